// gfx950 kernels of the KDA decode / spec-verify core.
//
// Sources (page titles, sections):
//   [kda]      "vllm.models.kimi_k3.amd.specialized_decode.mono.attention.kda",
//              module docstring, the role table's "kda tasks" row (what a
//              recurrence CTA does and in which order) and the functions
//              kda_conv, kda_gates, kda_recur and kda_norm.
//   [prepared] "vllm.models.kimi_k3.nvidia.specialized_decode.cutedsl.kda.prepared",
//              PreparedKda._operands (packed projection row), PreparedKda.__init__
//              (weights prepared once: fp32 norm weight, exp of A_log).
//
// Per (request, head) unit this kernel resolves the slots, loads everything
// it needs from memory before any arithmetic (the small per-token inputs
// first, then the 64 KiB fp32 state tile), runs the width-4 conv with SiLU,
// the gate contraction on the matrix cores and the decay gate, then for each
// token the l2 scales, decay, delta-rule update and output, storing the
// state after every token, and finally the gated RMSNorm of each token's 128
// outputs into bf16 core_out and the shifted conv windows.
//
// One workgroup owns one (request, head) unit for all L tokens: 8 waves of 64,
// wave w holding state rows v = 16w .. 16w + 15 in registers across the token
// loop (the pages split a head into eight 16-row v-chunks on separate CTAs
// that trade q/k and norm partials through mailboxes; here the eight chunks
// are the eight waves of one workgroup and the hand-offs go through LDS).
// One-token calls and grids of at most one unit a CU use 16 waves of 8 rows.
//
// Lane layout of the state: lane l of wave w holds rows 16w + (l >> 3) and
// 16w + 8 + (l >> 3) (16 waves: row 8w + (l >> 3)), columns 32m + 4(l & 7) ..
// +3 for m = 0..3. One dwordx4 load or store instruction therefore covers
// eight full 128-byte lines (eight rows x 128 B), and a row's dot product is
// an 8-lane reduction done with three DPP steps.
#include "kda_internal.h"

#include <algorithm>

namespace kda {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float bf16_to_f32(uint32_t bits) {
    return __uint_as_float(bits << 16);
}

// Round to nearest even (gfx950 converts fp32 -> bf16 in hardware).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// The bf16 value nearest x (ties to even), back in fp32: a bf16 hand-off.
__device__ __forceinline__ float round_bf16(float x) {
    return bf16_to_f32(f32_to_bf16(x));
}

__device__ __forceinline__ float exp_fast(float x) {
    return __builtin_amdgcn_exp2f(x * kLog2e);
}

// 1 / (1 + e^-x): saturates to 0 at -inf and 1 at +inf without overflow.
__device__ __forceinline__ float sigmoid(float x) {
    return __builtin_amdgcn_rcpf(1.0f + exp_fast(-x));
}

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// Sum over the 8 lanes l with the same l >> 3 (one state row).
__device__ __forceinline__ float sum8(float x) {
    x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]: partner lane ^ 1
    x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]: partner lane ^ 2
    x += dpp<0x141>(x);  // row_half_mirror: partner lane 7 - i of the 8
    return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m, 64);
    return x;
}

__device__ __forceinline__ float dot4(f32x4 a, f32x4 b, float acc) {
    acc = __builtin_fmaf(a.x, b.x, acc);
    acc = __builtin_fmaf(a.y, b.y, acc);
    acc = __builtin_fmaf(a.z, b.z, acc);
    acc = __builtin_fmaf(a.w, b.w, acc);
    return acc;
}

template <int L, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void kda_core_kernel(const CoreParams p) {
    static_assert(WAVES == 8 || WAVES == 16, "8 or 16 waves a (request, head) unit");
    constexpr int N = kHeadDim;
    constexpr int RW = N / WAVES;        // state rows a wave holds: 16 or 8
    constexpr int G = RW / 8;            // 8-row groups a lane holds: 2 or 1
    constexpr int NT = 64 * WAVES;
    const int H = p.heads;
    const int D = H * N;
    // XCD-blocked unit order: the dispatcher sends workgroup b to XCD b % 8, so
    // XCD x takes a contiguous block of (request, head) units (measured 4 %
    // faster than request-major order on MI355X for the 64 x 8 verify and the
    // 256-request decode batches; any order is correct).
    int unit = blockIdx.x;
    {
        const int q = (p.requests * H) >> 3;
        if ((int)blockIdx.x < 8 * q) unit = (blockIdx.x & 7) * q + (blockIdx.x >> 3);
    }
    const int r = unit / H;
    const int h = unit - r * H;
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;

    __shared__ float s_qkv[L][3 * N];   // conv outputs q | k | v (raw: l2 scales applied later)
    __shared__ float s_eg[L][N];        // e^g per key channel
    __shared__ float s_gate[L][N];      // output gate (raw)
    __shared__ float s_o[L][N];         // recurrence outputs
    __shared__ float s_braw[L];
    // conv windows after each token in the dim-first layout: channel cl's three
    // inputs at 3 cl .. 3 cl + 2 (the global order of one head's q, k, v runs)
    __shared__ __attribute__((aligned(16))) uint16_t s_win[L][3 * N * 3];

    // ---- slot resolution ([prepared] run: slots [B], or [>= B, q] + accepted).
    // The accepted count and the slot row are loaded together and the carried
    // slot is picked among the loaded values, so one round trip to memory
    // precedes the state stream.
    const int32_t* srow = p.slots + (int64_t)r * p.slots_row_stride;
    // unconditional load (the slot row stands in for a missing accepted array),
    // so that it issues together with the slot loads
    const int a_raw = *(p.accepted != nullptr ? p.accepted + r : srow);
    int dst[L];
#pragma unroll
    for (int t = 0; t < L; ++t) dst[t] = srow[t];
    const int a = p.accepted != nullptr ? a_raw : 1;
    bool ok = a >= 1 && a <= L;
    int src = dst[0];
#pragma unroll
    for (int t = 0; t < L; ++t) {
        ok = ok && (unsigned)dst[t] < (unsigned)p.num_slots;
        if (t == a - 1) src = dst[t];
    }
    if (ok && p.claims != nullptr) {   // distinct-destination check (opt-in)
#pragma unroll
        for (int t = 0; t < L; ++t) ok = ok && p.claims[dst[t]] == 1;
    }
    if (!ok) {  // uniform across the workgroup: skip the whole request
        if (h == 0 && tid == 0) atomicAdd(p.err_count, 1);
        return;
    }

    const int64_t row0 = (int64_t)r * L;
    const uint16_t* prow = p.projected + row0 * p.pitch;

    // ---- small inputs first: conv window + x (waves 0-5), gate + beta (6-7)
    const bool conv_thread = tid < 3 * N;
    const bool gate_thread = !conv_thread && (WAVES == 8 || tid < 4 * N);   // 16 waves: 8-15 neither
    const int cl = conv_thread ? tid : tid - 3 * N;   // conv channel, or gate column
    const int cs = cl >> 7;                           // 0 q, 1 k, 2 v
    const int cj = cl & (N - 1);
    const int64_t cch = (int64_t)cs * D + (int64_t)h * N + cj;   // channel in 0 .. 3D
    uint32_t win[kWidth - 1];
    uint32_t xb[L];
    float cw[kWidth];
    float cb = 0.0f;
    uint32_t braw = 0;
    if (conv_thread) {
        const int64_t cbase = (int64_t)src * p.conv_slot_stride + cch * p.conv_dim_stride;
#pragma unroll
        for (int m = 0; m < kWidth - 1; ++m) win[m] = p.conv[cbase + m * p.conv_pos_stride];
#pragma unroll
        for (int t = 0; t < L; ++t) xb[t] = prow[t * p.pitch + cch];
        // the channel's four taps in one 16-byte load: the small loads issued
        // before the state stream are on the path to it, and four dword loads
        // here measured 2 us slower for the 64 x 8 verify batch
        const f32x4 w4 = *reinterpret_cast<const f32x4*>(p.conv_w + cch * kWidth);
        cw[0] = w4.x; cw[1] = w4.y; cw[2] = w4.z; cw[3] = w4.w;
        cb = p.conv_b[cch];
    } else if (gate_thread) {
#pragma unroll
        for (int t = 0; t < L; ++t) xb[t] = prow[t * p.pitch + 3 * (int64_t)D + (int64_t)h * N + cj];
        // unconditional (clamped row): a load under a per-lane branch here makes
        // the compiler wait for every outstanding load before these waves issue
        // their state stream
        braw = prow[min(cj, L - 1) * p.pitch + 4 * (int64_t)D + kFaRank + h];
    }

    // ---- gate MFMA operands: wave w < 8 computes outputs 16w .. 16w + 15 of the head
    const bool mfma_wave = WAVES == 8 || wave < 8;
    const int mn = lane & 15;        // A row (token) / B column (output)
    const int kg = lane >> 4;        // which 8 of each 32-wide K step
    const int i_out = (WAVES == 8 ? wave : (wave & 7)) * 16 + mn;
    bf16x8 bfrag[4];
    if (mfma_wave) {
        const uint16_t* fb = p.f_b + (int64_t)(h * N + i_out) * kFaRank + 8 * kg;
#pragma unroll
        for (int s = 0; s < 4; ++s)
            bfrag[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(fb + 32 * s));
    } else {
#pragma unroll
        for (int s = 0; s < 4; ++s) bfrag[s] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
    }
    bf16x8 afrag[4];
    if (mfma_wave && mn < L && !p.fa_u16) {   // rows are only 4-byte aligned: dword loads
        const uint32_t* fa = reinterpret_cast<const uint32_t*>(prow + mn * p.pitch + 4 * (int64_t)D + 8 * kg);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            u32x4 v = {fa[16 * s + 0], fa[16 * s + 1], fa[16 * s + 2], fa[16 * s + 3]};
            afrag[s] = __builtin_bit_cast(bf16x8, v);
        }
    } else if (mfma_wave && mn < L) {         // odd pitch or base: 2-byte loads
        const uint16_t* fa = prow + mn * p.pitch + 4 * (int64_t)D + 8 * kg;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            uint32_t w[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
                w[e] = (uint32_t)fa[32 * s + 2 * e] | ((uint32_t)fa[32 * s + 2 * e + 1] << 16);
            afrag[s] = __builtin_bit_cast(bf16x8, u32x4{w[0], w[1], w[2], w[3]});
        }
    } else {
#pragma unroll
        for (int s = 0; s < 4; ++s) afrag[s] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
    }
    const float dtv = mfma_wave ? p.dt_bias[h * N + i_out] : 0.0f;
    const float aexp = p.a_exp[h];
    float nw0 = 0.0f, nw1 = 0.0f;
    if (wave < L) {
        nw0 = p.norm_w[h * N + 2 * lane];
        nw1 = p.norm_w[h * N + 2 * lane + 1];
    }

    // ---- the carried state: 64 KiB a unit, read once. A one-token call
    // overwrites the tile it reads (in place), and a plain load would leave its
    // lines in L2 just before the non-temporal stores replace them; there the
    // load is non-temporal too. With L > 1 the tokens write other slots and
    // plain loads measured faster on MI355X.
    const int rsub = lane >> 3;
    const int csub = (lane & 7) * 4;
    const int64_t unit_off = (int64_t)h * N * N + (int64_t)(wave * RW + rsub) * N + csub;
    // A bare barrier (no fence, no wait for data) before the state stream: every
    // wave's small loads above enter the CU's memory pipeline ahead of any
    // wave's 8 KiB share of the tile. Without it, the waves issued last (the v
    // conv and gate waves) find their conv and gate inputs queued behind the
    // other waves' state loads, and the first barrier below waits for them
    // (measured 3 % slower for the 64 x 8 verify batch on MI355X). The early
    // return above is uniform across the workgroup, so every wave arrives here.
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
    f32x4 S[G][4];
    {
        const float* sb = p.state + (int64_t)src * p.state_slot_stride + unit_off;
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const f32x4* ptr = reinterpret_cast<const f32x4*>(sb + g * 8 * N + 32 * m);
                S[g][m] = (L == 1) ? __builtin_nontemporal_load(ptr) : *ptr;
            }
    }

    // ---- conv update + SiLU; the window after token t goes to slot dst[t]
    if (conv_thread) {
        float w0 = bf16_to_f32(win[0]), w1 = bf16_to_f32(win[1]), w2 = bf16_to_f32(win[2]);
        uint32_t b0 = win[0], b1 = win[1], b2 = win[2];
#pragma unroll
        for (int t = 0; t < L; ++t) {
            const float x = bf16_to_f32(xb[t]);
            float pre = __builtin_fmaf(cw[0], w0, cb);
            pre = __builtin_fmaf(cw[1], w1, pre);
            pre = __builtin_fmaf(cw[2], w2, pre);
            pre = __builtin_fmaf(cw[3], x, pre);
            const float y = pre * sigmoid(pre);
            s_qkv[t][cl] = p.handoff_bf16 ? round_bf16(y) : y;
            w0 = w1; w1 = w2; w2 = x;
            b0 = b1; b1 = b2; b2 = xb[t];
            if (p.conv_dim_first16) {   // staged; written below with 16-byte stores
                s_win[t][3 * cl] = (uint16_t)b0;
                s_win[t][3 * cl + 1] = (uint16_t)b1;
                s_win[t][3 * cl + 2] = (uint16_t)b2;
            } else {
                uint16_t* cw_out = p.conv + (int64_t)dst[t] * p.conv_slot_stride + cch * p.conv_dim_stride;
                cw_out[0] = (uint16_t)b0;
                cw_out[p.conv_pos_stride] = (uint16_t)b1;
                cw_out[2 * p.conv_pos_stride] = (uint16_t)b2;
            }
        }
    } else if (gate_thread) {
#pragma unroll
        for (int t = 0; t < L; ++t) s_gate[t][cj] = bf16_to_f32(xb[t]);
        if (cj < L) s_braw[cj] = bf16_to_f32(braw);
    }

    // ---- g1 = f_b f_a on MFMA (tokens padded to 16), then the lower-bound gate
    if (mfma_wave) {
        f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int s = 0; s < 4; ++s)
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afrag[s], bfrag[s], acc, 0, 0, 0);
        // lane holds tokens 4 kg + i, output column mn
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = 4 * kg + i;
            if (t < L) {
                const float g1 = p.handoff_bf16 ? round_bf16(acc[i]) : acc[i];
                const float g = p.lb * sigmoid(aexp * (g1 + dtv));
                s_eg[t][i_out] = exp_fast(g);
            }
        }
    }
    __syncthreads();

    // ---- the recurrence over the L tokens, a state stored per token. Every
    // wave takes the l2norm scales of q and k (and k . q) itself from the raw
    // conv outputs: a lane's 16 columns, summed over the 8 lanes of a row, cover
    // all 128 channels (the same reduction as the row dot products), so no
    // second barrier is needed. With k_hat = ks k and q_hat = qs q:
    //   (S k_hat) = ks (S k), (S q_hat) = qs (S q), k_hat . q_hat = ks qs (k . q).
#pragma unroll
    for (int t = 0; t < L; ++t) {
        f32x4 eg[4], kk[4], qq[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            eg[m] = *reinterpret_cast<const f32x4*>(&s_eg[t][32 * m + csub]);
            qq[m] = *reinterpret_cast<const f32x4*>(&s_qkv[t][32 * m + csub]);
            kk[m] = *reinterpret_cast<const f32x4*>(&s_qkv[t][N + 32 * m + csub]);
        }
        float sq = 0.0f, sk = 0.0f, skq = 0.0f;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            sq = dot4(qq[m], qq[m], sq);
            sk = dot4(kk[m], kk[m], sk);
            skq = dot4(kk[m], qq[m], skq);
        }
        const float qs = p.q_scale * __builtin_amdgcn_rsqf(sum8(sq) + p.l2_eps);
        const float ks = __builtin_amdgcn_rsqf(sum8(sk) + p.l2_eps);
        const float kq = qs * ks * sum8(skq);     // k_hat . q_hat
        const float beta = sigmoid(s_braw[t]);
        float* dp = p.state + (int64_t)dst[t] * p.state_slot_stride + unit_off;
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const int row = wave * RW + g * 8 + rsub;
            float a = 0.0f, b = 0.0f;
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                S[g][m] *= eg[m];                 // decay: column i scaled by e^g_i
                a = dot4(S[g][m], kk[m], a);      // (S k)_row, decayed state
                b = dot4(S[g][m], qq[m], b);      // (S q)_row, decayed state
            }
            a = ks * sum8(a);                     // (S k_hat)_row
            b = qs * sum8(b);                     // (S q_hat)_row
            const float bu = beta * (s_qkv[t][2 * N + row] - a);
            // o = (S_decayed + bu k_hat^T) q_hat = b + bu (k_hat . q_hat)
            const float o = __builtin_fmaf(bu, kq, b);
            const float buk = bu * ks;            // rank-1 update along k_hat = ks k
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                S[g][m] += buk * kk[m];
                __builtin_nontemporal_store(S[g][m],
                                            reinterpret_cast<f32x4*>(dp + g * 8 * N + 32 * m));
            }
            if ((lane & 7) == 0) s_o[t][row] = p.handoff_bf16 ? round_bf16(o) : o;
        }
    }
    __syncthreads();

    // ---- gated RMSNorm over the head's 128 outputs -> bf16 core_out: wave t for token t
    if (wave < L) {
        const int t = wave;
        const float o0 = s_o[t][2 * lane], o1 = s_o[t][2 * lane + 1];
        const float ss = wave_sum(o0 * o0 + o1 * o1);
        const float rstd = __builtin_amdgcn_rsqf(ss * (1.0f / N) + p.norm_eps);
        const float y0 = o0 * rstd * nw0 * sigmoid(s_gate[t][2 * lane]);
        const float y1 = o1 * rstd * nw1 * sigmoid(s_gate[t][2 * lane + 1]);
        const uint32_t packed = f32_to_bf16(y0) | (f32_to_bf16(y1) << 16);
        uint32_t* op = reinterpret_cast<uint32_t*>(p.out + (row0 + t) * D + (int64_t)h * N + 2 * lane);
        *op = packed;
    }

    // ---- coalesced conv window stores (dim-first pool): per token, the head's
    // q, k and v windows are 3 runs of 128 channels x 3 bf16 = 768 B, i.e.
    // 48 chunks of 16 B each; 2-byte stores at a 6-byte stride cost far more
    // than their bytes. Issued last, after the state stores and core_out, so they
    // do not queue ahead of the state traffic that bounds the kernel; s_win is
    // filled before the first barrier and never overwritten.
    if (p.conv_dim_first16) {
        constexpr int kChunks = 3 * 48;
        for (int c = tid; c < L * kChunks; c += NT) {
            const int t = c / kChunks, k = c - t * kChunks, s = k / 48;
            int slot = dst[0];
#pragma unroll
            for (int u = 1; u < L; ++u)
                if (t == u) slot = dst[u];
            uint16_t* out = p.conv + (int64_t)slot * p.conv_slot_stride +
                            ((int64_t)s * D + (int64_t)h * N) * 3 + (k - s * 48) * 8;
            *reinterpret_cast<u32x4*>(out) = *reinterpret_cast<const u32x4*>(&s_win[t][8 * k]);
        }
    }
}

// Element i of a small weight given as bf16 or fp32.
__device__ __forceinline__ float load_weight(const void* p, int64_t i, bool bf16) {
    return bf16 ? bf16_to_f32(static_cast<const uint16_t*>(p)[i]) : static_cast<const float*>(p)[i];
}

// Weight preparation ([prepared] PreparedKda.__init__): conv weight [3D][1][W]
// -> fp32 [3D][W] (the nn.Conv1d order, widened: a channel's taps are one
// 16-byte row; the prepared page's decode layout [3][W][D] would take four
// loads a channel here), bias -> fp32
// (zeros if absent), f_b copied, A_log -> exp(A_log), dt_bias -> fp32, norm
// weight expanded to fp32 [H][128]. One grid-stride pass over all items.
__global__ void kda_prepare_kernel(const PrepareParams in, const PreparedWeights out) {
    const int64_t H = in.heads, D = H * kHeadDim, C = 3 * D;
    const int64_t n_w = C * kWidth, n_b = C, n_fb = D * kFaRank, n_a = H, n_dt = D,
                  n_nw = H * kHeadDim;
    const int64_t total = n_w + n_b + n_fb + n_a + n_dt + n_nw;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total;
         e += (int64_t)gridDim.x * blockDim.x) {
        int64_t i = e;
        if (i < n_w) {   // i = c * W + j: the nn.Conv1d order
            out.conv_w[i] = bf16_to_f32(in.conv_weight[i]);
            continue;
        }
        i -= n_w;
        if (i < n_b) {
            out.conv_b[i] = in.conv_bias ? bf16_to_f32(in.conv_bias[i]) : 0.0f;
            continue;
        }
        i -= n_b;
        if (i < n_fb) {
            out.f_b[i] = in.f_b[i];
            continue;
        }
        i -= n_fb;
        if (i < n_a) {
            out.a_exp[i] = expf(load_weight(in.A_log, i, in.A_log_bf16));
            continue;
        }
        i -= n_a;
        if (i < n_dt) {
            out.dt_bias[i] = load_weight(in.dt_bias, i, in.dt_bias_bf16);
            continue;
        }
        i -= n_dt;
        out.norm_w[i] = load_weight(in.norm_weight, (i / kHeadDim) * in.norm_head_stride + i % kHeadDim,
                                    in.norm_weight_bf16);
    }
}

__global__ void kda_zero_kernel(int32_t* p, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0;
}

// One thread per request: the request's validity under the core kernel's
// rules, then one claim per token on its destination slot (or the claims'
// reset after the core kernel has read them). The claim counts reach the core
// kernel through stream order; a slot claimed more than once in the call
// makes every request naming it skip.
template <int L>
__global__ __launch_bounds__(256) void kda_claim_kernel(const CoreParams p, int32_t* claims, int clear) {
    const int r = blockIdx.x * 256 + threadIdx.x;
    if (r >= p.requests) return;
    const int32_t* srow = p.slots + (int64_t)r * p.slots_row_stride;
    const int a = p.accepted != nullptr ? p.accepted[r] : 1;
    bool ok = a >= 1 && a <= L;
    int dst[L];
#pragma unroll
    for (int t = 0; t < L; ++t) {
        dst[t] = srow[t];
        ok = ok && (unsigned)dst[t] < (unsigned)p.num_slots;
    }
    if (!ok) return;
#pragma unroll
    for (int t = 0; t < L; ++t) {
        if (clear)
            claims[dst[t]] = 0;
        else
            atomicAdd(claims + dst[t], 1);
    }
}

template <int L>
hipError_t launch_claims_t(const CoreParams& p, int32_t* claims, bool clear, hipStream_t s) {
    const unsigned blocks = (unsigned)((p.requests + 255) / 256);
    hipLaunchKernelGGL((kda_claim_kernel<L>), dim3(blocks), dim3(256), 0, s, p, claims, clear ? 1 : 0);
    return hipGetLastError();
}

// Waves a unit (measured on MI355X, one device, alternating runs): sixteen 8-row
// waves for every one-token call (in-place decode: 73.8 against 77.5 us for
// 256 requests x 12 heads, 21.4 against 22.6 for 64, although only one such
// workgroup fits a CU) and for grids of at most one unit a CU, where a unit's
// per-token arithmetic would otherwise sit exposed between its store bursts
// (verify 16 x 4: 12.4 against 13.2 us); eight 16-row waves, two units a CU,
// for larger multi-token grids (verify 64 x 8: 78.3 against 78.9 us). "One
// unit a CU" counts the device's compute units (256 on a whole MI355X, fewer
// on a partition of one).
template <int L>
hipError_t launch_core_t(const CoreParams& p, hipStream_t s) {
    const dim3 grid((unsigned)(p.requests * p.heads));
    if constexpr (L == 1) {
        hipLaunchKernelGGL((kda_core_kernel<1, 16>), grid, dim3(1024), 0, s, p);
    } else {
        if ((int64_t)p.requests * p.heads <= p.cu_count)
            hipLaunchKernelGGL((kda_core_kernel<L, 16>), grid, dim3(1024), 0, s, p);
        else
            hipLaunchKernelGGL((kda_core_kernel<L, 8>), grid, dim3(512), 0, s, p);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prepare(const PrepareParams& in, const PreparedWeights& out, hipStream_t s) {
    hipLaunchKernelGGL(kda_prepare_kernel, dim3(256), dim3(256), 0, s, in, out);
    return hipGetLastError();
}

hipError_t launch_zero(int32_t* p, int64_t n, hipStream_t s) {
    const int64_t blocks = std::min<int64_t>(1024, (n + 255) / 256);
    hipLaunchKernelGGL(kda_zero_kernel, dim3((unsigned)std::max<int64_t>(blocks, 1)), dim3(256), 0, s, p, n);
    return hipGetLastError();
}

hipError_t launch_claims(int tokens, const CoreParams& p, int32_t* claims, bool clear, hipStream_t s) {
    switch (tokens) {
        case 1: return launch_claims_t<1>(p, claims, clear, s);
        case 2: return launch_claims_t<2>(p, claims, clear, s);
        case 3: return launch_claims_t<3>(p, claims, clear, s);
        case 4: return launch_claims_t<4>(p, claims, clear, s);
        case 5: return launch_claims_t<5>(p, claims, clear, s);
        case 6: return launch_claims_t<6>(p, claims, clear, s);
        case 7: return launch_claims_t<7>(p, claims, clear, s);
        case 8: return launch_claims_t<8>(p, claims, clear, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_core(int tokens, const CoreParams& p, hipStream_t s) {
    switch (tokens) {
        case 1: return launch_core_t<1>(p, s);
        case 2: return launch_core_t<2>(p, s);
        case 3: return launch_core_t<3>(p, s);
        case 4: return launch_core_t<4>(p, s);
        case 5: return launch_core_t<5>(p, s);
        case 6: return launch_core_t<6>(p, s);
        case 7: return launch_core_t<7>(p, s);
        case 8: return launch_core_t<8>(p, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace kda
