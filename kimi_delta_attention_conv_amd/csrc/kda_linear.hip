// gfx950 projection kernel around the KDA core: Y[M][N] = X[M][K] W[N][K]^T,
// bf16 inputs, fp32 accumulation on MFMA, bf16 output.
//
// Sources (page titles, sections):
//   "vllm.models.kimi_k3.amd.specialized_decode.mono.attention.kda", module
//   docstring, gemv role: in_proj produces the packed q|k|v|g|f_a|beta row,
//   16 weight rows to a group, tokens on the other side of the product.
//   "vllm.models.kimi_k3.amd.specialized_decode.mono.attention.back", module
//   docstring and stage_o: o_proj over the core rows (K = 1536 local), an
//   MFMA GEMV with the token dimension padded to 16.
//
// Four GEMM kernels, chosen by the row count M and K, and a slice sum:
//
// Skinny (M <= 16 when K is a multiple of 64 but not of 128, up to 64 rows
// when K is not a multiple of 64): both operands are K-contiguous (rows of X,
// rows of the nn.Linear weight W), so
// every lane reads 64 contiguous bytes of one row per 128-wide K block and
// feeds v_mfma_f32_16x16x32_bf16 directly from registers. Within a K block,
// lane group kg (= lane >> 4) hands K elements 8 (kg + 4q) .. +8 to MFMA K
// step q; A and B use the same assignment, so the product is unchanged. A
// workgroup computes 16 * NT output columns for 16 * MT rows; its waves take
// the K blocks round-robin and their partial tiles are summed through LDS in
// wave order (a fixed order: results do not depend on timing).
//
// Direct-to-LDS (K a multiple of 128, or K a multiple of 64 and M > 16): BM x
// BN tiles, X and W blocks loaded straight into a ring of LDS stages; with a
// caller's workspace and a long K (33 to 256 rows) the same kernel splits K
// over 4 slices of workgroups and linear_split_sum adds the fp32 slices in
// slice order. Pipelined (above 256 rows, K >= 4096, tiles filling three
// quarters to all but one of the CUs): the same tiles and arithmetic with the
// fragment reads overlapping the MFMAs and the idle CUs loading the tiles' W
// lines ahead of them. Tiled (M > 64, other K): 128 x 64 tiles staged through
// registers.
#include "kda_internal.h"

#include <atomic>

namespace kda {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kKBlock = 128;

// 16 bytes, or zero without a load when `ok` is false. (The skinny kernel
// measured faster with this guarded form than with clamped unconditional
// loads; the tiled kernel below loads unconditionally instead.)
__device__ __forceinline__ bf16x8 load8(const uint16_t* p, bool ok) {
    const u32x4 z = {0u, 0u, 0u, 0u};
    return __builtin_bit_cast(bf16x8, ok ? *reinterpret_cast<const u32x4*>(p) : z);
}

__device__ __forceinline__ uint16_t to_bf16(float f) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

template <int MT, int NT, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void linear_skinny_kernel(const LinearParams p) {
    const int n0 = blockIdx.x * (16 * NT);
    const int m0 = blockIdx.y * (16 * MT);
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int mn = lane & 15;   // B column (output n) / A row (token m) of this lane
    const int kg = lane >> 4;   // which 32-wide slice of each K block

    // out-of-range rows read nothing and are zero
    const uint16_t* wrow[NT];
    bool n_ok[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        const int n = n0 + 16 * j + mn;
        n_ok[j] = n < p.N;
        wrow[j] = p.W + (int64_t)(n_ok[j] ? n : p.N - 1) * p.K;
    }
    const uint16_t* xrow[MT];
    bool m_ok[MT];
#pragma unroll
    for (int i = 0; i < MT; ++i) {
        const int m = m0 + 16 * i + mn;
        m_ok[i] = m < p.M;
        xrow[i] = p.X + (int64_t)(m_ok[i] ? m : p.M - 1) * p.x_pitch;
    }

    f32x4 acc[MT][NT];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    const int nkb = (p.K + kKBlock - 1) / kKBlock;
    for (int kb = wave; kb < nkb; kb += WAVES) {
        // K step q of this lane uses elements 8 (kg + 4q) .. +8 of the block:
        // the 4 lanes of a row read 64 contiguous bytes per load instruction
        const int kbase = kb * kKBlock + 8 * kg;
        bf16x8 b[NT][4];
#pragma unroll
        for (int j = 0; j < NT; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                b[j][q] = load8(wrow[j] + kbase + 32 * q, n_ok[j] && kbase + 32 * q + 8 <= p.K);
#pragma unroll
        for (int i = 0; i < MT; ++i) {
            bf16x8 a[4];
#pragma unroll
            for (int q = 0; q < 4; ++q)
                a[q] = load8(xrow[i] + kbase + 32 * q, m_ok[i] && kbase + 32 * q + 8 <= p.K);
#pragma unroll
            for (int j = 0; j < NT; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[q], b[j][q], acc[i][j], 0, 0, 0);
        }
    }

    // sum the waves' partial tiles in wave order; lane holds rows 4 kg + r
    // (r = 0..3) of each 16-row tile, column mn of each 16-column tile
    __shared__ float red[WAVES][MT * NT * 4][64];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) red[wave][(i * NT + j) * 4 + r][lane] = acc[i][j][r];
    __syncthreads();
    for (int e = threadIdx.x; e < MT * NT * 4 * 64; e += 64 * WAVES) {
        const int ijr = e >> 6, l = e & 63;
        float s = red[0][ijr][l];
#pragma unroll
        for (int w = 1; w < WAVES; ++w) s += red[w][ijr][l];
        const int i = (ijr >> 2) / NT, j = (ijr >> 2) % NT;
        const int m = m0 + 16 * i + 4 * (l >> 4) + (ijr & 3);
        const int nn = n0 + 16 * j + (l & 15);
        if (m < p.M && nn < p.N) p.Y[(int64_t)m * p.y_pitch + nn] = to_bf16(s);
    }
}

// Tiled kernel for larger M: a workgroup of 4 waves computes a BM x BN tile
// (waves 2 x 2, each (BM/2) x (BN/2) as 16 x 16 MFMA tiles). K advances in
// blocks of 64: each block of X and W rows is staged through LDS (rows padded
// by 16 bytes) and the next block's global loads are in flight while the
// current one is multiplied, with one barrier per block.
constexpr int kTileK = 64;
constexpr int kLdsRow = kTileK + 8;   // elements; 144-byte rows

template <int BM, int BN, int DEPTH>
__global__ __launch_bounds__(256) void linear_tiled_kernel(const LinearParams p) {
    constexpr int TM = BM / 32;            // 16-row tiles per wave
    constexpr int TN = BN / 32;            // 16-column tiles per wave
    constexpr int A_LD = BM * 8 / 256;     // 16-byte pieces of the X block per thread
    constexpr int B_LD = BN * 8 / 256;     // 16-byte pieces of the W block per thread
    __shared__ __attribute__((aligned(16))) uint16_t sA[2][BM][kLdsRow];
    __shared__ __attribute__((aligned(16))) uint16_t sB[2][BN][kLdsRow];

    // XCD-aware tile order: workgroup g runs on XCD g % 8; XCD x takes a
    // contiguous range of tiles, M-blocks of one N-block adjacent, so the
    // workgroups that share a W slab (and the X rows) meet in one XCD's L2.
    const int mblocks = (p.M + BM - 1) / BM;
    const int tiles = mblocks * ((p.N + BN - 1) / BN);
    int t = blockIdx.x;
    {
        const int q = tiles >> 3;
        if ((int)blockIdx.x < 8 * q) t = (blockIdx.x & 7) * q + (blockIdx.x >> 3);
    }
    const int m0 = (t % mblocks) * BM;
    const int n0 = (t / mblocks) * BN;
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int wm = wave >> 1, wn = wave & 1;
    const int mn = lane & 15, kg = lane >> 4;

    // Register stages of the global -> LDS copy: stage d holds K block kb with
    // kb % DEPTH == d, so DEPTH - 1 blocks are in flight while one is
    // multiplied. Piece q of a thread is piece q * 256 + tid of the block:
    // row piece / 8, K elements 8 * (piece % 8) .. +8, so 8 consecutive lanes
    // read one 128-byte row segment.
    u32x4 ra[DEPTH][A_LD], rb[DEPTH][B_LD];
    const int nkb = (p.K + kTileK - 1) / kTileK;
    // Addresses are clamped into the matrices, so every load is valid and
    // unconditional (a branch around each load would make the compiler wait
    // for all outstanding loads at the loop head, serialising the prefetch):
    // rows past M of X and past N of W only feed outputs that are never
    // stored, and blocks past the end are never copied to LDS. Only K elements
    // past K (a K that is not a multiple of 64) are zeroed, at the LDS store of
    // the last block.
    auto gload = [&](u32x4 (&a)[A_LD], u32x4 (&b)[B_LD], int kb) {
#pragma unroll
        for (int q = 0; q < A_LD; ++q) {
            const int piece = q * 256 + tid, row = piece >> 3, k = kb * kTileK + 8 * (piece & 7);
            a[q] = *reinterpret_cast<const u32x4*>(
                p.X + (int64_t)min(m0 + row, p.M - 1) * p.x_pitch + min(k, p.K - 8));
        }
#pragma unroll
        for (int q = 0; q < B_LD; ++q) {
            const int piece = q * 256 + tid, row = piece >> 3, k = kb * kTileK + 8 * (piece & 7);
            b[q] = *reinterpret_cast<const u32x4*>(
                p.W + (int64_t)min(n0 + row, p.N - 1) * p.K + min(k, p.K - 8));
        }
    };
    auto lstore = [&](const u32x4 (&a)[A_LD], const u32x4 (&b)[B_LD], int buf, int kb) {
        const bool tail = kb * kTileK + kTileK > p.K;   // uniform
#pragma unroll
        for (int q = 0; q < A_LD; ++q) {
            const int piece = q * 256 + tid;
            const bool ok = !tail || kb * kTileK + 8 * (piece & 7) + 8 <= p.K;
            *reinterpret_cast<u32x4*>(&sA[buf][piece >> 3][8 * (piece & 7)]) =
                ok ? a[q] : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int q = 0; q < B_LD; ++q) {
            const int piece = q * 256 + tid;
            const bool ok = !tail || kb * kTileK + 8 * (piece & 7) + 8 <= p.K;
            *reinterpret_cast<u32x4*>(&sB[buf][piece >> 3][8 * (piece & 7)]) =
                ok ? b[q] : u32x4{0u, 0u, 0u, 0u};
        }
    };

    f32x4 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

#pragma unroll
    for (int d = 0; d < DEPTH; ++d) gload(ra[d], rb[d], d);
    lstore(ra[0], rb[0], 0, 0);
    __syncthreads();
    for (int base = 0; base < nkb; base += DEPTH) {
#pragma unroll
        for (int u = 0; u < DEPTH; ++u) {
            const int kb = base + u;
            if (kb >= nkb) break;
            const int buf = kb & 1;
            // stage u held block kb (now in LDS): refill it with block kb + DEPTH
            gload(ra[u], rb[u], kb + DEPTH);
#pragma unroll
            for (int s = 0; s < kTileK / 32; ++s) {
                bf16x8 a[TM], b[TN];
#pragma unroll
                for (int i = 0; i < TM; ++i)
                    a[i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(
                        &sA[buf][wm * (BM / 2) + 16 * i + mn][32 * s + 8 * kg]));
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    b[j] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(
                        &sB[buf][wn * (BN / 2) + 16 * j + mn][32 * s + 8 * kg]));
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
            }
            if (kb + 1 < nkb) lstore(ra[(u + 1) % DEPTH], rb[(u + 1) % DEPTH], buf ^ 1, kb + 1);
            __syncthreads();
        }
    }

    // lane holds rows 4 kg + r (r = 0..3) of each 16-row tile, column mn
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int n = n0 + wn * (BN / 2) + 16 * j + mn;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = m0 + wm * (BM / 2) + 16 * i + 4 * kg + r;
                if (m < p.M && n < p.N) p.Y[(int64_t)m * p.y_pitch + n] = to_bf16(acc[i][j][r]);
            }
        }
}

// Direct-to-LDS kernel for M > 64 and K a multiple of 64. A workgroup of
// WGM x WGN waves computes a BM x BN tile; K advances in blocks of 64 through a
// ring of STAGES LDS buffers that gfx950's global_load_lds_dwordx4 fills without
// passing through registers, STAGES - 1 blocks ahead of the block multiplied.
// One explicit vmcnt wait and one barrier per block: register-staged copies
// made the compiler wait for every load in flight at the loop head, which left
// each block's global latency exposed.
//
// LDS per stage: [BM + BN rows][64 k] bf16 (X rows, then W rows), 128-byte rows
// without padding. A direct load writes 64 lanes x 16 bytes contiguously, so
// each wave load fills 8 rows; lane l fetches chunk (l & 7) ^ (l >> 3) of its
// row, which places chunk c of row r at position c ^ (r & 7). The MFMA
// fragment reads (16 rows, one chunk each) then hit 16 distinct bank groups.
//
// With KS = 2 the waves form two groups that take the two 32-wide halves of
// every K block (each wave's fragment reads per block halve while its tile
// stays large); the groups' partial tiles are summed through LDS at the end.
//
// A stage holds SUB consecutive 64-wide K blocks (each in the layout above),
// so one wait and one barrier cover SUB blocks and each row is fetched in
// SUB x 128-byte runs.
//
// With SPLIT > 1 the K range is cut into SPLIT equal slices, one workgroup a
// (tile, slice); each writes its fp32 tile to p.part in fragment order (every
// lane's four accumulators as one 16-byte run, lanes contiguous) and
// linear_split_sum adds the slices in slice order. The slices of a tile are
// consecutive workgroups, so with the round-robin placement of workgroups on
// the 8 XCDs (SPLIT dividing 8) each XCD works on one K slice and its L2 holds
// that slice of X for all of its workgroups.
template <int BM, int BN, int STAGES, int WGM, int WGN, int KS, int SUB, int SPLIT>
__global__ __launch_bounds__(64 * WGM * WGN * KS) void linear_lds_kernel(const LinearParams p) {
    static_assert(KS == 1 || KS == 2, "K split of a 64-wide block into 1 or 2 parts");
    constexpr int WAVES = WGM * WGN * KS;
    constexpr int ROWS = BM + BN;
    constexpr int LPB = ROWS / (8 * WAVES);        // direct loads per thread per K block
    constexpr int TM = BM / WGM / 16, TN = BN / WGN / 16;   // 16 x 16 tiles per wave
    static_assert(LPB * 8 * WAVES == ROWS, "rows must split into whole wave loads");
    __shared__ __attribute__((aligned(1024))) uint16_t sm[STAGES][SUB][ROWS * 64];

    static_assert(SPLIT == 1 || 8 % SPLIT == 0, "K slices map onto the 8 XCDs");
    const int mblocks = (p.M + BM - 1) / BM;
    const int tiles = mblocks * ((p.N + BN - 1) / BN);
    int t = blockIdx.x, slice = 0;
    if (SPLIT > 1) {
        slice = blockIdx.x % SPLIT;
        t = blockIdx.x / SPLIT;
    } else {
        const int q = tiles >> 3;
        if ((int)blockIdx.x < 8 * q) t = (blockIdx.x & 7) * q + (blockIdx.x >> 3);
    }
    const int m0 = (t % mblocks) * BM;
    const int n0 = (t / mblocks) * BN;
    const int kc = p.K / SPLIT;                   // this workgroup's K slice
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int kh = wave / (WGM * WGN);            // K part of this wave's group
    const int slot = wave % (WGM * WGN);          // tile position within the group
    const int wm = slot / WGN, wn = slot % WGN;
    const int mn = lane & 15, kg = lane >> 4;

    // this lane's global source for load j of a block: row 8 (4 j + wave) + (lane >> 3)
    // of [A rows; B rows], chunk (lane & 7) ^ (lane >> 3)
    const uint16_t* src[LPB];
#pragma unroll
    for (int j = 0; j < LPB; ++j) {
        const int row = 8 * (WAVES * j + wave) + (lane >> 3);
        const int chunk = (lane & 7) ^ (lane >> 3);
        src[j] = (row < BM
            ? p.X + (int64_t)min(m0 + row, p.M - 1) * p.x_pitch
            : p.W + (int64_t)min(n0 + row - BM, p.N - 1) * p.K) + slice * kc + 8 * chunk;
    }
    const int nkb = kc / (64 * SUB);             // stages of K (the launch checks K % (64 SUB SPLIT))
    auto issue = [&](int kb) {
#if defined(__HIP_DEVICE_COMPILE__)   // the builtin's LDS operand has no host type
        const int st = kb % STAGES;
        const int kk = min(kb, nkb - 1) * 64 * SUB;     // past the end: a harmless re-read
#pragma unroll
        for (int j = 0; j < LPB; ++j)
#pragma unroll
            for (int u = 0; u < SUB; ++u)
                __builtin_amdgcn_global_load_lds(src[j] + kk + 64 * u, &sm[st][u][8 * (WAVES * j + wave) * 64],
                                                 16, 0, 0);
#endif
    };

    f32x4 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

#pragma unroll
    for (int s = 0; s < STAGES - 1; ++s) issue(s);
    for (int kb = 0; kb < nkb; ++kb) {
        // stage kb has landed once at most (STAGES - 2) stages of loads are outstanding
        constexpr int N = (STAGES - 2) * LPB * SUB;
        static_assert(N < 64, "the vmcnt field holds 6 bits");
        __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
        // a plain barrier: a fenced one would also wait for the direct loads still
        // in flight for later blocks; the memory clobber keeps LDS reads and new
        // direct loads on their side of it
        __asm__ volatile("s_barrier" ::: "memory");
        issue(kb + STAGES - 1);                   // into the stage read one block ago
#pragma unroll
        for (int u = 0; u < SUB; ++u) {
        const uint16_t* st = sm[kb % STAGES][u];
#pragma unroll
        for (int s = kh * (2 / KS); s < (kh + 1) * (2 / KS); ++s) {
            bf16x8 a[TM], b[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const int row = wm * (BM / WGM) + 16 * i + mn;
                const int pos = (4 * s + kg) ^ (row & 7);
                a[i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(st + row * 64 + 8 * pos));
            }
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int row = BM + wn * (BN / WGN) + 16 * j + mn;
                const int pos = (4 * s + kg) ^ (row & 7);
                b[j] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(st + row * 64 + 8 * pos));
            }
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
        }
        }
    }
    __builtin_amdgcn_s_waitcnt(0);   // no direct load may still target LDS at exit

    if (KS == 2) {   // group 1 parks its tiles in the (now idle) stages, group 0 adds them
        static_assert(KS == 1 || WGM * WGN * TM * TN * 256 * 4 <= (int)sizeof(sm), "room to reduce");
        float* red = reinterpret_cast<float*>(&sm[0][0][0]);
        __syncthreads();
        if (kh == 1) {
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        red[((slot * TM + i) * TN + j) * 256 + r * 64 + lane] = acc[i][j][r];
        }
        __syncthreads();
        if (kh == 1) return;
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    acc[i][j][r] += red[((slot * TM + i) * TN + j) * 256 + r * 64 + lane];
    }

    if (SPLIT > 1) {
        f32x4* out = reinterpret_cast<f32x4*>(p.part) +
                     (((int64_t)slice * tiles + t) * (WGM * WGN) + slot) * (TM * TN * 64);
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) out[(i * TN + j) * 64 + lane] = acc[i][j];
        return;
    }
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int n = n0 + wn * (BN / WGN) + 16 * j + mn;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = m0 + wm * (BM / WGM) + 16 * i + 4 * kg + r;
                if (m < p.M && n < p.N) p.Y[(int64_t)m * p.y_pitch + n] = to_bf16(acc[i][j][r]);
            }
        }
}

// Sum of the SPLIT fp32 slices of linear_lds_kernel's tiles, in slice order
// (a fixed order), rounded to bf16. One thread per fragment (one lane's four
// accumulators of one 16 x 16 tile): it reads that fragment's 16-byte run in
// every slice and writes the four outputs it holds.
template <int BM, int BN, int WGM, int WGN, int SPLIT>
__global__ __launch_bounds__(256) void linear_split_sum(const LinearParams p) {
    constexpr int TM = BM / WGM / 16, TN = BN / WGN / 16;
    const int mblocks = (p.M + BM - 1) / BM;
    const int64_t tiles = (int64_t)mblocks * ((p.N + BN - 1) / BN);
    const int64_t frags = tiles * (BM * BN / 4);          // fragments in one slice
    const int64_t f = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (f >= frags) return;
    const f32x4* part = reinterpret_cast<const f32x4*>(p.part);
    f32x4 sum = part[f];
#pragma unroll
    for (int k = 1; k < SPLIT; ++k) sum += part[k * frags + f];
    const int lane = (int)(f & 63);
    const int64_t q = f >> 6;                             // (tile, slot, i, j)
    const int ij = (int)(q % (TM * TN));
    const int slot = (int)((q / (TM * TN)) % (WGM * WGN));
    const int t = (int)(q / (TM * TN * WGM * WGN));
    const int i = ij / TN, j = ij % TN;
    const int n = (t / mblocks) * BN + (slot % WGN) * (BN / WGN) + 16 * j + (lane & 15);
    if (n >= p.N) return;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int m = (t % mblocks) * BM + (slot / WGN) * (BM / WGM) + 16 * i + 4 * (lane >> 4) + r;
        if (m < p.M) p.Y[(int64_t)m * p.y_pitch + n] = to_bf16(sum[r]);
    }
}

template <int BM, int BN>
int64_t split_floats(const LinearParams& p, int split) {
    return (int64_t)split * ((p.N + BN - 1) / BN) * ((p.M + BM - 1) / BM) * BM * BN;
}

template <int BM, int BN, int STAGES, int WGM, int WGN, int KS, int SUB = 1, int SPLIT = 1>
hipError_t launch_lds(const LinearParams& p, hipStream_t s) {
    if (p.K % (64 * SUB * SPLIT) != 0) return hipErrorInvalidValue;
    if (SPLIT > 1 && (p.part == nullptr || p.part_floats < split_floats<BM, BN>(p, SPLIT)))
        return hipErrorInvalidValue;
    const int64_t tiles = (int64_t)((p.N + BN - 1) / BN) * ((p.M + BM - 1) / BM);
    hipLaunchKernelGGL((linear_lds_kernel<BM, BN, STAGES, WGM, WGN, KS, SUB, SPLIT>),
                       dim3((unsigned)(tiles * SPLIT)), dim3(64 * WGM * WGN * KS), 0, s, p);
    if (SPLIT > 1) {
        const int64_t frags = tiles * (BM * BN / 4);
        hipLaunchKernelGGL((linear_split_sum<BM, BN, WGM, WGN, SPLIT>), dim3((unsigned)((frags + 255) / 256)),
                           dim3(256), 0, s, p);
    }
    return hipGetLastError();
}

// Pipelined direct-to-LDS kernel with prefetching workgroups, for shapes
// whose 128 x 128 tiles fill three quarters to all but one of the CUs (above
// 256 rows with a K of at least 4096: in_proj at 512 rows makes 200 tiles for
// 256 CUs). It repeats linear_lds_kernel<128, 128, *, 2, 4, 2>'s arithmetic bit
// for bit (same tiles, waves, K halves and summation order) with two changes:
//
// * Software pipelining of the fragments: after the barrier that publishes
//   block kb + 1, each wave reads block kb + 1's fragments and only then issues
//   block kb's MFMAs, on fragments read one step earlier, so the LDS reads that
//   follow every barrier overlap matrix work. The slot of block kb - 1, whose
//   fragments every wave has consumed before reaching that barrier, takes block
//   kb + STAGES - 1. The direct loads use the buffer (MUBUF) form: while a
//   FLAT-encoded global_load_lds is in flight, the compiler's wait-count pass
//   waits for every LDS read before any fragment is used, which undoes the
//   overlap. Byte offsets are 32-bit (the dispatch checks both matrices fit).
// * Prefetching workgroups: those launched past the tiles run on CUs the tiles
//   leave idle and load, K block by K block, a share of the W lines that the
//   tiles of their XCD are about to read (into a private LDS scratch; never
//   waited for until they exit), so that the tiles' own loads find those lines
//   in L2 or the Infinity Cache rather than in HBM. Measured on MI355X at 512
//   rows, the weight stream is what bounds the kernel: with W lines resident in
//   L2 a timing copy takes 46.8 us, with X lines resident instead 66.9 us, as
//   long as with neither (66 us). The prefetching workgroups bring the kernel
//   from 66 to 53-54 us; prefetching the X lines as well (shared by every column
//   block of an XCD, and cheap for the tiles) cost 4 us of that. With many more
//   idle CUs (384 rows: 150 tiles, 106 prefetching workgroups) prefetching ran
//   far ahead of the tiles and evicted lines before use, which was slower:
//   hence the three-quarter rule in the dispatch.

// Share of one XCD's upcoming W lines for a prefetching workgroup (tile t runs
// on XCD t / (tiles / 8) in the XCD-blocked order of the tile kernels).
template <int BN, int THREADS>
__device__ __forceinline__ void prefetch_share(const LinearParams& p, int tiles, int mblocks, uint16_t* lds) {
#if defined(__HIP_DEVICE_COMPILE__)
    const int q = tiles >> 3;
    if (q == 0) return;
    const int x = blockIdx.x & 7;                       // this workgroup's XCD
    const int extra = (int)gridDim.x - tiles;
    const int v0 = ((x - tiles) % 8 + 8) % 8;           // first prefetching workgroup on XCD x
    const int npf = (extra - v0 + 7) / 8;               // prefetching workgroups on XCD x
    const int jpf = ((int)blockIdx.x - tiles) / 8;
    const int n_lo = (x * q / mblocks) * BN;
    const int n_hi = min(p.N, ((x * q + q - 1) / mblocks + 1) * BN);
    const int rows = n_hi - n_lo;                       // the XCD's W rows
    const int nk = p.K / 64;
    const int wv = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    // a thread takes whole rows and walks them in K order, so each wave touches
    // its rows' lines block by block
    for (int r = jpf + npf * (int)threadIdx.x; r < rows; r += npf * THREADS) {
        const uint16_t* rp = p.W + (int64_t)(n_lo + r) * p.K;
        for (int kb = 0; kb < nk; ++kb)   // one 4-byte load a 128-byte line
            __builtin_amdgcn_global_load_lds(rp + kb * 64, lds + wv * 128, 4, 0, 0);
    }
    __builtin_amdgcn_s_waitcnt(0);   // no direct load may still target LDS at exit
#endif
}

template <int BM, int BN, int STAGES, int WGM, int WGN, int KS>
__global__ __launch_bounds__(64 * WGM * WGN * KS) void linear_pipe_kernel(const LinearParams p) {
    static_assert(KS == 1 || KS == 2, "K split of a 64-wide block into 1 or 2 parts");
    static_assert(STAGES >= 3, "a slot being filled, one being read, one consumed");
    constexpr int WAVES = WGM * WGN * KS;
    constexpr int ROWS = BM + BN;
    constexpr int LPB = ROWS / (8 * WAVES);           // direct loads per thread per K block
    constexpr int TM = BM / WGM / 16, TN = BN / WGN / 16;
    constexpr int SPW = 2 / KS;                       // 32-wide K steps a wave takes per block
    static_assert(LPB * 8 * WAVES == ROWS, "rows must split into whole wave loads");
    static_assert((BM / 8) % WAVES == 0, "a wave load lies wholly in X or in W");
    __shared__ __attribute__((aligned(1024))) uint16_t sm[STAGES][ROWS * 64];

    const int mblocks = (p.M + BM - 1) / BM;
    const int tiles = mblocks * ((p.N + BN - 1) / BN);
    if ((int)blockIdx.x >= tiles) {
        prefetch_share<BN, 64 * WAVES>(p, tiles, mblocks, &sm[0][0]);
        return;
    }
    int t = blockIdx.x;
    {
        const int q = tiles >> 3;
        if ((int)blockIdx.x < 8 * q) t = (blockIdx.x & 7) * q + (blockIdx.x >> 3);
    }
    const int m0 = (t % mblocks) * BM;
    const int n0 = (t / mblocks) * BN;
    // the wave index in a scalar register: the direct loads' LDS address (M0)
    // is then provably uniform, with no per-lane loop around each load
    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int kh = wave / (WGM * WGN);
    const int slot = wave % (WGM * WGN);
    const int wm = slot / WGN, wn = slot % WGN;
    const int mn = lane & 15, kg = lane >> 4;

    // byte offset of this lane's 16 bytes of load j of a block (the layout of
    // linear_lds_kernel: row 8 (WAVES j + wave) + (lane >> 3) of [X rows; W rows],
    // chunk (lane & 7) ^ (lane >> 3))
    uint32_t voff[LPB];
#pragma unroll
    for (int j = 0; j < LPB; ++j) {
        const int row = 8 * (WAVES * j + wave) + (lane >> 3);
        const int chunk = (lane & 7) ^ (lane >> 3);
        voff[j] = (uint32_t)(row < BM ? (int64_t)min(m0 + row, p.M - 1) * p.x_pitch
                                      : (int64_t)min(n0 + row - BM, p.N - 1) * p.K) * 2u + 16u * chunk;
    }
    const int nkb = p.K / 64;
#if defined(__HIP_DEVICE_COMPILE__)
    // no range check in the descriptors: every offset is clamped into its matrix
    // (an extent computed here made the compiler treat them as per-lane values)
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc((void*)p.X, (short)0, -1, 0x00020000);
    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc((void*)p.W, (short)0, -1, 0x00020000);
#endif
    auto issue = [&](int kb) {
#if defined(__HIP_DEVICE_COMPILE__)
        const int st = kb % STAGES;
        const uint32_t kk = (uint32_t)min(kb, nkb - 1) * 128u;   // past the end: a harmless re-read
#pragma unroll
        for (int j = 0; j < LPB; ++j)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                (WAVES * j < BM / 8) ? rx : rw,
                (__attribute__((address_space(3))) void*)&sm[st][8 * (WAVES * j + wave) * 64], 16,
                voff[j] + kk, 0, 0, 0);
#endif
    };
    auto read = [&](int kb, bf16x8 (&a)[SPW][TM], bf16x8 (&b)[SPW][TN]) {
        const uint16_t* st = sm[kb % STAGES];
#pragma unroll
        for (int ss = 0; ss < SPW; ++ss) {
            const int s = kh * SPW + ss;
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const int row = wm * (BM / WGM) + 16 * i + mn;
                const int pos = (4 * s + kg) ^ (row & 7);
                a[ss][i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(st + row * 64 + 8 * pos));
            }
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int row = BM + wn * (BN / WGN) + 16 * j + mn;
                const int pos = (4 * s + kg) ^ (row & 7);
                b[ss][j] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(st + row * 64 + 8 * pos));
            }
        }
    };
    f32x4 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    auto mma = [&](const bf16x8 (&a)[SPW][TM], const bf16x8 (&b)[SPW][TN]) {
#pragma unroll
        for (int ss = 0; ss < SPW; ++ss)
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[ss][i], b[ss][j], acc[i][j], 0, 0, 0);
    };
    // vmcnt: block kb + 1 has landed once at most STAGES - 3 later blocks of this
    // wave's loads are outstanding (STAGES - 2 before the loop); lgkmcnt: the
    // fragments of block kb were read one step earlier, so only this step's
    // NR reads may still be in flight
    constexpr int NW = (STAGES - 3) * LPB, N0 = (STAGES - 2) * LPB, NR = SPW * (TM + TN);
    static_assert(N0 < 64 && NR < 16, "the vmcnt field holds 6 bits, lgkmcnt 4");
    auto step = [&](int kb, const bf16x8 (&ca)[SPW][TM], const bf16x8 (&cb)[SPW][TN],
                    bf16x8 (&na)[SPW][TM], bf16x8 (&nb)[SPW][TN]) {
        // unconditional, so that no control-flow join makes the compiler wait
        // for these reads before the MFMAs: in the last step, block kb + 1 is a
        // landed copy of the last block, read and never used
        __builtin_amdgcn_s_waitcnt((NW & 15) | ((NW >> 4) << 14) | (7 << 4) | (15 << 8));
        __asm__ volatile("s_barrier" ::: "memory");
        issue(kb + STAGES - 1);
        read(kb + 1, na, nb);
        __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4) | (NR << 8));
        __builtin_amdgcn_sched_barrier(0);
        mma(ca, cb);
        __builtin_amdgcn_sched_barrier(0);
    };

#pragma unroll
    for (int s = 0; s < STAGES - 1; ++s) issue(s);
    __builtin_amdgcn_s_waitcnt((N0 & 15) | ((N0 >> 4) << 14) | (7 << 4) | (15 << 8));
    __asm__ volatile("s_barrier" ::: "memory");
    bf16x8 a0[SPW][TM], b0[SPW][TN], a1[SPW][TM], b1[SPW][TN];
    read(0, a0, b0);
    // settle the prologue's LDS and scalar loads here, so that the loop header's
    // wait state holds only fragment reads
    __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4) | (0 << 8));
    int kb = 0;
    for (; kb + 2 <= nkb; kb += 2) {
        step(kb, a0, b0, a1, b1);
        step(kb + 1, a1, b1, a0, b0);
    }
    if (kb < nkb) step(kb, a0, b0, a1, b1);
    __builtin_amdgcn_s_waitcnt(0);   // no direct load may still target LDS at exit

    if (KS == 2) {   // group 1 parks its tiles in the (now idle) stages, group 0 adds them
        static_assert(KS == 1 || WGM * WGN * TM * TN * 256 * 4 <= (int)sizeof(sm), "room to reduce");
        float* red = reinterpret_cast<float*>(&sm[0][0]);
        __syncthreads();
        if (kh == 1) {
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        red[((slot * TM + i) * TN + j) * 256 + r * 64 + lane] = acc[i][j][r];
        }
        __syncthreads();
        if (kh == 1) return;
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    acc[i][j][r] += red[((slot * TM + i) * TN + j) * 256 + r * 64 + lane];
    }
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int n = n0 + wn * (BN / WGN) + 16 * j + mn;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = m0 + wm * (BM / WGM) + 16 * i + 4 * kg + r;
                if (m < p.M && n < p.N) p.Y[(int64_t)m * p.y_pitch + n] = to_bf16(acc[i][j][r]);
            }
        }
}

// 128 x 128 tiles of 2 x 4 waves per K half, 4 stages (128 KB of LDS), and as
// many prefetching workgroups as the tiles leave CUs idle.
bool pipe_shape(const LinearParams& p) {
    const int64_t tiles = (int64_t)((p.N + 127) / 128) * ((p.M + 127) / 128);
    return p.M > 256 && p.K >= 4096 && p.K % 64 == 0 && p.cu_count > 0 && tiles < p.cu_count &&
           4 * tiles >= 3 * (int64_t)p.cu_count && (int64_t)p.M * p.x_pitch * 2 <= INT32_MAX &&
           (int64_t)p.N * p.K * 2 <= INT32_MAX;
}

hipError_t launch_pipe(const LinearParams& p, hipStream_t s) {
    // one workgroup a CU: the tiles first, then the prefetching workgroups
    hipLaunchKernelGGL((linear_pipe_kernel<128, 128, 4, 2, 4, 2>), dim3((unsigned)p.cu_count), dim3(1024), 0, s,
                       p);
    return hipGetLastError();
}

template <int MT, int NT, int WAVES>
hipError_t launch_skinny(const LinearParams& p, hipStream_t s) {
    const dim3 grid((unsigned)((p.N + 16 * NT - 1) / (16 * NT)), (unsigned)((p.M + 16 * MT - 1) / (16 * MT)));
    hipLaunchKernelGGL((linear_skinny_kernel<MT, NT, WAVES>), grid, dim3(64 * WAVES), 0, s, p);
    return hipGetLastError();
}

template <int BM, int BN, int DEPTH>
hipError_t launch_tiled(const LinearParams& p, hipStream_t s) {
    const int64_t tiles = (int64_t)((p.N + BN - 1) / BN) * ((p.M + BM - 1) / BM);
    hipLaunchKernelGGL((linear_tiled_kernel<BM, BN, DEPTH>), dim3((unsigned)tiles), dim3(256), 0, s, p);
    return hipGetLastError();
}

// The K split, for 33 to 256 rows with a long K: one tile covers up to 64,
// 128 or 256 rows x 128 columns (X is read once per 128 columns, W once per
// tile) and 4 K slices make ~200 workgroups for the W stream, at the cost of
// the fp32 slices and a second launch. With a short K (o_proj) or beyond 256
// rows that cost outweighs the gain.
constexpr int kSplit = 4;
bool split_shape(int32_t M, int32_t K) {
    return M > 32 && M <= 256 && K >= 4096 && K % (64 * kSplit) == 0;
}

}  // namespace

int64_t linear_workspace_floats(int32_t M, int32_t N, int32_t K) {
    if (M < 1 || N < 1 || !split_shape(M, K)) return 0;
    LinearParams p{};
    p.M = M;
    p.N = N;
    p.K = K;
    if (M <= 64) return split_floats<64, 128>(p, kSplit);
    if (M <= 128) return split_floats<128, 128>(p, kSplit);
    return split_floats<256, 128>(p, kSplit);
}

hipError_t launch_linear(const LinearParams& p, hipStream_t s) {
    // shapes measured on MI355X at the projections' sizes (7168 -> 6284,
    // 1536 -> 7168). With a workspace, 33 to 256 rows and K >= 4096, 4 K
    // slices of 64 x 128 tiles (2 x 2 waves per K half) up to 64 rows,
    // 128 x 128 (2 x 4) up to 128 and 256 x 128 (4 x 2, 3 stages) up to 256.
    // With K a multiple of 128 and up to 64 rows, the
    // direct-to-LDS kernel with two 64-wide K blocks a stage: 16 x 32 tiles
    // (6 stages) up to 16 rows, 32 x 32 up to 32 and 32 x 64 up to 64 (4
    // stages), one wave or wave pair on each 32-wide K half of a block. Above
    // 64 rows (K a multiple of 64): 128 x 64 tiles of 4 x 2 waves with 4 stages
    // up to 256 rows; 128 x 128 tiles of 2 x 4 waves per K half (16 waves) with
    // 3 stages beyond, in the pipelined kernel with 4 stages and prefetching
    // workgroups on the idle CUs when K >= 4096 and those tiles fill three
    // quarters to all but one of the CUs (in_proj at 385 to 512 rows). K a
    // multiple of 64 only: one K block a stage up to 64 rows (the skinny kernel
    // up to 16). Other K: the skinny kernel up to 64 rows and the
    // register-staged kernel above.
    if (split_shape(p.M, p.K) && p.part != nullptr &&
        p.part_floats >= linear_workspace_floats(p.M, p.N, p.K)) {
        if (p.M <= 64) return launch_lds<64, 128, 4, 2, 2, 2, 1, kSplit>(p, s);
        if (p.M <= 128) return launch_lds<128, 128, 3, 2, 4, 2, 1, kSplit>(p, s);
        return launch_lds<256, 128, 3, 4, 2, 2, 1, kSplit>(p, s);
    }
    if (pipe_shape(p)) return launch_pipe(p, s);
    if (p.K % 128 == 0 && p.M <= 64) {
        if (p.M <= 16) return launch_lds<16, 32, 6, 1, 1, 2, 2>(p, s);
        if (p.M <= 32) return launch_lds<32, 32, 4, 1, 1, 2, 2>(p, s);
        return launch_lds<32, 64, 4, 1, 2, 2, 2>(p, s);
    }
    if (p.K % 64 == 0) {
        if (p.M <= 16) return launch_skinny<1, 2, 8>(p, s);
        if (p.M <= 32) return launch_lds<32, 32, 8, 1, 1, 2>(p, s);
        if (p.M <= 64) return launch_lds<32, 64, 6, 1, 2, 2>(p, s);
        if (p.M <= 256) return launch_lds<128, 64, 4, 4, 2, 1>(p, s);
        return launch_lds<128, 128, 3, 2, 4, 2>(p, s);
    }
    if (p.M <= 16) return launch_skinny<1, 2, 8>(p, s);
    if (p.M <= 32) return launch_skinny<2, 2, 8>(p, s);
    if (p.M <= 64) return launch_skinny<4, 2, 8>(p, s);
    return launch_tiled<128, 64, 2>(p, s);
}

int32_t current_device_cus() {
    static std::atomic<int32_t> cus[64] = {};   // per device, 0 until first read
    int d = -1;
    if (hipGetDevice(&d) != hipSuccess || d < 0 || d >= 64) return 0;
    int32_t n = cus[d].load(std::memory_order_relaxed);
    if (n == 0) {
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, d) != hipSuccess) return 0;
        n = v;
        cus[d].store(n, std::memory_order_relaxed);
    }
    return n;
}

}  // namespace kda
