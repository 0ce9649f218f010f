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
// Both operands are K-contiguous (rows of X, rows of the nn.Linear weight W),
// so every lane reads 64 contiguous bytes of one row per 128-wide K block and
// feeds v_mfma_f32_16x16x32_bf16 directly from registers. Within a K block,
// lane group kg (= lane >> 4) owns K elements 32kg .. 32kg + 31 and hands
// 8 of them to each of the 4 MFMA K steps; A and B use the same assignment,
// so the product is unchanged.
//
// A workgroup computes 16 output columns for 16 * MT rows; its 4 waves take
// the K blocks round-robin and their partial tiles are summed through LDS in
// wave order (a fixed order: results do not depend on timing).
#include "kda_internal.h"

namespace kda {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kLinWaves = 4;
constexpr int kLinThreads = 64 * kLinWaves;
constexpr int kKBlock = 128;

__device__ __forceinline__ bf16x8 load8(const uint16_t* p, bool ok) {
    const u32x4 z = {0u, 0u, 0u, 0u};
    return __builtin_bit_cast(bf16x8, ok ? *reinterpret_cast<const u32x4*>(p) : z);
}

__device__ __forceinline__ uint16_t to_bf16(float f) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

template <int MT>
__global__ __launch_bounds__(kLinThreads) void linear_skinny_kernel(const LinearParams p) {
    const int n0 = blockIdx.x * 16;
    const int m0 = blockIdx.y * (16 * MT);
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int mn = lane & 15;   // B column (output n) / A row (token m) of this lane
    const int kg = lane >> 4;   // which 32-wide slice of each K block

    // out-of-range rows read a valid row and are zeroed
    const int n = n0 + mn;
    const bool n_ok = n < p.N;
    const uint16_t* wrow = p.W + (int64_t)(n_ok ? n : p.N - 1) * p.K;
    const uint16_t* xrow[MT];
    bool m_ok[MT];
#pragma unroll
    for (int i = 0; i < MT; ++i) {
        const int m = m0 + 16 * i + mn;
        m_ok[i] = m < p.M;
        xrow[i] = p.X + (int64_t)(m_ok[i] ? m : p.M - 1) * p.x_pitch;
    }

    f32x4 acc[MT];
#pragma unroll
    for (int i = 0; i < MT; ++i) acc[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    const int nkb = (p.K + kKBlock - 1) / kKBlock;
    for (int kb = wave; kb < nkb; kb += kLinWaves) {
        const int kbase = kb * kKBlock + 32 * kg;
        bf16x8 b[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) b[j] = load8(wrow + kbase + 8 * j, n_ok && kbase + 8 * j + 8 <= p.K);
#pragma unroll
        for (int i = 0; i < MT; ++i) {
            bf16x8 a[4];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                a[j] = load8(xrow[i] + kbase + 8 * j, m_ok[i] && kbase + 8 * j + 8 <= p.K);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[j], b[j], acc[i], 0, 0, 0);
        }
    }

    // sum the 4 waves' partial tiles in wave order; lane holds rows 4 kg + r
    // (r = 0..3) of each 16-row tile, column mn
    __shared__ float red[kLinWaves][MT * 4][64];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) red[wave][i * 4 + r][lane] = acc[i][r];
    __syncthreads();
    for (int e = threadIdx.x; e < MT * 4 * 64; e += kLinThreads) {
        const int ir = e >> 6, l = e & 63;
        float s = red[0][ir][l];
#pragma unroll
        for (int w = 1; w < kLinWaves; ++w) s += red[w][ir][l];
        const int m = m0 + 16 * (ir >> 2) + 4 * (l >> 4) + (ir & 3);
        const int nn = n0 + (l & 15);
        if (m < p.M && nn < p.N) p.Y[(int64_t)m * p.y_pitch + nn] = to_bf16(s);
    }
}

template <int MT>
hipError_t launch_t(const LinearParams& p, hipStream_t s) {
    const dim3 grid((unsigned)((p.N + 15) / 16), (unsigned)((p.M + 16 * MT - 1) / (16 * MT)));
    hipLaunchKernelGGL(linear_skinny_kernel<MT>, grid, dim3(kLinThreads), 0, s, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_linear(const LinearParams& p, hipStream_t s) {
    if (p.M <= 16) return launch_t<1>(p, s);
    if (p.M <= 32) return launch_t<2>(p, s);
    return launch_t<4>(p, s);
}

}  // namespace kda
