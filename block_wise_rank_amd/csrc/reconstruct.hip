// Rebuild X_hat_b = A_b B_b for a list of blocks (decoded factors, fp32
// arithmetic).  Only the listed blocks are rebuilt (evolve.pub review of arXiv
// 2609.29913, FAQ).  Grid: (listed block, 64-token tile); the decoded B_b
// (r x 128) and the decoded 64-token slice of A_b^T (r x 64) are staged in LDS
// and each thread accumulates 32 tokens of one feature column.
#include "common.hpp"
#include "kernels.hpp"

namespace milo {
namespace {

template <int F>
__device__ __forceinline__ float load_code(const uint8_t *p, int64_t idx) {
    if constexpr (F == kF32) return reinterpret_cast<const float *>(p)[idx];
    else if constexpr (F == kBF16) return bf16_bits_to_f32(reinterpret_cast<const uint16_t *>(p)[idx]);
    else return static_cast<float>(reinterpret_cast<const int8_t *>(p)[idx]);
}

template <int F, int OUT>
__global__ __launch_bounds__(256) void reconstruct_kernel(
    const uint8_t *__restrict__ arena, const int32_t *__restrict__ rank,
    const int64_t *__restrict__ a_off, const int64_t *__restrict__ b_off,
    const float *__restrict__ a_scale, const float *__restrict__ b_scale, int T,
    const int32_t *__restrict__ ids, void *__restrict__ out) {
    __shared__ __align__(16) float Bs[kD * kD];
    __shared__ float As[kD * 64];
    const int n = blockIdx.x;
    const int id = ids[n];
    const int t0 = blockIdx.y * 64;
    const int tid = threadIdx.x;
    const int r = rank[id];
    const uint8_t *Ab = arena + a_off[id];
    const uint8_t *Bb = arena + b_off[id];
    for (int e = tid; e < r * kD; e += 256) {
        float v = load_code<F>(Bb, e);
        if constexpr (F == kI8) v *= b_scale[static_cast<int64_t>(id) * kD + e / kD];
        Bs[e] = v;
    }
    for (int e = tid; e < r * 64; e += 256) {
        const int i = e >> 6, tt = e & 63;
        float v = load_code<F>(Ab, static_cast<int64_t>(i) * T + t0 + tt);
        if constexpr (F == kI8) v *= a_scale[static_cast<int64_t>(id) * T + t0 + tt];
        As[e] = v;
    }
    __syncthreads();
    const int j = tid & 127, half = tid >> 7;
    float acc[32];
#pragma unroll
    for (int u = 0; u < 32; ++u) acc[u] = 0.f;
    for (int i = 0; i < r; ++i) {
        const float b = Bs[i * kD + j];
        const float *a = As + i * 64 + half * 32;
#pragma unroll
        for (int u = 0; u < 32; ++u) acc[u] = fmaf(a[u], b, acc[u]);
    }
    const int64_t row = static_cast<int64_t>(n) * T + t0 + half * 32;
#pragma unroll
    for (int u = 0; u < 32; ++u) {
        if constexpr (OUT == kF32)
            static_cast<float *>(out)[(row + u) * kD + j] = acc[u];
        else
            static_cast<uint16_t *>(out)[(row + u) * kD + j] = f32_to_bf16_bits(acc[u]);
    }
}

}  // namespace

hipError_t launch_reconstruct(const void *arena, int f_type, const int32_t *rank,
                              const int64_t *a_off, const int64_t *b_off, const float *a_scale,
                              const float *b_scale, int block_len, const int32_t *ids, int n_ids,
                              void *out, int out_type, hipStream_t st) {
    if (n_ids <= 0) return hipSuccess;
    const dim3 grid(static_cast<unsigned>(n_ids), static_cast<unsigned>(block_len / 64));
    const uint8_t *ar = static_cast<const uint8_t *>(arena);
#define MILO_RECON(F, O)                                                                         \
    hipLaunchKernelGGL((reconstruct_kernel<F, O>), grid, dim3(256), 0, st, ar, rank, a_off,      \
                       b_off, a_scale, b_scale, block_len, ids, out)
    if (f_type == kF32) {
        if (out_type == kF32) MILO_RECON(kF32, kF32); else MILO_RECON(kF32, kBF16);
    } else if (f_type == kBF16) {
        if (out_type == kF32) MILO_RECON(kBF16, kF32); else MILO_RECON(kBF16, kBF16);
    } else {
        if (out_type == kF32) MILO_RECON(kI8, kF32); else MILO_RECON(kI8, kBF16);
    }
#undef MILO_RECON
    return hipGetLastError();
}

}  // namespace milo
