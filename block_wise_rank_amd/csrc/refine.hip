// Singular values as sigma_i = ||X_b v_i||, then the eigenvectors sorted by
// descending sigma with a sign convention (largest-magnitude entry positive).
//
// The eigenvalues of an fp32 Gram are only accurate to about u * ||G||, which
// is too coarse for the small singular values (sigma^2 ~ 1e-5 next to
// sigma_0^2 ~ 1).  The norm ||X v_i|| is a Rayleigh quotient: its error is
// second order in the eigenvector error, so recomputing it directly from X
// gives singular values accurate to a few fp32 ulps of sigma_0.
//
// Y^T = V^T X^T runs on bf16 MFMA with fp32 accumulation.  For fp32 X both
// operands are split exactly into three bf16 terms, keeping the products whose
// term orders sum to <= 2.  For bf16 X (exact as it stands) V is split into two
// terms, which leaves a perturbation delta of V with |delta| <= 2^-17 |v|; its
// effect on ||X v|| is first order only through v . delta (relative 2^-17) and
// otherwise second order (||X delta||^2 / 2 sigma <= sigma_0^2 2^-35 / sigma),
// far inside the singular values' tolerance.  One workgroup (4 waves) per block;
// wave w owns eigenvectors 32w .. 32w + 31 and keeps their fragments in
// registers while it streams every 32-token tile of X straight from memory
// (8 consecutive features per lane = one 16-byte load for bf16).
#include "common.hpp"
#include "kernels.hpp"

namespace milo {
namespace {

template <int NX>
__global__ __launch_bounds__(256) void refine_kernel(const void *__restrict__ x,
                                                     const int64_t *__restrict__ row0,
                                                     int64_t row_stride, int T,
                                                     float *__restrict__ vt,
                                                     float *__restrict__ sigma) {
    __shared__ __align__(16) float Vs[kD * kD];  // 64 KiB, row i = eigenvector i
    __shared__ float ss[kD];       // sum of squares per eigenvector
    __shared__ float sig[kD];
    __shared__ int perm[kD];
    __shared__ float sgn[kD];
    __shared__ float ninv[kD];     // 1 / ||v_i||

    const int blk = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    float *vblk = vt + static_cast<int64_t>(blk) * kD * kD;
    constexpr int NV = kD * kD / 4 / 256;  // float4 of V per thread
    float4 vr[NV];
#pragma unroll
    for (int k = 0; k < NV; ++k) vr[k] = reinterpret_cast<const float4 *>(vblk)[tid + 256 * k];
#pragma unroll
    for (int k = 0; k < NV; ++k) reinterpret_cast<float4 *>(Vs)[tid + 256 * k] = vr[k];
    __syncthreads();

    // A fragments: row i = 32 * wave + lane % 32, k slots j = 16 ks + 8 (lane / 32) + e.
    // Thousands of fp32 rotations leave each eigenvector's norm off by ~1e-5: the
    // fragments are built from v_i / ||v_i|| (so that ||X v|| measures sigma and
    // B = V_r^T is orthonormal), and the same pass finds the row's sign: its
    // largest-magnitude entry (first one on ties) is made positive.
    constexpr int NT = NX == 1 ? 2 : 3;  // terms of V
    u16x8_t fa[NT][8];
    {
        const int i = 32 * wave + (lane & 31), h = lane >> 5;
        float v[8][8];
        float ssq = 0.f;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            const float4 p0 = *reinterpret_cast<const float4 *>(Vs + i * kD + 16 * ks + 8 * h);
            const float4 p1 = *reinterpret_cast<const float4 *>(Vs + i * kD + 16 * ks + 8 * h + 4);
            v[ks][0] = p0.x; v[ks][1] = p0.y; v[ks][2] = p0.z; v[ks][3] = p0.w;
            v[ks][4] = p1.x; v[ks][5] = p1.y; v[ks][6] = p1.z; v[ks][7] = p1.w;
#pragma unroll
            for (int e = 0; e < 8; ++e) ssq = fmaf(v[ks][e], v[ks][e], ssq);
        }
        ssq += __shfl_xor(ssq, 32, 64);
        const float nrm = sqrtf(ssq);
        const float inv = nrm > 0.f ? 1.f / nrm : 0.f;
        float best = -1.f, bval = 0.f;
        int bidx = 0;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float a = v[ks][e] * inv;
                if (fabsf(a) > best) {  // indices increase along the lane's slots
                    best = fabsf(a);
                    bidx = 16 * ks + 8 * h + e;
                    bval = a;
                }
                uint16_t hi, mi, lo;
                split3_bf16(a, hi, mi, lo);
                fa[0][ks][e] = hi;
                fa[1][ks][e] = mi;
                if constexpr (NT == 3) fa[NT - 1][ks][e] = lo;
            }
        const float ob = __shfl_xor(best, 32, 64), ov = __shfl_xor(bval, 32, 64);
        const int oi = __shfl_xor(bidx, 32, 64);
        if (ob > best || (ob == best && oi < bidx)) bval = ov;
        if (h == 0) {
            ninv[i] = inv;
            sgn[i] = (bval < 0.f) ? -1.f : 1.f;
        }
    }

    const int64_t base = row0 ? row0[blk] : static_cast<int64_t>(blk) * T * row_stride;
    float acc2[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) acc2[r] = 0.f;

    // bf16 X: the next 32-token tile's fragments are loaded while this tile's
    // products run (one tile of latency cover).
    u16x8_t xb[NX == 1 ? 8 : 1];
    auto load_x = [&](int t0) {
        if constexpr (NX == 1) {
            const uint16_t *xr = static_cast<const uint16_t *>(x) + base +
                                 static_cast<int64_t>(t0 + (lane & 31)) * row_stride + 8 * (lane >> 5);
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) xb[ks] = *reinterpret_cast<const u16x8_t *>(xr + 16 * ks);
        }
    };
    load_x(0);
    for (int t0 = 0; t0 < T; t0 += 32) {
        const int t = t0 + (lane & 31);
        f32x16_t acc = zero16(), acc1 = zero16();
        u16x8_t cur[NX == 1 ? 8 : 1];
        if constexpr (NX == 1) {
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) cur[ks] = xb[ks];
            load_x(t0 + 32 < T ? t0 + 32 : t0);  // the last tile reloads itself (unused)
            // keep the scheduler from sinking those loads back between the products
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            const int j0 = 16 * ks + 8 * (lane >> 5);
            if constexpr (NX == 1) {
                // two independent accumulation chains (even / odd k-steps)
                f32x16_t &a = (ks & 1) ? acc1 : acc;
                a = mfma32x32x16(fa[0][ks], cur[ks], a);
                a = mfma32x32x16(fa[1][ks], cur[ks], a);
            } else {
                const float *xr = static_cast<const float *>(x) + base +
                                  static_cast<int64_t>(t) * row_stride + j0;
                const float4 v0 = reinterpret_cast<const float4 *>(xr)[0];
                const float4 v1 = reinterpret_cast<const float4 *>(xr)[1];
                const float f[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
                u16x8_t fb[3];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    uint16_t h, m, l;
                    split3_bf16(f[e], h, m, l);
                    fb[0][e] = h;
                    fb[1][e] = m;
                    fb[2][e] = l;
                }
#pragma unroll
                for (int sa = 0; sa < 3; ++sa)
#pragma unroll
                    for (int sb = 0; sb < 3; ++sb)
                        if (sa + sb <= 2) acc = mfma32x32x16(fa[sa < NT ? sa : 0][ks], fb[sb], acc);
            }
        }
        if constexpr (NX == 1) acc += acc1;
#pragma unroll
        for (int r = 0; r < 16; ++r) acc2[r] += acc[r] * acc[r];
    }
    // acc2[r] belongs to row i = 32 wave + 8 (r / 4) + 4 (lane / 32) + r % 4, token lane % 32.
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const float tot = half_sum(acc2[r]);
        if ((lane & 31) == 0) ss[32 * wave + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3)] = tot;
    }
    __syncthreads();

    // Sort descending (rank by counting; ties keep index order) and fix signs.
    if (tid < kD) sig[tid] = sqrtf(ss[tid]);
    __syncthreads();
    if (tid < kD) {
        const float si = sig[tid];
        int pos = 0;
        for (int j = 0; j < kD; ++j) {
            const float sj = sig[j];
            pos += (sj > si) || (sj == si && j < tid);
        }
        perm[pos] = tid;
        ss[pos] = si;  // sorted values (ss is free again)
    }
    __syncthreads();
    if (tid < kD) sigma[static_cast<int64_t>(blk) * kD + tid] = ss[tid];
    for (int e4 = tid; e4 < kD * kD / 4; e4 += 256) {
        const int pos = e4 >> 5, j = 4 * (e4 & 31);
        const int src = perm[pos];
        const float g = sgn[src], iv = ninv[src];
        const float4 a = *reinterpret_cast<const float4 *>(Vs + src * kD + j);
        reinterpret_cast<float4 *>(vblk)[e4] = make_float4(g * (a.x * iv), g * (a.y * iv), g * (a.z * iv), g * (a.w * iv));
    }
}

}  // namespace

hipError_t launch_refine(const void *x, int x_type, const int64_t *row0, int64_t row_stride,
                         int block_len, int n_blocks, float *vt, float *sigma, hipStream_t st) {
    if (n_blocks <= 0) return hipSuccess;
    if (x_type == kBF16)
        hipLaunchKernelGGL(refine_kernel<1>, dim3(static_cast<unsigned>(n_blocks)), dim3(256), 0,
                           st, x, row0, row_stride, block_len, vt, sigma);
    else
        hipLaunchKernelGGL(refine_kernel<3>, dim3(static_cast<unsigned>(n_blocks)), dim3(256), 0,
                           st, x, row0, row_stride, block_len, vt, sigma);
    return hipGetLastError();
}

}  // namespace milo
