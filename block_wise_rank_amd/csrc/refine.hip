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
    const int64_t base = row0 ? row0[blk] : static_cast<int64_t>(blk) * T * row_stride;
    // bf16 X streams through a ring of four 32-token tiles in LDS (the V
    // area, free once the fragments are built).  Each wave loads a quarter of
    // a tile (rows 8 w .. 8 w + 7, two 16-byte loads per lane) four tiles
    // ahead, so that the workgroup keeps four distinct tiles in flight
    // instead of every wave loading every tile.  Rows are padded to 272
    // bytes: the 16-byte fragment reads of 32 consecutive rows fall on
    // distinct banks.
    constexpr int kRowB = kD * 2 + 16;
    constexpr int kSlot = 32 * kRowB;
    static_assert(4 * kSlot <= kD * kD * 4, "the ring fits in the V area");
    uint8_t *ring = reinterpret_cast<uint8_t *>(Vs);
    const int n_tiles = T / 32;
    const uint8_t *xg = static_cast<const uint8_t *>(x) + base * 2;
    const int lr = 8 * wave + (lane >> 4);  // rows lr and lr + 4 of a tile
    const uint8_t *xl = xg + static_cast<int64_t>(lr) * row_stride * 2 + 16 * (lane & 15);
    const int64_t x4 = static_cast<int64_t>(4) * row_stride * 2, x32 = static_cast<int64_t>(32) * row_stride * 2;
    auto load_q = [&](uint4 &ra, uint4 &rb, int tile) __attribute__((always_inline)) {
        const int tt = tile < n_tiles ? tile : n_tiles - 1;  // past the end: the last tile again
        const uint8_t *p0 = xl + tt * x32;
        ra = *reinterpret_cast<const uint4 *>(p0);
        rb = *reinterpret_cast<const uint4 *>(p0 + x4);
    };
    auto store_q = [&](const uint4 &ra, const uint4 &rb, int tile) __attribute__((always_inline)) {
        uint8_t *p0 = ring + (tile & 3) * kSlot + lr * kRowB + 16 * (lane & 15);
        *reinterpret_cast<uint4 *>(p0) = ra;
        *reinterpret_cast<uint4 *>(p0 + 4 * kRowB) = rb;
    };
    // tile k waits in (qka, qkb), k = tile % 4, until it is stored, one tile before its use
    uint4 q0a, q0b, q1a, q1b, q2a, q2b, q3a, q3b;
    constexpr int NV = kD * kD / 4 / 256;  // float4 of V per thread
    float4 vr[NV];
#pragma unroll
    for (int k = 0; k < NV; ++k) vr[k] = reinterpret_cast<const float4 *>(vblk)[tid + 256 * k];
    // the first five X tiles are in flight while V is prepared
    uint4 ra, rb;
    if constexpr (NX == 1) {
        load_q(ra, rb, 0);
        load_q(q1a, q1b, 1);
        load_q(q2a, q2b, 2);
        load_q(q3a, q3b, 3);
        load_q(q0a, q0b, 4);
    }
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

    float acc2[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) acc2[r] = 0.f;

    if constexpr (NX == 1) {
        __syncthreads();  // every wave has read V: its LDS is free
        store_q(ra, rb, 0);
        __syncthreads();
        auto step = [&](uint4 &na, uint4 &nb, int t) __attribute__((always_inline)) {
            // B fragments of tile t: token lane % 32, features 16 ks + 8 (lane / 32) ..
            const uint8_t *src = ring + (t & 3) * kSlot + (lane & 31) * kRowB + 16 * (lane >> 5);
            u16x8_t cur[8];
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) cur[ks] = *reinterpret_cast<const u16x8_t *>(src + 32 * ks);
            f32x16_t acc = zero16(), acc1 = zero16();
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) {
                // two independent accumulation chains (even / odd k-steps)
                f32x16_t &a = (ks & 1) ? acc1 : acc;
                a = mfma32x32x16(fa[0][ks], cur[ks], a);
                a = mfma32x32x16(fa[1][ks], cur[ks], a);
            }
            store_q(na, nb, t + 1);  // its slot was last read in tile t - 3
            load_q(na, nb, t + 5);
            acc += acc1;
#pragma unroll
            for (int r = 0; r < 16; ++r) acc2[r] += acc[r] * acc[r];
            __syncthreads();
        };
        int t = 0;
        for (; t + 4 <= n_tiles; t += 4) {
            step(q1a, q1b, t);
            step(q2a, q2b, t + 1);
            step(q3a, q3b, t + 2);
            step(q0a, q0b, t + 3);
        }
        if (t < n_tiles) {  // block_len % 64 == 0: an even number of tiles, so two remain
            step(q1a, q1b, t);
            step(q2a, q2b, t + 1);
        }
    } else {
        for (int t0 = 0; t0 < T; t0 += 32) {
            const int t = t0 + (lane & 31);
            f32x16_t acc = zero16();
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) {
                const int j0 = 16 * ks + 8 * (lane >> 5);
                const float *xr = static_cast<const float *>(x) + base + static_cast<int64_t>(t) * row_stride + j0;
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
#pragma unroll
            for (int r = 0; r < 16; ++r) acc2[r] += acc[r] * acc[r];
        }
    }
    // V again (the X ring overwrote its LDS copy): DMA'd from memory into the V
    // area, 1 KiB per wave instruction, while the sums are reduced and sorted
    // (every wave's last ring read is behind the loop's final barrier)
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        const int m = 16 * wave + k;
        __builtin_amdgcn_global_load_lds(
            (const __attribute__((address_space(1))) void *)(reinterpret_cast<const uint8_t *>(vblk) + 1024 * m + 16 * lane),
            (__attribute__((address_space(3))) void *)(reinterpret_cast<uint8_t *>(Vs) + 1024 * m), 16, 0, 0);
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
    // sorted, signed, unit-norm rows (the DMA of V has landed before the barrier)
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();
#pragma unroll
    for (int k = 0; k < NV; ++k) {
        const int e4 = tid + 256 * k, pos = e4 >> 5, j = 4 * (e4 & 31);
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
