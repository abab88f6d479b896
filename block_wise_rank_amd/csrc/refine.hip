// Singular values as sigma_i = ||X_b v_i||, sorted descending, with the order
// and a per-row scale (sign and 1/||v_i||) written for the projection.
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
// wave w owns eigenvectors 32w .. 32w + 31 and builds their fragments straight
// from memory, keeping them in registers for the whole block.
//
// The eigenvectors are not rewritten: the projection reads row perm[i] of the
// eigensolver's output for sorted rank i and multiplies it by scale[i] = sign /
// ||v||, the same value the sorted row would have held.
//
// bf16 X streams through an 8-slot ring of 32-token tiles in LDS, filled by LDS
// DMA (global_load_lds, 16 bytes per lane, no registers) seven tiles ahead of
// use, so that a workgroup keeps 56 KiB of loads in flight: at the latency of a
// loaded HBM that is what streaming at full bandwidth needs with two
// workgroups per CU.  A tile is 32 unpadded 256-byte rows; a row's 16-byte
// chunk c sits at chunk c ^ (row % 16), so the fragment reads of 16 consecutive
// rows cover every bank.  The DMA lane that writes physical chunk p of row r
// loads logical chunk p ^ (r % 16).
#include "common.hpp"
#include "kernels.hpp"

namespace milo {
namespace {

constexpr int kRing = 8;                 // tiles in the ring
constexpr int kAhead = kRing - 1;        // tiles loaded ahead of use
constexpr int kTileB = 32 * kD * 2;      // bytes of one bf16 tile
constexpr int kDmaPerWave = kTileB / 1024 / 4;  // 1 KiB DMA instructions per wave and tile

// s_waitcnt immediate: at most n vector memory operations outstanding.
constexpr int vmcnt_imm(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }

// 32-bit LDS address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) void *)p));
}

// Eight 16-byte LDS reads at addr[k] + off, waited for inside the same asm block.
__device__ __forceinline__ void read8_lds(u16x8_t (&out)[8], const uint32_t (&addr)[8], uint32_t off) {
    typedef int v4i __attribute__((ext_vector_type(4)));
    v4i r0, r1, r2, r3, r4, r5, r6, r7;
    asm volatile(
        "ds_read_b128 %0, %8\n\t"
        "ds_read_b128 %1, %9\n\t"
        "ds_read_b128 %2, %10\n\t"
        "ds_read_b128 %3, %11\n\t"
        "ds_read_b128 %4, %12\n\t"
        "ds_read_b128 %5, %13\n\t"
        "ds_read_b128 %6, %14\n\t"
        "ds_read_b128 %7, %15\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3), "=&v"(r4), "=&v"(r5), "=&v"(r6), "=&v"(r7)
        : "v"(addr[0] + off), "v"(addr[1] + off), "v"(addr[2] + off), "v"(addr[3] + off),
          "v"(addr[4] + off), "v"(addr[5] + off), "v"(addr[6] + off), "v"(addr[7] + off)
        : "memory");
    out[0] = __builtin_bit_cast(u16x8_t, r0);
    out[1] = __builtin_bit_cast(u16x8_t, r1);
    out[2] = __builtin_bit_cast(u16x8_t, r2);
    out[3] = __builtin_bit_cast(u16x8_t, r3);
    out[4] = __builtin_bit_cast(u16x8_t, r4);
    out[5] = __builtin_bit_cast(u16x8_t, r5);
    out[6] = __builtin_bit_cast(u16x8_t, r6);
    out[7] = __builtin_bit_cast(u16x8_t, r7);
}

template <int NX>
__global__ __launch_bounds__(256) void refine_kernel(const void *__restrict__ x,
                                                     const int64_t *__restrict__ row0,
                                                     int64_t row_stride, int T,
                                                     const float *__restrict__ vt,
                                                     float *__restrict__ sigma,
                                                     int32_t *__restrict__ perm_out,
                                                     float *__restrict__ scale_out) {
    __shared__ __align__(16) uint8_t ring[NX == 1 ? kRing * kTileB : 16];
    __shared__ float ss[kD];       // sum of squares per eigenvector
    __shared__ float sig[kD];
    __shared__ float scl[kD];      // sign / ||v_i|| by original index

    const int blk = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const float *vblk = vt + static_cast<int64_t>(blk) * kD * kD;
    const int64_t base = row0 ? row0[blk] : static_cast<int64_t>(blk) * T * row_stride;
    const int n_tiles = T / 32;

    // A fragments: row i = 32 * wave + lane % 32, k slots j = 16 ks + 8 (lane / 32) + e,
    // loaded before the first tiles' DMA so that they arrive first.
    const int i = 32 * wave + (lane & 31), h = lane >> 5;
    float v[8][8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
        const float4 p0 = *reinterpret_cast<const float4 *>(vblk + i * kD + 16 * ks + 8 * h);
        const float4 p1 = *reinterpret_cast<const float4 *>(vblk + i * kD + 16 * ks + 8 * h + 4);
        v[ks][0] = p0.x; v[ks][1] = p0.y; v[ks][2] = p0.z; v[ks][3] = p0.w;
        v[ks][4] = p1.x; v[ks][5] = p1.y; v[ks][6] = p1.z; v[ks][7] = p1.w;
    }

    // DMA of tile tau (clamped to the last tile) into slot tau % kRing: wave w
    // writes rows 8 w .. 8 w + 7 (two 1 KiB instructions of four rows each).
    const uint8_t *xg = static_cast<const uint8_t *>(x) + base * 2;
    const int dr = lane >> 4, dp = lane & 15;  // row within an instruction, physical chunk
    auto dma = [&](int tau) __attribute__((always_inline)) {
        if constexpr (NX == 1) {
            const int tt = tau < n_tiles ? tau : n_tiles - 1;
#pragma unroll
            for (int k = 0; k < kDmaPerWave; ++k) {
                const int j = kDmaPerWave * wave + k;       // instruction: rows 4 j .. 4 j + 3
                const int r = 4 * j + dr;
                const uint8_t *src = xg + (static_cast<int64_t>(32 * tt + r) * row_stride) * 2 + 16 * (dp ^ (r & 15));
                __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)src,
                                                 (__attribute__((address_space(3))) void *)(ring + (tau % kRing) * kTileB + 1024 * j),
                                                 16, 0, 0);
            }
        }
    };
    if constexpr (NX == 1) {
#pragma unroll
        for (int tau = 0; tau < kAhead; ++tau) dma(tau);
        // every prologue DMA is issued before the fragment build waits for V
        __builtin_amdgcn_sched_barrier(0);
    }

    // Thousands of fp32 rotations leave each eigenvector's norm off by ~1e-5: the
    // fragments are built from v_i / ||v_i|| (so that ||X v|| measures sigma and
    // B = V_r^T is orthonormal), and the same pass finds the row's sign: its
    // largest-magnitude entry (first one on ties) is made positive.
    constexpr int NT = NX == 1 ? 2 : 3;  // terms of V
    u16x8_t fa[NT][8];
    {
        float ssq = 0.f;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks)
#pragma unroll
            for (int e = 0; e < 8; ++e) ssq = fmaf(v[ks][e], v[ks][e], ssq);
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
        if (h == 0) scl[i] = (bval < 0.f) ? -inv : inv;
    }

    float acc2[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) acc2[r] = 0.f;

    if constexpr (NX == 1) {
        // B fragments of a tile: token n = lane % 32, logical chunk 2 ks + h of its row
        const int n = lane & 31;
        uint32_t roff[8];  // LDS byte addresses in slot 0
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) roff[ks] = lds_addr(ring) + n * (kD * 2) + 16 * ((2 * ks + h) ^ (n & 15));
        for (int t = 0; t < n_tiles; ++t) {
            // this wave's part of tile t has landed (each later tile added
            // kDmaPerWave operations); the barrier makes every part visible and
            // frees slot (t - 1) % kRing for the tile kAhead ahead
            __builtin_amdgcn_s_waitcnt(vmcnt_imm((kAhead - 1) * kDmaPerWave));
            __syncthreads();
            dma(t + kAhead);
            // The tile's fragments, read in one asm block that also waits for
            // them: the compiler then sees no LDS read that the DMAs in flight
            // might write (it would wait for all of them), and no result is
            // used before it has arrived.
            const uint32_t so = (t % kRing) * kTileB;
            u16x8_t cur[8];
            read8_lds(cur, roff, so);
            f32x16_t acc = zero16(), acc1 = zero16();
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) {
                // two independent accumulation chains (even / odd k-steps)
                f32x16_t &a = (ks & 1) ? acc1 : acc;
                a = mfma32x32x16(fa[0][ks], cur[ks], a);
                a = mfma32x32x16(fa[1][ks], cur[ks], a);
            }
            acc += acc1;
#pragma unroll
            for (int r = 0; r < 16; ++r) acc2[r] += acc[r] * acc[r];
        }
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // the trailing (discarded) tiles have landed
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
                    uint16_t hh, m, l;
                    split3_bf16(f[e], hh, m, l);
                    fb[0][e] = hh;
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
    // acc2[r] belongs to row i = 32 wave + 8 (r / 4) + 4 (lane / 32) + r % 4, token lane % 32.
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const float tot = half_sum(acc2[r]);
        if ((lane & 31) == 0) ss[32 * wave + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3)] = tot;
    }
    __syncthreads();

    // Sort descending (rank by counting; ties keep index order).
    if (tid < kD) sig[tid] = sqrtf(ss[tid]);
    __syncthreads();
    if (tid < kD) {
        const float si = sig[tid];
        int pos = 0;
        for (int j = 0; j < kD; ++j) {
            const float sj = sig[j];
            pos += (sj > si) || (sj == si && j < tid);
        }
        const int64_t o = static_cast<int64_t>(blk) * kD + pos;
        sigma[o] = si;
        perm_out[o] = tid;
        scale_out[o] = scl[tid];
    }
}

}  // namespace

hipError_t launch_refine(const void *x, int x_type, const int64_t *row0, int64_t row_stride,
                         int block_len, int n_blocks, const float *vt, float *sigma, int32_t *perm,
                         float *scale, hipStream_t st) {
    if (n_blocks <= 0) return hipSuccess;
    if (x_type == kBF16)
        hipLaunchKernelGGL(refine_kernel<1>, dim3(static_cast<unsigned>(n_blocks)), dim3(256), 0,
                           st, x, row0, row_stride, block_len, vt, sigma, perm, scale);
    else
        hipLaunchKernelGGL(refine_kernel<3>, dim3(static_cast<unsigned>(n_blocks)), dim3(256), 0,
                           st, x, row0, row_stride, block_len, vt, sigma, perm, scale);
    return hipGetLastError();
}

}  // namespace milo
