// Batched Gram matrices G_b = X_b^T X_b of 128-wide KV blocks on bf16 MFMA.
//
// The contraction runs over tokens, but the cache is token-major, so each
// 64-token tile is staged in LDS and MFMA fragments (8 consecutive tokens of one
// feature per lane) are gathered with 16-bit LDS reads.  The row pitch of 264
// bytes puts the two lane halves of a wave (tokens 8 apart) on disjoint bank
// sets.  fp32 inputs are split exactly into three bf16 terms and the six
// products with term-order sum <= 2 are accumulated, which keeps the Gram
// accurate to fp32 level; bf16 inputs are exact in one term.
//
// One workgroup (4 waves) per (block, token split); wave w owns the 64 x 64
// quadrant (w / 2, w % 2) of G as 2 x 2 tiles of 32 x 32.
//
// bf16 inputs (the method's cache) have their own kernel: tiles stream through
// an LDS ring filled by DMA several tiles ahead, and the fragments are read with
// transposing LDS loads (two per fragment instead of eight 16-bit reads).
#include "common.hpp"
#include "kernels.hpp"

namespace milo {
namespace {

constexpr int kTT = 64;      // tokens per LDS tile
constexpr int kPitch = 132;  // LDS row pitch in 16-bit elements (264 bytes)

template <int NX>
__global__ __launch_bounds__(256) void gram_kernel(const void *__restrict__ x,
                                                   const int64_t *__restrict__ row0,
                                                   int64_t row_stride, int T, int splits,
                                                   float *__restrict__ gpart) {
    __shared__ __align__(16) uint16_t tile[NX][kTT * kPitch];
    const int blk = blockIdx.x / splits;
    const int sp = blockIdx.x - blk * splits;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int span = T / splits;
    const int t_begin = sp * span;
    const int64_t base = row0 ? row0[blk] : static_cast<int64_t>(blk) * T * row_stride;
    const int mb = wave >> 1, nb = wave & 1;

    f32x16_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = zero16();

    for (int t0 = t_begin; t0 < t_begin + span; t0 += kTT) {
        if constexpr (NX == 1) {
            const uint16_t *xb = static_cast<const uint16_t *>(x) + base;
#pragma unroll
            for (int c = tid; c < kTT * 16; c += 256) {
                const int r = c >> 4, cc = c & 15;
                const uint4 v = *reinterpret_cast<const uint4 *>(
                    xb + static_cast<int64_t>(t0 + r) * row_stride + cc * 8);
                uint2 *dst = reinterpret_cast<uint2 *>(&tile[0][r * kPitch + cc * 8]);
                dst[0] = make_uint2(v.x, v.y);
                dst[1] = make_uint2(v.z, v.w);
            }
        } else {
            const float *xb = static_cast<const float *>(x) + base;
#pragma unroll
            for (int c = tid; c < kTT * 32; c += 256) {
                const int r = c >> 5, cc = c & 31;
                const float4 v = *reinterpret_cast<const float4 *>(
                    xb + static_cast<int64_t>(t0 + r) * row_stride + cc * 4);
                const float f[4] = {v.x, v.y, v.z, v.w};
                uint16_t h[3][4];
#pragma unroll
                for (int e = 0; e < 4; ++e) split3_bf16(f[e], h[0][e], h[1][e], h[2][e]);
#pragma unroll
                for (int s = 0; s < NX; ++s) {
                    uint2 w;
                    w.x = static_cast<uint32_t>(h[s][0]) | (static_cast<uint32_t>(h[s][1]) << 16);
                    w.y = static_cast<uint32_t>(h[s][2]) | (static_cast<uint32_t>(h[s][3]) << 16);
                    *reinterpret_cast<uint2 *>(&tile[s][r * kPitch + cc * 4]) = w;
                }
            }
        }
        __syncthreads();

#pragma unroll
        for (int ks = 0; ks < kTT; ks += 16) {
            const int tok = ks + 8 * (lane >> 5);
            u16x8_t fa[NX][2], fb[NX][2];
#pragma unroll
            for (int s = 0; s < NX; ++s)
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const int fA = 64 * mb + 32 * i + (lane & 31);
                    const int fB = 64 * nb + 32 * i + (lane & 31);
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        fa[s][i][e] = tile[s][(tok + e) * kPitch + fA];
                        fb[s][i][e] = tile[s][(tok + e) * kPitch + fB];
                    }
                }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) {
#pragma unroll
                    for (int sa = 0; sa < NX; ++sa)
#pragma unroll
                        for (int sb = 0; sb < NX; ++sb)
                            if (sa + sb <= 2) acc[i][j] = mfma32x32x16(fa[sa][i], fb[sb][j], acc[i][j]);
                }
        }
        __syncthreads();
    }

    float *g = gpart + (static_cast<int64_t>(blk) * splits + sp) * kD * kD;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = 64 * mb + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                const int col = 64 * nb + 32 * j + (lane & 31);
                g[row * kD + col] = acc[i][j][r];
            }
}

// bf16 X streams through a ring of kGRing 32-token tiles in LDS, filled by LDS
// DMA (global_load_lds, 16 bytes per lane, no registers) kGAhead tiles ahead of
// use; wave w moves rows 8 w .. 8 w + 7 of every tile.  Rows are 256 bytes,
// unpadded; a row's 16-byte chunk c sits at chunk c ^ 4 (row % 4).  A
// transposing read of 64 lanes touches rows {0..3, 8..11} (plus a multiple of
// 4) and four consecutive chunks of each; with the swizzle the eight rows fall
// on four distinct groups of four chunks, two rows each, so every bank is hit
// exactly twice (512 bytes in two passes), as with a padded row.
constexpr int kGT = 32;                      // tokens per ring tile
constexpr int kGRing = 6;                    // ring slots (48 KiB: three workgroups per CU)
constexpr int kGAhead = kGRing - 1;          // tiles in flight ahead of use
constexpr int kGTileB = kGT * kD * 2;        // bytes of one tile
constexpr int kGDma = kGTileB / 1024 / 4;    // 1 KiB DMA instructions per wave and tile

// s_waitcnt immediate: at most n vector memory operations outstanding.
constexpr int vmcnt_imm(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) void *)p));
}

// The sixteen transposing reads of one tile (four fragment bases, two k-steps
// of 16 tokens, two 4-row halves), waited for inside the same asm block: the
// compiler then sees no LDS read that the DMAs in flight might write (it would
// wait for all of them), and no result is used before it has arrived.
__device__ __forceinline__ void read_tile_tr(u16x4_t (&o)[16], const uint32_t (&b)[4], uint32_t so) {
    typedef short v4s __attribute__((ext_vector_type(4)));
    v4s r[16];
    const uint32_t a0 = b[0] + so, a1 = b[1] + so, a2 = b[2] + so, a3 = b[3] + so;
    asm volatile(
        "ds_read_b64_tr_b16 %0, %16\n\t"
        "ds_read_b64_tr_b16 %1, %16 offset:1024\n\t"
        "ds_read_b64_tr_b16 %2, %17\n\t"
        "ds_read_b64_tr_b16 %3, %17 offset:1024\n\t"
        "ds_read_b64_tr_b16 %4, %18\n\t"
        "ds_read_b64_tr_b16 %5, %18 offset:1024\n\t"
        "ds_read_b64_tr_b16 %6, %19\n\t"
        "ds_read_b64_tr_b16 %7, %19 offset:1024\n\t"
        "ds_read_b64_tr_b16 %8, %16 offset:4096\n\t"
        "ds_read_b64_tr_b16 %9, %16 offset:5120\n\t"
        "ds_read_b64_tr_b16 %10, %17 offset:4096\n\t"
        "ds_read_b64_tr_b16 %11, %17 offset:5120\n\t"
        "ds_read_b64_tr_b16 %12, %18 offset:4096\n\t"
        "ds_read_b64_tr_b16 %13, %18 offset:5120\n\t"
        "ds_read_b64_tr_b16 %14, %19 offset:4096\n\t"
        "ds_read_b64_tr_b16 %15, %19 offset:5120\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]),
          "=&v"(r[7]), "=&v"(r[8]), "=&v"(r[9]), "=&v"(r[10]), "=&v"(r[11]), "=&v"(r[12]), "=&v"(r[13]),
          "=&v"(r[14]), "=&v"(r[15])
        : "v"(a0), "v"(a1), "v"(a2), "v"(a3)
        : "memory");
#pragma unroll
    for (int k = 0; k < 16; ++k) o[k] = __builtin_bit_cast(u16x4_t, r[k]);
}

__global__ __launch_bounds__(256) void gram_bf16_kernel(const uint16_t *__restrict__ x,
                                                        const int64_t *__restrict__ row0,
                                                        int64_t row_stride, int T, int splits,
                                                        float *__restrict__ gpart) {
    __shared__ __align__(16) uint8_t ring[kGRing * kGTileB];
    const int blk = blockIdx.x / splits;
    const int sp = blockIdx.x - blk * splits;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int span = T / splits;
    const int t_begin = sp * span;
    const int n_tiles = span / kGT;
    const uint8_t *xb = reinterpret_cast<const uint8_t *>(x + (row0 ? row0[blk] : static_cast<int64_t>(blk) * T * row_stride)) +
                        static_cast<int64_t>(t_begin) * row_stride * 2;
    const int mb = wave >> 1, nb = wave & 1;
    const int g = lane >> 4, j = lane & 15;  // 16-lane group, lane within it

    // DMA of tile tau (clamped to the last tile) into slot tau % kGRing: lane L
    // of instruction q writes row 4 q + L / 16, physical chunk L % 16.
    auto dma = [&](int tau) __attribute__((always_inline)) {
        const int tt = tau < n_tiles ? tau : n_tiles - 1;
#pragma unroll
        for (int k = 0; k < kGDma; ++k) {
            const int q = kGDma * wave + k;
            const int r = 4 * q + (lane >> 4), c = (lane & 15) ^ (4 * (r & 3));
            const uint8_t *src = xb + (static_cast<int64_t>(kGT * tt + r) * row_stride) * 2 + 16 * c;
            __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)src,
                                             (__attribute__((address_space(3))) void *)(ring + (tau % kGRing) * kGTileB + 1024 * q),
                                             16, 0, 0);
        }
    };
#pragma unroll
    for (int tau = 0; tau < kGAhead; ++tau) dma(tau);

    // Fragment bases in slot 0: lane (g, j) reads features f + 16 (g % 2) + 4 (j % 4) .. + 3
    // of rows 8 (g / 2) + j / 4 (and + 4) of a 16-token k-step, f = 64 mb + 32 i (A) or
    // 64 nb + 32 i (B), i.e. column j of rows r0 .. r0 + 3 as a transposing read delivers it.
    const int rr = 8 * (g >> 1) + (j >> 2);
    uint32_t fbase[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int f = (q < 2 ? 64 * mb + 32 * q : 64 * nb + 32 * (q - 2)) + 16 * (g & 1) + 4 * (j & 3);
        fbase[q] = lds_addr(ring) + rr * (kD * 2) + 16 * ((f >> 3) ^ (4 * (rr & 3))) + 2 * (f & 7);
    }

    f32x16_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) acc[i][jj] = zero16();

    for (int t = 0; t < n_tiles; ++t) {
        // this wave's part of tile t has landed (each later tile added kGDma
        // operations); the barrier makes every part visible and frees slot
        // (t - 1) % kGRing for the tile kGAhead ahead
        __builtin_amdgcn_s_waitcnt(vmcnt_imm((kGAhead - 1) * kGDma));
        __syncthreads();
        dma(t + kGAhead);
        u16x4_t o[16];
        read_tile_tr(o, fbase, (t % kGRing) * kGTileB);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const u16x8_t fa0 = cat8(o[8 * ks + 0], o[8 * ks + 1]), fa1 = cat8(o[8 * ks + 2], o[8 * ks + 3]);
            const u16x8_t fb0 = cat8(o[8 * ks + 4], o[8 * ks + 5]), fb1 = cat8(o[8 * ks + 6], o[8 * ks + 7]);
            acc[0][0] = mfma32x32x16(fa0, fb0, acc[0][0]);
            acc[0][1] = mfma32x32x16(fa0, fb1, acc[0][1]);
            acc[1][0] = mfma32x32x16(fa1, fb0, acc[1][0]);
            acc[1][1] = mfma32x32x16(fa1, fb1, acc[1][1]);
        }
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // the trailing (discarded) tiles have landed

    float *gp = gpart + (static_cast<int64_t>(blk) * splits + sp) * kD * kD;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = 64 * mb + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                const int col = 64 * nb + 32 * jj + (lane & 31);
                gp[row * kD + col] = acc[i][jj][r];
            }
}

}  // namespace

hipError_t launch_gram(const void *x, int x_type, const int64_t *row0, int64_t row_stride,
                       int block_len, int n_blocks, int splits, float *gpart, hipStream_t st) {
    if (n_blocks <= 0) return hipSuccess;
    const dim3 grid(static_cast<unsigned>(n_blocks * splits));
    if (x_type == kBF16)
        hipLaunchKernelGGL(gram_bf16_kernel, grid, dim3(256), 0, st, static_cast<const uint16_t *>(x), row0,
                           row_stride, block_len, splits, gpart);
    else
        hipLaunchKernelGGL(gram_kernel<3>, grid, dim3(256), 0, st, x, row0, row_stride, block_len,
                           splits, gpart);
    return hipGetLastError();
}

}  // namespace milo
