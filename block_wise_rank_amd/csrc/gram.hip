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
// bf16 inputs (the method's cache) have their own kernel: tiles are
// double-buffered in LDS with the next tile's loads in flight during the
// current tile's products, and the fragments are read with transposing LDS
// loads (two per fragment instead of eight 16-bit reads), from rows of 288
// bytes so that the 4 rows x 64 bytes of a half-wave's read cover every bank
// exactly twice.
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

constexpr int kBP = 288;  // LDS row pitch in bytes (bf16 kernel)

__global__ __launch_bounds__(256) void gram_bf16_kernel(const uint16_t *__restrict__ x,
                                                        const int64_t *__restrict__ row0,
                                                        int64_t row_stride, int T, int splits,
                                                        float *__restrict__ gpart) {
    __shared__ __align__(16) uint8_t tile[2][kTT * kBP];
    const int blk = blockIdx.x / splits;
    const int sp = blockIdx.x - blk * splits;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int span = T / splits;
    const int t_begin = sp * span;
    const uint16_t *xb = x + (row0 ? row0[blk] : static_cast<int64_t>(blk) * T * row_stride);
    const int mb = wave >> 1, nb = wave & 1;
    const int g = lane >> 4, j = lane & 15;  // 16-lane group, lane within it

    f32x16_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) acc[i][jj] = zero16();

    // tile loads: token row c >> 4, 16-byte piece c & 15 for c = tid + 256 u
    const int64_t off0 = static_cast<int64_t>(tid >> 4) * row_stride + (tid & 15) * 8;
    const int64_t rstep = 16 * row_stride;  // c + 256 is 16 token rows further
    const int so = (tid >> 4) * kBP + (tid & 15) * 16;
    uint4 x0, x1, x2, x3;
    auto load = [&](int t0) {
        const uint16_t *p = xb + static_cast<int64_t>(t0) * row_stride + off0;
        x0 = *reinterpret_cast<const uint4 *>(p);
        x1 = *reinterpret_cast<const uint4 *>(p + rstep);
        x2 = *reinterpret_cast<const uint4 *>(p + 2 * rstep);
        x3 = *reinterpret_cast<const uint4 *>(p + 3 * rstep);
    };
    const int n_tiles = span / kTT;
    load(t_begin);
    for (int it = 0; it < n_tiles; ++it) {
        uint8_t *tb = tile[it & 1];
        *reinterpret_cast<uint4 *>(tb + so) = x0;
        *reinterpret_cast<uint4 *>(tb + so + 16 * kBP) = x1;
        *reinterpret_cast<uint4 *>(tb + so + 32 * kBP) = x2;
        *reinterpret_cast<uint4 *>(tb + so + 48 * kBP) = x3;
        if (it + 1 < n_tiles) load(t_begin + (it + 1) * kTT);
        __syncthreads();
#pragma unroll
        for (int ks = 0; ks < kTT; ks += 16) {
            // lane (g, j): features base + 16 (g % 2) + j, tokens ks + 8 (g / 2) + 4 h + 0..3
            const uint8_t *rowp = tb + (ks + 8 * (g >> 1) + (j >> 2)) * kBP + (16 * (g & 1) + 4 * (j & 3)) * 2;
            u16x8_t fa[2], fb[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const uint8_t *pa = rowp + (64 * mb + 32 * i) * 2;
                const uint8_t *pb = rowp + (64 * nb + 32 * i) * 2;
                fa[i] = cat8(lds_read_tr16(pa), lds_read_tr16(pa + 4 * kBP));
                fb[i] = cat8(lds_read_tr16(pb), lds_read_tr16(pb + 4 * kBP));
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int jj = 0; jj < 2; ++jj) acc[i][jj] = mfma32x32x16(fa[i], fb[jj], acc[i][jj]);
        }
    }

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
