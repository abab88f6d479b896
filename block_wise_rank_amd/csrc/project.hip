// Factor pairs of each block from its sorted right singular vectors:
//   B_b = V_r^T (r_b x d rows), stored in the factor dtype;
//   A_b = X_b B~_b^T with B~_b the STORED (rounded or quantised) B_b, so that the
//         rebuilt block A_b B~_b is X_b projected on the stored basis;
//   A_b is written transposed (rank-major, r_b rows of T tokens).
// INT8: every row of B_b (one per rank) and every row of A_b (one per token)
// gets an absmax scale s = max|row| / 127 and codes rint(x / s) clamped to
// +-127, decided in fp32.
// 4-bit: A_b = X_b B_b^T with the fp32-accurate B_b (the products are the
// fp32 storage's, bit for bit), then every run of 32 consecutive elements of a
// rank row of A^T (tokens) and of B (features) gets s = max|run| / 7 and codes
// rint(x / s) in [-7, 7], decided in fp32.
// 2-bit: the same runs with s = max|run| / 3 and a code c in 0..3 for the
// level (2c - 3) s nearest to x: |x / s| >= 2 (the fp32 quotient) takes the
// outer level of x's sign, else the inner one; x = 0 and s = 0 give code 2.
//
// A^T = B~ X^T runs on bf16 MFMA (M = rank, N = token, K = feature): the
// fragments of B~ stay in registers (one 32-rank tile per wave) while 32-token
// tiles of X stream in as 16-byte loads of 8 consecutive features.  fp32
// storage splits V (and fp32 X) into three bf16 terms for fp32-accurate
// products.  Grid: (block, 256-token part).
//
// bf16 X -> bf16 factors (the storage the method runs on) has its own kernel:
// 1024-token parts (B fragments built twice per 2048-token block instead of
// eight times), the next X tile loaded while the current one's products run,
// and each wave's 32 rank rows collected for 128 tokens in LDS so that A^T is
// written as whole 256-byte row pieces with 16-byte stores.
#include "common.hpp"
#include "kernels.hpp"

namespace milo {
namespace {

constexpr int kTokensPerWG = 256;

// 4-bit B row i: this lane holds features 16 ks + 8 (lane / 32) + e of it, so
// the 32-feature run g sits in k-steps 2 g and 2 g + 1 of this lane and of
// lane ^ 32.  Every lane takes part (cross-lane max); `store` picks the writers.
__device__ __forceinline__ void store_b_i4(const float (&v)[8][8], int i, int r, int lane, bool store,
                                           uint8_t *Bb) {
    float sB4[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        float m = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) m = fmaxf(m, fmaxf(fabsf(v[2 * g][e]), fabsf(v[2 * g + 1][e])));
        m = fmaxf(m, __shfl_xor(m, 32, 64));
        sB4[g] = __fdiv_rn(m, 7.f);
    }
    if (!store) return;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
        const float sg = sB4[ks >> 1];
        uint32_t w = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float c = sg > 0.f ? rintf(__fdiv_rn(v[ks][e], sg)) : 0.f;
            c = fminf(fmaxf(c, -7.f), 7.f);
            w |= (static_cast<uint32_t>(static_cast<int>(c)) & 0xfu) << (4 * e);
        }
        *reinterpret_cast<uint32_t *>(Bb + static_cast<int64_t>(i) * (kD / 2) + 8 * ks + 4 * (lane >> 5)) = w;
    }
    if (lane < 32)
        *reinterpret_cast<float4 *>(Bb + static_cast<int64_t>(r) * (kD / 2) + 16 * i) =
            make_float4(sB4[0], sB4[1], sB4[2], sB4[3]);
}

// 2-bit code of x in a run of scale s.  The quotient's test fl(|x| / s) >= 2
// holds exactly when |x| >= 2 s: 2 s is exact in fp32, and any fp32 value below
// 2 s has a quotient of at most 2 - 2^-23, which rounds below 2.  So no division
// is needed for the same decision.
__device__ __forceinline__ uint32_t code2(float x, float s) {
    if (!(s > 0.f)) return 2u;
    const bool outer = fabsf(x) >= 2.f * s;
    return x < 0.f ? (outer ? 0u : 1u) : (outer ? 3u : 2u);
}

// 2-bit B row i (the lane layout of store_b_i4): codes of features 16 ks +
// 8 (lane / 32) .. + 7 as one 16-bit piece, then the row's four run scales.
__device__ __forceinline__ void store_b_i2(const float (&v)[8][8], int i, int r, int lane, bool store,
                                           uint8_t *Bb) {
    float sB4[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        float m = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) m = fmaxf(m, fmaxf(fabsf(v[2 * g][e]), fabsf(v[2 * g + 1][e])));
        m = fmaxf(m, __shfl_xor(m, 32, 64));
        sB4[g] = __fdiv_rn(m, 3.f);
    }
    if (!store) return;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
        uint32_t h = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) h |= code2(v[ks][e], sB4[ks >> 1]) << (2 * e);
        *reinterpret_cast<uint16_t *>(Bb + static_cast<int64_t>(i) * (kD / 4) + 4 * ks + 2 * (lane >> 5)) =
            static_cast<uint16_t>(h);
    }
    if (lane < 32)
        *reinterpret_cast<float4 *>(Bb + static_cast<int64_t>(r) * (kD / 4) + 16 * i) =
            make_float4(sB4[0], sB4[1], sB4[2], sB4[3]);
}

template <int NX, int OUT>
__global__ __launch_bounds__(256) void project_kernel(
    const void *__restrict__ x, const int64_t *__restrict__ row0, int64_t row_stride, int T,
    const float *__restrict__ vt, const int32_t *__restrict__ perm, const float *__restrict__ vscale,
    const int32_t *__restrict__ rank,
    const int64_t *__restrict__ a_off, const int64_t *__restrict__ b_off,
    uint8_t *__restrict__ arena, float *__restrict__ a_scale, float *__restrict__ b_scale) {
    constexpr int NS = (OUT == kF32 || OUT == kI4 || OUT == kI2) ? 3 : 1;  // bf16 terms of the B operand
    __shared__ float sB_rows[kD];
    __shared__ float tmax[4][32];

    const int blk = blockIdx.x, part = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r = rank[blk];
    const int t_begin = part * kTokensPerWG;
    const int t_end = min(T, t_begin + kTokensPerWG);
    if (r == 0) {
        if constexpr (OUT == kI8)
            for (int t = t_begin + tid; t < t_end; t += 256) a_scale[static_cast<int64_t>(blk) * T + t] = 0.f;
        return;
    }
    const int ebytes = OUT == kF32 ? 4 : (OUT == kBF16 ? 2 : 1);
    uint8_t *Ab = arena + a_off[blk];
    uint8_t *Bb = arena + b_off[blk];

    // ---- B fragments: row i = 32 wave + lane % 32, k slots j = 16 ks + 8 (lane / 32) + e.
    const int i = 32 * wave + (lane & 31);
    const bool row_ok = i < r;
    // sorted rank i: row perm[i] of the eigensolver's output times vscale[i]
    const int vsrc = row_ok ? perm[static_cast<int64_t>(blk) * kD + i] : 0;
    const float vsc = row_ok ? vscale[static_cast<int64_t>(blk) * kD + i] : 0.f;
    const float *vrow = vt + static_cast<int64_t>(blk) * kD * kD + static_cast<int64_t>(vsrc) * kD;
    float v[8][8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
        if (row_ok) {
            const float4 a = *reinterpret_cast<const float4 *>(vrow + 16 * ks + 8 * (lane >> 5));
            const float4 b = *reinterpret_cast<const float4 *>(vrow + 16 * ks + 8 * (lane >> 5) + 4);
            v[ks][0] = a.x * vsc; v[ks][1] = a.y * vsc; v[ks][2] = a.z * vsc; v[ks][3] = a.w * vsc;
            v[ks][4] = b.x * vsc; v[ks][5] = b.y * vsc; v[ks][6] = b.z * vsc; v[ks][7] = b.w * vsc;
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) v[ks][e] = 0.f;
        }
    }
    float sB = 1.f;
    if constexpr (OUT == kI8) {
        float m = 0.f;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks)
#pragma unroll
            for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(v[ks][e]));
        m = fmaxf(m, __shfl_xor(m, 32, 64));
        sB = __fdiv_rn(m, 127.f);
    }
    u16x8_t fa[NS][8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            if constexpr (OUT == kF32 || OUT == kI4 || OUT == kI2) {
                uint16_t h, mm, l;
                split3_bf16(v[ks][e], h, mm, l);
                fa[0][ks][e] = h;
                fa[1 % NS][ks][e] = mm;
                fa[2 % NS][ks][e] = l;
            } else if constexpr (OUT == kBF16) {
                fa[0][ks][e] = f32_to_bf16_bits(v[ks][e]);
            } else {
                float q = sB > 0.f ? rintf(__fdiv_rn(v[ks][e], sB)) : 0.f;
                q = fminf(fmaxf(q, -127.f), 127.f);
                v[ks][e] = q;  // keep the code for the B store
                fa[0][ks][e] = f32_to_bf16_bits(q);  // |q| <= 127 is exact in bf16
            }
        }

    // ---- B rows (first part only) and B scales.
    if constexpr (OUT == kI4) store_b_i4(v, i, r, lane, part == 0 && row_ok, Bb);
    if constexpr (OUT == kI2) store_b_i2(v, i, r, lane, part == 0 && row_ok, Bb);
    if (OUT != kI4 && OUT != kI2 && part == 0 && row_ok) {
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            const int j0 = 16 * ks + 8 * (lane >> 5);
            uint8_t *dst = Bb + (static_cast<int64_t>(i) * kD + j0) * ebytes;
            if constexpr (OUT == kF32) {
                float4 *d4 = reinterpret_cast<float4 *>(dst);
                d4[0] = make_float4(v[ks][0], v[ks][1], v[ks][2], v[ks][3]);
                d4[1] = make_float4(v[ks][4], v[ks][5], v[ks][6], v[ks][7]);
            } else if constexpr (OUT == kBF16) {
                *reinterpret_cast<u16x8_t *>(dst) = fa[0][ks];
            } else {
                uint2 w;
                w.x = (static_cast<uint32_t>(static_cast<uint8_t>(static_cast<int8_t>(v[ks][0])))) |
                      (static_cast<uint32_t>(static_cast<uint8_t>(static_cast<int8_t>(v[ks][1]))) << 8) |
                      (static_cast<uint32_t>(static_cast<uint8_t>(static_cast<int8_t>(v[ks][2]))) << 16) |
                      (static_cast<uint32_t>(static_cast<uint8_t>(static_cast<int8_t>(v[ks][3]))) << 24);
                w.y = (static_cast<uint32_t>(static_cast<uint8_t>(static_cast<int8_t>(v[ks][4])))) |
                      (static_cast<uint32_t>(static_cast<uint8_t>(static_cast<int8_t>(v[ks][5]))) << 8) |
                      (static_cast<uint32_t>(static_cast<uint8_t>(static_cast<int8_t>(v[ks][6]))) << 16) |
                      (static_cast<uint32_t>(static_cast<uint8_t>(static_cast<int8_t>(v[ks][7]))) << 24);
                *reinterpret_cast<uint2 *>(dst) = w;
            }
        }
        if constexpr (OUT == kI8)
            if (lane < 32) b_scale[static_cast<int64_t>(blk) * kD + i] = sB;
    }
    if constexpr (OUT == kI8) {
        if (lane < 32) sB_rows[i] = row_ok ? sB : 0.f;
        __syncthreads();
    }

    const int64_t base = row0 ? row0[blk] : static_cast<int64_t>(blk) * T * row_stride;
    const bool wave_active = 32 * wave < r;
    for (int t0 = t_begin; t0 < t_end; t0 += 32) {
        const int t = t0 + (lane & 31);
        f32x16_t acc = zero16();
        if (wave_active) {
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) {
                const int j0 = 16 * ks + 8 * (lane >> 5);
                if constexpr (NX == 1) {
                    const u16x8_t fb = *reinterpret_cast<const u16x8_t *>(
                        static_cast<const uint16_t *>(x) + base + static_cast<int64_t>(t) * row_stride + j0);
#pragma unroll
                    for (int s = 0; s < NS; ++s) acc = mfma32x32x16(fa[s][ks], fb, acc);
                } else {
                    const float *xr = static_cast<const float *>(x) + base +
                                      static_cast<int64_t>(t) * row_stride + j0;
                    const float4 a = reinterpret_cast<const float4 *>(xr)[0];
                    const float4 b = reinterpret_cast<const float4 *>(xr)[1];
                    const float f[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
                    u16x8_t fb[3];
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        uint16_t h, mm, l;
                        split3_bf16(f[e], h, mm, l);
                        fb[0][e] = h;
                        fb[1][e] = mm;
                        fb[2][e] = l;
                    }
#pragma unroll
                    for (int sa = 0; sa < NS; ++sa)
#pragma unroll
                        for (int sb = 0; sb < 3; ++sb)
                            if (sa + sb <= 2) acc = mfma32x32x16(fa[sa][ks], fb[sb], acc);
                }
            }
        }
        // acc[q]: rank row i' = 32 wave + 8 (q / 4) + 4 (lane / 32) + q % 4, token t.
        if constexpr (OUT == kI4) {
            // 32-token run of row i' = this tile: lanes of one half hold it
            if (wave_active) {
#pragma unroll
                for (int q = 0; q < 16; ++q) {
                    const int ir = 32 * wave + 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);
                    float m = fabsf(acc[q]);
#pragma unroll
                    for (int o = 1; o < 32; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
                    const float sA = __fdiv_rn(m, 7.f);
                    float c = sA > 0.f ? rintf(__fdiv_rn(acc[q], sA)) : 0.f;
                    c = fminf(fmaxf(c, -7.f), 7.f);
                    // eight tokens' nibbles into one word (token t0 + 8k + e at bits 4e)
                    uint32_t w = (static_cast<uint32_t>(static_cast<int>(c)) & 0xfu) << (4 * (lane & 7));
                    w |= __shfl_xor(w, 1, 64);
                    w |= __shfl_xor(w, 2, 64);
                    w |= __shfl_xor(w, 4, 64);
                    if (ir < r) {
                        if ((lane & 7) == 0)
                            *reinterpret_cast<uint32_t *>(Ab + static_cast<int64_t>(ir) * (T / 2) + t / 2) = w;
                        if ((lane & 31) == 0)
                            *reinterpret_cast<float *>(Ab + static_cast<int64_t>(r) * (T / 2) +
                                                       (static_cast<int64_t>(ir) * (T / kI4Group) + t0 / kI4Group) * 4) = sA;
                    }
                }
            }
        } else if constexpr (OUT == kI2) {
            // 32-token run of row i' = this tile, held by the lanes of one half
            if (wave_active) {
#pragma unroll
                for (int q = 0; q < 16; ++q) {
                    const int ir = 32 * wave + 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);
                    float m = fabsf(acc[q]);
#pragma unroll
                    for (int o = 1; o < 32; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
                    const float sA = __fdiv_rn(m, 3.f);
                    // sixteen tokens' codes into one word (token t0 + 16k + e at bits 2e)
                    uint32_t w = code2(acc[q], sA) << (2 * (lane & 15));
                    w |= __shfl_xor(w, 1, 64);
                    w |= __shfl_xor(w, 2, 64);
                    w |= __shfl_xor(w, 4, 64);
                    w |= __shfl_xor(w, 8, 64);
                    if (ir < r) {
                        if ((lane & 15) == 0)
                            *reinterpret_cast<uint32_t *>(Ab + static_cast<int64_t>(ir) * (T / 4) + t / 4) = w;
                        if ((lane & 31) == 0)
                            *reinterpret_cast<float *>(Ab + static_cast<int64_t>(r) * (T / 4) +
                                                       (static_cast<int64_t>(ir) * (T / kI4Group) + t0 / kI4Group) * 4) = sA;
                    }
                }
            }
        } else if constexpr (OUT != kI8) {
            if (wave_active) {
#pragma unroll
                for (int q = 0; q < 16; ++q) {
                    const int ir = 32 * wave + 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);
                    if (ir < r) {
                        if constexpr (OUT == kF32)
                            reinterpret_cast<float *>(Ab)[static_cast<int64_t>(ir) * T + t] = acc[q];
                        else
                            reinterpret_cast<uint16_t *>(Ab)[static_cast<int64_t>(ir) * T + t] =
                                f32_to_bf16_bits(acc[q]);
                    }
                }
            }
        } else {
            float val[16];
            float m = 0.f;
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const int ir = 32 * wave + 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);
                val[q] = (ir < r) ? acc[q] * sB_rows[ir] : 0.f;
                m = fmaxf(m, fabsf(val[q]));
            }
            m = fmaxf(m, __shfl_xor(m, 32, 64));
            if (lane < 32) tmax[wave][lane] = m;
            __syncthreads();
            const int tl = lane & 31;
            const float mt = fmaxf(fmaxf(tmax[0][tl], tmax[1][tl]), fmaxf(tmax[2][tl], tmax[3][tl]));
            const float sA = __fdiv_rn(mt, 127.f);
            if (wave_active) {
#pragma unroll
                for (int q = 0; q < 16; ++q) {
                    const int ir = 32 * wave + 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);
                    if (ir < r) {
                        float c = sA > 0.f ? rintf(__fdiv_rn(val[q], sA)) : 0.f;
                        c = fminf(fmaxf(c, -127.f), 127.f);
                        reinterpret_cast<int8_t *>(Ab)[static_cast<int64_t>(ir) * T + t] =
                            static_cast<int8_t>(c);
                    }
                }
            }
            if (wave == 0 && lane < 32) a_scale[static_cast<int64_t>(blk) * T + t] = sA;
            __syncthreads();
        }
    }
}

constexpr int kPartBF = 1024;   // tokens per workgroup (bf16 path)
constexpr int kStageT = 128;    // tokens collected per flush
constexpr int kStageP = 264;    // LDS pitch (bytes) of a staged rank row (256 B + 8)

// Cooperative stream of a block part's bf16 rows through LDS: four 32-token
// slots of 272-byte rows (the 16-byte reads of 32 consecutive rows fall on
// distinct banks).  Wave w loads rows 8 w .. 8 w + 7 of a tile (two 16-byte
// loads per lane) four tiles ahead of its use, so that the workgroup keeps four
// distinct tiles in flight instead of every wave loading every tile.
// compute(t, cur) receives tile t's B fragments (token lane % 32, features
// 16 ks + 8 (lane / 32) + e).  Every wave of the workgroup must take part;
// n_tiles is even.
constexpr int kXRowB = kD * 2 + 16;
constexpr int kXSlot = 32 * kXRowB;

template <typename F>
__device__ __forceinline__ void stream_x_ring(uint8_t *ring, const uint16_t *xrow0, int64_t row_stride,
                                              int n_tiles, int wave, int lane, F &&compute) {
    const int lr = 8 * wave + (lane >> 4);  // rows lr and lr + 4 of a tile
    const uint8_t *xl = reinterpret_cast<const uint8_t *>(xrow0) + static_cast<int64_t>(lr) * row_stride * 2 +
                        16 * (lane & 15);
    const int64_t x4 = 8 * row_stride, x32 = 64 * row_stride;  // bytes of 4 and of 32 rows
    auto load_q = [&](uint4 &ra, uint4 &rb, int tile) __attribute__((always_inline)) {
        const int tt = tile < n_tiles ? tile : n_tiles - 1;  // past the end: the last tile again
        const uint8_t *p0 = xl + tt * x32;
        ra = *reinterpret_cast<const uint4 *>(p0);
        rb = *reinterpret_cast<const uint4 *>(p0 + x4);
    };
    auto store_q = [&](const uint4 &ra, const uint4 &rb, int tile) __attribute__((always_inline)) {
        uint8_t *p0 = ring + (tile & 3) * kXSlot + lr * kXRowB + 16 * (lane & 15);
        *reinterpret_cast<uint4 *>(p0) = ra;
        *reinterpret_cast<uint4 *>(p0 + 4 * kXRowB) = rb;
    };
    auto step = [&](uint4 &na, uint4 &nb, int t) __attribute__((always_inline)) {
        const uint8_t *src = ring + (t & 3) * kXSlot + (lane & 31) * kXRowB + 16 * (lane >> 5);
        u16x8_t cur[8];
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) cur[ks] = *reinterpret_cast<const u16x8_t *>(src + 32 * ks);
        compute(t, cur);
        store_q(na, nb, t + 1);  // its slot was last read in tile t - 3
        load_q(na, nb, t + 5);
        __syncthreads();
    };
    // tile k waits in (qka, qkb), k = tile % 4, until it is stored, one tile before its use
    uint4 q0a, q0b, q1a, q1b, q2a, q2b, q3a, q3b;
    {
        uint4 ra, rb;
        load_q(ra, rb, 0);
        load_q(q1a, q1b, 1);
        load_q(q2a, q2b, 2);
        load_q(q3a, q3b, 3);
        load_q(q0a, q0b, 4);
        store_q(ra, rb, 0);
    }
    __syncthreads();
    int t = 0;
    for (; t + 4 <= n_tiles; t += 4) {
        step(q1a, q1b, t);
        step(q2a, q2b, t + 1);
        step(q3a, q3b, t + 2);
        step(q0a, q0b, t + 3);
    }
    if (t < n_tiles) {  // an even number of tiles: two remain
        step(q1a, q1b, t);
        step(q2a, q2b, t + 1);
    }
}

__global__ __launch_bounds__(256) void project_bf16_kernel(
    const uint16_t *__restrict__ x, const int64_t *__restrict__ row0, int64_t row_stride, int T,
    const float *__restrict__ vt, const int32_t *__restrict__ perm, const float *__restrict__ vscale,
    const int32_t *__restrict__ rank,
    const int64_t *__restrict__ a_off, const int64_t *__restrict__ b_off, uint8_t *__restrict__ arena) {
    __shared__ __align__(16) uint8_t stage[4][32 * kStageP];
    __shared__ __align__(16) uint8_t xring[4 * kXSlot];
    const int blk = blockIdx.x, part = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = rank[blk];
    if (r == 0) return;  // uniform over the workgroup
    const bool active = 32 * wave < r;  // the wave has rank rows (all waves stream X)
    const int t_begin = part * kPartBF;
    const int t_end = min(T, t_begin + kPartBF);
    uint16_t *Ab = reinterpret_cast<uint16_t *>(arena + a_off[blk]);
    uint16_t *Bb = reinterpret_cast<uint16_t *>(arena + b_off[blk]);

    // B~ fragments: rank row i = 32 wave + lane % 32, features 16 ks + 8 (lane / 32) + e
    const int i = 32 * wave + (lane & 31);
    const bool row_ok = i < r;
    // sorted rank i: row perm[i] of the eigensolver's output times vscale[i]
    const int vsrc = row_ok ? perm[static_cast<int64_t>(blk) * kD + i] : 0;
    const float vsc = row_ok ? vscale[static_cast<int64_t>(blk) * kD + i] : 0.f;
    const float *vrow = vt + static_cast<int64_t>(blk) * kD * kD + static_cast<int64_t>(vsrc) * kD;
    u16x8_t fa[8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
        float4 a = make_float4(0.f, 0.f, 0.f, 0.f), b = a;
        if (row_ok) {
            a = *reinterpret_cast<const float4 *>(vrow + 16 * ks + 8 * (lane >> 5));
            b = *reinterpret_cast<const float4 *>(vrow + 16 * ks + 8 * (lane >> 5) + 4);
            a = make_float4(a.x * vsc, a.y * vsc, a.z * vsc, a.w * vsc);
            b = make_float4(b.x * vsc, b.y * vsc, b.z * vsc, b.w * vsc);
        }
        const uint32_t w0 = f32x2_to_bf16x2_bits(a.x, a.y), w1 = f32x2_to_bf16x2_bits(a.z, a.w);
        const uint32_t w2 = f32x2_to_bf16x2_bits(b.x, b.y), w3 = f32x2_to_bf16x2_bits(b.z, b.w);
        fa[ks] = __builtin_bit_cast(u16x8_t, make_uint4(w0, w1, w2, w3));
        if (part == 0 && row_ok)  // B row i, features 16 ks + 8 (lane / 32) ..
            *reinterpret_cast<uint4 *>(Bb + i * kD + 16 * ks + 8 * (lane >> 5)) = make_uint4(w0, w1, w2, w3);
    }

    const uint16_t *xp = x + (row0 ? row0[blk] : static_cast<int64_t>(blk) * T * row_stride) +
                         static_cast<int64_t>(t_begin) * row_stride;
    uint8_t *stg = stage[wave];
    stream_x_ring(xring, xp, row_stride, (t_end - t_begin) / 32, wave, lane,
                  [&](int t, const u16x8_t (&xc)[8]) __attribute__((always_inline)) {
        if (!active) return;
        const int t0 = t_begin + 32 * t;
        f32x16_t acc = zero16(), acc1 = zero16();
#pragma unroll
        for (int ks = 0; ks < 8; ks += 2) {
            acc = mfma32x32x16(fa[ks], xc[ks], acc);
            acc1 = mfma32x32x16(fa[ks + 1], xc[ks + 1], acc1);
        }
        acc += acc1;
        // acc[q]: rank row 8 (q / 4) + 4 (lane / 32) + q % 4 of this wave, token lane % 32
        const int tt = (t0 - t_begin) & (kStageT - 1);
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const int row = 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);
            *reinterpret_cast<uint16_t *>(stg + row * kStageP + (tt + (lane & 31)) * 2) = f32_to_bf16_bits(acc[q]);
        }
        if (tt + 32 == kStageT || t0 + 32 >= t_end) {
            // flush: 32 rows x (tt + 32) tokens; 16 lanes per row, 16 bytes each
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            const int n16 = (tt + 32) / 8;  // 16-byte pieces per row
            const int tok0 = t0 + 32 - (tt + 32);
#pragma unroll
            for (int rr = 0; rr < 32; rr += 4) {
                const int row = rr + (lane >> 4), piece = lane & 15;
                const int ir = 32 * wave + row;
                if (ir < r && piece < n16)
                    *reinterpret_cast<uint4 *>(Ab + static_cast<int64_t>(ir) * T + tok0 + 8 * piece) =
                        *reinterpret_cast<const uint4 *>(stg + row * kStageP + piece * 16);
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }
    });
}

// bf16 X -> fp32, 4-bit or 2-bit factors: the B operand in three bf16 terms
// (the products are fp32-accurate and identical for all three storages, so the
// codes are those of the fp32 factors), 1024-token parts, X through the LDS
// ring above.  Each wave's 32 rank rows are collected in LDS as fp32 for 64
// tokens; the flush writes fp32 rows as whole pieces, or quantises each 32-token
// run (one run per lane: max, scale, codes) and writes its code bytes (16 for
// 4-bit, 8 for 2-bit) and its scale.
constexpr int kRunP = 36;           // LDS floats per staged 32-token run (16-byte aligned pieces)
constexpr int kRowP = 2 * kRunP;    // LDS floats per staged rank row (64 tokens)

template <int OUT>
__global__ __launch_bounds__(256, 2) void project_split_kernel(
    const uint16_t *__restrict__ x, const int64_t *__restrict__ row0, int64_t row_stride, int T,
    const float *__restrict__ vt, const int32_t *__restrict__ perm, const float *__restrict__ vscale,
    const int32_t *__restrict__ rank,
    const int64_t *__restrict__ a_off, const int64_t *__restrict__ b_off, uint8_t *__restrict__ arena) {
    __shared__ __align__(16) float stage[4][32 * kRowP];
    __shared__ __align__(16) uint8_t xring[4 * kXSlot];
    const int blk = blockIdx.x, part = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = rank[blk];
    if (r == 0) return;  // uniform over the workgroup
    const bool active = 32 * wave < r;  // the wave has rank rows (all waves stream X)
    const int t_begin = part * kPartBF;
    const int t_end = min(T, t_begin + kPartBF);
    uint8_t *Ab = arena + a_off[blk];
    uint8_t *Bb = arena + b_off[blk];

    // B fragments: rank row i = 32 wave + lane % 32, features 16 ks + 8 (lane / 32) + e
    const int i = 32 * wave + (lane & 31);
    const bool row_ok = i < r;
    // sorted rank i: row perm[i] of the eigensolver's output times vscale[i]
    const int vsrc = row_ok ? perm[static_cast<int64_t>(blk) * kD + i] : 0;
    const float vsc = row_ok ? vscale[static_cast<int64_t>(blk) * kD + i] : 0.f;
    const float *vrow = vt + static_cast<int64_t>(blk) * kD * kD + static_cast<int64_t>(vsrc) * kD;
    float v[8][8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
        float4 a = make_float4(0.f, 0.f, 0.f, 0.f), b = a;
        if (row_ok) {
            a = *reinterpret_cast<const float4 *>(vrow + 16 * ks + 8 * (lane >> 5));
            b = *reinterpret_cast<const float4 *>(vrow + 16 * ks + 8 * (lane >> 5) + 4);
            a = make_float4(a.x * vsc, a.y * vsc, a.z * vsc, a.w * vsc);
            b = make_float4(b.x * vsc, b.y * vsc, b.z * vsc, b.w * vsc);
        }
        v[ks][0] = a.x; v[ks][1] = a.y; v[ks][2] = a.z; v[ks][3] = a.w;
        v[ks][4] = b.x; v[ks][5] = b.y; v[ks][6] = b.z; v[ks][7] = b.w;
        if constexpr (OUT == kF32)
            if (part == 0 && row_ok) {
                float4 *d4 = reinterpret_cast<float4 *>(Bb + (static_cast<int64_t>(i) * kD + 16 * ks + 8 * (lane >> 5)) * 4);
                d4[0] = a;
                d4[1] = b;
            }
    }
    if constexpr (OUT == kI4) store_b_i4(v, i, r, lane, part == 0 && row_ok, Bb);
    if constexpr (OUT == kI2) store_b_i2(v, i, r, lane, part == 0 && row_ok, Bb);
    u16x8_t fa[3][8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            uint16_t h, mm, l;
            split3_bf16(v[ks][e], h, mm, l);
            fa[0][ks][e] = h;
            fa[1][ks][e] = mm;
            fa[2][ks][e] = l;
        }

    const uint16_t *xp = x + (row0 ? row0[blk] : static_cast<int64_t>(blk) * T * row_stride) +
                         static_cast<int64_t>(t_begin) * row_stride;
    float *stg = stage[wave];
    stream_x_ring(xring, xp, row_stride, (t_end - t_begin) / 32, wave, lane,
                  [&](int t, const u16x8_t (&xc)[8]) __attribute__((always_inline)) {
        if (!active) return;
        const int t0 = t_begin + 32 * t;
        f32x16_t acc = zero16(), acc1 = zero16();
#pragma unroll
        for (int ks = 0; ks < 8; ks += 2)
#pragma unroll
            for (int s = 0; s < 3; ++s) {
                acc = mfma32x32x16(fa[s][ks], xc[ks], acc);
                acc1 = mfma32x32x16(fa[s][ks + 1], xc[ks + 1], acc1);
            }
        acc += acc1;
        // acc[q]: rank row 8 (q / 4) + 4 (lane / 32) + q % 4 of this wave, token lane % 32
        const int g = t & 1;  // run of the 64-token flush (the part has an even number of tiles)
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const int row = 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);
            stg[row * kRowP + g * kRunP + (lane & 31)] = acc[q];
        }
        if (g == 1) {
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            const int tok0 = t0 - 32;  // first token of the flush
            if constexpr (OUT == kF32) {
                // 32 rows x 64 tokens: 16 lanes per row, 16-byte pieces of 4 tokens
#pragma unroll
                for (int rr = 0; rr < 32; rr += 4) {
                    const int row = rr + (lane >> 4), piece = lane & 15;
                    const int ir = 32 * wave + row;
                    if (ir < r)
                        *reinterpret_cast<float4 *>(Ab + (static_cast<int64_t>(ir) * T + tok0 + 4 * piece) * 4) =
                            *reinterpret_cast<const float4 *>(stg + row * kRowP + (piece >> 3) * kRunP + 4 * (piece & 7));
                }
            } else if constexpr (OUT == kI2) {
                // 64 runs (32 rows x 2), one per lane: 8 code bytes and a scale each
                const int row = lane >> 1, gg = lane & 1;
                const int ir = 32 * wave + row;
                const float4 *src = reinterpret_cast<const float4 *>(stg + row * kRowP + gg * kRunP);
                float m = 0.f;
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const float4 a = src[k];
                    m = fmaxf(fmaxf(m, fmaxf(fabsf(a.x), fabsf(a.y))), fmaxf(fabsf(a.z), fabsf(a.w)));
                }
                const float sA = __fdiv_rn(m, 3.f);
                uint32_t w[2] = {0u, 0u};
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const float4 a = src[k];
                    const float f[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) w[k >> 2] |= code2(f[e], sA) << (2 * (4 * (k & 3) + e));
                }
                if (ir < r) {
                    *reinterpret_cast<uint2 *>(Ab + static_cast<int64_t>(ir) * (T / 4) + (tok0 + 32 * gg) / 4) =
                        make_uint2(w[0], w[1]);
                    *reinterpret_cast<float *>(Ab + static_cast<int64_t>(r) * (T / 4) +
                                               (static_cast<int64_t>(ir) * (T / kI4Group) + tok0 / kI4Group + gg) * 4) = sA;
                }
            } else {
                // 64 runs (32 rows x 2), one per lane
                const int row = lane >> 1, gg = lane & 1;
                const int ir = 32 * wave + row;
                const float4 *src = reinterpret_cast<const float4 *>(stg + row * kRowP + gg * kRunP);
                float m = 0.f;
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const float4 a = src[k];
                    m = fmaxf(fmaxf(m, fmaxf(fabsf(a.x), fabsf(a.y))), fmaxf(fabsf(a.z), fabsf(a.w)));
                }
                const float sA = __fdiv_rn(m, 7.f);
                // code = rint(x / s) with the IEEE quotient.  x * fl(1 / s) is within
                // 1e-6 of x / s (|x / s| <= 7.5), and so is fl(x / s): unless x * (1 / s)
                // lies within 1e-5 of a half-integer, both round to the same code.
                // A run with such an element (rare) takes every code from the quotient.
                const float inv = sA > 0.f ? __fdiv_rn(1.f, sA) : 0.f;
                uint32_t w[4] = {0u, 0u, 0u, 0u};
                bool near = false;
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const float4 a = src[k];
                    const float f[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float qf = f[e] * inv;
                        float c = rintf(qf);
                        near |= fabsf(qf - c) > 0.5f - 1e-5f;
                        c = fminf(fmaxf(c, -7.f), 7.f);
                        w[k >> 1] |= (static_cast<uint32_t>(static_cast<int>(c)) & 0xfu) << (4 * (4 * (k & 1) + e));
                    }
                }
                if (near) {
#pragma unroll
                    for (int k = 0; k < 4; ++k) w[k] = 0u;
#pragma unroll
                    for (int k = 0; k < 8; ++k) {
                        const float4 a = src[k];
                        const float f[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const float c = fminf(fmaxf(rintf(__fdiv_rn(f[e], sA)), -7.f), 7.f);
                            w[k >> 1] |= (static_cast<uint32_t>(static_cast<int>(c)) & 0xfu) << (4 * (4 * (k & 1) + e));
                        }
                    }
                }
                if (ir < r) {
                    *reinterpret_cast<uint4 *>(Ab + static_cast<int64_t>(ir) * (T / 2) + (tok0 + 32 * gg) / 2) =
                        make_uint4(w[0], w[1], w[2], w[3]);
                    *reinterpret_cast<float *>(Ab + static_cast<int64_t>(r) * (T / 2) +
                                               (static_cast<int64_t>(ir) * (T / kI4Group) + tok0 / kI4Group + gg) * 4) = sA;
                }
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }
    });
}

}  // namespace

hipError_t launch_project(const void *x, int x_type, const int64_t *row0, int64_t row_stride,
                          int block_len, int n_blocks, const float *vt, const int32_t *perm,
                          const float *vscale, const int32_t *rank,
                          const int64_t *a_off, const int64_t *b_off, void *arena, int out_type,
                          float *a_scale, float *b_scale, hipStream_t st) {
    if (n_blocks <= 0) return hipSuccess;
    if (x_type == kBF16 && out_type == kBF16) {
        const dim3 g(static_cast<unsigned>(n_blocks), static_cast<unsigned>((block_len + kPartBF - 1) / kPartBF));
        hipLaunchKernelGGL(project_bf16_kernel, g, dim3(256), 0, st, static_cast<const uint16_t *>(x), row0,
                           row_stride, block_len, vt, perm, vscale, rank, a_off, b_off, static_cast<uint8_t *>(arena));
        return hipGetLastError();
    }
    if (x_type == kBF16 && (out_type == kF32 || out_type == kI4 || out_type == kI2)) {
        const dim3 g(static_cast<unsigned>(n_blocks), static_cast<unsigned>((block_len + kPartBF - 1) / kPartBF));
        const uint16_t *xb = static_cast<const uint16_t *>(x);
        uint8_t *ar = static_cast<uint8_t *>(arena);
        if (out_type == kF32)
            hipLaunchKernelGGL(project_split_kernel<kF32>, g, dim3(256), 0, st, xb, row0, row_stride, block_len, vt,
                               perm, vscale, rank, a_off, b_off, ar);
        else if (out_type == kI4)
            hipLaunchKernelGGL(project_split_kernel<kI4>, g, dim3(256), 0, st, xb, row0, row_stride, block_len, vt,
                               perm, vscale, rank, a_off, b_off, ar);
        else
            hipLaunchKernelGGL(project_split_kernel<kI2>, g, dim3(256), 0, st, xb, row0, row_stride, block_len, vt,
                               perm, vscale, rank, a_off, b_off, ar);
        return hipGetLastError();
    }
    const dim3 grid(static_cast<unsigned>(n_blocks),
                    static_cast<unsigned>((block_len + kTokensPerWG - 1) / kTokensPerWG));
    uint8_t *ar = static_cast<uint8_t *>(arena);
#define MILO_PROJECT(NX, OUT)                                                                     \
    hipLaunchKernelGGL((project_kernel<NX, OUT>), grid, dim3(256), 0, st, x, row0, row_stride,    \
                       block_len, vt, perm, vscale, rank, a_off, b_off, ar, a_scale, b_scale)
    if (x_type == kF32 && out_type == kF32)
        MILO_PROJECT(3, kF32);
    else if (x_type == kBF16 && out_type == kI8)
        MILO_PROJECT(1, kI8);
    else if (x_type == kF32 && out_type == kBF16)
        MILO_PROJECT(3, kBF16);
    else if (x_type == kF32 && out_type == kI4)
        MILO_PROJECT(3, kI4);
    else if (x_type == kF32 && out_type == kI2)
        MILO_PROJECT(3, kI2);
    else
        MILO_PROJECT(3, kI8);
#undef MILO_PROJECT
    return hipGetLastError();
}

}  // namespace milo
