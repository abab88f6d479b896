// Decode attention over compressed KV blocks (one layer, one decode step).
//
// For every selected block the kernel rebuilds key tiles from the factors,
// K_hat^T = B_k^T A_k^T, applies RoPE at the tokens' absolute positions, forms
// the logits of the G query heads that share the KV head, runs an online
// softmax, and accumulates the value side in rank space, u += P A_v, applying
// B_v once per split: o = u B_v ((p A_v) B_v, so V is never rebuilt).  The
// retrieved blocks' factors are rebuilt right before attention (evolve.pub
// review of arXiv 2609.29913, Summary; FAQ); keys were compressed before RoPE
// (ai4snews digest, Figure 1 caption), so RoPE is applied to rebuilt keys.
//
// Work split (flash-decoding style): one workgroup per (sequence, KV head,
// selected block, token split); the partial (max, sum, unnormalised output)
// triples are merged by decode_combine_kernel with log-sum-exp weights.  The
// uncompressed recent tail runs through the same code with identity factors
// (keys and values read directly, token-major).
//
// RoPE: logit_t = (R_{pq} q) . (R_{p0+t} k_t) = (R_{pq-p0} q) . (R_t k_t) for a
// 32-token tile starting at position p0.  Each tile's rotated queries are
// precomputed per workgroup (angles reduced in fp64), and R_t for t < 32 is a
// per-lane register table, so per token only the key rotation by R_t remains.
//
// MFMA usage (bf16 in, fp32 accumulate; fp32 factors are split into two bf16
// terms, three products):
//   K^T tile   v_mfma_f32_32x32x16_bf16, M = head dim j, N = token, K = rank;
//              B_k fragments live in LDS, A_k^T (rank-major in the arena) is
//              gathered 8 ranks x 1 token per lane straight from memory;
//   logits     32x32x16, M = query head (G <= 16 rows used), N = token,
//              K = head dim, in a k-order that matches the K^T accumulator;
//   P A_v      v_mfma_f32_16x16x32_bf16, M = query head, N = rank, K = token,
//              A_v^T read as 16-byte rows of 8 consecutive tokens.
#include <math.h>

#include "common.hpp"
#include "kernels.hpp"

namespace milo {
namespace {

constexpr int kTile = 32;
constexpr int kWaves = 4;
constexpr double kTwoPi = 6.283185307179586476925286766559;
constexpr float kLog2e = 1.4426950408889634f;

struct LdsLayout {
    int bk, qf, scratch, pt, alpha, kst, total;
};

__host__ __device__ inline int align16(int v) { return (v + 15) & ~15; }

// Staging pitch (bytes) of one 32-token rank row of an A_k tile: the row plus 8
// bytes, so rows 8 apart (the two lane halves of a transposed read) fall on
// disjoint LDS banks.  fp32 factors bypass the staging buffer.
__host__ __device__ inline int kst_pitch(int esize) { return esize == 4 ? 0 : 32 * esize + 8; }

// All offsets in bytes.  scratch holds the prologue tables (RoPE table, the
// queries, theta) and is reused for the end-of-split merge.
__host__ __device__ inline LdsLayout lds_layout(int ns, int n_tiles, int G, bool tail, int esize) {
    LdsLayout L;
    const int bk = tail ? 0 : ns * 4 * 8 * 64 * 8 * 2;
    const int qf = ns * n_tiles * 8 * 2 * G * 8 * 2;
    const int prologue = 32 * 64 * 8 + G * 128 * 4 + 64 * 8;
    const int merge = kWaves * G * 128 * 4 + 2 * kWaves * 16 * 4;
    const int scratch = prologue > merge ? prologue : merge;
    const int kst = tail ? 0 : kWaves * 128 * kst_pitch(esize);
    L.bk = 0;
    L.qf = align16(L.bk + bk);
    L.scratch = align16(L.qf + qf);
    L.pt = align16(L.scratch + scratch);
    L.alpha = align16(L.pt + kWaves * ns * 16 * 32 * 2);
    L.kst = align16(L.alpha + 128 * 4);  // alpha per wave (64 floats), or 128 B-row scales
    L.total = align16(L.kst + kst);
    return L;
}

// Order this wave's LDS writes before its later LDS reads of other lanes' data
// (LDS executes a wave's operations in order; the fences stop the compiler from
// reordering across this point).
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Copy nbytes (a multiple of 16) from global memory to LDS in rounds of 4 KiB
// per 4 chunks per thread: each round issues all its loads before any store.
__device__ __forceinline__ void copy_to_lds(uint8_t *dst, const uint8_t *src, int nbytes) {
    const int n = nbytes >> 4;
    for (int base = 0; base < n; base += 1024) {
        uint4 v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            v[i] = reinterpret_cast<const uint4 *>(src)[min(base + static_cast<int>(threadIdx.x) + 256 * i, n - 1)];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = base + threadIdx.x + 256 * i;
            if (c < n) reinterpret_cast<uint4 *>(dst)[c] = v[i];
        }
    }
}

template <int F>
__device__ __forceinline__ float load_elem(const uint8_t *base, int64_t idx) {
    if constexpr (F == kF32) return reinterpret_cast<const float *>(base)[idx];
    else if constexpr (F == kBF16) return bf16_bits_to_f32(reinterpret_cast<const uint16_t *>(base)[idx]);
    else return static_cast<float>(reinterpret_cast<const int8_t *>(base)[idx]);
}

// Split an fp32 value into NS bf16 terms (NS = 1: round; NS = 2: hi + lo).
template <int NS>
__device__ __forceinline__ void to_terms(float v, uint16_t (&t)[2]) {
    t[0] = f32_to_bf16_bits(v);
    if constexpr (NS == 2) t[1] = f32_to_bf16_bits(v - bf16_bits_to_f32(t[0]));
}

template <int F, bool TAIL>
__global__ __launch_bounds__(256) void decode_partial_kernel(const DecodeParams p) {
    constexpr int NS = (F == kF32) ? 2 : 1;
    extern __shared__ __align__(16) uint8_t lds[];
    const int G = p.group;
    const int n_tiles = p.split_len / kTile;
    const int tiles_per_wave = n_tiles / kWaves;
    constexpr int ES = (F == kF32) ? 4 : (F == kBF16 ? 2 : 1);
    const LdsLayout L = lds_layout(NS, n_tiles, G, TAIL, ES);
    uint16_t *bk = reinterpret_cast<uint16_t *>(lds + L.bk);
    uint16_t *qf = reinterpret_cast<uint16_t *>(lds + L.qf);
    float2 *rope_tab = reinterpret_cast<float2 *>(lds + L.scratch);
    float *qs = reinterpret_cast<float *>(lds + L.scratch + 32 * 64 * 8);
    double *theta = reinterpret_cast<double *>(lds + L.scratch + 32 * 64 * 8 + G * 128 * 4);
    float *us = reinterpret_cast<float *>(lds + L.scratch);            // merge (aliases the tables)
    float *wm = us + kWaves * G * 128;
    float *wl = wm + kWaves * 16;
    uint16_t *pt = reinterpret_cast<uint16_t *>(lds + L.pt);
    float *alpha_s = reinterpret_cast<float *>(lds + L.alpha);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int tl_ = lane & 31, hf_ = lane >> 5;
    const int s = blockIdx.z, h = blockIdx.y, sp = blockIdx.x;
    const int Hkv = p.n_kv_heads;
    const int T = p.block_len;

    // ---- which tokens this workgroup covers
    int split_index, tok0 = 0, valid = 0, fid = -1, rk = 0, rv = 0;
    int64_t pos0 = 0;
    if constexpr (!TAIL) {
        const int e = sp / p.block_splits, c = sp - e * p.block_splits;
        split_index = sp;
        int b = e;
        bool ok = true;
        if (p.sel_ptr) {
            const int beg = p.sel_ptr[s], cnt = p.sel_ptr[s + 1] - beg;
            ok = e < cnt;
            if (ok) b = p.sel_blk[beg + e];
            ok = ok && b >= 0 && b < p.blocks_per_seq;
        }
        if (ok) {
            fid = (s * Hkv + h) * p.blocks_per_seq + b;
            rk = p.k_rank[fid];
            rv = p.v_rank[fid];
            tok0 = c * p.split_len;
            pos0 = static_cast<int64_t>(b) * T + tok0;
            valid = p.split_len;
        }
    } else {
        split_index = p.n_sel * p.block_splits + sp;
        tok0 = sp * p.split_len;
        const int len = min(p.tail_len[s], p.tail_cap);  // never read past the tail buffer
        valid = min(max(len - tok0, 0), p.split_len);
        pos0 = p.tail_pos0[s] + tok0;
    }
    const int64_t pidx = static_cast<int64_t>(s * Hkv + h) * p.n_splits + split_index;
    float *ml = p.part_ml + pidx * G * 2;
    float *po = p.part_o + pidx * G * kD;
    if (valid == 0) {
        if (tid < G) {
            ml[2 * tid] = -INFINITY;
            ml[2 * tid + 1] = 0.f;
        }
        return;
    }

    // ---- prologue: theta, queries, in-tile RoPE table, rotated query fragments
    if (tid < 64) theta[tid] = exp2(-(2.0 * tid / 128.0) * log2(p.rope_base));
    {
        // the G query heads of this KV head are consecutive rows of q
        const int64_t q0 = (static_cast<int64_t>(s) * p.n_q_heads + h * G) * kD;
        float qv[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int e = min(tid + 256 * i, G * kD - 1);
            qv[i] = p.q_type == kF32 ? static_cast<const float *>(p.q)[q0 + e]
                                     : bf16_bits_to_f32(static_cast<const uint16_t *>(p.q)[q0 + e]);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if (tid + 256 * i < G * kD) qs[tid + 256 * i] = qv[i];
    }
    __syncthreads();
    for (int e = tid; e < 32 * 64; e += 256) {
        const int t = e >> 6, j = e & 63;
        float sn, cs;  // angle < 32 rad: fp32 sincos is accurate after its own reduction
        sincosf(static_cast<float>(static_cast<double>(t) * theta[j]), &sn, &cs);
        rope_tab[e] = make_float2(cs, sn);
    }
    const int qf_term = n_tiles * 8 * 2 * G * 8;  // elements per bf16 term
    const int64_t qpos = p.q_pos[s];
    for (int e = tid; e < n_tiles * 64; e += 256) {
        const int tl = e >> 6, j = e & 63;
        double a = static_cast<double>(qpos - (pos0 + tl * kTile)) * theta[j];
        a -= kTwoPi * rint(a / kTwoPi);  // exact enough in fp64 for positions < 2^40
        float snf, csf;
        sincosf(static_cast<float>(a), &snf, &csf);
        const double sn = snf, cs = csf;
#pragma unroll 1
        for (int g = 0; g < G; ++g) {
            const double x1 = qs[g * kD + j], x2 = qs[g * kD + j + 64];
            const float y[2] = {static_cast<float>(x1 * cs - x2 * sn),
                                static_cast<float>(x1 * sn + x2 * cs)};
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const int jj = j + 64 * half;
                const int jt = jj >> 5, rem = jj & 31;
                const int kk = 2 * jt + (rem >> 4);
                const int hf = (rem >> 2) & 1;
                const int slot = 4 * ((rem >> 3) & 1) + (rem & 3);
                const int idx = (((tl * 8 + kk) * 2 + hf) * G + g) * 8 + slot;
                uint16_t tv[2];
                to_terms<NS>(y[half], tv);
#pragma unroll
                for (int st = 0; st < NS; ++st) qf[st * qf_term + idx] = tv[st];
            }
        }
    }
    int KS = 0;
    const uint8_t *Ak = nullptr, *Av = nullptr, *Bv = nullptr;
    if constexpr (!TAIL) {
        KS = (rk + 15) >> 4;
        Ak = p.k_arena + p.k_aoff[fid];
        Av = p.v_arena + p.v_aoff[fid];
        Bv = p.v_arena + p.v_boff[fid];
        const uint8_t *Bk = p.k_arena + p.k_boff[fid];
        if constexpr (F != kF32) {
            // rows of B_k (and their INT8 scales) -> LDS, then into MFMA fragment order
            uint8_t *tmp = lds + L.kst;
            float *bsc = reinterpret_cast<float *>(lds + L.alpha);  // free until the main loop
            copy_to_lds(tmp, Bk, rk * kD * ES);
            if constexpr (F == kI8)
                if (tid < rk) bsc[tid] = p.k_bscale[static_cast<int64_t>(fid) * kD + tid];
            __syncthreads();
            for (int q = tid; q < 4 * 8 * 64; q += 256) {
                const int ln = q & 63, ks = (q >> 6) & 7, jt = q >> 9;
                if (ks >= KS) continue;
                const int j = 32 * jt + (ln & 31), r0 = 16 * ks + 8 * (ln >> 5);
                u16x8_t ch;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int r = r0 + e;
                    float v = 0.f;
                    if (r < rk) {
                        if constexpr (F == kBF16)
                            v = bf16_bits_to_f32(reinterpret_cast<const uint16_t *>(tmp)[r * kD + j]);
                        else
                            v = static_cast<float>(reinterpret_cast<const int8_t *>(tmp)[r * kD + j]) * bsc[r];
                    }
                    ch[e] = f32_to_bf16_bits(v);
                }
                *reinterpret_cast<u16x8_t *>(bk + q * 8) = ch;
            }
            __syncthreads();  // the staging area is reused for A_k tiles
        } else {
            for (int e = tid; e < KS * 16 * kD; e += 256) {
                const int r = e >> 7, j = e & 127;
                const float v = r < rk ? load_elem<F>(Bk, e) : 0.f;
                const int jt = j >> 5, ln = (j & 31) + 32 * ((r >> 3) & 1);
                const int idx = ((jt * 8 + (r >> 4)) * 64 + ln) * 8 + (r & 7);
                uint16_t tv[2];
                to_terms<NS>(v, tv);
#pragma unroll
                for (int st = 0; st < NS; ++st) bk[st * (4 * 8 * 64 * 8) + idx] = tv[st];
            }
        }
    }
    // P^T staging rows g >= G stay zero for the whole split.
    for (int e = tid; e < kWaves * NS * 16 * 32; e += 256) pt[e] = 0;
    __syncthreads();
    float rc[2][16], rsn[2][16];
#pragma unroll
    for (int jt = 0; jt < 2; ++jt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int j = 32 * jt + 8 * (i >> 2) + 4 * hf_ + (i & 3);
            const float2 v = rope_tab[tl_ * 64 + j];
            rc[jt][i] = v.x;
            rsn[jt][i] = v.y;
        }

    // ---- main loop over this wave's tiles (contiguous tiles per wave)
    float m_run[8], l_run[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        m_run[i] = -INFINITY;
        l_run[i] = 0.f;
    }
    f32x4_t u[8];
#pragma unroll
    for (int n = 0; n < 8; ++n) u[n] = zero4();
    const int NTU = TAIL ? 8 : (rv + 15) >> 4;
    const float lscale = p.softmax_scale * kLog2e;
    uint16_t *my_pt = pt + wave * NS * 16 * 32;
    const int tile0 = wave * tiles_per_wave;

    // A_k tiles (bf16 / int8): 16-byte coalesced loads of LPR lanes per rank row,
    // staged rank-major in this wave's LDS buffer and read back transposed
    // (8 ranks of one token per lane).  Rows past rk reuse row rk - 1 (finite
    // values; their B_k fragment rows are zero).
    constexpr int RB = 32 * ES;                 // bytes of one rank row of a tile
    constexpr int LPR = RB / 16 > 0 ? RB / 16 : 1;
    constexpr int RPI = 64 / LPR;               // rank rows per load instruction
    constexpr int NI = 128 / RPI;               // load instructions for 128 ranks
    constexpr int KP = (F == kF32) ? 16 : 32 * ES + 8;  // staging pitch (bytes)
    uint8_t *kst = lds + L.kst + wave * 128 * KP;
    const int rk_pad = KS * 16;
    uint4 kraw[F == kF32 ? 1 : NI];
    auto load_k = [&](int tl) {
        if constexpr (F != kF32 && !TAIL) {
            const int tt0 = tok0 + tl * kTile;
#pragma unroll
            for (int c = 0; c < NI; ++c)
                if (c * RPI < rk_pad) {
                    const int r = min(c * RPI + lane / LPR, rk - 1);
                    kraw[c] = *reinterpret_cast<const uint4 *>(
                        Ak + (static_cast<int64_t>(r) * T + tt0) * ES + (lane % LPR) * 16);
                }
        }
    };
    // A_v fragments for P A_v (16x16x32 B operand): rank column 16 n + lane % 16,
    // tokens tb .. tb + 7.  bf16: one 16-byte load; int8: 8 bytes; fp32: 32 bytes.
    u16x8_t vraw[F == kF32 ? 1 : 8];
    auto load_v = [&](int tl) {
        if constexpr (F != kF32 && !TAIL) {
            const int tb = tok0 + tl * kTile + 8 * (lane >> 4);
#pragma unroll
            for (int n = 0; n < 8; ++n)
                if (n < NTU) {
                    const int col = min(16 * n + (lane & 15), rv - 1);
                    if constexpr (F == kBF16) {
                        vraw[n] = *reinterpret_cast<const u16x8_t *>(
                            reinterpret_cast<const uint16_t *>(Av) + static_cast<int64_t>(col) * T + tb);
                    } else {
                        const uint2 w = *reinterpret_cast<const uint2 *>(Av + static_cast<int64_t>(col) * T + tb);
                        vraw[n][0] = static_cast<uint16_t>(w.x & 0xffff);
                        vraw[n][1] = static_cast<uint16_t>(w.x >> 16);
                        vraw[n][2] = static_cast<uint16_t>(w.y & 0xffff);
                        vraw[n][3] = static_cast<uint16_t>(w.y >> 16);
                    }
                }
        }
    };
    // Pipeline: the staging buffer holds tile it while its keys are rebuilt; the
    // A_k registers already hold tile it + 1 and A_v registers tile it.  Each
    // wait therefore covers loads issued a whole tile earlier.
    auto stage_k = [&]() {
        if constexpr (F != kF32 && !TAIL) {
#pragma unroll
            for (int c = 0; c < NI; ++c)
                if (c * RPI < rk_pad) {
                    uint8_t *dst = kst + (c * RPI + lane / LPR) * KP + (lane % LPR) * 16;
                    reinterpret_cast<uint2 *>(dst)[0] = make_uint2(kraw[c].x, kraw[c].y);
                    reinterpret_cast<uint2 *>(dst)[1] = make_uint2(kraw[c].z, kraw[c].w);
                }
            wave_lds_sync();
        }
    };
    load_k(tile0);
    stage_k();
    load_v(tile0);
    if (tiles_per_wave > 1) load_k(tile0 + 1);

    for (int it = 0; it < tiles_per_wave; ++it) {
        const int tl = tile0 + it;
        const int tloc = tl * kTile;           // offset within the split
        const int t = tok0 + tloc + tl_;       // this lane's token (block- or tail-local)
        const bool tok_ok = tloc + tl_ < valid;

        // ---- K^T tile: kacc[jt][i] = k_hat[t][32 jt + 8 (i/4) + 4 hf + i%4]
        f32x16_t kacc[4];
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) kacc[jt] = zero16();
        if constexpr (!TAIL) {
            for (int ks = 0; ks < KS; ++ks) {
                u16x8_t af[NS];
                if constexpr (F == kBF16) {
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        af[0][e] = *reinterpret_cast<const uint16_t *>(kst + (16 * ks + 8 * hf_ + e) * KP + tl_ * 2);
                } else if constexpr (F == kI8) {
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        af[0][e] = f32_to_bf16_bits(static_cast<float>(
                            *reinterpret_cast<const int8_t *>(kst + (16 * ks + 8 * hf_ + e) * KP + tl_)));
                } else {
                    float v[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int r = 16 * ks + 8 * hf_ + e;
                        v[e] = load_elem<F>(Ak, static_cast<int64_t>(min(r, rk - 1)) * T + t);
                        if (r >= rk) v[e] = 0.f;
                    }
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        uint16_t tv[2];
                        to_terms<NS>(v[e], tv);
#pragma unroll
                        for (int st = 0; st < NS; ++st) af[st][e] = tv[st];
                    }
                }
#pragma unroll
                for (int jt = 0; jt < 4; ++jt) {
#pragma unroll
                    for (int sa = 0; sa < NS; ++sa) {
                        const u16x8_t bf = *reinterpret_cast<const u16x8_t *>(
                            bk + sa * (4 * 8 * 64 * 8) + ((jt * 8 + ks) * 64 + lane) * 8);
#pragma unroll
                        for (int sb = 0; sb < NS; ++sb)
                            if (sa + sb < NS) kacc[jt] = mfma32x32x16(bf, af[sb], kacc[jt]);
                    }
                }
            }
        } else {
            const int tc = min(t, tok0 + valid - 1);  // clamped: masked lanes read a valid row
            const int64_t row = ((static_cast<int64_t>(s) * Hkv + h) * p.tail_cap + tc) * kD;
#pragma unroll
            for (int jt = 0; jt < 4; ++jt)
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    const int j0 = 32 * jt + 8 * q4 + 4 * hf_;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        kacc[jt][4 * q4 + e] =
                            load_elem<F>(static_cast<const uint8_t *>(p.tail_k), row + j0 + e);
                }
        }
        // RoPE by the in-tile offset (pairs j, j + 64 sit in kacc[jt], kacc[jt + 2])
#pragma unroll
        for (int jt = 0; jt < 2; ++jt)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float k1 = kacc[jt][i], k2 = kacc[jt + 2][i];
                kacc[jt][i] = k1 * rc[jt][i] - k2 * rsn[jt][i];
                kacc[jt + 2][i] = k1 * rsn[jt][i] + k2 * rc[jt][i];
            }
        // logits S[g][t] over 8 k-steps of 16 head dims
        f32x16_t S = zero16();
        const bool q_lane = tl_ < G;
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
            const int jt = kk >> 1, h2 = kk & 1;
            u16x8_t kf[NS];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                uint16_t tv[2];
                to_terms<NS>(kacc[jt][8 * h2 + e], tv);
#pragma unroll
                for (int st = 0; st < NS; ++st) kf[st][e] = tv[st];
            }
#pragma unroll
            for (int sa = 0; sa < NS; ++sa) {
                u16x8_t qv;
                if (q_lane)
                    qv = *reinterpret_cast<const u16x8_t *>(
                        qf + sa * qf_term + (((tl * 8 + kk) * 2 + hf_) * G + tl_) * 8);
                else
#pragma unroll
                    for (int e = 0; e < 8; ++e) qv[e] = 0;
#pragma unroll
                for (int sb = 0; sb < NS; ++sb)
                    if (sa + sb < NS) S = mfma32x32x16(qv, kf[sb], S);
            }
        }
        // online softmax (log2 domain); S[i] holds head g = 8 (i/4) + 4 hf + i%4, token tl_
        float tscale = lscale;
        float vscale = 1.f;
        if constexpr (F == kI8 && !TAIL) {
            tscale *= p.k_ascale[static_cast<int64_t>(fid) * T + t];
            vscale = p.v_ascale[static_cast<int64_t>(fid) * T + t];
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int g = 8 * (i >> 2) + 4 * hf_ + (i & 3);
            const float x = tok_ok ? S[i] * tscale : -INFINITY;
            const float mt = half_max(x);
            const float mn = fmaxf(m_run[i], mt);
            const bool none = (mn == -INFINITY);
            const float alpha = none ? 1.f : exp2f(m_run[i] - mn);
            const float pr = none ? 0.f : exp2f(x - mn);
            l_run[i] = l_run[i] * alpha + half_sum(pr);
            m_run[i] = mn;
            if (g < G) {
                uint16_t tv[2];
                to_terms<NS>(pr * vscale, tv);
#pragma unroll
                for (int st = 0; st < NS; ++st) my_pt[(st * 16 + g) * 32 + tl_] = tv[st];
                if (tl_ == 0) alpha_s[wave * 16 + g] = alpha;
            }
        }
        wave_lds_sync();
        // u = u * alpha + P A_v   (u rows: g = 4 (lane/16) + i, columns: rank 16 n + lane%16)
        {
            const int g0 = 4 * (lane >> 4);
            float al[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) al[i] = (g0 + i < G) ? alpha_s[wave * 16 + g0 + i] : 1.f;
            u16x8_t pf[NS];
#pragma unroll
            for (int st = 0; st < NS; ++st)
                pf[st] = *reinterpret_cast<const u16x8_t *>(my_pt + (st * 16 + (lane & 15)) * 32 + 8 * (lane >> 4));
            const int tb = tok0 + tloc + 8 * (lane >> 4);  // first of this lane's 8 tokens
#pragma unroll
            for (int n = 0; n < 8; ++n) {
                if (n < NTU) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) u[n][i] *= al[i];
                    const int col = 16 * n + (lane & 15);
                    u16x8_t vf[NS];
                    if constexpr (!TAIL && F == kBF16) {
                        vf[0] = vraw[n];
                        if (col >= rv)
#pragma unroll
                            for (int e = 0; e < 8; ++e) vf[0][e] = 0;
                    } else if constexpr (!TAIL && F == kI8) {
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const int8_t c8 = static_cast<int8_t>((vraw[n][e >> 1] >> (8 * (e & 1))) & 0xff);
                            vf[0][e] = col < rv ? f32_to_bf16_bits(static_cast<float>(c8)) : 0;
                        }
                    } else if constexpr (!TAIL) {
                        const int cc = min(col, rv - 1);
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            uint16_t tv[2];
                            const float v = col < rv ? load_elem<F>(Av, static_cast<int64_t>(cc) * T + tb + e) : 0.f;
                            to_terms<NS>(v, tv);
#pragma unroll
                            for (int st = 0; st < NS; ++st) vf[st][e] = tv[st];
                        }
                    } else {
                        const int64_t rowb = (static_cast<int64_t>(s) * Hkv + h) * p.tail_cap;
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const bool ok = tb + e - tok0 < valid;
                            const int te = ok ? tb + e : tok0;
                            float v = load_elem<F>(static_cast<const uint8_t *>(p.tail_v), (rowb + te) * kD + col);
                            if (!ok) v = 0.f;
                            uint16_t tv[2];
                            to_terms<NS>(v, tv);
#pragma unroll
                            for (int st = 0; st < NS; ++st) vf[st][e] = tv[st];
                        }
                    }
#pragma unroll
                    for (int sa = 0; sa < NS; ++sa)
#pragma unroll
                        for (int sb = 0; sb < NS; ++sb)
                            if (sa + sb < NS) u[n] = mfma16x16x32(pf[sa], vf[sb], u[n]);
                }
            }
        }
        if (it + 1 < tiles_per_wave) {
            wave_lds_sync();  // this tile's staged keys have been read
            stage_k();
            load_v(tl + 1);
            if (it + 2 < tiles_per_wave) load_k(tl + 2);
        }
    }

    // ---- merge the four waves and apply B_v
    __syncthreads();  // the scratch region (RoPE table, queries) is dead from here on
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int g = 8 * (i >> 2) + 4 * hf_ + (i & 3);
        if (g < G && tl_ == 0) {
            wm[wave * 16 + g] = m_run[i];
            wl[wave * 16 + g] = l_run[i];
        }
    }
#pragma unroll
    for (int n = 0; n < 8; ++n)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int g = 4 * (lane >> 4) + i;
            if (n < NTU && g < G) us[(wave * G + g) * kD + 16 * n + (lane & 15)] = u[n][i];
        }
    const uint8_t *bv_src = Bv;
    if constexpr (!TAIL && F != kF32) {
        // B_v rows (and INT8 scales) -> LDS; the A_k staging area is free now
        copy_to_lds(lds + L.kst, Bv, rv * kD * ES);
        if constexpr (F == kI8)
            if (tid < rv) reinterpret_cast<float *>(lds + L.alpha)[tid] = p.v_bscale[static_cast<int64_t>(fid) * kD + tid];
        bv_src = lds + L.kst;
    }
    __syncthreads();
    for (int e = tid; e < G * kD; e += 256) {
        const int g = e >> 7, j = e & 127;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) M = fmaxf(M, wm[w * 16 + g]);
        float coef[kWaves];
        float Lsum = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float mw = wm[w * 16 + g];
            coef[w] = (mw == -INFINITY) ? 0.f : exp2f(mw - M);
            Lsum += coef[w] * wl[w * 16 + g];
        }
        float o = 0.f;
        if constexpr (!TAIL) {
            for (int r = 0; r < rv; ++r) {
                float uw = 0.f;
#pragma unroll
                for (int w = 0; w < kWaves; ++w) uw += coef[w] * us[(w * G + g) * kD + r];
                float bv = load_elem<F>(bv_src, static_cast<int64_t>(r) * kD + j);
                if constexpr (F == kI8) bv *= reinterpret_cast<const float *>(lds + L.alpha)[r];
                o += uw * bv;
            }
        } else {
#pragma unroll
            for (int w = 0; w < kWaves; ++w) o += coef[w] * us[(w * G + g) * kD + j];
        }
        po[g * kD + j] = o;
        if (j == 0) {
            ml[2 * g] = M;
            ml[2 * g + 1] = Lsum;
        }
    }
}

// One workgroup per (sequence, query head): the split maxima and weights are
// computed by all threads in parallel, then thread j sums its output column.
template <int OT>
__global__ __launch_bounds__(128) void decode_combine_kernel(const DecodeParams p) {
    __shared__ float coef[1024];
    __shared__ float red[2];
    const int hq = blockIdx.x, s = blockIdx.y, tid = threadIdx.x;
    const int G = p.group;
    const int h = hq / G, g = hq - h * G;
    const int64_t base = static_cast<int64_t>(s * p.n_kv_heads + h) * p.n_splits;
    float num = 0.f, den_part = 0.f;
    // chunks of up to 1024 splits (the weights of one chunk fit in LDS)
    float M = -INFINITY;
    for (int sp = tid; sp < p.n_splits; sp += 128) M = fmaxf(M, p.part_ml[((base + sp) * G + g) * 2]);
    M = wave_max(M);
    if ((tid & 63) == 0) red[tid >> 6] = M;
    __syncthreads();
    M = fmaxf(red[0], red[1]);
    __syncthreads();
    for (int c0 = 0; c0 < p.n_splits; c0 += 1024) {
        const int cn = min(1024, p.n_splits - c0);
        for (int i = tid; i < cn; i += 128) {
            const float m = p.part_ml[((base + c0 + i) * G + g) * 2];
            const float c = (m == -INFINITY || M == -INFINITY) ? 0.f : exp2f(m - M);
            coef[i] = c;
            den_part += c * p.part_ml[((base + c0 + i) * G + g) * 2 + 1];
        }
        __syncthreads();
        for (int i = 0; i < cn; ++i) {
            const float c = coef[i];
            if (c != 0.f) num += c * p.part_o[((base + c0 + i) * G + g) * kD + tid];
        }
        __syncthreads();
    }
    den_part = wave_sum(den_part);
    if ((tid & 63) == 0) red[tid >> 6] = den_part;
    __syncthreads();
    const float den = red[0] + red[1];
    const float o = den > 0.f ? num / den : 0.f;
    const int64_t oi = (static_cast<int64_t>(s) * p.n_q_heads + hq) * kD + tid;
    if constexpr (OT == kF32)
        static_cast<float *>(p.out)[oi] = o;
    else
        static_cast<uint16_t *>(p.out)[oi] = f32_to_bf16_bits(o);
}

template <int F, bool TAIL>
hipError_t launch_partial(const DecodeParams &p, dim3 grid, hipStream_t st) {
    constexpr int NS = (F == kF32) ? 2 : 1;
    constexpr int ES = (F == kF32) ? 4 : (F == kBF16 ? 2 : 1);
    const LdsLayout L = lds_layout(NS, p.split_len / kTile, p.group, TAIL, ES);
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(decode_partial_kernel<F, TAIL>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, L.total);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((decode_partial_kernel<F, TAIL>), grid, dim3(256), L.total, st, p);
    return hipGetLastError();
}

}  // namespace

bool decode_split_fits(int f_type, int tail_type, bool has_tail, int G, int split) {
    constexpr int kMaxLds = 160 * 1024;
    const int esz = f_type == kF32 ? 4 : (f_type == kBF16 ? 2 : 1);
    const int ns = f_type == kF32 ? 2 : 1;
    if (lds_layout(ns, split / kTile, G, false, esz).total > kMaxLds) return false;
    if (has_tail) {
        const int tns = tail_type == kF32 ? 2 : 1;
        if (lds_layout(tns, split / kTile, G, true, tail_type == kF32 ? 4 : 2).total > kMaxLds) return false;
    }
    return true;
}

size_t decode_workspace_bytes(const DecodeParams &p) {
    const size_t n = static_cast<size_t>(p.batch) * p.n_kv_heads * p.n_splits * p.group;
    const size_t ml = (n * 2 * sizeof(float) + 255) / 256 * 256;
    return ml + n * kD * sizeof(float);
}

hipError_t launch_decode_blocks(const DecodeParams &p, hipStream_t st) {
    const dim3 grid(static_cast<unsigned>(p.n_sel * p.block_splits), static_cast<unsigned>(p.n_kv_heads),
                    static_cast<unsigned>(p.batch));
    if (p.f_type == kBF16) return launch_partial<kBF16, false>(p, grid, st);
    if (p.f_type == kI8) return launch_partial<kI8, false>(p, grid, st);
    return launch_partial<kF32, false>(p, grid, st);
}

hipError_t launch_decode_tail(const DecodeParams &p, hipStream_t st) {
    const dim3 grid(static_cast<unsigned>(p.tail_splits), static_cast<unsigned>(p.n_kv_heads),
                    static_cast<unsigned>(p.batch));
    if (p.tail_type == kBF16) return launch_partial<kBF16, true>(p, grid, st);
    return launch_partial<kF32, true>(p, grid, st);
}

hipError_t launch_decode_combine(const DecodeParams &p, hipStream_t st) {
    const dim3 cgrid(static_cast<unsigned>(p.n_q_heads), static_cast<unsigned>(p.batch));
    if (p.out_type == kF32)
        hipLaunchKernelGGL(decode_combine_kernel<kF32>, cgrid, dim3(128), 0, st, p);
    else
        hipLaunchKernelGGL(decode_combine_kernel<kBF16>, cgrid, dim3(128), 0, st, p);
    return hipGetLastError();
}

}  // namespace milo
