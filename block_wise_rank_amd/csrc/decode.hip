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
// Work split (flash-decoding style): one workgroup of 8 waves per (sequence,
// KV head, selected block, token split); wave w takes the 32-token tiles
// w, w + 8, ... of the split, so the 8 waves read neighbouring stretches of
// every factor row at once.  The partial (max, sum, unnormalised output)
// triples of the splits are merged by decode_combine_kernel with log-sum-exp
// weights.  The uncompressed recent tail runs through the same code with the
// keys and values read directly (token-major) and B_v = I.
//
// RoPE: logit_t = (R_{pq} q) . (R_{p0+t} k_t) = (R_{pq-p0} q) . (R_t k_t) for a
// tile starting at position p0.  A table of (cos, sin)((pq - p0) theta_j) per
// tile (angles reduced in fp64) rotates the queries, which stay in registers,
// at the start of each tile; a 32 x 64 table of (cos, sin)(t theta_j) rotates
// the rebuilt keys.
//
// MFMA usage: v_mfma_f32_16x16x32_bf16 throughout (bf16 in, fp32 accumulate;
// fp32 factors are split into two bf16 terms, three products).  Lane l = 16 c
// + n of a wave holds, in every accumulator, row 4 c + i (i < 4) of column n.
//   K^T tile  M = head dim, N = token, K = rank: B_k^T fragments were built in
//             LDS once per workgroup; A_k^T (rank-major in the arena) is staged
//             per wave in LDS (XOR-swizzled 16-byte chunks) and read back
//             8 ranks x 1 token per lane.
//   logits^T  M = token, N = query head, K = head dim.  The K^T accumulators
//             feed the A operand in place: k-slot e < 4 of k-step kk is head
//             dim 16 kk + 4 c + e, slot e >= 4 is dim 64 + 16 kk + 4 c + e - 4,
//             which also keeps each RoPE pair (j, j + 64) inside one lane.
//   u^T       M = rank, N = query head, K = token: the probabilities feed the
//             B operand in place (k-slot e < 4 is token 4 c + e, e >= 4 is
//             token 16 + 4 c + e - 4) and A_v^T rows are read as two 8-byte
//             pieces in the same token order.
// Every lane owns one query head (its column n) in the logits, the softmax
// state and u, so rescaling needs no communication; the tile maximum is
// reduced over the four lane groups with two shuffles.
#include <math.h>

#include "common.hpp"
#include "kernels.hpp"

namespace milo {
namespace {

constexpr int kTile = 32;
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kMaxLds = 160 * 1024;
constexpr int kMaxDevices = 64;
constexpr double kTwoPi = 6.283185307179586476925286766559;
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kUP = 132;   // pitch (floats) of per-head u rows in the merge
constexpr int kTVP = 264;  // pitch (bytes) of staged tail V rows (32 tokens x 128 dims)
// Row pitches of the in-tile RoPE table (float2) and of the queries (float): 528
// bytes, so the 16-byte reads of 8 consecutive rows fall on distinct banks.
constexpr int kRP = 66;
constexpr int kQP = 132;
// Grouped low-bit factors: 4- or 2-bit codes with an fp32 scale per 32
// consecutive elements of a rank row (codes of all rows first, then scales).
__host__ __device__ constexpr bool is_q(int f) { return f == kI4 || f == kI2; }
__host__ __device__ constexpr int qbits(int f) { return f == kI4 ? 4 : 2; }
// bytes one rank takes in a B part (d codes, then d / 32 scales)
__host__ __device__ constexpr int q_b_bytes(int f) { return kD * qbits(f) / 8 + 4 * (kD / kI4Group); }

// Quantised B_k: offset of its decoded bf16 rows in the staging area, past the
// raw codes and scales of up to 128 ranks (at most 80 bytes each)
constexpr int kBkRows4 = 128 * q_b_bytes(kI4);

__host__ __device__ constexpr int align16(int v) { return (v + 15) & ~15; }

// A_k staging pitch per rank row of a 32-token tile (bytes); fp32 factors are
// read straight from memory.
// 4- and 2-bit factors are dequantised into the bf16 layout as they are staged.
__host__ __device__ inline int stage_pitch(int f) { return (f == kBF16 || is_q(f)) ? 64 : (f == kI8 ? 40 : 0); }

struct LdsLayout {
    int ang, qs, bk, rope, base, stage, loop_end;      // loop phase
    int uw, mlw, uacc, merge_end;                       // merge phase (aliases the loop phase)
    int bvraw, bvrows;                                  // 4-bit B_v: codes, decoded rows
    int total;
};

// Merge-phase areas: per-wave u rows, per-wave (m, l), merged u
constexpr int kMergeEnd = align16(align16(align16(kWaves * 16 * kUP * 4) + kWaves * 16 * 2 * 4) + 16 * kUP * 4);
// Quantised B_v: its codes and scales (at most 128 x 80 bytes) land in the last
// 10 KiB of the staging area, the staging rows of waves 6 and 7; the decoded
// bf16 rows (128 x 256 bytes) go between the merge areas and them, which needs
// the staging area to start at least this far in
constexpr int kBvRaw = kWaves * 128 * 64 - 128 * q_b_bytes(kI4);
constexpr int kI4StageMin = kMergeEnd + 128 * kD * 2 - kBvRaw;

__host__ __device__ inline LdsLayout lds_layout(int f, int ns, int n_tiles, bool tail, int G) {
    LdsLayout L;
    L.ang = 0;
    L.qs = align16(L.ang + 64 * 8);
    L.bk = align16(L.qs + G * kQP * 4);  // the G query heads (lanes n >= G reuse head G - 1)
    L.rope = align16(L.bk + (tail ? 0 : ns * 8 * 4 * 64 * 16));
    L.base = align16(L.rope + 32 * kRP * 8);
    L.stage = align16(L.base + n_tiles * 64 * 8);
    if (is_q(f) && !tail && L.stage < kI4StageMin) L.stage = kI4StageMin;
    int stage = 0;
    if (!tail) stage = kWaves * 128 * stage_pitch(f);
    else if (f == kBF16) stage = kWaves * 32 * kTVP;
    // the B_k rows for the fragment build are staged in this area too
    const int bk_rows = (tail || f == kF32) ? 0 : (is_q(f) ? 128 * q_b_bytes(f) : 128 * kD * (f == kBF16 ? 2 : 1));
    if (stage < bk_rows) stage = bk_rows;
    L.loop_end = align16(L.stage + stage);
    L.uw = 0;
    L.mlw = align16(L.uw + kWaves * 16 * kUP * 4);
    L.uacc = align16(L.mlw + kWaves * 16 * 2 * 4);
    L.merge_end = align16(L.uacc + 16 * kUP * 4);
    L.bvraw = L.stage + kBvRaw;
    L.bvrows = L.stage > L.merge_end ? L.stage : L.merge_end;
    L.total = L.loop_end > L.merge_end ? L.loop_end : L.merge_end;
    return L;
}

__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// s_waitcnt immediate that waits until at most n vector memory operations of
// this wave are outstanding (expcnt and lgkmcnt left at their maxima).
constexpr int vmcnt_imm(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }

// c ? a : b for a condition uniform over the wave, as one scalar select (a
// select the compiler turned into branches would leave the number of memory
// operations in flight unknown on the joined path, and it would then wait for
// all of them).
__device__ __forceinline__ const uint8_t *pick_uniform(bool c, const void *a, const void *b) {
    const uint64_t x = c ? reinterpret_cast<uint64_t>(a) : reinterpret_cast<uint64_t>(b);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(x));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(x >> 32));
    return reinterpret_cast<const uint8_t *>(static_cast<uint64_t>(hi) << 32 | lo);
}

// Value, in units of its run's scale, of code k (0..7) of eight consecutive
// codes held in the low bits of w: a two's-complement nibble (4-bit), or the
// level 2c - 3 of a 2-bit code c.
template <int F>
__device__ __forceinline__ float qval(uint32_t w, int k) {
    if constexpr (F == kI4) return static_cast<float>(static_cast<int32_t>(w << (28 - 4 * k)) >> 28);
    else return static_cast<float>(static_cast<int>((w >> (2 * k)) & 3u) * 2 - 3);
}

// The 32 codes of one run starting at p as four words of eight codes each.
template <int F>
__device__ __forceinline__ void run_words(const uint8_t *p, uint32_t (&w4)[4]) {
    if constexpr (F == kI4) {
        const uint4 c = *reinterpret_cast<const uint4 *>(p);
        w4[0] = c.x; w4[1] = c.y; w4[2] = c.z; w4[3] = c.w;
    } else {
        const uint2 c = *reinterpret_cast<const uint2 *>(p);
        w4[0] = c.x & 0xffffu; w4[1] = c.x >> 16; w4[2] = c.y & 0xffffu; w4[3] = c.y >> 16;
    }
}

// A run of 32 codes (scale sc) -> 16 words of bf16 pairs, element order kept.
template <int F>
__device__ __forceinline__ void decode_run(const uint32_t (&w4)[4], float sc, uint32_t (&hw)[16]) {
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            hw[4 * c + e] = f32x2_to_bf16x2_bits(qval<F>(w4[c], 2 * e) * sc, qval<F>(w4[c], 2 * e + 1) * sc);
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

// 8 floats -> NS bf16 fragments
template <int NS>
__device__ __forceinline__ void frag_terms(const float (&v)[8], u16x8_t (&f)[NS]) {
    if constexpr (NS == 1) {
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
            const uint32_t w = f32x2_to_bf16x2_bits(v[e], v[e + 1]);
            f[0][e] = static_cast<uint16_t>(w & 0xffff);
            f[0][e + 1] = static_cast<uint16_t>(w >> 16);
        }
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            uint16_t t[2];
            to_terms<NS>(v[e], t);
            f[0][e] = t[0];
            f[1][e] = t[1];
        }
    }
}

// Byte offset of (rank row r, token t) in a bf16 A_k staging tile (64-byte
// rows): the two 16-token halves of a row swap places in rows with bit 1 set.
// A transposing read of one half-wave touches rows r0 .. r0 + 3 and r0 + 8 ..
// r0 + 11 (r0 a multiple of 4) x 32 bytes of one half; the swap spreads them
// over all 32 banks twice, the minimum for 256 bytes.
__device__ __forceinline__ int stage_off_bf16(int r, int t) {
    return r * 64 + ((((t >> 4) ^ ((r >> 1) & 1))) << 5) + ((t & 15) << 1);
}
__device__ __forceinline__ int stage_off_i8(int r, int t) {
    return r * 40 + ((((t >> 4) ^ ((r >> 4) & 1))) << 4) + (t & 15);
}

// One split's partial result (m, l, unnormalised o) of the G query heads of
// (sequence blockIdx.z, KV head blockIdx.y): split sp of the selected blocks,
// or of the uncompressed tail (TAIL; F is then the tail's element type).
template <int F, bool TAIL>
__device__ __forceinline__ void decode_partial(const DecodeParams &p, const int sp, uint8_t *lds) {
    constexpr int NS = (F == kF32) ? 2 : 1;
    constexpr int ES = (F == kF32) ? 4 : (F == kBF16 ? 2 : 1);  // 4- and 2-bit: see below
    constexpr int QRB = is_q(F) ? kTile * qbits(F) / 8 : 0;      // code bytes of a 32-token run
    const int G = p.group;
    const int n_tiles = p.split_len / kTile;
    const LdsLayout L = lds_layout(F, NS, n_tiles, TAIL, G);
    float2 *ang = reinterpret_cast<float2 *>(lds + L.ang);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c4 = lane >> 4, ln = lane & 15;
    const int s = blockIdx.z, h = blockIdx.y;
    const int Hkv = p.n_kv_heads;
    const int T = p.block_len;

    // ---- which tokens this workgroup covers
    int split_index, tok0 = 0, valid = 0, fid = -1, rk = 0, rv = 0;
    int64_t pos0 = 0, ka_off = 0, va_off = 0, kb_off = 0, vb_off = 0;
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
        // every metadata load is issued at once (index 0 stands in when the
        // selection entry is invalid; nothing is read through it then)
        const int fs = ok ? (s * Hkv + h) * p.blocks_per_seq + b : 0;
        const int rk_s = p.k_rank[fs], rv_s = p.v_rank[fs];
        ka_off = p.k_aoff[fs];
        va_off = p.v_aoff[fs];
        kb_off = p.k_boff[fs];
        vb_off = p.v_boff[fs];
        if (ok) {
            fid = fs;
            rk = rk_s;
            rv = rv_s;
            tok0 = c * p.split_len;
            pos0 = static_cast<int64_t>(b) * T + tok0;
            valid = p.split_len;
        }
    } else {
        split_index = p.n_sel * p.block_splits + sp;
        tok0 = sp * p.split_len;
        if (p.tail_seg_pos) {
            // segment m holds its first tail_seg_valid tokens at tail_seg_pos + i;
            // a split never straddles two segments (split_len divides tail_seg_len)
            const int m = tok0 / p.tail_seg_len, off = tok0 - m * p.tail_seg_len;
            const int64_t si = static_cast<int64_t>(s) * (p.tail_cap / p.tail_seg_len) + m;
            const int sv = min(max(p.tail_seg_valid[si], 0), p.tail_seg_len);
            valid = min(max(sv - off, 0), p.split_len);
            pos0 = p.tail_seg_pos[si] + off;
        } else {
            const int len = min(p.tail_len[s], p.tail_cap);  // never read past the tail buffer
            valid = min(max(len - tok0, 0), p.split_len);
            pos0 = p.tail_pos0[s] + tok0;
        }
        rk = rv = kD;
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
    const int tiles_valid = (valid + kTile - 1) / kTile;
    const int KS = (rk + 31) >> 5;    // 32-rank k-steps of the key rebuild
    const int NTU = (rv + 15) >> 4;   // 16-rank row tiles of u

    const uint8_t *Ak = nullptr, *Av = nullptr, *Bv = nullptr, *Bk = nullptr;
    if constexpr (!TAIL) {
        Ak = p.k_arena + ka_off;
        Av = p.v_arena + va_off;
        Bv = p.v_arena + vb_off;
        Bk = p.k_arena + kb_off;
    }
    // ---- per-wave A_k staging (bf16 / int8 blocks) and tail V staging
    uint8_t *stg = lds + L.stage;
    if constexpr (!TAIL) stg += wave * 128 * stage_pitch(F);
    else stg += wave * 32 * kTVP;

    // A_k tile loads: 16-byte pieces, LPR lanes per rank row; rows past rk
    // repeat row rk - 1 (finite; their B_k fragment rows are zero).
    constexpr int RB = is_q(F) ? QRB : kTile * ES;  // bytes of one rank row of a tile
    constexpr int LPR = RB / 16 > 0 ? RB / 16 : 1;  // lanes per row
    constexpr int RPI = 64 / LPR;                   // rows per load instruction
    constexpr int NI = 128 / RPI;                   // load instructions for 128 ranks
    uint4 kraw[(F == kF32 || is_q(F) || TAIL) ? 1 : NI];
    // 4- and 2-bit: lane L stages, for ci = 0..7, the 16 bytes that the bf16 DMA
    // would write (row 16 ci + L / 4, physical chunk L % 4): 8 codes and their
    // row's scale for the tile.  Consecutive lanes then write consecutive 16 bytes.
    uint32_t kcode[(is_q(F) && !TAIL) ? 8 : 1];
    float kscl[(is_q(F) && !TAIL) ? 8 : 1];
    const int rk_pad = KS * 32;
    // Every load instruction is issued (rows clamped to rk - 1; identical
    // addresses coalesce), which keeps the registers free of partial paths.
    auto load_k = [&](int tile) {
        if constexpr (F != kF32 && !TAIL) {
            if (rk > 0) {
                const int tt0 = tok0 + tile * kTile;
                if constexpr (is_q(F)) {
                    const int pp = lane & 3;
                    constexpr int QB = qbits(F);
#pragma unroll
                    for (int ci = 0; ci < 8; ++ci) {
                        const int rp = 16 * ci + (lane >> 2);  // staging row
                        const int r = min(rp, rk - 1);         // rows past rk repeat the last
                        const int pc = ((((pp >> 1) ^ ((rp >> 1) & 1))) << 1) | (pp & 1);  // logical chunk
                        const uint32_t co = static_cast<uint32_t>(r * (T * QB / 8) + (tt0 + 8 * pc) * QB / 8);
                        if constexpr (F == kI4) kcode[ci] = *reinterpret_cast<const uint32_t *>(Ak + co);
                        else kcode[ci] = *reinterpret_cast<const uint16_t *>(Ak + co);
                        kscl[ci] = *reinterpret_cast<const float *>(
                            Ak + static_cast<uint32_t>(rk * (T * QB / 8) + (r * (T / kI4Group) + tt0 / kI4Group) * 4));
                    }
                } else {
#pragma unroll
                    for (int ci = 0; ci < NI; ++ci) {
                        // 32-bit offsets from the block's (uniform) base keep each address in one register
                        const int r = min(ci * RPI + lane / LPR, rk - 1);
                        const uint32_t off = static_cast<uint32_t>((r * T + tt0) * ES + (lane % LPR) * 16);
                        kraw[ci] = *reinterpret_cast<const uint4 *>(Ak + off);
                    }
                }
            }
        }
    };
    auto stage_k = [&](uint8_t *sdst) {
        if constexpr (F != kF32 && !TAIL) {
            if constexpr (is_q(F)) {
#pragma unroll
                for (int ci = 0; ci < 8; ++ci)
                    if (16 * ci < rk_pad) {  // uniform
                        uint32_t hw[4];
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            hw[e] = f32x2_to_bf16x2_bits(qval<F>(kcode[ci], 2 * e) * kscl[ci],
                                                         qval<F>(kcode[ci], 2 * e + 1) * kscl[ci]);
                        *reinterpret_cast<uint4 *>(sdst + 1024 * ci + 16 * lane) = make_uint4(hw[0], hw[1], hw[2], hw[3]);
                    }
            } else {
#pragma unroll
                for (int ci = 0; ci < NI; ++ci)
                    if (ci * RPI < rk_pad) {  // uniform
                        const int r = ci * RPI + lane / LPR;
                        if constexpr (F == kBF16) {
                            // 16-byte piece lane % LPR = tokens 8 (lane % LPR) .. + 7
                            uint8_t *dst = sdst + stage_off_bf16(r, 8 * (lane % LPR));
                            reinterpret_cast<uint2 *>(dst)[0] = make_uint2(kraw[ci].x, kraw[ci].y);
                            reinterpret_cast<uint2 *>(dst)[1] = make_uint2(kraw[ci].z, kraw[ci].w);
                        } else {
                            uint8_t *dst = sdst + r * 40 + (((lane % LPR) ^ ((r >> 4) & 1)) << 4);
                            reinterpret_cast<uint2 *>(dst)[0] = make_uint2(kraw[ci].x, kraw[ci].y);
                            reinterpret_cast<uint2 *>(dst)[1] = make_uint2(kraw[ci].z, kraw[ci].w);
                        }
                    }
            }
            wave_lds_sync();
        }
    };
    // bf16 blocks, tiles after the first: the tile's A_k^T goes from memory
    // straight into this wave's staging rows (LDS DMA, 16 bytes per lane, no
    // registers).  Instruction ci fills rows 16 ci .. 16 ci + 15; lane L writes
    // bytes 16 L of them, i.e. row 16 ci + L / 4 at 16 (L % 4), which is where
    // stage_off_bf16 puts the row's tokens 8 pc .. 8 pc + 7 for the pc below.
    // All eight instructions are issued without branches (rows past rk repeat
    // row rk - 1; rk = 0 reads the first bytes of q).
    auto dma_k = [&](int tile, uint8_t *sdst) {
        if constexpr (F == kBF16 && !TAIL) {
            const int tt0 = tok0 + tile * kTile;
            const int hh = (lane >> 1) & 1, lo = lane & 1;
            const uint8_t *base = pick_uniform(rk > 0, Ak, p.q);
            const int rlast = max(rk - 1, 0), on = rk > 0 ? 2 : 0;  // rk = 0: offset 0
#pragma unroll
            for (int ci = 0; ci < 8; ++ci) {
                const int r = 16 * ci + (lane >> 2);
                const int pc = ((hh ^ ((r >> 1) & 1)) << 1) | lo;
                const uint32_t off = static_cast<uint32_t>((min(r, rlast) * T + tt0 + 8 * pc) * on);
                __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)(base + off),
                                                 (__attribute__((address_space(3))) void *)(sdst + 1024 * ci), 16, 0, 0);
            }
        }
    };
    // bf16 blocks: B_v rows (256 bytes each) DMA'd into the staging rows of
    // waves 4..7 once their last rebuild is done (wave w: rows 32 (w - 4) ..
    // + 31, four rows per instruction), for the o = u B_v product of the merge.
    // That half of the staging lies past the merge's own LDS areas.
    auto dma_bv = [&](uint8_t *sdst) {
        if constexpr (F == kBF16 && !TAIL) {
            const uint8_t *base = pick_uniform(rv > 0, Bv, p.q);
            const int rlast = max(rv - 1, 0), on = rv > 0 ? 1 : 0;  // rv = 0: offset 0
#pragma unroll
            for (int ci = 0; ci < 8; ++ci) {
                const int row = 32 * (wave - 4) + 4 * ci + (lane >> 4);
                const uint32_t off = static_cast<uint32_t>((min(row, rlast) * (kD * 2) + 16 * (lane & 15)) * on);
                __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)(base + off),
                                                 (__attribute__((address_space(3))) void *)(sdst + 1024 * ci), 16, 0, 0);
            }
        }
    };
    // A_v^T pieces: rank 16 mr + ln, tokens 8 c .. 8 c + 7 of the tile (the
    // token order of the tiles below makes them the lane's eight P slots)
    uint4 vraw[(F == kF32 || TAIL) ? 1 : 8];
    auto load_v = [&](int tile) {
        if constexpr (F != kF32 && !TAIL) {
            const int t0 = tok0 + tile * kTile, tb = t0 + 8 * c4;
            if constexpr (F == kBF16) {
                // always 8 loads, without branches (rv = 0 reads the first bytes of q)
                const uint8_t *base = pick_uniform(rv > 0, Av, p.q);
                const int rlast = max(rv - 1, 0), on = rv > 0 ? 2 : 0;  // rv = 0: offset 0
#pragma unroll
                for (int mr = 0; mr < 8; ++mr) {
                    const uint32_t off = static_cast<uint32_t>((min(16 * mr + ln, rlast) * T + tb) * on);
                    vraw[mr] = *reinterpret_cast<const uint4 *>(base + off);
                }
            } else if (rv > 0) {
#pragma unroll
                for (int mr = 0; mr < 8; ++mr) {
                    const int row = min(16 * mr + ln, rv - 1);
                    if constexpr (is_q(F)) {
                        // codes of tokens tb .. tb + 7, and the scale of the tile's run
                        constexpr int QB = qbits(F);
                        const uint32_t co = static_cast<uint32_t>(row * (T * QB / 8) + tb * QB / 8);
                        uint32_t w;
                        if constexpr (F == kI4) w = *reinterpret_cast<const uint32_t *>(Av + co);
                        else w = *reinterpret_cast<const uint16_t *>(Av + co);
                        const float sc = *reinterpret_cast<const float *>(
                            Av + static_cast<uint32_t>(rv * (T * QB / 8) + (row * (T / kI4Group) + t0 / kI4Group) * 4));
                        vraw[mr] = make_uint4(w, __float_as_uint(sc), 0u, 0u);
                    } else {
                        const uint2 w = *reinterpret_cast<const uint2 *>(Av + static_cast<uint32_t>(row * T + tb));
                        vraw[mr] = make_uint4(w.x, w.y, 0u, 0u);
                    }
                }
            }
        }
    };

    // ---- prologue.  Every global load of the prologue (B_k rows, queries, the
    // RoPE tables, the first tile's factors) is issued before any is used.
    const int wt0 = wave;  // first tile of this wave
    const bool has_tile = wt0 < tiles_valid;
    if (has_tile) {
        load_k(wt0);
        load_v(wt0);
    }
    // B_k part of the arena as raw 16-byte chunks (4- and 2-bit: rk code rows of
    // d/2 or d/4 bytes, then rk x d/32 fp32 scales)
    constexpr int BKB = is_q(F) ? q_b_bytes(F) : kD * ES;  // bytes per rank
    constexpr int NBK = (F == kF32 || TAIL) ? 1 : (128 * BKB / 16 + kThreads - 1) / kThreads;
    uint4 bkraw[NBK];
    const int n16 = (F == kF32 || TAIL) ? 0 : (rk * BKB) >> 4;
    if constexpr (F != kF32 && !TAIL) {
        // rk = 0: the (discarded) loads read the first bytes of q instead
        const uint4 *src = reinterpret_cast<const uint4 *>(n16 > 0 ? Bk : static_cast<const uint8_t *>(p.q));
        const int last = n16 > 0 ? n16 - 1 : 0;
#pragma unroll
        for (int i = 0; i < NBK; ++i) bkraw[i] = src[min(tid + kThreads * i, last)];
    }
    // The remaining loads are issued unconditionally (indices clamped) so that
    // none is sunk into the branch that uses it, and used in issue order.
    float bsc_v = 0.f;
    if constexpr (F == kI8 && !TAIL) bsc_v = p.k_bscale[static_cast<int64_t>(fid) * kD + (tid & (kD - 1))];
    const float4 rope_v = reinterpret_cast<const float4 *>(p.rope_tab)[tid];      // entries 2 tid, 2 tid + 1
    const float4 rope_w = reinterpret_cast<const float4 *>(p.rope_tab)[tid + kThreads];
    constexpr int NST = kMaxTiles * 64 / 2 / kThreads;                               // float4 per thread
    float4 step_v[NST];
#pragma unroll
    for (int i = 0; i < NST; ++i) step_v[i] = reinterpret_cast<const float4 *>(p.step_tab)[tid + kThreads * i];
    // G query heads: 4 consecutive values per thread (rows >= G are zero)
    const int64_t q0 = (static_cast<int64_t>(s) * p.n_q_heads + h * G) * kD;
    const int qe0 = 4 * tid;  // < 16 * 128
    const int64_t qi = q0 + min(qe0, G * kD - 4);
    const bool q32 = p.q_type == kF32;
    const uint8_t *qb = static_cast<const uint8_t *>(p.q) + qi * (q32 ? 4 : 2);
    const uint2 qlo = *reinterpret_cast<const uint2 *>(qb), qhi = *reinterpret_cast<const uint2 *>(qb + (q32 ? 8 : 0));
    const uint4 qraw = make_uint4(qlo.x, qlo.y, qhi.x, qhi.y);
    const double theta_v = p.theta[tid & 63];
    const int64_t qpos = p.q_pos[s];

    if constexpr (F != kF32 && !TAIL) {
        // B_k rows -> the A_k staging area (free until the main loop); chunks past
        // the rows repeat the last one and are never read
        uint8_t *tmp = lds + L.stage;
#pragma unroll
        for (int i = 0; i < NBK; ++i) reinterpret_cast<uint4 *>(tmp)[tid + kThreads * i] = bkraw[i];
        if constexpr (F == kI8)
            if (tid < rk) reinterpret_cast<float *>(tmp + 128 * kD)[tid] = bsc_v;  // after the rows
    }
    {
        float2 *rw = reinterpret_cast<float2 *>(lds + L.rope);
        const int r0 = 2 * tid, r1 = 2 * (tid + kThreads);
        *reinterpret_cast<float4 *>(rw + (r0 >> 6) * kRP + (r0 & 63)) = rope_v;
        *reinterpret_cast<float4 *>(rw + (r1 >> 6) * kRP + (r1 & 63)) = rope_w;
    }
    {
        float qv[4];
        if (q32) {
            qv[0] = __uint_as_float(qraw.x); qv[1] = __uint_as_float(qraw.y);
            qv[2] = __uint_as_float(qraw.z); qv[3] = __uint_as_float(qraw.w);
        } else {
            qv[0] = bf16_bits_to_f32(qraw.x & 0xffff); qv[1] = bf16_bits_to_f32(qraw.x >> 16);
            qv[2] = bf16_bits_to_f32(qraw.y & 0xffff); qv[3] = bf16_bits_to_f32(qraw.y >> 16);
        }
        float *qw = reinterpret_cast<float *>(lds + L.qs);
        if (qe0 < G * kD)
            *reinterpret_cast<float4 *>(qw + (qe0 >> 7) * kQP + (qe0 & 127)) = make_float4(qv[0], qv[1], qv[2], qv[3]);
    }
    if (tid < 64) {
        // rotation of the queries relative to the split's first token, (pq - p0) theta_j
        double a = static_cast<double>(qpos - pos0) * theta_v;
        a -= kTwoPi * rint(a / kTwoPi);  // exact enough in fp64 for positions < 2^40
        float sn, cs;
        sincosf(static_cast<float>(a), &sn, &cs);
        ang[tid] = make_float2(cs, sn);
    }
    __syncthreads();
    // per-tile query rotation (pq - p0 - 32 tile) theta_j = angle difference
    {
        float2 *bw = reinterpret_cast<float2 *>(lds + L.base);
#pragma unroll
        for (int i = 0; i < NST; ++i) {
            const int e = 2 * (tid + kThreads * i);  // entries e, e + 1 (same tile)
            if (e < tiles_valid * 64) {
                const float4 st = step_v[i];
                const float2 a0 = ang[e & 63], a1 = ang[(e + 1) & 63];
                // (cos, sin)(A - B) = (cA cB + sA sB, sA cB - cA sB)
                bw[e] = make_float2(a0.x * st.x + a0.y * st.y, a0.y * st.x - a0.x * st.y);
                bw[e + 1] = make_float2(a1.x * st.z + a1.y * st.w, a1.y * st.z - a1.x * st.w);
            }
        }
    }
    if constexpr (!TAIL) {
        uint16_t *bk = reinterpret_cast<uint16_t *>(lds + L.bk);
        const uint8_t *tmp = lds + L.stage;
        const float *bsc = reinterpret_cast<const float *>(tmp + 128 * kD);  // int8 only
        // 4- and 2-bit: B_k's rows are first decoded into bf16 rows (row r at 256 r
        // bytes, after the raw codes and scales), so that the fragments come from
        // them by the bf16 path's transposing reads.  Thread t: row t / 4, dims
        // 32 (t % 4) ..
        uint8_t *rows4 = lds + L.stage + kBkRows4;
        if constexpr (is_q(F)) {
            constexpr int CRB = kD * qbits(F) / 8;  // code bytes of a B row
            const int r = tid >> 2, qd = tid & 3;
            uint32_t hw[16];
            if (r < rk) {
                uint32_t w4[4];
                run_words<F>(tmp + r * CRB + qd * (CRB / 4), w4);
                const float sc = reinterpret_cast<const float *>(tmp + rk * CRB)[r * (kD / kI4Group) + qd];
                decode_run<F>(w4, sc, hw);
            } else {
#pragma unroll
                for (int k = 0; k < 16; ++k) hw[k] = 0u;
            }
            uint4 *dst = reinterpret_cast<uint4 *>(rows4 + r * (kD * 2) + 64 * qd);
#pragma unroll
            for (int c = 0; c < 4; ++c) dst[c] = make_uint4(hw[4 * c], hw[4 * c + 1], hw[4 * c + 2], hw[4 * c + 3]);
            __syncthreads();
        }
        for (int q = tid; q < 8 * 4 * 64; q += kThreads) {
            const int l2 = q & 63, ks = (q >> 6) & 3, mt = q >> 8;
            if (ks >= KS) continue;
            const int j = 16 * mt + (l2 & 15), r0 = 32 * ks + 8 * (l2 >> 4);
            if constexpr (F == kBF16 || is_q(F)) {
                // ranks r0 .. r0 + 7 of dim j by two transposing reads of the staged
                // rows (lane (c, i) of a 16-lane group addresses row r0 + i / 4 (+ 4),
                // dims 16 mt + 4 (i % 4) ..); rows past rk (repeats) become zero
                const uint8_t *p0 = (is_q(F) ? rows4 : tmp) + (r0 + ((l2 & 15) >> 2)) * (kD * 2) + (16 * mt + 4 * (l2 & 3)) * 2;
                u16x8_t f0 = cat8(lds_read_tr16(p0), lds_read_tr16(p0 + 4 * kD * 2));
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (r0 + e >= rk) f0[e] = 0;
                *reinterpret_cast<u16x8_t *>(bk + q * 8) = f0;
                continue;
            }
            float v[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int r = r0 + e;
                v[e] = 0.f;
                if (r < rk) {
                    if constexpr (F == kI8) v[e] = static_cast<float>(reinterpret_cast<const int8_t *>(tmp)[r * kD + j]) * bsc[r];
                    else v[e] = load_elem<F>(Bk, static_cast<int64_t>(r) * kD + j);
                }
            }
            u16x8_t f[NS];
            frag_terms<NS>(v, f);
#pragma unroll
            for (int st = 0; st < NS; ++st) *reinterpret_cast<u16x8_t *>(bk + (st * 2048 + q) * 8) = f[st];
        }
    }
    __syncthreads();  // tables, fragments; the staging area is free again
    // Lane (c, n) owns query head n: column n of every accumulator.

    float m_run = -INFINITY, l_run = 0.f;
    f32x4_t u[8];
#pragma unroll
    for (int mr = 0; mr < 8; ++mr) u[mr] = zero4();
    const float lscale = p.softmax_scale * kLog2e;

    // Pipeline: the staging buffer holds this tile's A_k^T while its keys are
    // rebuilt; A_v^T pieces are loaded a whole tile ahead.  bf16: the next
    // tile's A_k^T is DMA'd into the staging rows as soon as the rebuild has
    // read them.  Other formats: it is loaded into registers at the start of
    // the tile and staged at its end.
    const int my_tiles = tiles_valid > wave ? (tiles_valid - 1 - wave) / kWaves + 1 : 0;
    if (my_tiles > 0) stage_k(stg);
    if constexpr (F == kBF16 && !TAIL) {
        // Every prologue load has landed by now (the first tile's A_v pieces
        // included).  Some are used only inside branches (the query rows, the
        // first wave's angles, part of the step table); left pending on the
        // paths that skip them, they would be carried into the tile loop, where
        // with LDS DMA in flight the compiler waits for all memory operations
        // (vmcnt(0)) at the first reuse of their registers, in every tile.
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        asm volatile("" ::: "memory");
    }
    // bf16 blocks: a tile's u update (u = alpha u + A_v^T P^T) runs at the top
    // of the next tile, right after the wait for that tile's DMA.  While an LDS
    // DMA is in flight the compiler waits for every memory operation (vmcnt(0))
    // before any use of a loaded register, so the A_v pieces are used only
    // where nothing newer is in flight: a tile's pieces are loaded at its top
    // and used at the next top, and its softmax weights wait in pf_prev.
    u16x8_t pf_prev = {};
    float alpha_prev = 1.f;
    bool rescale_prev = false;
    auto u_update_bf16 = [&]() {
#pragma unroll
        for (int mr = 0; mr < 8; ++mr)
            if (mr < NTU) {
                if (rescale_prev) u[mr] *= alpha_prev;
                u[mr] = mfma16x16x32(__builtin_bit_cast(u16x8_t, vraw[mr]), pf_prev, u[mr]);
            }
    };
    // The loop reaches LDS through two restrict pointers, the staging rows and
    // the tables (disjoint regions), so that the compiler knows the staging DMA
    // does not write what the table reads load.
    auto main_loop = [&](uint8_t *__restrict__ sg, const uint8_t *__restrict__ tb) {
    const float2 *rope = reinterpret_cast<const float2 *>(tb + L.rope);
    const float2 *basetab = reinterpret_cast<const float2 *>(tb + L.base);
    const uint16_t *bkf = reinterpret_cast<const uint16_t *>(tb + L.bk);
    const float *qrow = reinterpret_cast<const float *>(tb + L.qs) + min(ln, G - 1) * kQP;
    uint8_t *stg = sg;
    for (int it = 0; it < my_tiles; ++it) {
        const int tile = wave + kWaves * it;
        const int tt0 = tok0 + tile * kTile;  // first token of the tile (block- or tail-local)

        // The two waves of a SIMD (w, w + 4) take turns at the higher issue
        // priority, tile by tile, so that they finish together.
        if ((it + (wave >> 2)) & 1) __builtin_amdgcn_s_setprio(1);
        else __builtin_amdgcn_s_setprio(0);
        if constexpr (F == kBF16 && !TAIL) {
            if (it > 0) {
                // this tile's DMA and the previous tile's A_v pieces have landed
                __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
                asm volatile("" ::: "memory");
                u_update_bf16();  // the previous tile's
                load_v(tile);     // used at the next top (the first tile's came with the prologue)
            }
        } else if (it + 1 < my_tiles) {
            load_k(tile + kWaves);  // a whole tile of latency cover
        }

        // ---- this tile's rotated query fragments, dims 16 kk + 4 c + i and + 64
        u16x8_t qf[NS][4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const float4 *bp = reinterpret_cast<const float4 *>(basetab + tile * 64 + 16 * kk + 4 * c4);
            const float4 b01 = bp[0], b23 = bp[1];
            const float cs[4] = {b01.x, b01.z, b23.x, b23.z}, sn[4] = {b01.y, b01.w, b23.y, b23.w};
            const float4 qa = *reinterpret_cast<const float4 *>(qrow + 16 * kk + 4 * c4);
            const float4 qb = *reinterpret_cast<const float4 *>(qrow + 64 + 16 * kk + 4 * c4);
            const float q1[4] = {qa.x, qa.y, qa.z, qa.w}, q2[4] = {qb.x, qb.y, qb.z, qb.w};
            float v[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                v[i] = q1[i] * cs[i] - q2[i] * sn[i];
                v[4 + i] = q1[i] * sn[i] + q2[i] * cs[i];
            }
            u16x8_t f[NS];
            frag_terms<NS>(v, f);
#pragma unroll
            for (int st = 0; st < NS; ++st) qf[st][kk] = f[st];
        }

        // ---- per half nt: K^T (acc[mt][i] = k_hat[token tk(nt, ln)][dim 16 mt + 4 c + i]),
        // RoPE by the in-tile offset, logits^T S[nt][i] = logit(token tk(nt, 4 c + i), head ln),
        // where tk(nt, 4 c + i) = 8 c + 4 nt + i: lane (c, n)'s eight P values are then
        // tokens 8 c .. 8 c + 7 (slot 4 nt + i), which one 16-byte A_v load holds
        f32x4_t S[2];
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            const int t = 8 * (ln >> 2) + 4 * nt + (ln & 3);
            asm volatile("" ::: "memory");
            f32x4_t acc[8];
            if constexpr (!TAIL) {
#pragma unroll
                for (int mt = 0; mt < 8; ++mt) acc[mt] = zero4();
                for (int ks = 0; ks < KS; ++ks) {
                    const bool first = ks == 0;  // zero accumulator input (inline constant)
                    u16x8_t bfr[NS];
                    if constexpr (F == kBF16 || is_q(F)) {
                        // ranks 32 ks + 8 c .. + 7 of token t by two transposing reads: lane
                        // (c, j) addresses rank row 32 ks + 8 c + j / 4 (+ 4), tokens
                        // 8 (j % 4) + 4 nt .. + 3, and lane (c, j) receives token tk(nt, j)
                        const int row = 32 * ks + 8 * c4 + (ln >> 2);
                        const uint8_t *p0 = stg + stage_off_bf16(row, 8 * (ln & 3) + 4 * nt);
                        bfr[0] = cat8(lds_read_tr16(p0), lds_read_tr16(p0 + 4 * 64));
                    } else if constexpr (F == kI8) {
                        float v[8];
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            v[e] = static_cast<float>(*reinterpret_cast<const int8_t *>(stg + stage_off_i8(32 * ks + 8 * c4 + e, t)));
                        frag_terms<1>(v, reinterpret_cast<u16x8_t(&)[1]>(bfr));
                    } else {
                        float v[8];
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const int r = 32 * ks + 8 * c4 + e;
                            v[e] = r < rk ? load_elem<F>(Ak, static_cast<int64_t>(r) * T + tt0 + t) : 0.f;
                        }
                        frag_terms<NS>(v, bfr);
                    }
#pragma unroll
                    for (int sa = 0; sa < NS; ++sa) {
                        // all eight fragment reads in flight before the first product
                        u16x8_t a[8];
#pragma unroll
                        for (int mt = 0; mt < 8; ++mt)
                            a[mt] = *reinterpret_cast<const u16x8_t *>(bkf + ((sa * 2048) + (mt * 4 + ks) * 64 + lane) * 8);
                        // (the scheduler would otherwise interleave reads and products
                        // two at a time, serialising the LDS round trips)
                        if constexpr (NS == 1) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                        for (int mt = 0; mt < 8; ++mt)
#pragma unroll
                            for (int sb = 0; sb < NS; ++sb)
                                if (sa + sb < NS)
                                    acc[mt] = mfma16x16x32(a[mt], bfr[sb], (first && sa + sb == 0) ? zero4() : acc[mt]);
                    }
                }
            } else {
                // tail keys straight from memory (rows past the valid length repeat the last one)
                const int64_t rowb = (static_cast<int64_t>(s) * Hkv + h) * p.tail_cap;
                const int tk = min(tt0 + t, tok0 + valid - 1);
                const uint8_t *kp = static_cast<const uint8_t *>(p.tail_k) + (rowb + tk) * kD * ES;
#pragma unroll
                for (int mt = 0; mt < 8; ++mt) {
                    const int j0 = 16 * mt + 4 * c4;
                    if constexpr (F == kF32) {
                        const float4 w = *reinterpret_cast<const float4 *>(kp + j0 * 4);
                        acc[mt][0] = w.x; acc[mt][1] = w.y; acc[mt][2] = w.z; acc[mt][3] = w.w;
                    } else {
                        const uint2 w = *reinterpret_cast<const uint2 *>(kp + j0 * 2);
                        acc[mt][0] = bf16_bits_to_f32(w.x & 0xffff);
                        acc[mt][1] = bf16_bits_to_f32(w.x >> 16);
                        acc[mt][2] = bf16_bits_to_f32(w.y & 0xffff);
                        acc[mt][3] = bf16_bits_to_f32(w.y >> 16);
                    }
                }
            }
            if constexpr (F == kBF16 && !TAIL) {
                if (nt == 1) {
                    // both halves have read the staged tile: the next one may land
                    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
                    asm volatile("" ::: "memory");
                    if (it + 1 < my_tiles) dma_k(tile + kWaves, stg);
                    else if (wave >= 4) dma_bv(stg);
                }
            }
            // keep the table reads below after the rebuild (registers)
            asm volatile("" ::: "memory");
            S[nt] = zero4();
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const float4 *rp = reinterpret_cast<const float4 *>(rope + t * kRP + 16 * kk + 4 * c4);
                const float4 r01 = rp[0], r23 = rp[1];
                const float cs[4] = {r01.x, r01.z, r23.x, r23.z}, sn[4] = {r01.y, r01.w, r23.y, r23.w};
                float v[8];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float k1 = acc[kk][i], k2 = acc[kk + 4][i];
                    v[i] = k1 * cs[i] - k2 * sn[i];
                    v[4 + i] = k1 * sn[i] + k2 * cs[i];
                }
                u16x8_t kf[NS];
                frag_terms<NS>(v, kf);
#pragma unroll
                for (int sa = 0; sa < NS; ++sa)
#pragma unroll
                    for (int sb = 0; sb < NS; ++sb)
                        if (sa + sb < NS) S[nt] = mfma16x16x32(kf[sa], qf[sb][kk], S[nt]);
            }
        }


        // ---- online softmax (log2 domain) for head ln over this tile's 32 tokens
        float sc[2][4], vs[2][4];
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                sc[nt][i] = lscale;
                vs[nt][i] = 1.f;
            }
        if constexpr (F == kI8 && !TAIL) {
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                const int64_t ti = static_cast<int64_t>(fid) * T + tt0 + 8 * c4 + 4 * nt;
                const float4 ka = *reinterpret_cast<const float4 *>(p.k_ascale + ti);
                const float4 va = *reinterpret_cast<const float4 *>(p.v_ascale + ti);
                sc[nt][0] *= ka.x; sc[nt][1] *= ka.y; sc[nt][2] *= ka.z; sc[nt][3] *= ka.w;
                vs[nt][0] = va.x; vs[nt][1] = va.y; vs[nt][2] = va.z; vs[nt][3] = va.w;
            }
        }
        float x[2][4];
        float tmax = -INFINITY;
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bool ok = !TAIL || tile * kTile + 8 * c4 + 4 * nt + i < valid;
                x[nt][i] = ok ? S[nt][i] * sc[nt][i] : -INFINITY;
                tmax = fmaxf(tmax, x[nt][i]);
            }
        tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
        const float mn = fmaxf(m_run, tmax);
        const bool none = (mn == -INFINITY);
        const float alpha = none ? 1.f : __builtin_amdgcn_exp2f(m_run - mn);
        float pv[8], psum = 0.f;
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float pr = none ? 0.f : __builtin_amdgcn_exp2f(x[nt][i] - mn);
                psum += pr;
                pv[4 * nt + i] = pr * vs[nt][i];
            }
        l_run = l_run * alpha + psum;
        m_run = mn;

        // ---- u^T = alpha u^T + A_v^T P^T (the rescale is skipped when no head's maximum moved)
        u16x8_t pf[NS];
        frag_terms<NS>(pv, pf);
        const bool rescale = __any(alpha != 1.f);
        if constexpr (F == kBF16 && !TAIL) {
            pf_prev = pf[0];
            alpha_prev = alpha;
            rescale_prev = rescale;
        } else if constexpr (!TAIL && F != kF32) {
#pragma unroll
            for (int mr = 0; mr < 8; ++mr)
                if (mr < NTU) {
                    if (rescale) u[mr] *= alpha;
                    u16x8_t af;
                    if constexpr (is_q(F)) {
                        const float sc = __uint_as_float(vraw[mr].y);
                        float v[8];
#pragma unroll
                        for (int e = 0; e < 8; ++e) v[e] = qval<F>(vraw[mr].x, e) * sc;
                        u16x8_t f[1];
                        frag_terms<1>(v, f);
                        af = f[0];
                    } else {
                        float v[8];
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            v[e] = static_cast<float>(static_cast<int8_t>((vraw[mr].x >> (8 * e)) & 0xff));
                            v[4 + e] = static_cast<float>(static_cast<int8_t>((vraw[mr].y >> (8 * e)) & 0xff));
                        }
                        u16x8_t f[1];
                        frag_terms<1>(v, f);
                        af = f[0];
                    }
                    u[mr] = mfma16x16x32(af, pf[0], u[mr]);
                }
        } else if constexpr (!TAIL) {
            // fp32 factors: A_v^T pieces straight from memory, two terms
#pragma unroll
            for (int mr = 0; mr < 8; ++mr)
                if (mr < NTU) {
                    if (rescale) u[mr] *= alpha;
                    const int row = min(16 * mr + ln, rv - 1);
                    float v[8];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        v[e] = load_elem<F>(Av, static_cast<int64_t>(row) * T + tt0 + 8 * c4 + e);
                        v[4 + e] = load_elem<F>(Av, static_cast<int64_t>(row) * T + tt0 + 8 * c4 + 4 + e);
                    }
                    u16x8_t af[NS];
                    frag_terms<NS>(v, af);
#pragma unroll
                    for (int sa = 0; sa < NS; ++sa)
#pragma unroll
                        for (int sb = 0; sb < NS; ++sb)
                            if (sa + sb < NS) u[mr] = mfma16x16x32(af[sa], pf[sb], u[mr]);
                }
        } else {
            // tail values: dims play the role of ranks (B_v = I)
            const int64_t rowb = (static_cast<int64_t>(s) * Hkv + h) * p.tail_cap;
            const int tlast = tok0 + valid - 1;
            if constexpr (F == kBF16) {
                // stage the 32 x 128 tile token-major, read 8 tokens of one dim per lane
#pragma unroll
                for (int q4 = 0; q4 < 8; ++q4) {
                    const int ch = lane + 64 * q4;  // 16-byte chunk: token ch / 16, dims 8 (ch % 16) ..
                    const int t = min(tt0 + (ch >> 4), tlast);
                    const uint4 w = *reinterpret_cast<const uint4 *>(static_cast<const uint8_t *>(p.tail_v) +
                                                                     ((rowb + t) * kD + 8 * (ch & 15)) * 2);
                    uint8_t *dst = stg + (ch >> 4) * kTVP + (ch & 15) * 16;
                    reinterpret_cast<uint2 *>(dst)[0] = make_uint2(w.x, w.y);
                    reinterpret_cast<uint2 *>(dst)[1] = make_uint2(w.z, w.w);
                }
                wave_lds_sync();
            }
#pragma unroll
            for (int mr = 0; mr < 8; ++mr) {
                if (rescale) u[mr] *= alpha;
                const int dim = 16 * mr + ln;
                u16x8_t af[NS];
                if constexpr (F == kBF16) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int tt = 8 * c4 + e;
                        af[0][e] = *reinterpret_cast<const uint16_t *>(stg + tt * kTVP + dim * 2);
                    }
                } else {
                    float v[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int tt = 8 * c4 + e;
                        const int t = min(tt0 + tt, tlast);
                        v[e] = reinterpret_cast<const float *>(p.tail_v)[(rowb + t) * kD + dim];
                    }
                    frag_terms<NS>(v, af);
                }
#pragma unroll
                for (int sa = 0; sa < NS; ++sa)
#pragma unroll
                    for (int sb = 0; sb < NS; ++sb)
                        if (sa + sb < NS) u[mr] = mfma16x16x32(af[sa], pf[sb], u[mr]);
            }
            if constexpr (F == kBF16) wave_lds_sync();  // staging reused by the next tile
        }

        if constexpr (F == kBF16 && !TAIL) {
            // (this tile's A_v pieces were loaded at its top)
        } else if (it + 1 < my_tiles) {
            load_v(tile + kWaves);
            wave_lds_sync();  // this tile's staged keys have been read
            stage_k(stg);
        }
    }
    };
    main_loop(stg, lds);
    __builtin_amdgcn_s_setprio(0);
    if constexpr (F == kBF16 && !TAIL) {
        if (my_tiles == 0 && wave >= 4) dma_bv(stg);
        // the DMAs land before the barrier that starts the merge
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        asm volatile("" ::: "memory");
        if (my_tiles > 0) u_update_bf16();  // the last tile's
    }
    if constexpr (is_q(F) && !TAIL) {
        // B_v's code rows and scales (rv x 80 or rv x 48 bytes, at most 640 16-byte chunks)
        // go by LDS DMA into the last 10 KiB of the staging area, chunk c at byte
        // 16 c: the staging rows of waves 6 (chunks 0 .. 127) and 7 (128 .. 639),
        // which each writes only once its own tiles are done (chunks past the last
        // repeat it).  They land before the second barrier of the merge.
        if (wave >= 6) {
            const int n16v = rv * q_b_bytes(F) / 16;
            const uint8_t *base = pick_uniform(n16v > 0, Bv, p.q);
            const int last = max(n16v - 1, 0), on = n16v > 0 ? 16 : 0;
            uint8_t *dst = lds + L.bvraw;
            const int ninst = wave == 6 ? 2 : 8;
            const int cbase = wave == 6 ? 0 : 128;
#pragma unroll
            for (int k = 0; k < 8; ++k)
                if (k < ninst) {
                    const int c0 = cbase + 64 * k;
                    const uint32_t off = static_cast<uint32_t>(min(c0 + lane, last) * on);
                    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)(base + off),
                                                     (__attribute__((address_space(3))) void *)(dst + 16 * c0), 16, 0, 0);
                }
        }
    }

    // ---- merge the waves (log-sum-exp) and apply B_v
    l_run += __shfl_xor(l_run, 16, 64);
    l_run += __shfl_xor(l_run, 32, 64);
    __syncthreads();  // loop-phase LDS is dead from here on
    float *uw = reinterpret_cast<float *>(lds + L.uw);
    float *mlw = reinterpret_cast<float *>(lds + L.mlw);
    float *uacc = reinterpret_cast<float *>(lds + L.uacc);
    if (c4 == 0) {
        mlw[(wave * 16 + ln) * 2] = m_run;
        mlw[(wave * 16 + ln) * 2 + 1] = l_run;
    }
#pragma unroll
    for (int mr = 0; mr < 8; ++mr)
        if (mr < NTU)
            *reinterpret_cast<f32x4_t *>(uw + (wave * 16 + ln) * kUP + 16 * mr + 4 * c4) = u[mr];
    const int KSV = (rv + 31) >> 5;  // 32-rank k-steps of u B_v
    const int rpad = TAIL ? kD : KSV * 32;
    // B_v fragments for o = u B_v (lane: dim 16 w + n, ranks 32 ks + 8 c + e), read
    // straight from memory now so that their latency overlaps the merge
    u16x8_t bvf[NS][4];
    if constexpr (F == kBF16 && !TAIL) {
        // lane (c, j): ranks 32 ks + 8 c .. + 7 of dim 16 w + j by two transposing
        // reads of the staged rows (lane (c, j) addresses row 32 ks + 8 c + j / 4
        // (+ 4), dims 16 w + 4 (j % 4) .. + 3); rows past rv repeat row rv - 1,
        // and u is zero there
        const uint8_t *bvl = lds + L.stage + 4 * 128 * stage_pitch(F);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            if (ks < KSV) {
                const uint8_t *p0 = bvl + (32 * ks + 8 * c4 + (ln >> 2)) * (kD * 2) + (16 * wave + 4 * (ln & 3)) * 2;
                bvf[0][ks] = cat8(lds_read_tr16(p0), lds_read_tr16(p0 + 4 * kD * 2));
            }
    } else if constexpr (!TAIL && !is_q(F)) {
        if (rv > 0) {
            const int dim = 16 * wave + ln;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                float v[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int r = 32 * ks + 8 * c4 + e;
                    const int rc = min(r, rv - 1);
                    float x = load_elem<F>(Bv, static_cast<int64_t>(rc) * kD + dim);
                    if constexpr (F == kI8) x *= p.v_bscale[static_cast<int64_t>(fid) * kD + rc];
                    v[e] = r < rv ? x : 0.f;
                }
                u16x8_t f[NS];
                frag_terms<NS>(v, f);
#pragma unroll
                for (int st = 0; st < NS; ++st) bvf[st][ks] = f[st];
            }
        }
    }
    if constexpr (is_q(F) && !TAIL) {
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // the B_v DMA has landed (before the barrier)
        asm volatile("" ::: "memory");
    }
    __syncthreads();
    if constexpr (is_q(F) && !TAIL) {
        // quantised B_v -> bf16 rows (row r at 256 r bytes), the bf16 path's layout
        // for the transposing fragment reads below.  Thread t: row t / 4, dims
        // 32 (t % 4) .. + 31; rows past rv are zero.
        constexpr int CRB = kD * qbits(F) / 8;
        const uint8_t *bv4 = lds + L.bvraw;
        const int r = tid >> 2, qd = tid & 3;
        uint32_t hw[16];
        if (r < rv) {
            uint32_t w4[4];
            run_words<F>(bv4 + r * CRB + qd * (CRB / 4), w4);
            const float sc = reinterpret_cast<const float *>(bv4 + rv * CRB)[r * (kD / kI4Group) + qd];
            decode_run<F>(w4, sc, hw);
        } else {
#pragma unroll
            for (int k = 0; k < 16; ++k) hw[k] = 0u;
        }
        uint4 *dst = reinterpret_cast<uint4 *>(lds + L.bvrows + r * (kD * 2) + 64 * qd);
#pragma unroll
        for (int c = 0; c < 4; ++c) dst[c] = make_uint4(hw[4 * c], hw[4 * c + 1], hw[4 * c + 2], hw[4 * c + 3]);
    }
    {
        // thread t: head g = t / 32, ranks t % 32 + 32 j; the head's wave weights
        // exp2(m_w - M) are computed once per thread
        static_assert(kThreads == 16 * 32, "one head per 32 threads");
        const int g = tid >> 5;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) M = fmaxf(M, mlw[(w * 16 + g) * 2]);
        float cf[kWaves];
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float mw = mlw[(w * 16 + g) * 2];
            cf[w] = (mw == -INFINITY) ? 0.f : exp2f(mw - M);
        }
        for (int r = tid & 31; r < rpad; r += 32) {
            float uvs = 0.f;
#pragma unroll
            for (int w = 0; w < kWaves; ++w)
                if (cf[w] != 0.f && r < rv) uvs += cf[w] * uw[(w * 16 + g) * kUP + r];
            uacc[g * kUP + r] = uvs;
        }
    }
    if (tid < G) {  // (max, sum) of every head, also when rpad == 0 (rank-0 values)
        float M = -INFINITY, Ls = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) M = fmaxf(M, mlw[(w * 16 + tid) * 2]);
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float mw = mlw[(w * 16 + tid) * 2];
            Ls += (mw == -INFINITY ? 0.f : exp2f(mw - M)) * mlw[(w * 16 + tid) * 2 + 1];
        }
        ml[2 * tid] = M;
        ml[2 * tid + 1] = Ls;
    }
    __syncthreads();
    if constexpr (is_q(F) && !TAIL) {
        // quantised B_v fragments from the rows decoded above, as for bf16
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            if (ks < KSV) {
                const uint8_t *p0 = lds + L.bvrows + (32 * ks + 8 * c4 + (ln >> 2)) * (kD * 2) + (16 * wave + 4 * (ln & 3)) * 2;
                bvf[0][ks] = cat8(lds_read_tr16(p0), lds_read_tr16(p0 + 4 * kD * 2));
            }
    }
    if constexpr (TAIL) {
        for (int e = tid; e < G * kD; e += kThreads) po[e] = uacc[(e >> 7) * kUP + (e & 127)];
    } else {
        // o^T tile of wave w: dims 16 w .. 16 w + 15 = u (16 x rpad) B_v (rpad x 128)
        f32x4_t o = zero4();
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            if (ks < KSV) {
                const float4 *up = reinterpret_cast<const float4 *>(uacc + ln * kUP + 32 * ks + 8 * c4);
                const float4 ua = up[0], ub = up[1];
                const float v[8] = {ua.x, ua.y, ua.z, ua.w, ub.x, ub.y, ub.z, ub.w};
                u16x8_t af[NS];
                frag_terms<NS>(v, af);
#pragma unroll
                for (int sa = 0; sa < NS; ++sa)
#pragma unroll
                    for (int sb = 0; sb < NS; ++sb)
                        if (sa + sb < NS) o = mfma16x16x32(af[sa], bvf[sb][ks], o);
            }
        }
        // o[i]: head 4 c + i, dim 16 w + ln
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int g = 4 * c4 + i;
            if (g < G) po[g * kD + 16 * wave + ln] = o[i];
        }
    }
}

// One workgroup per (sequence, query head): the split maxima and weights are
// computed by all threads in parallel; thread (k, j) then sums dimension j over
// the splits k, k + kCG, ... (eight loads in flight), and the kCG partial sums
// are added in group order.
constexpr int kCG = 4;  // split groups per output column

template <int OT>
__global__ __launch_bounds__(kD * kCG) void decode_combine_kernel(const DecodeParams p) {
    __shared__ float coef[1024];
    __shared__ float red[kD * kCG / 64];
    __shared__ float part[kCG][kD];
    const int hq = blockIdx.x, s = blockIdx.y, tid = threadIdx.x;
    const int dim = tid & (kD - 1), grp = tid / kD;
    const int lane = tid & 63, wave = tid >> 6;
    constexpr int kNW = kD * kCG / 64;
    constexpr int kNT = kD * kCG;
    const int G = p.group;
    const int h = hq / G, g = hq - h * G;
    const int64_t base = static_cast<int64_t>(s * p.n_kv_heads + h) * p.n_splits;
    float num = 0.f, den_part = 0.f;
    // chunks of up to 1024 splits (the weights of one chunk fit in LDS)
    float M = -INFINITY;
    for (int sp = tid; sp < p.n_splits; sp += kNT) M = fmaxf(M, p.part_ml[((base + sp) * G + g) * 2]);
    M = wave_max(M);
    if (lane == 0) red[wave] = M;
    __syncthreads();
    M = red[0];
#pragma unroll
    for (int w = 1; w < kNW; ++w) M = fmaxf(M, red[w]);
    __syncthreads();
    for (int c0 = 0; c0 < p.n_splits; c0 += 1024) {
        const int cn = min(1024, p.n_splits - c0);
        for (int i = tid; i < cn; i += kNT) {
            const float m = p.part_ml[((base + c0 + i) * G + g) * 2];
            const float c = (m == -INFINITY || M == -INFINITY) ? 0.f : exp2f(m - M);
            coef[i] = c;
            den_part += c * p.part_ml[((base + c0 + i) * G + g) * 2 + 1];
        }
        __syncthreads();
        // eight loads in flight at a time (indices clamped; a split with weight 0
        // may hold stale values, which the select keeps out), summed in order
        for (int i0 = grp; i0 < cn; i0 += 8 * kCG) {
            float v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = p.part_o[((base + c0 + min(i0 + kCG * u, cn - 1)) * G + g) * kD + dim];
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (i0 + kCG * u < cn) {
                    const float c = coef[i0 + kCG * u];
                    num += c != 0.f ? c * v[u] : 0.f;
                }
        }
        __syncthreads();
    }
    part[grp][dim] = num;
    den_part = wave_sum(den_part);
    if (lane == 0) red[wave] = den_part;
    __syncthreads();
    if (grp == 0) {
        float den = 0.f;
#pragma unroll
        for (int w = 0; w < kNW; ++w) den += red[w];
        float o = part[0][dim];
#pragma unroll
        for (int k = 1; k < kCG; ++k) o += part[k][dim];
        o = den > 0.f ? o / den : 0.f;
        const int64_t oi = (static_cast<int64_t>(s) * p.n_q_heads + hq) * kD + dim;
        if constexpr (OT == kF32)
            static_cast<float *>(p.out)[oi] = o;
        else
            static_cast<uint16_t *>(p.out)[oi] = f32_to_bf16_bits(o);
    }
}

// One launch for every split of a call: workgroup x < n_sel * block_splits
// runs split x of the selected blocks (factor type F), the rest run the
// tail's splits (element type TF; TF < 0: no tail).  The partials are merged
// by decode_combine_kernel, a launch of its own: a merge inside this kernel by
// its last workgroup would need a device-scope release from every workgroup,
// which writes back the issuing XCD's L2 each time.
template <int F, int TF>
__global__ __launch_bounds__(kThreads) void decode_kernel(const DecodeParams p) {
    extern __shared__ __align__(16) uint8_t lds[];
    const int nb = p.n_sel * p.block_splits;
    const int x = blockIdx.x;
    if constexpr (TF < 0) {
        decode_partial<F, false>(p, x, lds);
    } else {
        if (x < nb) decode_partial<F, false>(p, x, lds);
        else decode_partial<TF, true>(p, x - nb, lds);
    }
}

// RoPE tables shared by every workgroup of one call: theta_j = base^(-2j/128),
// (cos, sin)(t theta_j) for t < 32, and (cos, sin)(32 tile theta_j) for the
// tile offsets of a split (angles reduced in fp64).
__global__ __launch_bounds__(256) void decode_tables_kernel(double rope_base, double *theta, float2 *rope,
                                                            float2 *step) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    const int j = i & 63;
    const double th = exp2(-(static_cast<double>(j) / 64.0) * log2(rope_base));
    if (i < 64) theta[i] = th;
    if (i < 32 * 64) {
        float sn, cs;  // angle < 32 rad: fp32 sincos is accurate after its own reduction
        sincosf(static_cast<float>(static_cast<double>(i >> 6) * th), &sn, &cs);
        rope[i] = make_float2(cs, sn);
    }
    if (i < kMaxTiles * 64) {
        double a = 32.0 * static_cast<double>(i >> 6) * th;
        a -= kTwoPi * rint(a / kTwoPi);
        float sn, cs;
        sincosf(static_cast<float>(a), &sn, &cs);
        step[i] = make_float2(cs, sn);
    }
}

template <int F, int TF>
hipError_t launch_decode_kernel(const DecodeParams &p, hipStream_t st) {
    constexpr int NS = (F == kF32) ? 2 : 1;
    const int n_tiles = p.split_len / kTile;
    int lds = lds_layout(F, NS, n_tiles, false, p.group).total;
    if constexpr (TF >= 0) {
        const int tl = lds_layout(TF, TF == kF32 ? 2 : 1, n_tiles, true, p.group).total;
        lds = lds > tl ? lds : tl;
    }
    // The kernel's dynamic LDS limit is raised to the CU's maximum once per
    // device, so that a launch recorded into a graph is a plain launch.
    static bool limit_set[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices || !limit_set[dev]) {
        e = hipFuncSetAttribute(reinterpret_cast<const void *>(decode_kernel<F, TF>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, kMaxLds);
        if (e != hipSuccess) return e;
        if (dev >= 0 && dev < kMaxDevices) limit_set[dev] = true;
    }
    if (lds > kMaxLds) return hipErrorInvalidValue;
    const dim3 grid(static_cast<unsigned>(p.n_splits), static_cast<unsigned>(p.n_kv_heads),
                    static_cast<unsigned>(p.batch));
    hipLaunchKernelGGL((decode_kernel<F, TF>), grid, dim3(kThreads), lds, st, p);
    return hipGetLastError();
}

template <int F>
hipError_t launch_decode_f(const DecodeParams &p, hipStream_t st) {
    if (p.tail_splits == 0) return launch_decode_kernel<F, -1>(p, st);
    if (p.tail_type == kBF16) return launch_decode_kernel<F, kBF16>(p, st);
    return launch_decode_kernel<F, kF32>(p, st);
}

}  // namespace

bool decode_split_fits(int f_type, int tail_type, bool has_tail, int G, int split) {
    const int ns = f_type == kF32 ? 2 : 1;
    const LdsLayout L = lds_layout(f_type, ns, split / kTile, false, G);
    if (L.total > kMaxLds) return false;
    // bf16: B_v is staged in the upper half of the staging rows during the merge
    if (f_type == kBF16 && L.merge_end > L.stage + kWaves / 2 * 128 * stage_pitch(kBF16)) return false;
    if (is_q(f_type) && L.bvrows + 128 * kD * 2 > L.bvraw) return false;
    if (has_tail) {
        const int tns = tail_type == kF32 ? 2 : 1;
        if (lds_layout(tail_type, tns, split / kTile, true, G).total > kMaxLds) return false;
    }
    return true;
}

size_t decode_table_bytes() {
    return (64 * sizeof(double) + (32 + kMaxTiles) * 64 * sizeof(float2) + 255) / 256 * 256;
}

size_t decode_workspace_bytes(const DecodeParams &p) {
    const size_t n = static_cast<size_t>(p.batch) * p.n_kv_heads * p.n_splits * p.group;
    const size_t ml = (n * 2 * sizeof(float) + 255) / 256 * 256;
    const size_t po = (n * kD * sizeof(float) + 255) / 256 * 256;
    return ml + po + decode_table_bytes();
}

hipError_t launch_decode_tables(const DecodeParams &p, hipStream_t st) {
    hipLaunchKernelGGL(decode_tables_kernel, dim3(kMaxTiles * 64 / 256), dim3(256), 0, st, p.rope_base, p.theta,
                       p.rope_tab, p.step_tab);
    return hipGetLastError();
}

hipError_t launch_decode_combine(const DecodeParams &p, hipStream_t st) {
    const dim3 cgrid(static_cast<unsigned>(p.n_q_heads), static_cast<unsigned>(p.batch));
    if (p.out_type == kF32)
        hipLaunchKernelGGL(decode_combine_kernel<kF32>, cgrid, dim3(kD * kCG), 0, st, p);
    else
        hipLaunchKernelGGL(decode_combine_kernel<kBF16>, cgrid, dim3(kD * kCG), 0, st, p);
    return hipGetLastError();
}

hipError_t launch_decode(const DecodeParams &p, hipStream_t st) {
    if (p.n_splits == 0) return hipSuccess;
    if (p.n_sel * p.block_splits == 0 || p.f_type == kBF16) return launch_decode_f<kBF16>(p, st);
    if (p.f_type == kI8) return launch_decode_f<kI8>(p, st);
    if (p.f_type == kI4) return launch_decode_f<kI4>(p, st);
    if (p.f_type == kI2) return launch_decode_f<kI2>(p, st);
    return launch_decode_f<kF32>(p, st);
}

}  // namespace milo
