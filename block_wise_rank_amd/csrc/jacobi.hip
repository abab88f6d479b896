// Batched symmetric eigensolve of 128 x 128 Gram matrices by cyclic two-sided
// Jacobi; the matrix lives in LDS and the eigenvectors in registers.
//
// A Jacobi rotation of the pair (p, q) of G = X^T X is the same rotation a
// one-sided (Hestenes) Jacobi step applies to columns p, q of X, computed from
// alpha = G_pp, beta = G_qq, gamma = G_pq (Golub & Van Loan, Matrix
// Computations, sec. 8.5 and 8.6): zeta = (beta - alpha) / (2 gamma),
// t = sign(zeta) / (|zeta| + sqrt(1 + zeta^2)), c = 1/sqrt(1 + t^2), s = c t;
// afterwards G_pp = alpha - t gamma, G_qq = beta + t gamma, G_pq = 0.
//
// Ordering: the round-robin ("circle") tournament.  Positions 0..127 form 64
// slots, slot P = positions (P, 127 - P) (its first and second row); in round
// k position 0 holds index 0 and position i >= 1 holds index
// 1 + (i - 1 + k) mod 127.  One round's 64 pairs are disjoint, so their
// rotations commute and are applied together; 127 rounds make a sweep, after
// which every index is back at its starting position.  Between rounds the
// index at position i >= 2 moves to position i - 1, the one at position 1 to
// position 127, and index 0 stays.
//
// Everything is kept in position space, where that movement is the same in
// every round:
//  * Eigenvectors: wave w holds slots 8w .. 8w + 7, both rows of each slot, two
//    components per lane.  A rotation is lane-local; between rounds the rows
//    shift one slot along the ring (first rows down, second rows up), inside
//    the registers except for the 14 rows that cross a wave boundary, which go
//    through a small double-buffered LDS exchange area.
//  * Off-diagonal 2 x 2 blocks of G between slots P < Q (2016 of them): four
//    role arrays (first-first, first-second, second-first, second-second), each
//    indexed by block, double-buffered.  After a round's rotation every element
//    moves to the block and role its two positions have in the next round: a
//    fixed permutation, tabulated at compile time.  A lane reads its blocks and
//    writes the rotated elements to their next places in the other buffer;
//    neighbouring lanes own neighbouring blocks, so both sides are consecutive
//    words (no bank conflicts) and no address depends on the round.
//  * Each pair's own element G_pq (positions P and 127 - P) is not in a block:
//    it is kept in a register of the lane that computes that pair's rotation.
//  * Rotation parameters: the element of the pair that slot P' holds in round
//    k + 1 is the second-first element of block (P' - 1, P' + 1) of round k (the
//    ends of the ring differ slightly), and its new diagonal entries come from
//    the rotations of pairs P' - 1 and P' + 1.  Wave 7's lane P' rotates that
//    block in round k and immediately computes round k + 1's rotation of pair
//    P'; parameters are double-buffered in LDS, the other per-pair state stays
//    in wave 7's registers.  One barrier per round.
//
// Scaled rotations (the square-root-free bookkeeping of "fast Givens", Golub &
// Van Loan sec. 5.1.13, applied to both sides): the row and column of G and
// the row of V^T at a position are stored divided by a scale s.  The rotation
// (c, s = c t) of pair (p, q) then becomes R_p <- R_p - alpha R_q,
// R_q <- beta R_p + R_q with alpha = t s_q / s_p, beta = t s_p / s_q, and
// s_p, s_q <- c s_p, c s_q: two FMAs per element instead of four products.
// Scales only shrink (c >= 1/sqrt 2), so after rounds 63 and 126 of a sweep G
// and V^T are multiplied back by them and the scales restart at 1; stored
// values stay within 2^32 of the true ones.  Rotation parameters are computed
// from true values (diagonal entries are tracked unscaled, g = s_p s_q G_pq).
//
// A pair whose rotation is the identity has alpha = beta = 0, which moves its
// rows unchanged.  Cyclic Jacobi converges quadratically once the off-diagonal
// part is small (Golub & Van Loan sec. 8.5.3): a sweep whose every relative
// off-diagonal |g| / sqrt|a b| was at most stop_tol leaves them near
// stop_tol^2, so with stop_tol = sqrt(tol) such a sweep ends the solve without
// the sweep that would only confirm it.
#include "common.hpp"
#include "kernels.hpp"

namespace milo {
namespace {

constexpr int kThreads = 512;                     // 8 waves
constexpr int kNW = kThreads / 64;
constexpr int kBlocks = 64 * 63 / 2;              // 2016 off-diagonal 2 x 2 blocks
constexpr int kGeneric = kBlocks - 64;            // blocks not feeding the next round's rotations
constexpr int kGenLanes = kThreads - 64;          // waves 0..6 (wave 7 computes the next round's rotations)
constexpr int kPerLane = (kGeneric + kGenLanes - 1) / kGenLanes;
constexpr int kRoleWords = kBlocks;               // one role array
constexpr int kBufWords = 4 * kRoleWords;         // one buffer of G
constexpr int kGBytes = 2 * kBufWords * 4;
constexpr int kPrmBytes = 2 * 64 * 8;             // (alpha, beta) per pair, double-buffered
constexpr int kXchBytes = 2 * 2 * (kNW - 1) * 64 * 8;
constexpr int kStabBytes = 128 * 4;               // scales by position at renormalisation
constexpr int kRecBytes = 64 * 16;                // per pair (new a, new b, scale a, scale b)
constexpr int kLdsBytes = kGBytes + kPrmBytes + kXchBytes + kStabBytes + 16 + kRecBytes;  // + flags
static_assert(kLdsBytes <= 80 * 1024, "two workgroups per CU");
static_assert(kPerLane == 5, "generic block slots per lane");
static_assert(kBufWords * 4 < 65536, "16-bit byte offsets within a buffer");

// ---- the tournament in position space (compile time) ----
constexpr int next_pos(int p) { return p == 0 ? 0 : (p == 1 ? 127 : p - 1); }
constexpr int slot_of(int p) { return p <= 63 ? p : 127 - p; }
constexpr int role_of(int p) { return p <= 63 ? 0 : 1; }  // 0: first row, 1: second row
constexpr int pos_of(int slot, int role) { return role == 0 ? slot : 127 - slot; }
constexpr int rowmajor_index(int P, int Q) { return P * 63 - P * (P - 1) / 2 + (Q - P - 1); }  // P < Q
// The next round's pair P' lies in block (Pa, Pb) of this round, element role kSel.
constexpr int next_pair_a(int Pn) { return Pn == 0 ? 0 : (Pn == 63 ? 62 : Pn - 1); }
constexpr int next_pair_b(int Pn) { return Pn == 0 ? 1 : (Pn == 63 ? 63 : Pn + 1); }
constexpr int next_pair_role(int Pn) { return Pn == 0 ? 0 : (Pn == 63 ? 3 : 2); }
constexpr bool next_pair_block(int P, int Q) {
    return Q == P + 2 || (P == 0 && Q == 1) || (P == 62 && Q == 63);
}
// Storage index of block (P, Q), P < Q: the 64 next-pair blocks first, in the
// order of the pair they feed (so wave 7's lanes read consecutive words), then
// the generic blocks in row-major order.
constexpr int block_index(int P, int Q) {
    if (next_pair_block(P, Q)) return P == 0 && Q == 1 ? 0 : (P == 62 && Q == 63 ? 63 : P + 1);
    // next-pair blocks before (P, Q) in row-major order: (0, 1), (p, p + 2) for
    // p < P, and (P, P + 2) when it precedes Q
    const int before = 1 + (P < 62 ? P : 62) + (P <= 61 && P + 2 < Q ? 1 : 0);
    return 64 + rowmajor_index(P, Q) - before;
}
// Word offset (role * kRoleWords + block) of the element at positions (a, b),
// or -1 - slot when both positions are one slot's pair.
constexpr int element_word(int a, int b) {
    const int sa = slot_of(a), sb = slot_of(b);
    if (sa == sb) return -1 - sa;
    return sa < sb ? (2 * role_of(a) + role_of(b)) * kRoleWords + block_index(sa, sb)
                   : (2 * role_of(b) + role_of(a)) * kRoleWords + block_index(sb, sa);
}

struct Tables {
    uint16_t pq[kBlocks];          // P | Q << 8 of block i
    uint16_t gen[kGeneric];        // generic blocks, row-major
    uint16_t dst[kBlocks][4];      // next-round byte offset (within a buffer) of each role
    uint16_t pair_dst[64];         // next-round byte offset of pair P's own element
};

constexpr Tables make_tables() {
    Tables t{};
    int n = 0, g = 0;
    for (int P = 0; P < 64; ++P)
        for (int Q = P + 1; Q < 64; ++Q) {
            const int b = block_index(P, Q);
            t.pq[b] = static_cast<uint16_t>(P | (Q << 8));
            if (!next_pair_block(P, Q)) t.gen[g++] = static_cast<uint16_t>(b);
            for (int r = 0; r < 4; ++r) {
                const int w = element_word(next_pos(pos_of(P, r >> 1)), next_pos(pos_of(Q, r & 1)));
                t.dst[b][r] = static_cast<uint16_t>(w >= 0 ? 4 * w : 0xffff);  // 0xffff: a pair's element
            }
            ++n;
        }
    for (int P = 0; P < 64; ++P)
        t.pair_dst[P] = static_cast<uint16_t>(4 * element_word(next_pos(P), next_pos(127 - P)));
    return t;
}

__constant__ Tables kTab = make_tables();

// Compile-time checks of the move map: the pair elements of round k + 1 come
// exactly from the next-pair blocks' selected roles, generic blocks only move
// into blocks, and every pair element moves into a block.
constexpr bool check_tables() {
    const Tables t = make_tables();
    for (int Pn = 0; Pn < 64; ++Pn) {
        const int b = block_index(next_pair_a(Pn), next_pair_b(Pn));
        if (b != Pn) return false;
        if (element_word(next_pos(pos_of(next_pair_a(Pn), next_pair_role(Pn) >> 1)),
                         next_pos(pos_of(next_pair_b(Pn), next_pair_role(Pn) & 1))) != -1 - Pn)
            return false;
        if (t.dst[b][next_pair_role(Pn)] != 0xffff) return false;
        if (element_word(next_pos(Pn), next_pos(127 - Pn)) < 0) return false;
    }
    for (int i = 0; i < kGeneric; ++i) {
        if (t.gen[i] != 64 + i) return false;
        for (int r = 0; r < 4; ++r)
            if (t.dst[t.gen[i]][r] == 0xffff) return false;
    }
    return true;
}
static_assert(check_tables(), "position-space move map");

__device__ __forceinline__ float &lds_at(uint8_t *base, unsigned byte_off) {
    return *reinterpret_cast<float *>(base + byte_off);
}

struct Rot {
    float c, t, na, nb;
    bool rot;
};

// Rotation annihilating g of the 2 x 2 block [a g; g b] (identity below tolerance).
__device__ __forceinline__ Rot jacobi_rotation(float a, float b, float g, float tol) {
    Rot r{1.f, 0.f, a, b, false};  // (c, t, new a, new b)
    if (g != 0.f && g * g > tol * tol * fabsf(a * b)) {
        // Any (c, s) with c^2 + s^2 = 1 to working precision keeps the transform
        // orthogonal, so 1-ulp reciprocals are enough here.
        const float zeta = 0.5f * (b - a) * __builtin_amdgcn_rcpf(g);
        const float az = fabsf(zeta);
        const float t = az > 1e18f ? 0.5f * __builtin_amdgcn_rcpf(zeta)
                                   : copysignf(__builtin_amdgcn_rcpf(az + sqrtf(1.f + zeta * zeta)), zeta);
        if (t != 0.f) {  // an infinite zeta (g negligible next to b - a) needs no rotation
            r.c = __builtin_amdgcn_rsqf(1.f + t * t);
            r.t = t;
            r.na = a - t * g;
            r.nb = b + t * g;
            r.rot = true;
        }
    }
    return r;
}

// (g0, g1, g2, g3) = (first-first, first-second, second-first, second-second)
// of block (P, Q): rows by pair P's (alpha, beta), then columns by pair Q's.
__device__ __forceinline__ void rotate_block(float (&g)[4], float2 p, float2 q) {
    const float h11 = fmaf(-p.x, g[2], g[0]), h12 = fmaf(-p.x, g[3], g[1]);
    const float h21 = fmaf(p.y, g[0], g[2]), h22 = fmaf(p.y, g[1], g[3]);
    g[0] = fmaf(-q.x, h12, h11);
    g[1] = fmaf(q.y, h11, h12);
    g[2] = fmaf(-q.x, h22, h21);
    g[3] = fmaf(q.y, h21, h22);
}

__global__ __launch_bounds__(kThreads, 4) void jacobi_kernel(const float *__restrict__ gpart, int splits,
                                                             float *__restrict__ vt_out,
                                                             int32_t *__restrict__ sweeps_out,
                                                             int max_sweeps, float tol, float stop_tol) {
    extern __shared__ __align__(16) uint8_t smem[];
    uint8_t *G = smem;                                                        // [2][4][kBlocks]
    float2 *prm = reinterpret_cast<float2 *>(smem + kGBytes);                 // [2][64] (alpha, beta)
    float2 *xch = reinterpret_cast<float2 *>(smem + kGBytes + kPrmBytes);     // [2][2][7][64]
    float *stab = reinterpret_cast<float *>(smem + kGBytes + kPrmBytes + kXchBytes);  // [128]
    int *flags = reinterpret_cast<int *>(smem + kGBytes + kPrmBytes + kXchBytes + kStabBytes);
    // Per pair, after the current round's rotation: its diagonal entries (true)
    // and the scales of its first and second row.  Only wave 7 touches it; a
    // round reads its neighbours' entries before any lane rewrites its own, so
    // one buffer suffices.
    float4 *rec = reinterpret_cast<float4 *>(smem + kGBytes + kPrmBytes + kXchBytes + kStabBytes + 16);

    const int blk = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const float *src = gpart + static_cast<int64_t>(blk) * splits * kD * kD;
    auto gram = [&](int a, int b) {
        float s = 0.f;
        for (int p = 0; p < splits; ++p) s += src[static_cast<int64_t>(p) * kD * kD + a * kD + b];
        return s;
    };
    // Round 0: position = index, so block (P, Q) role r holds G[pos(P)][pos(Q)].
    for (int e = tid; e < kBufWords; e += kThreads) {
        const int r = e / kRoleWords, b = e - r * kRoleWords;
        const int code = kTab.pq[b];
        reinterpret_cast<float *>(G)[e] = gram(pos_of(code & 0xff, r >> 1), pos_of(code >> 8, r & 1));
    }
    if (tid == 0) {
        flags[0] = 0;
        flags[1] = 0;
    }

    // Wave 7 state of pair Pn = lane: its own element (stored form, before this
    // round's rotation) and whether this round rotates it.
    const int Pn = lane;
    const int Pa = next_pair_a(Pn), Pb = next_pair_b(Pn), sel = next_pair_role(Pn);
    const int sblk = block_index(Pa, Pb);  // = Pn
    float gp = 0.f;
    bool rotp = false;
    if (wave == kNW - 1) {
        const float a = gram(Pn, Pn), b = gram(127 - Pn, 127 - Pn);
        gp = gram(Pn, 127 - Pn);
        const Rot r = jacobi_rotation(a, b, gp, tol);  // scales start at 1: alpha = beta = t
        prm[Pn] = make_float2(r.t, r.t);
        rec[Pn] = make_float4(r.na, r.nb, r.c, r.c);
        rotp = r.rot;
        if (r.rot && gp * gp > stop_tol * stop_tol * fabsf(a * b)) flags[0] = 1;
    }

    // Eigenvector rows of this wave's slots: F = first rows, S = second rows
    // (components 2 lane, 2 lane + 1); initially slot P holds indices P, 127 - P.
    float2 F[8], S[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int P = 8 * wave + j, c0 = 2 * lane;
        F[j] = make_float2(c0 == P ? 1.f : 0.f, c0 + 1 == P ? 1.f : 0.f);
        S[j] = make_float2(c0 == 127 - P ? 1.f : 0.f, c0 + 1 == 127 - P ? 1.f : 0.f);
    }
    // Generic blocks of this lane (waves 0..6): entries tid, tid + 448, ... of the
    // generic list.  code = P | Q << 6 | block << 12; dst = next byte offsets of
    // the four roles, two per word.
    int code[kPerLane];
    uint32_t dst[kPerLane][2];
#pragma unroll
    for (int j = 0; j < kPerLane; ++j) {
        const int i = tid + kGenLanes * j;
        const bool has = wave < kNW - 1 && i < kGeneric;
        const int b = has ? kTab.gen[i] : 0;
        const int pq = kTab.pq[b];
        code[j] = (pq & 0xff) | ((pq >> 8) << 6) | (b << 12);
        dst[j][0] = kTab.dst[b][0] | (static_cast<uint32_t>(kTab.dst[b][1]) << 16);
        dst[j][1] = kTab.dst[b][2] | (static_cast<uint32_t>(kTab.dst[b][3]) << 16);
    }
    const bool has4 = wave < kNW - 1 && tid + kGenLanes * (kPerLane - 1) < kGeneric;  // slot 4 is partial
    // wave 7: next places of the special block's three other roles and of the
    // pair's own element
    const uint32_t sdst0 = kTab.dst[sblk][0] | (static_cast<uint32_t>(kTab.dst[sblk][1]) << 16);
    const uint32_t sdst1 = kTab.dst[sblk][2] | (static_cast<uint32_t>(kTab.dst[sblk][3]) << 16);
    const uint32_t pdst = kTab.pair_dst[Pn];
    __syncthreads();

    int used = -max_sweeps;
    int gk = 0;  // rounds done so far (parity selects the buffers)
    for (int sweep = 0; sweep < max_sweeps; ++sweep) {
        for (int kr = 0; kr < 127; ++kr, ++gk) {
            int k = kr;
            asm volatile("" : "+s"(k));
            const int cb = gk & 1;
            const float2 *pc = prm + cb * 64;
            uint8_t *cur = G + cb * (kBufWords * 4);
            uint8_t *nxt = G + (cb ^ 1) * (kBufWords * 4);
            // rounds after which G and V^T are multiplied back by their scales
            const bool renorm = (k == 63) | (k == 126);
            const bool last_round = (k == 126);

            // ---- eigenvector rows: rotate (identity when alpha = beta = 0), shift
            // along the ring, send the ends
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float2 ab = pc[8 * wave + j];
                const float2 f = F[j], s = S[j];
                F[j] = make_float2(fmaf(-ab.x, s.x, f.x), fmaf(-ab.x, s.y, f.y));
                S[j] = make_float2(fmaf(ab.y, f.x, s.x), fmaf(ab.y, f.y, s.y));
            }
            // Round k + 1's position i holds round k's position i + 1 (127 -> 1 wraps
            // to 1 -> 127): first rows move down one slot, second rows up one slot.
            float2 *xo = xch + cb * 2 * (kNW - 1) * 64;
            if (wave > 0) xo[(wave - 1) * 64 + lane] = F[0];
            if (wave < kNW - 1) xo[((kNW - 1) + wave) * 64 + lane] = S[7];
            {
                const float2 f1 = F[1], s7 = S[7];
#pragma unroll
                for (int j = 0; j < 7; ++j)
                    if (j > 0 || wave > 0) F[j] = F[j + 1];  // index 0 never moves
                if (wave == kNW - 1) F[7] = s7;
#pragma unroll
                for (int j = 7; j >= 1; --j) S[j] = S[j - 1];
                if (wave == 0) S[0] = f1;
            }

            if (wave == kNW - 1) {
                __builtin_amdgcn_s_setprio(2);  // the round's longest chain goes first on its SIMD
                // ---- wave 7: this pair's own element moves into a block; block
                // (Pa, Pb) is rotated, its selected element becomes the element of
                // round k + 1's pair Pn, whose rotation is computed here.
                lds_at(nxt, pdst) = rotp ? 0.f : gp;
                const float2 A = pc[Pa], B = pc[Pb];
                const float4 RA = rec[Pa], RB = rec[Pb];
                float h[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) h[e] = lds_at(cur, (e * kRoleWords + sblk) * 4);
                rotate_block(h, A, B);
                // the other three roles move on (the selected one's slot is unused)
                const float gn = sel == 0 ? h[0] : (sel == 2 ? h[2] : h[3]);
                if (sel != 0) lds_at(nxt, sdst0 & 0xffffu) = h[0];
                lds_at(nxt, sdst0 >> 16) = h[1];
                if (sel != 2) lds_at(nxt, sdst1 & 0xffffu) = h[2];
                if (sel != 3) lds_at(nxt, sdst1 >> 16) = h[3];
                // new diagonal entries and scales of the rows that form pair Pn next
                // round (pair Pa's second row and pair Pb's first row; ends differ)
                const float an = Pn == 0 ? RA.x : (Pn == 63 ? RB.y : RB.x);
                const float bn = Pn == 0 ? RB.x : RA.y;
                const float sfa = Pn == 0 ? RA.z : (Pn == 63 ? RB.w : RB.z);
                const float sfb = Pn == 0 ? RB.z : RA.w;
                const float gt = gn * sfa * sfb;
                Rot r = jacobi_rotation(an, bn, gt, tol);
                float s1 = sfa, s2 = sfb;
                gp = gn;
                if (renorm) {  // uniform: scales gathered by next-round position, restart at 1
                    stab[Pn] = sfa;
                    stab[127 - Pn] = sfb;
                    s1 = s2 = 1.f;
                    gp = gn * sfa * sfb;
                }
                float al = r.t * (s2 * __builtin_amdgcn_rcpf(s1)), be = r.t * (s1 * __builtin_amdgcn_rcpf(s2));
                if ((al == 0.f) | (be == 0.f)) {  // negligible rotation: none
                    r = Rot{1.f, 0.f, an, bn, false};
                    al = be = 0.f;
                }
                prm[(cb ^ 1) * 64 + Pn] = make_float2(al, be);
                rec[Pn] = make_float4(r.na, r.nb, s1 * r.c, s2 * r.c);
                rotp = r.rot;
                if (r.rot && gt * gt > stop_tol * stop_tol * fabsf(an * bn))
                    flags[(sweep + (last_round ? 1 : 0)) & 1] = 1;
                __builtin_amdgcn_s_setprio(0);
            } else {
                // ---- waves 0..6: generic blocks, two at a time (loads, then stores)
#pragma unroll
                for (int j0 = 0; j0 < kPerLane; j0 += 2) {
                    const int nb = j0 + 2 <= kPerLane ? 2 : kPerLane - j0;
                    float g[2][4];
                    float2 cp[2], cq[2];
                    bool on[2];
#pragma unroll
                    for (int i = 0; i < nb; ++i) {
                        const int c = code[j0 + i];
                        on[i] = j0 + i < kPerLane - 1 || has4;
                        cp[i] = pc[c & 63];
                        cq[i] = pc[(c >> 6) & 63];
                        if (on[i]) {
#pragma unroll
                            for (int e = 0; e < 4; ++e) g[i][e] = lds_at(cur, (e * kRoleWords + (c >> 12)) * 4);
                        }
                    }
#pragma unroll
                    for (int i = 0; i < nb; ++i)
                        if (on[i]) {
                            rotate_block(g[i], cp[i], cq[i]);
                            lds_at(nxt, dst[j0 + i][0] & 0xffffu) = g[i][0];
                            lds_at(nxt, dst[j0 + i][0] >> 16) = g[i][1];
                            lds_at(nxt, dst[j0 + i][1] & 0xffffu) = g[i][2];
                            lds_at(nxt, dst[j0 + i][1] >> 16) = g[i][3];
                        }
                }
            }
            if (k == 1 && tid == 0) flags[(sweep + 1) & 1] = 0;
            __syncthreads();

            // ---- receive the rows that crossed a wave boundary
            const float2 *xi = xch + cb * 2 * (kNW - 1) * 64;
            if (wave < kNW - 1) F[7] = xi[wave * 64 + lane];
            if (wave > 0) S[0] = xi[((kNW - 1) + wave - 1) * 64 + lane];

            // ---- multiply G and V^T back by the scales (gathered by position above)
            if (renorm) {
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const float sf = stab[8 * wave + j], ss = stab[127 - 8 * wave - j];
                    F[j] = make_float2(F[j].x * sf, F[j].y * sf);
                    S[j] = make_float2(S[j].x * ss, S[j].y * ss);
                }
                float *gn = reinterpret_cast<float *>(nxt);
                for (int e = tid; e < kBufWords; e += kThreads) {
                    const int r = e / kRoleWords, b = e - r * kRoleWords;
                    const int pq = kTab.pq[b];
                    gn[e] *= stab[pos_of(pq & 0xff, r >> 1)] * stab[pos_of(pq >> 8, r & 1)];
                }
                __syncthreads();
            }
        }
        const int rot = flags[sweep & 1];
        if (!rot) {
            used = sweep + 1;
            break;
        }
    }

    // 127 rounds per sweep: slot P again holds indices P and 127 - P.
    float2 *dstv = reinterpret_cast<float2 *>(vt_out + static_cast<int64_t>(blk) * kD * kD);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int P = 8 * wave + j;
        dstv[P * 64 + lane] = F[j];
        dstv[(127 - P) * 64 + lane] = S[j];
    }
    if (tid == 0 && sweeps_out) sweeps_out[blk] = used;
}

}  // namespace

hipError_t launch_jacobi(const float *gpart, int splits, int n_blocks, float *vt, int32_t *sweeps,
                         int max_sweeps, float tol, float stop_tol, hipStream_t st) {
    if (n_blocks <= 0) return hipSuccess;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(jacobi_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(jacobi_kernel, dim3(static_cast<unsigned>(n_blocks)), dim3(kThreads), kLdsBytes, st,
                       gpart, splits, vt, sweeps, max_sweeps, tol, stop_tol);
    return hipGetLastError();
}

}  // namespace milo
