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
// rows unchanged.  The solve ends at the first half of a sweep (after round
// 63 or 126, where the scales are folded back anyway) that closes 127
// consecutive rounds, every pair once, in which every relative off-diagonal
// |g| / sqrt|a b| was at most stop_tol, without the rounds that would only
// confirm it: cyclic Jacobi converges quadratically once the
// off-diagonal part is small (Golub & Van Loan sec. 8.5.3), but for clustered
// eigenvalues that says little about each eigenvector.  The accuracy of the
// singular values rests instead on the pass that follows, which recomputes
// them as Rayleigh quotients ||X v|| (second order in the eigenvector error,
// and within a cluster a mix of nearly equal values); stop_tol is chosen by
// measurement against the oracle.
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
constexpr int kBatch = 2;                         // generic blocks whose loads are issued together
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
static_assert(check_tables(), "position-space move map");  // includes gen[i] == 64 + i


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

// LDS of one workgroup; static, so that its address is known and every offset
// below folds into the LDS instructions' immediate field.
__shared__ __align__(16) uint8_t g_lds[kLdsBytes];
constexpr int kPrmOff = kGBytes;                                   // [2][64] (alpha, beta)
constexpr int kXchOff = kPrmOff + kPrmBytes;                       // [2][2][7][64] rows crossing waves
constexpr int kStabOff = kXchOff + kXchBytes;                      // [128] scales by position
constexpr int kFlagOff = kStabOff + kStabBytes;                    // "this half sweep ends the solve"
// Per pair, after the current round's rotation: its diagonal entries (true) and
// the scales of its first and second row.  Only wave 7 touches it; a round reads
// its neighbours' entries before any lane rewrites its own, so one buffer suffices.
constexpr int kRecOff = kFlagOff + 16;
__device__ __forceinline__ float &lds_f(uint32_t byte_off) { return *reinterpret_cast<float *>(g_lds + byte_off); }
__device__ __forceinline__ float2 &lds_f2(uint32_t byte_off) { return *reinterpret_cast<float2 *>(g_lds + byte_off); }
__device__ __forceinline__ float4 &lds_f4(uint32_t byte_off) { return *reinterpret_cast<float4 *>(g_lds + byte_off); }
__device__ __forceinline__ int &lds_i(uint32_t byte_off) { return *reinterpret_cast<int *>(g_lds + byte_off); }

// Registers of one lane for the whole solve.
struct LaneState {
    // Eigenvector rows of this wave's slots (components 2 lane, 2 lane + 1): F =
    // first rows, S = second rows.  The rows of a wave move one slot per round
    // along its F and S rings; the rings are renamed instead of moved: in phase
    // ph (= rounds done mod 8) logical first-row slot j lives in F[(j + ph) & 7]
    // and logical second-row slot j in S[(j - ph) & 7].
    float2 F[8], S[8];
    // Byte offsets of this lane's blocks, kept unpacked so that every LDS access
    // of a round is one register plus an immediate (the buffer's offset).
    // Waves 0..6, generic slot j = entry tid + 448 j of the generic list, i.e.
    // block 64 + tid + 448 j: gb = slot 0's read offset (slot j's is gb + 1792 j),
    // pq = the (alpha, beta) offsets of P and Q (low and high half), d = the
    // next-round offsets of its four roles (two per word).  Wave 7 (no generic
    // blocks) keeps in gb and d[0] the special block's read offset and next-round
    // role offsets, in pq[1] the pair element's next-round offset, and in d[1],
    // d[2] and d[3] its pair's (alpha, beta) and record (see the round below).
    uint32_t gb, pq[kPerLane], d[kPerLane][2];
    float gp;    // wave 7: this pair's own element (stored form, before this round's rotation)
    bool rotp;   // wave 7: whether this round rotates it
    bool has4;   // generic slot 4 is in use (it is partial)
};

struct Solve {
    int k, sweep, used;     // round within the sweep, sweeps done, result (rounds)
    int run;                // wave 7: consecutive rounds below stop_tol, the next round included
    bool fin;               // wave 7: the next round ends the solve
    int wave, lane, tid, sel, blk, max_sweeps;
    float tol, stop_tol;
    float *vt_out;
    int32_t *sweeps_out;
};

// V^T rows out, by position after the last round (after whole sweeps slot P
// holds indices P and 127 - P again, otherwise a permutation of them: the
// refine pass that follows sorts the vectors by their singular values).
template <int NPH>
__device__ __forceinline__ void write_rows(const LaneState &L, const Solve &C, int ln) {
    float2 *dstv = reinterpret_cast<float2 *>(C.vt_out + static_cast<int64_t>(C.blk) * kD * kD) + ln;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int P = 8 * C.wave + j;
        dstv[P * 64] = L.F[(j + NPH) & 7];
        dstv[(127 - P) * 64] = L.S[(j - NPH) & 7];
    }
}

// Eigenvector rows of one round: rotate (identity when alpha = beta = 0), shift
// along the ring, send the ends.  pc = this round's (alpha, beta) table.
template <int PH>
__device__ __forceinline__ void rotate_rows(LaneState &L, uint32_t pc, int wave, int ln, uint32_t xb) {
    constexpr int f0 = PH & 7, f1 = (PH + 1) & 7, s7 = (7 - PH) & 7;
    float4 ab[4];  // this wave's eight pairs, as broadcast reads
#pragma unroll
    for (int j = 0; j < 4; ++j) ab[j] = lds_f4(pc + 64 * wave + 16 * j);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const float al = (j & 1) ? ab[j >> 1].z : ab[j >> 1].x;
        const float be = (j & 1) ? ab[j >> 1].w : ab[j >> 1].y;
        float2 &fr = L.F[(j + PH) & 7], &sr = L.S[(j - PH) & 7];
        const float2 f = fr, s = sr;
        fr = make_float2(fmaf(-al, s.x, f.x), fmaf(-al, s.y, f.y));
        sr = make_float2(fmaf(be, f.x, s.x), fmaf(be, f.y, s.y));
    }
    // computed here (not sunk past the barrier, where they would cost copies)
    asm volatile("" : "+v"(L.F[0]), "+v"(L.F[1]), "+v"(L.F[2]), "+v"(L.F[3]), "+v"(L.F[4]), "+v"(L.F[5]),
                      "+v"(L.F[6]), "+v"(L.F[7]));
    asm volatile("" : "+v"(L.S[0]), "+v"(L.S[1]), "+v"(L.S[2]), "+v"(L.S[3]), "+v"(L.S[4]), "+v"(L.S[5]),
                      "+v"(L.S[6]), "+v"(L.S[7]));
    // Round k + 1's position i holds round k's position i + 1 (127 -> 1 wraps to
    // 1 -> 127): first rows move down one slot, second rows up one slot.  After
    // the renaming, F[f0] is logical slot 7 and S[s7] logical slot 0.
    if (wave > 0) lds_f2(xb + 8 * ((wave - 1) * 64 + ln)) = L.F[f0];
    if (wave < kNW - 1) lds_f2(xb + 8 * (((kNW - 1) + wave) * 64 + ln)) = L.S[s7];
    if (wave == 0) {  // position 0 stays, position 1 wraps to 127 (this wave's S slot 0)
        const float2 p1 = L.F[f1];
        L.F[f1] = L.F[f0];
        L.S[s7] = p1;
    }
    if (wave == kNW - 1) L.F[f0] = L.S[s7];  // position 64 -> 63
}

// Lane l of wave 7 receives the value of lane l - 1 (shr) or l + 1 (shl); the
// end lane keeps its own, which is what pairs 0 and 63 need.
__device__ __forceinline__ float lane_prev(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), 0x138, 0xf, 0xf, false));
}
__device__ __forceinline__ float lane_next(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), 0x130, 0xf, 0xf, false));
}

// One round of the tournament in phase PH; true once the solve has ended (the
// rows are then written out).
template <int PH>
__device__ __forceinline__ bool jacobi_round(LaneState &L, Solve &C) {
    constexpr int cb = PH & 1;                        // buffer parity
    constexpr uint32_t cur = cb * (kBufWords * 4), nxt = (cb ^ 1) * (kBufWords * 4);
    constexpr uint32_t pc = kPrmOff + cb * 512, pn = kPrmOff + (cb ^ 1) * 512;
    constexpr uint32_t xb = kXchOff + cb * (2 * (kNW - 1) * 64 * 8);
    constexpr int f0 = PH & 7, f1 = (PH + 1) & 7, s7 = (7 - PH) & 7;
    const int wave = C.wave;
    int k = C.k;
    asm volatile("" : "+s"(k));
    int ln = C.lane;
    asm volatile("" : "+v"(ln));
    // unpacked in every round: hoisted out of the loop the halves would take
    // registers the round needs
#pragma unroll
    for (int j = 0; j < kPerLane; ++j) asm volatile("" : "+v"(L.pq[j]), "+v"(L.d[j][0]), "+v"(L.d[j][1]));
    // rounds after which G and V^T are multiplied back by their scales, and
    // after which the solve can end (wave 7 knows it one round ahead and
    // flags it; the others read the flag after the round)
    const bool renorm = (k == 63) | (k == 126);
    const bool last_round = (k == 126);

    if (wave == kNW - 1) {
        __builtin_amdgcn_s_setprio(2);  // the round's longest chain goes first on its SIMD
        // ---- wave 7: this pair's own element moves into a block; block (Pa, Pb)
        // is rotated, its selected element becomes the element of round k + 1's
        // pair Pn = lane, whose rotation is computed here.
        const int sel = C.sel;
        // the special block, written last round by the lanes that moved its elements
        float h[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) h[e] = lds_f(cur + L.gb + e * kRoleWords * 4);
        lds_f(nxt + L.pq[1]) = L.rotp ? 0.f : L.gp;
        // this round's (alpha, beta) and records of pairs Pa = lane - 1 and Pb =
        // lane + 1, computed last round by those lanes (held in unused slot registers)
        const float wal = __uint_as_float(L.d[1][0]), wbe = __uint_as_float(L.d[1][1]);
        const float4 wrc = make_float4(__uint_as_float(L.d[2][0]), __uint_as_float(L.d[2][1]),
                                       __uint_as_float(L.d[3][0]), __uint_as_float(L.d[3][1]));
        // this wave's rows (pairs 56 .. 63) while the block is in flight
        rotate_rows<PH>(L, pc, wave, ln, xb);
        const float2 A = make_float2(lane_prev(wal), lane_prev(wbe)), B = make_float2(lane_next(wal), lane_next(wbe));
        rotate_block(h, A, B);
        const float4 RA = make_float4(lane_prev(wrc.x), lane_prev(wrc.y), lane_prev(wrc.z), lane_prev(wrc.w));
        const float4 RB = make_float4(lane_next(wrc.x), lane_next(wrc.y), lane_next(wrc.z), lane_next(wrc.w));
        // the other three roles move on (the selected one's slot is unused)
        const float gn = sel == 0 ? h[0] : (sel == 2 ? h[2] : h[3]);
        if (sel != 0) lds_f(nxt + (L.d[0][0] & 0xffffu)) = h[0];
        lds_f(nxt + (L.d[0][0] >> 16)) = h[1];
        if (sel != 2) lds_f(nxt + (L.d[0][1] & 0xffffu)) = h[2];
        if (sel != 3) lds_f(nxt + (L.d[0][1] >> 16)) = h[3];
        // new diagonal entries and scales of the rows that form pair Pn next round
        // (pair Pa's second row and pair Pb's first row; the ends differ)
        const bool first = ln == 0, last = ln == 63;
        const float an = first ? RA.x : (last ? RB.y : RB.x);
        const float bn = first ? RB.x : RA.y;
        const float sfa = first ? RA.z : (last ? RB.w : RB.z);
        const float sfb = first ? RB.z : RA.w;
        const float gt = gn * sfa * sfb;
        Rot r = jacobi_rotation(an, bn, gt, C.tol);
        float s1 = sfa, s2 = sfb;
        L.gp = gn;
        if (renorm) {  // uniform: scales gathered by next-round position, restart at 1
            lds_f(kStabOff + 4 * ln) = sfa;
            lds_f(kStabOff + 4 * (127 - ln)) = sfb;
            s1 = s2 = 1.f;
            L.gp = gn * sfa * sfb;
        }
        float al = r.t * (s2 * __builtin_amdgcn_rcpf(s1)), be = r.t * (s1 * __builtin_amdgcn_rcpf(s2));
        if ((al == 0.f) | (be == 0.f)) {  // negligible rotation: none
            r = Rot{1.f, 0.f, an, bn, false};
            al = be = 0.f;
        }
        lds_f2(pn + 8 * ln) = make_float2(al, be);
        L.d[1][0] = __float_as_uint(al);
        L.d[1][1] = __float_as_uint(be);
        L.d[2][0] = __float_as_uint(r.na);
        L.d[2][1] = __float_as_uint(r.nb);
        L.d[3][0] = __float_as_uint(s1 * r.c);
        L.d[3][1] = __float_as_uint(s2 * r.c);
        L.rotp = r.rot;
        // every pair once in the 127 rounds up to the next one below stop_tol,
        // and the next round ends a half sweep: it ends the solve
        const bool big = __any(r.rot && gt * gt > C.stop_tol * C.stop_tol * fabsf(an * bn));
        C.run = big ? 0 : C.run + 1;
        C.fin = C.run >= 127 && (k == 62 || k == 125);
        if (C.fin && ln == 0) lds_i(kFlagOff) = 1;
        __builtin_amdgcn_s_setprio(0);
    } else {
        rotate_rows<PH>(L, pc, wave, ln, xb);
        // ---- waves 0..6: generic blocks, kBatch at a time (loads, then stores)
#pragma unroll
        for (int j0 = 0; j0 < kPerLane; j0 += kBatch) {
            const int nb = j0 + kBatch <= kPerLane ? kBatch : kPerLane - j0;
            float g[kBatch][4];
            float2 cp[kBatch], cq[kBatch];
            bool on[kBatch];
#pragma unroll
            for (int i = 0; i < nb; ++i) {
                const int j = j0 + i;
                on[i] = j < kPerLane - 1 || L.has4;
                cp[i] = lds_f2(pc + (L.pq[j] & 0xffffu));
                cq[i] = lds_f2(pc + (L.pq[j] >> 16));
                if (on[i]) {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        g[i][e] = lds_f(cur + L.gb + 4 * kGenLanes * j + e * kRoleWords * 4);
                }
            }
#pragma unroll
            for (int i = 0; i < nb; ++i)
                if (on[i]) {
                    rotate_block(g[i], cp[i], cq[i]);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const uint32_t w = L.d[j0 + i][e >> 1];
                        lds_f(nxt + ((e & 1) ? w >> 16 : w & 0xffffu)) = g[i][e];
                    }
                }
        }
    }
    __syncthreads();

    // ---- receive the rows that crossed a wave boundary
    if (wave < kNW - 1) L.F[f0] = lds_f2(xb + 8 * (wave * 64 + ln));
    if (wave > 0) L.S[s7] = lds_f2(xb + 8 * (((kNW - 1) + wave - 1) * 64 + ln));
    // after a half sweep: does the solve end here (flag written by wave 7 last round)
    const bool final = renorm && __builtin_amdgcn_readfirstlane(lds_i(kFlagOff)) != 0;

    // ---- multiply G and V^T back by the scales (gathered by position above)
    if (renorm) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float sf = lds_f(kStabOff + 4 * (8 * wave + j)), ss = lds_f(kStabOff + 4 * (127 - 8 * wave - j));
            float2 &fr = L.F[(j + PH + 1) & 7], &sr = L.S[(j - PH - 1) & 7];
            fr = make_float2(fr.x * sf, fr.y * sf);
            sr = make_float2(sr.x * ss, sr.y * ss);
        }
        if (!final) {
            for (int e = C.tid; e < kBufWords; e += kThreads) {
                const int r = e / kRoleWords, b = e - r * kRoleWords;
                const int c = kTab.pq[b];
                lds_f(nxt + 4 * e) *= lds_f(kStabOff + 4 * pos_of(c & 0xff, r >> 1)) *
                                      lds_f(kStabOff + 4 * pos_of(c >> 8, r & 1));
            }
            __syncthreads();
        }
    }

    // ---- the end of the solve: converged, or the last round of the last sweep
    if (final || (last_round && C.sweep + 1 == C.max_sweeps)) {
        if (final) C.used = C.sweep * 127 + k + 1;
        write_rows<(PH + 1) & 7>(L, C, ln);
        if (C.tid == 0 && C.sweeps_out) C.sweeps_out[C.blk] = C.used * 64;  // 64 rotations a round
        return true;
    }
    if (last_round) {
        ++C.sweep;
        C.k = 0;
    } else {
        C.k = k + 1;
    }
    return false;
}

__global__ __launch_bounds__(kThreads, 4) void jacobi_kernel(const float *__restrict__ gpart, int splits,
                                                             float *__restrict__ vt_out,
                                                             int32_t *__restrict__ sweeps_out,
                                                             int max_sweeps, float tol, float stop_tol) {
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
        lds_f(4 * e) = gram(pos_of(code & 0xff, r >> 1), pos_of(code >> 8, r & 1));
    }
    if (tid == 0) lds_i(kFlagOff) = 0;

    LaneState L;
    const int Pn = lane;
    const int Pa = next_pair_a(Pn), Pb = next_pair_b(Pn), sel = next_pair_role(Pn);
    const int sblk = block_index(Pa, Pb);  // = Pn
    // initially slot P holds indices P, 127 - P
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int P = 8 * wave + j, c0 = 2 * lane;
        L.F[j] = make_float2(c0 == P ? 1.f : 0.f, c0 + 1 == P ? 1.f : 0.f);
        L.S[j] = make_float2(c0 == 127 - P ? 1.f : 0.f, c0 + 1 == 127 - P ? 1.f : 0.f);
    }
#pragma unroll
    for (int j = 0; j < kPerLane; ++j) {
        const int i = tid + kGenLanes * j;
        const bool has = wave < kNW - 1 && i < kGeneric;
        const int b = wave == kNW - 1 ? (j == 0 ? sblk : 0) : (has ? kTab.gen[i] : 0);
        const int c = kTab.pq[b];
        if (j == 0) L.gb = 4u * b;
        L.pq[j] = 8u * (c & 0xff) | (8u * (c >> 8)) << 16;
#pragma unroll
        for (int e = 0; e < 2; ++e) L.d[j][e] = kTab.dst[b][2 * e] | static_cast<uint32_t>(kTab.dst[b][2 * e + 1]) << 16;
    }
    if (wave == kNW - 1) L.pq[1] = kTab.pair_dst[Pn];
    // Wave 7: the rotation of pair Pn = lane for round 0; its (alpha, beta) and
    // record stay in slot registers this wave does not use otherwise.
    L.gp = 0.f;
    L.rotp = false;
    int run0 = 0;
    if (wave == kNW - 1) {
        const float a = gram(Pn, Pn), b = gram(127 - Pn, 127 - Pn);
        L.gp = gram(Pn, 127 - Pn);
        const Rot r = jacobi_rotation(a, b, L.gp, tol);  // scales start at 1: alpha = beta = t
        lds_f2(kPrmOff + 8 * Pn) = make_float2(r.t, r.t);
        L.d[1][0] = L.d[1][1] = __float_as_uint(r.t);
        L.d[2][0] = __float_as_uint(r.na);
        L.d[2][1] = __float_as_uint(r.nb);
        L.d[3][0] = L.d[3][1] = __float_as_uint(r.c);
        L.rotp = r.rot;
        run0 = __any(r.rot && L.gp * L.gp > stop_tol * stop_tol * fabsf(a * b)) ? 0 : 1;
    }
    // opaque from here on: kept as whole registers, not repacked
#pragma unroll
    for (int j = 0; j < kPerLane; ++j)
        asm volatile("" : "+v"(L.pq[j]), "+v"(L.d[j][0]), "+v"(L.d[j][1]));
    asm volatile("" : "+v"(L.gb));
    L.has4 = wave < kNW - 1 && tid + kGenLanes * (kPerLane - 1) < kGeneric;  // slot 4 is partial
    __syncthreads();

    Solve C{0, 0, -max_sweeps * 127, run0, false, wave, lane, tid, sel, blk, max_sweeps, tol, stop_tol, vt_out,
            sweeps_out};
    // The rows kept for this path spill 24 registers (written before the first
    // sweep, read after the last, outside the round loop); the builds without
    // that spill schedule the round loop worse and solve 1.6% slower.
    if (max_sweeps <= 0) {
        write_rows<0>(L, C, lane);
        if (tid == 0 && sweeps_out) sweeps_out[blk] = C.used * 64;
        return;
    }
    for (;;) {
        if (jacobi_round<0>(L, C)) return;
        if (jacobi_round<1>(L, C)) return;
        if (jacobi_round<2>(L, C)) return;
        if (jacobi_round<3>(L, C)) return;
        if (jacobi_round<4>(L, C)) return;
        if (jacobi_round<5>(L, C)) return;
        if (jacobi_round<6>(L, C)) return;
        if (jacobi_round<7>(L, C)) return;
    }
}

}  // namespace

hipError_t launch_jacobi(const float *gpart, int splits, int n_blocks, float *vt, int32_t *sweeps,
                         int max_sweeps, float tol, float stop_tol, int n_cus, hipStream_t st) {
    if (n_blocks <= 0) return hipSuccess;
    // Fewer blocks than CUs: a little dynamic LDS puts each workgroup past half
    // of a CU's LDS, so that no two share a CU (one alone runs its rounds faster,
    // and concurrent calls on other streams spread over the idle CUs instead).
    const size_t extra = n_blocks < n_cus ? 160 * 1024 / 2 - kLdsBytes + 1024 : 0;
    hipLaunchKernelGGL(jacobi_kernel, dim3(static_cast<unsigned>(n_blocks)), dim3(kThreads), extra, st,
                       gpart, splits, vt, sweeps, max_sweeps, tol, stop_tol);
    return hipGetLastError();
}

}  // namespace milo
