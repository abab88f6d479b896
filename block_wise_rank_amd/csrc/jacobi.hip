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
// slots, slot P = positions (P, 127 - P); in round k position 0 holds index 0
// and position i >= 1 holds index 1 + (i - 1 + k) mod 127.  One round's 64
// pairs are disjoint, so their rotations commute and are applied together;
// 127 rounds make a sweep.  From one round to the next every index except 0
// moves to the neighbouring position, which is what the layout exploits:
//
//  * Eigenvectors: wave w holds slots 8w .. 8w + 7, both rows of each slot, two
//    components per lane.  A rotation is lane-local; between rounds the rows
//    shift one slot along the ring (first rows down, second rows up), inside
//    the registers except for the 14 rows that cross a wave boundary, which go
//    through a small double-buffered LDS exchange area.
//  * Off-diagonal 2 x 2 blocks (slot P, slot Q), P < Q, of G: 2016 per round.
//    G's upper triangle is indexed by matrix index (pitch 129 puts G[a][b] on
//    bank (a + b) mod 32 whichever triangle is addressed).
//  * Rotation parameters: the two indices of round k + 1's pair P' sit in
//    slots P' + 1 (first row) and P' - 1 (second row) of round k (the ends of
//    the ring differ slightly), so their off-diagonal entry is an
//    element of block (P' - 1, P' + 1) and their new diagonal entries come from
//    the rotations of pairs P' - 1 and P' + 1.  The lane that rotates that block
//    in round k therefore has everything round k + 1's rotation P' needs and
//    computes it at once; parameters and new diagonal entries of every pair are
//    double-buffered in LDS.  One barrier per round.
//
// Scaled rotations (the square-root-free bookkeeping of "fast Givens", Golub &
// Van Loan sec. 5.1.13, applied to both sides): row i of G and of V^T is stored
// divided by a scale s_i.  The rotation (c, s = c t) of pair (p, q) then becomes
// R_p <- R_p - alpha R_q, R_q <- beta R_p + R_q with alpha = t s_q / s_p,
// beta = t s_p / s_q, and s_p, s_q <- c s_p, c s_q: two FMAs per element
// instead of four products.  Scales only shrink (c >= 1/sqrt 2), so every 63 or
// 64 rounds (at rounds 63 and 126 of a sweep) G and V^T are multiplied back by
// them and the scales restart at 1; stored values stay within 2^32 of the true
// ones.  Rotation parameters are computed from true values (diagonal entries
// are tracked unscaled, g = s_p s_q G_pq).
//
// Pairs whose rotation is the identity (already orthogonal to tolerance) skip
// their LDS traffic, so late sweeps cost little.  Cyclic Jacobi converges
// quadratically once the off-diagonal part is small (Golub & Van Loan sec. 8.5.3):
// a sweep whose every relative off-diagonal |g| / sqrt|a b| was at most
// stop_tol leaves them near stop_tol^2, so with stop_tol = sqrt(tol) such a
// sweep ends the solve without the sweep that would only confirm it.
// Diagonal entries are never stored in G.
#include "common.hpp"
#include "kernels.hpp"

namespace milo {
namespace {

constexpr int kGP = 129;              // LDS pitch of G (floats)
constexpr int kThreads = 512;         // 8 waves
constexpr int kNW = kThreads / 64;
constexpr int kGWords = 16384;        // G's upper triangle ends at 126 * 129 + 127
constexpr int kPrmBytes = 2 * 64 * 8;  // (alpha, beta) per pair, double-buffered
constexpr int kXchBytes = 2 * 2 * (kNW - 1) * 64 * 8;
constexpr int kLdsBytes = kGWords * 4 + kPrmBytes + kXchBytes;  // <= 80 KiB: two blocks per CU
constexpr int kGeneric = 2016 - 64;   // off-diagonal blocks not needed for the next round's rotations
constexpr int kGenLanes = kThreads - 64;  // waves 0..6 (wave 7 computes the next round's rotations)
constexpr int kPerLane = (kGeneric + kGenLanes - 1) / kGenLanes;
static_assert(kLdsBytes <= 80 * 1024, "two workgroups per CU");
static_assert(kPerLane == 5, "generic block slots per lane");

// G's cells below and on the diagonal are free and hold small tables:
//  * the two convergence flags (by sweep parity: a rotation above stop_tol
//    happened) at row 2, columns 0 and 1;
//  * the scales by matrix index, gathered at renormalisation, on the diagonal
//    (index 127's diagonal cell lies past the triangle: row 3, column 0);
//  * per pair and buffer, (new diagonal of the first and second index, their
//    new scales), as float4 at rows 64..79, columns < 35 (16-byte aligned).
constexpr int kFlagWord = 2 * kGP;
__device__ __forceinline__ int scale_word(int i) { return i < 127 ? i * (kGP + 1) : 3 * kGP; }
static_assert(126 * (kGP + 1) < kGWords, "diagonal cells of indices 0..126 lie inside G");
__device__ __forceinline__ int rec_word(int buf, int P) {
    const int e = buf * 64 + P, r = 64 + (e >> 3);
    return ((r * kGP + 3) & ~3) + 4 * (e & 7);
}
static_assert(((79 * kGP + 3) & ~3) + 4 * 7 + 3 < 79 * kGP + 64, "records stay below the diagonal");

// Block (P, Q) holds the next round's pair iff Q == P + 2, or it is (0, 1) or (62, 63).
constexpr bool next_pair_block(int P, int Q) {
    return Q == P + 2 || (P == 0 && Q == 1) || (P == 62 && Q == 63);
}

struct BlockTable {
    uint16_t pq[kGeneric];  // P | Q << 8, row-major over P < Q
};

constexpr BlockTable make_block_table() {
    BlockTable t{};
    int n = 0;
    for (int P = 0; P < 64; ++P)
        for (int Q = P + 1; Q < 64; ++Q)
            if (!next_pair_block(P, Q)) t.pq[n++] = static_cast<uint16_t>(P | (Q << 8));
    return t;
}

__constant__ BlockTable kBlocks = make_block_table();

// Matrix index at position `pos` in round k (0 <= k < 127).
__device__ __forceinline__ int index_at(int pos, int k) {
    if (pos == 0) return 0;
    const unsigned u = static_cast<unsigned>(pos - 1 + k);
    return static_cast<int>(min(u, u - 127u)) + 1;
}

__device__ __forceinline__ int gidx(int a, int b) {
    return static_cast<int>(__umul24(static_cast<unsigned>(min(a, b)), kGP)) + max(a, b);
}

// LDS byte offsets of G's elements for every generic block of every lane in
// every round of a sweep: [round][lane][kPerLane blocks x 4 elements, padded to
// 24].  The tournament's index arithmetic is the same for every matrix, so it is
// tabulated once (2.7 MB, L2-resident) and each lane loads its 48 bytes a round
// ahead.  Byte offsets of the upper triangle end below 64 KiB, so 16 bits hold them.
constexpr int kAddrPad = 24;
constexpr int kAddrVec = kAddrPad * 2 / 16;  // uint4 per lane and round
static_assert(kGWords * 4 <= 65536, "16-bit LDS offsets");
static_assert(4 * kPerLane <= kAddrPad, "table row");
__device__ __align__(16) uint16_t g_gen_addr[127 * kGenLanes * kAddrPad];

__global__ __launch_bounds__(256) void jacobi_table_kernel() {
    const int i = blockIdx.x * 256 + threadIdx.x;  // (round, lane, block slot)
    if (i >= 127 * kGenLanes * kPerLane) return;
    const int j = i % kPerLane, g = (i / kPerLane) % kGenLanes, k = i / (kPerLane * kGenLanes);
    uint16_t *out = g_gen_addr + (k * kGenLanes + g) * kAddrPad + 4 * j;
    const int bi = g + kGenLanes * j;
    if (bi >= kGeneric) {
        out[0] = out[1] = out[2] = out[3] = 0;
        return;
    }
    const int code = kBlocks.pq[bi];
    const int P = code & 0xff, Q = code >> 8;
    const int p1 = index_at(P, k), q1 = index_at(127 - P, k);
    const int p2 = index_at(Q, k), q2 = index_at(127 - Q, k);
    out[0] = static_cast<uint16_t>(4 * gidx(p1, p2));
    out[1] = static_cast<uint16_t>(4 * gidx(p1, q2));
    out[2] = static_cast<uint16_t>(4 * gidx(q1, p2));
    out[3] = static_cast<uint16_t>(4 * gidx(q1, q2));
}

__device__ __forceinline__ float &lds_at(float *base, unsigned byte_off) {
    return *reinterpret_cast<float *>(reinterpret_cast<char *>(base) + byte_off);
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

__global__ __launch_bounds__(kThreads, 4) void jacobi_kernel(const float *__restrict__ gpart, int splits,
                                                             float *__restrict__ vt_out,
                                                             int32_t *__restrict__ sweeps_out,
                                                             int max_sweeps, float tol, float stop_tol) {
    extern __shared__ __align__(16) float smem[];
    float *G = smem;
    int *flags = reinterpret_cast<int *>(smem + kFlagWord);                   // [2] by sweep parity
    float2 *prm = reinterpret_cast<float2 *>(smem + kGWords);                 // [2][64] (alpha, beta)
    float2 *xch = reinterpret_cast<float2 *>(smem + kGWords + kPrmBytes / 4);  // [2][2][7][64]

    const int blk = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const float *src = gpart + static_cast<int64_t>(blk) * splits * kD * kD;
    for (int e = tid; e < kD * kD; e += kThreads) {
        const int i = e >> 7, j = e & 127;
        if (i < j) {
            float s = 0.f;
            for (int p = 0; p < splits; ++p) s += src[static_cast<int64_t>(p) * kD * kD + e];
            G[i * kGP + j] = s;
        }
    }
    if (tid == 0) {
        flags[0] = 0;
        flags[1] = 0;
    }
    __syncthreads();

    // Round 0 of sweep 0: pair P = (P, 127 - P).
    if (wave == kNW - 1) {
        const int x = lane, y = 127 - lane;
        float a = 0.f, b = 0.f;
        for (int p = 0; p < splits; ++p) {
            a += src[static_cast<int64_t>(p) * kD * kD + x * kD + x];
            b += src[static_cast<int64_t>(p) * kD * kD + y * kD + y];
        }
        const float g = G[x * kGP + y];
        const Rot r = jacobi_rotation(a, b, g, tol);  // scales start at 1: alpha = beta = t
        prm[lane] = make_float2(r.t, r.t);
        *reinterpret_cast<float4 *>(G + rec_word(0, lane)) = make_float4(r.na, r.nb, r.c, r.c);
        if (r.rot) {
            G[x * kGP + y] = 0.f;
            if (g * g > stop_tol * stop_tol * fabsf(a * b)) flags[0] = 1;
        }
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
    // Generic blocks of this lane (waves 0..6): table entries tid, tid + 448, ...
    int bq[kPerLane];
#pragma unroll
    for (int j = 0; j < kPerLane; ++j) {
        const int i = tid + kGenLanes * j;
        bq[j] = (wave < kNW - 1 && i < kGeneric) ? kBlocks.pq[i] : -1;
    }
    // The next-pair block of this lane (wave 7 only): lane = next round's pair P'.
    const int Pn = lane;
    const int Pa = Pn == 0 ? 0 : (Pn == 63 ? 62 : Pn - 1);
    const int Pb = Pn == 0 ? 1 : (Pn == 63 ? 63 : Pn + 1);
    const int sel = Pn == 0 ? 0 : (Pn == 63 ? 3 : 2);  // element (p1 p2) / (q1 q2) / (q1 p2)
    // This lane's row of the offset table (wave 7 reads a valid row it never uses).
    const uint4 *arow = reinterpret_cast<const uint4 *>(g_gen_addr) + (tid < kGenLanes ? tid : tid - 64) * kAddrVec;
    uint4 ta[kAddrVec];
#pragma unroll
    for (int v = 0; v < kAddrVec; ++v) ta[v] = arow[v];
    __syncthreads();

    int used = -max_sweeps;
    int gk = 0;  // rounds done so far (parity selects the buffers)
    for (int sweep = 0; sweep < max_sweeps; ++sweep) {
        for (int kr = 0; kr < 127; ++kr, ++gk) {
            // Opaque copy of the round: recomputing the indices each round keeps
            // them out of per-index induction registers.
            int k = kr;
            asm volatile("" : "+s"(k));
            const int cb = gk & 1;
            const float2 *pc = prm + cb * 64;
            // rounds after which G and V^T are multiplied back by their scales
            const bool renorm = (k == 63) | (k == 126);

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

            // ---- next round's rotations (wave 7): rotate block (Pa, Pb), then the
            // pair of round k + 1 formed by one of its elements
            const bool last_round = (k == 126);
            if (wave == kNW - 1) {
                const float2 A = pc[Pa], B = pc[Pb];
                const float4 DA = *reinterpret_cast<const float4 *>(G + rec_word(cb, Pa));
                const float4 DB = *reinterpret_cast<const float4 *>(G + rec_word(cb, Pb));
                const int p1 = index_at(Pa, k), q1 = index_at(127 - Pa, k);
                const int p2 = index_at(Pb, k), q2 = index_at(127 - Pb, k);
                const int sa[4] = {gidx(p1, p2), gidx(p1, q2), gidx(q1, p2), gidx(q1, q2)};
                const int asel = sel == 0 ? sa[0] : (sel == 2 ? sa[2] : sa[3]);
                const bool sact = (A.x != 0.f) | (B.x != 0.f);
                float h[4];
                if (sact) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) h[e] = G[sa[e]];
                    const float r11 = fmaf(-A.x, h[2], h[0]), r12 = fmaf(-A.x, h[3], h[1]);
                    const float r21 = fmaf(A.y, h[0], h[2]), r22 = fmaf(A.y, h[1], h[3]);
                    h[0] = fmaf(-B.x, r12, r11);
                    h[1] = fmaf(B.y, r11, r12);
                    h[2] = fmaf(-B.x, r22, r21);
                    h[3] = fmaf(B.y, r21, r22);
                } else {
                    const float v = G[asel];
                    h[0] = h[2] = h[3] = v;
                    h[1] = 0.f;
                }
                const float gn = sel == 0 ? h[0] : (sel == 2 ? h[2] : h[3]);
                // new diagonal entries and scales of the pair's first and second index
                const float an = Pn == 0 ? DA.x : (Pn == 63 ? DB.y : DB.x);
                const float bn = Pn == 0 ? DB.x : DA.y;
                const float sfa = Pn == 0 ? DA.z : (Pn == 63 ? DB.w : DB.z);
                const float sfb = Pn == 0 ? DB.z : DA.w;
                const float gt = gn * sfa * sfb;
                Rot r = jacobi_rotation(an, bn, gt, tol);
                const int kn = last_round ? 0 : k + 1;
                float s1 = sfa, s2 = sfb;
                if (renorm) {  // uniform: the scales are gathered by index and restart at 1
                    G[scale_word(index_at(Pn, kn))] = sfa;
                    G[scale_word(index_at(127 - Pn, kn))] = sfb;
                    s1 = s2 = 1.f;
                }
                const float ratio = s2 * __builtin_amdgcn_rcpf(s1);
                float al = r.t * ratio, be = r.t * __builtin_amdgcn_rcpf(ratio);
                if ((al == 0.f) | (be == 0.f)) {  // negligible rotation: none
                    r = Rot{1.f, 0.f, an, bn, false};
                    al = be = 0.f;
                }
                prm[(cb ^ 1) * 64 + Pn] = make_float2(al, be);
                *reinterpret_cast<float4 *>(G + rec_word(cb ^ 1, Pn)) = make_float4(r.na, r.nb, s1 * r.c, s2 * r.c);
                const float gw = r.rot ? 0.f : gn;
                if (sel == 0) h[0] = gw;
                else if (sel == 2) h[2] = gw;
                else h[3] = gw;
                if (sact) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) G[sa[e]] = h[e];
                } else if (r.rot) {
                    G[asel] = 0.f;
                }
                if (r.rot && gt * gt > stop_tol * stop_tol * fabsf(an * bn))
                    flags[(sweep + (last_round ? 1 : 0)) & 1] = 1;
            }


            // ---- generic off-diagonal blocks (waves 0..6), two at a time: loads first, then stores
            {
                // next round's offsets (round 0 after the sweep's last): each uint4
                // of the table row is reloaded once its two blocks are done
                const int kn = k == 126 ? 0 : k + 1;
                const uint4 *anext = arow + kn * kGenLanes * kAddrVec;
#pragma unroll
                for (int j0 = 0; j0 < kPerLane; j0 += 2) {
                    if (wave == kNW - 1) break;  // uniform
                    const uint4 tv = ta[j0 / 2];
                    const unsigned aw[4] = {tv.x, tv.y, tv.z, tv.w};
                    unsigned ad[2][4];
                    float gv[2][4];
                    float2 c1[2], c2[2];
                    bool act[2];
#pragma unroll
                    for (int i = 0; i < 2; ++i) {
                        const int code = j0 + i < kPerLane ? bq[j0 + i] : -1;
                        act[i] = code >= 0;
                        const int P = act[i] ? (code & 0xff) : 0, Q = act[i] ? (code >> 8) : 1;
                        c1[i] = pc[P];
                        c2[i] = pc[Q];
                        act[i] = act[i] & ((c1[i].x != 0.f) | (c2[i].x != 0.f));
                        ad[i][0] = aw[2 * i] & 0xffffu;
                        ad[i][1] = aw[2 * i] >> 16;
                        ad[i][2] = aw[2 * i + 1] & 0xffffu;
                        ad[i][3] = aw[2 * i + 1] >> 16;
                    }
#pragma unroll
                    for (int i = 0; i < 2; ++i)
                        if (act[i]) {
#pragma unroll
                            for (int e = 0; e < 4; ++e) gv[i][e] = lds_at(G, ad[i][e]);
                        }
#pragma unroll
                    for (int i = 0; i < 2; ++i)
                        if (act[i]) {
                            // rows of pair P, then columns of pair Q
                            const float a1 = c1[i].x, b1 = c1[i].y, a2 = c2[i].x, b2 = c2[i].y;
                            const float h11 = fmaf(-a1, gv[i][2], gv[i][0]), h12 = fmaf(-a1, gv[i][3], gv[i][1]);
                            const float h21 = fmaf(b1, gv[i][0], gv[i][2]), h22 = fmaf(b1, gv[i][1], gv[i][3]);
                            lds_at(G, ad[i][0]) = fmaf(-a2, h12, h11);
                            lds_at(G, ad[i][1]) = fmaf(b2, h11, h12);
                            lds_at(G, ad[i][2]) = fmaf(-a2, h22, h21);
                            lds_at(G, ad[i][3]) = fmaf(b2, h21, h22);
                        }
                    ta[j0 / 2] = anext[j0 / 2];
                }
            }
            if (k == 1 && tid == 0) flags[(sweep + 1) & 1] = 0;
            __syncthreads();

            // ---- receive the rows that crossed a wave boundary
            const float2 *xi = xch + cb * 2 * (kNW - 1) * 64;
            if (wave < kNW - 1) F[7] = xi[wave * 64 + lane];
            if (wave > 0) S[0] = xi[((kNW - 1) + wave - 1) * 64 + lane];

            // ---- multiply G and V^T back by the scales (gathered by index above)
            if (renorm) {
                const int kn = k == 126 ? 0 : k + 1;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const float sf = G[scale_word(index_at(8 * wave + j, kn))];
                    const float ss = G[scale_word(index_at(127 - 8 * wave - j, kn))];
                    F[j] = make_float2(F[j].x * sf, F[j].y * sf);
                    S[j] = make_float2(S[j].x * ss, S[j].y * ss);
                }
                const float sj = G[scale_word(tid & 127)];
                for (int e = tid; e < kD * kD; e += kThreads) {
                    const int i = e >> 7, j = e & 127;
                    if (i < j) G[i * kGP + j] *= G[scale_word(i)] * sj;
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
    float2 *dst = reinterpret_cast<float2 *>(vt_out + static_cast<int64_t>(blk) * kD * kD);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int P = 8 * wave + j;
        dst[P * 64 + lane] = F[j];
        dst[(127 - P) * 64 + lane] = S[j];
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
    // Refilled on the caller's stream before every solve, so the solve never
    // depends on another stream's work; concurrent fills write identical values.
    constexpr int kTabThreads = 127 * kGenLanes * kPerLane;
    hipLaunchKernelGGL(jacobi_table_kernel, dim3((kTabThreads + 255) / 256), dim3(256), 0, st);
    hipLaunchKernelGGL(jacobi_kernel, dim3(static_cast<unsigned>(n_blocks)), dim3(kThreads), kLdsBytes, st,
                       gpart, splits, vt, sweeps, max_sweeps, tol, stop_tol);
    return hipGetLastError();
}

}  // namespace milo
