// Batched symmetric eigensolve of 128 x 128 Gram matrices by cyclic two-sided
// Jacobi, held entirely in LDS (one workgroup of 16 waves per block).
//
// A Jacobi rotation of the pair (p, q) of G = X^T X is the same rotation a
// one-sided (Hestenes) Jacobi step applies to columns p, q of X, computed from
// alpha = G_pp, beta = G_qq, gamma = G_pq (Golub & Van Loan, Matrix
// Computations, sec. 8.5 and 8.6): zeta = (beta - alpha) / (2 gamma),
// t = sign(zeta) / (|zeta| + sqrt(1 + zeta^2)), c = 1/sqrt(1 + t^2), s = c t.
//
// Ordering: the round-robin ("circle") tournament on 128 indices gives 127
// rounds of 64 disjoint pairs per sweep, so one round's rotations commute and
// are applied together.  Per round:
//   A  wave 0 computes the 64 rotations and updates the 2 x 2 diagonal blocks,
//      while waves 1..15 apply the previous round's rotations to the
//      eigenvector rows;
//   B  all waves update the 2016 off-diagonal 2 x 2 blocks of the upper
//      triangle (G_PQ <- J_P^T G_PQ J_Q).
// G is kept as its upper triangle inside a 128 x 129 array (pitch 129 puts
// G[a][b] on bank (a + b) mod 32 whichever triangle is addressed); the
// eigenvectors are rows of a 128 x 128 array.  Pairs whose rotation is the
// identity (already orthogonal to tolerance) skip their LDS traffic, so late
// sweeps cost little.  A sweep without any rotation ends the solve.
#include "common.hpp"
#include "kernels.hpp"

namespace milo {
namespace {

constexpr int kGP = 129;  // LDS pitch of G (floats)

__device__ __forceinline__ int tournament_player(int pos, int round) {
    return pos == 0 ? 0 : 1 + (pos - 1 + round) % 127;
}

__device__ __forceinline__ int gidx(int a, int b) {
    return a < b ? a * kGP + b : b * kGP + a;
}

constexpr int kThreads = 1024;  // 16 waves
constexpr int kNW = kThreads / 64;

// Rotate eigenvector rows p, q for the pairs first, first + stride, ... (< 64) of
// one round.  All loads of the batch are issued before any store, so the wave
// keeps up to 2 * NP LDS requests in flight instead of one dependent chain.
template <int NP>
__device__ __forceinline__ void rotate_vectors(float *V, const float *rc, const float *rs,
                                               const int *rp, const int *rq, int first,
                                               int stride, int lane) {
    float c[NP], sn[NP];
    int p[NP], q[NP];
    bool act[NP];
#pragma unroll
    for (int i = 0; i < NP; ++i) {
        const int P = first + i * stride;
        act[i] = P < 64;
        const int Pc = act[i] ? P : 0;
        c[i] = rc[Pc];
        sn[i] = rs[Pc];
        p[i] = rp[Pc];
        q[i] = rq[Pc];
        act[i] = act[i] && sn[i] != 0.f;  // uniform over the wave
    }
    float2 a[NP], b[NP];
    float2 *V2 = reinterpret_cast<float2 *>(V);
#pragma unroll
    for (int i = 0; i < NP; ++i)
        if (act[i]) {
            a[i] = V2[p[i] * (kD / 2) + lane];
            b[i] = V2[q[i] * (kD / 2) + lane];
        }
#pragma unroll
    for (int i = 0; i < NP; ++i)
        if (act[i]) {
            V2[p[i] * (kD / 2) + lane] = make_float2(c[i] * a[i].x - sn[i] * b[i].x, c[i] * a[i].y - sn[i] * b[i].y);
            V2[q[i] * (kD / 2) + lane] = make_float2(sn[i] * a[i].x + c[i] * b[i].x, sn[i] * a[i].y + c[i] * b[i].y);
        }
}

__global__ __launch_bounds__(kThreads) void jacobi_kernel(const float *__restrict__ gpart, int splits,
                                                          float *__restrict__ vt_out,
                                                          int32_t *__restrict__ sweeps_out,
                                                          int max_sweeps, float tol) {
    extern __shared__ __align__(16) float smem[];
    float *G = smem;            // 128 x 129
    float *V = smem + kD * kGP; // 128 x 128, row i = eigenvector i
    __shared__ float rc[2][64], rs[2][64];
    __shared__ int rp[2][64], rq[2][64];
    __shared__ int any_rot;

    const int blk = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const float *src = gpart + static_cast<int64_t>(blk) * splits * kD * kD;
    for (int e = tid; e < kD * kD; e += kThreads) {
        float s = 0.f;
        for (int p = 0; p < splits; ++p) s += src[static_cast<int64_t>(p) * kD * kD + e];
        const int i = e >> 7, j = e & 127;
        G[i * kGP + j] = s;
        V[e] = (i == j) ? 1.f : 0.f;
    }
    if (tid == 0) any_rot = 0;
    __syncthreads();

    int used = -max_sweeps;
    for (int sweep = 0; sweep < max_sweeps; ++sweep) {
        for (int k = 0; k < 127; ++k) {
            const int buf = k & 1;
            if (wave == 0) {
                // Phase A: the 64 rotations of this round (one pair per lane).
                const int P = lane;
                const int p = tournament_player(P, k), q = tournament_player(127 - P, k);
                const int pq = gidx(p, q);
                const float a = G[p * kGP + p], b = G[q * kGP + q], g = G[pq];
                float c = 1.f, s = 0.f;
                if (fabsf(g) > tol * sqrtf(fabsf(a) * fabsf(b))) {
                    // Any (c, s) with c^2 + s^2 = 1 to working precision keeps the
                    // transform orthogonal, so 1-ulp reciprocals are enough here.
                    const float zeta = 0.5f * (b - a) * __builtin_amdgcn_rcpf(g);
                    const float az = fabsf(zeta);
                    const float t = az > 1e18f ? 0.5f * __builtin_amdgcn_rcpf(zeta)
                                               : copysignf(__builtin_amdgcn_rcpf(az + sqrtf(1.f + zeta * zeta)), zeta);
                    c = __builtin_amdgcn_rsqf(1.f + t * t);
                    s = c * t;
                    G[p * kGP + p] = a - t * g;
                    G[q * kGP + q] = b + t * g;
                    G[pq] = 0.f;
                    any_rot = 1;
                }
                rc[buf][P] = c;
                rs[buf][P] = s;
                rp[buf][P] = p;
                rq[buf][P] = q;
            } else if (k > 0) {
                // Meanwhile waves 1..15 apply the previous round to the eigenvectors.
                rotate_vectors<5>(V, rc[buf ^ 1], rs[buf ^ 1], rp[buf ^ 1], rq[buf ^ 1], wave - 1,
                                  kNW - 1, lane);
            }
            __syncthreads();

            // Phase B: off-diagonal 2 x 2 blocks (P < Q).  Wave-row wr pairs block-row
            // wr (63 - wr blocks) with block-row 62 - wr (wr + 1 blocks): 64 lanes.
            // Each wave owns wave-rows wave and wave + 16, loaded as one batch.
            int P[2], Q[2];
            bool act[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int wr = wave + kNW * i;
                act[i] = true;
                if (wr < 31) {
                    if (lane < 63 - wr) {
                        P[i] = wr;
                        Q[i] = wr + 1 + lane;
                    } else {
                        P[i] = 62 - wr;
                        Q[i] = lane;
                    }
                } else {
                    act[i] = lane < 32;
                    P[i] = 31;
                    Q[i] = 32 + (lane & 31);
                }
            }
            float c1[2], s1[2], c2[2], s2[2];
            int i11[2], i12[2], i21[2], i22[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                c1[i] = rc[buf][P[i]];
                s1[i] = rs[buf][P[i]];
                c2[i] = rc[buf][Q[i]];
                s2[i] = rs[buf][Q[i]];
                const int p1 = rp[buf][P[i]], q1 = rq[buf][P[i]];
                const int p2 = rp[buf][Q[i]], q2 = rq[buf][Q[i]];
                i11[i] = gidx(p1, p2);
                i12[i] = gidx(p1, q2);
                i21[i] = gidx(q1, p2);
                i22[i] = gidx(q1, q2);
                act[i] = act[i] && !(s1[i] == 0.f && s2[i] == 0.f);
            }
            float g11[2], g12[2], g21[2], g22[2];
#pragma unroll
            for (int i = 0; i < 2; ++i)
                if (act[i]) {
                    g11[i] = G[i11[i]];
                    g12[i] = G[i12[i]];
                    g21[i] = G[i21[i]];
                    g22[i] = G[i22[i]];
                }
#pragma unroll
            for (int i = 0; i < 2; ++i)
                if (act[i]) {
                    // rows of pair P, then columns of pair Q
                    const float h11 = c1[i] * g11[i] - s1[i] * g21[i], h12 = c1[i] * g12[i] - s1[i] * g22[i];
                    const float h21 = s1[i] * g11[i] + c1[i] * g21[i], h22 = s1[i] * g12[i] + c1[i] * g22[i];
                    G[i11[i]] = c2[i] * h11 - s2[i] * h12;
                    G[i12[i]] = s2[i] * h11 + c2[i] * h12;
                    G[i21[i]] = c2[i] * h21 - s2[i] * h22;
                    G[i22[i]] = s2[i] * h21 + c2[i] * h22;
                }
            __syncthreads();
        }
        // The last round (126, buffer 0) still has to reach the eigenvectors.
        rotate_vectors<4>(V, rc[0], rs[0], rp[0], rq[0], wave, kNW, lane);
        __syncthreads();
        const int rot = any_rot;
        __syncthreads();
        if (tid == 0) any_rot = 0;
        if (!rot) {
            used = sweep + 1;
            break;
        }
    }

    float *dst = vt_out + static_cast<int64_t>(blk) * kD * kD;
    for (int e = tid; e < kD * kD / 4; e += kThreads)
        reinterpret_cast<float4 *>(dst)[e] = reinterpret_cast<const float4 *>(V)[e];
    if (tid == 0 && sweeps_out) sweeps_out[blk] = used;
}

}  // namespace

hipError_t launch_jacobi(const float *gpart, int splits, int n_blocks, float *vt, int32_t *sweeps,
                         int max_sweeps, float tol, hipStream_t st) {
    if (n_blocks <= 0) return hipSuccess;
    const size_t lds = sizeof(float) * (kD * kGP + kD * kD);
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(jacobi_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       static_cast<int>(lds));
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(jacobi_kernel, dim3(static_cast<unsigned>(n_blocks)), dim3(kThreads), lds, st,
                       gpart, splits, vt, sweeps, max_sweeps, tol);
    return hipGetLastError();
}

}  // namespace milo
