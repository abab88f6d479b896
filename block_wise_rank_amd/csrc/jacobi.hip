// Batched symmetric eigensolve of 128 x 128 Gram matrices by cyclic two-sided
// Jacobi, held entirely in LDS (one workgroup of 8 waves per block).
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
//      while waves 1..7 apply the previous round's rotations to the
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

// Rotate eigenvector rows p, q for the pairs first, first + stride, ... of one round.
__device__ __forceinline__ void rotate_vectors(float *V, const float *rc, const float *rs,
                                               const int *rp, const int *rq, int first,
                                               int stride, int lane) {
    for (int P = first; P < 64; P += stride) {
        const float s = rs[P];
        if (s == 0.f) continue;  // uniform over the wave
        const float c = rc[P];
        float2 *vp = reinterpret_cast<float2 *>(V + rp[P] * kD) + lane;
        float2 *vq = reinterpret_cast<float2 *>(V + rq[P] * kD) + lane;
        const float2 a = *vp, b = *vq;
        *vp = make_float2(c * a.x - s * b.x, c * a.y - s * b.y);
        *vq = make_float2(s * a.x + c * b.x, s * a.y + c * b.y);
    }
}

__global__ __launch_bounds__(512) void jacobi_kernel(const float *__restrict__ gpart, int splits,
                                                     float *__restrict__ vt_out,
                                                     int32_t *__restrict__ sweeps_out,
                                                     int max_sweeps, float tol) {
    extern __shared__ float smem[];
    float *G = smem;            // 128 x 129
    float *V = smem + kD * kGP; // 128 x 128, row i = eigenvector i
    __shared__ float rc[2][64], rs[2][64];
    __shared__ int rp[2][64], rq[2][64];
    __shared__ int any_rot;

    const int blk = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const float *src = gpart + static_cast<int64_t>(blk) * splits * kD * kD;
    for (int e = tid; e < kD * kD; e += 512) {
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
                const int P = lane;
                const int p = tournament_player(P, k), q = tournament_player(127 - P, k);
                const int pq = gidx(p, q);
                const float a = G[p * kGP + p], b = G[q * kGP + q], g = G[pq];
                float c = 1.f, s = 0.f;
                if (fabsf(g) > tol * sqrtf(fabsf(a) * fabsf(b))) {
                    const float zeta = (b - a) / (2.f * g);
                    const float t = fabsf(zeta) > 1e18f
                                        ? 0.5f / zeta
                                        : copysignf(1.f, zeta) / (fabsf(zeta) + sqrtf(1.f + zeta * zeta));
                    c = 1.f / sqrtf(1.f + t * t);
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
                rotate_vectors(V, rc[buf ^ 1], rs[buf ^ 1], rp[buf ^ 1], rq[buf ^ 1], wave - 1, 7,
                               lane);
            }
            __syncthreads();

            // Off-diagonal 2 x 2 blocks (P < Q).  Wave-row wr pairs block-row wr
            // (63 - wr blocks) with block-row 62 - wr (wr + 1 blocks): 64 lanes.
            for (int wr = wave; wr < 32; wr += 8) {
                int P, Q;
                if (wr < 31) {
                    if (lane < 63 - wr) {
                        P = wr;
                        Q = wr + 1 + lane;
                    } else {
                        P = 62 - wr;
                        Q = lane;
                    }
                } else {
                    if (lane >= 32) continue;
                    P = 31;
                    Q = 32 + lane;
                }
                const float s1 = rs[buf][P], s2 = rs[buf][Q];
                if (s1 == 0.f && s2 == 0.f) continue;
                const float c1 = rc[buf][P], c2 = rc[buf][Q];
                const int p1 = rp[buf][P], q1 = rq[buf][P];
                const int p2 = rp[buf][Q], q2 = rq[buf][Q];
                const int i11 = gidx(p1, p2), i12 = gidx(p1, q2);
                const int i21 = gidx(q1, p2), i22 = gidx(q1, q2);
                const float g11 = G[i11], g12 = G[i12], g21 = G[i21], g22 = G[i22];
                // rows of pair P, then columns of pair Q
                const float h11 = c1 * g11 - s1 * g21, h12 = c1 * g12 - s1 * g22;
                const float h21 = s1 * g11 + c1 * g21, h22 = s1 * g12 + c1 * g22;
                G[i11] = c2 * h11 - s2 * h12;
                G[i12] = s2 * h11 + c2 * h12;
                G[i21] = c2 * h21 - s2 * h22;
                G[i22] = s2 * h21 + c2 * h22;
            }
            __syncthreads();
        }
        // The last round (126, buffer 0) still has to reach the eigenvectors.
        rotate_vectors(V, rc[0], rs[0], rp[0], rq[0], wave, 8, lane);
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
    for (int e = tid; e < kD * kD / 4; e += 512)
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
    hipLaunchKernelGGL(jacobi_kernel, dim3(static_cast<unsigned>(n_blocks)), dim3(512), lds, st,
                       gpart, splits, vt, sweeps, max_sweeps, tol);
    return hipGetLastError();
}

}  // namespace milo
