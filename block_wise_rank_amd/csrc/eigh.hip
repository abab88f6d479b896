// Batched symmetric eigensolve of 128 x 128 Gram matrices: Householder
// tridiagonalisation, then implicit symmetric QR steps with Wilkinson shifts on
// the tridiagonal matrix, the rotations accumulated into the rows of Q (Golub &
// Van Loan, Matrix Computations, sec. 8.3: tridiagonalisation 8.3.1, the
// implicit shifted QR step 8.3.3-8.3.5).
//
// Two kernels, one workgroup of 128 threads (two waves) per matrix, thread r
// owning row r in registers:
//  * tridiag_kernel: G = Q T Q^T with Q = H_0 H_1 ... H_125,
//    H_k = I - beta_k v_k v_k^T, v_k zero in entries 0..k.  Step k forms v_k
//    from column k below the diagonal (held, by symmetry, as entry k of every
//    row), p = beta A v, w = p - (beta/2)(p^T v) v and A <- A - v w^T - w v^T:
//    two barriers per step, the vectors exchanged through small double-buffered
//    LDS arrays.  The reflectors go to the Gram's own workspace area (no longer
//    needed once summed), the diagonal and off-diagonal of T to the first two
//    rows of the eigenvector area.
//  * ql_kernel: thread r forms row r of Q (e_r^T H_0 H_1 ... H_125, reflector
//    entries read as wave-uniform scalar loads) and then applies every rotation
//    of the QR steps to it: V = Q Z, where Z holds the eigenvectors of T, so
//    row r of V is entry r of every eigenvector and the result leaves as rows of
//    V^T with coalesced stores.  The QR steps themselves (a short dependent
//    chain per rotation) are computed redundantly by every lane of each wave
//    from the wave's own copy of T in LDS, so the two waves never wait for each
//    other.  The chase over rows l .. m of the unreduced bottom block is
//    unrolled over the rotation index, with uniform branches skipping to l and
//    leaving at m, which keeps every row entry at a fixed register.
//
// Deflation: e_j is negligible when |e_j| <= u (|d_j| + |d_{j+1}|),
// u = 2^-23.  After every QR step the bottom block shrinks past negligible
// entries and its top is the entry above the lowest negligible one below it
// (flags for all j from one lane-parallel test and two ballots).  The Gram is
// scaled by a power of two (1 / its largest diagonal entry, rounded to a power
// of two) so that squares stay clear of the fp32 range limits; the scale does
// not change the eigenvectors, and the singular values are recomputed from X
// afterwards (the Rayleigh quotients ||X v||).
#include "common.hpp"
#include "kernels.hpp"

namespace milo {
namespace {

constexpr int kThreads = kD;     // one thread per row, two waves
constexpr int kRefl = kD - 2;    // reflectors H_0 .. H_125
constexpr int kBetaRow = kD - 2; // row of the reflector area holding beta_k
constexpr float kDeflTol = 1.1920929e-7f;  // 2^-23

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
    return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
    return v;
}

__global__ __launch_bounds__(kThreads) void tridiag_kernel(float *__restrict__ gpart, int splits,
                                                          float *__restrict__ vt) {
    const int blk = blockIdx.x, r = threadIdx.x, lane = r & 63, wave = r >> 6;
    float *src = gpart + static_cast<int64_t>(blk) * splits * kD * kD;
    float *tri = vt + static_cast<int64_t>(blk) * kD * kD;  // row 0: d, row 1: e
    __shared__ float4 xb[2][kD / 4], vb[2][kD / 4], pb[2][kD / 4];
    __shared__ float red[2][2][2];
    __shared__ float smax[2];

    float a[kD];
    {
        const float4 *row = reinterpret_cast<const float4 *>(src + r * kD);
#pragma unroll
        for (int j = 0; j < kD / 4; ++j) {
            float4 t = row[j];
            for (int p = 1; p < splits; ++p) {
                const float4 u = row[static_cast<int64_t>(p) * kD * kD / 4 + j];
                t.x += u.x; t.y += u.y; t.z += u.z; t.w += u.w;
            }
            a[4 * j] = t.x; a[4 * j + 1] = t.y; a[4 * j + 2] = t.z; a[4 * j + 3] = t.w;
        }
    }
    float dr = 0.f;
    for (int p = 0; p < splits; ++p) dr += src[static_cast<int64_t>(p) * kD * kD + r * kD + r];
    const float wm = wave_max(fabsf(dr));
    if (lane == 0) smax[wave] = wm;
    __syncthreads();  // also: every read of the Gram partials is done before reflectors overwrite them
    const float mx = fmaxf(smax[0], smax[1]);
    const float sc = mx > 0.f ? ldexpf(1.f, -ilogbf(mx)) : 1.f;
#pragma unroll
    for (int j = 0; j < kD; ++j) a[j] *= sc;

    float *hv = src;
    for (int k = 0; k < kRefl; ++k) {
        const int par = k & 1;
        float akk, ak1;  // entries k and k + 1 of row r (k is uniform: a branch, not an indexed read)
        switch (k) {
#define MILO_PICK(K)      \
    case K:               \
        akk = a[K];       \
        ak1 = a[(K) + 1]; \
        break;
#define MILO_PICK8(K0)                                                                              \
    MILO_PICK(K0) MILO_PICK(K0 + 1) MILO_PICK(K0 + 2) MILO_PICK(K0 + 3) MILO_PICK(K0 + 4) MILO_PICK(K0 + 5) \
    MILO_PICK(K0 + 6) MILO_PICK(K0 + 7)
            MILO_PICK8(0) MILO_PICK8(8) MILO_PICK8(16) MILO_PICK8(24) MILO_PICK8(32) MILO_PICK8(40)
            MILO_PICK8(48) MILO_PICK8(56) MILO_PICK8(64) MILO_PICK8(72) MILO_PICK8(80) MILO_PICK8(88)
            MILO_PICK8(96) MILO_PICK8(104) MILO_PICK8(112) MILO_PICK(120) MILO_PICK(121) MILO_PICK(122)
            MILO_PICK(123) MILO_PICK(124)
            default:
                akk = a[125];
                ak1 = a[126];
                break;
#undef MILO_PICK8
#undef MILO_PICK
        }
        const float xk = r > k ? akk : 0.f;
        reinterpret_cast<float *>(xb[par])[r] = xk;
        const float s2 = wave_sum(xk * xk);
        if (lane == 0) red[par][0][wave] = s2;
        if (r == k) tri[k] = akk;
        __syncthreads();
        const float nx2 = red[par][0][0] + red[par][0][1];
        const float x1 = reinterpret_cast<const float *>(xb[par])[k + 1];
        float alpha = 0.f, beta = 0.f;
        if (nx2 > 0.f) {
            const float nx = sqrtf(nx2);
            alpha = x1 >= 0.f ? -nx : nx;
            beta = 1.f / (nx2 + fabsf(x1) * nx);  // 2 / v^T v
        }
        const float vr = xk - (r == k + 1 ? alpha : 0.f);
        float dot = 0.f;
#pragma unroll
        for (int j = 0; j < kD / 4; ++j) {
            const float4 x = xb[par][j];
            dot = fmaf(a[4 * j], x.x, dot);
            dot = fmaf(a[4 * j + 1], x.y, dot);
            dot = fmaf(a[4 * j + 2], x.z, dot);
            dot = fmaf(a[4 * j + 3], x.w, dot);
        }
        dot = fmaf(-alpha, ak1, dot);
        const float pr = r > k ? beta * dot : 0.f;
        reinterpret_cast<float *>(vb[par])[r] = vr;
        reinterpret_cast<float *>(pb[par])[r] = pr;
        const float pv = wave_sum(pr * vr);
        if (lane == 0) red[par][1][wave] = pv;
        hv[k * kD + r] = vr;
        if (r == 0) {
            hv[kBetaRow * kD + k] = beta;
            tri[kD + k] = alpha;
        }
        __syncthreads();
        const float K = 0.5f * beta * (red[par][1][0] + red[par][1][1]);
        const float wr = fmaf(-K, vr, pr);
#pragma unroll
        for (int j = 0; j < kD / 4; ++j) {
            const float4 p = pb[par][j], v = vb[par][j];
            const float pj[4] = {p.x, p.y, p.z, p.w}, vj[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float wj = fmaf(-K, vj[i], pj[i]);
                a[4 * j + i] = fmaf(-vr, wj, fmaf(-wr, vj[i], a[4 * j + i]));
            }
        }
    }
    if (r == kD - 2) tri[kD - 2] = a[kD - 2];
    if (r == kD - 1) {
        tri[kD - 1] = a[kD - 1];
        tri[kD + kD - 2] = a[kD - 2];
    }
}

__global__ __launch_bounds__(kThreads) void ql_kernel(const float *__restrict__ gpart, int splits,
                                                     float *__restrict__ vt, int32_t *__restrict__ rot_out,
                                                     int max_steps) {
    const int blk = blockIdx.x, r = threadIdx.x, lane = r & 63, wave = r >> 6;
    const float *hv = gpart + static_cast<int64_t>(blk) * splits * kD * kD;
    float *out = vt + static_cast<int64_t>(blk) * kD * kD;
    // per wave: D[0..127] = diagonal, E[j + 1] = T[j][j+1] (E[0], E[128], E[129] pads)
    __shared__ float sd[2][kD + 4], se[2][kD + 4];
    float *D = sd[wave], *E = se[wave];
    D[lane] = out[lane];
    D[lane + 64] = out[lane + 64];
    E[lane + 1] = out[kD + lane];
    E[lane + 65] = lane + 64 < kD - 1 ? out[kD + lane + 64] : 0.f;
    if (lane == 0) {
        E[0] = 0.f;
        E[kD + 1] = 0.f;
    }
    __syncthreads();  // every read of T is done before the rows of V^T overwrite it

    // row r of Q = e_r^T H_0 H_1 ... H_125
    float y[kD];
#pragma unroll
    for (int j = 0; j < kD; ++j) y[j] = j == r ? 1.f : 0.f;
    for (int k = 0; k < kRefl; ++k) {
        const float *v = hv + k * kD;
        float t0 = 0.f, t1 = 0.f;
#pragma unroll
        for (int j = 0; j < kD; j += 2) {
            t0 = fmaf(y[j], v[j], t0);
            t1 = fmaf(y[j + 1], v[j + 1], t1);
        }
        const float t = (t0 + t1) * hv[kBetaRow * kD + k];
#pragma unroll
        for (int j = 0; j < kD; ++j) y[j] = fmaf(-t, v[j], y[j]);
    }

    int m = kD - 1, steps = 0, rotations = 0;
    bool capped = false;
    for (;;) {
        // negligible off-diagonal entries: bit j of (lo, hi) for e_j, j = lane, lane + 64
        const auto negl = [&](int j) {
            return fabsf(E[j + 1]) <= kDeflTol * (fabsf(D[j]) + fabsf(D[j + 1]));
        };
        const uint64_t lo = __ballot(negl(lane));
        const uint64_t hi = __ballot(lane + 64 >= kD - 1 || negl(lane + 64));
        // bottom of the unreduced block: the last non-negligible e_j with j < m
        int jb = -1;
        {
            const uint64_t hm = m > 64 ? (~hi & ((m - 64 >= 64) ? ~0ull : ((1ull << (m - 64)) - 1))) : 0ull;
            if (hm) {
                jb = 64 + 63 - __builtin_clzll(hm);
            } else {
                const uint64_t lm = ~lo & (m >= 64 ? ~0ull : ((1ull << m) - 1));
                if (lm) jb = 63 - __builtin_clzll(lm);
            }
        }
        if (jb < 0) break;
        m = jb + 1;
        // top: one past the last negligible e_j with j < m - 1
        int l = 0;
        {
            const int t = m - 1;
            const uint64_t hm = t > 64 ? (hi & ((1ull << (t - 64)) - 1)) : 0ull;
            if (hm) {
                l = 64 + 64 - __builtin_clzll(hm);
            } else {
                const uint64_t lm = lo & (t >= 64 ? ~0ull : ((1ull << t) - 1));
                if (lm) l = 64 - __builtin_clzll(lm);
            }
        }
        if (steps == max_steps) {
            capped = true;
            break;
        }
        ++steps;
        rotations += m - l;
        // Wilkinson shift: the eigenvalue of the trailing 2 x 2 nearer its last entry
        float mu;
        {
            const float p = D[m - 1], b = D[m], g = E[m];
            const float del = 0.5f * (p - b);
            const float h = sqrtf(fmaf(del, del, g * g));
            mu = b - g * g / (del + (del >= 0.f ? h : -h));
        }
        const float keep = E[l];  // T[l-1][l]: the first rotation writes this slot
        float a = D[l], f = E[l + 1], x = a - mu, z = f;
        // the chase over rows l .. m, one rotation per index K (rows/columns K, K + 1):
        // (c, s) zeroes the bulge z against x; a, f are the current T[K][K],
        // T[K][K+1], and b, en the untouched T[K+1][K+1], T[K+1][K+2]
#pragma unroll
        for (int K = 0; K < kD - 1; ++K) {
            if (K < l) continue;
            if (K >= m) break;
            const float b = D[K + 1], en = E[K + 2];
            const float q = fmaf(x, x, z * z);
            const float rs = q > 0.f ? __builtin_amdgcn_rsqf(q) : 0.f;
            const float c = q > 0.f ? x * rs : 1.f, s = z * rs;
            E[K] = q * rs;  // T[K-1][K] (at K = l this slot is restored below)
            const float cc = c * c, ss = s * s, cs = c * s;
            const float t2 = 2.f * cs * f;
            D[K] = fmaf(cc, a, fmaf(ss, b, t2));
            const float an = fmaf(ss, a, fmaf(cc, b, -t2));
            x = fmaf(cs, b - a, (cc - ss) * f);
            a = an;
            z = s * en;
            f = c * en;
            const float y0 = y[K], y1 = y[K + 1];
            y[K] = fmaf(c, y0, s * y1);
            y[K + 1] = fmaf(c, y1, -s * y0);
        }
        E[m] = x;
        D[m] = a;
        E[l] = keep;
    }
#pragma unroll
    for (int c = 0; c < kD; ++c) out[c * kD + r] = y[c];
    if (r == 0 && rot_out) rot_out[blk] = capped ? -rotations : rotations;
}

}  // namespace

hipError_t launch_tridiag(float *gpart, int splits, int n_blocks, float *vt, hipStream_t st) {
    if (n_blocks <= 0) return hipSuccess;
    hipLaunchKernelGGL(tridiag_kernel, dim3(static_cast<unsigned>(n_blocks)), dim3(kThreads), 0, st, gpart, splits,
                       vt);
    return hipGetLastError();
}

hipError_t launch_ql(const float *gpart, int splits, int n_blocks, float *vt, int32_t *rotations, int max_steps,
                     hipStream_t st) {
    if (n_blocks <= 0) return hipSuccess;
    hipLaunchKernelGGL(ql_kernel, dim3(static_cast<unsigned>(n_blocks)), dim3(kThreads), 0, st, gpart, splits, vt,
                       rotations, max_steps);
    return hipGetLastError();
}

}  // namespace milo
