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
//    LDS arrays; rows and columns already reduced are skipped.  The reflectors go to the Gram's own workspace area (no longer
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
// Deflation: e_j is negligible when |e_j| <= u max(|d_j| + |d_{j+1}|, 1),
// u = 2^-23 (1: the scale of G's largest diagonal entry, below).  After every QR step the bottom block shrinks past negligible
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
constexpr int kRing = 12, kAhead = 10;      // rotation staging of the apply kernel (steps)
constexpr int kSetupEvery = 8;              // passes of the chain kernel between step starts
static_assert(kSetupEvery <= 32, "a lane's buffered flags fit one word");

// Sum over the wave by DPP (no LDS round trips): within each row of 16 lanes
// by quad permutes and row rotations, then across rows by the row broadcasts
// of lanes 15 and 31; the total ends in lane 63 and is returned to every lane.
template <int Ctrl, int RowMask>
__device__ __forceinline__ float dpp_add(float v) {
    const int o = __builtin_amdgcn_update_dpp(0, __float_as_int(v), Ctrl, RowMask, 0xf, false);
    return v + __int_as_float(o);
}

__device__ __forceinline__ float wave_sum(float v) {
    v = dpp_add<0xB1, 0xf>(v);   // quad_perm [1, 0, 3, 2]
    v = dpp_add<0x4E, 0xf>(v);   // quad_perm [2, 3, 0, 1]
    v = dpp_add<0x124, 0xf>(v);  // row_ror:4
    v = dpp_add<0x128, 0xf>(v);  // row_ror:8: every lane holds its row's sum
    v = dpp_add<0x142, 0xa>(v);  // row_bcast:15 into rows 1 and 3
    v = dpp_add<0x143, 0xc>(v);  // row_bcast:31 into rows 2 and 3
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
    return v;
}

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3))) void tridiag_kernel(float *__restrict__ gpart, int splits,
                                                          float *__restrict__ vt) {
    const int blk = blockIdx.x, r = threadIdx.x, lane = r & 63;
    const int wave = __builtin_amdgcn_readfirstlane(r >> 6);
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
        // Rows and columns 0..k are done: v and p vanish there, so a wave whose
        // rows are all <= k skips the products, and so does every group of
        // eight columns <= k (uniform branches).
        const bool live = 64 * wave + 63 > k;
        // The loops below run over segments of 16 columns, skipping those with
        // every column <= k; within a segment the LDS operands of each group of
        // columns are loaded one group ahead, so that only a segment's first
        // load waits (the columns <= k of a segment that is run add exact zeros:
        // x, v and p vanish there).  (Segments of 32 wasted more zero updates,
        // a branch per group exposed every load.)
        float dot = 0.f;
        if (live) {
#pragma unroll
            for (int sg = 0; sg < 8; ++sg) {
                if (16 * sg + 15 <= k) continue;
                float4 xn0 = xb[par][4 * sg], xn1 = xb[par][4 * sg + 1];
#pragma unroll
                for (int j = 4 * sg; j < 4 * sg + 4; j += 2) {  // columns 4j .. 4j + 7
                    const float4 x = xn0, x2 = xn1;
                    if (j + 2 < 4 * sg + 4) {
                        xn0 = xb[par][j + 2];
                        xn1 = xb[par][j + 3];
                    }
                    dot = fmaf(a[4 * j], x.x, dot);
                    dot = fmaf(a[4 * j + 1], x.y, dot);
                    dot = fmaf(a[4 * j + 2], x.z, dot);
                    dot = fmaf(a[4 * j + 3], x.w, dot);
                    dot = fmaf(a[4 * j + 4], x2.x, dot);
                    dot = fmaf(a[4 * j + 5], x2.y, dot);
                    dot = fmaf(a[4 * j + 6], x2.z, dot);
                    dot = fmaf(a[4 * j + 7], x2.w, dot);
                }
            }
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
        // A - v w^T - w v^T with w = p - K v is A - v p^T - (p - 2 K v) v^T
        const float K = 0.5f * beta * (red[par][1][0] + red[par][1][1]);
        const float ur = fmaf(-2.f * K, vr, pr);
        if (live) {
#pragma unroll
            for (int sg = 0; sg < 8; ++sg) {
                if (16 * sg + 15 <= k) continue;
                float4 pn = pb[par][4 * sg], vn = vb[par][4 * sg];
#pragma unroll
                for (int j = 4 * sg; j < 4 * sg + 4; ++j) {  // columns 4j .. 4j + 3
                    const float4 p = pn, v = vn;
                    if (j + 1 < 4 * sg + 4) {
                        pn = pb[par][j + 1];
                        vn = vb[par][j + 1];
                    }
                    a[4 * j] = fmaf(-vr, p.x, fmaf(-ur, v.x, a[4 * j]));
                    a[4 * j + 1] = fmaf(-vr, p.y, fmaf(-ur, v.y, a[4 * j + 1]));
                    a[4 * j + 2] = fmaf(-vr, p.z, fmaf(-ur, v.z, a[4 * j + 2]));
                    a[4 * j + 3] = fmaf(-vr, p.w, fmaf(-ur, v.w, a[4 * j + 3]));
                }
            }
        }
    }
    if (r == kD - 2) tri[kD - 2] = a[kD - 2];
    if (r == kD - 1) {
        tri[kD - 1] = a[kD - 1];
        tri[kD + kD - 2] = a[kD - 2];
    }
}

// T is scaled so that G's largest diagonal entry lies in [1, 2): the floor of 1
// keeps entries far below that scale from being resolved to full relative
// accuracy (the fp32 Gram carries errors of that order anyway, and the singular
// values are recomputed from X).
__device__ __forceinline__ bool negligible(float e, float d0, float d1) {
    return fabsf(e) <= kDeflTol * fmaxf(fabsf(d0) + fabsf(d1), 1.f);
}

// Highest bit j < lim of a 128-bit mask (four words) that is set, or -1.
__device__ __forceinline__ int highest_below(const uint32_t (&w)[4], int lim) {
    int j = -1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int n = lim - 32 * i;  // bits of word i below lim
        const uint32_t keep = n >= 32 ? ~0u : (n > 0 ? (1u << n) - 1u : 0u);
        const uint32_t x = w[i] & keep;
        j = x ? 32 * i + 31 - __builtin_clz(x) : j;
    }
    return j;
}

// Bits j0 .. j0 + n - 1 (n <= 32, within the 128) of the mask set from the low
// n bits of v.
__device__ __forceinline__ void set_bits(uint32_t (&w)[4], int j0, int n, uint32_t v) {
    const int w0 = j0 >> 5, sh = j0 & 31;
    uint32_t lo = 0u, hi = 0u;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        lo = i == w0 ? w[i] : lo;
        hi = i == w0 + 1 ? w[i] : hi;
    }
    uint64_t both = static_cast<uint64_t>(hi) << 32 | lo;
    const uint64_t keep = (n >= 32 ? 0xffffffffull : ((1ull << n) - 1)) << sh;
    both = (both & ~keep) | ((static_cast<uint64_t>(v) << sh) & keep);
    lo = static_cast<uint32_t>(both);
    hi = static_cast<uint32_t>(both >> 32);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        w[i] = i == w0 ? lo : w[i];
        w[i] = i == w0 + 1 ? hi : w[i];
    }
}

__device__ __forceinline__ void set_bit(uint32_t (&w)[4], int j, bool on) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t bit = (j >> 5) == i ? 1u << (j & 31) : 0u;
        w[i] = on ? (w[i] | bit) : (w[i] & ~bit);
    }
}

// The QR iteration of 64 tridiagonal matrices per wave, one per lane: every
// pass of the loop takes one rotation of each lane's current step, or starts
// its next step.  T lives in LDS as [row][lane] (each lane its own column, so
// no bank conflicts whatever row each lane is at); the negligible off-diagonal
// entries are kept as a per-lane 128-bit mask, updated as the chase writes
// them, from which each step's block [l, m] follows: m - 1 is the last entry
// above the converged bottom that is not negligible, l is one past the last
// negligible entry above it.  Each step's rotations (c, s) and its header go to
// the block's stream area in order.
// L matrices per wave (lanes L .. 63 idle): the LDS copy of T takes
// (kD + 2) * 8 bytes per matrix, so L sets how many waves a CU holds (64: two,
// 48: three, 36: four), and the launcher picks L so that a call's waves fill
// the CUs in as few rounds as possible.
template <int L>
__global__ __launch_bounds__(64) void qr_chain_kernel(const float *__restrict__ vt, int n_blocks,
                                                      uint8_t *__restrict__ stream, int32_t *__restrict__ counts,
                                                      int32_t *__restrict__ rot_out) {
    static_assert(L >= 1 && L <= 64, "one lane per matrix");
    const int lane = threadIdx.x, b = blockIdx.x * L + lane;
    const bool own = lane < L;  // only these lanes touch the LDS copy
    const bool act = own && b < n_blocks;
    __shared__ float Ds[kD + 2][L], Es[kD + 2][L];  // d_j, e_j = T[j][j+1] (rows 127.. pads)
    if (own) {
        const float4 *tri = reinterpret_cast<const float4 *>(vt + static_cast<int64_t>(act ? b : 0) * kD * kD);
#pragma unroll 4
        for (int q = 0; q < kD / 4; ++q) {
            const float4 dv = act ? tri[q] : make_float4(0.f, 0.f, 0.f, 0.f);
            const float4 ev = act ? tri[kD / 4 + q] : make_float4(0.f, 0.f, 0.f, 0.f);
            Ds[4 * q][lane] = dv.x; Ds[4 * q + 1][lane] = dv.y; Ds[4 * q + 2][lane] = dv.z; Ds[4 * q + 3][lane] = dv.w;
            Es[4 * q][lane] = ev.x; Es[4 * q + 1][lane] = ev.y; Es[4 * q + 2][lane] = ev.z;
            Es[4 * q + 3][lane] = 4 * q + 3 < kD - 1 ? ev.w : 0.f;
        }
        Ds[kD][lane] = Ds[kD + 1][lane] = 0.f;
        Es[kD][lane] = Es[kD + 1][lane] = 0.f;
    }
    uint32_t nm[4] = {0u, 0u, 0u, 0u};
    if (own) {
#pragma unroll
        for (int j = 0; j < kD - 1; ++j)
            if (negligible(Es[j][lane], Ds[j][lane], Ds[j + 1][lane])) nm[j >> 5] |= 1u << (j & 31);
    }

    uint8_t *mine = stream + static_cast<int64_t>(act ? b : 0) * kStreamBytes;
    float2 *rot = reinterpret_cast<float2 *>(mine) + kRotPad;
    uint32_t *hdr = reinterpret_cast<uint32_t *>(mine + sizeof(float) * 2 * (kRotCap + 2 * kRotPad));
    // st: 0 ready for its next step, 1 in a chase, 2 done, 3 chase ended (its
    // closing writes pending).  Steps end and start only in every kSetupEvery-th
    // pass, so that their code (far longer than a rotation's) runs in few
    // passes; a lane whose chase has ended waits for that pass.
    int m = kD - 1, l = 0, K = 0, steps = 0, rots = 0, st = act ? 0 : 2;
    bool capped = false;
    float g = 0.f, p = 0.f, sn = 1.f, cn = 1.f, dk = 0.f, dk1 = 0.f, ek = 0.f, dprev = 0.f;
    // A rotation's LDS writes are issued at the start of the next pass (before
    // that pass's reads), so that waiting for those reads never waits for them.
    int wk = -1;      // d_wk (and e_{wk-1} when we_on) still to be written
    bool we_on = false;
    float wd = 0.f, we = 0.f;
    // Negligibility of the e_j a chase writes, j = fj .. fj + fn - 1, kept as the
    // bits of fv until the next step-start pass merges them into the mask (only
    // step starts read it; at most kSetupEvery rotations come between).
    int fj = 0, fn = 0;
    uint32_t fv = 0u;
    for (int pass = 0; __any(st != 2); ++pass) {
        if (wk >= 0) {
            if (we_on) Es[wk - 1][lane] = we;
            Ds[wk][lane] = wd;
            wk = -1;
        }
        if (pass % kSetupEvery == 0) {
            if (fn > 0) {
                set_bits(nm, fj, fn, fv);
                fn = 0;
                fv = 0u;
            }
            if (st == 3) {
                const float dm = dk - p;  // d_m
                Ds[m][lane] = dm;
                Es[m - 1][lane] = g;
                set_bit(nm, m - 1, negligible(g, dprev, dm));
                if (l > 0) set_bit(nm, l - 1, negligible(Es[l - 1][lane], Ds[l - 1][lane], Ds[l][lane]));
                if (m < kD - 1) set_bit(nm, m, negligible(Es[m][lane], dm, Ds[m + 1][lane]));
                st = 0;
            }
            if (st == 0) {
                uint32_t nc[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) nc[i] = ~nm[i];
                const int jb = highest_below(nc, m);  // last non-negligible e_j, j < m
                if (jb < 0) {
                    st = 2;
                } else {
                    const int mm = jb + 1, ll = highest_below(nm, mm - 1) + 1;
                    if (steps == kStepCap || rots + (mm - ll) > kRotCap) {
                        capped = true;
                        st = 2;
                    } else {
                        m = mm;
                        l = ll;
                        hdr[steps] = static_cast<uint32_t>(l) | static_cast<uint32_t>(m) << 16;
                        ++steps;
                        // Wilkinson shift from the trailing 2 x 2, carried as g = d_l - mu
                        // (the shift only steers convergence: rcp and sqrt at their
                        // hardware accuracy)
                        const float em = Es[m - 1][lane], dm = Ds[m][lane];
                        const float g0 = (Ds[m - 1][lane] - dm) * __builtin_amdgcn_rcpf(2.f * em);
                        const float h = __builtin_amdgcn_sqrtf(fmaf(g0, g0, 1.f));
                        dk = Ds[l][lane];
                        dk1 = Ds[l + 1][lane];
                        ek = Es[l][lane];
                        g = dk - dm + em * __builtin_amdgcn_rcpf(g0 + (g0 >= 0.f ? h : -h));
                        p = 0.f;
                        sn = cn = 1.f;
                        K = l;
                        st = 1;
                    }
                }
            }
        }
        if (st == 1) {
            // rotation K (rows/columns K, K + 1) zeroes the bulge f = s e_K against
            // g; p carries the change of the diagonal entry the next one starts
            // from.  With q = f^2 + g^2, c = g / sqrt q, s = f / sqrt q and
            // w = (d_{K+1} - d_K + p) f + 2 g b (b = c_prev e_K):
            // p' = f w / q, g' = g w / q - b.
            const float dn = Ds[K + 2][lane], en = Es[K + 1][lane];
            const float f = sn * ek, bb = cn * ek;
            const float q = fmaf(f, f, g * g);
            const bool ok = q > 0.f;  // f = g = 0: the identity (c = 1, s = 0)
            const float g2 = dk - p;
            const float w = fmaf(dk1 - g2, f, 2.f * (g * bb));
            const float rs = __builtin_amdgcn_rsqf(ok ? q : 1.f);
            const float rs2 = rs * rs;
            p = (f * w) * rs2;
            const float dK = g2 + p;
            const float gn = fmaf(g * w, rs2, -bb);
            sn = f * rs;
            cn = ok ? g * rs : 1.f;
            g = ok ? gn : bb;
            we_on = K > l;
            if (we_on) {
                we = q * rs;  // e_{K-1}
                if (fn == 0) fj = K - 1;
                fv |= static_cast<uint32_t>(negligible(we, dprev, dK)) << fn;
                ++fn;
            }
            wk = K;
            wd = dK;
            dprev = dK;
            rot[rots] = make_float2(cn, sn);
            ++rots;
            dk = dk1;
            dk1 = dn;
            ek = en;
            ++K;
            if (K == m) st = 3;
        }
    }
    if (act) {
        counts[2 * b] = steps;
        counts[2 * b + 1] = rots;
        if (rot_out) rot_out[b] = capped ? -rots : rots;
    }
}

// Row r of Q = e_r^T H_0 H_1 ... H_125, the reflectors staged through LDS eight
// at a time (double-buffered, the next group's loads in flight during the
// current group) by threads tid < 128; v_k vanishes in entries 0..k, so each
// reflector skips the groups of eight entries it does not touch.  Every thread
// of the workgroup calls it (it holds barriers); a thread with r >= 128 holds
// no row and only stages.
__device__ __forceinline__ void form_q_row(float (&y)[kD], const float *__restrict__ hv, int r, int tid,
                                           float4 (*hb)[8][kD / 4], float *beta, float (*gp)[4]) {
#pragma unroll
    for (int j = 0; j < kD; ++j) y[j] = j == r ? 1.f : 0.f;
    if (tid < kRefl) beta[tid] = hv[kBetaRow * kD + tid];
    // thread tid stages entries 8 (tid & 15) .. + 7 of reflector 8 c + (tid >> 4)
    const bool stager = tid < kD;
    const int rr = (tid >> 4) & 7, cc = 2 * (tid & 15);
    const float4 *src = reinterpret_cast<const float4 *>(hv);
    float4 a0 = make_float4(0.f, 0.f, 0.f, 0.f), a1 = a0;
    if (stager) {
        a0 = src[rr * (kD / 4) + cc];
        a1 = src[rr * (kD / 4) + cc + 1];
    }
    for (int c = 0; c < kD / 8; ++c) {
        if (stager) {
            hb[c & 1][rr][cc] = a0;
            hb[c & 1][rr][cc + 1] = a1;
            // v_k . v_k+1 for the group's pairs (k = 8c + 2p): the stagers of
            // reflectors 2p and 2p + 1 hold the same entries 16 lanes apart;
            // products, then the sum over the 16 lanes of a row by DPP
            const float o[8] = {__shfl_xor(a0.x, 16), __shfl_xor(a0.y, 16), __shfl_xor(a0.z, 16),
                                __shfl_xor(a0.w, 16), __shfl_xor(a1.x, 16), __shfl_xor(a1.y, 16),
                                __shfl_xor(a1.z, 16), __shfl_xor(a1.w, 16)};
            float g = a0.x * o[0];
            g = fmaf(a0.y, o[1], g);
            g = fmaf(a0.z, o[2], g);
            g = fmaf(a0.w, o[3], g);
            g = fmaf(a1.x, o[4], g);
            g = fmaf(a1.y, o[5], g);
            g = fmaf(a1.z, o[6], g);
            g = fmaf(a1.w, o[7], g);
            g = dpp_add<0xB1, 0xf>(g);   // quad_perm [1, 0, 3, 2]
            g = dpp_add<0x4E, 0xf>(g);   // quad_perm [2, 3, 0, 1]
            g = dpp_add<0x124, 0xf>(g);  // row_ror:4
            g = dpp_add<0x128, 0xf>(g);  // row_ror:8: the row's sum in every lane
            if ((tid & 31) == 0) gp[c & 1][(tid >> 5) & 3] = g;
        }
        __syncthreads();
        if (stager && c + 1 < kD / 8) {
            const int k = 8 * (c + 1) + rr;
            const bool in = k < kRefl;
            a0 = in ? src[k * (kD / 4) + cc] : make_float4(0.f, 0.f, 0.f, 0.f);
            a1 = in ? src[k * (kD / 4) + cc + 1] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
        if (r >= kD) continue;  // uniform: a wave without rows
        // two reflectors at a time: with t = y.v_k and t' = y.v_k+1,
        // y H_k H_k+1 = y - s v_k - s' v_k+1, s = beta_k t,
        // s' = beta_k+1 (t' - s v_k.v_k+1): one pass of dots and one of
        // updates for the pair (v_k+1 vanishes where v_k does)
#pragma unroll 1
        for (int i = 0; i < 8; i += 2) {
            const int k = 8 * c + i;
            if (k >= kRefl) break;
            const float4 *v = hb[c & 1][i], *w = hb[c & 1][i + 1];
            float t0 = 0.f, t1 = 0.f, q0 = 0.f, q1 = 0.f;
#pragma unroll
            for (int j = 0; j < kD; j += 8) {
                if (j + 7 <= k) continue;
                const float4 u0 = v[j / 4], u1 = v[j / 4 + 1], w0 = w[j / 4], w1 = w[j / 4 + 1];
                t0 = fmaf(y[j], u0.x, t0);
                t1 = fmaf(y[j + 1], u0.y, t1);
                t0 = fmaf(y[j + 2], u0.z, t0);
                t1 = fmaf(y[j + 3], u0.w, t1);
                t0 = fmaf(y[j + 4], u1.x, t0);
                t1 = fmaf(y[j + 5], u1.y, t1);
                t0 = fmaf(y[j + 6], u1.z, t0);
                t1 = fmaf(y[j + 7], u1.w, t1);
                q0 = fmaf(y[j], w0.x, q0);
                q1 = fmaf(y[j + 1], w0.y, q1);
                q0 = fmaf(y[j + 2], w0.z, q0);
                q1 = fmaf(y[j + 3], w0.w, q1);
                q0 = fmaf(y[j + 4], w1.x, q0);
                q1 = fmaf(y[j + 5], w1.y, q1);
                q0 = fmaf(y[j + 6], w1.z, q0);
                q1 = fmaf(y[j + 7], w1.w, q1);
            }
            const float t = (t0 + t1) * beta[k];
            const float tn = fmaf(-t, gp[c & 1][i >> 1], q0 + q1) * beta[k + 1];
#pragma unroll
            for (int j = 0; j < kD; j += 8) {
                if (j + 7 <= k) continue;
                const float4 u0 = v[j / 4], u1 = v[j / 4 + 1], w0 = w[j / 4], w1 = w[j / 4 + 1];
                y[j] = fmaf(-t, u0.x, fmaf(-tn, w0.x, y[j]));
                y[j + 1] = fmaf(-t, u0.y, fmaf(-tn, w0.y, y[j + 1]));
                y[j + 2] = fmaf(-t, u0.z, fmaf(-tn, w0.z, y[j + 2]));
                y[j + 3] = fmaf(-t, u0.w, fmaf(-tn, w0.w, y[j + 3]));
                y[j + 4] = fmaf(-t, u1.x, fmaf(-tn, w1.x, y[j + 4]));
                y[j + 5] = fmaf(-t, u1.y, fmaf(-tn, w1.y, y[j + 5]));
                y[j + 6] = fmaf(-t, u1.z, fmaf(-tn, w1.z, y[j + 6]));
                y[j + 7] = fmaf(-t, u1.w, fmaf(-tn, w1.w, y[j + 7]));
            }
        }
    }
}

// The rotation of rows/columns K, K + 1 applied to a row of V (columns of V
// are eigenvectors; the rotation mixes two of them).
__device__ __forceinline__ void rotate_pair(float &y0, float &y1, float c, float s) {
    const float a = y0, b = y1;
    y0 = fmaf(s, b, c * a);
    y1 = fmaf(c, b, -s * a);
}

// Thread r forms row r of Q and applies every recorded rotation to it (V = Q Z,
// Z the eigenvectors of T), then writes entry r of every eigenvector: the rows
// of V^T, coalesced.  Each step's rotations are staged into LDS by the
// workgroup's first wave (LDS DMA, kAhead steps ahead of their use), then
// applied by every thread to its row with the rotation index unrolled, so that
// each row entry stays at a fixed register.
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3))) void qr_apply_kernel(const float *__restrict__ gpart, int splits,
                                                           const uint8_t *__restrict__ stream,
                                                           const int32_t *__restrict__ counts,
                                                           float *__restrict__ vt) {
    const int blk = blockIdx.x, r = threadIdx.x, lane = r & 63;
    const int wave = __builtin_amdgcn_readfirstlane(r >> 6);
    const float *hv = gpart + static_cast<int64_t>(blk) * splits * kD * kD;
    const uint8_t *mine = stream + static_cast<int64_t>(blk) * kStreamBytes;
    const float2 *rot = reinterpret_cast<const float2 *>(mine) + kRotPad;
    const uint32_t *hdr = reinterpret_cast<const uint32_t *>(mine + sizeof(float) * 2 * (kRotCap + 2 * kRotPad));
    __shared__ float4 hb[2][8][kD / 4];
    __shared__ float beta[kD];
    __shared__ float4 cs[kRing][kD / 2];  // ring of steps: rotation K of a step at (c, s) pair K
    __shared__ uint32_t hs[kStepCap];
    const int S = __builtin_amdgcn_readfirstlane(counts[2 * blk]);
    for (int t = r; t < S; t += kThreads) hs[t] = hdr[t];

    float y[kD];
    __shared__ float gpair[2][4];
    form_q_row(y, hv, r, r, hb, beta, gpair);  // its barriers make hs visible

    // Step t's rotations sit at rot[pos_t ..] and its rows in hs[t].  Wave 0
    // copies each step into ring slot t % kRing by LDS DMA kAhead steps ahead of
    // its use (the stream comes from HBM): the 128 rotation slots from pos_t - l_t on, so that rotation K lands
    // at pair K (the slots outside [l, m) belong to neighbouring steps or the
    // padding and are applied as the identity).
    int pos = 0, tf = 0;
    const auto fetch = [&]() {
        if (tf < S) {
            const uint32_t h = __builtin_amdgcn_readfirstlane(hs[tf]);  // uniform: scalar branches below
            const int l = static_cast<int>(h & 0xffffu), n = static_cast<int>(h >> 16) - l;
            if (wave == 0)
                __builtin_amdgcn_global_load_lds(
                    (const __attribute__((address_space(1))) void *)(rot + pos - l + 2 * lane),
                    (__attribute__((address_space(3))) void *)(cs[tf % kRing]), 16, 0, 0);
            pos += n;
            ++tf;
        }
    };
    // at most n DMAs outstanding (n < kAhead)
    const auto wait_dma = [](int n) {
        switch (n < 0 ? 0 : n) {
#define MILO_WAIT(N) \
    case N:          \
        __builtin_amdgcn_s_waitcnt(0x0F70 | (N)); \
        break;
            MILO_WAIT(0) MILO_WAIT(1) MILO_WAIT(2) MILO_WAIT(3) MILO_WAIT(4) MILO_WAIT(5) MILO_WAIT(6)
            MILO_WAIT(7) MILO_WAIT(8)
#undef MILO_WAIT
            default:
                __builtin_amdgcn_s_waitcnt(0x0F70 | (kAhead - 1));
        }
    };
    // After step t's DMA has landed: the identity into the slots of its first and
    // last groups of eight that lie outside [l, m) (they hold neighbouring
    // steps' rotations or padding).
    const auto identity_edges = [&](int t) {
        if (t < S && wave == 0) {
            const uint32_t h = __builtin_amdgcn_readfirstlane(hs[t]);
            const int l = static_cast<int>(h & 0xffffu), m = static_cast<int>(h >> 16);
            const int lo = l & ~7, hi = (m + 7) & ~7;
            const int K = lane < 8 ? lo + lane : m + (lane - 8);  // 8 slots below l, up to 8 from m
            if ((lane < 8 && K < l) || (lane >= 8 && lane < 16 && K < hi && K < kD))
                reinterpret_cast<float2 *>(cs[t % kRing])[K] = make_float2(1.f, 0.f);
        }
    };
    static_assert(kAhead - 1 <= 15 && kAhead < kRing, "DMA ring");
    for (int i = 0; i < kAhead; ++i) fetch();
    wait_dma(tf - 1);
    identity_edges(0);
    __syncthreads();
    for (int t = 0; t < S; ++t) {
        fetch();  // step t + kAhead
        const uint32_t h = __builtin_amdgcn_readfirstlane(hs[t]);
        const int l = static_cast<int>(h & 0xffffu), m = static_cast<int>(h >> 16);
        const float4 *cst = cs[t % kRing];
        // whole groups of eight rotations (the slots of a group outside [l, m)
        // hold the identity)
#pragma unroll
        for (int K0 = 0; K0 < kD - 1; K0 += 8) {
            if (K0 + 8 <= l) continue;
            if (K0 >= m) break;
            float c8[8], s8[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float4 v = cst[K0 / 2 + i];
                c8[2 * i] = v.x;
                s8[2 * i] = v.y;
                c8[2 * i + 1] = v.z;
                s8[2 * i + 1] = v.w;
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int K = K0 + i;
                if (K >= kD - 1) break;
                rotate_pair(y[K], y[K + 1], c8[i], s8[i]);
            }
        }
        wait_dma(tf - (t + 2));  // step t + 1 has landed; the later steps may be in flight
        identity_edges(t + 1);
        __syncthreads();
    }
#pragma unroll
    for (int c = 0; c < kD; ++c) vt[static_cast<int64_t>(blk) * kD * kD + c * kD + r] = y[c];
}

}  // namespace

hipError_t launch_tridiag(float *gpart, int splits, int n_blocks, float *vt, hipStream_t st) {
    if (n_blocks <= 0) return hipSuccess;
    hipLaunchKernelGGL(tridiag_kernel, dim3(static_cast<unsigned>(n_blocks)), dim3(kThreads), 0, st, gpart, splits,
                       vt);
    return hipGetLastError();
}

hipError_t launch_qr_chain(const float *vt, int n_blocks, void *stream, int32_t *counts, int32_t *rotations,
                           int n_cus, hipStream_t st) {
    if (n_blocks <= 0) return hipSuccess;
    // a wave's time is its lanes' dependent chains, nearly whatever L is, so the
    // launch takes about (rounds of resident waves) x (one wave's time): take the
    // L with the fewest rounds, the smaller L on a tie (its longest chain is
    // shorter and its waves spread over more SIMDs)
    const int lanes[3] = {64, 48, 36}, per_cu[3] = {2, 3, 4};  // 160 KiB of LDS / ((kD + 2) * 8 * L)
    int pick = 0;
    int64_t best = -1;
    for (int i = 0; i < 3; ++i) {
        const int64_t waves = (n_blocks + lanes[i] - 1) / lanes[i];
        const int64_t slots = static_cast<int64_t>(n_cus > 0 ? n_cus : 1) * per_cu[i];
        const int64_t rounds = (waves + slots - 1) / slots;
        if (best < 0 || rounds <= best) {
            best = rounds;
            pick = i;
        }
    }
    const int L = lanes[pick];
    const dim3 grid(static_cast<unsigned>((n_blocks + L - 1) / L));
    uint8_t *sp = static_cast<uint8_t *>(stream);
    if (L == 64)
        hipLaunchKernelGGL(qr_chain_kernel<64>, grid, dim3(64), 0, st, vt, n_blocks, sp, counts, rotations);
    else if (L == 48)
        hipLaunchKernelGGL(qr_chain_kernel<48>, grid, dim3(64), 0, st, vt, n_blocks, sp, counts, rotations);
    else
        hipLaunchKernelGGL(qr_chain_kernel<36>, grid, dim3(64), 0, st, vt, n_blocks, sp, counts, rotations);
    return hipGetLastError();
}

hipError_t launch_qr_apply(const float *gpart, int splits, int n_blocks, const void *stream, const int32_t *counts,
                           float *vt, hipStream_t st) {
    if (n_blocks <= 0) return hipSuccess;
    hipLaunchKernelGGL(qr_apply_kernel, dim3(static_cast<unsigned>(n_blocks)), dim3(kThreads), 0, st, gpart, splits,
                       static_cast<const uint8_t *>(stream), counts, vt);
    return hipGetLastError();
}

}  // namespace milo
