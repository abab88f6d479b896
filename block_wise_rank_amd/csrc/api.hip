// libmilo C ABI: host-side validation, workspace planning and kernel sequencing.
// Every check runs before anything is enqueued, so a failing call writes nothing.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/milo.h"
#include "kernels.hpp"

namespace {

thread_local std::string g_last_error;

// Measurement aid: while enabled on a thread, every kernel launched by that
// thread's calls is bracketed by HIP events on the call's stream.
struct ProfRecord {
    const char *name;
    hipEvent_t start, stop;
};
struct ProfState {
    bool on = false;
    std::vector<hipEvent_t> pool;
    size_t next = 0;
    std::vector<ProfRecord> recs;
};
thread_local ProfState g_prof;

hipEvent_t prof_event() {
    if (g_prof.next < g_prof.pool.size()) return g_prof.pool[g_prof.next++];
    hipEvent_t ev = nullptr;
    if (hipEventCreate(&ev) != hipSuccess) return nullptr;
    g_prof.pool.push_back(ev);
    g_prof.next = g_prof.pool.size();
    return ev;
}

// Run a launcher (returning hipError_t) with optional event brackets.
template <typename Fn>
hipError_t timed(const char *name, hipStream_t s, Fn &&fn) {
    hipEvent_t a = nullptr, b = nullptr;
    if (g_prof.on && (a = prof_event())) hipEventRecord(a, s);
    hipError_t e = fn();
    if (g_prof.on && a && (b = prof_event())) {
        hipEventRecord(b, s);
        g_prof.recs.push_back({name, a, b});
    }
    return e;
}

milo_status fail(milo_status s, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return s;
}

milo_status ok() {
    g_last_error.clear();
    return MILO_OK;
}

milo_status hip_fail(hipError_t e, const char *what) {
    return fail(MILO_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

int elem_bytes(milo_dtype t) { return t == MILO_F32 ? 4 : (t == MILO_BF16 ? 2 : 1); }
bool factor_dtype_ok(milo_dtype t) {
    return t == MILO_F32 || t == MILO_BF16 || t == MILO_I8 || t == MILO_I4 || t == MILO_I2;
}
bool grouped(milo_dtype t) { return t == MILO_I4 || t == MILO_I2; }
int kernel_type(milo_dtype t) {
    switch (t) {
        case MILO_F32: return milo::kF32;
        case MILO_BF16: return milo::kBF16;
        case MILO_I8: return milo::kI8;
        case MILO_I4: return milo::kI4;
        default: return milo::kI2;
    }
}
// Bytes one rank takes in a block's A part (n = T elements) and B part (n = d):
// MILO_I4 holds half a byte per element, MILO_I2 a quarter, both with an fp32
// scale per 32 elements after the codes.
int64_t rank_bytes(milo_dtype t, int n) {
    if (t == MILO_I4) return n / 2 + 4 * (n / 32);
    if (t == MILO_I2) return n / 4 + 4 * (n / 32);
    return static_cast<int64_t>(n) * elem_bytes(t);
}
int64_t a_rank_bytes(milo_dtype t, int T) { return rank_bytes(t, T); }
int64_t b_rank_bytes(milo_dtype t, int d) { return rank_bytes(t, d); }

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

constexpr int kD = 128;
// The Jacobi eigensolve of small launches: at most 30 sweeps; pairs below 1e-6
// relative are not rotated.  It ends after the first half sweep that closes 127
// consecutive rounds whose relative off-diagonals all stayed below 2.5e-3:
// quadratic convergence leaves them far smaller, and the singular values are then
// recomputed as Rayleigh quotients ||X v||, second order in the eigenvector
// error.  Over 28 pools of the long-context workload the worst singular value
// error is 1.8% of its tolerance at 9.2 sweeps on average; half sweeps at 3e-3
// raise it to 3.5%, whole sweeps at 5e-3 to 14%, and 1e-2 exceeds it.
constexpr int kMaxSweeps = 30;
constexpr float kJacobiTol = 1e-6f;
constexpr float kJacobiStopTol = 2.5e-3f;
// Launches of at most this many blocks per CU take the Jacobi eigensolve (about
// 1.2 ms for two blocks per CU, a workgroup's latency); larger ones take
// Householder + QR, whose rotation chain is sequential per block (about 4 ms
// whatever the launch) but whose throughput is three times the Jacobi's.
constexpr int kJacobiBlocksPerCu = 8;
constexpr size_t kMat = sizeof(float) * kD * kD;  // one 128 x 128 fp32 matrix

// Split the token dimension of the Gram when there are too few blocks to fill
// the chip (partials are summed in a fixed order by the eigensolver).
int gram_splits(int n_blocks, int block_len) {
    int s = 1;
    while (n_blocks * s < 512 && s < 8 && (block_len / (s * 2)) % 64 == 0 && block_len / (s * 2) >= 64)
        s *= 2;
    return s;
}

size_t tables_bytes(int n_pools) {
    return align_up(sizeof(int32_t) * (n_pools + 1), 256) + align_up(sizeof(int64_t) * n_pools, 256) * 2;
}

// Per block: the sorted order of its eigenvectors and their scales (refine -> project).
constexpr size_t kOrder = sizeof(int32_t) * kD + sizeof(float) * kD;
// Per block, besides its Gram partials and eigenvectors: the QR iteration's
// step and rotation counts and its recorded rotations (milo::kStreamBytes).
constexpr size_t kEigExtra = kOrder + 2 * sizeof(int32_t) + milo::kStreamBytes;

size_t chunk_bytes(int n_blocks, int block_len) {
    const int s = gram_splits(n_blocks, block_len);
    return static_cast<size_t>(n_blocks) * ((s + 1) * kMat + kEigExtra);
}

milo_status check_pools(const int32_t *pool_ptr, int32_t n_pools, const int64_t *budget,
                        int32_t n_blocks) {
    if (n_pools < 0) return fail(MILO_E_INVALID, "n_pools must be >= 0 (got %d)", n_pools);
    if (!pool_ptr) return fail(MILO_E_INVALID, "pool_ptr is NULL");
    if (n_pools > 0 && !budget) return fail(MILO_E_INVALID, "budget is NULL");
    if (pool_ptr[0] != 0) return fail(MILO_E_INVALID, "pool_ptr[0] must be 0 (got %d)", pool_ptr[0]);
    for (int p = 0; p < n_pools; ++p) {
        if (pool_ptr[p + 1] < pool_ptr[p])
            return fail(MILO_E_INVALID, "pool_ptr must be non-decreasing (pool %d)", p);
        if (budget[p] < 0) return fail(MILO_E_INVALID, "budget[%d] is negative", p);
    }
    if (pool_ptr[n_pools] != n_blocks)
        return fail(MILO_E_INVALID, "pool_ptr[n_pools] = %d but n_blocks = %d", pool_ptr[n_pools],
                    n_blocks);
    return MILO_OK;
}

// Compute units of the current device (looked up once per device).
milo_status device_cus(int *n) {
    static std::mutex mu;
    static int cus[64] = {};
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    std::lock_guard<std::mutex> lock(mu);
    if (dev >= 0 && dev < 64 && cus[dev] > 0) {
        *n = cus[dev];
        return MILO_OK;
    }
    int v = 0;
    e = hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute(multiprocessor count)");
    if (dev >= 0 && dev < 64) cus[dev] = v;
    *n = v;
    return MILO_OK;
}

int64_t pool_ranks(const int32_t *pool_ptr, const int64_t *budget, int p, int k) {
    const int64_t cap = static_cast<int64_t>(pool_ptr[p + 1] - pool_ptr[p]) * k;
    return budget[p] < cap ? budget[p] : cap;
}

}  // namespace

extern "C" {

int milo_abi_version(void) { return MILO_ABI_VERSION; }

const char *milo_last_error(void) { return g_last_error.c_str(); }

const char *milo_status_string(milo_status s) {
    switch (s) {
        case MILO_OK: return "MILO_OK";
        case MILO_E_INVALID: return "MILO_E_INVALID";
        case MILO_E_UNSUPPORTED: return "MILO_E_UNSUPPORTED";
        case MILO_E_WORKSPACE: return "MILO_E_WORKSPACE";
        case MILO_E_HIP: return "MILO_E_HIP";
    }
    return "MILO_E_UNKNOWN";
}

size_t milo_arena_bytes(milo_dtype dtype, int32_t block_len, int32_t head_dim,
                        const int32_t *pool_ptr, int32_t n_pools, const int64_t *budget) {
    if (!factor_dtype_ok(dtype)) {
        fail(MILO_E_INVALID, "unknown dtype %d", static_cast<int>(dtype));
        return 0;
    }
    if (block_len <= 0 || head_dim <= 0) {
        fail(MILO_E_INVALID, "block_len and head_dim must be positive");
        return 0;
    }
    if (!pool_ptr || n_pools < 0 || (n_pools > 0 && !budget)) {
        fail(MILO_E_INVALID, "invalid pool table");
        return 0;
    }
    const int k = block_len < head_dim ? block_len : head_dim;
    size_t total = 0;
    for (int p = 0; p < n_pools; ++p) {
        if (pool_ptr[p + 1] < pool_ptr[p] || budget[p] < 0) {
            fail(MILO_E_INVALID, "invalid pool %d", p);
            return 0;
        }
        total += static_cast<size_t>(pool_ranks(pool_ptr, budget, p, k)) *
                 static_cast<size_t>(a_rank_bytes(dtype, block_len) + b_rank_bytes(dtype, head_dim));
    }
    g_last_error.clear();
    return total;
}

size_t milo_compress_workspace_bytes(int32_t n_blocks, int32_t block_len, int32_t head_dim) {
    (void)head_dim;
    if (n_blocks < 0 || block_len <= 0) return 0;
    // pool tables are sized for the worst case of one pool per block
    return tables_bytes(n_blocks) + chunk_bytes(n_blocks, block_len);
}

static milo_status read_policy(const milo_alloc_options *alloc, int *policy, uint64_t *seed) {
    if (!alloc) return MILO_OK;
    if (alloc->policy != MILO_ALLOC_ENTROPY && alloc->policy != MILO_ALLOC_UNIFORM &&
        alloc->policy != MILO_ALLOC_RANDOM)
        return fail(MILO_E_INVALID, "unknown allocation policy %d", static_cast<int>(alloc->policy));
    *policy = static_cast<int>(alloc->policy);
    *seed = alloc->seed;
    return MILO_OK;
}

milo_status milo_compress_blocks(const milo_blocks *in, const int32_t *pool_ptr, int32_t n_pools,
                                 const int64_t *budget, double eps2, float *sigma_out,
                                 double *objective_out, milo_factors *out, int32_t *sweeps_out,
                                 void *workspace, size_t *workspace_bytes, void *stream) {
    return milo_compress_blocks_ex(in, pool_ptr, n_pools, budget, eps2, sigma_out, objective_out, out,
                                   sweeps_out, nullptr, workspace, workspace_bytes, stream);
}

milo_status milo_compress_blocks_ex(const milo_blocks *in, const int32_t *pool_ptr, int32_t n_pools,
                                    const int64_t *budget, double eps2, float *sigma_out,
                                    double *objective_out, milo_factors *out, int32_t *sweeps_out,
                                    const milo_alloc_options *alloc, void *workspace,
                                    size_t *workspace_bytes, void *stream) {
    int policy = milo::kAllocEntropy;
    uint64_t seed = 0;
    if (milo_status st = read_policy(alloc, &policy, &seed); st != MILO_OK) return st;
    if (!in) return fail(MILO_E_INVALID, "in is NULL");
    if (!out) return fail(MILO_E_INVALID, "out is NULL");
    if (!workspace_bytes) return fail(MILO_E_INVALID, "workspace_bytes is NULL");
    if (in->head_dim != kD) return fail(MILO_E_UNSUPPORTED, "head_dim must be 128 (got %d)", in->head_dim);
    if (in->block_len < 128 || in->block_len % 64 != 0)
        return fail(MILO_E_UNSUPPORTED, "block_len must be a multiple of 64 and >= 128 (got %d)",
                    in->block_len);
    if (in->n_blocks < 0) return fail(MILO_E_INVALID, "n_blocks must be >= 0");
    if (in->dtype != MILO_F32 && in->dtype != MILO_BF16)
        return fail(MILO_E_UNSUPPORTED, "input dtype must be MILO_F32 or MILO_BF16");
    if (in->row_stride < in->head_dim)
        return fail(MILO_E_INVALID, "row_stride (%lld) must be >= head_dim",
                    static_cast<long long>(in->row_stride));
    const int xe = elem_bytes(in->dtype);
    if ((in->row_stride * xe) % 16 != 0)
        return fail(MILO_E_INVALID, "row_stride must keep rows 16-byte aligned");
    if (in->n_blocks > 0 && (!in->x || !aligned(in->x, 16)))
        return fail(MILO_E_INVALID, "x must be a non-NULL 16-byte aligned device pointer");
    if (!(eps2 > 0.0) || !std::isfinite(eps2)) return fail(MILO_E_INVALID, "eps2 must be finite and > 0");
    milo_status st = check_pools(pool_ptr, n_pools, budget, in->n_blocks);
    if (st != MILO_OK) return st;
    if (in->n_blocks > 0 && !sigma_out) return fail(MILO_E_INVALID, "sigma_out is NULL");
    // factor set
    if (!factor_dtype_ok(out->dtype))
        return fail(MILO_E_UNSUPPORTED, "unsupported factor dtype %d", static_cast<int>(out->dtype));
    if (grouped(out->dtype) && in->block_len % 128 != 0)
        return fail(MILO_E_UNSUPPORTED, "MILO_I4 / MILO_I2 factors need block_len a multiple of 128");
    if (out->n_blocks != in->n_blocks || out->block_len != in->block_len || out->head_dim != in->head_dim)
        return fail(MILO_E_INVALID, "factor set geometry does not match the blocks");
    const size_t need_arena = milo_arena_bytes(out->dtype, in->block_len, in->head_dim, pool_ptr, n_pools, budget);
    if (in->n_blocks > 0) {
        if (!out->rank || !out->a_off || !out->b_off)
            return fail(MILO_E_INVALID, "factor rank/a_off/b_off must be set");
        if (need_arena > 0 && (!out->arena || !aligned(out->arena, 256)))
            return fail(MILO_E_INVALID, "arena must be a non-NULL 256-byte aligned device pointer");
        if (out->arena_bytes < need_arena)
            return fail(MILO_E_INVALID, "arena_bytes %zu < %zu needed", out->arena_bytes, need_arena);
        if (out->dtype == MILO_I8 && (!out->a_scale || !out->b_scale))
            return fail(MILO_E_INVALID, "MILO_I8 factors need a_scale and b_scale");
    }
    // workspace plan: pool tables, then per-chunk Gram partials + eigenvectors
    const size_t tab = tables_bytes(n_pools);
    const size_t full = tab + chunk_bytes(in->n_blocks, in->block_len);
    int max_pool = 0;
    for (int p = 0; p < n_pools; ++p) max_pool = std::max(max_pool, pool_ptr[p + 1] - pool_ptr[p]);
    // a chunk needs at least one Gram partial, the eigenvectors, their order and
    // the QR iteration's record per block
    const size_t minimum = tab + static_cast<size_t>(max_pool) * (2 * kMat + kEigExtra);
    if (!workspace || *workspace_bytes < minimum) {
        *workspace_bytes = full;
        return fail(MILO_E_WORKSPACE, "workspace of %zu bytes needed (minimum %zu)", full, minimum);
    }
    if (!aligned(workspace, 256)) return fail(MILO_E_INVALID, "workspace must be 256-byte aligned");
    const size_t ws_cap = *workspace_bytes;

    hipStream_t s = static_cast<hipStream_t>(stream);
    int n_cus = 0;
    if (milo_status cs = device_cus(&n_cus); cs != MILO_OK) return cs;
    const int T = in->block_len;
    const int k = T < kD ? T : kD;
    const int a_bpr = static_cast<int>(a_rank_bytes(out->dtype, T)), b_bpr = static_cast<int>(b_rank_bytes(out->dtype, kD));
    const int x_type = in->dtype == MILO_F32 ? milo::kF32 : milo::kBF16;
    const int f_type = kernel_type(out->dtype);

    // pool tables -> device
    uint8_t *ws = static_cast<uint8_t *>(workspace);
    int32_t *d_pool_ptr = reinterpret_cast<int32_t *>(ws);
    int64_t *d_budget = reinterpret_cast<int64_t *>(ws + align_up(sizeof(int32_t) * (n_pools + 1), 256));
    int64_t *d_base = reinterpret_cast<int64_t *>(reinterpret_cast<uint8_t *>(d_budget) +
                                                  align_up(sizeof(int64_t) * n_pools, 256));
    std::vector<int64_t> base(n_pools);
    int64_t acc = 0;
    for (int p = 0; p < n_pools; ++p) {
        base[p] = acc;
        acc += pool_ranks(pool_ptr, budget, p, k) * static_cast<int64_t>(a_bpr + b_bpr);
    }
    hipError_t e;
    if (n_pools > 0) {
        e = hipMemcpyAsync(d_pool_ptr, pool_ptr, sizeof(int32_t) * (n_pools + 1), hipMemcpyHostToDevice, s);
        if (e != hipSuccess) return hip_fail(e, "pool table upload");
        e = hipMemcpyAsync(d_budget, budget, sizeof(int64_t) * n_pools, hipMemcpyHostToDevice, s);
        if (e != hipSuccess) return hip_fail(e, "budget upload");
        e = hipMemcpyAsync(d_base, base.data(), sizeof(int64_t) * n_pools, hipMemcpyHostToDevice, s);
        if (e != hipSuccess) return hip_fail(e, "pool base upload");
    }
    uint8_t *chunk_ws = ws + tab;
    const size_t chunk_cap = ws_cap - tab;

    const uint8_t *xb = static_cast<const uint8_t *>(in->x);
    int p0 = 0;
    while (p0 < n_pools) {
        // grow the chunk while its workspace fits
        int p1 = p0 + 1;
        while (p1 < n_pools &&
               static_cast<size_t>(pool_ptr[p1 + 1] - pool_ptr[p0]) * (2 * kMat + kEigExtra) <= chunk_cap)
            ++p1;
        const int b0 = pool_ptr[p0], nb = pool_ptr[p1] - b0;
        if (nb > 0) {
            // Gram token splits: enough workgroups to fill the chip, within the workspace.
            const int fit = static_cast<int>((chunk_cap - static_cast<size_t>(nb) * kEigExtra) /
                                             (static_cast<size_t>(nb) * kMat)) - 1;
            int splits = gram_splits(nb, T);
            while (splits > 1 && splits > fit) splits /= 2;  // powers of two keep T / splits % 64 == 0
            float *gpart = reinterpret_cast<float *>(chunk_ws);
            float *vt = reinterpret_cast<float *>(chunk_ws + static_cast<size_t>(nb) * splits * kMat);
            int32_t *vperm = reinterpret_cast<int32_t *>(reinterpret_cast<uint8_t *>(vt) + static_cast<size_t>(nb) * kMat);
            float *vscale = reinterpret_cast<float *>(vperm + static_cast<size_t>(nb) * kD);
            int32_t *qr_counts = reinterpret_cast<int32_t *>(vscale + static_cast<size_t>(nb) * kD);
            uint8_t *qr_stream = reinterpret_cast<uint8_t *>(qr_counts + 2 * static_cast<size_t>(nb));
            // block b of the chunk: row0 points into the caller's table, else blocks back to back
            const int64_t *row0 = in->row0 ? in->row0 + b0 : nullptr;
            const void *xc = in->row0 ? static_cast<const void *>(xb)
                                      : static_cast<const void *>(xb + static_cast<size_t>(b0) * T * in->row_stride * xe);
            float *sig = sigma_out + static_cast<size_t>(b0) * kD;
            if ((e = timed("gram", s, [&] { return milo::launch_gram(xc, x_type, row0, in->row_stride, T, nb, splits, gpart, s); })) != hipSuccess)
                return hip_fail(e, "gram launch");
            int32_t *rot_out = sweeps_out ? sweeps_out + b0 : nullptr;
            if (nb <= kJacobiBlocksPerCu * n_cus) {
                if ((e = timed("jacobi", s, [&] {
                         return milo::launch_jacobi(gpart, splits, nb, vt, rot_out, kMaxSweeps, kJacobiTol,
                                                    kJacobiStopTol, n_cus, s);
                     })) != hipSuccess)
                    return hip_fail(e, "jacobi launch");
            } else {
                if ((e = timed("tridiag", s, [&] { return milo::launch_tridiag(gpart, splits, nb, vt, s); })) !=
                    hipSuccess)
                    return hip_fail(e, "tridiagonalisation launch");
                if ((e = timed("qr_chain", s, [&] {
                         return milo::launch_qr_chain(vt, nb, qr_stream, qr_counts, rot_out, n_cus, s);
                     })) != hipSuccess)
                    return hip_fail(e, "QR iteration launch");
                if ((e = timed("qr_apply", s, [&] {
                         return milo::launch_qr_apply(gpart, splits, nb, qr_stream, qr_counts, vt, s);
                     })) != hipSuccess)
                    return hip_fail(e, "QR rotation launch");
            }
            if ((e = timed("refine", s, [&] { return milo::launch_refine(xc, x_type, row0, in->row_stride, T, nb, vt, sig, vperm, vscale, s); })) != hipSuccess)
                return hip_fail(e, "refine launch");
            if ((e = timed("alloc", s, [&] {
                     return milo::launch_alloc(sig, kD, k, d_pool_ptr, d_budget, d_base, p0, p1 - p0, b0,
                                               eps2, out->rank, objective_out, out->a_off, out->b_off, a_bpr,
                                               b_bpr, policy, seed, s);
                 })) != hipSuccess)
                return hip_fail(e, "alloc launch");
            if ((e = timed("project", s, [&] {
                     return milo::launch_project(
                         xc, x_type, row0, in->row_stride, T, nb, vt, vperm, vscale, out->rank + b0, out->a_off + b0,
                         out->b_off + b0, out->arena, f_type,
                         out->a_scale ? out->a_scale + static_cast<size_t>(b0) * T : nullptr,
                         out->b_scale ? out->b_scale + static_cast<size_t>(b0) * kD : nullptr, s);
                 })) != hipSuccess)
                return hip_fail(e, "project launch");
        } else {
            if ((e = milo::launch_alloc(sigma_out, kD, k, d_pool_ptr, d_budget, d_base, p0, p1 - p0, b0,
                                        eps2, out->rank, objective_out, out->a_off, out->b_off, a_bpr,
                                        b_bpr, policy, seed, s)) != hipSuccess)
                return hip_fail(e, "alloc launch");
        }
        p0 = p1;
    }
    return ok();
}

milo_status milo_allocate_ranks(const float *sigma, int32_t n_blocks, int32_t head_dim,
                                int32_t max_rank, const int32_t *pool_ptr, int32_t n_pools,
                                const int64_t *budget, double eps2, int32_t *rank_out,
                                double *objective_out, void *workspace, size_t *workspace_bytes,
                                void *stream) {
    return milo_allocate_ranks_ex(sigma, n_blocks, head_dim, max_rank, pool_ptr, n_pools, budget, eps2,
                                  rank_out, objective_out, nullptr, workspace, workspace_bytes, stream);
}

milo_status milo_allocate_ranks_ex(const float *sigma, int32_t n_blocks, int32_t head_dim,
                                   int32_t max_rank, const int32_t *pool_ptr, int32_t n_pools,
                                   const int64_t *budget, double eps2, int32_t *rank_out,
                                   double *objective_out, const milo_alloc_options *alloc,
                                   void *workspace, size_t *workspace_bytes, void *stream) {
    int policy = milo::kAllocEntropy;
    uint64_t seed = 0;
    if (milo_status st = read_policy(alloc, &policy, &seed); st != MILO_OK) return st;
    if (head_dim <= 0) return fail(MILO_E_INVALID, "head_dim must be > 0");
    if (max_rank < 1 || max_rank > head_dim)
        return fail(MILO_E_INVALID, "max_rank must be in [1, head_dim] (got %d)", max_rank);
    if (n_blocks < 0) return fail(MILO_E_INVALID, "n_blocks must be >= 0");
    if (n_blocks > 0 && (!sigma || !rank_out)) return fail(MILO_E_INVALID, "sigma and rank_out must be set");
    if (!(eps2 > 0.0) || !std::isfinite(eps2)) return fail(MILO_E_INVALID, "eps2 must be finite and > 0");
    if (!workspace_bytes) return fail(MILO_E_INVALID, "workspace_bytes is NULL");
    milo_status st = check_pools(pool_ptr, n_pools, budget, n_blocks);
    if (st != MILO_OK) return st;
    const size_t need = tables_bytes(n_pools);
    if (!workspace || *workspace_bytes < need) {
        *workspace_bytes = need;
        return fail(MILO_E_WORKSPACE, "workspace of %zu bytes needed", need);
    }
    if (!aligned(workspace, 256)) return fail(MILO_E_INVALID, "workspace must be 256-byte aligned");
    if (n_pools == 0) return ok();
    hipStream_t s = static_cast<hipStream_t>(stream);
    uint8_t *ws = static_cast<uint8_t *>(workspace);
    int32_t *d_pool_ptr = reinterpret_cast<int32_t *>(ws);
    int64_t *d_budget = reinterpret_cast<int64_t *>(ws + align_up(sizeof(int32_t) * (n_pools + 1), 256));
    hipError_t e;
    if ((e = hipMemcpyAsync(d_pool_ptr, pool_ptr, sizeof(int32_t) * (n_pools + 1), hipMemcpyHostToDevice, s)) != hipSuccess ||
        (e = hipMemcpyAsync(d_budget, budget, sizeof(int64_t) * n_pools, hipMemcpyHostToDevice, s)) != hipSuccess)
        return hip_fail(e, "pool table upload");
    e = timed("alloc", s, [&] {
        return milo::launch_alloc(sigma, head_dim, max_rank, d_pool_ptr, d_budget, nullptr, 0, n_pools, 0,
                                  eps2, rank_out, objective_out, nullptr, nullptr, 0, 0, policy, seed, s);
    });
    if (e != hipSuccess) return hip_fail(e, "alloc launch");
    return ok();
}

milo_status milo_reconstruct(const milo_factors *f, const int32_t *block_ids, int32_t n_ids,
                             void *x_out, milo_dtype out_dtype, void *stream) {
    return milo_reconstruct_ex(f, block_ids, n_ids, x_out, nullptr, out_dtype, stream);
}

milo_status milo_reconstruct_ex(const milo_factors *f, const int32_t *block_ids, int32_t n_ids,
                                void *x_out, const int64_t *out_off, milo_dtype out_dtype, void *stream) {
    if (!f) return fail(MILO_E_INVALID, "factor set is NULL");
    if (f->head_dim != kD) return fail(MILO_E_UNSUPPORTED, "head_dim must be 128");
    if (f->block_len < 128 || f->block_len % 64 != 0)
        return fail(MILO_E_UNSUPPORTED, "block_len must be a multiple of 64 and >= 128");
    if (!factor_dtype_ok(f->dtype)) return fail(MILO_E_INVALID, "unknown factor dtype");
    if (grouped(f->dtype) && f->block_len % 128 != 0)
        return fail(MILO_E_UNSUPPORTED, "MILO_I4 / MILO_I2 factors need block_len a multiple of 128");
    if (out_dtype != MILO_F32 && out_dtype != MILO_BF16)
        return fail(MILO_E_UNSUPPORTED, "out_dtype must be MILO_F32 or MILO_BF16");
    if (n_ids < 0) return fail(MILO_E_INVALID, "n_ids must be >= 0");
    if (n_ids == 0) return ok();
    if (!block_ids || !x_out) return fail(MILO_E_INVALID, "block_ids and x_out must be set");
    if (!f->rank || !f->a_off || !f->b_off || !f->arena)
        return fail(MILO_E_INVALID, "factor set pointers must be set");
    if (f->dtype == MILO_I8 && (!f->a_scale || !f->b_scale))
        return fail(MILO_E_INVALID, "MILO_I8 factors need scales");
    const int ft = kernel_type(f->dtype);
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = timed("reconstruct", s, [&] {
        return milo::launch_reconstruct(f->arena, ft, f->rank, f->a_off, f->b_off, f->a_scale,
                                        f->b_scale, f->block_len, block_ids, n_ids, x_out, out_off,
                                        out_dtype == MILO_F32 ? milo::kF32 : milo::kBF16, s);
    });
    if (e != hipSuccess) return hip_fail(e, "reconstruct launch");
    return ok();
}

milo_status milo_fetch_blocks(const milo_factors *host, const milo_factors *dev, const int32_t *blocks,
                              int32_t n, void *stream) {
    if (!host || !dev) return fail(MILO_E_INVALID, "host and dev factor sets must be given");
    if (host->dtype != dev->dtype) return fail(MILO_E_INVALID, "host and dev dtypes differ");
    if (!factor_dtype_ok(host->dtype)) return fail(MILO_E_INVALID, "unknown factor dtype");
    if (host->n_blocks != dev->n_blocks || host->block_len != dev->block_len || host->head_dim != dev->head_dim)
        return fail(MILO_E_INVALID, "host and dev geometries differ");
    if (host->n_blocks < 0 || host->block_len < 1 || host->head_dim < 1) return fail(MILO_E_INVALID, "bad geometry");
    if (dev->arena_bytes < host->arena_bytes) return fail(MILO_E_INVALID, "dev arena smaller than host arena");
    if (n < 0) return fail(MILO_E_INVALID, "n must be >= 0");
    if (n == 0) return ok();
    if (!blocks) return fail(MILO_E_INVALID, "blocks must be set");
    if (!host->rank || !host->a_off || !host->b_off || !host->arena || !dev->arena)
        return fail(MILO_E_INVALID, "factor set pointers must be set");
    const bool i8 = host->dtype == MILO_I8;
    if (i8 && (!host->a_scale || !host->b_scale || !dev->a_scale || !dev->b_scale))
        return fail(MILO_E_INVALID, "MILO_I8 factors need scales");
    const int64_t T = host->block_len, d = host->head_dim, cap = static_cast<int64_t>(host->arena_bytes);
    if (grouped(host->dtype) && (T % 32 != 0 || d % 32 != 0))
        return fail(MILO_E_INVALID, "MILO_I4 / MILO_I2 geometry must hold whole 32-element groups");
    const int64_t abpr = a_rank_bytes(host->dtype, static_cast<int>(T)), bbpr = b_rank_bytes(host->dtype, static_cast<int>(d));
    // byte runs [begin, end) of the arena, and of the two scale arrays, in list order
    struct Run { int64_t b, e; };
    std::vector<Run> arena, sa, sb;
    auto add = [](std::vector<Run> &v, int64_t b, int64_t e) {
        if (e <= b) return;
        if (!v.empty() && v.back().e == b) v.back().e = e;
        else v.push_back({b, e});
    };
    for (int32_t i = 0; i < n; ++i) {
        const int32_t id = blocks[i];
        if (id < 0 || id >= host->n_blocks) return fail(MILO_E_INVALID, "block id %d out of range", id);
        const int64_t r = host->rank[id];
        if (r < 0 || r > (T < d ? T : d)) return fail(MILO_E_INVALID, "block %d has rank %lld", id, (long long)r);
        const int64_t a0 = host->a_off[id], b0 = host->b_off[id];
        if (a0 < 0 || b0 < 0 || a0 + r * abpr > cap || b0 + r * bbpr > cap)
            return fail(MILO_E_INVALID, "block %d reaches past the arena", id);
        add(arena, a0, a0 + r * abpr);
        add(arena, b0, b0 + r * bbpr);
        if (i8) {
            add(sa, static_cast<int64_t>(id) * T * 4, (static_cast<int64_t>(id) + 1) * T * 4);
            add(sb, static_cast<int64_t>(id) * d * 4, (static_cast<int64_t>(id) + 1) * d * 4);
        }
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = timed("fetch", s, [&] {
        auto copy = [&](const std::vector<Run> &v, const void *src, void *dst) {
            for (const Run &q : v) {
                hipError_t r = hipMemcpyAsync(static_cast<uint8_t *>(dst) + q.b, static_cast<const uint8_t *>(src) + q.b,
                                              static_cast<size_t>(q.e - q.b), hipMemcpyHostToDevice, s);
                if (r != hipSuccess) return r;
            }
            return hipSuccess;
        };
        hipError_t r = copy(arena, host->arena, dev->arena);
        if (r == hipSuccess && i8) r = copy(sa, host->a_scale, dev->a_scale);
        if (r == hipSuccess && i8) r = copy(sb, host->b_scale, dev->b_scale);
        return r;
    });
    if (e != hipSuccess) return hip_fail(e, "fetch copies");
    return ok();
}

}  // extern "C"

namespace {

// milo_decode_attention's work with the scratch given explicitly: `ws` of
// `ws_bytes` bytes (the caller's workspace, or this device's static scratch).
milo_status decode_attention(const milo_decode_args *a, size_t *workspace_needed, void *ws, size_t ws_bytes,
                             void *stream) {
    if (!a) return fail(MILO_E_INVALID, "args is NULL");
    if (a->head_dim != kD) return fail(MILO_E_UNSUPPORTED, "head_dim must be 128 (got %d)", a->head_dim);
    if (a->batch < 0) return fail(MILO_E_INVALID, "batch must be >= 0");
    if (a->n_kv_heads < 1 || a->n_q_heads < 1 || a->n_q_heads % a->n_kv_heads != 0)
        return fail(MILO_E_INVALID, "n_q_heads must be a positive multiple of n_kv_heads");
    const int G = a->n_q_heads / a->n_kv_heads;
    if (G > 16) return fail(MILO_E_UNSUPPORTED, "at most 16 query heads per KV head (got %d)", G);
    if (!a->k || !a->v) return fail(MILO_E_INVALID, "k and v factor sets must be given");
    const milo_factors *k = a->k, *v = a->v;
    if (k->dtype != v->dtype) return fail(MILO_E_UNSUPPORTED, "K and V factors must share a dtype");
    if (!factor_dtype_ok(k->dtype)) return fail(MILO_E_INVALID, "unknown factor dtype");
    if (k->head_dim != kD || v->head_dim != kD) return fail(MILO_E_UNSUPPORTED, "factor head_dim must be 128");
    if (k->block_len != v->block_len) return fail(MILO_E_INVALID, "K and V block_len differ");
    const int T = k->block_len;
    if (T < 128 || T % 64 != 0) return fail(MILO_E_UNSUPPORTED, "block_len must be a multiple of 64 and >= 128");
    if (grouped(k->dtype) && T % 128 != 0)
        return fail(MILO_E_UNSUPPORTED, "MILO_I4 / MILO_I2 factors need block_len a multiple of 128");
    if (a->blocks_per_seq < 0) return fail(MILO_E_INVALID, "blocks_per_seq must be >= 0");
    const int64_t need_blocks = static_cast<int64_t>(a->batch) * a->n_kv_heads * a->blocks_per_seq;
    if (k->n_blocks < need_blocks || v->n_blocks < need_blocks)
        return fail(MILO_E_INVALID, "factor sets hold fewer than batch * n_kv_heads * blocks_per_seq blocks");
    if (need_blocks > 0) {
        if (!k->rank || !k->a_off || !k->b_off || !k->arena || !v->rank || !v->a_off || !v->b_off || !v->arena)
            return fail(MILO_E_INVALID, "factor set pointers must be set");
        if (k->dtype == MILO_I8 && (!k->a_scale || !k->b_scale || !v->a_scale || !v->b_scale))
            return fail(MILO_E_INVALID, "MILO_I8 factors need scales");
    }
    if (a->q_dtype != MILO_F32 && a->q_dtype != MILO_BF16) return fail(MILO_E_UNSUPPORTED, "q_dtype must be F32 or BF16");
    if (a->out_dtype != MILO_F32 && a->out_dtype != MILO_BF16) return fail(MILO_E_UNSUPPORTED, "out_dtype must be F32 or BF16");
    if (a->batch > 0 && (!a->q || !a->q_pos || !a->out)) return fail(MILO_E_INVALID, "q, q_pos and out must be set");
    if (a->batch > 0 && !aligned(a->q, 16)) return fail(MILO_E_INVALID, "q must be 16-byte aligned");
    if (need_blocks > 0 && (!aligned(k->arena, 16) || !aligned(v->arena, 16)))
        return fail(MILO_E_INVALID, "factor arenas must be 16-byte aligned");
    if (a->sel_ptr) {
        if (!a->sel_blk && a->sel_max > 0) return fail(MILO_E_INVALID, "sel_blk is NULL");
        if (a->sel_max < 0 || a->sel_max > a->blocks_per_seq)
            return fail(MILO_E_INVALID, "sel_max must be in [0, blocks_per_seq]");
    }
    const bool tail = a->tail_k != nullptr;
    const bool segs = a->tail_seg_pos != nullptr;
    if (segs && !tail) return fail(MILO_E_INVALID, "tail_seg_pos needs tail_k");
    if (tail) {
        if (!a->tail_v) return fail(MILO_E_INVALID, "tail_v must be set");
        if (segs) {
            if (!a->tail_seg_valid) return fail(MILO_E_INVALID, "tail_seg_valid must be set with tail_seg_pos");
            if (a->tail_seg_len <= 0 || a->tail_seg_len % 128 != 0 || a->tail_cap % a->tail_seg_len != 0)
                return fail(MILO_E_UNSUPPORTED, "tail_seg_len must be a positive multiple of 128 dividing tail_cap");
        } else if (!a->tail_len || !a->tail_pos0) {
            return fail(MILO_E_INVALID, "tail_len and tail_pos0 must be set");
        }
        if (a->tail_cap <= 0 || a->tail_cap % 64 != 0) return fail(MILO_E_UNSUPPORTED, "tail_cap must be a positive multiple of 64");
        if (a->tail_dtype != MILO_F32 && a->tail_dtype != MILO_BF16) return fail(MILO_E_UNSUPPORTED, "tail_dtype must be F32 or BF16");
        const int te = elem_bytes(a->tail_dtype);
        if (!aligned(a->tail_k, 16) || !aligned(a->tail_v, 16) || te == 0)
            return fail(MILO_E_INVALID, "tail buffers must be 16-byte aligned");
    }
    if (!(a->rope_base > 1.0) || !std::isfinite(a->rope_base)) return fail(MILO_E_INVALID, "rope_base must be finite and > 1");
    if (!std::isfinite(a->softmax_scale)) return fail(MILO_E_INVALID, "softmax_scale must be finite");
    const int ftype = kernel_type(k->dtype);
    const int ttype = a->tail_dtype == MILO_F32 ? milo::kF32 : milo::kBF16;
    int split = a->split_len;
    if (split == 0) {
        // The longest split that still gives a workgroup to every CU (256),
        // counting the tail's: each split pays a prologue (B_k fragments,
        // rotated queries) and a merge, and one workgroup fills a CU (its LDS
        // and registers), so more, shorter splits only add rounds of those.
        const int64_t units = static_cast<int64_t>(a->batch) * a->n_kv_heads *
                              (a->sel_ptr ? a->sel_max : a->blocks_per_seq);
        const int64_t tail_units = tail ? static_cast<int64_t>(a->batch) * a->n_kv_heads : 0;
        split = 128;
        for (int c = 2048; c > 128; c /= 2)
            if (T % c == 0 && (!segs || a->tail_seg_len % c == 0) &&
                units * (T / c) + tail_units * ((a->tail_cap + c - 1) / c) >= 256 &&
                milo::decode_split_fits(ftype, ttype, tail, G, c)) {
                split = c;
                break;
            }
    }
    if (split < 128 || split % 128 != 0 || T % split != 0 || split > 32 * milo::kMaxTiles)
        return fail(MILO_E_UNSUPPORTED, "split_len must be a multiple of 128, at most 2048, dividing block_len");
    if (segs && a->tail_seg_len % split != 0)
        return fail(MILO_E_UNSUPPORTED, "split_len %d must divide tail_seg_len %d", split, a->tail_seg_len);
    if (!milo::decode_split_fits(ftype, ttype, tail, G, split))
        return fail(MILO_E_UNSUPPORTED, "split_len %d needs more LDS than a workgroup has for %d query heads per KV head", split, G);

    milo::DecodeParams p{};
    p.q = a->q;
    p.q_type = a->q_dtype == MILO_F32 ? milo::kF32 : milo::kBF16;
    p.q_pos = a->q_pos;
    p.batch = a->batch;
    p.n_q_heads = a->n_q_heads;
    p.n_kv_heads = a->n_kv_heads;
    p.group = G;
    p.f_type = kernel_type(k->dtype);
    p.block_len = T;
    p.blocks_per_seq = a->blocks_per_seq;
    p.k_rank = k->rank; p.v_rank = v->rank;
    p.k_aoff = k->a_off; p.k_boff = k->b_off; p.v_aoff = v->a_off; p.v_boff = v->b_off;
    p.k_arena = static_cast<const uint8_t *>(k->arena);
    p.v_arena = static_cast<const uint8_t *>(v->arena);
    p.k_ascale = k->a_scale; p.k_bscale = k->b_scale; p.v_ascale = v->a_scale; p.v_bscale = v->b_scale;
    p.sel_ptr = a->sel_ptr;
    p.sel_blk = a->sel_blk;
    p.n_sel = a->sel_ptr ? a->sel_max : a->blocks_per_seq;
    p.tail_k = a->tail_k;
    p.tail_v = a->tail_v;
    p.tail_type = a->tail_dtype == MILO_F32 ? milo::kF32 : milo::kBF16;
    p.tail_cap = tail ? a->tail_cap : 0;
    p.tail_len = a->tail_len;
    p.tail_pos0 = a->tail_pos0;
    p.tail_seg_pos = segs ? a->tail_seg_pos : nullptr;
    p.tail_seg_valid = segs ? a->tail_seg_valid : nullptr;
    p.tail_seg_len = segs ? a->tail_seg_len : 0;
    p.rope_base = a->rope_base;
    p.softmax_scale = a->softmax_scale;
    p.out = a->out;
    p.out_type = a->out_dtype == MILO_F32 ? milo::kF32 : milo::kBF16;
    p.split_len = split;
    p.block_splits = T / split;
    p.tail_splits = tail ? (a->tail_cap + split - 1) / split : 0;
    p.n_splits = p.n_sel * p.block_splits + p.tail_splits;

    const size_t need = milo::decode_workspace_bytes(p);
    if (workspace_needed) *workspace_needed = need;
    if (!ws || ws_bytes < need)
        return fail(MILO_E_WORKSPACE, "workspace of %zu bytes needed (%zu given)", need, ws ? ws_bytes : 0);
    if (!aligned(ws, 256)) return fail(MILO_E_INVALID, "workspace must be 256-byte aligned");
    const size_t n = static_cast<size_t>(p.batch) * p.n_kv_heads * p.n_splits * G;
    const size_t ml_bytes = align_up(n * 2 * sizeof(float), 256), po_bytes = align_up(n * kD * sizeof(float), 256);
    p.part_ml = static_cast<float *>(ws);
    p.part_o = reinterpret_cast<float *>(static_cast<uint8_t *>(ws) + ml_bytes);
    uint8_t *tabs = static_cast<uint8_t *>(ws) + ml_bytes + po_bytes;
    p.theta = reinterpret_cast<double *>(tabs);
    p.rope_tab = reinterpret_cast<float2 *>(tabs + 64 * sizeof(double));
    p.step_tab = p.rope_tab + 32 * 64;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (p.batch == 0) return ok();
    hipError_t e = hipSuccess;
    if ((e = timed("decode_tables", s, [&] { return milo::launch_decode_tables(p, s); })) != hipSuccess)
        return hip_fail(e, "decode table launch");
    if ((e = timed("decode", s, [&] { return milo::launch_decode(p, s); })) != hipSuccess)
        return hip_fail(e, "decode launch");
    if ((e = timed("decode_combine", s, [&] { return milo::launch_decode_combine(p, s); })) != hipSuccess)
        return hip_fail(e, "decode combine launch");
    return ok();
}

// Scratch of milo_decode_attention_noalloc: a static device array, so that the
// entry point never allocates.  Every GPU the library runs on holds its own copy
// for the life of the process.  In host code `scratch` only names the symbol;
// its device address, per device, comes from hipGetSymbolAddress and is kept
// here, set once per device on the first call there.
constexpr size_t kScratchBytes = MILO_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices] = {};

milo_status device_scratch(void **ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(MILO_E_UNSUPPORTED, "device ordinal %d beyond %d", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
        if (!p) return fail(MILO_E_HIP, "hipGetSymbolAddress(scratch) gave NULL");
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return MILO_OK;
}

}  // namespace

extern "C" {

milo_status milo_decode_attention(const milo_decode_args *a, size_t *workspace_needed, void *stream) {
    if (!a) return fail(MILO_E_INVALID, "args is NULL");
    return decode_attention(a, workspace_needed, a->workspace, a->workspace_bytes, stream);
}

milo_status milo_decode_attention_noalloc(const milo_decode_args *a, void *stream) {
    if (!a) return fail(MILO_E_INVALID, "args is NULL");
    void *ws = nullptr;
    if (milo_status st = device_scratch(&ws); st != MILO_OK) return st;
    size_t need = 0;
    const milo_status st = decode_attention(a, &need, ws, kScratchBytes, stream);
    if (st == MILO_E_WORKSPACE)
        return fail(MILO_E_WORKSPACE, "the call needs %zu bytes of scratch; milo_decode_attention_noalloc "
                    "has %zu (MILO_NOALLOC_SCRATCH_BYTES)", need, kScratchBytes);
    return st;
}

int milo_profile_enable(int on) {
    const int prev = g_prof.on ? 1 : 0;
    g_prof.on = on != 0;
    return prev;
}

int milo_profile_read(const char **names, int32_t *launches, double *total_ms, int cap) {
    std::vector<const char *> keys;
    std::vector<int32_t> cnt;
    std::vector<double> ms;
    for (const ProfRecord &r : g_prof.recs) {
        float t = 0.f;
        if (hipEventSynchronize(r.stop) != hipSuccess || hipEventElapsedTime(&t, r.start, r.stop) != hipSuccess) {
            fail(MILO_E_HIP, "profile event failed");
            g_prof.recs.clear();
            g_prof.next = 0;
            return -1;
        }
        size_t i = 0;
        while (i < keys.size() && std::strcmp(keys[i], r.name) != 0) ++i;
        if (i == keys.size()) {
            keys.push_back(r.name);
            cnt.push_back(0);
            ms.push_back(0.0);
        }
        cnt[i] += 1;
        ms[i] += t;
    }
    g_prof.recs.clear();
    g_prof.next = 0;
    const int n = static_cast<int>(keys.size());
    for (int i = 0; i < n && i < cap; ++i) {
        if (names) names[i] = keys[i];
        if (launches) launches[i] = cnt[i];
        if (total_ms) total_ms[i] = ms[i];
    }
    return n;
}

}  // extern "C"
