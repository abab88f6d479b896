// Global rank allocation within a pool of blocks.
//
// The allocation maximises sum_b sum_{i < r_b} log(1 + sigma_{b,i}^2 / eps^2)
// under sum_b r_b <= R by handing out one rank at a time to the block with the
// largest marginal gain (evolve.pub review of arXiv 2609.29913, Strengths,
// Eqs 5-7).  The gain is strictly increasing in sigma and every block's
// singular values are non-increasing, so the greedy hands out exactly the R'
// = min(R, n k) largest singular values of the pool in the order
// (sigma desc, block asc, index asc), and r_b counts block b's share.  This
// kernel computes that selection directly:
//   1. the R'-th largest sigma, tau, by a bitwise search over the fp32 bit
//      patterns (monotone for sigma >= 0): 31 rounds, each counting the keys
//      >= a candidate.  Pools of up to 8192 keys hold them in registers (32 per
//      thread) and each round is a register count plus one barrier; larger pools
//      count per block with a binary search over its sorted row;
//   2. every value > tau is taken; the remaining R' - #{> tau} ranks go to the
//      values == tau in block order (an exclusive scan over the blocks).
// Exact integer work on fp32 keys: the ranks do not depend on eps, and equal
// the greedy's bit for bit.  One workgroup of 256 threads per pool; thread t
// owns a contiguous run of blocks so prefix sums follow block order.
//
// The same selection serves the equal-budget comparisons the greedy is ablated
// against (same review, Strengths, on Fig. 5(d)):
//   uniform  block j of the pool gets floor(R'/n) ranks, one more if j < R' mod n;
//   random   the R' (block, index) slots with the largest 32-bit keys, key =
//            high half of SplitMix64 output 1 + (pool << 32 | j << 8 | i) for the
//            caller's seed (Steele, Lea & Flood 2014, Stafford's finaliser 13):
//            a uniformly random R'-subset of the slots; a block's rank is the
//            number of its slots taken.  Keys are not sorted within a block, so
//            they are counted by a scan instead of a binary search.
#include "common.hpp"
#include "kernels.hpp"

namespace milo {
namespace {

__device__ __forceinline__ uint64_t splitmix64(uint64_t seed, uint64_t c) {
    uint64_t z = seed + c * 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

__device__ __forceinline__ uint32_t random_key(uint64_t seed, int pool, int j, int i) {
    const uint64_t c = (static_cast<uint64_t>(static_cast<uint32_t>(pool)) << 32) |
                       (static_cast<uint64_t>(j) << 8) | static_cast<uint64_t>(i);
    return static_cast<uint32_t>(splitmix64(seed, c + 1) >> 32);
}

// Number of block j's random keys that are >= c.
__device__ __forceinline__ int count_ge_random(uint64_t seed, int pool, int j, int k, uint32_t c) {
    int n = 0;
    for (int i = 0; i < k; ++i) n += random_key(seed, pool, j, i) >= c;
    return n;
}

__device__ __forceinline__ uint32_t key_bits(float s) {
    const uint32_t u = __float_as_uint(s);
    return (u >> 31) ? 0u : u;  // -0.0 (or any negative) counts as 0
}

// Number of leading entries of a non-increasing row whose key is >= c.
__device__ __forceinline__ int count_ge(const float *row, int k, uint32_t c) {
    int lo = 0, hi = k;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (key_bits(row[mid]) >= c)
            lo = mid + 1;
        else
            hi = mid;
    }
    return lo;
}

template <typename Tv>
__device__ Tv block_sum(Tv v, Tv *red) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) v += __shfl_xor(v, o, 64);
    __syncthreads();
    if (lane == 0) red[wave] = v;
    __syncthreads();
    Tv tot = red[0] + red[1] + red[2] + red[3];
    return tot;
}

// Exclusive prefix over the 256 threads (thread order), returns the prefix:
// an inclusive scan inside each wave (shuffles), then the totals of the waves
// before (one barrier).  buf holds at least 4 entries.
__device__ int64_t block_exclusive_scan(int64_t v, int64_t *buf) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int64_t x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int64_t y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
    }
    __syncthreads();  // earlier readers of buf are done
    if (lane == 63) buf[wave] = x;
    __syncthreads();
    int64_t before = 0;
    for (int w = 0; w < wave; ++w) before += buf[w];
    return before + x - v;
}

constexpr int kKeysPerThread = 32;  // pools of up to 8192 keys are searched in registers

__global__ __launch_bounds__(256) void alloc_kernel(
    const float *__restrict__ sigma, int pitch, int k, const int32_t *__restrict__ pool_ptr,
    const int64_t *__restrict__ budget, const int64_t *__restrict__ pool_base, int pool_lo,
    int blk_lo, double eps2, int32_t *__restrict__ rank, double *__restrict__ objective,
    int64_t *__restrict__ a_off, int64_t *__restrict__ b_off, int a_bpr, int b_bpr, int policy,
    uint64_t seed) {
    __shared__ int64_t red64[4];
    __shared__ int red32[2][4];
    __shared__ int s_ge[256], s_gt[256], s_rank[256];
    __shared__ double redd[4];
    __shared__ int64_t scan_buf[256];

    const int pool = pool_lo + blockIdx.x;
    const int b_lo = pool_ptr[pool], b_hi = pool_ptr[pool + 1];
    const int n = b_hi - b_lo;
    const int tid = threadIdx.x;
    const int per = (n + 255) / 256;
    const int my_lo = b_lo + tid * per;
    const int my_hi = min(b_hi, my_lo + per);
    const int64_t cap = static_cast<int64_t>(n) * k;
    const int64_t R = budget[pool] < cap ? budget[pool] : cap;

    const bool rnd = policy == kAllocRandom;
    // keys of block b that are >= c
    auto count = [&](int b, uint32_t c) {
        return rnd ? count_ge_random(seed, pool, b - b_lo, k, c)
                   : count_ge(sigma + static_cast<int64_t>(b - blk_lo) * pitch, k, c);
    };

    // 1. tau = key of the R-th largest value (only needed when 0 < R < cap).
    uint32_t tau = 0;
    const bool partial = R > 0 && R < cap && policy != kAllocUniform;
    // small pools: keys in registers, per-block counts and the objective spread
    // over all threads (a thread owns at most one block then)
    const bool cached = cap <= 256 * kKeysPerThread && n <= 256;
    if (partial && cached) {
        // keys in registers: thread t holds keys t, t + 256, ... of the pool in
        // (block, index) order; padding keys are 0, which no candidate (>= 1)
        // counts, exactly as a zero sigma
        uint32_t keys[kKeysPerThread];
#pragma unroll
        for (int q = 0; q < kKeysPerThread; ++q) {
            const int idx = tid + 256 * q;
            uint32_t key = 0;
            if (idx < cap) {
                const int j = idx / k, i = idx - j * k;
                key = rnd ? random_key(seed, pool, j, i)
                          : key_bits(sigma[static_cast<int64_t>(b_lo + j - blk_lo) * pitch + i]);
            }
            keys[q] = key;
        }
        const int lane = tid & 63, wave = tid >> 6;
        for (int bit = rnd ? 31 : 30, round = 0; bit >= 0; --bit, ++round) {  // sigma keys have a clear sign bit
            const uint32_t cand = tau | (1u << bit);
            int cnt = 0;
#pragma unroll
            for (int q = 0; q < kKeysPerThread; ++q) cnt += keys[q] >= cand ? 1 : 0;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) cnt += __shfl_xor(cnt, o, 64);
            // two buffers: a wave writes round r + 1's counts only after every wave
            // has passed round r's barrier, that is after all reads of round r - 1
            if (lane == 0) red32[round & 1][wave] = cnt;
            __syncthreads();
            const int64_t tot = static_cast<int64_t>(red32[round & 1][0]) + red32[round & 1][1] +
                                red32[round & 1][2] + red32[round & 1][3];
            if (tot >= R) tau = cand;  // uniform decision
        }
        // per block: keys >= tau and keys > tau
        for (int j = tid; j < n; j += 256) s_ge[j] = s_gt[j] = 0;
        __syncthreads();
#pragma unroll
        for (int q = 0; q < kKeysPerThread; ++q) {
            const int idx = tid + 256 * q;
            if (idx < cap) {
                const int j = idx / k;
                if (keys[q] >= tau) atomicAdd(&s_ge[j], 1);
                if (keys[q] > tau) atomicAdd(&s_gt[j], 1);
            }
        }
        __syncthreads();
    } else if (partial) {
        for (int bit = rnd ? 31 : 30; bit >= 0; --bit) {  // sigma keys have a clear sign bit
            const uint32_t cand = tau | (1u << bit);
            int64_t cnt = 0;
            for (int b = my_lo; b < my_hi; ++b) cnt += count(b, cand);
            cnt = block_sum<int64_t>(cnt, red64);
            if (cnt >= R) tau = cand;  // uniform decision
        }
    }

    // 2. ranks: strictly greater values, then ties in block order.
    auto ge_gt = [&](int b, int &ge, int &gt) {
        if (cached) {
            ge = s_ge[b - b_lo];
            gt = s_gt[b - b_lo];
        } else {
            ge = count(b, tau);
            gt = tau == 0xffffffffu ? 0 : count(b, tau + 1);
        }
    };
    int64_t gt_sum = 0, eq_sum = 0;
    for (int b = my_lo; b < my_hi; ++b) {
        if (partial) {
            int ge, gt;
            ge_gt(b, ge, gt);
            gt_sum += gt;
            eq_sum += ge - gt;
        }
    }
    int64_t need = 0, eq_before = 0;
    if (partial) {
        const int64_t gt_tot = block_sum<int64_t>(gt_sum, red64);
        need = R - gt_tot;
        eq_before = block_exclusive_scan(eq_sum, scan_buf);
    }
    int64_t rank_sum = 0;
    double obj = 0.0;
    for (int b = my_lo; b < my_hi; ++b) {
        const float *row = sigma + static_cast<int64_t>(b - blk_lo) * pitch;
        int r;
        if (policy == kAllocUniform) {
            const int j = b - b_lo;
            r = static_cast<int>(R / n + (j < R % n ? 1 : 0));
        } else if (!partial) {
            r = R == 0 ? 0 : k;
        } else {
            int ge, gt;
            ge_gt(b, ge, gt);
            int64_t extra = need - eq_before;
            extra = extra < 0 ? 0 : (extra > ge - gt ? ge - gt : extra);
            eq_before += ge - gt;
            r = gt + static_cast<int>(extra);
        }
        rank[b] = r;
        rank_sum += r;
        if (cached) {
            s_rank[b - b_lo] = r;
        } else {
            for (int i = 0; i < r; ++i) {
                const double s = static_cast<double>(row[i]);
                obj += log1p(s * s / eps2);
            }
        }
    }
    if (cached) {
        __syncthreads();
        for (int q = 0; q < kKeysPerThread; ++q) {
            const int idx = tid + 256 * q;
            if (idx < cap) {
                const int j = idx / k, i = idx - j * k;
                if (i < s_rank[j]) {
                    const double s = static_cast<double>(sigma[static_cast<int64_t>(b_lo + j - blk_lo) * pitch + i]);
                    obj += log1p(s * s / eps2);
                }
            }
        }
    }
    // Objective (reduction order is fixed by the thread layout: deterministic).
    {
        const int lane = tid & 63, wave = tid >> 6;
        double v = obj;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) v += __shfl_xor(v, o, 64);
        __syncthreads();
        if (lane == 0) redd[wave] = v;
        __syncthreads();
        if (tid == 0 && objective) objective[pool] = ((redd[0] + redd[1]) + redd[2]) + redd[3];
    }
    // Arena offsets: the pool's blocks are laid out back to back in block order,
    // each as A^T (r x T) followed by B (r x d); a rank takes a_bpr bytes of A
    // and b_bpr bytes of B.
    if (a_off) {
        const int64_t before = block_exclusive_scan(rank_sum, scan_buf);
        int64_t off = pool_base[pool] + before * (a_bpr + b_bpr);
        for (int b = my_lo; b < my_hi; ++b) {
            const int r = rank[b];
            a_off[b] = off;
            b_off[b] = off + static_cast<int64_t>(r) * a_bpr;
            off += static_cast<int64_t>(r) * (a_bpr + b_bpr);
        }
    }
}

}  // namespace

hipError_t launch_alloc(const float *sigma, int sigma_pitch, int max_rank, const int32_t *pool_ptr,
                        const int64_t *budget, const int64_t *pool_base, int pool_lo, int n_pools,
                        int blk_lo, double eps2, int32_t *rank, double *objective, int64_t *a_off,
                        int64_t *b_off, int a_bpr, int b_bpr, int policy, uint64_t seed,
                        hipStream_t st) {
    if (n_pools <= 0) return hipSuccess;
    hipLaunchKernelGGL(alloc_kernel, dim3(static_cast<unsigned>(n_pools)), dim3(256), 0, st, sigma,
                       sigma_pitch, max_rank, pool_ptr, budget, pool_base, pool_lo, blk_lo, eps2,
                       rank, objective, a_off, b_off, a_bpr, b_bpr, policy, seed);
    return hipGetLastError();
}

}  // namespace milo
