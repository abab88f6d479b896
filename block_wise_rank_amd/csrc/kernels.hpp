// Host-side launchers of the libmilo kernels (one translation unit per kernel
// family; each launcher lives next to its kernel).  All launches are
// asynchronous on the given stream.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace milo {

enum ElemType : int { kF32 = 0, kBF16 = 1, kI8 = 2, kI4 = 3, kI2 = 4 };
// 4-bit factors: symmetric codes in [-7, 7], two per byte (element 2k in the low
// nibble), one fp32 scale per kI4Group consecutive elements of a row.
// 2-bit factors: codes c in 0..3 for the levels (2c - 3) s, four per byte
// (element 4k + j in bits 2j, 2j + 1 of byte k), one fp32 scale s per kI4Group
// consecutive elements of a row.
constexpr int kI4Group = 32;
// Rank allocation policies (values of milo_alloc_policy).
enum AllocPolicy : int { kAllocEntropy = 0, kAllocUniform = 1, kAllocRandom = 2 };

// G_b = X_b^T X_b, written as `splits` partial sums per block:
// gpart[(b * splits + s) * 128 * 128 + i * 128 + j].
hipError_t launch_gram(const void *x, int x_type, const int64_t *row0, int64_t row_stride,
                       int block_len, int n_blocks, int splits, float *gpart, hipStream_t st);

// Eigenvectors of the 128 x 128 Grams in three launches.
//  * launch_tridiag reduces each Gram (the sum of its `splits` partials in
//    gpart) to tridiagonal form by Householder reflections, keeping the
//    reflectors in the block's first partial and the tridiagonal matrix in
//    vt[b].
//  * launch_qr_chain runs the implicit shifted QR steps on the tridiagonal
//    matrices, one per lane (64, 48 or 36 per wave: the fewest rounds of
//    resident waves on the n_cus CUs, then the fewest per wave), and records each block's plane rotations in its
//    stream area: up to kRotCap rotations (c, s) after kRotPad unused slots,
//    kRotPad more unused slots, then up to kStepCap step headers (first row |
//    last row << 16); counts[b] = (steps, rotations).
//    rotations[b] (may be null) = the rotations, negated when a cap stopped
//    the iteration.
//  * launch_qr_apply forms the rows of Q from the reflectors, applies the
//    recorded rotations to them and writes the eigenvectors as the rows of
//    vt[b] (in no particular order, unit length to working accuracy).
constexpr int kRotCap = 20480;  // rotations per block (about 11.5 k are taken on planted Grams)
constexpr int kStepCap = 512;   // QR steps per block (about 170 are taken)
constexpr int kRotPad = 128;     // rotation slots before and after a block's rotations
constexpr size_t kStreamBytes = sizeof(float) * 2 * (kRotCap + 2 * kRotPad) + sizeof(uint32_t) * kStepCap;
hipError_t launch_tridiag(float *gpart, int splits, int n_blocks, float *vt, hipStream_t st);
hipError_t launch_qr_chain(const float *vt, int n_blocks, void *stream, int32_t *counts, int32_t *rotations,
                           int n_cus, hipStream_t st);
hipError_t launch_qr_apply(const float *gpart, int splits, int n_blocks, const void *stream, const int32_t *counts,
                           float *vt, hipStream_t st);

// The eigensolve of launches with few blocks (at most eight per CU), where each
// block's latency counts: parallel-order cyclic Jacobi on G_b (the sum of the
// partials) in LDS, 64 disjoint rotations per round.  Pairs with
// |g| <= tol sqrt|a b| are not rotated; the solve ends after the first half
// sweep that closes 127 rounds with no rotation above stop_tol.  vt[b][i][:] =
// eigenvector i (unsorted); sweeps[b] (may be null) = 64 x the rounds used
// (64 rotations a round), negative when max_sweeps sweeps were reached.
hipError_t launch_jacobi(const float *gpart, int splits, int n_blocks, float *vt,
                         int32_t *sweeps, int max_sweeps, float tol, float stop_tol, int n_cus,
                         hipStream_t st);

// sigma_i = ||X_b v_i|| in fp32-accurate arithmetic, sorted descending into
// sigma[b][0..128); perm[b][k] = the eigenvector (row of vt[b]) of sorted rank k
// and scale[b][k] = its sign (largest-magnitude entry made positive) / ||v||:
// sorted row k of V^T is scale[b][k] * vt[b][perm[b][k]][:].
hipError_t launch_refine(const void *x, int x_type, const int64_t *row0, int64_t row_stride,
                         int block_len, int n_blocks, const float *vt, float *sigma, int32_t *perm,
                         float *scale, hipStream_t st);

// Rank allocation for pools [pool_lo, pool_lo + n_pools) of the device pool
// tables under `policy` (seed: the random policy's generator seed): ranks of
// blocks, per-pool objective (may be null), and when a_off is non-null the
// arena offsets (pool_base[p] + prefix of rank * (a_bpr + b_bpr): a rank's
// bytes in the A and in the B part of a block).
hipError_t launch_alloc(const float *sigma, int sigma_pitch, int max_rank,
                        const int32_t *pool_ptr, const int64_t *budget, const int64_t *pool_base,
                        int pool_lo, int n_pools, int blk_lo, double eps2, int32_t *rank,
                        double *objective, int64_t *a_off, int64_t *b_off, int a_bpr,
                        int b_bpr, int policy, uint64_t seed, hipStream_t st);

// Factor pairs from the eigenvectors (sorted rank k = scale[b][k] *
// vt[b][perm[b][k]], see launch_refine) and ranks: A_b^T (rank-major) and B_b
// rows into the arena, plus INT8 scales.
hipError_t launch_project(const void *x, int x_type, const int64_t *row0, int64_t row_stride,
                          int block_len, int n_blocks, const float *vt, const int32_t *perm,
                          const float *vscale, const int32_t *rank,
                          const int64_t *a_off, const int64_t *b_off, void *arena,
                          int out_type, float *a_scale, float *b_scale, hipStream_t st);

// X_hat = A B for the listed blocks; block i's rows start at element out_off[i]
// of out (out_off null: i * block_len * 128).
hipError_t launch_reconstruct(const void *arena, int f_type, const int32_t *rank,
                              const int64_t *a_off, const int64_t *b_off, const float *a_scale,
                              const float *b_scale, int block_len, const int32_t *ids, int n_ids,
                              void *out, const int64_t *out_off, int out_type, hipStream_t st);

struct DecodeParams {
    const void *q;
    int q_type;
    const int64_t *q_pos;
    int batch, n_q_heads, n_kv_heads, group;
    // factor sets (same storage type)
    int f_type;
    int block_len, blocks_per_seq;
    const int32_t *k_rank, *v_rank;
    const int64_t *k_aoff, *k_boff, *v_aoff, *v_boff;
    const uint8_t *k_arena, *v_arena;
    const float *k_ascale, *k_bscale, *v_ascale, *v_bscale;
    // selection
    const int32_t *sel_ptr, *sel_blk;
    int n_sel;  // splits-per-block slots reserved per sequence (sel_max or blocks_per_seq)
    // tail
    const void *tail_k, *tail_v;
    int tail_type, tail_cap;
    const int32_t *tail_len;
    const int64_t *tail_pos0;
    // segmented tail (tail_seg_pos non-null): [batch][tail_cap / tail_seg_len]
    // start positions and valid token counts of segments of tail_seg_len slots
    const int64_t *tail_seg_pos;
    const int32_t *tail_seg_valid;
    int tail_seg_len;
    double rope_base;
    float softmax_scale;
    void *out;
    int out_type;
    int split_len;
    int block_splits;  // block_len / split_len
    int tail_splits;   // tail_cap / split_len (0 without tail)
    int n_splits;      // n_sel * block_splits + tail_splits
    float *part_ml;    // [batch][Hkv][n_splits][group][2]  (m, l) in log2 units
    float *part_o;     // [batch][Hkv][n_splits][group][128]
    // RoPE tables, rebuilt by launch_decode_tables each call (workspace):
    double *theta;     // [64] base^(-2j/128)
    float2 *rope_tab;  // [32][64] (cos, sin)(t theta_j), t < 32
    float2 *step_tab;  // [kMaxTiles][64] (cos, sin)(32 tile theta_j)
};
constexpr int kMaxTiles = 64;  // 32-token tiles per split (split_len <= 2048)

// Whether a split of `split` tokens fits the decode kernels' LDS budget.
bool decode_split_fits(int f_type, int tail_type, bool has_tail, int G, int split);
// Workspace: the partials (m, l; then o), then the tables.
size_t decode_workspace_bytes(const DecodeParams &p);
size_t decode_table_bytes();
// The RoPE tables; one launch for the partial results of the compressed-block
// splits and of the tail splits; the log-sum-exp merge into the output.
hipError_t launch_decode_tables(const DecodeParams &p, hipStream_t st);
hipError_t launch_decode(const DecodeParams &p, hipStream_t st);
hipError_t launch_decode_combine(const DecodeParams &p, hipStream_t st);

}  // namespace milo
