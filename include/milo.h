/*
 * milo.h -- C ABI of libmilo: block-wise low-rank compression of a KV cache and
 * decode attention over the compressed blocks (the MILO method), for AMD
 * Instinct MI355X (gfx950).
 *
 * Method sources, cited by page and section:
 *   [REV] evolve.pub AI review of "MILO: Efficient Many-shot In-Context Learning
 *         with Block-wise Low-rank Compression" (arXiv 2609.29913): Summary,
 *         Strengths (rank allocation, Eqs 5-7), FAQ.
 *   [ABS] shd-paper.top digest of the paper: English abstract; method section
 *         ("technical framework": blocking, block-level low-rank compression,
 *         dynamic rank-budget allocation).
 *   [DIG] ai4snews digest: arXivInterpretation; Figure 1 caption (pre-RoPE keys).
 *
 * Conventions shared by every call
 *   - Tensor pointers are DEVICE pointers unless the comment says "host".
 *     Sizes are element counts unless they say "bytes".
 *   - The caller owns every buffer.  The library never allocates device memory,
 *     never frees, and never synchronises; it enqueues kernels on `stream` (a
 *     hipStream_t passed as void*, NULL = the default stream) and returns.
 *     Outputs are valid once the stream has reached that point; inputs must
 *     stay alive until then.  Small host arrays (pool tables) are copied to the
 *     device inside the call, so they may be freed when the call returns.
 *   - Every argument is validated on the host before anything is enqueued, so a
 *     call that returns an error has written nothing.  Errors are status codes;
 *     nothing is thrown across the ABI.  milo_last_error() gives a
 *     human-readable reason for the last failure on the calling thread.
 *   - head_dim must be 128 and block_len a multiple of 64 with block_len >= 128
 *     (MILO_E_UNSUPPORTED otherwise).
 *   - Calls on the same stream are ordered; calls on different streams that
 *     share an output or workspace buffer race.
 */
#ifndef MILO_H
#define MILO_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MILO_ABI_VERSION 4

typedef enum milo_status {
    MILO_OK = 0,
    MILO_E_INVALID = 1,     /* null pointer, negative or inconsistent size, bad CSR       */
    MILO_E_UNSUPPORTED = 2, /* head_dim != 128, block_len not a multiple of 64 or < 128, */
                            /* or an unsupported dtype combination                        */
    MILO_E_WORKSPACE = 3,   /* workspace missing or too small; *_bytes holds the need   */
    MILO_E_HIP = 4          /* a HIP runtime call or a kernel launch failed              */
} milo_status;

typedef enum milo_dtype {
    MILO_F32 = 0,
    MILO_BF16 = 1,
    MILO_I8 = 2, /* factor storage only: per-row absmax INT8 with fp32 scales */
    MILO_I4 = 3, /* factor storage only: 4-bit codes, an fp32 scale per 32 elements */
    MILO_I2 = 4  /* factor storage only: 2-bit codes, an fp32 scale per 32 elements */
} milo_dtype;

/*
 * A batch of KV blocks to compress (the cache cut into fixed-size blocks of
 * block_len tokens, each holding several in-context examples: [DIG]
 * arXivInterpretation; [ABS] abstract).  Block b is the block_len x head_dim
 * matrix X_b whose token row t starts at element row0[b] + t * row_stride of x.
 * K blocks must hold keys BEFORE rotary embedding ([REV] Summary; [DIG] Fig. 1).
 */
typedef struct milo_blocks {
    const void *x;         /* device, element type `dtype` (MILO_F32 or MILO_BF16)       */
    milo_dtype dtype;
    const int64_t *row0;   /* device [n_blocks] element offsets, or NULL meaning          */
                           /* row0[b] = b * block_len * row_stride (blocks back to back)  */
    int64_t row_stride;    /* elements between consecutive token rows, >= head_dim        */
    int32_t n_blocks;
    int32_t block_len;     /* T */
    int32_t head_dim;      /* d, must be 128 */
} milo_blocks;

/*
 * Compressed blocks: X_b ~= A_b B_b with A_b = X_b V_r (T x r_b) and
 * B_b = V_r^T (r_b x d), V_r the leading r_b right singular vectors of X_b
 * ([REV] Summary and FAQ: a per-block SVD, the cache kept per block in
 * low-rank form).  Layout in the arena, for block b:
 *   A_b is stored TRANSPOSED, rank-major: r_b rows of block_len elements,
 *       row i = column i of A_b, at byte offset a_off[b];
 *   B_b is stored as r_b rows of head_dim elements at byte offset b_off[b].
 * Element type `dtype`: MILO_F32, MILO_BF16, MILO_I8, MILO_I4 or MILO_I2 (codes).  For MILO_I8
 * every row of A_b (one per token) has a scale a_scale[b*block_len + t] and
 * every row of B_b (one per rank) a scale b_scale[b*head_dim + i]; the decoded
 * value is code * scale.
 * MILO_I4 (block_len a multiple of 128; the composition with low-bit KV
 * quantisation of [REV] Key claims and FAQ, with this library's own group-wise
 * quantiser): each row is cut into runs of 32 consecutive elements, each with
 * an fp32 scale s = max|run| / 7 and codes rint(x / s) in [-7, 7] (decided in
 * fp32), decoded value code * s.  Codes are two's-complement nibbles, two per
 * byte, element 2k in the low nibble.  A_b's part at a_off[b]: the r_b code rows
 * (block_len / 2 bytes each), then the r_b x (block_len / 32) scales.  B_b's
 * part at b_off[b]: the r_b code rows (head_dim / 2 bytes each), then the
 * r_b x (head_dim / 32) scales.  a_scale / b_scale are not used (NULL).  A_b
 * is computed from the fp32-accurate B_b before either is quantised.
 * MILO_I2 (block_len a multiple of 128; the lowest width of that composition):
 * the same runs of 32 elements, each with an fp32 scale s = max|run| / 3 and
 * a code c in 0..3 per element standing for (2c - 3) s, the level nearest to
 * x: with q = x / s in fp32, |q| >= 2 takes the outer level of x's sign,
 * |q| < 2 the inner one (x = 0 takes +s; a run with s = 0 has codes 2).  Four
 * codes per byte, element 4k + j in bits 2j, 2j + 1 of byte k.  A_b's part:
 * the r_b code rows (block_len / 4 bytes each), then the r_b x (block_len / 32)
 * scales; B_b's part: the r_b code rows (head_dim / 4 bytes each), then the
 * r_b x (head_dim / 32) scales.
 * milo_compress_blocks writes rank, a_off, b_off, the arena and the scales;
 * the caller sizes the arena with milo_arena_bytes().
 */
typedef struct milo_factors {
    milo_dtype dtype;
    int32_t n_blocks;
    int32_t block_len;
    int32_t head_dim;
    int32_t *rank;         /* device [n_blocks]                                  */
    int64_t *a_off;        /* device [n_blocks], bytes from arena                */
    int64_t *b_off;        /* device [n_blocks], bytes from arena                */
    void *arena;           /* device, 256-byte aligned                           */
    size_t arena_bytes;
    float *a_scale;        /* device [n_blocks * block_len], MILO_I8 only, else NULL */
    float *b_scale;        /* device [n_blocks * head_dim],  MILO_I8 only, else NULL */
} milo_factors;

/*
 * milo_compress_blocks -- per-block SVD of every block, global rank allocation
 * per pool, and the factor pairs ([REV] Summary; [ABS] method section).
 *
 *  in          blocks to compress (K blocks pre-RoPE, or V blocks).
 *  pool_ptr    host [n_pools + 1], CSR over blocks: pool p is the run of blocks
 *              [pool_ptr[p], pool_ptr[p+1]); pool_ptr[0] = 0,
 *              pool_ptr[n_pools] = n_blocks, non-decreasing.
 *  budget      host [n_pools], the global rank budget R_p of each pool (>= 0).
 *  eps2        eps^2 of the gain log(1 + sigma^2/eps^2) ([REV] Summary and
 *              Strengths, Eqs 5-7); > 0.  The ranks do not depend on it, only
 *              the reported objective does.
 *  sigma_out   device [n_blocks][head_dim] fp32: singular values of each block,
 *              descending.
 *  objective_out device [n_pools] fp64 (may be NULL): sum over the pool of the
 *              gains of the ranks handed out.
 *  out         factor set: dtype, n_blocks, block_len, head_dim must match `in`;
 *              rank/a_off/b_off/arena (and scales for MILO_I8) must be set.
 *              Within each pool exactly min(R_p, n_p * min(T, d)) ranks are
 *              handed out: the R_p largest singular values of the pool in the
 *              order (sigma desc, block asc, index asc), which is what the
 *              greedy on the gains selects.
 *  sweeps_out  device [n_blocks] int32 (may be NULL): the work of each block's
 *              eigensolve, as the number of plane rotations it applied.  Calls
 *              of more than eight blocks per compute unit reduce each Gram to
 *              tridiagonal form and run implicit shifted QR steps (0 rotations
 *              for a block that is diagonal once reduced; capped at 512 steps
 *              and 20480 rotations per block); smaller calls run a parallel
 *              Jacobi eigensolve (64 rotations per round, capped at 30 sweeps of
 *              127 rounds).  Negated if a cap stopped the iteration (the
 *              results are then those of its last step).  (ABI version 4;
 *              versions 2 and 3 counted Jacobi sweeps and rounds.)  The
 *              call returns before its kernels run, so it cannot report this in
 *              its status: a caller that must know passes sweeps_out and checks
 *              it once the stream has reached the call.
 *  workspace   device scratch; *workspace_bytes its size.  With workspace ==
 *              NULL or a size below what one pool needs, returns
 *              MILO_E_WORKSPACE and sets *workspace_bytes to the size that
 *              processes every block in one pass.  Any size >= the largest
 *              pool's need works: pools are then processed in chunks.
 * Supported dtype pairs (in -> factors): F32 or BF16 -> any of F32, BF16, I8, I4, I2.
 */
milo_status milo_compress_blocks(const milo_blocks *in, const int32_t *pool_ptr, int32_t n_pools,
                                 const int64_t *budget, double eps2, float *sigma_out,
                                 double *objective_out, milo_factors *out, int32_t *sweeps_out,
                                 void *workspace, size_t *workspace_bytes, void *stream);

/*
 * Rank allocation policies.  MILO_ALLOC_ENTROPY is the method's allocation (the
 * greedy on the gains, above).  The other two are the equal-budget allocations
 * the method is compared with ([REV] Strengths, on Fig. 5(d)); both hand out
 * exactly R' = min(R_p, n_p * k) ranks per pool, k = min(block_len, head_dim):
 *  MILO_ALLOC_UNIFORM  block j of the pool (j = 0 .. n_p - 1) gets
 *                      floor(R'/n_p) ranks, one more when j < R' mod n_p;
 *  MILO_ALLOC_RANDOM   the R' (block, index) slots with the largest keys, key of
 *                      slot (j, i) of pool p = the high 32 bits of output number
 *                      1 + (p << 32 | j << 8 | i) of SplitMix64 seeded with
 *                      `seed` (Steele, Lea & Flood 2014; Stafford's finaliser
 *                      13), equal keys to the smaller block, then the smaller
 *                      index: a uniformly random R'-subset of the pool's slots;
 *                      block j's rank is the number of its slots taken.
 * Every policy takes each block's leading singular vectors and reports the same
 * objective: the sum of log(1 + sigma^2/eps^2) over the ranks handed out.
 */
typedef enum { MILO_ALLOC_ENTROPY = 0, MILO_ALLOC_UNIFORM = 1, MILO_ALLOC_RANDOM = 2 } milo_alloc_policy;
typedef struct {
    milo_alloc_policy policy;
    uint64_t seed;  /* MILO_ALLOC_RANDOM only */
} milo_alloc_options;

/*
 * milo_compress_blocks_ex -- milo_compress_blocks with the allocation policy
 * chosen by `alloc` (NULL: MILO_ALLOC_ENTROPY, identical to
 * milo_compress_blocks).  Returns MILO_E_INVALID for an unknown policy.
 */
milo_status milo_compress_blocks_ex(const milo_blocks *in, const int32_t *pool_ptr, int32_t n_pools,
                                    const int64_t *budget, double eps2, float *sigma_out,
                                    double *objective_out, milo_factors *out, int32_t *sweeps_out,
                                    const milo_alloc_options *alloc, void *workspace,
                                    size_t *workspace_bytes, void *stream);

/*
 * milo_allocate_ranks -- the rank allocation alone ([REV] Strengths, Eqs 5-7),
 * on caller-supplied singular values.
 *  sigma       device [n_blocks][head_dim] fp32, every row non-increasing and
 *              >= 0 (results are unspecified otherwise).
 *  max_rank    k = ranks a block can hold (1..head_dim); only sigma[b][0..k) count.
 *  pool_ptr, budget, eps2  as for milo_compress_blocks (host arrays).
 *  rank_out    device [n_blocks] int32.
 *  objective_out device [n_pools] fp64 or NULL.
 *  workspace   device scratch for the pool tables; with NULL or too small a
 *              size returns MILO_E_WORKSPACE and sets *workspace_bytes.
 */
milo_status milo_allocate_ranks(const float *sigma, int32_t n_blocks, int32_t head_dim,
                                int32_t max_rank, const int32_t *pool_ptr, int32_t n_pools,
                                const int64_t *budget, double eps2, int32_t *rank_out,
                                double *objective_out, void *workspace, size_t *workspace_bytes,
                                void *stream);

/* milo_allocate_ranks under the policy chosen by `alloc` (NULL: entropy).  The
 * uniform and random policies do not read sigma for the ranks, only for the
 * objective; k = max_rank. */
milo_status milo_allocate_ranks_ex(const float *sigma, int32_t n_blocks, int32_t head_dim,
                                   int32_t max_rank, const int32_t *pool_ptr, int32_t n_pools,
                                   const int64_t *budget, double eps2, int32_t *rank_out,
                                   double *objective_out, const milo_alloc_options *alloc,
                                   void *workspace, size_t *workspace_bytes, void *stream);

/*
 * milo_reconstruct -- rebuild X_hat_b = A_b B_b (decoded) for the listed blocks
 * only ([REV] FAQ: only the blocks a query needs are rebuilt).
 *  block_ids   device [n_ids], each in [0, f->n_blocks).
 *  x_out       device [n_ids][block_len][head_dim], MILO_F32 or MILO_BF16.
 */
milo_status milo_reconstruct(const milo_factors *f, const int32_t *block_ids, int32_t n_ids,
                             void *x_out, milo_dtype out_dtype, void *stream);

/*
 * milo_reconstruct_ex -- milo_reconstruct writing block i's block_len rows at
 * element offset out_off[i] of x_out instead of i * block_len * head_dim, so
 * that rebuilt blocks land where a staging cache keeps them (for example per
 * sequence and KV head, next to an uncompressed tail).
 *  out_off  device [n_ids] int64, or NULL (= milo_reconstruct).  Each offset
 *           must be a multiple of 8 (16-byte aligned rows); the regions of
 *           different ids must not overlap.  Device values are not validated.
 */
milo_status milo_reconstruct_ex(const milo_factors *f, const int32_t *block_ids, int32_t n_ids,
                                void *x_out, const int64_t *out_off, milo_dtype out_dtype, void *stream);

/*
 * milo_fetch_blocks -- host-offloaded compressed cache: bring the factors of
 * the listed blocks from a factor set kept in host memory into a device factor
 * set of the same layout ([REV] Summary and FAQ: the compressed cache is
 * offloaded to CPU memory, on one L4 GPU, and only the blocks a query needs are
 * brought back and rebuilt; the throughput figures are measured against
 * offloading the full cache).
 *  host    factor set whose arena (and, for MILO_I8, a_scale / b_scale) is in
 *          pinned host memory (hipHostMalloc; pageable memory works, but the
 *          copies then do not overlap other work), and whose rank / a_off /
 *          b_off are HOST arrays.  Only read.
 *  dev     factor set with the same dtype, n_blocks, block_len and head_dim and
 *          arena_bytes >= host's; its arena (and scales) are device memory.
 *          Its metadata arrays are not touched and must hold host's values: the
 *          layout is shared, so a fetched block sits at the same arena offsets
 *          (and scale rows) in both sets, and decode over dev reads exactly the
 *          fetched blocks.
 *  blocks  host [n]: block ids, each in [0, n_blocks); any order, repeats
 *          allowed.  Ranges that continue the previous block's in the list are
 *          fetched with one copy (a whole pool in id order is one copy).
 *  stream  the copies are asynchronous DMA on this stream; the host arrays are
 *          read during the call only.
 * Errors (nothing copied): MILO_E_INVALID for missing pointers, mismatched
 * geometry, ids out of range or offsets reaching past arena_bytes.
 */
milo_status milo_fetch_blocks(const milo_factors *host, const milo_factors *dev, const int32_t *blocks,
                              int32_t n, void *stream);

/*
 * Decode attention over compressed blocks for one layer ([REV] Summary: the
 * retrieved blocks' low-rank factors are rebuilt before sparse attention).
 * Sequence s, query head hq uses KV head h = hq / (n_q_heads / n_kv_heads).
 * Factor block id of block b of sequence s and KV head h:
 *      (s * n_kv_heads + h) * blocks_per_seq + b.
 * Token t of block b is at absolute position b * block_len + t; tail token i of
 * sequence s at tail_pos0[s] + i.  RoPE (half-split pairs, angle
 * pos * rope_base^(-2j/d)) is applied to the query at q_pos[s] and to every
 * rebuilt key at its position; logits are scaled by softmax_scale.
 */
typedef struct milo_decode_args {
    const void *q;            /* device [batch][n_q_heads][head_dim], pre-RoPE, 16-byte */
                              /* aligned (the factor arenas must be 16-byte aligned too) */
    milo_dtype q_dtype;       /* MILO_F32 or MILO_BF16                                  */
    const int64_t *q_pos;     /* device [batch]                                         */
    int32_t batch;
    int32_t n_q_heads;        /* multiple of n_kv_heads; at most 16 per KV head        */
    int32_t n_kv_heads;
    int32_t head_dim;         /* 128                                                    */
    const milo_factors *k;    /* host struct describing the K factor set               */
    const milo_factors *v;    /* host struct describing the V factor set (same blocks) */
    int32_t blocks_per_seq;
    const int32_t *sel_ptr;   /* device CSR [batch + 1] over sel_blk, or NULL = every   */
    const int32_t *sel_blk;   /* block; entries of a sequence ascending and distinct,   */
    int32_t sel_max;          /* in [0, blocks_per_seq).  sel_max (host) bounds the     */
                              /* entries per sequence; ignored when sel_ptr is NULL.    */
    const void *tail_k;       /* device [batch][n_kv_heads][tail_cap][head_dim], keys   */
    const void *tail_v;       /* pre-RoPE, or NULL for no uncompressed tail             */
    milo_dtype tail_dtype;    /* MILO_F32 or MILO_BF16                                  */
    int32_t tail_cap;         /* multiple of 64 when tail_k != NULL                     */
    const int32_t *tail_len;  /* device [batch], 0..tail_cap                            */
    const int64_t *tail_pos0; /* device [batch]                                         */
    double rope_base;         /* > 1, e.g. 1e6                                           */
    float softmax_scale;      /* e.g. 1/sqrt(head_dim)                                   */
    void *out;                /* device [batch][n_q_heads][head_dim]                    */
    milo_dtype out_dtype;     /* MILO_F32 or MILO_BF16                                  */
    int32_t split_len;        /* tokens per work split: multiple of 128, at most 2048,   */
                              /* dividing block_len, whose workgroup fits the LDS for   */
                              /* the call's query heads per KV head; 0 picks the        */
                              /* longest such split that still gives >= 256             */
                              /* workgroups, the tail's included (else 128)             */
    void *workspace;          /* device scratch: per-split partial results and the     */
                              /* RoPE tables of the call (256-byte aligned)             */
    size_t workspace_bytes;
    /* Segmented uncompressed part (ABI version 2), for caches that hold blocks
     * rebuilt at their own positions next to the recent tail ([REV] FAQ: only
     * the blocks a query needs are rebuilt, then attended sparsely).  With
     * tail_seg_pos non-NULL, sequence s's tail_cap slots are tail_cap /
     * tail_seg_len segments of tail_seg_len slots; segment m holds its first
     * tail_seg_valid[s][m] tokens (0..tail_seg_len), token i of it at position
     * tail_seg_pos[s][m] + i; tail_len and tail_pos0 are then not read (may be
     * NULL).  tail_seg_len is a multiple of 128 dividing tail_cap, and the
     * split must divide it (the default split does).                        */
    const int64_t *tail_seg_pos;   /* device [batch][tail_cap / tail_seg_len] or NULL */
    const int32_t *tail_seg_valid; /* device [batch][tail_cap / tail_seg_len]        */
    int32_t tail_seg_len;
} milo_decode_args;

/*
 * milo_decode_attention -- one decode step of one layer.  With
 * a->workspace == NULL or a->workspace_bytes too small it returns
 * MILO_E_WORKSPACE and stores the size needed in *workspace_needed (may be NULL).
 * K and V factor sets must use the same storage dtype (F32, BF16 or I8).
 */
milo_status milo_decode_attention(const milo_decode_args *a, size_t *workspace_needed,
                                  void *stream);

/*
 * milo_decode_attention_noalloc -- milo_decode_attention for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  Same arguments, kernels and results
 * as milo_decode_attention, except that a->workspace and a->workspace_bytes are
 * ignored: the scratch (split partials and RoPE tables) is a static device
 * array of MILO_NOALLOC_SCRATCH_BYTES per GPU, held by every GPU the library
 * runs on until the process ends.  The call allocates nothing (its first call
 * on a device looks up that device's array address, once).
 *  - A call that needs more scratch than that returns MILO_E_WORKSPACE and
 *    enqueues nothing; milo_last_error() gives the size it needs (the default
 *    split of every supported geometry with up to 16 x 2 KV heads x 64 blocks
 *    of 2048 tokens and 8 query heads per KV head needs about 8.5 MiB).
 *  - Every call on one GPU uses that GPU's one array: calls that overlap on a
 *    GPU (different streams, or other host threads) race and must not be
 *    issued; calls ordered on one stream are fine.  Nothing in the array needs
 *    to start at zero: each call writes every partial it reads.
 */
#define MILO_NOALLOC_SCRATCH_BYTES (32u << 20)
milo_status milo_decode_attention_noalloc(const milo_decode_args *a, void *stream);

/* Arena bytes for a factor set: sum over pools of min(R_p, n_p * min(T, d))
 * ranks, each costing (block_len + head_dim) elements of dtype.  Host only.
 * Returns 0 and sets the last error on invalid input. */
size_t milo_arena_bytes(milo_dtype dtype, int32_t block_len, int32_t head_dim,
                        const int32_t *pool_ptr, int32_t n_pools, const int64_t *budget);

/* Workspace bytes milo_compress_blocks needs to process `n_blocks` blocks of
 * the given geometry in one pass (host only). */
size_t milo_compress_workspace_bytes(int32_t n_blocks, int32_t block_len, int32_t head_dim);

/*
 * Measurement aid (not part of the method): while enabled, every kernel that
 * the calling thread's libmilo calls launch is bracketed by a pair of HIP
 * events recorded on the call's stream.  milo_profile_read waits for the
 * recorded kernels, fills up to `cap` entries (kernel name -- a static string
 * --, launch count, total milliseconds; any output pointer may be NULL),
 * clears the record and returns the number of distinct kernels, or -1 if an
 * event failed.  State is per thread; events are created on first use and
 * reused.  milo_profile_enable returns the previous setting.
 */
int milo_profile_enable(int on);
int milo_profile_read(const char **names, int32_t *launches, double *total_ms, int cap);

const char *milo_status_string(milo_status s);
const char *milo_last_error(void);
int milo_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MILO_H */
