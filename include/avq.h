/*
 * avq.h -- C interface of libavq, the AVQ-Attention forward pass on AMD
 * Instinct MI355X (gfx950).
 *
 * Method: "AVQ-Attention: Adaptive Vector-Quantized Attention" (arXiv
 * 2607.12789v1).  The forward pass is two calls:
 *
 *   avq_assign_aggregate   the VQ precompute of Sec. 4.2 / Algorithm 1:
 *                          two-level assignment of every key and the per-
 *                          codeword value sums and key counts of Eq. 3.
 *   avq_attention_fwd      the attention of Sec. 4.3 / Algorithm 2: count-
 *                          weighted attention over the parents (Eq. 6), the
 *                          per-query-tile importance (Eq. 7), top-P parent
 *                          selection, and the child correction (Eq. 8, Eq. 9).
 *
 * Conventions shared by both calls
 * --------------------------------
 * Pointers are device pointers (memory from hipMalloc or any allocator that
 * returns device memory), owned by the caller.  The library allocates no
 * device or host memory, keeps no results between calls and is safe to call
 * from several host threads (calls sharing a workspace must not overlap).  Calls are asynchronous on `stream` (a
 * hipStream_t; NULL is the default stream).
 *
 * Shapes (all row-major and contiguous):
 *   bh = b*H + h indexes (batch, head); BH = B*H.
 *   Mt = M0 * (1 + C) codewords per head: rows 0..M0-1 are the parents; the C
 *   children of parent m are rows M0 + m*C ... M0 + m*C + C - 1 (Alg. 1 input
 *   layout).  The codebook is per head and shared across the batch.
 *   Each parent must equal the mean of its C children (Sec. 4.1, Eq. 5).  If
 *   it does not, avq_attention_fwd still returns Algorithm 2's value, but that
 *   value no longer equals attention over the refined codebook.
 *
 * dtype: AVQ_F32 (float) or AVQ_BF16 (bfloat16) for Q, K, V and the codebook.
 * Value sums, counts and outputs are float / int32 in both cases.
 *
 * Supported sizes: d in {64, 128}; 1 <= M0 <= 512; 0 <= C <= 16.  C = 0 is a
 * flat codebook of M0 codewords (plain VQ attention, the pages' fused flat-VQ
 * baseline of Sec. 5): keys are assigned to the nearest codeword only, and
 * the attention call then requires P = 0.
 * B, H, N >= 0 (any of them zero makes the call a no-op, except that
 * avq_assign_aggregate still zeroes vsum and counts when B*H > 0).
 * Every pointer argument must be 16-byte aligned.
 *
 * Errors: every call returns AVQ_OK (0) or a negative status.  Arguments are
 * validated on the host before anything is launched; on a validation error
 * nothing is written.  A launch failure returns AVQ_ERR_HIP; faults that occur
 * while a kernel runs surface at the caller's next synchronisation.
 */
#ifndef AVQ_H
#define AVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define AVQ_OK 0
#define AVQ_ERR_NULL (-1)        /* a required pointer is NULL */
#define AVQ_ERR_SHAPE (-2)       /* a size is out of range */
#define AVQ_ERR_DTYPE (-3)       /* unknown dtype */
#define AVQ_ERR_ALIGN (-4)       /* a pointer is not 16-byte aligned */
#define AVQ_ERR_UNSUPPORTED (-5) /* valid but unsupported (d, M0, C, block_q) */
#define AVQ_ERR_HIP (-6)         /* the HIP runtime reported an error */
#define AVQ_ERR_WORKSPACE (-7)   /* workspace missing or too small */
#define AVQ_ERR_SCRATCH (-8)     /* more than avq_attention_fwd_noalloc's static scratch */

/* Size of the static device scratch behind avq_attention_fwd_noalloc (per GPU). */
#define AVQ_NOALLOC_SCRATCH_BYTES (8u << 20)

#define AVQ_F32 0
#define AVQ_BF16 1

/*
 * Two-level VQ assignment and aggregation (Sec. 4.2, Algorithm 1; Eq. 2, 3).
 *
 * For every key of every (batch, head): the nearest parent by squared
 * Euclidean distance (lowest index on equal distances), then the C children
 * of that parent in order, keeping a child only if strictly closer than the
 * best child so far; the key moves to that child only if it is strictly
 * closer than the parent.  Every key adds its value and a count of one to
 * its parent row (a parent row holds its whole cluster); a key that moved also
 * adds them to its child row.
 *
 *   K, V      in  [BH, N, d]  dtype
 *   codebook  in  [H, Mt, d]  dtype
 *   vsum      out [BH, Mt, d] float   value sums (zeroed by the call first)
 *   counts    out [BH, Mt]    int32   key counts (zeroed by the call first)
 *   assign    out [BH, N]     int32   final row of every key (its child row
 *                                     if it moved, else its parent row), or
 *                                     NULL to skip
 *
 * Value sums are accumulated with floating-point atomics, so their rounding
 * depends on the order keys are added in; counts and assignments are exact.
 */
int avq_assign_aggregate(const void* K, const void* V, const void* codebook,
                         int B, int H, int N, int d, int M0, int C, int dtype,
                         float* vsum, int32_t* counts, int32_t* assign,
                         void* stream);

/*
 * avq_assign_aggregate that also sums the keys per codeword, for the codebook
 * update of the training recipe (App. A, Eq. 11): in the same pass,
 *   ksum  out [B*H, Mt, d] float: sum of the keys of every codeword over the
 *         same sets as vsum (parents their whole cell, children the keys that
 *         moved to them),
 * exactly what avq_assign_aggregate(K, K, ...) would write to its vsum, but
 * without a second assignment pass and second read of the keys from HBM.
 * ksum must not be NULL (AVQ_ERR_NULL) and must be 16-byte aligned; every
 * other argument, output and error is that of avq_assign_aggregate.
 */
int avq_assign_aggregate_kv(const void* K, const void* V, const void* codebook, int B, int H,
                            int N, int d, int M0, int C, int dtype, float* vsum,
                            int32_t* counts, int32_t* assign, float* ksum, void* stream);

/*
 * avq_assign_aggregate without the zero fill: this batch's value sums and
 * counts (Eq. 3) are added to what vsum and counts already hold, so several
 * batches of keys, or the keys of one sequence given in parts, accumulate
 * into one set of aggregates (the sums of Eq. 3 over the union of the
 * batches).  Every argument, layout and error is that of
 * avq_assign_aggregate; the caller zero-fills vsum and counts before the
 * first batch (avq_attention_fwd_prepared can do it as it consumes them).
 */
int avq_assign_aggregate_accum(const void* K, const void* V, const void* codebook, int B,
                               int H, int N, int d, int M0, int C, int dtype, float* vsum,
                               int32_t* counts, int32_t* assign, void* stream);

/*
 * Bytes of device workspace avq_attention_fwd needs for these sizes (0 if the
 * sizes are invalid).  The workspace holds the value sums of every codeword
 * converted to the operand format of the weighted-value products and a copy
 * of the counts; it is written and read by one call of avq_attention_fwd and
 * carries nothing between such calls.  avq_attention_prepare and avq_attention_fwd_prepared
 * split that call in two around the same workspace.
 */
size_t avq_attention_workspace_size(int B, int H, int d, int M0, int C,
                                    int dtype);

/*
 * AVQ attention forward (Sec. 4.3, Algorithm 2; Eq. 6-9, Sec. C and D).
 *
 * Queries are processed in tiles of block_q consecutive tokens (the last tile
 * may be partial); the tile is the unit of parent selection.  For each tile:
 *   s_ij = scale * Q_i . C_j for the parents j; m_i = max over parents with
 *   n_j > 0 (Eq. 18); A_ij = exp(s_ij - m_i), zero where n_j = 0;
 *   X_i = sum_j A_ij Vsum_j, Z_i = sum_j A_ij n_j (Eq. 6);
 *   w_j = sum_{i in tile} A_ij n_j / Z_i (Eq. 7);
 *   the P parents of largest w (ties to the lower index) are refined: for
 *   their children c, s_ic = scale * Q_i . C_c,
 *   s_ip = mean over the C children of s_ic (Eq. 8, needs Eq. 5),
 *   dA_ic = exp(s_ic - m_i) - exp(s_ip - m_i), zero where n_c = 0 (Eq. 9,
 *   Sec. D), X_i += sum_c dA_ic Vsum_c, Z_i += sum_c dA_ic n_c;
 *   Y_i = X_i / Z_i.
 * The stabiliser m_i is raised (and the accumulators rescaled) only when a
 * larger logit exceeds it by a factor 2^8; the result does not depend on it.
 * When M0 > 64 the parents are processed in tiles of 64 and the exact
 * denominator Z_i is completed in a first pass before the importances are
 * formed in a second pass.
 *
 *   Q          in  [BH, N, d]  dtype
 *   codebook   in  [H, Mt, d]  dtype
 *   vsum       in  [BH, Mt, d] float  (from avq_assign_aggregate)
 *   counts     in  [BH, Mt]    int32  (from avq_assign_aggregate)
 *   P          0 <= P <= M0 (P = 0: plain VQ attention over the parents);
 *              P must be 0 when C = 0 (AVQ_ERR_SHAPE otherwise)
 *   block_q    query tile: 32, 64 or 128 (one wave of 64 lanes per 32 queries)
 *   scale      logit scale, > 0 (1/sqrt(d) in the usual convention, Sec. 3.1)
 *   Y          out [BH, N, d] float
 *   topp       out [BH, ceil(N/block_q), P] int32, the selected parents of
 *              each tile in ascending order, or NULL to skip
 *   importance out [BH, ceil(N/block_q), M0] float, w_j per tile, or NULL
 *   workspace  device memory of at least avq_attention_workspace_size()
 *              bytes (AVQ_ERR_WORKSPACE otherwise); overwritten by the call
 *
 * Precision (bf16 inputs): logits use bf16 inputs with float accumulation;
 * the weighted value sums use fp16 operands (weights in [-2^8, 2^8], value
 * sums scaled by one power of two per (batch, head)) with float accumulation;
 * softmax bookkeeping, denominators and importances are float.  fp32 inputs
 * use float throughout.
 */
int avq_attention_fwd(const void* Q, const void* codebook, const float* vsum,
                      const int32_t* counts, int B, int H, int N, int d, int M0,
                      int C, int dtype, int P, int block_q, float scale,
                      float* Y, int32_t* topp, float* importance,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * AVQ attention forward with the approximate tiled denominator of App. B
 * (Eq. 13-14) for the importances.  The parents are visited in tiles of 64;
 * after tile J the importances of its parents are formed at once with
 *   Z~_i(J) = N / N_seen(J) * (sum over the tiles t <= J of sum_{j in t} A_ij n_j),
 *   w_j = sum_{i in tile} A_ij n_j / Z~_i(J),
 * where N_seen(J) counts the keys of the parents of tiles 0..J and N all keys
 * (w_j = 0 while N_seen(J) = 0), so no second pass over the parents is made.
 * Everything else -- the selection, the refinement and Y with its exact
 * denominator -- is as in avq_attention_fwd, and so are the arguments,
 * layouts, workspace and errors.  With M0 <= 64 (one tile) the result equals
 * avq_attention_fwd's.
 */
int avq_attention_fwd_approx(const void* Q, const void* codebook, const float* vsum,
                             const int32_t* counts, int B, int H, int N, int d, int M0,
                             int C, int dtype, int P, int block_q, float scale,
                             float* Y, int32_t* topp, float* importance,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * AVQ attention forward with the query tiles taken in a given token order
 * (Sec. 4.3 and Fig. 3: the queries of an image are put in the order of a
 * Gilbert space-filling curve, so that each tile of block_q consecutive
 * positions along the curve is a compact 2-D region and shares one parent
 * selection; App. H, Tab. 8 compares curve, raster and random orders).
 *
 * Tile t holds the queries of the rows query_order[t*block_q + i],
 * 0 <= i < block_q (the last tile may be partial), and the output of each
 * query goes to its own row of Y, so Y is in the row order of Q whatever the
 * query order.  With query_order[i] = i this is avq_attention_fwd (or
 * avq_attention_fwd_approx when approx_denominator is nonzero); topp and
 * importance are indexed by tile, in the given order.
 *
 *   query_order  in  [N] int32 device array, 4-byte aligned, shared by every
 *                (batch, head): a permutation of 0 .. N-1.  An entry outside
 *                [0, N) makes its position empty: it adds nothing to its
 *                tile's importances and no row is written for it.  A row
 *                named twice is written twice (which value stays is
 *                unspecified); a row never named is not written.
 *   approx_denominator  nonzero: the importances of avq_attention_fwd_approx
 *
 * Every other argument, layout, the workspace and the errors are those of
 * avq_attention_fwd; a NULL query_order is AVQ_ERR_NULL (when B*H and N are
 * not zero).
 */
int avq_attention_fwd_ordered(const void* Q, const void* codebook, const float* vsum,
                              const int32_t* counts, int B, int H, int N, int d, int M0,
                              int C, int dtype, int P, int block_q, float scale,
                              const int32_t* query_order, int approx_denominator,
                              float* Y, int32_t* topp, float* importance,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * The two halves of avq_attention_fwd, for callers that attend several query
 * batches to one set of aggregates (Eq. 3: the value sums and counts depend
 * on the keys only), that keep the aggregates' buffers across calls, and to
 * time the attention kernel on its own.
 *
 * avq_attention_prepare converts the value sums (Eq. 3, from
 * avq_assign_aggregate) into the operands of the weighted-value products
 * (Eq. 6 and 9) and copies the counts, both into the workspace: one or two
 * launches, reading vsum and counts and writing the workspace.  Q, codebook
 * and P play no part, and N is not needed.
 *
 * avq_attention_fwd_prepared is then the rest of avq_attention_fwd for one
 * query batch: the attention kernel alone, reading the operands and counts
 * from a workspace that avq_attention_prepare filled with the same B, H, d,
 * M0, C and dtype, unchanged since; it does not write the workspace, so any
 * number of such calls may follow one preparation, also concurrently on
 * different streams once the preparation has completed.  Given those, its
 * outputs are bit for bit those of avq_attention_fwd on the same arguments.
 * A workspace not prepared so gives unspecified (but memory-safe) outputs.
 *
 *   clear_vsum    NULL, or [B*H, Mt, d] float, 16-byte aligned: zero-filled
 *                 by the call (every element)
 *   clear_counts  NULL, or [B*H, Mt] int32, 16-byte aligned: zero-filled
 * The attention kernel reads neither the value sums nor the counts once they
 * are prepared, so passing the buffers avq_attention_prepare read leaves them
 * zero, ready for the next avq_assign_aggregate_accum, with no separate fill
 * launch (the fill is spread over the attention kernel's workgroups; with
 * N = 0 the call only fills).  They must not be read or written by other
 * work in flight meanwhile, and calls sharing one preparation must not clear
 * a buffer that another of them reads.
 *
 * Arguments, layouts and errors are otherwise those of avq_attention_fwd;
 * prepare checks only what it uses (vsum, counts, the workspace and the
 * sizes).
 */
int avq_attention_prepare(const float* vsum, const int32_t* counts, int B, int H, int d,
                          int M0, int C, int dtype, void* workspace,
                          size_t workspace_bytes, void* stream);
int avq_attention_fwd_prepared(const void* Q, const void* codebook, int B, int H, int N,
                               int d, int M0, int C, int dtype, int P, int block_q,
                               float scale, float* Y, int32_t* topp, float* importance,
                               const void* workspace, size_t workspace_bytes,
                               float* clear_vsum, int32_t* clear_counts, void* stream);

/*
 * avq_attention_fwd without a workspace argument, for callers that cannot
 * allocate device memory around the call (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation).  It computes exactly what
 * avq_attention_fwd computes, with the same kernels, arguments (minus
 * workspace and workspace_bytes), layouts and errors, and allocates nothing:
 * the operands avq_attention_fwd keeps in its workspace live in a static
 * device array of AVQ_NOALLOC_SCRATCH_BYTES (8 MiB) that every GPU the
 * library runs on holds from the library's load to the end of the process.
 * Its address on a GPU is looked up on the first call made with that GPU
 * current.
 *
 * Limit: calls whose avq_attention_workspace_size() exceeds
 * AVQ_NOALLOC_SCRATCH_BYTES return AVQ_ERR_SCRATCH and write nothing (bf16,
 * d = 64, M0 = 64, C = 8 fits B*H <= 110; d = 128, M0 = 256, C = 8 fits
 * B*H <= 13).
 *
 * Concurrency: every call on one GPU uses that GPU's one scratch array, and
 * each call overwrites what it uses before reading it (nothing carries over
 * from an earlier call).  Calls on one GPU must therefore not overlap: two
 * calls in flight at once -- on different streams, or from different host
 * threads -- race on the scratch and give wrong results.  Calls on one stream
 * run one after another and are safe.
 */
int avq_attention_fwd_noalloc(const void* Q, const void* codebook, const float* vsum,
                              const int32_t* counts, int B, int H, int N, int d, int M0,
                              int C, int dtype, int P, int block_q, float scale,
                              float* Y, int32_t* topp, float* importance, void* stream);

/*
 * Codebook update step of the training recipe (App. A, Eq. 11 and Eq. 12;
 * Sec. 4.1, Fig. 2): one step of EMA online k-means on the hierarchical
 * codebook of every head, with the parent-child constraint restored.
 *
 *   ksum     in  [B*H, Mt, d] float: this batch's keys summed per codeword,
 *                parents over their whole cell and children over the keys
 *                that moved to them -- the vsum of avq_assign_aggregate
 *                called with the keys as the values (V = K)
 *   counts   in  [B*H, Mt] int32: the matching key counts (its counts)
 *   decay    the EMA decay lambda, 0 <= decay <= 1
 *   S        in/out [H, Mt, d] float: EMA key sums S_x (Eq. 11)
 *   Nema     in/out [H, Mt] float: EMA key counts N_x (Eq. 11)
 *   codebook in/out [H, Mt, d] float: the codeword positions
 *
 * For every head h and codeword x, with the batch totals over b = 0..B-1:
 *   S_x <- decay S_x + (1 - decay) sum_b ksum[b*H+h, x]
 *   N_x <- decay N_x + (1 - decay) sum_b counts[b*H+h, x]
 * a parent moves to its mean S_p / N_p (it keeps its position while
 * N_p = 0), and its children to the minimiser of sum_c N_c |M_c - C_pc|^2
 * with mean_c C_pc = C_p, M_c = S_c / N_c (Eq. 12):
 *   C_pc = M_c - delta / (N_c sigma), delta = sum_c M_c - C C_p,
 *   sigma = sum_c 1 / N_c.
 * A child with N_c = 0 has no mean: its current position stands for M_c, and
 * the children without mass share the whole residual equally (the limit of
 * Eq. 12 as their mass goes to zero), the others keeping their means.  With
 * C = 0 every codeword moves to its mean.  Arithmetic is float; the
 * constraint then holds to float rounding (a bf16 copy of the codebook for
 * the forward calls holds it to bf16 rounding).
 *
 * Sizes: d >= 1, C <= 16, H*M0 <= 2^30 (AVQ_ERR_UNSUPPORTED otherwise); B may
 * be 0 (pure decay; ksum and counts may then be NULL).  All pointers 4-byte
 * aligned (AVQ_ERR_ALIGN).  S, Nema and codebook are updated in place; the
 * three must not overlap each other or the inputs.  Allocates nothing.
 */
int avq_codebook_update(const float* ksum, const int32_t* counts, int B, int H, int d, int M0,
                        int C, float decay, float* S, float* Nema, float* codebook,
                        void* stream);

/* Human-readable name of a status code (static string). */
const char* avq_status_string(int status);

/* Library version: major * 10000 + minor * 100 + patch. */
int avq_version(void);

#ifdef __cplusplus
}
#endif

#endif /* AVQ_H */
