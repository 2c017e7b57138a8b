/*
 * tp_layer.h - C ABI of libtplayer: one tensor-parallel rank's share of a
 * Megatron-style GPT Transformer layer (causal self-attention block and MLP
 * block), forward and backward, on AMD Instinct MI355X (gfx950).
 *
 * The method (paper-graph summary of "Efficient Large-Scale Language Model
 * Training on GPU Clusters Using Megatron-LM", section 3, "Tensor Model
 * Parallelism: The Megatron Partitioning"; interview book "Distributed
 * training", section 2.6):
 *   MLP block:        U_r = H W1[:, f_r] + b1[f_r];  Z_r = GELU(U_r);
 *                     partial_r = Z_r W2[f_r, :]      (column split, then row split)
 *   attention block:  QKV_r = X [Wq|Wk|Wv][:, c_r] + b_qkv[c_r]  (whole heads);
 *                     per head causal softmax(Q K^T / sqrt(d)) V;
 *                     partial_r = C_r Wo[c_r, :]       (row split)
 *   The all-reduce (g forward, f backward) is NOT performed by the rank
 *   calls: each call ends in a per-rank partial sum, exactly where the
 *   all-reduce would sit. The replicated output bias and the residual are
 *   added after the all-reduce (the fused bias + dropout + residual add of
 *   the paper-graph page's "Computation Optimizations", without dropout);
 *   on one GPU tp_reduce_partials does the sum and that add in one pass.
 *
 * Shapes (t = ranks, r = rank, T = s*b tokens, d = h/a, a_r = a/t heads per rank):
 *   activations: token-major [s, b, h], row index sigma*b + beta, row-major.
 *   weights W[d_in, d_out], row-major, Y = X W.
 *   c_r = columns [r h/t, (r+1) h/t) of each of Wq, Wk, Wv; f_r = [r 4h/t, (r+1) 4h/t).
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers, 16-byte aligned, owned by the
 *     caller; the library never allocates, frees or keeps them.
 *   - Element type is given by `dtype`: TP_BF16 (storage bf16, fp32
 *     accumulation) or TP_FP32 (fp32 throughout).
 *   - GELU is the erf form x Phi(x); the kernels evaluate Phi with the
 *     rational approximation of Abramowitz & Stegun 7.1.26 (within 3e-7 of
 *     the exact Phi in fp32), for GELU and for GELU' = Phi + x phi.
 *   - `stream` is a hipStream_t (NULL = default stream). Work is enqueued
 *     asynchronously; nothing synchronizes the host.
 *   - Outputs and gradients are overwritten, never accumulated.
 *   - Return value: TP_OK (0) or a negative TP_E* code; no exceptions or
 *     aborts cross the ABI. tp_strerror() describes a code; for TP_EHIP it
 *     returns the HIP error text of the calling thread's last failure.
 *   - `rank` selects no code path: every rank does the same work on the
 *     shards it is given. It is validated (0 <= rank < t) and documents
 *     which shards the caller must pass.
 */
#ifndef TP_LAYER_H
#define TP_LAYER_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

enum tp_dtype { TP_BF16 = 0, TP_FP32 = 1 };
enum tp_block { TP_ATTN = 0, TP_MLP = 1 };

enum tp_status {
  TP_OK = 0,
  TP_EINVAL = -1,        /* non-positive dims, h % a, a % t (heads stay whole), rank not in [0,t), bad enum */
  TP_EUNSUPPORTED = -2,  /* s, b*s, d or h/t not a multiple of 16, or a matrix of
                            2^31 or more elements (the tile loaders use 32-bit
                            byte offsets within an operand) */
  TP_ENULL = -3,         /* a required pointer is NULL */
  TP_EALIGN = -4,        /* a pointer is not 16-byte aligned */
  TP_EWORKSPACE = -5,    /* workspace_bytes < tp_workspace_bytes(...) */
  TP_EHIP = -6,          /* a HIP launch failed */
  TP_ESCRATCH = -7       /* tp_layer_bwd_noalloc: the call needs more than tp_noalloc_scratch_bytes() */
};

/* Rank-local weights of one block.
 *   TP_ATTN: w_in  = [Wq[:,c_r] | Wk[:,c_r] | Wv[:,c_r]]  [h, 3h/t]
 *            b_in  = [bq[c_r] | bk[c_r] | bv[c_r]]         [3h/t]
 *            w_out = Wo[c_r, :]                            [h/t, h]
 *            b_out = bo (replicated)                       [h]
 *   TP_MLP:  w_in  = W1[:, f_r] [h, 4h/t];  b_in = b1[f_r] [4h/t]
 *            w_out = W2[f_r, :] [4h/t, h];  b_out = b2 (replicated) [h]
 * b_out is not read by the rank calls (it is added after the all-reduce, see
 * tp_reduce_partials) and may be NULL there.                                 */
typedef struct {
  const void *w_in, *b_in, *w_out, *b_out;
} tp_block_weights;

/* Rank-local gradients, same shapes as tp_block_weights. dw_in, db_in and
 * dw_out are this rank's shards of the unsharded gradients (weight gradients
 * need no tensor-parallel communication); db_out is the full [h] gradient of
 * the replicated bias, computed identically on every rank. */
typedef struct {
  void *dw_in, *db_in, *dw_out, *db_out;
} tp_block_grads;

/* Pure host validation, no HIP call: TP_OK or TP_EINVAL / TP_EUNSUPPORTED.
 * Heads must divide evenly by t ("parallelism" blog, Attention). Every
 * matrix of the call must hold fewer than 2^31 elements: [T, h], [T, 4h/t],
 * the weight shards (up to [h, 4h/t]) and, on the materialised attention
 * path (fp32, or d not in {64, 96, 128, 160}), one [s, s] score matrix.   */
int tp_check_args(int h, int a, int s, int b, int t, int rank, int dtype, int block);

/* Bytes of activations that tp_layer_fwd(block, rank) saves for
 * tp_layer_bwd(block, rank) (what the backward reads of the forward: the
 * activation memory per layer of the interview book "Distributed training",
 * section 2.2, for one rank's shards). ATTN keeps QKV_r [T,3h/t] and the context C_r
 * [T,h/t] (also in fp32 for bf16); with bf16 and d in {64, 96, 128, 160}
 * (fused attention) also the bf16 rounding residuals of Q_r and K_r [T,2h/t]
 * and one log-sum-exp per query and head, otherwise the causal softmax P_r
 * [b*a_r, s, s]. MLP keeps U_r and Z_r [T,4h/t]. 0 on invalid arguments. */
size_t tp_saved_bytes(int h, int a, int s, int b, int t, int dtype, int block);

/* Scratch bytes needed by both tp_layer_fwd and tp_layer_bwd of `block`:
 * the gradient temporaries of the chain rule ("parallelism" blog, "The
 * backward pass": dC, D = rowsum(dC * C), dQKV for ATTN; dU for MLP), the
 * score matrix of the materialised attention path, and fp32 partial tiles
 * of split-K / stream-K GEMMs and of the fused attention's chunks. Owned by
 * the caller, 16-byte aligned; its contents do not outlive a call, so one
 * buffer of the larger of the two blocks' sizes serves every call on a
 * stream. 0 on invalid args.                                                */
size_t tp_workspace_bytes(int h, int a, int s, int b, int t, int dtype, int block);

/* Forward of rank `rank`'s share of `block` (paper-graph page, section 3,
 * "Tensor Model Parallelism: The Megatron Partitioning": the first GEMM of a
 * block split by columns, the second by rows, so the block ends in a partial
 * sum that the g all-reduce adds up; "parallelism" blog, "The MLP, with real
 * numbers" and "Attention").
 *   x          [T, h]  block input, replicated on every rank (f = identity)
 *   w          rank-local weights (see tp_block_weights)
 *   y_partial  [T, h]  out: this rank's partial C_r Wo_r (ATTN) or Z_r W2_r
 *                      (MLP). x + b_out + sum over ranks = block output.
 *   saved      tp_saved_bytes(...) bytes, out: activations for the backward
 *   workspace  tp_workspace_bytes(...) bytes of scratch
 * ATTN: QKV GEMM + bias, causal scaled softmax per head, P V, output GEMM.
 * MLP:  FC1 GEMM with fused bias + GELU, FC2 GEMM.                           */
int tp_layer_fwd(int h, int a, int s, int b, int t, int rank, int dtype, int block,
                 const void *x, const tp_block_weights *w, void *y_partial, void *saved,
                 void *workspace, size_t workspace_bytes, void *stream);

/* Backward of rank `rank`'s share of `block` ("parallelism" blog, "The
 * backward pass": weight gradients are local to the rank; the input
 * gradient is a partial sum that f's backward all-reduce adds up).
 *   x, w       as passed to tp_layer_fwd
 *   saved      as written by tp_layer_fwd(block, rank), unchanged
 *   dy         [T, h] gradient of the block output, replicated (g's backward
 *              is the identity)
 *   dx_partial [T, h] out: this rank's partial of dL/dx through its shards.
 *              dy + sum over ranks (f's backward all-reduce, then the
 *              residual gradient) = dL/dx.
 *   g          out: rank-local gradients (see tp_block_grads)
 * Chain rule: "parallelism" blog, "The backward pass"; the softmax backward
 * uses dS = P * (dP - rowsum(dC * C)).                                       */
int tp_layer_bwd(int h, int a, int s, int b, int t, int rank, int dtype, int block,
                 const void *x, const tp_block_weights *w, const void *saved, const void *dy,
                 void *dx_partial, const tp_block_grads *g,
                 void *workspace, size_t workspace_bytes, void *stream);

/* tp_layer_bwd without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc). The workspace is a buffer the
 * library holds in device memory (a file-scope array of
 * tp_noalloc_scratch_bytes() = 256 MiB, one copy on each GPU it runs on,
 * kept until the process ends); the call allocates and frees nothing.
 * Arguments, results and errors as tp_layer_bwd, plus TP_ESCRATCH when
 * tp_workspace_bytes(h, a, s, b, t, dtype, block) exceeds the buffer (e.g.
 * the attention block of h=2304, a=24, s=2048, b=4, t=1 needs 289 MiB).
 * Every call on one GPU shares that GPU's buffer: calls that overlap in time
 * on one GPU (different streams or threads without ordering) race and give
 * wrong results. Calls in order on one stream are safe.                    */
size_t tp_noalloc_scratch_bytes(void);
int tp_layer_bwd_noalloc(int h, int a, int s, int b, int t, int rank, int dtype, int block,
                         const void *x, const tp_block_weights *w, const void *saved, const void *dy,
                         void *dx_partial, const tp_block_grads *g, void *stream);

/* Stand-in for the all-reduce on one GPU, fused with the bias + residual add
 * that follows it:
 *   out[i, j] = sum_{r<t} partials[r, i, j] + bias[j] + residual[i, j]
 * summed in rank order in fp32 and rounded once ("parallelism" blog, "First:
 * the three collectives": an all-reduce is the element-wise sum).
 *   partials  [t, rows, cols] contiguous; bias [cols] or NULL;
 *   residual  [rows, cols] or NULL; out [rows, cols] (must not alias partials).
 * cols must be a multiple of 8. Forward: bias = b_out, residual = block input;
 * backward: bias = NULL, residual = the block output's gradient.             */
int tp_reduce_partials(int dtype, long rows, long cols, int t, const void *partials, const void *bias,
                       const void *residual, void *out, void *stream);

/* Backward with full activation recomputation ("Distributed training"
 * interview book, section 2.2: full recomputation keeps only the layer input
 * and pays a second forward pass; paper-graph page, "FLOP Counting and
 * Training Time Estimation": recomputation adds one forward pass to the
 * count). Same result as tp_layer_fwd followed by tp_layer_bwd, bit for bit,
 * without keeping any activation between the two calls:
 *   scratch  tp_saved_bytes(...) bytes of device memory, overwritten: the
 *            forward is re-run into it up to (not including) the block's
 *            output product, whose result the backward does not read; the
 *            buffer can be shared by every layer, since nothing in it
 *            outlives the call.
 * Other arguments, ownership and errors as tp_layer_bwd.                     */
int tp_layer_bwd_recompute(int h, int a, int s, int b, int t, int rank, int dtype, int block,
                           const void *x, const tp_block_weights *w, const void *dy, void *dx_partial,
                           const tp_block_grads *g, void *scratch,
                           void *workspace, size_t workspace_bytes, void *stream);

/* LayerNorm of `rows` tokens of width h, fused with the bias + residual add
 * that precedes it. With sequence parallelism ("parallelism" blog post,
 * "Sequence parallelism: the parts TP leaves behind") a rank runs it on its
 * own slice of the sequence: between the reduce-scatter that ends one block
 * and the all-gather that feeds the next, it adds the output bias and the
 * residual and applies the next LayerNorm.
 *   v       = x + residual + bias, rounded once to dtype (residual, bias may
 *             be NULL); written to sum_out [rows, h] if sum_out is not NULL
 *   y       = (v - mean(v)) / sqrt(var(v) + eps) * gamma + beta, per row,
 *             mean and biased variance over the h features, in fp32
 *   stats   [rows, 2] fp32: mean and 1/sqrt(var + eps) of each row
 * gamma == NULL: add only (then beta, y and stats are not used and sum_out
 * is required); otherwise beta, y and stats are required.
 *   x, residual, sum_out, y  [rows, h];  bias, gamma, beta [h]
 * h must be a multiple of 8 and at most 32768 (bf16) or 16384 (fp32)
 * (TP_EUNSUPPORTED); eps >= 0 and finite (TP_EINVAL). stats needs 8-byte
 * alignment, every other pointer 16 (TP_EALIGN). y and sum_out must not
 * alias the inputs of another row. rows == 0: TP_OK, nothing is read or
 * written. The page does not write LayerNorm out: this is the textbook
 * definition.                                                                */
int tp_layernorm_fwd(int dtype, long rows, long h, float eps, const void *x, const void *bias,
                     const void *residual, const void *gamma, const void *beta, void *sum_out, void *y,
                     float *stats, void *stream);

/* Backward of tp_layernorm_fwd for the gradient dy of its output y:
 *   x_hat = (v - mean) rstd,  g = dy * gamma
 *   dx     = rstd (g - mean_h(g) - x_hat mean_h(g x_hat)) + dresid
 *   dgamma = sum over the rows of dy x_hat,  dbeta = sum over the rows of dy
 *   v      [rows, h] the LayerNorm input (tp_layernorm_fwd's sum_out, or its
 *          x when no residual or bias was added); stats as written by it
 *   dresid [rows, h] gradient reaching v through the residual path, or NULL
 *   dx     [rows, h] out; dgamma, dbeta [h] out, both or neither (NULL).
 * With sequence parallelism the rows are the rank's own tokens, so dgamma
 * and dbeta are this rank's partial sums: their sum over the ranks (the
 * all-reduce of the replicated LayerNorm weights' gradients) is the full
 * gradient. dx must not alias dy or v. Sizes, alignment and errors as
 * tp_layernorm_fwd; rows == 0 writes zeros to dgamma and dbeta (if given)
 * and reads nothing else.                                                    */
int tp_layernorm_bwd(int dtype, long rows, long h, const void *dy, const void *v, const float *stats,
                     const void *gamma, const void *dresid, void *dx, void *dgamma, void *dbeta, void *stream);

/* General GEMM on the same MFMA kernels and the same launch planning as the
 * layer's weight GEMMs (whole waves of 256x256 tiles, stream-K over a partial
 * last wave, or split-K for few tiles; every sum in a fixed order):
 *   C[M,N] = alpha * op(A) op(B) (+ bias[N]).
 *   a_kmajor: A stored [M, lda] (element (m,k) at A[m*lda+k]) if 1, else
 *             stored [K, lda] (element (m,k) at A[k*lda+m]).
 *   b_kmajor: B stored [N, ldb] (element (k,n) at B[n*ldb+k]) if 1, else
 *             stored [K, ldb] (element (k,n) at B[k*ldb+n]).
 *   bias may be NULL. C has leading dimension ldc. M, N, K multiples of 16;
 *   leading dimensions multiples of 8 (TP_EUNSUPPORTED otherwise, and when
 *   A, B or C spans 2^31 or more elements, rows x leading dimension).
 *   workspace: device scratch of at least tp_gemm_workspace_bytes(dtype, M,
 *   N, K) bytes, 256-byte aligned, owned by the caller (NULL when that size is
 *   0); TP_EWORKSPACE if smaller. Used by the tests to check each operand
 *   layout and launch plan on its own.                                        */
size_t tp_gemm_workspace_bytes(int dtype, int M, int N, int K);
int tp_gemm(int dtype, int M, int N, int K, float alpha,
            const void *A, long lda, int a_kmajor, const void *B, long ldb, int b_kmajor,
            const void *bias, void *C, long ldc, void *workspace, size_t workspace_bytes, void *stream);

/* Opt-in profiling of the library's own launches. While enabled, every
 * kernel group the library enqueues (one GEMM with its split-K reduction,
 * the softmax, a column sum, ...) is bracketed by two HIP events on the
 * call's stream and tagged with its role ("fc1_fwd", "scores", "reduce",
 * ...), its algorithmic FLOPs (2MNK; attention products count the full s x s
 * square, as the paper-graph page's FLOP formula does) and its algorithmic
 * HBM bytes (each operand read once, each result written once).
 * tp_prof_enable(1) clears the records and starts; tp_prof_enable(0) stops.
 * tp_prof_read waits for the recorded events, sums them per role into `out`
 * (up to max_entries), clears the records and returns the number of roles
 * seen (or a negative TP_E* code). Event timing adds a few microseconds per
 * recorded group; leave it off for throughput measurements.                */
typedef struct {
  char name[24];
  int launches;
  double ms;
  double flops;
  double bytes;
} tp_prof_entry;

int tp_prof_enable(int on);
int tp_prof_read(tp_prof_entry *out, int max_entries);

const char *tp_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* TP_LAYER_H */
