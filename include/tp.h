/*
 * tp.h - tensor-parallel sharded linear layer Y = X W on one MI355X (gfx950).
 *
 * The operation follows these web pages on tensor parallelism:
 *   [TP-topic]  "Tensor Parallelism" topic page, chipfoundryservices.com
 *   [AI-gloss]  "Tensor Parallelism" entry, AI Glossary, aiforbusinessandlife.com
 *   [DLwPT]     "Tensor parallelism" concept page, Deep Learning with PyTorch 2e
 *
 * A weight W of logical shape [K, Nout] (rows = input features, columns =
 * output features, Y = X W) is split over N logical shards, either by output
 * columns (W = [W_0, ..., W_{N-1}], [TP-topic] "Column-Wise Parallelism") or
 * by rows, i.e. the contracted dimension (W = [W_0; ...; W_{N-1}] with X split
 * to match, [TP-topic] "Row-Wise Parallelism"). Shard s always owns the s-th
 * contiguous block; N must divide the split dimension. All N shards (or a
 * range of them) run on the one GPU, so the pages' all-gather becomes a
 * concatenation in device memory and their all-reduce becomes an fp32 sum of
 * partials in ascending shard order.
 *
 * Conventions shared by every entry point
 *   Memory      Every tp_matrix points to device memory owned by the caller.
 *               The library allocates and frees nothing; descriptors are read
 *               before the call returns. Apart from tp_mlp_noalloc's scratch
 *               array (see there) it keeps no mutable global state.
 *   Streams     Work is enqueued on `stream` (a hipStream_t; NULL = the null
 *               stream) and the call returns without waiting. Inputs must
 *               stay alive and unchanged until the stream has passed the work.
 *   Errors      Every argument is checked on the host before any HIP call; on
 *               failure the call returns the status and enqueues nothing. A
 *               failed launch returns TP_ERR_HIP. No C++ exception crosses
 *               this interface.
 *   Dtypes      X and W share one dtype. TP_BF16 runs on the bf16 matrix cores
 *               with fp32 accumulation; TP_F32 runs an fp32 FMA path (exact on
 *               integer-valued inputs whose partial sums stay below 2^24).
 *               Partials and sums are fp32. bf16 outputs are rounded to
 *               nearest-even from the fp32 result.
 *   Layout      Row-major. `ld` is the distance in elements between rows.
 *               Leading dimensions or pointers that are not 16-byte aligned,
 *               or widths that are not multiples of 8, select a slower
 *               element-guarded kernel; they are not an error.
 *   Aliasing    An output may not overlap any input (TP_ERR_ALIAS).
 *   Empty       A zero-sized output is a successful no-op. K = 0 gives act(0).
 */
#ifndef TP_H
#define TP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum tp_status {
  TP_OK = 0,
  TP_ERR_NULL = 1,         /* a descriptor, data pointer or out-parameter is NULL */
  TP_ERR_DTYPE = 2,        /* unsupported dtype, or X and W dtypes differ, or P not fp32 */
  TP_ERR_SHAPE = 3,        /* negative size, or shapes that do not chain (X.cols != W.rows, ...) */
  TP_ERR_INDIVISIBLE = 4,  /* N < 1 or N does not divide the split dimension */
  TP_ERR_SHARD_RANGE = 5,  /* s0 < 0, ns < 1 or s0 + ns > N */
  TP_ERR_STRIDE = 6,       /* ld shorter than a row, or shard blocks that overlap */
  TP_ERR_ALIAS = 7,        /* an output overlaps an input */
  TP_ERR_WORKSPACE = 8,    /* workspace missing or smaller than required */
  TP_ERR_HIP = 9,          /* a kernel launch failed */
  TP_ERR_TOO_LARGE = 10    /* a size exceeds the 32-bit tile/launch limits of the kernels */
} tp_status;

typedef enum tp_dtype { TP_F32 = 0, TP_BF16 = 1 } tp_dtype;

/*
 * Which dimension is split: W's output columns, W's rows (the contracted
 * dimension), or the token rows of the activations (sequence parallelism).
 */
typedef enum tp_axis { TP_SPLIT_COLS = 0, TP_SPLIT_ROWS = 1, TP_SPLIT_TOKENS = 2 } tp_axis;

typedef enum tp_act { TP_ACT_NONE = 0, TP_ACT_GELU = 1 } tp_act;

/*
 * A row-major matrix in device memory, possibly stored as shard blocks.
 *   ptr           element [0][0] (of block 0 when shard_stride > 0)
 *   dtype         tp_dtype
 *   rows, cols    the LOGICAL shape, as defined by each entry point
 *   ld            elements between consecutive rows (of one block when shard_stride > 0)
 *   shard_stride  0: the blocks are slices of one row-major matrix;
 *                 > 0: shard-major storage, block j starts shard_stride
 *                 elements after block j-1 (each block has its own rows with
 *                 row stride ld); blocks may not overlap.
 */
typedef struct tp_matrix {
  void* ptr;
  int32_t dtype;
  int32_t reserved; /* padding, ignored */
  int64_t rows;
  int64_t cols;
  int64_t ld;
  int64_t shard_stride;
} tp_matrix;

/*
 * Column-parallel linear ([TP-topic] "Column-Wise Parallelism"; [AI-gloss]
 * "Worked example", column split). For s = s0 .. s0+ns-1, shard s computes
 *     Y_j = act(X W_s),  j = s - s0,
 * where W_s = W[:, s*Nout/N : (s+1)*Nout/N] and the activation is elementwise
 * on the fp32 result ([TP-topic] "Megatron-LM Tensor Parallelism": applied on
 * each shard without exchange; TP_ACT_GELU = x * Phi(x), Phi(x) = (1 + erf(x /
 * sqrt 2)) / 2, evaluated in fp32 to within 5e-7 of the exact value).
 *   X  [M, K], shard_stride 0 (the same X reaches every shard).
 *   W  logical [K, Nout], N | Nout. shard_stride 0: W_s is the column slice
 *      above (ld >= Nout); > 0: W_s is the [K, Nout/N] block at
 *      ptr + s*shard_stride with row stride ld (ld >= Nout/N).
 *   Y  logical [M, ns*Nout/N], dtype TP_F32 or TP_BF16. shard_stride 0: Y_j is
 *      written at columns j*Nout/N (the concatenation, [TP-topic]
 *      "Column-Wise Parallelism": output combination); > 0: Y_j is the
 *      [M, Nout/N] block at ptr + j*shard_stride (outputs left partitioned,
 *      [AI-gloss] "Worked example").
 */
tp_status tp_col_linear(const tp_matrix* X, const tp_matrix* W, int32_t N, int32_t s0, int32_t ns,
                        int32_t act, const tp_matrix* Y, void* stream);

/*
 * Row-parallel linear, partial products only ([TP-topic] "Row-Wise
 * Parallelism"; [AI-gloss] "Worked example", split along the input
 * dimension). For s = s0 .. s0+ns-1, shard s computes the fp32 partial
 *     P_j = X_s W_s,  j = s - s0,
 * with X_s = X[:, s*K/N : (s+1)*K/N] and W_s = W[s*K/N : (s+1)*K/N, :].
 *   X  logical [M, K], N | K. shard_stride 0: X_s is the column slice; > 0:
 *      X_s is the [M, K/N] block at ptr + s*shard_stride (e.g. the
 *      partitioned output of a column-parallel layer).
 *   W  logical [K, Nout]. shard_stride 0: W_s is the row slice; > 0: the
 *      [K/N, Nout] block at ptr + s*shard_stride.
 *   P  dtype TP_F32, rows = M, cols = Nout; P_j at ptr + j*shard_stride with
 *      row stride ld. shard_stride may be 0 only when ns = 1.
 * Combine the partials with tp_reduce_partials(axis = TP_SPLIT_ROWS).
 */
tp_status tp_row_linear(const tp_matrix* X, const tp_matrix* W, int32_t N, int32_t s0, int32_t ns,
                        const tp_matrix* P, void* stream);

/*
 * Combine n shard outputs ([AI-gloss] "Check your understanding": outputs
 * for the same coordinates are added, outputs for different coordinates are
 * concatenated; [TP-topic] "Tensor Parallelism Fundamentals").
 *   P     n blocks of [rows, cols] at ptr + j*shard_stride, row stride ld,
 *         dtype TP_F32 (axis ROWS) or TP_F32 / TP_BF16 (axis COLS, TOKENS).
 *   axis  TP_SPLIT_ROWS: the contracted dimension was split, so
 *           Y = P_0 + P_1 + ... + P_{n-1}, fp32, in ascending j
 *         (the single-GPU form of the all-reduce);
 *         TP_SPLIT_COLS: the output columns were split, so
 *           Y = [P_0 | P_1 | ... | P_{n-1}]  (Y.cols = n*cols; the all-gather);
 *         TP_SPLIT_TOKENS: the token rows were split, so the blocks are
 *           stacked in order, Y = [P_0; P_1; ...; P_{n-1}] (Y.rows = n*rows;
 *           the all-gather of the token shards before attention, [TP-topic]
 *           "Sequence Parallelism Extension").
 *   Y     [rows, cols] (ROWS), [rows, n*cols] (COLS) or [n*rows, cols]
 *         (TOKENS), dtype TP_F32 or TP_BF16 (ROWS: rounded from the fp32 sum;
 *         COLS, TOKENS: converted, exact when P and Y share a dtype),
 *         Y.shard_stride must be 0.
 */
tp_status tp_reduce_partials(const tp_matrix* P, int32_t n, int32_t axis, const tp_matrix* Y, void* stream);

/*
 * Megatron-style tensor-parallel MLP forward ([TP-topic] "Megatron-LM Tensor
 * Parallelism": the first linear split by columns, the activation on each
 * shard, the second linear split by rows, one sum at the end):
 *     Y = sum_{s=s0}^{s0+ns-1} act(X W1_s) W2_s        (fp32, ascending s)
 * with W1_s = W1[:, s*F/N : (s+1)*F/N] and W2_s = W2[s*F/N : (s+1)*F/N, :];
 * the same slice of the intermediate width F indexes both, so the
 * intermediate H_s = act(X W1_s) never leaves its shard. With bf16 inputs H_s
 * is rounded to bf16 before the second product.
 *   X   [M, d], shard_stride 0.       W1 logical [d, F], N | F.
 *   W2  logical [F, Dout].            shard_stride as in tp_col_linear (W1)
 *                                     and tp_row_linear (W2).
 *   Y   [M, Dout], TP_F32, shard_stride 0.
 *   workspace, *workspace_bytes
 *       device scratch for H, the partials and, for 32 rows or fewer, the
 *       first product's K-chunk sums (size depends on the shapes).
 *       If workspace is NULL the required size is stored in *workspace_bytes
 *       and TP_OK is returned with nothing enqueued (only shapes, dtypes and
 *       strides are checked then; data pointers may be NULL); otherwise
 *       *workspace_bytes must be at least that size. The workspace must not
 *       overlap any operand. It may be reused once the stream has passed
 *       the call.
 */
tp_status tp_mlp(const tp_matrix* X, const tp_matrix* W1, const tp_matrix* W2, int32_t N, int32_t s0,
                 int32_t ns, int32_t act, void* workspace, size_t* workspace_bytes, const tp_matrix* Y,
                 void* stream);

/*
 * tp_mlp without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, hosts
 * that forbid allocation). Same arguments, result and kernels as tp_mlp; the
 * intermediate and the partials live in a scratch array built into the
 * library, one copy per GPU, tp_mlp_noalloc_max_scratch() bytes (64 MiB),
 * held from the loading of the library until the process ends. The call
 * allocates and frees nothing. Shapes whose tp_mlp workspace exceeds that
 * size return TP_ERR_TOO_LARGE with nothing enqueued. The scratch array's
 * device address is looked up on the first call made with a device current;
 * that device must be the one `stream` belongs to. Every call on one GPU
 * shares that GPU's array and leaves its contents behind: calls that may run
 * at the same time on one GPU (different streams, or host threads) race
 * and must be ordered by the caller; calls on one stream are ordered by it.
 */
tp_status tp_mlp_noalloc(const tp_matrix* X, const tp_matrix* W1, const tp_matrix* W2, int32_t N, int32_t s0,
                         int32_t ns, int32_t act, const tp_matrix* Y, void* stream);

/* Bytes of the per-GPU scratch array tp_mlp_noalloc uses. */
size_t tp_mlp_noalloc_max_scratch(void);

/*
 * Backward passes. The pages pair every forward collective with a backward
 * one ([TP-topic] "Megatron-LM Tensor Parallelism": the identity operator of
 * the forward pass becomes an all-reduce in the backward pass and vice versa;
 * "Communication Optimization": the backward pass all-reduces gradients with
 * the forward volume; "Memory Distribution": each shard computes the
 * gradients of its own 1/N of the weights). Given dY, the gradient of a loss
 * with respect to the forward output, these return the gradients with
 * respect to X and the executed shards of W. Gradients are fp32-accumulated;
 * dtype rules, layouts and errors are those of the forward calls. Either
 * output descriptor may be NULL to skip that gradient (not both).
 */

/*
 * Backward of tp_col_linear with act = NONE. X is replicated in the forward
 * pass, so its gradient is a sum over shards (the backward all-reduce):
 *     dX  = sum_j P_j,   P_j = dY_j W_s^T   (fp32 partials, j = s - s0)
 *     dW_j = X^T dY_j                       (the gradient of W_s)
 *   X, W   as in tp_col_linear.
 *   dY     logical [M, ns*Nout/N], the layout of tp_col_linear's Y (dtype of X).
 *   dXp    TP_F32 partials, rows = M, cols = K, P_j at ptr + j*shard_stride
 *          (shard_stride may be 0 only when ns = 1); sum them with
 *          tp_reduce_partials(axis = TP_SPLIT_ROWS).
 *   dW     logical [K, ns*Nout/N], TP_F32 or TP_BF16: shard_stride 0 puts dW_j
 *          at columns j*Nout/N; > 0 puts it at ptr + j*shard_stride.
 */
tp_status tp_col_linear_backward(const tp_matrix* X, const tp_matrix* W, const tp_matrix* dY, int32_t N,
                                 int32_t s0, int32_t ns, const tp_matrix* dXp, const tp_matrix* dW,
                                 void* stream);

/*
 * Backward of tp_row_linear. The forward output is the sum of the partials,
 * so every shard receives the whole dY, and the gradient of each input block
 * stays on its shard (no exchange):
 *     dX_j = dY W_s^T,   dW_j = X_s^T dY,   j = s - s0
 *   X, W   as in tp_row_linear.
 *   dY     [M, Nout], dtype of X, shard_stride 0.
 *   dX     logical [M, ns*K/N], TP_F32 or TP_BF16: shard_stride 0 puts dX_j at
 *          columns j*K/N (the layout of X's executed blocks); > 0 at
 *          ptr + j*shard_stride.
 *   dW     logical [ns*K/N, Nout], TP_F32 or TP_BF16: shard_stride 0 puts dW_j
 *          at rows j*K/N; > 0 at ptr + j*shard_stride.
 */
tp_status tp_row_linear_backward(const tp_matrix* X, const tp_matrix* W, const tp_matrix* dY, int32_t N,
                                 int32_t s0, int32_t ns, const tp_matrix* dX, const tp_matrix* dW,
                                 void* stream);

/*
 * Backward of tp_mlp. With Z_s = X W1_s and H_s = act(Z_s):
 *     dH_s = dY W2_s^T,  dZ_s = dH_s * act'(Z_s)  (elementwise),
 *     dW2_s = H_s^T dY,  dW1_s = X^T dZ_s,
 *     dX = sum_s dZ_s W1_s^T                  (fp32, ascending s)
 * H_s and Z_s are recomputed from X (they are not kept by tp_mlp). With bf16
 * inputs Z_s, H_s and dZ_s are rounded to bf16 before they feed a product.
 *   X, W1, W2, act, workspace, *workspace_bytes   as in tp_mlp (the workspace
 *          holds Z, H, dZ and the partials of dX; NULL queries its size).
 *   dY     [M, Dout], dtype of X, shard_stride 0.
 *   dX     [M, d], TP_F32, shard_stride 0, or NULL.
 *   dW1    logical [d, ns*F/N] as dW of tp_col_linear_backward, or NULL.
 *   dW2    logical [ns*F/N, Dout] as dW of tp_row_linear_backward, or NULL.
 */
tp_status tp_mlp_backward(const tp_matrix* X, const tp_matrix* W1, const tp_matrix* W2, const tp_matrix* dY,
                          int32_t N, int32_t s0, int32_t ns, int32_t act, void* workspace,
                          size_t* workspace_bytes, const tp_matrix* dX, const tp_matrix* dW1,
                          const tp_matrix* dW2, void* stream);

/*
 * Attention for the heads of the executed shards, the step between the
 * column-parallel QKV projection and the row-parallel output projection
 * ([TP-topic] figure "Tensor Parallelism — Split Layers Across GPUs", panel
 * "Attention Head Parallelism": each shard computes full attention for its
 * own subset of heads, which do not interact; under grouped-query attention
 * the query heads are split evenly and the shared key/value heads
 * replicated; "Megatron-LM Tensor Parallelism", attention layer splitting).
 * Shard s holds hq = heads/N query heads and hkv = kv_heads/N key/value heads
 * (hkv = 1, a replicated head, when kv_heads < N). For every query head h of
 * every executed shard and every sequence of seq_len consecutive tokens:
 *     O_h = softmax(Q_h K_g^T / sqrt(head_dim)) V_g,   g = h / (hq / hkv),
 * causal (token i attends to tokens 0..i of its sequence) when causal = 1.
 *   QKV  logical [M, ns*(hq + 2 hkv)*head_dim], the layout of tp_col_linear's
 *        Y: shard j's block holds its query heads, then its key heads, then
 *        its value heads, head-major, head_dim columns each.
 *   A    logical [M, ns*hq*head_dim], dtype of QKV; shard j's block holds its
 *        query heads' outputs in order: the X of the row-parallel W_o.
 *   M must be a multiple of seq_len. bf16 with head_dim 64 or 128 runs on the
 *   matrix cores (fp32 scores and softmax; each probability enters the
 *   product with V as a bf16 pair, its rounded value and rounded remainder,
 *   which hold it to about 2^-17 of itself; normalized by the fp32 sum of the
 *   probabilities); other cases take an fp32 element-wise kernel limited to seq_len <= 8192
 *   (TP_ERR_TOO_LARGE beyond). At most 65535 executed query heads (ns*hq) and
 *   65535 sequences per call (TP_ERR_TOO_LARGE beyond).
 */
tp_status tp_attention(const tp_matrix* QKV, int32_t N, int32_t s0, int32_t ns, int32_t heads, int32_t kv_heads,
                       int32_t head_dim, int64_t seq_len, int32_t causal, const tp_matrix* A, void* stream);

/*
 * The sequence-parallel boundary after a row-parallel layer ([TP-topic]
 * "Sequence Parallelism Extension": LayerNorm and dropout run on token
 * shards, each shard holding M/N of the M tokens; the all-reduce of the
 * row-parallel partials becomes a reduce-scatter, and an all-gather restores
 * the full sequence before attention). For the tokens of shards
 * s = s0 .. s0+ns-1 (token shard s owns rows s*M/N .. (s+1)*M/N - 1), with i
 * the executed token row (i = 0 .. ns*M/N - 1, global row s0*M/N + i):
 *     x_i  = R_i + keep_i * (P_0 + ... + P_{n-1})_i / (1 - p_drop)
 *            (the reduce-scatter: the fp32 partial sum of this token slice
 *             only, in ascending order; then dropout and the residual add)
 *     X1_i = x_i                                  (the new residual stream)
 *     Y_i  = (x_i - mean(x_i)) / sqrt(var(x_i) + eps) * gamma + beta
 * with mean and var the mean and biased variance over the d features of the
 * row, computed in fp32.
 *   P      n blocks of [M, d], TP_F32, block t at ptr + t*shard_stride (the
 *          output of tp_row_linear over all tokens); shard_stride may be 0
 *          only when n = 1. N | M.
 *   R      NULL (no residual) or logical [ns*M/N, d], TP_F32 or TP_BF16: the
 *          residual rows of the executed token shards. shard_stride 0: one
 *          matrix, token shard j at rows j*M/N; > 0: the [M/N, d] block of
 *          token shard j at ptr + j*shard_stride.
 *   keep   NULL (no dropout) or device bytes [ns*M/N, d], row stride d, each
 *          0 (dropped) or 1 (kept); the mask is an input, drawn by the caller.
 *   p_drop the drop probability, 0 <= p_drop < 1 (checked only with keep).
 *   gamma, beta  device fp32 [d].  eps  >= 0.
 *   X1     NULL or logical [ns*M/N, d], TP_F32, layout as R.
 *   Y      logical [ns*M/N, d], TP_F32 or TP_BF16, layout as R.
 * No output may overlap an input (an in-place residual update is rejected
 * with TP_ERR_ALIAS). Rows of up to 16384 aligned features stay in registers
 * (the partials are read once); wider or unaligned rows take a kernel that
 * reads them three times.
 */
tp_status tp_sp_layernorm(const tp_matrix* P, int32_t n, const tp_matrix* R, const uint8_t* keep, float p_drop,
                          const float* gamma, const float* beta, float eps, int32_t N, int32_t s0, int32_t ns,
                          const tp_matrix* X1, const tp_matrix* Y, void* stream);

/* A static, human-readable name for a status code (never NULL). */
const char* tp_status_string(int32_t status);

/* Version of this interface: (major << 16) | minor. 1.1 added tp_sp_layernorm and TP_SPLIT_TOKENS. */
int32_t tp_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TP_H */
