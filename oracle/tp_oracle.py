"""Oracle for the tensor-parallel sharded linear layer Y = X W (test infrastructure).

TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the CPU
baseline leg of the benchmark may import this module; the product path (the
HIP library and its Python binding) never does, and this module imports
nothing from it.

Everything here is plain float64 numpy, computed shard by shard in the order
the tensor-parallelism pages describe, so that the split, concatenation and
summation steps are themselves checked and not only the final product.
Inputs are the exact values the GPU receives (bfloat16 or float32 values held
in float32 arrays); they are widened to float64 before any arithmetic.
The one library primitive used as a step is the float64 matrix product
``numpy.matmul``; the Gaussian error function comes from ``scipy.special.erf``.

Sources (the web pages on tensor parallelism this library implements):
  [TP-topic]   "Tensor Parallelism" topic page, chipfoundryservices.com
  [AI-gloss]   "Tensor Parallelism" entry, AI Glossary, aiforbusinessandlife.com
  [DLwPT]      "Tensor parallelism" concept page, Deep Learning with PyTorch 2e (liveBook)

Pins (tests/test_oracle.py): the worked example of [AI-gloss] "Worked example"
(fixture tests/golden/worked_example.json), brute force against pure-Python
loops on small integer inputs, the split invariants for every shard count
dividing the split dimension, textbook values of the normal CDF for GeLU and
an independent Taylor-series error function, and mutation tests that plant
plausible mistakes here and check that a pin catches each one.
The backward functions are pinned against central finite differences of the
forward functions above, against the unsharded gradients for every shard
count, against brute force, and by their own mutation tests.
Readings where the pages are silent: W is [in, out] row-major and Y = X W;
blocks are contiguous and shard s takes the s-th; N must divide the split
dimension; the MLP activation is the exact GeLU x * Phi(x); the intermediate
H is kept in float64 here (the GPU rounds it to bfloat16); partial sums are
added in ascending shard order.
"""
from __future__ import annotations

import numpy as np
from scipy.special import erf as _erf

__all__ = [
    "widen",
    "matmul",
    "col_block",
    "row_block",
    "x_block",
    "concat_cols",
    "reduce_sum",
    "gelu",
    "apply_act",
    "col_shard_outputs",
    "col_linear",
    "row_partials",
    "row_linear",
    "mlp_shard_partials",
    "mlp",
    "transpose",
    "gelu_grad",
    "act_grad",
    "split_cols",
    "col_linear_backward",
    "row_linear_backward",
    "mlp_backward",
    "attention_shard",
    "attention",
    "shard_qkv_columns",
    "token_rows",
    "layernorm",
    "sp_layernorm",
    "all_gather_rows",
]

ACTS = ("none", "gelu")


def widen(a) -> np.ndarray:
    """Exact widening of the received values (float32 / bfloat16 held in float32) to float64."""
    return np.asarray(a, dtype=np.float64)


def matmul(a, b) -> np.ndarray:
    """C[m, n] = sum_k A[m, k] * B[k, n] in float64.

    The definition of the matrix product named by [DLwPT] "Related concepts"
    (entries of the result are sums of products of rows of the first factor
    with columns of the second); the float64 library product is the step.
    """
    a = widen(a)
    b = widen(b)
    if a.ndim != 2 or b.ndim != 2 or a.shape[1] != b.shape[0]:
        raise ValueError(f"matmul shape mismatch {a.shape} x {b.shape}")
    return a @ b


def _check_split(dim: int, n: int, what: str) -> int:
    """Even split only: each shard owns dim / n contiguous indices ([TP-topic] figure, '[d, d/N]')."""
    if n < 1 or dim % n != 0:
        raise ValueError(f"{what}: {n} shards do not evenly divide {dim}")
    return dim // n


def col_block(w, n: int, s: int) -> np.ndarray:
    """W_s of the column-wise split W = [W_1, ..., W_N]: columns s*Nout/N .. (s+1)*Nout/N - 1.

    [TP-topic] "Column-Wise Parallelism"; [AI-gloss] "How it works" (split W by output columns).
    """
    w = np.asarray(w)
    width = _check_split(w.shape[1], n, "column split")
    return w[:, s * width:(s + 1) * width]


def row_block(w, n: int, s: int) -> np.ndarray:
    """W_s of the row-wise split W = [W_1; ...; W_N]: rows s*K/N .. (s+1)*K/N - 1.

    [TP-topic] "Row-Wise Parallelism" (W stacked vertically, input split to match).
    """
    w = np.asarray(w)
    height = _check_split(w.shape[0], n, "row split")
    return w[s * height:(s + 1) * height, :]


def x_block(x, n: int, s: int) -> np.ndarray:
    """X_s: the input columns matching row block s of W ([TP-topic] "Row-Wise Parallelism")."""
    x = np.asarray(x)
    width = _check_split(x.shape[1], n, "input split")
    return x[:, s * width:(s + 1) * width]


def concat_cols(blocks) -> np.ndarray:
    """Place column-shard outputs side by side, block 0 first.

    The combine step of the column split ([TP-topic] "Column-Wise Parallelism",
    all-gather / concatenation; [AI-gloss] "Check your understanding": outputs
    at different coordinates are concatenated).
    """
    return np.concatenate([widen(b) for b in blocks], axis=1)


def reduce_sum(partials) -> np.ndarray:
    """Sum partial outputs that share coordinates, in ascending shard order, float64.

    The combine step of the row split ([TP-topic] "Row-Wise Parallelism",
    Y = sum_i Y_i via all-reduce; [AI-gloss] "Check your understanding":
    contributions to the same coordinates are added).
    """
    partials = list(partials)
    if not partials:
        raise ValueError("reduce_sum needs at least one partial")
    total = widen(partials[0]).copy()
    for p in partials[1:]:
        total = total + widen(p)
    return total


def gelu(x) -> np.ndarray:
    """Exact GeLU: x * Phi(x) = 0.5 * x * (1 + erf(x / sqrt(2))), float64.

    The pages name only an activation applied to each shard on its own
    ([TP-topic] "Megatron-LM Tensor Parallelism", MLP splitting); the exact
    erf form of GeLU is the reading taken here.
    """
    x = widen(x)
    return 0.5 * x * (1.0 + _erf(x / np.sqrt(2.0)))


def apply_act(y, act: str) -> np.ndarray:
    if act == "none":
        return widen(y)
    if act == "gelu":
        return gelu(y)
    raise ValueError(f"unknown activation {act!r}")


def col_shard_outputs(x, w, n: int, act: str = "none", s0: int = 0, ns: int | None = None):
    """Y_s = act(X W_s) for s in s0 .. s0+ns-1 ([TP-topic] "Column-Wise Parallelism").

    X is replicated to every shard; each shard's block of output columns is
    computed independently (the activation, being elementwise, needs no exchange).
    """
    ns = n - s0 if ns is None else ns
    return [apply_act(matmul(x, col_block(w, n, s)), act) for s in range(s0, s0 + ns)]


def col_linear(x, w, n: int, act: str = "none", s0: int = 0, ns: int | None = None) -> np.ndarray:
    """Column-parallel linear: concatenation of the column-shard outputs."""
    return concat_cols(col_shard_outputs(x, w, n, act, s0, ns))


def row_partials(x, w, n: int, s0: int = 0, ns: int | None = None):
    """P_s = X_s W_s for s in s0 .. s0+ns-1 ([TP-topic] "Row-Wise Parallelism")."""
    ns = n - s0 if ns is None else ns
    return [matmul(x_block(x, n, s), row_block(w, n, s)) for s in range(s0, s0 + ns)]


def row_linear(x, w, n: int, s0: int = 0, ns: int | None = None) -> np.ndarray:
    """Row-parallel linear: sum of the partials."""
    return reduce_sum(row_partials(x, w, n, s0, ns))


def mlp_shard_partials(x, w1, w2, n: int, act: str = "gelu", s0: int = 0, ns: int | None = None):
    """Per-shard outputs of the Megatron MLP pair ([TP-topic] "Megatron-LM Tensor Parallelism").

    Shard s applies the column block s of W1, the activation on its own
    columns, then the row block s of W2; both blocks cover the same slice
    s*F/N .. (s+1)*F/N of the intermediate width, which is why the
    intermediate H never leaves its shard ([TP-topic] "Row-Wise Parallelism":
    the input is already split by the preceding column-wise layer).
    H stays float64 here.
    """
    ns = n - s0 if ns is None else ns
    out = []
    for s in range(s0, s0 + ns):
        h_s = apply_act(matmul(x, col_block(w1, n, s)), act)
        out.append(matmul(h_s, row_block(w2, n, s)))
    return out


def mlp(x, w1, w2, n: int, act: str = "gelu", s0: int = 0, ns: int | None = None) -> np.ndarray:
    """Y = sum_s act(X W1_s) W2_s, the single sum closing the MLP pair."""
    return reduce_sum(mlp_shard_partials(x, w1, w2, n, act, s0, ns))


# ----------------------------------------------------------------------------- backward passes
#
# The pages pair each forward collective with one in the backward pass
# ([TP-topic] "Megatron-LM Tensor Parallelism": identity operators of the
# forward pass become all-reduces in the backward pass and the reverse;
# "Communication Optimization": gradients are all-reduced with the forward
# volume; "Memory Distribution": each shard computes the gradients of its own
# 1/N of the weights). They do not write the gradients out; the ones below are
# the chain rule for Y = X W: with dY the gradient of a loss with respect to Y,
# the gradient with respect to X is dY W^T and with respect to W is X^T dY.


def transpose(a) -> np.ndarray:
    """The transposed matrix (rows become columns), float64."""
    return widen(a).T


def gelu_grad(x) -> np.ndarray:
    """Derivative of the exact GeLU: Phi(x) + x phi(x), phi(x) = exp(-x^2/2) / sqrt(2 pi), float64."""
    x = widen(x)
    return 0.5 * (1.0 + _erf(x / np.sqrt(2.0))) + x * np.exp(-0.5 * x * x) / np.sqrt(2.0 * np.pi)


def act_grad(z, act: str) -> np.ndarray:
    if act == "none":
        return np.ones_like(widen(z))
    if act == "gelu":
        return gelu_grad(z)
    raise ValueError(f"unknown activation {act!r}")


def split_cols(y, ns: int):
    """The ns equal column blocks of y, in order (the inverse of concat_cols)."""
    y = widen(y)
    width = _check_split(y.shape[1], ns, "columns")
    return [y[:, j * width:(j + 1) * width] for j in range(ns)]


def col_linear_backward(x, w, dy, n: int, s0: int = 0, ns: int | None = None):
    """Backward of the column split (no activation).

    X reaches every shard unchanged in the forward pass, so its gradient is the
    sum of the shards' contributions (the backward all-reduce):
        dX = sum_j P_j, P_j = dY_j W_s^T;   dW_s = X^T dY_j   (j = s - s0).
    dy is [M, ns*Nout/N] (shard j's block at columns j*Nout/N).
    Returns (the partials P_j, the weight-gradient blocks dW_s).
    """
    ns = n - s0 if ns is None else ns
    dys = split_cols(dy, ns)
    partials = [matmul(dys[j], transpose(col_block(w, n, s0 + j))) for j in range(ns)]
    dws = [matmul(transpose(x), dys[j]) for j in range(ns)]
    return partials, dws


def row_linear_backward(x, w, dy, n: int, s0: int = 0, ns: int | None = None):
    """Backward of the row split.

    The forward output is the sum of the partials, so every shard receives the
    whole dY, and each shard's input block keeps its own gradient (no exchange):
        dX_s = dY W_s^T,   dW_s = X_s^T dY.
    Returns (the input-gradient blocks dX_s, the weight-gradient blocks dW_s).
    """
    ns = n - s0 if ns is None else ns
    dxs = [matmul(dy, transpose(row_block(w, n, s))) for s in range(s0, s0 + ns)]
    dws = [matmul(transpose(x_block(x, n, s)), dy) for s in range(s0, s0 + ns)]
    return dxs, dws


def mlp_backward(x, w1, w2, dy, n: int, act: str = "gelu", s0: int = 0, ns: int | None = None):
    """Backward of the Megatron MLP pair, shard by shard, float64 throughout.

    With Z_s = X W1_s and H_s = act(Z_s) (recomputed here):
        dH_s = dY W2_s^T  (the row-split layer: dY reaches every shard),
        dZ_s = dH_s * act'(Z_s)  (elementwise, inside the shard),
        dW2_s = H_s^T dY,  dW1_s = X^T dZ_s,
        dX = sum_s dZ_s W1_s^T  (the column-split layer: the backward all-reduce,
             ascending shard order).
    Returns (dX, dW1 as the concatenation of the dW1_s, dW2 as the dW2_s stacked by rows).
    """
    ns = n - s0 if ns is None else ns
    partials, dw1, dw2 = [], [], []
    dy = widen(dy)
    for s in range(s0, s0 + ns):
        w1s, w2s = col_block(w1, n, s), row_block(w2, n, s)
        z = matmul(x, w1s)
        h = apply_act(z, act)
        dz = matmul(dy, transpose(w2s)) * act_grad(z, act)
        dw2.append(matmul(transpose(h), dy))
        dw1.append(matmul(transpose(x), dz))
        partials.append(matmul(dz, transpose(w1s)))
    return reduce_sum(partials), concat_cols(dw1), np.vstack(dw2)


# ----------------------------------------------------------------------------- attention per head subset
#
# [TP-topic] figure "Tensor Parallelism — Split Layers Across GPUs", panel
# "Attention Head Parallelism": the heads are split evenly over the shards and
# each shard computes full attention for its own heads (the heads do not
# interact); with grouped-query attention the query heads are split evenly and
# the shared key/value heads are replicated. Section "Megatron-LM Tensor
# Parallelism": the Q, K, V projections are split by columns (so each shard's
# block of the fused QKV output holds its own heads) and the output projection
# by rows. Readings taken where the pages are silent: a shard's QKV block holds
# its query heads, then its key heads, then its value heads, head-major with
# head_dim columns each; scores are scaled by 1/sqrt(head_dim); the model is a
# decoder (causal: a token attends to itself and earlier tokens of its own
# sequence) unless causal is False; tokens are consecutive sequences of
# seq_len tokens; query head h of a shard uses key/value head h // (hq / hkv).


def _softmax_rows(s) -> np.ndarray:
    """exp(s - max) / sum, row by row; -inf entries contribute zero."""
    m = np.max(s, axis=1, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=1, keepdims=True)


def attention_shard(qkv_block, hq: int, hkv: int, head_dim: int, seq_len: int, causal: bool = True) -> np.ndarray:
    """Attention of one shard's heads: qkv_block [M, (hq + 2 hkv) head_dim] -> [M, hq head_dim], float64."""
    qkv_block = widen(qkv_block)
    m_rows = qkv_block.shape[0]
    if qkv_block.shape[1] != (hq + 2 * hkv) * head_dim:
        raise ValueError("QKV block width does not match the head counts")
    if hkv < 1 or hq % hkv != 0:
        raise ValueError("query heads must be a multiple of key/value heads")
    if seq_len < 1 or m_rows % seq_len != 0:
        raise ValueError("tokens must be whole sequences")
    group = hq // hkv
    out = np.zeros((m_rows, hq * head_dim))
    koff, voff = hq * head_dim, (hq + hkv) * head_dim
    for r0 in range(0, m_rows, seq_len):
        rows = slice(r0, r0 + seq_len)
        for h in range(hq):
            kv = h // group
            q = qkv_block[rows, h * head_dim:(h + 1) * head_dim]
            k = qkv_block[rows, koff + kv * head_dim:koff + (kv + 1) * head_dim]
            v = qkv_block[rows, voff + kv * head_dim:voff + (kv + 1) * head_dim]
            s = matmul(q, transpose(k)) / np.sqrt(head_dim)
            if causal:
                s = np.where(np.tril(np.ones((seq_len, seq_len), dtype=bool)), s, -np.inf)
            out[rows, h * head_dim:(h + 1) * head_dim] = matmul(_softmax_rows(s), v)
    return out


def _heads_per_shard(heads: int, kv_heads: int, n: int):
    hq = _check_split(heads, n, "query heads")
    if kv_heads >= n:
        hkv = _check_split(kv_heads, n, "key/value heads")
    else:
        if kv_heads < 1 or n % kv_heads != 0:
            raise ValueError("shards must split the key/value heads evenly or replicate them evenly")
        hkv = 1
    return hq, hkv


def attention(qkv, n: int, heads: int, kv_heads: int, head_dim: int, seq_len: int, causal: bool = True,
              s0: int = 0, ns: int | None = None) -> np.ndarray:
    """Attention of the executed shards, concatenated: qkv [M, ns * block] (shard j's block at
    columns j * block, block = (hq + 2 hkv) head_dim) -> [M, ns * hq * head_dim]."""
    ns = n - s0 if ns is None else ns
    hq, hkv = _heads_per_shard(heads, kv_heads, n)
    blocks = split_cols(qkv, ns)
    return concat_cols([attention_shard(b, hq, hkv, head_dim, seq_len, causal) for b in blocks])


def shard_qkv_columns(heads: int, kv_heads: int, head_dim: int, n: int, s: int) -> np.ndarray:
    """Column indices, into an unsharded [Q heads | K heads | V heads] projection output, of shard s's
    QKV block: its query heads, then its key/value heads (a replicated copy when kv_heads < n)."""
    hq, hkv = _heads_per_shard(heads, kv_heads, n)
    group = heads // kv_heads
    q_heads = list(range(s * hq, (s + 1) * hq))
    kv = sorted({h // group for h in q_heads})
    if len(kv) != hkv:
        raise ValueError("a shard's query heads must share its key/value heads")
    cols = []
    for h in q_heads:
        cols += list(range(h * head_dim, (h + 1) * head_dim))
    for base in (heads, heads + kv_heads):
        for g in kv:
            cols += list(range((base + g) * head_dim, (base + g + 1) * head_dim))
    return np.array(cols)


# ----------------------------------------------------------------------------- sequence parallelism
#
# [TP-topic] "Sequence Parallelism Extension": LayerNorm and Dropout are not
# split by tensor parallelism, so the tokens are split over the shards for
# them (each shard processes a subset of the tokens), with an all-gather
# before attention (every token attends to every token) and a reduction after
# it. On one device the all-reduce of the row-parallel partials splits into a
# reduce-scatter (each token shard sums the partials of its own tokens, in
# ascending shard order) and an all-gather (the token shards side by side
# again). Readings: token shard s owns rows s*M/N .. (s+1)*M/N - 1; LayerNorm
# normalizes each token over the hidden dimension with the biased variance,
# (x - mean) / sqrt(var + eps) * gamma + beta; dropout is inverted dropout
# with a caller-supplied 0/1 keep mask, applied to the reduced partials before
# the residual is added (x = residual + keep * sum / (1 - p)).


def token_rows(m: int, n: int, s: int) -> slice:
    """The token rows of token shard s of n (contiguous, even split)."""
    rows = _check_split(m, n, "tokens")
    return slice(s * rows, (s + 1) * rows)


def layernorm(x, gamma, beta, eps: float) -> np.ndarray:
    """Per-row LayerNorm over the last dimension, float64, biased variance."""
    x = widen(x)
    mean = np.mean(x, axis=1, keepdims=True)
    var = np.mean((x - mean) ** 2, axis=1, keepdims=True)
    return (x - mean) / np.sqrt(var + eps) * widen(gamma)[None, :] + widen(beta)[None, :]


def sp_layernorm(partials, residual, keep, p_drop: float, gamma, beta, eps: float, n: int, s0: int = 0,
                 ns: int | None = None):
    """Reduce-scatter, dropout, residual add and LayerNorm for the tokens of shards s0 .. s0+ns-1.

    partials: the row-parallel fp32 partials [M, d] (a list, summed in order);
    residual: [M, d] or None; keep: 0/1 [M, d] or None (no dropout).
    Returns (x, y) for the executed token rows: x the pre-norm sum (the new
    residual stream), y the normalized output.
    """
    ns = n - s0 if ns is None else ns
    partials = list(partials)
    m = widen(partials[0]).shape[0]
    rows = slice(token_rows(m, n, s0).start, token_rows(m, n, s0 + ns - 1).stop)
    x = reduce_sum([widen(pj)[rows] for pj in partials])
    if keep is not None:
        x = x * widen(keep)[rows] / (1.0 - p_drop)
    if residual is not None:
        x = x + widen(residual)[rows]
    return x, layernorm(x, gamma, beta, eps)


def all_gather_rows(blocks) -> np.ndarray:
    """Token shards stacked back in order (the all-gather before attention)."""
    return np.vstack([widen(b) for b in blocks])
