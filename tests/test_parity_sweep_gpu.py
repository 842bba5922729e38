"""GPU parity over a seeded sweep of shapes, against the float64 oracle.

Each case draws its own sizes from a fixed seed: the token count M crosses the
skinny (M <= 32), large-tile and partial-tile paths; K, the shard width and the
shard count N take values that leave ragged k tails and partial column tiles;
a few cases use sizes that are not multiples of 8 and so take the element-wise
path. Column-parallel, row-parallel (partials, then the ascending-order sum),
the MLP pair and the backward pass of each are checked element by element
within the bars of tests/parity.py, and so are attention (head counts,
grouped key/value heads, head sizes, sequence lengths and counts, causal or
not, shard subsets) and the sequence-parallel LayerNorm (token and shard
counts, widths, partial counts, dropout rates, dtypes).
"""
import numpy as np
import pytest
import torch

import oracle
import tensor_sharded_linear_amd as tp
from synthetic import normal_bf16
from parity import assert_close, bf16_tensor, host, note

pytestmark = pytest.mark.gpu

CASES = 12


def draw(case: int, kind: int):
    """Sizes of one case: (M, K, width, N, s0, ns, act, out_dtype, aligned)."""
    rng = np.random.default_rng([7000 + kind, case])
    aligned = case % 4 != 3
    M = int(rng.choice([int(rng.integers(1, 33)), int(rng.integers(33, 700))]))
    N = int(rng.integers(1, 5))
    step = 8 if aligned else 1
    K = step * int(rng.integers(1, 1100 // step + 1))
    width = step * int(rng.integers(1, 400 // step + 1))
    s0 = int(rng.integers(0, N))
    ns = int(rng.integers(1, N - s0 + 1))
    act = "gelu" if rng.random() < 0.5 else "none"
    out_dtype = torch.bfloat16 if rng.random() < 0.5 else torch.float32
    return M, K, width, N, s0, ns, act, out_dtype, aligned


@pytest.mark.parametrize("case", range(CASES))
def test_sweep_col(case):
    M, K, width, N, s0, ns, act, out_dtype, aligned = draw(case, 0)
    xb, x = normal_bf16((M, K), 1.0, 7100 + case, 0)
    wb, w = normal_bf16((K, width * N), 0.02, 7100 + case, 1)
    note(f"sweep col case={case} M={M} K={K} width={width} N={N} s0={s0} ns={ns} act={act} out={out_dtype}")
    got = host(tp.col_linear(bf16_tensor(xb), bf16_tensor(wb), N, s0=s0, ns=ns, act=act, out_dtype=out_dtype))
    ref = np.concatenate(oracle.col_shard_outputs(x, w, N, act, s0=s0, ns=ns), axis=1)
    assert_close(got, ref, f"col case {case}", stored_bf16=out_dtype == torch.bfloat16)


@pytest.mark.parametrize("case", range(CASES))
def test_sweep_row(case):
    M, Kb, width, N, s0, ns, _, _, aligned = draw(case, 1)
    K = Kb * N  # the split dimension must divide evenly
    nout = width
    xb, x = normal_bf16((M, K), 1.0, 7200 + case, 0)
    wb, w = normal_bf16((K, nout), 0.02, 7200 + case, 1)
    note(f"sweep row case={case} M={M} K={K} Nout={nout} N={N} s0={s0} ns={ns}")
    P = tp.row_linear(bf16_tensor(xb), bf16_tensor(wb), N, s0=s0, ns=ns)
    ph = host(P)
    refs = oracle.row_partials(x, w, N)[s0:s0 + ns]
    for j, p in enumerate(refs):
        assert_close(ph[j], p, f"row case {case} partial {s0 + j}")
    assert_close(host(tp.reduce_partials(P)), oracle.reduce_sum(refs), f"row case {case} sum")


@pytest.mark.parametrize("case", range(CASES))
def test_sweep_mlp(case):
    M, d, fw, N, s0, ns, act, _, aligned = draw(case, 2)
    F = fw * N
    xb, x = normal_bf16((M, d), 1.0, 7300 + case, 0)
    w1b, w1 = normal_bf16((d, F), 0.02, 7300 + case, 1)
    w2b, w2 = normal_bf16((F, d), 0.02, 7300 + case, 2)
    note(f"sweep mlp case={case} M={M} d={d} F={F} N={N} s0={s0} ns={ns} act={act}")
    got = host(tp.mlp(bf16_tensor(xb), bf16_tensor(w1b), bf16_tensor(w2b), N, s0=s0, ns=ns, act=act))
    assert_close(got, oracle.mlp(x, w1, w2, N, act, s0, ns), f"mlp case {case}")


# ----------------------------------------------------------------------------- backward passes

BACKWARD_CASES = 8


@pytest.mark.parametrize("case", range(BACKWARD_CASES))
def test_sweep_col_backward(case):
    M, K, width, N, s0, ns, _, _, _ = draw(case, 3)
    xb, x = normal_bf16((M, K), 1.0, 7400 + case, 0)
    wb, w = normal_bf16((K, width * N), 0.02, 7400 + case, 1)
    yb, dy = normal_bf16((M, width * ns), 1.0, 7400 + case, 2)
    note(f"sweep col backward case={case} M={M} K={K} width={width} N={N} s0={s0} ns={ns}")
    P, G = tp.col_linear_backward(bf16_tensor(xb), bf16_tensor(wb), bf16_tensor(yb), N, s0, ns)
    partials, dws = oracle.col_linear_backward(x, w, dy, N, s0, ns)
    ph = host(P)
    for j in range(ns):
        assert_close(ph[j], partials[j], f"col backward case {case} dX partial {j}")
    assert_close(host(G), oracle.concat_cols(dws), f"col backward case {case} dW")


@pytest.mark.parametrize("case", range(BACKWARD_CASES))
def test_sweep_row_backward(case):
    M, Kb, nout, N, s0, ns, _, _, _ = draw(case, 4)
    K = Kb * N
    xb, x = normal_bf16((M, K), 1.0, 7500 + case, 0)
    wb, w = normal_bf16((K, nout), 0.02, 7500 + case, 1)
    yb, dy = normal_bf16((M, nout), 1.0, 7500 + case, 2)
    note(f"sweep row backward case={case} M={M} K={K} Nout={nout} N={N} s0={s0} ns={ns}")
    A, G = tp.row_linear_backward(bf16_tensor(xb), bf16_tensor(wb), bf16_tensor(yb), N, s0, ns)
    dxs, dws = oracle.row_linear_backward(x, w, dy, N, s0, ns)
    assert_close(host(A), oracle.concat_cols(dxs), f"row backward case {case} dX")
    assert_close(host(G), np.vstack(dws), f"row backward case {case} dW")


@pytest.mark.parametrize("case", range(BACKWARD_CASES))
def test_sweep_mlp_backward(case):
    M, d, fw, N, s0, ns, act, _, _ = draw(case, 5)
    F = fw * N
    xb, x = normal_bf16((M, d), 1.0, 7600 + case, 0)
    w1b, w1 = normal_bf16((d, F), 0.02, 7600 + case, 1)
    w2b, w2 = normal_bf16((F, d), 0.02, 7600 + case, 2)
    yb, dy = normal_bf16((M, d), 1.0, 7600 + case, 3)
    note(f"sweep mlp backward case={case} M={M} d={d} F={F} N={N} s0={s0} ns={ns} act={act}")
    dX, dW1, dW2 = tp.mlp_backward(bf16_tensor(xb), bf16_tensor(w1b), bf16_tensor(w2b), bf16_tensor(yb), N,
                                   s0=s0, ns=ns, act=act)
    rx, r1, r2 = oracle.mlp_backward(x, w1, w2, dy, N, act, s0, ns)
    assert_close(host(dX), rx, f"mlp backward case {case} dX")
    assert_close(host(dW1), r1, f"mlp backward case {case} dW1")
    assert_close(host(dW2), r2, f"mlp backward case {case} dW2")


# ----------------------------------------------------------------------------- attention and sequence parallelism

ATTN_CASES = 10


def draw_attention(case: int):
    """(heads, kv_heads, head_dim, n, s0, ns, seq_len, sequences, causal) of one attention case."""
    rng = np.random.default_rng([7700, case])
    n = int(rng.choice([1, 2, 4]))
    heads = n * int(rng.integers(1, 4))
    # key/value heads: a divisor of heads that is either split evenly or replicated (one per shard)
    options = [k for k in range(1, heads + 1) if heads % k == 0 and (k % n == 0 or (k < n and n % k == 0))]
    kv_heads = int(rng.choice(options))
    dh = int(rng.choice([64, 128]))
    s0 = int(rng.integers(0, n))
    ns = int(rng.integers(1, n - s0 + 1))
    seq_len = int(rng.integers(1, 600))
    sequences = int(rng.integers(1, 4))
    causal = bool(rng.random() < 0.7)
    return heads, kv_heads, dh, n, s0, ns, seq_len, sequences, causal


@pytest.mark.parametrize("case", range(ATTN_CASES))
def test_sweep_attention(case):
    from test_parity_attention_gpu import qkv_case

    heads, kv_heads, dh, n, s0, ns, L, B, causal = draw_attention(case)
    bits, q = qkv_case(B * L, heads, kv_heads, dh, n, ns, 7800 + case)
    note(f"sweep attention case={case} heads={heads} kv_heads={kv_heads} dh={dh} n={n} s0={s0} ns={ns} "
         f"L={L} B={B} causal={causal}")
    got = host(tp.attention(bf16_tensor(bits), n, heads, kv_heads, dh, L, causal, s0=s0, ns=ns))
    ref = oracle.attention(q, n, heads, kv_heads, dh, L, causal, s0, ns)
    assert_close(got, ref, f"attention case {case}", stored_bf16=True)


SP_CASES = 8


@pytest.mark.parametrize("case", range(SP_CASES))
def test_sweep_sp_layernorm(case):
    from test_parity_sp_gpu import run_case

    rng = np.random.default_rng([7900, case])
    N = int(rng.choice([1, 2, 4, 8]))
    M = N * int(rng.integers(1, 40))
    d = int(rng.choice([int(rng.integers(1, 300)), 4 * int(rng.integers(1, 1500))]))
    t = int(rng.integers(1, 9))
    s0 = int(rng.integers(0, N))
    ns = int(rng.integers(1, N - s0 + 1))
    p_drop = float(rng.choice([0.0, 0.1, 0.5]))
    r_bf16 = bool(rng.random() < 0.5)
    y_dtype = torch.bfloat16 if rng.random() < 0.5 else torch.float32
    run_case(8000 + case, t, M, d, N, s0, ns, p_drop=p_drop, r_bf16=r_bf16, y_dtype=y_dtype)
