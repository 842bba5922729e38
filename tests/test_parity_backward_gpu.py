"""GPU parity of the backward passes (through the C interface) against the float64 oracle.

Same method as test_parity_gpu.py: seeded synthetic inputs, the library on the
GPU and the oracle on the CPU on the same bits, compared exactly for
integer-valued inputs and within the bars of tests/parity.py otherwise.
Shapes span several 256 x 256 tiles with ragged tails, shard subsets,
shard-major stacks, the element-guarded path and the fp32 path; the
Megatron-size MLP backward is checked on sampled rows of dX and dW2 and
sampled columns of dW1, each of which the oracle computes exactly from the
inputs it depends on.
"""
import numpy as np
import pytest
import torch

import oracle
import tensor_sharded_linear_amd as tp
from synthetic import WORKLOADS, bf16_bits_from_f32, int_uniform_f32, normal_bf16, stratified_rows
from parity import assert_close, assert_exact, bf16_tensor, dev, f32_tensor, host, note

pytestmark = pytest.mark.gpu


def ints_bf16(shape, lo, hi, wid, tid):
    v = int_uniform_f32(shape, lo, hi, wid, tid)
    return bf16_bits_from_f32(v), v


# ----------------------------------------------------------------------------- column split


@pytest.mark.parametrize("M,K,width,N", [(300, 264, 136, 3), (64, 512, 256, 2), (257, 64, 40, 4)])
def test_col_backward_exact_integers(M, K, width, N):
    xb, x = ints_bf16((M, K), -1, 1, 1100 + M, 0)
    wb, w = ints_bf16((K, N * width), -1, 1, 1100 + M, 1)
    yb, dy = ints_bf16((M, N * width), -1, 1, 1100 + M, 2)
    note(f"col backward exact M={M} K={K} width={width} N={N}")
    P, G = tp.col_linear_backward(bf16_tensor(xb), bf16_tensor(wb), bf16_tensor(yb), N)
    partials, dws = oracle.col_linear_backward(x, w, dy, N)
    for j in range(N):
        assert_exact(host(P[j]), partials[j], f"dX partial {j}")
    assert_exact(host(G), oracle.concat_cols(dws), "dW")


def test_col_backward_float_subset_and_stacks():
    M, K, width, N, s0, ns = 520, 384, 200, 4, 1, 2
    xb, x = normal_bf16((M, K), 1.0, 1110, 0)
    wb, w = normal_bf16((K, N * width), 0.02, 1110, 1)
    yb, dy = normal_bf16((M, ns * width), 1.0, 1110, 2)
    X, W, dY = bf16_tensor(xb), bf16_tensor(wb), bf16_tensor(yb)
    partials, dws = oracle.col_linear_backward(x, w, dy, N, s0, ns)
    note("col backward float, shards 1..2 of 4, column-slice W")
    P, G = tp.col_linear_backward(X, W, dY, N, s0, ns)
    for j in range(ns):
        assert_close(host(P[j]), partials[j], f"dX partial {j}")
    assert_close(host(G), oracle.concat_cols(dws), "dW")
    note("col backward float, shard-major W and partitioned dY / dW")
    Ws = torch.stack([W[:, s * width:(s + 1) * width] for s in range(N)]).contiguous()
    dYp = torch.stack([dY[:, j * width:(j + 1) * width] for j in range(ns)]).contiguous()
    P2, G2 = tp.col_linear_backward(X, Ws, dYp, N, s0, ns, partitioned_dw=True, dw_dtype=torch.bfloat16)
    for j in range(ns):
        assert_close(host(P2[j]), partials[j], f"dX partial {j} (stacks)")
        assert_close(host(G2[j]), dws[j], f"dW block {j} (stacks, bf16)", stored_bf16=True)


# ----------------------------------------------------------------------------- row split


@pytest.mark.parametrize("M,K,Nout,N", [(300, 528, 392, 2), (600, 264, 520, 3)])
def test_row_backward_exact_integers(M, K, Nout, N):
    xb, x = ints_bf16((M, K), -1, 1, 1200 + M, 0)
    wb, w = ints_bf16((K, Nout), -1, 1, 1200 + M, 1)
    yb, dy = ints_bf16((M, Nout), -1, 1, 1200 + M, 2)
    note(f"row backward exact M={M} K={K} Nout={Nout} N={N}")
    A, G = tp.row_linear_backward(bf16_tensor(xb), bf16_tensor(wb), bf16_tensor(yb), N)
    dxs, dws = oracle.row_linear_backward(x, w, dy, N)
    assert_exact(host(A), oracle.concat_cols(dxs), "dX")
    assert_exact(host(G), np.vstack(dws), "dW")


def test_row_backward_float_subset_and_stacks():
    M, K, Nout, N, s0, ns = 400, 1024, 264, 4, 2, 2
    xb, x = normal_bf16((M, K), 1.0, 1210, 0)
    wb, w = normal_bf16((K, Nout), 0.02, 1210, 1)
    yb, dy = normal_bf16((M, Nout), 1.0, 1210, 2)
    X, W, dY = bf16_tensor(xb), bf16_tensor(wb), bf16_tensor(yb)
    dxs, dws = oracle.row_linear_backward(x, w, dy, N, s0, ns)
    note("row backward float, shards 2..3 of 4")
    A, G = tp.row_linear_backward(X, W, dY, N, s0, ns)
    assert_close(host(A), oracle.concat_cols(dxs), "dX")
    assert_close(host(G), np.vstack(dws), "dW")
    note("row backward float, shard-major X and W, partitioned outputs")
    kb = K // N
    Xs = torch.stack([X[:, s * kb:(s + 1) * kb] for s in range(N)]).contiguous()
    Ws = torch.stack([W[s * kb:(s + 1) * kb] for s in range(N)]).contiguous()
    A2, G2 = tp.row_linear_backward(Xs, Ws, dY, N, s0, ns, partitioned=True, dx_dtype=torch.bfloat16)
    for j in range(ns):
        assert_close(host(A2[j]), dxs[j], f"dX block {j} (stacks, bf16)", stored_bf16=True)
        assert_close(host(G2[j]), dws[j], f"dW block {j} (stacks)")


def test_backward_generic_path_and_fp32():
    # widths that are not multiples of 8 take the element-guarded kernel
    M, K, width, N = 37, 30, 10, 3
    xb, x = normal_bf16((M, K), 1.0, 1300, 0)
    wb, w = normal_bf16((K, N * width), 0.02, 1300, 1)
    yb, dy = normal_bf16((M, N * width), 1.0, 1300, 2)
    note("col backward, unaligned shapes")
    P, G = tp.col_linear_backward(bf16_tensor(xb), bf16_tensor(wb), bf16_tensor(yb), N)
    partials, dws = oracle.col_linear_backward(x, w, dy, N)
    for j in range(N):
        assert_close(host(P[j]), partials[j], f"unaligned dX partial {j}")
    assert_close(host(G), oracle.concat_cols(dws), "unaligned dW")
    # fp32 inputs: the exact fp32 path
    xf = int_uniform_f32((M, K), -3, 3, 1301, 0)
    wf = int_uniform_f32((K, N * width), -3, 3, 1301, 1)
    yf = int_uniform_f32((M, K), -3, 3, 1301, 2)
    note("row backward, fp32 exact")
    A, G = tp.row_linear_backward(f32_tensor(xf), f32_tensor(wf), f32_tensor(yf[:, :N * width]), N)
    dxs, dws = oracle.row_linear_backward(xf, wf, yf[:, :N * width], N)
    assert_exact(host(A), oracle.concat_cols(dxs), "fp32 dX")
    assert_exact(host(G), np.vstack(dws), "fp32 dW")


# ----------------------------------------------------------------------------- MLP pair


def test_mlp_backward_exact_integers_no_activation():
    M, d, F, N = 96, 64, 512, 4
    xb, x = ints_bf16((M, d), -1, 1, 1400, 0)
    w1b, w1 = ints_bf16((d, F), -1, 1, 1400, 1)
    w2b, w2 = ints_bf16((F, d), -1, 1, 1400, 2)
    yb, dy = ints_bf16((M, d), -1, 1, 1400, 3)
    note("mlp backward exact, act none")
    dX, dW1, dW2 = tp.mlp_backward(bf16_tensor(xb), bf16_tensor(w1b), bf16_tensor(w2b), bf16_tensor(yb), N,
                                   act="none")
    rx, r1, r2 = oracle.mlp_backward(x, w1, w2, dy, N, "none")
    assert_exact(host(dX), rx, "dX")
    assert_exact(host(dW1), r1, "dW1")
    assert_exact(host(dW2), r2, "dW2")


@pytest.mark.parametrize("M,d,F,N,s0,ns", [(300, 512, 2048, 4, 0, 4), (264, 256, 1536, 3, 1, 2),
                                           (256, 256, 1024, 1, 0, 1), (40, 512, 2048, 8, 0, 8)])
def test_mlp_backward_gelu(M, d, F, N, s0, ns):
    xb, x = normal_bf16((M, d), 1.0, 1500 + M, 0)
    w1b, w1 = normal_bf16((d, F), 0.02, 1500 + M, 1)
    w2b, w2 = normal_bf16((F, d), 0.02, 1500 + M, 2)
    yb, dy = normal_bf16((M, d), 1.0, 1500 + M, 3)
    note(f"mlp backward gelu M={M} d={d} F={F} N={N} s0={s0} ns={ns}")
    dX, dW1, dW2 = tp.mlp_backward(bf16_tensor(xb), bf16_tensor(w1b), bf16_tensor(w2b), bf16_tensor(yb), N,
                                   s0=s0, ns=ns)
    rx, r1, r2 = oracle.mlp_backward(x, w1, w2, dy, N, "gelu", s0, ns)
    assert_close(host(dX), rx, "dX")
    assert_close(host(dW1), r1, "dW1")
    assert_close(host(dW2), r2, "dW2")


def test_mlp_backward_workspace_off_the_vector_alignment():
    """A workspace 4 bytes past an aligned address: the recomputed pre-activation and the GeLU'
    product keep the large-tile kernel but store (and read) their workspace matrices one value
    at a time; the products that read workspace matrices as operands take the guarded kernel."""
    M, d, F, N = 300, 256, 1024, 2
    xb, x = normal_bf16((M, d), 1.0, 1190, 0)
    w1b, w1 = normal_bf16((d, F), 0.02, 1190, 1)
    w2b, w2 = normal_bf16((F, d), 0.02, 1190, 2)
    yb, dy = normal_bf16((M, d), 1.0, 1190, 3)
    X, W1, W2, dY = bf16_tensor(xb), bf16_tensor(w1b), bf16_tensor(w2b), bf16_tensor(yb)
    need = tp.mlp_backward_workspace_bytes(X, W1, W2, dY, N)
    ws = torch.empty(need + 4, dtype=torch.uint8, device=dev())[4:]
    note("mlp backward, workspace 4 bytes past alignment")
    dX, dW1, dW2 = tp.mlp_backward(X, W1, W2, dY, N, workspace=ws)
    rx, r1, r2 = oracle.mlp_backward(x, w1, w2, dy, N, "gelu")
    assert_close(host(dX), rx, "dX")
    assert_close(host(dW1), r1, "dW1")
    assert_close(host(dW2), r2, "dW2")


def test_mlp_backward_partial_outputs_and_fp32():
    M, d, F, N = 128, 64, 256, 2
    xb, x = normal_bf16((M, d), 1.0, 1600, 0)
    w1b, w1 = normal_bf16((d, F), 0.02, 1600, 1)
    w2b, w2 = normal_bf16((F, d), 0.02, 1600, 2)
    yb, dy = normal_bf16((M, d), 1.0, 1600, 3)
    X, W1, W2, dY = bf16_tensor(xb), bf16_tensor(w1b), bf16_tensor(w2b), bf16_tensor(yb)
    rx, r1, r2 = oracle.mlp_backward(x, w1, w2, dy, N)
    note("mlp backward: dW2 only, then dX only")
    a, g1, g2 = tp.mlp_backward(X, W1, W2, dY, N, dx=False, dw1=False)
    assert a is None and g1 is None
    assert_close(host(g2), r2, "dW2 alone")
    a, g1, g2 = tp.mlp_backward(X, W1, W2, dY, N, dw1=False, dw2=False)
    assert_close(host(a), rx, "dX alone")
    note("mlp backward: shard-major weights and gradients")
    width = F // N
    W1s = torch.stack([W1[:, s * width:(s + 1) * width] for s in range(N)]).contiguous()
    W2s = torch.stack([W2[s * width:(s + 1) * width] for s in range(N)]).contiguous()
    G1 = torch.empty((N, d, width), dtype=torch.float32, device=dev())
    G2 = torch.empty((N, width, d), dtype=torch.float32, device=dev())
    a, g1, g2 = tp.mlp_backward(X, W1s, W2s, dY, N, dw1=G1, dw2=G2)
    assert_close(host(a), rx, "dX (stacks)")
    assert_close(np.concatenate(list(host(g1)), axis=1), r1, "dW1 (stacks)")
    assert_close(np.concatenate(list(host(g2)), axis=0), r2, "dW2 (stacks)")
    note("mlp backward: fp32 inputs, exact integers, act none")
    xf = int_uniform_f32((24, 16), -2, 2, 1601, 0)
    w1f = int_uniform_f32((16, 36), -2, 2, 1601, 1)
    w2f = int_uniform_f32((36, 16), -2, 2, 1601, 2)
    yf = int_uniform_f32((24, 16), -2, 2, 1601, 3)
    a, g1, g2 = tp.mlp_backward(f32_tensor(xf), f32_tensor(w1f), f32_tensor(w2f), f32_tensor(yf), 3, act="none")
    fx, f1, f2 = oracle.mlp_backward(xf, w1f, w2f, yf, 3, "none")
    assert_exact(host(a), fx, "fp32 dX")
    assert_exact(host(g1), f1, "fp32 dW1")
    assert_exact(host(g2), f2, "fp32 dW2")


def test_backward_determinism_bitwise():
    M, d, F, N = 512, 512, 2048, 4
    xb, _ = normal_bf16((M, d), 1.0, 1700, 0)
    w1b, _ = normal_bf16((d, F), 0.02, 1700, 1)
    w2b, _ = normal_bf16((F, d), 0.02, 1700, 2)
    yb, _ = normal_bf16((M, d), 1.0, 1700, 3)
    X, W1, W2, dY = bf16_tensor(xb), bf16_tensor(w1b), bf16_tensor(w2b), bf16_tensor(yb)
    note("backward determinism: two runs")
    a = [t.clone() for t in tp.mlp_backward(X, W1, W2, dY, N)]
    b = [t.clone() for t in tp.mlp_backward(X, W1, W2, dY, N)]
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        assert torch.equal(u.view(torch.int32), v.view(torch.int32))


def test_mlp_backward_megatron_full_size():
    wl = WORKLOADS["megatron_mlp"]
    xb, x = normal_bf16((wl.M, wl.d), 1.0, wl.wid, 0)
    w1b, w1 = normal_bf16((wl.d, wl.F), 0.02, wl.wid, 1)
    w2b, w2 = normal_bf16((wl.F, wl.d), 0.02, wl.wid, 2)
    yb, dy = normal_bf16((wl.M, wl.d), 1.0, wl.wid, 4)
    note("megatron mlp backward full size: X [2048,4096], W1 [4096,16384], W2 [16384,4096], N=8")
    dX, dW1, dW2 = tp.mlp_backward(bf16_tensor(xb), bf16_tensor(w1b), bf16_tensor(w2b), bf16_tensor(yb), wl.N)
    gx, g1, g2 = host(dX), host(dW1), host(dW2)
    # dX: a row depends only on the same rows of X and dY
    rows = stratified_rows(wl.M, 11)
    rx, _, _ = oracle.mlp_backward(x[rows], w1, w2, dy[rows], wl.N)
    assert_close(gx[rows], rx, "dX sampled rows")
    # dW2 rows f and dW1 columns f depend on column f of Z = X W1 and row f of W2
    fs = stratified_rows(wl.F, 12)
    z = oracle.matmul(x, w1[:, fs])
    h = oracle.gelu(z)
    dz = oracle.matmul(dy, oracle.transpose(w2[fs, :])) * oracle.gelu_grad(z)
    assert_close(g2[fs, :], oracle.matmul(oracle.transpose(h), dy), "dW2 sampled rows")
    assert_close(g1[:, fs], oracle.matmul(oracle.transpose(x), dz), "dW1 sampled columns")
