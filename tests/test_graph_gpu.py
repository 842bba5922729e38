"""The library inside a captured HIP graph.

The entry points allocate nothing, wait for nothing and clear nothing with
memset, so a caller can capture them (here through torch's graph capture, whose
capture stream the binding passes as the launch stream) and replay the whole
step. Each test captures a step once, then replays it several times with new
inputs written in between by ordinary eager work, and checks every replay
bitwise against the same calls run eagerly on those inputs.
"""
import numpy as np
import pytest
import torch

import tensor_sharded_linear_amd as tp
from synthetic import normal_bf16
from parity import bf16_tensor, dev, note

pytestmark = pytest.mark.gpu

REPLAYS = 3


def inputs(seed, shapes, sigmas):
    return [bf16_tensor(normal_bf16(s, sig, seed, t)[0]) for t, (s, sig) in enumerate(zip(shapes, sigmas))]


def test_megatron_step_in_a_graph():
    M, d, F, N = 256, 512, 2048, 4
    x, w1, w2 = inputs(9100, [(M, d), (d, F), (F, d)], [1.0, 0.02, 0.02])
    h = torch.empty((M, F), dtype=torch.bfloat16, device=dev())
    p = torch.empty((N, M, d), dtype=torch.float32, device=dev())
    y = torch.empty((M, d), dtype=torch.float32, device=dev())
    y1 = torch.empty((M, d), dtype=torch.float32, device=dev())
    ws = torch.empty(tp.mlp_workspace_bytes(x, w1, w2, N), dtype=torch.uint8, device=dev())

    def step():
        tp.col_linear(x, w1, N, act="gelu", out=h)
        tp.row_linear(h, w2, N, out=p)
        tp.reduce_partials(p, "rows", out=y)
        tp.mlp(x, w1, w2, N, out=y1, workspace=ws)

    step()  # first use outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for r in range(REPLAYS):
        note(f"graph replay {r}")
        xs, = inputs(9200 + r, [(M, d)], [1.0])
        x.copy_(xs)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got, got1 = y.clone(), y1.clone()
        step()  # the same calls, eagerly, on the same inputs
        torch.cuda.synchronize()
        assert torch.equal(got, y), f"replay {r}: three-call step differs from eager"
        assert torch.equal(got1, y1), f"replay {r}: tp_mlp differs from eager"
        assert torch.equal(got, got1)


def test_decode_and_attention_in_a_graph():
    # a decode-shaped MLP (skinny kernels, split-K chunk sums in the workspace: K in
    # four, finished by the chunk-sum pass)
    M, d, F, N = 16, 1024, 4096, 8
    x, w1, w2 = inputs(9300, [(M, d), (d, F), (F, d)], [1.0, 0.02, 0.02])
    y = torch.empty((M, d), dtype=torch.float32, device=dev())
    ws = torch.empty(tp.mlp_workspace_bytes(x, w1, w2, N), dtype=torch.uint8, device=dev())
    # shard-major weights whose first product splits K in two: the second product
    # reads the chunk sums itself (12 column tiles of 256 per shard, K 1000)
    d2, width = 1000, 3000
    w1s, w2s = inputs(9350, [(N, d2, width), (N, width, d2)], [0.02, 0.02])
    x2, = inputs(9360, [(M, d2)], [1.0])
    y2 = torch.empty((M, d2), dtype=torch.float32, device=dev())
    ws2 = torch.empty(tp.mlp_workspace_bytes(x2, w1s, w2s, N), dtype=torch.uint8, device=dev())
    # causal attention over two sequences, 4 heads x 128 split over 2 shards
    heads, n, dh, L, B = 4, 2, 128, 320, 2
    qkv, = inputs(9400, [(B * L, (heads + 2 * heads) * dh)], [1.0])
    att = torch.empty((B * L, heads * dh), dtype=torch.bfloat16, device=dev())

    def step():
        tp.mlp(x, w1, w2, N, out=y, workspace=ws)
        tp.mlp(x2, w1s, w2s, N, out=y2, workspace=ws2)
        tp.attention(qkv, n, heads, heads, dh, L, True, out=att)

    step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for r in range(REPLAYS):
        note(f"graph replay {r}")
        xs, qs, x2s = inputs(9500 + r, [(M, d), (B * L, (heads + 2 * heads) * dh), (M, d2)], [1.0, 1.0, 1.0])
        x.copy_(xs)
        qkv.copy_(qs)
        x2.copy_(x2s)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got_y, got_y2, got_a = y.clone(), y2.clone(), att.clone()
        step()
        torch.cuda.synchronize()
        assert torch.equal(got_y, y), f"replay {r}: decode MLP differs from eager"
        assert torch.equal(got_y2, y2), f"replay {r}: decode MLP (chunk sums read by the second product) differs"
        assert torch.equal(got_a, att), f"replay {r}: attention differs from eager"


def test_backward_and_sequence_parallel_boundary_in_a_graph():
    M, d, F, N = 256, 512, 1024, 4
    x, w1, w2, dy = inputs(9600, [(M, d), (d, F), (F, d), (M, d)], [1.0, 0.02, 0.02, 1.0])
    dX = torch.empty((M, d), dtype=torch.float32, device=dev())
    dW1 = torch.empty((d, F), dtype=torch.float32, device=dev())
    dW2 = torch.empty((F, d), dtype=torch.float32, device=dev())
    ws = torch.empty(tp.mlp_backward_workspace_bytes(x, w1, w2, dy, N), dtype=torch.uint8, device=dev())
    # the sequence-parallel boundary on the row-parallel partials of the forward pass
    p = torch.empty((N, M, d), dtype=torch.float32, device=dev())
    h = torch.empty((M, F), dtype=torch.bfloat16, device=dev())
    gamma = torch.ones(d, dtype=torch.float32, device=dev())
    beta = torch.zeros(d, dtype=torch.float32, device=dev())
    ln = torch.empty((M, d), dtype=torch.bfloat16, device=dev())

    def step():
        tp.mlp_backward(x, w1, w2, dy, N, dx=dX, dw1=dW1, dw2=dW2, workspace=ws)
        tp.col_linear(x, w1, N, act="gelu", out=h)
        tp.row_linear(h, w2, N, out=p)
        tp.sp_layernorm(p, gamma, beta, N, residual=x, out=ln)

    step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for r in range(REPLAYS):
        note(f"graph replay {r}")
        xs, ys = inputs(9700 + r, [(M, d), (M, d)], [1.0, 1.0])
        x.copy_(xs)
        dy.copy_(ys)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in (dX, dW1, dW2, ln)]
        step()
        torch.cuda.synchronize()
        for name, a, b in zip(("dX", "dW1", "dW2", "LayerNorm"), got, (dX, dW1, dW2, ln)):
            assert torch.equal(a, b), f"replay {r}: {name} differs from eager"
