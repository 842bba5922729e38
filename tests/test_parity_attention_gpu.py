"""GPU parity of attention per head subset (tp_attention) against the float64 oracle.

Seeded synthetic QKV blocks, the library on the GPU and the oracle on the CPU
on the same bits, compared within the bars of tests/parity.py (the output is
stored in the input dtype, bf16 here, so the bf16 storage allowance applies;
nothing else is allowed: the kernel's own arithmetic must fit the plain bar).
Cases: causal and not, head_dim 128 and 64 on the matrix cores, sequence
lengths that leave ragged 128-query and 64-key blocks (with an odd number of
query blocks, and with many full key blocks before the ragged one), several sequences,
grouped-query attention with key/value heads split and replicated, shard
subsets, partitioned layouts, the element-wise path (fp32 and other head
sizes), and the attention-projection workload's full shape checked on two
of its eight shards.
"""
import numpy as np
import pytest
import torch

import oracle
import tensor_sharded_linear_amd as tp
from synthetic import WORKLOADS, bf16_bits_from_f32, f32_from_bf16_bits, normal_bf16, rng
from parity import assert_close, bf16_tensor, dev, f32_tensor, host, note

pytestmark = pytest.mark.gpu


def qkv_case(M, heads, kv_heads, dh, n, ns, wid, sigma=1.0):
    hq = heads // n
    hkv = kv_heads // n if kv_heads >= n else 1
    bits, vals = normal_bf16((M, ns * (hq + 2 * hkv) * dh), sigma, wid, 0)
    return bits, vals


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("dh,L,B", [(128, 200, 2), (128, 384, 1), (64, 130, 3), (128, 1000, 2), (64, 777, 1)])
def test_attention_mha(causal, dh, L, B):
    heads, n = 8, 2
    bits, q = qkv_case(B * L, heads, heads, dh, n, n, 2000 + dh + L)
    note(f"attention mha dh={dh} L={L} B={B} causal={causal}")
    got = host(tp.attention(bf16_tensor(bits), n, heads, heads, dh, L, causal))
    ref = oracle.attention(q, n, heads, heads, dh, L, causal)
    assert_close(got, ref, "attention", stored_bf16=True)


@pytest.mark.parametrize("heads,kv_heads,n", [(8, 2, 4), (16, 4, 2), (8, 1, 8)])
def test_attention_gqa(heads, kv_heads, n):
    dh, L = 128, 256
    bits, q = qkv_case(L, heads, kv_heads, dh, n, n, 2100 + heads + kv_heads + n)
    note(f"attention gqa heads={heads} kv_heads={kv_heads} n={n}")
    got = host(tp.attention(bf16_tensor(bits), n, heads, kv_heads, dh, L))
    assert_close(got, oracle.attention(q, n, heads, kv_heads, dh, L), "attention gqa", stored_bf16=True)


def test_attention_subset_partitioned_and_head_split():
    heads, kv_heads, dh, L, n = 8, 4, 128, 320, 4
    hq, hkv = 2, 1
    # an unsharded QKV projection output, split into the shards' blocks by the head layout
    fbits, full = normal_bf16((L, (heads + 2 * kv_heads) * dh), 1.0, 2200, 0)
    cols = [oracle.shard_qkv_columns(heads, kv_heads, dh, n, s) for s in range(n)]
    qkv_bits = np.concatenate([fbits[:, c] for c in cols], axis=1)
    qkv_vals = np.concatenate([full[:, c] for c in cols], axis=1)
    unsharded = oracle.attention_shard(full, heads, kv_heads, dh, L, True)
    note("attention: all shards vs unsharded attention over all heads")
    got = host(tp.attention(bf16_tensor(qkv_bits), n, heads, kv_heads, dh, L))
    assert_close(got, unsharded, "all shards = unsharded", stored_bf16=True)
    note("attention: shards 1..2 of 4, partitioned in and out")
    blk = (hq + 2 * hkv) * dh
    part = torch.stack([bf16_tensor(qkv_bits[:, s * blk:(s + 1) * blk]) for s in (1, 2)]).contiguous()
    got = host(tp.attention(part, n, heads, kv_heads, dh, L, s0=1, ns=2, partitioned=True))
    ref = oracle.attention(qkv_vals[:, blk:3 * blk], n, heads, kv_heads, dh, L, True, 1, 2)
    assert_close(np.concatenate(list(got), axis=1), ref, "subset partitioned", stored_bf16=True)


@pytest.mark.parametrize("big", [(4, 5, 6, 7), (0, 1, 2, 3)])
@pytest.mark.parametrize("causal", [True, False])
def test_attention_scores_far_apart_within_a_key_block(big, causal):
    """Keys at positions big (mod 8) score about 136 above the rest (natural-log units), so an
    offset other than the true row max would overflow exp. The kernel splits each 64-key block's
    scores of one query over two lanes in groups of 4 keys; both placements put the large scores
    on one side of that split."""
    dh, L = 128, 256
    g = rng(2400, 0)
    u = g.standard_normal(dh)
    q = 3.0 * u + 0.05 * g.standard_normal((L, dh))
    k = 0.05 * g.standard_normal((L, dh))
    rows = np.array([j for j in range(L) if j % 8 in big])
    k[rows] = 4.0 * u
    v = g.standard_normal((L, dh))
    bits = bf16_bits_from_f32(np.concatenate([q, k, v], axis=1).astype(np.float32))
    vals = f32_from_bf16_bits(bits).astype(np.float64)
    scores = vals[:, :dh] @ vals[:, dh:2 * dh].T / np.sqrt(dh)
    assert scores[:, rows].min() - np.delete(scores, rows, axis=1).max() > 100.0
    note(f"attention, scores far apart within a key block, big={big} causal={causal}")
    got = host(tp.attention(bf16_tensor(bits), 1, 1, 1, dh, L, causal))
    assert np.isfinite(got).all()
    assert_close(got, oracle.attention(vals, 1, 1, 1, dh, L, causal), "attention, far-apart scores", stored_bf16=True)


def test_attention_elementwise_path():
    heads, n, L = 4, 2, 37
    note("attention fp32 inputs (element-wise path)")
    g = np.random.default_rng([2300, 0])
    q = g.standard_normal((2 * L, 2 * (2 + 4) * 16)).astype(np.float32)
    got = host(tp.attention(f32_tensor(q), n, heads, heads, 16, L))
    assert_close(got, oracle.attention(q, n, heads, heads, 16, L), "fp32 attention")
    note("attention bf16 head_dim 32 (element-wise path)")
    bits, vals = qkv_case(3 * L, heads, 2, 32, n, n, 2301)
    got = host(tp.attention(bf16_tensor(bits), n, heads, 2, 32, L, False))
    assert_close(got, oracle.attention(vals, n, heads, 2, 32, L, False), "bf16 dh=32", stored_bf16=True)


def test_attention_row_stride_past_31_bits():
    """A QKV row stride whose sequence span reaches 2^31 bytes leaves the matrix-core kernel
    (31-bit buffer offsets within a sequence) for the element-wise one."""
    heads, n, dh, L = 4, 2, 128, 300
    bits, vals = qkv_case(L, heads, heads, dh, n, n, 2350)
    ld = 1 << 22  # bf16: 300 rows span more than 2^31 bytes
    big = torch.empty((L, ld), dtype=torch.bfloat16, device=dev())
    q = big[:, : bits.shape[1]]
    q.copy_(bf16_tensor(bits))
    note("attention with a 2^22-element QKV row stride (element-wise path)")
    got = host(tp.attention(q, n, heads, heads, dh, L))
    # the element-wise kernel keeps the probabilities in fp32: only the bf16 storage allowance applies
    assert_close(got, oracle.attention(vals, n, heads, heads, dh, L), "attention, huge stride", stored_bf16=True)
    del big


def test_attention_determinism():
    bits, _ = qkv_case(512, 8, 8, 128, 2, 2, 2400)
    x = bf16_tensor(bits)
    note("attention determinism")
    a = tp.attention(x, 2, 8, 8, 128, 512).clone()
    b = tp.attention(x, 2, 8, 8, 128, 512).clone()
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_attention_projection_workload_full_shape():
    # X [4096, 8192] -> QKV [4096, 24576] (8 shards of 8 heads x 128) -> attention over the
    # 4096 tokens as one causal sequence; shards 0 and 7 are checked against the oracle
    wl = WORKLOADS["attn_proj"]
    heads, dh = 64, 128
    xb, _ = normal_bf16((wl.M, wl.d), 1.0, wl.wid, 0)
    wb, _ = normal_bf16((wl.d, wl.F), 0.02, wl.wid, 1)
    note("attention block: QKV projection then attention at full size")
    qkv = tp.col_linear(bf16_tensor(xb), bf16_tensor(wb), wl.N)
    out = host(tp.attention(qkv, wl.N, heads, heads, dh, wl.M))
    qv = host(qkv)
    blk = 3 * (heads // wl.N) * dh
    oblk = (heads // wl.N) * dh
    for s in (0, wl.N - 1):
        qs = qv[:, s * blk:(s + 1) * blk]
        ref = oracle.attention_shard(qs, heads // wl.N, heads // wl.N, dh, wl.M, True)
        assert_close(out[:, s * oblk:(s + 1) * oblk], ref, f"shard {s}", stored_bf16=True)
