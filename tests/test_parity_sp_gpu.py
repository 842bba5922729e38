"""GPU parity of the sequence-parallel boundary (tp_sp_layernorm, tp_reduce_partials over tokens).

Seeded synthetic partials, residuals, keep masks and LayerNorm parameters, the
library on the GPU and the float64 oracle on the CPU on the same bits,
compared within the bars of tests/parity.py. Cases: every register-resident
width class (up to 16384 features) and the wide / unaligned / odd-width
element path, ragged token shards, shard subsets, one to eight partials,
dropout on and off, fp32 and bf16 residuals and outputs, partitioned
(shard-major) layouts, the token all-gather (exact), shard-by-shard runs
gathered back equal to one run over all shards (bitwise), determinism, and
the Megatron MLP block at full size followed by the sequence-parallel
LayerNorm, checked on sampled token rows.
"""
import numpy as np
import pytest
import torch

import oracle
import tensor_sharded_linear_amd as tp
from synthetic import WORKLOADS, keep_mask, normal_bf16, normal_f32, stratified_rows
from parity import assert_close, assert_exact, bf16_tensor, dev, f32_tensor, host, note

pytestmark = pytest.mark.gpu

EPS = 1e-5


def inputs(wid, t, M, d, p_drop, r_bf16):
    """Partials [t, M, d] fp32, residual (bits or values), keep mask, gamma, beta."""
    P = np.stack([normal_f32((M, d), 0.0, 1.0, wid, 100 + k) for k in range(t)])
    if r_bf16:
        rbits, res = normal_bf16((M, d), 1.0, wid, 4)
    else:
        rbits, res = None, normal_f32((M, d), 0.0, 1.0, wid, 4)
    keep = keep_mask((M, d), p_drop, wid, 5) if p_drop > 0 else None
    gamma = normal_f32((d,), 1.0, 0.1, wid, 6)
    beta = normal_f32((d,), 0.0, 0.1, wid, 7)
    return P, rbits, res, keep, gamma, beta


def run_case(wid, t, M, d, N, s0, ns, p_drop=0.1, r_bf16=True, y_dtype=torch.bfloat16, with_res=True,
             with_x1=True, partitioned=False):
    P, rbits, res, keep, gamma, beta = inputs(wid, t, M, d, p_drop, r_bf16)
    T = M // N
    rows = slice(s0 * T, (s0 + ns) * T)
    note(f"sp_layernorm t={t} M={M} d={d} N={N} s0={s0} ns={ns} p={p_drop} r_bf16={r_bf16} y={y_dtype} "
         f"res={with_res} x1={with_x1} partitioned={partitioned}")
    r_dev = None
    if with_res:
        r_dev = bf16_tensor(rbits[rows]) if r_bf16 else f32_tensor(res[rows])
        if partitioned:
            r_dev = r_dev.view(ns, T, d)
    k_dev = torch.from_numpy(np.ascontiguousarray(keep[rows])).to(dev()) if keep is not None else None
    got = tp.sp_layernorm(f32_tensor(P), f32_tensor(gamma), f32_tensor(beta), N, s0, ns, residual=r_dev,
                          keep=k_dev, p_drop=p_drop, eps=EPS, out_dtype=y_dtype, residual_out=with_x1,
                          partitioned=partitioned)
    y, x1 = got if with_x1 else (got, None)
    rx, ry = oracle.sp_layernorm(list(P), res if with_res else None, keep, p_drop, gamma, beta, EPS, N, s0, ns)
    yh = host(y).reshape(ns * T, d)
    assert_close(yh, ry, "sp_layernorm y", stored_bf16=y_dtype == torch.bfloat16)
    if with_x1:
        assert_close(host(x1).reshape(ns * T, d), rx, "sp_layernorm x")


@pytest.mark.parametrize("d", [64, 1000, 2052, 4096, 8192, 12288, 16384])
def test_sp_layernorm_widths(d):
    run_case(3000 + d % 97, 2, 24, d, 4, 1, 2)


@pytest.mark.parametrize("d", [1001, 16388])
def test_sp_layernorm_element_path(d):
    # odd width / beyond the register-resident limit: the three-read element kernel
    run_case(3100 + d % 89, 3, 12, d, 3, 0, 3, p_drop=0.2, r_bf16=False, y_dtype=torch.float32)


@pytest.mark.parametrize("t", [1, 3, 8])
def test_sp_layernorm_partials_count(t):
    run_case(3200 + t, t, 40, 768, 8, 2, 5, p_drop=0.0)


@pytest.mark.parametrize("r_bf16,y_dtype,with_res,with_x1", [
    (False, torch.float32, True, True),
    (True, torch.float32, True, False),
    (False, torch.bfloat16, False, True),
    (True, torch.bfloat16, False, False),
])
def test_sp_layernorm_dtypes_and_options(r_bf16, y_dtype, with_res, with_x1):
    run_case(3300 + 2 * int(r_bf16) + int(with_res), 2, 64, 1024, 2, 0, 2, p_drop=0.25, r_bf16=r_bf16,
             y_dtype=y_dtype, with_res=with_res, with_x1=with_x1)


def test_sp_layernorm_partitioned():
    run_case(3400, 4, 48, 512, 4, 1, 3, partitioned=True)


def test_sp_layernorm_unaligned_strides():
    # partials with a padded, odd row stride take the element kernel
    wid, t, M, d, N = 3500, 2, 16, 256, 2
    P, rbits, res, keep, gamma, beta = inputs(wid, t, M, d, 0.1, True)
    note("sp_layernorm unaligned partial stride")
    pad = torch.zeros((t, M, d + 1), dtype=torch.float32, device=dev())
    pad[:, :, :d] = f32_tensor(P)
    y = tp.sp_layernorm(pad[:, :, :d], f32_tensor(gamma), f32_tensor(beta), N, residual=bf16_tensor(rbits),
                        keep=torch.from_numpy(keep).to(dev()), p_drop=0.1, eps=EPS)
    _, ry = oracle.sp_layernorm(list(P), res, keep, 0.1, gamma, beta, EPS, N)
    assert_close(host(y), ry, "unaligned")


def test_sp_layernorm_constant_rows_give_beta():
    # a row whose sum is constant normalizes to zero: the output is beta (closed form)
    M, d, N = 8, 512, 2
    gamma = normal_f32((d,), 1.0, 0.1, 3600, 6)
    beta = normal_f32((d,), 0.0, 0.1, 3600, 7)
    P = np.full((1, M, d), 0.375, np.float32)
    note("sp_layernorm constant rows")
    y = host(tp.sp_layernorm(f32_tensor(P), f32_tensor(gamma), f32_tensor(beta), N, eps=EPS))
    assert_exact(y, np.tile(beta.astype(np.float64), (M, 1)), "constant rows -> beta")


def test_token_all_gather_exact():
    n, R, C = 4, 6, 200
    bits, vals = normal_bf16((n, R, C), 1.0, 3700, 0)
    note("reduce_partials axis=tokens (token all-gather)")
    got = host(tp.reduce_partials(bf16_tensor(bits), axis="tokens", out_dtype=torch.bfloat16))
    assert_exact(got, oracle.all_gather_rows(list(vals)), "token all-gather")
    got32 = host(tp.reduce_partials(f32_tensor(vals), axis="tokens"))
    assert_exact(got32, oracle.all_gather_rows(list(vals)), "token all-gather fp32")


def test_shard_by_shard_then_gather_equals_one_call():
    wid, t, M, d, N = 3800, 3, 64, 2048, 4
    P, rbits, res, keep, gamma, beta = inputs(wid, t, M, d, 0.1, True)
    T = M // N
    Pd, gd, bd = f32_tensor(P), f32_tensor(gamma), f32_tensor(beta)
    kd = torch.from_numpy(keep).to(dev())
    rd = bf16_tensor(rbits)
    note("sp_layernorm per token shard, then all-gather")
    whole = tp.sp_layernorm(Pd, gd, bd, N, residual=rd, keep=kd, p_drop=0.1, eps=EPS)
    parts = torch.stack([tp.sp_layernorm(Pd, gd, bd, N, s, 1, residual=rd[s * T:(s + 1) * T],
                                         keep=kd[s * T:(s + 1) * T].contiguous(), p_drop=0.1, eps=EPS)
                         for s in range(N)])
    gathered = tp.reduce_partials(parts, axis="tokens")
    torch.cuda.synchronize()
    assert torch.equal(gathered.view(torch.int32), whole.view(torch.int32))


def test_sp_layernorm_determinism():
    wid, t, M, d, N = 3900, 8, 32, 4096, 8
    P, rbits, res, keep, gamma, beta = inputs(wid, t, M, d, 0.1, True)
    args = (f32_tensor(P), f32_tensor(gamma), f32_tensor(beta), N)
    kw = dict(residual=bf16_tensor(rbits), keep=torch.from_numpy(keep).to(dev()), p_drop=0.1, eps=EPS,
              out_dtype=torch.bfloat16)
    note("sp_layernorm determinism")
    a = tp.sp_layernorm(*args, **kw).clone()
    b = tp.sp_layernorm(*args, **kw).clone()
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_megatron_mlp_then_sp_layernorm_full_size():
    # X [2048, 4096] -> column W1 + GeLU -> row W2 partials (8 shards) -> reduce-scatter over 8 token
    # shards, dropout 0.1, residual X, LayerNorm; sampled token rows against the oracle
    wl = WORKLOADS["megatron_mlp"]
    xb, x = normal_bf16((wl.M, wl.d), 1.0, wl.wid, 0)
    w1b, w1 = normal_bf16((wl.d, wl.F), 0.02, wl.wid, 1)
    w2b, w2 = normal_bf16((wl.F, wl.d), 0.02, wl.wid, 2)
    keep = keep_mask((wl.M, wl.d), 0.1, wl.wid, 5)
    gamma = normal_f32((wl.d,), 1.0, 0.1, wl.wid, 6)
    beta = normal_f32((wl.d,), 0.0, 0.1, wl.wid, 7)
    note("megatron mlp + sequence-parallel LayerNorm at full size")
    xd = bf16_tensor(xb)
    h = tp.col_linear(xd, bf16_tensor(w1b), wl.N, act="gelu", partitioned=True)
    p = tp.row_linear(h, bf16_tensor(w2b), wl.N)
    y, x1 = tp.sp_layernorm(p, f32_tensor(gamma), f32_tensor(beta), wl.N, residual=xd,
                            keep=torch.from_numpy(keep).to(dev()), p_drop=0.1, eps=EPS,
                            out_dtype=torch.bfloat16, residual_out=True, partitioned=True)
    yh = host(y).reshape(wl.M, wl.d)
    xh = host(x1).reshape(wl.M, wl.d)
    rows = stratified_rows(wl.M, seed=wl.M + 1)
    parts = oracle.mlp_shard_partials(x[rows], w1, w2, wl.N, "gelu")
    rx, ry = oracle.sp_layernorm(parts, x[rows], keep[rows], 0.1, gamma, beta, EPS, 1)
    assert_close(xh[rows], rx, "pre-norm sum, sampled rows")
    assert_close(yh[rows], ry, "LayerNorm output, sampled rows", stored_bf16=True)


def test_sp_layernorm_padded_strides():
    # partials and outputs with padded (16-byte aligned) row strides keep the register path
    wid, t, M, d, N = 3950, 3, 32, 1024, 4
    P, rbits, res, keep, gamma, beta = inputs(wid, t, M, d, 0.1, True)
    note("sp_layernorm padded strides")
    pp = torch.zeros((t, M, d + 64), dtype=torch.float32, device=dev())
    pp[:, :, :d] = f32_tensor(P)
    yb = torch.zeros((M, d + 32), dtype=torch.bfloat16, device=dev())
    xb = torch.zeros((M, d + 16), dtype=torch.float32, device=dev())
    tp.sp_layernorm(pp[:, :, :d], f32_tensor(gamma), f32_tensor(beta), N, residual=bf16_tensor(rbits),
                    keep=torch.from_numpy(keep).to(dev()), p_drop=0.1, eps=EPS, out=yb[:, :d], residual_out=xb[:, :d])
    rx, ry = oracle.sp_layernorm(list(P), res, keep, 0.1, gamma, beta, EPS, N)
    assert_close(host(yb[:, :d]), ry, "padded y", stored_bf16=True)
    assert_close(host(xb[:, :d]), rx, "padded x")
    # the padding columns are untouched
    assert torch.count_nonzero(yb[:, d:]).item() == 0 and torch.count_nonzero(xb[:, d:]).item() == 0


def test_token_all_gather_converts_bf16_to_f32():
    n, R, C = 3, 5, 64
    bits, vals = normal_bf16((n, R, C), 1.0, 3960, 0)
    note("reduce_partials axis=tokens bf16 -> fp32")
    got = host(tp.reduce_partials(bf16_tensor(bits), axis="tokens", out_dtype=torch.float32))
    assert_exact(got, oracle.all_gather_rows(list(vals)), "token all-gather bf16 -> fp32")
