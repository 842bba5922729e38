"""GPU parity: the HIP path (through the C interface) against the float64 oracle.

Every case draws seeded synthetic inputs (synthetic/), runs the library on
the GPU and the oracle on the CPU on the same bits, and compares element by
element: exactly for integer-valued inputs, else within the bars of
tests/parity.py. Full-size workloads are checked on seeded sampled rows,
which is exact because each output row depends only on its own input row.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import tensor_sharded_linear_amd as tp
from synthetic import WORKLOADS, int_uniform_f32, normal_bf16, stratified_rows
from parity import assert_close, assert_exact, bf16_tensor, dev, f32_tensor, host, note

pytestmark = pytest.mark.gpu


def ints_bf16(shape, lo, hi, wid, tid):
    """Small integers stored as bf16 (exactly representable): (bits, float32 values)."""
    from synthetic import bf16_bits_from_f32

    v = int_uniform_f32(shape, lo, hi, wid, tid)
    return bf16_bits_from_f32(v), v


# ----------------------------------------------------------------------------- the pages' worked example


def test_worked_example_fp32(golden_dir):
    with open(os.path.join(golden_dir, "worked_example.json")) as f:
        g = json.load(f)
    x = np.array(g["X"], np.float32)
    w = np.array(g["W"], np.float32)
    n = g["N"]
    X, W = f32_tensor(x), f32_tensor(w)
    note("worked example: tp_col_linear concat, N=2, fp32")
    assert_exact(host(tp.col_linear(X, W, n)), np.array(g["Y"]), "column split, concatenated")
    note("worked example: tp_col_linear partitioned")
    parts = host(tp.col_linear(X, W, n, partitioned=True))
    for s in range(n):
        assert_exact(parts[s], np.array(g["col_shard_outputs"][s]), f"column shard {s}")
    note("worked example: tp_row_linear + tp_reduce_partials")
    P = tp.row_linear(X, W, n)
    ph = host(P)
    for s in range(n):
        assert_exact(ph[s], np.array(g["row_partials"][s]), f"row partial {s}")
    assert_exact(host(tp.reduce_partials(P, "rows")), np.array(g["Y"]), "row partials summed")
    note("worked example: tp_reduce_partials concat of the column shards")
    cparts = tp.col_linear(X, W, n, partitioned=True)
    assert_exact(host(tp.reduce_partials(cparts, "cols")), np.array(g["Y"]), "column shards concatenated")


# ----------------------------------------------------------------------------- the tiny split check (exact)


def test_split_check_fp32_exact():
    wl = WORKLOADS["split_check"]
    x = int_uniform_f32((wl.M, wl.d), -4, 4, wl.wid, 0)
    w = int_uniform_f32((wl.d, wl.F), -4, 4, wl.wid, 1)
    X, W = f32_tensor(x), f32_tensor(w)
    ref = oracle.matmul(x, w)
    note("split check fp32: column split N=2")
    assert_exact(host(tp.col_linear(X, W, 2)), oracle.col_linear(x, w, 2), "column split")
    outs = host(tp.col_linear(X, W, 2, partitioned=True))
    for s, o in enumerate(oracle.col_shard_outputs(x, w, 2)):
        assert_exact(outs[s], o, f"column shard {s}")
    note("split check fp32: row split N=2")
    P = tp.row_linear(X, W, 2)
    for s, p in enumerate(oracle.row_partials(x, w, 2)):
        assert_exact(host(P)[s], p, f"row partial {s}")
    assert_exact(host(tp.reduce_partials(P)), oracle.row_linear(x, w, 2), "row split summed")
    assert_exact(host(tp.reduce_partials(P)), ref, "equals the unsharded product")


def test_split_check_bf16_exact():
    """The same integers in bf16 take the matrix-core kernels (few rows: the skinny kernel)."""
    wl = WORKLOADS["split_check"]
    xb, x = ints_bf16((wl.M, wl.d), -4, 4, wl.wid, 0)
    wb, w = ints_bf16((wl.d, wl.F), -4, 4, wl.wid, 1)
    X, W = bf16_tensor(xb), bf16_tensor(wb)
    note("split check bf16: column split, fp32 out")
    assert_exact(host(tp.col_linear(X, W, 2, out_dtype=torch.float32)), oracle.col_linear(x, w, 2), "column")
    note("split check bf16: row split")
    P = tp.row_linear(X, W, 2)
    assert_exact(host(tp.reduce_partials(P)), oracle.row_linear(x, w, 2), "row")


# ----------------------------------------------------------------------------- large-tile kernel


@pytest.mark.parametrize("M,K,width,N", [(300, 264, 264, 2), (512, 512, 256, 4), (257, 64, 40, 3), (1, 8, 256, 1)])
def test_mfma_exact_integers(M, K, width, N):
    """Integer bf16 inputs through the large-tile kernel: fp32 results must be exact."""
    nout = width * N
    xb, x = ints_bf16((M, K), -2, 2, 90 + M, 0)
    wb, w = ints_bf16((K, nout), -2, 2, 90 + M, 1)
    X, W = bf16_tensor(xb), bf16_tensor(wb)
    note(f"mfma exact: col M={M} K={K} width={width} N={N}")
    assert_exact(host(tp.col_linear(X, W, N, out_dtype=torch.float32)), oracle.col_linear(x, w, N), "column")
    if K % N == 0:
        note(f"mfma exact: row M={M} K={K} Nout={nout} N={N}")
        P = tp.row_linear(X, W, N)
        for s, p in enumerate(oracle.row_partials(x, w, N)):
            assert_exact(host(P[s]), p, f"row partial {s}")


@pytest.mark.parametrize("M,K,width,N,act", [
    (600, 520, 392, 2, "none"),
    (600, 520, 392, 2, "gelu"),
    (256, 1024, 256, 4, "gelu"),
    (777, 136, 136, 3, "none"),
])
def test_mfma_float_col(M, K, width, N, act):
    nout = width * N
    xb, x = normal_bf16((M, K), 1.0, 200 + M, 0)
    wb, w = normal_bf16((K, nout), 0.02, 200 + M, 1)
    X, W = bf16_tensor(xb), bf16_tensor(wb)
    for out_dtype in (torch.float32, torch.bfloat16):
        note(f"mfma col M={M} K={K} width={width} N={N} act={act} out={out_dtype}")
        got = host(tp.col_linear(X, W, N, act=act, out_dtype=out_dtype))
        assert_close(got, oracle.col_linear(x, w, N, act), f"col {act} {out_dtype}",
                     stored_bf16=out_dtype == torch.bfloat16)
    # a proper sub-range of shards, partitioned output
    if N >= 2:
        note(f"mfma col sub-range s0=1 ns={N - 1} partitioned")
        got = host(tp.col_linear(X, W, N, s0=1, ns=N - 1, act=act, partitioned=True, out_dtype=torch.float32))
        for j, o in enumerate(oracle.col_shard_outputs(x, w, N, act, s0=1, ns=N - 1)):
            assert_close(got[j], o, f"col shard {j + 1}")


@pytest.mark.parametrize("M,K,Nout,N", [(600, 1040, 392, 2), (300, 512, 768, 4), (1000, 96, 264, 3)])
def test_mfma_float_row(M, K, Nout, N):
    xb, x = normal_bf16((M, K), 1.0, 300 + M, 0)
    wb, w = normal_bf16((K, Nout), 0.02, 300 + M, 1)
    X, W = bf16_tensor(xb), bf16_tensor(wb)
    note(f"mfma row M={M} K={K} Nout={Nout} N={N}")
    P = tp.row_linear(X, W, N)
    ph = host(P)
    for s, p in enumerate(oracle.row_partials(x, w, N)):
        assert_close(ph[s], p, f"row partial {s}")
    assert_close(host(tp.reduce_partials(P)), oracle.row_linear(x, w, N), "row sum")


def test_shard_major_weights_and_inputs():
    """3-D shard-major stacks (block s at base + s * stride) for both splits."""
    M, K, width, N = 320, 256, 128, 4
    xb, x = normal_bf16((M, K), 1.0, 400, 0)
    wb, w = normal_bf16((N, K, width), 0.02, 400, 1)  # column blocks
    X, W = bf16_tensor(xb), bf16_tensor(wb)
    wfull = np.concatenate(list(w), axis=1)
    note("shard-major column weights")
    assert_close(host(tp.col_linear(X, W, N, out_dtype=torch.float32)), oracle.col_linear(x, wfull, N), "col")
    # row split with a shard-major input (the partitioned output of a column layer)
    xsb, xs = normal_bf16((N, M, 64), 1.0, 401, 0)
    w2b, w2 = normal_bf16((N, 64, 200), 0.02, 401, 1)
    note("shard-major row inputs and weights")
    P = tp.row_linear(bf16_tensor(xsb), bf16_tensor(w2b), N)
    xfull = np.concatenate(list(xs), axis=1)
    w2full = np.concatenate(list(w2), axis=0)
    for s, p in enumerate(oracle.row_partials(xfull, w2full, N)):
        assert_close(host(P[s]), p, f"row partial {s}")


# ----------------------------------------------------------------------------- guarded kernel


def test_generic_path_unaligned_strides():
    """Leading dimensions that are not multiples of 8 take the element-guarded kernel."""
    M, K, width, N = 70, 37, 21, 3
    xb, x = normal_bf16((M, K + 3), 1.0, 500, 0)  # row stride K+3, view of the first K columns
    wb, w = normal_bf16((K, width * N + 5), 0.02, 500, 1)
    X = bf16_tensor(xb)[:, :K]
    W = bf16_tensor(wb)[:, : width * N]
    note("generic path: bf16 unaligned col")
    got = host(tp.col_linear(X, W, N, act="gelu", out_dtype=torch.float32))
    assert_close(got, oracle.col_linear(x[:, :K], w[:, : width * N], N, "gelu"), "generic col")
    xi = int_uniform_f32((M, 36), -4, 4, 501, 0)
    wi = int_uniform_f32((36, 50), -4, 4, 501, 1)
    note("generic path: fp32 exact row")
    P = tp.row_linear(f32_tensor(xi), f32_tensor(wi), 4)
    assert_exact(host(tp.reduce_partials(P)), oracle.row_linear(xi, wi, 4), "generic row exact")


def test_large_tile_kernel_with_unaligned_outputs():
    """Outputs whose row stride or base address rule out 16-byte (fp32) or 8-byte (bf16) stores
    still run on the large-tile kernel, which then stores each value alone."""
    M, K, width, N = 300, 512, 264, 2
    xb, x = normal_bf16((M, K), 1.0, 510, 0)
    wb, w = normal_bf16((K, width * N), 0.02, 510, 1)
    X, W = bf16_tensor(xb), bf16_tensor(wb)
    ref = oracle.col_linear(x, w, N, "gelu")
    note("large-tile col, bf16 Y with a row stride of 2 mod 4 elements")
    Ybig = torch.zeros((M, width * N + 2), dtype=torch.bfloat16, device=dev())
    got = tp.col_linear(X, W, N, act="gelu", out=Ybig[:, : width * N])
    assert_close(host(got), ref, "col, bf16 Y stride 2 mod 4", stored_bf16=True)
    assert torch.count_nonzero(Ybig[:, width * N:]) == 0
    note("large-tile col, fp32 Y one element past a 16-byte boundary")
    Yf = torch.zeros(M * width * N + 1, dtype=torch.float32, device=dev())
    got = tp.col_linear(X, W, N, act="gelu", out=Yf[1:].view(M, width * N))
    assert_close(host(got), ref, "col, fp32 Y offset by one element")
    assert float(Yf[0]) == 0.0
    note("large-tile row partials with an odd row stride")
    hb, h = normal_bf16((M, 2 * K), 1.0, 511, 0)
    w2b, w2 = normal_bf16((2 * K, width), 0.02, 511, 1)
    Pbig = torch.zeros((2, M, width + 1), dtype=torch.float32, device=dev())
    P = tp.row_linear(bf16_tensor(hb), bf16_tensor(w2b), 2, out=Pbig[:, :, :width])
    parts = oracle.row_partials(h, w2, 2)
    for j in range(2):
        assert_close(host(P[j]), parts[j], f"row partial {j}, odd row stride")
    assert torch.count_nonzero(Pbig[:, :, width:]) == 0


def test_long_k_shorter_tile_groups_with_ragged_tiles():
    """K long enough (10496) that the large-tile kernel groups tiles 2 rows tall, with 3 row tiles
    (the last group 1 row tall) and a ragged column tile, for both splits."""
    M, K, width, N = 600, 10496, 264, 2
    xb, x = normal_bf16((M, K), 1.0, 520, 0)
    wb, w = normal_bf16((K, width * N), 0.02, 520, 1)
    note("long K: col, GeLU, 3 row tiles, ragged columns")
    got = host(tp.col_linear(bf16_tensor(xb), bf16_tensor(wb), N, act="gelu", out_dtype=torch.float32))
    assert_close(got, oracle.col_linear(x, w, N, "gelu"), "long-K col")
    hb, h = normal_bf16((M, K * N), 1.0, 521, 0)
    w2b, w2 = normal_bf16((K * N, width), 0.02, 521, 1)
    note("long K: row partials, 3 row tiles, ragged columns")
    P = tp.row_linear(bf16_tensor(hb), bf16_tensor(w2b), N)
    parts = oracle.row_partials(h, w2, N)
    for j in range(N):
        assert_close(host(P[j]), parts[j], f"long-K row partial {j}")


def test_row_strides_past_31_bits_take_the_guarded_path():
    """Row strides whose 256-row tile span reaches 2^31 bytes leave the large-tile kernel (its
    buffer offsets are 31-bit) for the element-guarded one, which addresses in 64 bits."""
    M, K, width, N = 300, 64, 64, 2
    xb, x = normal_bf16((M, K), 1.0, 510, 0)
    wb, w = normal_bf16((K, width * N), 0.02, 510, 1)
    ldx = 1 << 22  # bf16: 256 rows span 2^31 bytes
    big_x = torch.empty((M, ldx), dtype=torch.bfloat16, device=dev())
    X = big_x[:, :K]
    X.copy_(bf16_tensor(xb))
    W = bf16_tensor(wb)
    note("guarded path: col with a 2^22-element row stride on X")
    got = host(tp.col_linear(X, W, N, act="gelu"))
    assert_close(got, oracle.col_linear(x, w, N, "gelu"), "col, huge X stride", stored_bf16=True)
    ldy = 1 << 21  # fp32: 256 rows span 2^31 bytes
    big_y = torch.empty((M, ldy), dtype=torch.float32, device=dev())
    Y = big_y[:, : width * N]
    note("guarded path: col with a 2^21-element row stride on an fp32 Y")
    tp.col_linear(bf16_tensor(xb), W, N, out=Y)
    assert_close(host(Y), oracle.col_linear(x, w, N), "col, huge Y stride")
    note("guarded path: row partials with a 2^22-element row stride on X")
    assert_close(host(tp.reduce_partials(tp.row_linear(X, W, N))), oracle.row_linear(x, w, N), "row, huge X stride")
    del big_x, big_y


def test_more_shards_than_one_launch_grid_holds():
    """65540 row shards of one input feature each: the element-guarded products go out in
    several launches (65535 shards per grid), then the sum runs over all partials."""
    M, N, Nout = 2, 65540, 3
    x = int_uniform_f32((M, N), -2, 2, 520, 0)
    w = int_uniform_f32((N, Nout), -2, 2, 520, 1)
    note(f"row split into {N} shards (fp32, exact)")
    P = tp.row_linear(f32_tensor(x), f32_tensor(w), N)
    ph = host(P)
    want = oracle.row_partials(x, w, N)
    for s in (0, 1, 65534, 65535, 65536, N - 1):  # both sides of the launch boundary
        assert_exact(ph[s], want[s], f"partial {s}")
    assert_exact(host(tp.reduce_partials(P)), oracle.row_linear(x, w, N), "sum over 65540 partials")


# ----------------------------------------------------------------------------- skinny kernel


@pytest.mark.parametrize("M", [1, 4, 16, 17, 32])
def test_skinny_col_and_row(M):
    K, width, N = 1000, 192, 3
    xb, x = normal_bf16((M, K), 1.0, 600 + M, 0)
    wb, w = normal_bf16((K, width * N), 0.02, 600 + M, 1)
    X, W = bf16_tensor(xb), bf16_tensor(wb)
    note(f"skinny col M={M} K={K} width={width} N={N}")
    got = host(tp.col_linear(X, W, N, act="gelu", out_dtype=torch.float32))
    assert_close(got, oracle.col_linear(x, w, N, "gelu"), f"skinny col M={M}")
    Kr = 1200
    xb2, x2 = normal_bf16((M, Kr), 1.0, 650 + M, 0)
    wb2, w2 = normal_bf16((Kr, 264), 0.02, 650 + M, 1)
    note(f"skinny row M={M} K={Kr} N={N}")
    P = tp.row_linear(bf16_tensor(xb2), bf16_tensor(wb2), N)
    for s, p in enumerate(oracle.row_partials(x2, w2, N)):
        assert_close(host(P[s]), p, f"skinny row partial {s}")


def test_skinny_exact_integers():
    M, K, width, N = 16, 2048, 64, 4
    xb, x = ints_bf16((M, K), -1, 1, 700, 0)
    wb, w = ints_bf16((K, width * N), -2, 2, 700, 1)
    note("skinny exact integers")
    got = host(tp.col_linear(bf16_tensor(xb), bf16_tensor(wb), N, out_dtype=torch.float32))
    assert_exact(got, oracle.col_linear(x, w, N), "skinny col exact")


def test_skinny_wide_tiles_ragged():
    # Enough column tiles (>= 192 of 256 columns) that the skinny kernel takes
    # its 256-column tiles; the column count leaves a ragged last tile and the
    # per-shard K (264) a partial 32-row slice.
    M, K, Nout, N = 5, 2112, 6000, 8
    xb, x = normal_bf16((M, K), 1.0, 720, 0)
    wb, w = normal_bf16((K, Nout), 0.02, 720, 1)
    note(f"skinny wide row M={M} K={K} Nout={Nout} N={N}")
    P = tp.row_linear(bf16_tensor(xb), bf16_tensor(wb), N)
    for s, p in enumerate(oracle.row_partials(x, w, N)):
        assert_close(host(P[s]), p, f"skinny wide row partial {s}")
    xi, xf = ints_bf16((M, K), -1, 1, 721, 0)
    wi, wf = ints_bf16((K, Nout), -2, 2, 721, 1)
    P = tp.row_linear(bf16_tensor(xi), bf16_tensor(wi), N)
    for s, p in enumerate(oracle.row_partials(xf, wf, N)):
        assert_exact(host(P[s]), p, f"skinny wide row exact partial {s}")
    M2, K2, width = 16, 96, 6144
    xb2, x2 = normal_bf16((M2, K2), 1.0, 722, 0)
    wb2, w2 = normal_bf16((K2, width * N), 0.02, 722, 1)
    note(f"skinny wide col gelu M={M2} K={K2} Nout={width * N}")
    got = host(tp.col_linear(bf16_tensor(xb2), bf16_tensor(wb2), N, act="gelu", out_dtype=torch.float32))
    assert_close(got, oracle.col_linear(x2, w2, N, "gelu"), "skinny wide col gelu")


# Inside tp_mlp a skinny first product may split K in two; the second product
# then adds the two fp32 chunk sums (ascending), applies the activation and
# rounds to bf16 as it loads its token rows, with no finishing pass between.
# Cases (first product's tiles, second product's tiles, how the sums are laid out):
#  - shard-major weights, 8 shards: 12 tiles of 256 per shard (the last ragged,
#    3000 columns), K 1000 in chunks of 512; second product 128 columns wide;
#    sums one block per shard
#  - shard-major weights, shards 2..6 of 8 and 3 rows: 120 tiles of 128, two
#    chunks; sums one block per shard
#  - one [d, F] weight, 16 shards: 96 tiles of 256 over all shards' columns,
#    K 3072 in two chunks; second product 256 columns wide (192 tiles); sums
#    one block holding every shard's columns, at the 16 rows of a full fragment
#  - one token (a single decode step), shard-major weights, 8 shards
#  - one [d, F] weight, shards 3..12 of 16: 120 tiles of 128, two chunks; sums
#    one block whose rows are longer than the second product's K
CHUNKED_CASES = [(5, 1000, 3000, 8, 0, 8, True), (3, 1000, 3000, 8, 2, 5, True),
                 (16, 3072, 1536, 16, 0, 16, False), (1, 1000, 3000, 8, 0, 8, True),
                 (7, 3072, 1536, 16, 3, 10, False)]


@pytest.mark.parametrize("M,d,width,N,s0,ns,shard_major", CHUNKED_CASES)
def test_mlp_skinny_split_k_into_second_product(M, d, width, N, s0, ns, shard_major):
    seed = 730 + d + M
    # 256 nonzero columns of X: |H| <= 256, so H is exact in bf16 and the whole chain in fp32
    xi, xf = ints_bf16((M, d), -1, 1, seed, 0)
    keep = np.zeros(d, dtype=bool)
    keep[:128] = keep[d - 128:] = True
    xi[:, ~keep] = 0
    xf[:, ~keep] = 0
    if shard_major:
        w1i, w1f = ints_bf16((N, d, width), -1, 1, seed, 1)
        w2i, w2f = ints_bf16((N, width, d), -1, 1, seed, 2)
        w1full, w2full = np.concatenate(list(w1f), axis=1), np.concatenate(list(w2f), axis=0)
    else:
        w1i, w1f = ints_bf16((d, width * N), -1, 1, seed, 1)
        w2i, w2f = ints_bf16((width * N, d), -1, 1, seed, 2)
        w1full, w2full = w1f, w2f
    note(f"mlp skinny split-K exact M={M} d={d} width={width} N={N} s0={s0} ns={ns} shard_major={shard_major}")
    got = host(tp.mlp(bf16_tensor(xi), bf16_tensor(w1i), bf16_tensor(w2i), N, s0=s0, ns=ns, act="none"))
    assert_exact(got, oracle.mlp(xf, w1full, w2full, N, "none", s0, ns), "mlp skinny split-K exact")

    xb, x = normal_bf16((M, d), 1.0, seed + 1, 0)
    if shard_major:
        w1b, w1 = normal_bf16((N, d, width), 0.02, seed + 1, 1)
        w2b, w2 = normal_bf16((N, width, d), 0.02, seed + 1, 2)
        w1full, w2full = np.concatenate(list(w1), axis=1), np.concatenate(list(w2), axis=0)
    else:
        w1b, w1full = normal_bf16((d, width * N), 0.02, seed + 1, 1)
        w2b, w2full = normal_bf16((width * N, d), 0.02, seed + 1, 2)
    note(f"mlp skinny split-K gelu M={M} d={d} width={width} N={N} s0={s0} ns={ns} shard_major={shard_major}")
    got = host(tp.mlp(bf16_tensor(xb), bf16_tensor(w1b), bf16_tensor(w2b), N, s0=s0, ns=ns))
    assert_close(got, oracle.mlp(x, w1full, w2full, N, "gelu", s0, ns), "mlp skinny split-K gelu")


# ----------------------------------------------------------------------------- combine kernels


@pytest.mark.parametrize("rows,cols,n", [(33, 64, 3), (5, 7, 4), (128, 1000, 8), (1, 4, 1)])
def test_reduce_and_concat(rows, cols, n):
    g = np.random.default_rng(rows * 1000 + cols)
    p = g.standard_normal((n, rows, cols)).astype(np.float32)
    P = f32_tensor(p)
    note(f"reduce rows={rows} cols={cols} n={n}")
    got = host(tp.reduce_partials(P, "rows"))
    assert_close(got, oracle.reduce_sum(list(p)), "sum")
    # the fp32 sum in ascending shard order is reproduced exactly by sequential float32 adds
    seq = p[0].copy()
    for j in range(1, n):
        seq = (seq + p[j]).astype(np.float32)
    assert_exact(got, seq, "ascending-order fp32 sum")
    got16 = host(tp.reduce_partials(P, "rows", out_dtype=torch.bfloat16))
    assert_close(got16, oracle.reduce_sum(list(p)), "sum bf16 out", stored_bf16=True)
    note(f"concat rows={rows} cols={cols} n={n}")
    assert_exact(host(tp.reduce_partials(P, "cols")), oracle.concat_cols(list(p)), "concat")
    assert_close(host(tp.reduce_partials(P, "cols", out_dtype=torch.bfloat16)), oracle.concat_cols(list(p)),
                 "concat fp32 -> bf16", stored_bf16=True)
    note(f"concat of bf16 blocks rows={rows} cols={cols} n={n}, side by side and stacked by rows")
    from synthetic import bf16_bits_from_f32, f32_from_bf16_bits
    bits = bf16_bits_from_f32(p)
    vals = f32_from_bf16_bits(bits)
    Pb = bf16_tensor(bits)
    assert_exact(host(tp.reduce_partials(Pb, "cols", out_dtype=torch.bfloat16)), oracle.concat_cols(list(vals)),
                 "concat bf16")
    assert_exact(host(tp.reduce_partials(Pb, "tokens", out_dtype=torch.bfloat16)), oracle.all_gather_rows(list(vals)),
                 "token gather bf16")


# ----------------------------------------------------------------------------- MLP chain


def test_mlp_exact_integers_no_activation():
    M, d, F, N = 96, 256, 512, 4
    xb, x = ints_bf16((M, d), -1, 1, 800, 0)
    w1b, w1 = ints_bf16((d, F), -1, 1, 800, 1)
    w2b, w2 = ints_bf16((F, d), -1, 1, 800, 2)
    note("mlp exact, act none, N=4")
    got = host(tp.mlp(bf16_tensor(xb), bf16_tensor(w1b), bf16_tensor(w2b), N, act="none"))
    assert_exact(got, oracle.mlp(x, w1, w2, N, "none"), "mlp exact")
    note("mlp exact, act none, decode rows")
    got = host(tp.mlp(bf16_tensor(xb[:16]), bf16_tensor(w1b), bf16_tensor(w2b), N, act="none"))
    assert_exact(got, oracle.mlp(x[:16], w1, w2, N, "none"), "mlp exact decode")


@pytest.mark.parametrize("M,d,F,N,s0,ns", [(300, 512, 2048, 4, 0, 4), (300, 512, 2048, 4, 1, 2),
                                           (16, 1024, 4096, 8, 0, 8), (9, 512, 1536, 3, 0, 3),
                                           (256, 256, 1024, 1, 0, 1)])
def test_mlp_gelu(M, d, F, N, s0, ns):
    xb, x = normal_bf16((M, d), 1.0, 900 + M, 0)
    w1b, w1 = normal_bf16((d, F), 0.02, 900 + M, 1)
    w2b, w2 = normal_bf16((F, d), 0.02, 900 + M, 2)
    note(f"mlp gelu M={M} d={d} F={F} N={N} s0={s0} ns={ns}")
    got = host(tp.mlp(bf16_tensor(xb), bf16_tensor(w1b), bf16_tensor(w2b), N, s0=s0, ns=ns))
    assert_close(got, oracle.mlp(x, w1, w2, N, "gelu", s0, ns), "mlp gelu")


def test_mlp_fp32_exact():
    M, d, F, N = 8, 24, 36, 3
    x = int_uniform_f32((M, d), -2, 2, 950, 0)
    w1 = int_uniform_f32((d, F), -2, 2, 950, 1)
    w2 = int_uniform_f32((F, d), -2, 2, 950, 2)
    note("mlp fp32 exact act none")
    got = host(tp.mlp(f32_tensor(x), f32_tensor(w1), f32_tensor(w2), N, act="none"))
    assert_exact(got, oracle.mlp(x, w1, w2, N, "none"), "fp32 mlp")


@pytest.mark.parametrize("M,d,F,N,s0,ns", [(300, 512, 2048, 4, 0, 4), (300, 392, 1536, 3, 0, 3),
                                           (520, 264, 2048, 8, 2, 5), (64, 512, 1024, 2, 0, 2)])
def test_mlp_bitwise_equals_separate_calls(M, d, F, N, s0, ns):
    """tp_mlp must carry the bits of the three public calls it stands for: the column product with
    GeLU, the row partials of the executed shards, their sum in ascending shard order. The shapes
    have ragged row and column tiles and shard counts that are not multiples of 4."""
    xb, _ = normal_bf16((M, d), 1.0, 980 + M, 0)
    w1b, _ = normal_bf16((d, F), 0.02, 980 + M, 1)
    w2b, _ = normal_bf16((F, d), 0.02, 980 + M, 2)
    X, W1, W2 = bf16_tensor(xb), bf16_tensor(w1b), bf16_tensor(w2b)
    width = F // N
    note(f"mlp vs separate calls M={M} d={d} F={F} N={N} s0={s0} ns={ns}")
    y = tp.mlp(X, W1, W2, N, s0=s0, ns=ns)
    h = tp.col_linear(X, W1, N, s0=s0, ns=ns, act="gelu")
    p = tp.row_linear(h, W2[s0 * width:(s0 + ns) * width], ns)
    y2 = tp.reduce_partials(p)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int32), y2.view(torch.int32))
    note("mlp vs separate calls, second call on the same shapes")
    y3 = tp.mlp(X, W1, W2, N, s0=s0, ns=ns)
    torch.cuda.synchronize()
    assert torch.equal(y3.view(torch.int32), y2.view(torch.int32))


def test_empty_and_degenerate():
    xb, x = normal_bf16((0, 64), 1.0, 960, 0)
    wb, w = normal_bf16((64, 128), 0.02, 960, 1)
    note("empty M")
    out = tp.col_linear(bf16_tensor(xb), bf16_tensor(wb), 2)
    assert out.shape == (0, 128)
    # K = 0: the product is empty, so every output is act(0) = 0
    note("K = 0")
    X0 = torch.zeros((5, 0), dtype=torch.bfloat16, device=dev())
    W0 = torch.zeros((0, 16), dtype=torch.bfloat16, device=dev())
    got = host(tp.col_linear(X0, W0, 2, out_dtype=torch.float32, act="gelu"))
    assert_exact(got, np.zeros((5, 16)), "K=0")
    # one column per shard (N = Nout)
    xb, x = normal_bf16((40, 64), 1.0, 961, 0)
    wb, w = normal_bf16((64, 8), 0.02, 961, 1)
    note("N = Nout: one column per shard")
    got = host(tp.col_linear(bf16_tensor(xb), bf16_tensor(wb), 8, out_dtype=torch.float32))
    assert_close(got, oracle.col_linear(x, w, 8), "one column per shard")


def test_determinism_bitwise():
    M, d, F, N = 512, 1024, 4096, 8
    xb, _ = normal_bf16((M, d), 1.0, 970, 0)
    w1b, _ = normal_bf16((d, F), 0.02, 970, 1)
    w2b, _ = normal_bf16((F, d), 0.02, 970, 2)
    X, W1, W2 = bf16_tensor(xb), bf16_tensor(w1b), bf16_tensor(w2b)
    note("determinism: two mlp runs")
    a = tp.mlp(X, W1, W2, N).clone()
    b = tp.mlp(X, W1, W2, N).clone()
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    note("determinism: decode rows")
    a = tp.mlp(X[:16], W1, W2, N).clone()
    b = tp.mlp(X[:16], W1, W2, N).clone()
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))


# ----------------------------------------------------------------------------- full-size workloads


def _rows(m):
    """Rows checked at full size: the first and last row of every 256-row tile and one seeded row in
    every 32-row band (every output tile and every band of 32 accumulator rows inside it)."""
    return stratified_rows(m, seed=m)


def test_megatron_mlp_full_size():
    wl = WORKLOADS["megatron_mlp"]
    xb, x = normal_bf16((wl.M, wl.d), 1.0, wl.wid, 0)
    w1b, w1 = normal_bf16((wl.d, wl.F), 0.02, wl.wid, 1)
    w2b, w2 = normal_bf16((wl.F, wl.d), 0.02, wl.wid, 2)
    note("megatron mlp full size: X [2048,4096], W1 [4096,16384], W2 [16384,4096], N=8, all shards")
    got = host(tp.mlp(bf16_tensor(xb), bf16_tensor(w1b), bf16_tensor(w2b), wl.N))
    rows = _rows(wl.M)
    assert_close(got[rows], oracle.mlp(x[rows], w1, w2, wl.N, "gelu"), "megatron mlp sampled rows")


def test_attention_projections_full_size():
    wl = WORKLOADS["attn_proj"]
    xb, x = normal_bf16((wl.M, wl.d), 1.0, wl.wid, 0)
    wqb, wq = normal_bf16((wl.d, wl.F), 0.02, wl.wid, 1)
    wob, wo = normal_bf16((wl.d, wl.out), 0.02, wl.wid, 2)
    ab, a = normal_bf16((wl.M, wl.d), 1.0, wl.wid, 3)
    rows = _rows(wl.M)
    note("attention QKV column-parallel full size: X [4096,8192] Wqkv [8192,24576] N=8 -> bf16")
    X, Wq = bf16_tensor(xb), bf16_tensor(wqb)
    qkv = host(tp.col_linear(X, Wq, wl.N))
    ref = oracle.col_linear(x[rows], wq, wl.N)
    assert_close(qkv[rows], ref, "qkv sampled rows", stored_bf16=True)
    del qkv
    # the same product with fp32 output: the computed value itself, under the plain bar
    note("attention QKV column-parallel full size with fp32 output")
    qkv32 = tp.col_linear(X, Wq, wl.N, out_dtype=torch.float32)
    got32 = host(qkv32[torch.as_tensor(rows, device=qkv32.device)])
    del qkv32
    assert_close(got32, ref, "qkv fp32 sampled rows")
    note("attention output projection row-parallel full size: A [4096,8192] Wo [8192,8192] N=8")
    P = tp.row_linear(bf16_tensor(ab), bf16_tensor(wob), wl.N)
    Y = host(tp.reduce_partials(P))
    parts = oracle.row_partials(a[rows], wo, wl.N)
    Pr = host(P[:, torch.as_tensor(rows, device=P.device)])
    for s in range(wl.N):
        assert_close(Pr[s], parts[s], f"W_o partial {s}")
    assert_close(Y[rows], oracle.reduce_sum(parts), "W_o reduced")


def test_gpt3_mlp_one_shard_full_size():
    wl = WORKLOADS["gpt3_mlp_shard"]
    width = wl.F // wl.N
    xb, x = normal_bf16((wl.M, wl.d), 1.0, wl.wid, 0)
    w1b, w1 = normal_bf16((1, wl.d, width), 0.02, wl.wid, 1)   # shard 0 of W1 only
    w2b, w2 = normal_bf16((1, width, wl.d), 0.02, wl.wid, 2)   # shard 0 of W2 only
    note("gpt3-width mlp, shard 0 of 8: X [16384,12288], W1_0 [12288,6144], W2_0 [6144,12288]")
    got = host(tp.mlp(bf16_tensor(xb), bf16_tensor(w1b), bf16_tensor(w2b), wl.N, s0=0, ns=1))
    rows = _rows(wl.M)
    # shard 0 of an 8-way split is the whole of the stored block
    ref = oracle.mlp_shard_partials(x[rows], w1[0], w2[0], 1, "gelu")[0]
    assert_close(got[rows], ref, "gpt3 shard partial sampled rows")


def test_decode_mlp_full_size():
    wl = WORKLOADS["decode_mlp"]
    width = wl.F // wl.N
    xb, x = normal_bf16((wl.M, wl.d), 1.0, wl.wid, 0)
    w1b, w1 = normal_bf16((wl.N, wl.d, width), 0.02, wl.wid, 1)
    w2b, w2 = normal_bf16((wl.N, width, wl.d), 0.02, wl.wid, 2)
    note("decode mlp full size: X [16,8192], W1 8x[8192,3584], W2 8x[3584,8192]")
    got = host(tp.mlp(bf16_tensor(xb), bf16_tensor(w1b), bf16_tensor(w2b), wl.N))
    w1full = np.concatenate(list(w1), axis=1)
    w2full = np.concatenate(list(w2), axis=0)
    assert_close(got, oracle.mlp(x, w1full, w2full, wl.N, "gelu"), "decode mlp")
