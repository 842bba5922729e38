"""Pins of the float64 oracle against facts that do not come from the oracle itself.

Each pin is a function returning True when the oracle agrees with:
  * the worked example printed on the "Tensor Parallelism" entry of the AI
    Glossary (aiforbusinessandlife.com), section "Worked example";
  * pure-Python triple loops on small integer matrices (brute force);
  * the split invariants (concatenated column shards and summed row partials
    both equal the unsharded product) for every shard count dividing the
    split dimension, with each shard's block located by explicit index loops;
  * textbook values of the standard normal CDF and an independent
    Taylor-series error function for GeLU;
  * the MLP chain reduced to plain products (no activation) and, with GeLU,
    a pure-Python evaluation of the whole chain on tiny inputs;
  * row independence (a sampled row equals the same row of the full result).
The mutation tests at the end plant plausible mistakes in the oracle (on the
CPU) and check that at least one pin fails for each.
"""
import json
import math
import os
from decimal import Decimal, getcontext

import numpy as np
import pytest

import oracle
from oracle import tp_oracle
from synthetic import int_uniform_f32, normal_bf16, sample_rows

# ----------------------------------------------------------------------------- helpers


def bf_matmul(a, b):
    """Pure-Python triple loop, k ascending (independent of numpy's product)."""
    m, k = len(a), len(a[0]) if a else 0
    n = len(b[0]) if b else 0
    out = [[0.0] * n for _ in range(m)]
    for i in range(m):
        for j in range(n):
            acc = 0.0
            for t in range(k):
                acc += float(a[i][t]) * float(b[t][j])
            out[i][j] = acc
    return out


def tolist(a):
    return np.asarray(a, dtype=np.float64).tolist()


getcontext().prec = 60
_PI = Decimal("3.14159265358979323846264338327950288419716939937510582097494459")


def series_erf(x: float) -> float:
    """erf by its Maclaurin series, 2/sqrt(pi) * sum (-1)^n x^(2n+1) / (n! (2n+1)), in 60-digit decimals."""
    xd = Decimal(repr(x))
    total = Decimal(0)
    term = xd  # x^(2n+1) / n!
    n = 0
    while True:
        contrib = term / (2 * n + 1)
        total += contrib if n % 2 == 0 else -contrib
        n += 1
        term = term * xd * xd / n
        if abs(term) < Decimal(10) ** -50 and n > 5:
            break
    return float(2 * total / _PI.sqrt())


def series_gelu(x: float) -> float:
    return 0.5 * x * (1.0 + series_erf(x / math.sqrt(2.0)))


# Standard normal CDF values from printed tables (textbook constants).
PHI_TABLE = {
    0.0: 0.5,
    0.5: 0.6914624612740131,
    1.0: 0.8413447460685429,
    1.5: 0.9331927987311419,
    2.0: 0.9772498680518208,
    3.0: 0.9986501019683699,
}

# ----------------------------------------------------------------------------- pins


def load_worked(golden_dir):
    with open(os.path.join(golden_dir, "worked_example.json")) as f:
        return json.load(f)


def pin_worked_example(golden_dir) -> bool:
    g = load_worked(golden_dir)
    x = np.array(g["X"], dtype=np.float32)
    w = np.array(g["W"], dtype=np.float32)
    n = g["N"]
    y = np.array(g["Y"], dtype=np.float64)
    ok = np.array_equal(tp_oracle.matmul(x, w), y)
    cols = tp_oracle.col_shard_outputs(x, w, n)
    ok &= len(cols) == n and all(np.array_equal(c, np.array(e)) for c, e in zip(cols, g["col_shard_outputs"]))
    ok &= np.array_equal(tp_oracle.col_linear(x, w, n), y)
    parts = tp_oracle.row_partials(x, w, n)
    ok &= len(parts) == n and all(np.array_equal(p, np.array(e)) for p, e in zip(parts, g["row_partials"]))
    ok &= np.array_equal(tp_oracle.row_linear(x, w, n), y)
    # the combine rule: the row partials share the output's coordinates (added),
    # the column outputs hold disjoint coordinates (concatenated)
    ok &= all(p.shape == y.shape for p in parts)
    ok &= sum(c.shape[1] for c in cols) == y.shape[1]
    return bool(ok)


def pin_bruteforce_matmul() -> bool:
    g = np.random.default_rng(11)
    for m in range(1, 6):
        for k in range(1, 6):
            for n in range(1, 6):
                a = g.integers(-4, 5, size=(m, k)).astype(np.float32)
                b = g.integers(-4, 5, size=(k, n)).astype(np.float32)
                if tolist(tp_oracle.matmul(a, b)) != bf_matmul(tolist(a), tolist(b)):
                    return False
    return True


def divisors(v):
    return [d for d in range(1, v + 1) if v % d == 0]


def pin_split_invariants() -> bool:
    g = np.random.default_rng(12)
    for (m, k, nout) in [(3, 8, 12), (2, 6, 6), (1, 4, 10), (4, 12, 8)]:
        x = g.integers(-4, 5, size=(m, k)).astype(np.float32)
        w = g.integers(-4, 5, size=(k, nout)).astype(np.float32)
        full = bf_matmul(tolist(x), tolist(w))
        wl, xl = tolist(w), tolist(x)
        for n in divisors(nout):
            width = nout // n
            outs = tp_oracle.col_shard_outputs(x, w, n)
            for s, o in enumerate(outs):
                blk = [[wl[r][c] for c in range(s * width, (s + 1) * width)] for r in range(k)]
                if tolist(o) != bf_matmul(xl, blk):
                    return False
            if tolist(tp_oracle.col_linear(x, w, n)) != full:
                return False
            # a sub-range of shards
            if n >= 2:
                sub = tp_oracle.col_linear(x, w, n, s0=1, ns=n - 1)
                want = [row[width:] for row in full]
                if tolist(sub) != want:
                    return False
        for n in divisors(k):
            height = k // n
            parts = tp_oracle.row_partials(x, w, n)
            for s, p in enumerate(parts):
                xs = [[xl[r][c] for c in range(s * height, (s + 1) * height)] for r in range(m)]
                ws = [wl[r] for r in range(s * height, (s + 1) * height)]
                if tolist(p) != bf_matmul(xs, ws):
                    return False
            if tolist(tp_oracle.row_linear(x, w, n)) != full:
                return False
    return True


def pin_gelu() -> bool:
    ok = True
    for x, phi in PHI_TABLE.items():
        ok &= abs(float(tp_oracle.gelu(np.array([x]))[0]) - x * phi) <= 1e-15 * max(1.0, abs(x))
        ok &= abs(float(tp_oracle.gelu(np.array([-x]))[0]) - (-x) * (1.0 - phi)) <= 1e-15 * max(1.0, abs(x))
    grid = np.linspace(-6.0, 6.0, 97)
    got = tp_oracle.gelu(grid)
    # odd part: gelu(x) - gelu(-x) = x
    ok &= bool(np.all(np.abs((got - tp_oracle.gelu(-grid)) - grid) <= 1e-14 * np.maximum(1.0, np.abs(grid))))
    for x, v in zip(grid.tolist(), got.tolist()):
        ok &= abs(v - series_gelu(x)) <= 1e-13 * max(1.0, abs(x))
    return bool(ok)


def pin_mlp() -> bool:
    g = np.random.default_rng(13)
    ok = True
    for (m, d, f, n) in [(3, 6, 8, 2), (2, 4, 12, 3), (4, 8, 8, 4), (1, 5, 6, 6)]:
        x = g.integers(-1, 2, size=(m, d)).astype(np.float32)
        w1 = g.integers(-1, 2, size=(d, f)).astype(np.float32)
        w2 = g.integers(-2, 3, size=(f, d)).astype(np.float32)
        full = bf_matmul(bf_matmul(tolist(x), tolist(w1)), tolist(w2))
        ok &= tolist(tp_oracle.mlp(x, w1, w2, n, act="none")) == full
        # with GeLU: pure-Python chain with the series erf, shard by shard
        xl, w1l, w2l = tolist(x), tolist(w1), tolist(w2)
        width = f // n
        want = [[0.0] * d for _ in range(m)]
        for s in range(n):
            cols = range(s * width, (s + 1) * width)
            h = [[series_gelu(sum(xl[i][t] * w1l[t][c] for t in range(d))) for c in cols] for i in range(m)]
            p = [[sum(h[i][j] * w2l[s * width + j][c] for j in range(width)) for c in range(d)] for i in range(m)]
            want = [[want[i][c] + p[i][c] for c in range(d)] for i in range(m)]
        got = tp_oracle.mlp(x, w1, w2, n, act="gelu")
        ok &= bool(np.max(np.abs(got - np.array(want))) <= 1e-12)
        # a proper sub-range of shards is the same sum restricted to those shards
        if n >= 2:
            sub = tp_oracle.mlp(x, w1, w2, n, act="none", s0=1, ns=n - 1)
            w1s = w1[:, width:]
            w2s = w2[width:, :]
            ok &= tolist(sub) == bf_matmul(bf_matmul(xl, tolist(w1s)), tolist(w2s))
    return bool(ok)


def pin_sampled_rows() -> bool:
    _, x = normal_bf16((40, 32), 1.0, 99, 0)
    _, w1 = normal_bf16((32, 64), 0.02, 99, 1)
    _, w2 = normal_bf16((64, 24), 0.02, 99, 2)
    rows = sample_rows(40, 7, seed=3)
    full = tp_oracle.mlp(x, w1, w2, 4)
    part = tp_oracle.mlp(x[rows], w1, w2, 4)
    return bool(np.array_equal(full[rows], part))


ALL_PINS = ["worked", "bruteforce", "split", "gelu", "mlp", "rows"]


def run_pins(golden_dir):
    return {
        "worked": pin_worked_example(golden_dir),
        "bruteforce": pin_bruteforce_matmul(),
        "split": pin_split_invariants(),
        "gelu": pin_gelu(),
        "mlp": pin_mlp(),
        "rows": pin_sampled_rows(),
    }


# ----------------------------------------------------------------------------- tests


def test_worked_example(golden_dir):
    assert pin_worked_example(golden_dir)


def test_matmul_bruteforce():
    assert pin_bruteforce_matmul()


def test_split_invariants_every_divisor():
    assert pin_split_invariants()


def test_gelu_textbook_and_series():
    assert pin_gelu()


def test_mlp_chain():
    assert pin_mlp()


def test_sampled_rows_are_exact():
    assert pin_sampled_rows()


def test_uneven_split_rejected():
    x = np.ones((2, 6), np.float32)
    w = np.ones((6, 10), np.float32)
    with pytest.raises(ValueError):
        tp_oracle.col_linear(x, w, 4)
    with pytest.raises(ValueError):
        tp_oracle.row_linear(x, w, 4)


def test_split_check_workload_exact_and_integer():
    """The tiny split-check workload: integer results, exactly representable in float32."""
    x = int_uniform_f32((4, 64), -4, 4, 1, 0)
    w = int_uniform_f32((64, 128), -4, 4, 1, 1)
    y = oracle.matmul(x, w)
    assert np.array_equal(oracle.col_linear(x, w, 2), y)
    assert np.array_equal(oracle.row_linear(x, w, 2), y)
    assert np.all(y == np.round(y)) and np.max(np.abs(y)) < 2 ** 24


# ----------------------------------------------------------------------------- mutations


def _mut_col_block_shift(w, n, s):
    return ORIG["col_block"](w, n, (s + 1) % n)


def _mut_row_block_strided(w, n, s):
    w = np.asarray(w)
    return w[s::n, :]


def _mut_reduce_drop_last(partials):
    partials = list(partials)
    return ORIG["reduce_sum"](partials[:-1] if len(partials) > 1 else partials)


def _mut_reduce_subtract(partials):
    partials = list(partials)
    total = tp_oracle.widen(partials[0]).copy()
    for p in partials[1:]:
        total = total - tp_oracle.widen(p)
    return total


def _mut_gelu_sign(x):
    x = tp_oracle.widen(x)
    from scipy.special import erf

    return 0.5 * x * (1.0 - erf(x / np.sqrt(2.0)))


def _mut_gelu_scale(x):
    x = tp_oracle.widen(x)
    from scipy.special import erf

    return 0.5 * x * (1.0 + erf(x / 2.0))


def _mut_matmul_drop_k(a, b):
    a = tp_oracle.widen(a)
    b = tp_oracle.widen(b)
    if a.shape[1] <= 1:
        return a @ b * 0.5
    return a[:, :-1] @ b[:-1, :]


def _mut_matmul_transposed(a, b):
    a = tp_oracle.widen(a)
    b = tp_oracle.widen(b)
    if b.shape[0] == b.shape[1]:
        return a @ b.T
    return a @ b + 1e-3


def _mut_concat_reversed(blocks):
    return np.concatenate([tp_oracle.widen(b) for b in list(blocks)[::-1]], axis=1)


def _mut_mlp_pairing(x, w1, w2, n, act="gelu", s0=0, ns=None):
    ns = n - s0 if ns is None else ns
    out = []
    for s in range(s0, s0 + ns):
        h = tp_oracle.apply_act(tp_oracle.matmul(x, tp_oracle.col_block(w1, n, s)), act)
        out.append(tp_oracle.matmul(h, tp_oracle.row_block(w2, n, (s + 1) % n)))
    return out


ORIG = {name: getattr(tp_oracle, name) for name in ("col_block", "reduce_sum")}

MUTATIONS = {
    "col_block_shift": ("col_block", _mut_col_block_shift),
    "row_block_strided": ("row_block", _mut_row_block_strided),
    "reduce_drop_last": ("reduce_sum", _mut_reduce_drop_last),
    "reduce_subtract": ("reduce_sum", _mut_reduce_subtract),
    "gelu_sign": ("gelu", _mut_gelu_sign),
    "gelu_scale": ("gelu", _mut_gelu_scale),
    "matmul_drop_k": ("matmul", _mut_matmul_drop_k),
    "matmul_transposed": ("matmul", _mut_matmul_transposed),
    "concat_reversed": ("concat_cols", _mut_concat_reversed),
    "mlp_pairing": ("mlp_shard_partials", _mut_mlp_pairing),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch, golden_dir):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(tp_oracle, attr, fn)
    results = run_pins(golden_dir)
    assert not all(results.values()), f"mutation {name} passed every pin: {results}"
