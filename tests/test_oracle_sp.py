"""Pins of the oracle's sequence-parallel LayerNorm path against facts that do not come from it.

Each pin returns True when the oracle agrees with:
  * pure-Python loops (statistics by explicit sums, math.sqrt) on small inputs,
    with and without residual and dropout;
  * closed forms: a constant row normalizes to zero, so its output is beta;
    a two-value row [a, b] normalizes to -+1 / sqrt(1 + eps / ((a - b) / 2)^2);
  * invariants: with eps = 0 the normalized row is unchanged by x -> alpha x + c
    (alpha > 0); the normalized row (gamma = 1, beta = 0) has mean 0 and
    variance var / (var + eps);
  * the token split ([TP-topic] "Sequence Parallelism Extension"): the token
    shards' results stacked in order (the all-gather) equal the computation
    over all tokens, and any shard range is the matching row slice; the
    reduce-scatter sums the partials in ascending order.
Mutation tests plant plausible mistakes and check that a pin fails for each.
"""
import math

import numpy as np
import pytest

from oracle import tp_oracle


def rng(seed):
    return np.random.default_rng([99, seed])


def loops(partials, residual, keep, p, gamma, beta, eps, rows):
    out_x, out_y = [], []
    d = len(gamma)
    for r in rows:
        x = [0.0] * d
        for pj in partials:
            for c in range(d):
                x[c] += float(pj[r][c])
        if keep is not None:
            x = [x[c] * float(keep[r][c]) / (1.0 - p) for c in range(d)]
        if residual is not None:
            x = [x[c] + float(residual[r][c]) for c in range(d)]
        mean = sum(x) / d
        var = sum((v - mean) ** 2 for v in x) / d
        out_x.append(x)
        out_y.append([(x[c] - mean) / math.sqrt(var + eps) * float(gamma[c]) + float(beta[c]) for c in range(d)])
    return np.array(out_x), np.array(out_y)


def pin_bruteforce_loops():
    g = rng(1)
    m, d, n = 8, 12, 4
    partials = [g.standard_normal((m, d)) for _ in range(n)]
    residual = g.standard_normal((m, d))
    keep = (g.random((m, d)) > 0.3).astype(np.float64)
    gamma, beta = g.standard_normal(d), g.standard_normal(d)
    ok = True
    for res, kp in ((None, None), (residual, None), (residual, keep)):
        for s0, ns in ((0, n), (1, 2)):
            x, y = tp_oracle.sp_layernorm(partials, res, kp, 0.3, gamma, beta, 1e-5, n, s0, ns)
            rows = range(s0 * (m // n), (s0 + ns) * (m // n))
            lx, ly = loops(partials, res, kp, 0.3, gamma, beta, 1e-5, rows)
            ok &= bool(np.allclose(x, lx, rtol=1e-13, atol=1e-13) and np.allclose(y, ly, rtol=1e-12, atol=1e-12))
    return ok


def pin_closed_forms():
    d = 6
    gamma, beta = np.linspace(0.5, 2.0, d), np.linspace(-1.0, 1.0, d)
    ok = bool(np.array_equal(tp_oracle.layernorm(np.full((1, d), 3.25), gamma, beta, 1e-5)[0], beta))
    a, b, eps = 2.0, -1.0, 1e-3
    y = tp_oracle.layernorm(np.array([[a, b]]), np.ones(2), np.zeros(2), eps)[0]
    want = 1.0 / math.sqrt(1.0 + eps / ((a - b) / 2.0) ** 2)
    ok &= abs(y[0] - want) < 1e-15 and abs(y[1] + want) < 1e-15
    return ok


def pin_invariants():
    g = rng(2)
    x = g.standard_normal((5, 16))
    ones, zeros = np.ones(16), np.zeros(16)
    base = tp_oracle.layernorm(x, ones, zeros, 0.0)
    ok = bool(np.allclose(tp_oracle.layernorm(3.5 * x + 7.0, ones, zeros, 0.0), base, rtol=1e-12, atol=1e-12))
    eps = 0.1
    y = tp_oracle.layernorm(x, ones, zeros, eps)
    var = np.var(x, axis=1)
    ok &= bool(np.allclose(y.mean(axis=1), 0.0, atol=1e-14))
    ok &= bool(np.allclose(y.var(axis=1), var / (var + eps), rtol=1e-12))
    return ok


def pin_token_split():
    g = rng(3)
    m, d, n = 12, 8, 3
    partials = [g.standard_normal((m, d)) for _ in range(4)]
    residual = g.standard_normal((m, d))
    gamma, beta = g.standard_normal(d), g.standard_normal(d)
    xa, ya = tp_oracle.sp_layernorm(partials, residual, None, 0.0, gamma, beta, 1e-5, 1)  # one shard: all tokens
    # the reduce-scatter written out here, in ascending partial order
    total = partials[0].copy()
    for pj in partials[1:]:
        total = total + pj
    ok = bool(np.array_equal(xa, total + residual))
    shards = [tp_oracle.sp_layernorm(partials, residual, None, 0.0, gamma, beta, 1e-5, n, s, 1) for s in range(n)]
    ok &= bool(np.array_equal(tp_oracle.all_gather_rows([t[1] for t in shards]), ya))
    ok &= bool(np.array_equal(tp_oracle.all_gather_rows([t[0] for t in shards]), xa))
    x12, y12 = tp_oracle.sp_layernorm(partials, residual, None, 0.0, gamma, beta, 1e-5, n, 1, 2)
    ok &= bool(np.array_equal(y12, ya[4:12]) and np.array_equal(x12, xa[4:12]))
    return ok


PINS = {
    "bruteforce_loops": pin_bruteforce_loops,
    "closed_forms": pin_closed_forms,
    "invariants": pin_invariants,
    "token_split": pin_token_split,
}


def run_pins():
    out = {}
    for name, fn in PINS.items():
        try:
            out[name] = bool(fn())
        except Exception:
            out[name] = False
    return out


@pytest.mark.parametrize("name", sorted(PINS))
def test_sp_pin(name):
    assert PINS[name](), name


# ----------------------------------------------------------------------------- mutations

ORIG_LN = tp_oracle.layernorm
ORIG_SP = tp_oracle.sp_layernorm
ORIG_ROWS = tp_oracle.token_rows


def _ln_unbiased(x, gamma, beta, eps):
    x = tp_oracle.widen(x)
    mean = np.mean(x, axis=1, keepdims=True)
    var = np.var(x, axis=1, keepdims=True, ddof=1)
    return (x - mean) / np.sqrt(var + eps) * gamma + beta


def _ln_eps_outside(x, gamma, beta, eps):
    x = tp_oracle.widen(x)
    mean = np.mean(x, axis=1, keepdims=True)
    var = np.mean((x - mean) ** 2, axis=1, keepdims=True)
    return (x - mean) / (np.sqrt(var) + eps) * gamma + beta


def _ln_wrong_axis(x, gamma, beta, eps):
    x = tp_oracle.widen(x)
    mean = np.mean(x, axis=0, keepdims=True)
    var = np.mean((x - mean) ** 2, axis=0, keepdims=True)
    return (x - mean) / np.sqrt(var + eps) * gamma + beta


def _rows_shifted(m, n, s):
    r = m // n
    return slice(((s + 1) % n) * r, ((s + 1) % n + 1) * r)


def _sp_no_dropout_scale(partials, residual, keep, p_drop, gamma, beta, eps, n, s0=0, ns=None):
    return ORIG_SP(partials, residual, keep, 0.0, gamma, beta, eps, n, s0, ns)


def _sp_residual_dropped(partials, residual, keep, p_drop, gamma, beta, eps, n, s0=0, ns=None):
    return ORIG_SP(partials, None, keep, p_drop, gamma, beta, eps, n, s0, ns)


MUTATIONS = {
    "unbiased_variance": ("layernorm", _ln_unbiased),
    "eps_outside_sqrt": ("layernorm", _ln_eps_outside),
    "stats_over_tokens": ("layernorm", _ln_wrong_axis),
    "token_rows_shifted": ("token_rows", _rows_shifted),
    "dropout_not_rescaled": ("sp_layernorm", _sp_no_dropout_scale),
    "residual_dropped": ("sp_layernorm", _sp_residual_dropped),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_sp_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(tp_oracle, attr, fn)
    results = run_pins()
    assert not all(results.values()), f"mutation {name} passed every pin: {results}"
