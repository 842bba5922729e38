"""Pins of the oracle's backward passes against facts that do not come from those functions.

Each pin returns True when the backward oracle agrees with:
  * central finite differences of the forward oracle (itself pinned in
    test_oracle.py) for the column split, the row split and the MLP pair with
    and without GeLU: the gradient of L = sum(G * f(X, W)) is, by definition,
    the limit of (L(W + h E) - L(W - h E)) / 2h;
  * the unsharded gradients dY W^T and X^T dY for every shard count that
    divides the split dimension (integer inputs, exact), and the
    shard-range subsets as slices of the full-range results;
  * pure-Python loops for dY W^T and X^T dY on small integers;
  * closed-form facts of the GeLU derivative: GeLU'(0) = 1/2,
    GeLU'(x) + GeLU'(-x) = 1, textbook values Phi(1) + phi(1), and finite
    differences of the pinned GeLU.
The mutation tests plant plausible mistakes in the backward oracle (on the
CPU) and check that at least one pin fails for each.
"""
import math

import numpy as np
import pytest

from oracle import tp_oracle
from synthetic import int_uniform_f32

# ----------------------------------------------------------------------------- helpers


def fd_grad(loss, a, h=1e-5):
    """Central finite-difference gradient of the scalar function loss(a) at a (float64)."""
    a = np.array(a, dtype=np.float64)
    g = np.zeros_like(a)
    for idx in np.ndindex(*a.shape):
        e = np.zeros_like(a)
        e[idx] = h
        g[idx] = (loss(a + e) - loss(a - e)) / (2 * h)
    return g


def close(a, b, rtol=1e-6, atol=1e-7):
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    return a.shape == b.shape and bool(np.allclose(a, b, rtol=rtol, atol=atol))


def rng(seed):
    return np.random.default_rng([77, seed])


# ----------------------------------------------------------------------------- pins


def pin_col_finite_differences():
    g = rng(1)
    x, w = g.standard_normal((3, 4)), g.standard_normal((4, 6))
    n = 3
    dy = g.standard_normal((3, 6))
    partials, dws = tp_oracle.col_linear_backward(x, w, dy, n)
    dx = tp_oracle.reduce_sum(partials)
    dw = tp_oracle.concat_cols(dws)
    fx = fd_grad(lambda a: float(np.sum(dy * tp_oracle.col_linear(a, w, n))), x)
    fw = fd_grad(lambda b: float(np.sum(dy * tp_oracle.col_linear(x, b, n))), w)
    return close(dx, fx) and close(dw, fw)


def pin_row_finite_differences():
    g = rng(2)
    x, w = g.standard_normal((3, 6)), g.standard_normal((6, 4))
    n = 3
    dy = g.standard_normal((3, 4))
    dxs, dws = tp_oracle.row_linear_backward(x, w, dy, n)
    dx = tp_oracle.concat_cols(dxs)
    dw = np.vstack(dws)
    fx = fd_grad(lambda a: float(np.sum(dy * tp_oracle.row_linear(a, w, n))), x)
    fw = fd_grad(lambda b: float(np.sum(dy * tp_oracle.row_linear(x, b, n))), w)
    return close(dx, fx) and close(dw, fw)


def pin_mlp_finite_differences():
    ok = True
    for act in ("gelu", "none"):
        g = rng(3 if act == "gelu" else 4)
        x, w1, w2 = g.standard_normal((3, 4)), g.standard_normal((4, 6)), g.standard_normal((6, 5))
        n = 2
        dy = g.standard_normal((3, 5))
        dx, dw1, dw2 = tp_oracle.mlp_backward(x, w1, w2, dy, n, act)
        f = lambda a, b, c: float(np.sum(dy * tp_oracle.mlp(a, b, c, n, act)))  # noqa: E731
        ok &= close(dx, fd_grad(lambda a: f(a, w1, w2), x))
        ok &= close(dw1, fd_grad(lambda b: f(x, b, w2), w1))
        ok &= close(dw2, fd_grad(lambda c: f(x, w1, c), w2))
    return ok


def pin_unsharded_every_divisor():
    x = int_uniform_f32((5, 12), -3, 3, 90, 0)
    w = int_uniform_f32((12, 12), -3, 3, 90, 1)
    dy = int_uniform_f32((5, 12), -3, 3, 90, 2)
    dxt = tp_oracle.widen(dy) @ tp_oracle.widen(w).T  # written out here, not the oracle's matmul
    dwt = tp_oracle.widen(x).T @ tp_oracle.widen(dy)
    ok = True
    for n in (1, 2, 3, 4, 6, 12):
        partials, dws = tp_oracle.col_linear_backward(x, w, dy, n)
        ok &= np.array_equal(sum(partials), dxt)
        ok &= np.array_equal(np.concatenate(dws, axis=1), dwt)
        dxs, dws = tp_oracle.row_linear_backward(x, w, dy, n)
        ok &= np.array_equal(np.concatenate(dxs, axis=1), dxt)
        ok &= np.array_equal(np.vstack(dws), dwt)
        # a shard range is the matching slice of the full-range result
        if n >= 3:
            k = 12 // n
            p_sub, dw_sub = tp_oracle.col_linear_backward(x, w, np.asarray(dy)[:, k:3 * k], n, 1, 2)
            ok &= np.array_equal(p_sub[0], tp_oracle.widen(dy)[:, k:2 * k] @ tp_oracle.widen(w)[:, k:2 * k].T)
            ok &= np.array_equal(np.concatenate(dw_sub, axis=1), dwt[:, k:3 * k])
            dx_sub, dw_sub = tp_oracle.row_linear_backward(x, w, dy, n, 1, 2)
            ok &= np.array_equal(np.concatenate(dx_sub, axis=1), dxt[:, k:3 * k])
            ok &= np.array_equal(np.vstack(dw_sub), dwt[k:3 * k, :])
    return bool(ok)


def pin_bruteforce_loops():
    xa = int_uniform_f32((3, 4), -2, 2, 91, 0)
    wa = int_uniform_f32((4, 6), -2, 2, 91, 1)
    dya = int_uniform_f32((3, 6), -2, 2, 91, 2)
    x, w, dy_col = xa.tolist(), wa.tolist(), dya.tolist()
    n = 2
    # column split: dX = dY W^T summed over shards, dW = X^T dY
    dx = [[sum(dy_col[i][j] * w[k][j] for j in range(6)) for k in range(4)] for i in range(3)]
    dw = [[sum(x[i][k] * dy_col[i][j] for i in range(3)) for j in range(6)] for k in range(4)]
    partials, dws = tp_oracle.col_linear_backward(xa, wa, dya, n)
    ok = np.array_equal(tp_oracle.reduce_sum(partials), np.array(dx))
    ok &= np.array_equal(tp_oracle.concat_cols(dws), np.array(dw))
    # row split: X [3, 4] split in 2 along its columns, W [4, 6] by rows
    dxs, dws = tp_oracle.row_linear_backward(xa, wa, dya, n)
    ok &= np.array_equal(tp_oracle.concat_cols(dxs), np.array(dx))
    ok &= np.array_equal(np.vstack(dws), np.array(dw))
    return bool(ok)


def _phi(x):
    return math.exp(-0.5 * x * x) / math.sqrt(2 * math.pi)


def pin_gelu_grad_facts():
    ok = float(tp_oracle.gelu_grad(np.array([0.0]))[0]) == 0.5
    xs = np.linspace(-8, 8, 161)
    ok &= bool(np.allclose(tp_oracle.gelu_grad(xs) + tp_oracle.gelu_grad(-xs), 1.0, rtol=0, atol=1e-15))
    # Phi(1) and phi(1) from tables of the standard normal distribution
    ok &= abs(float(tp_oracle.gelu_grad(np.array([1.0]))[0]) - (0.8413447460685429 + 0.24197072451914337)) < 1e-15
    ok &= abs(float(tp_oracle.gelu_grad(np.array([-2.0]))[0]) - (0.022750131948179195 - 2 * _phi(2.0))) < 1e-15
    h = 1e-5
    fd = (tp_oracle.gelu(xs + h) - tp_oracle.gelu(xs - h)) / (2 * h)
    ok &= bool(np.allclose(fd, tp_oracle.gelu_grad(xs), rtol=0, atol=1e-9))
    return bool(ok)


PINS = {
    "col_finite_differences": pin_col_finite_differences,
    "row_finite_differences": pin_row_finite_differences,
    "mlp_finite_differences": pin_mlp_finite_differences,
    "unsharded_every_divisor": pin_unsharded_every_divisor,
    "bruteforce_loops": pin_bruteforce_loops,
    "gelu_grad_facts": pin_gelu_grad_facts,
}


def run_pins():
    results = {}
    for name, fn in PINS.items():
        try:
            results[name] = bool(fn())
        except Exception:  # a crash is a failed pin
            results[name] = False
    return results


@pytest.mark.parametrize("name", sorted(PINS))
def test_backward_pin(name):
    assert PINS[name](), name


# ----------------------------------------------------------------------------- mutations

ORIG = {name: getattr(tp_oracle, name) for name in ("gelu_grad", "col_block", "x_block", "reduce_sum")}


def _mut_gelu_grad_sign(x):
    x = tp_oracle.widen(x)
    return ORIG["gelu_grad"](x) - 2 * x * np.exp(-0.5 * x * x) / np.sqrt(2 * np.pi)


def _mut_gelu_grad_cdf_only(x):
    x = tp_oracle.widen(x)
    return ORIG["gelu_grad"](x) - x * np.exp(-0.5 * x * x) / np.sqrt(2 * np.pi)


def _mut_col_bwd_pairing(x, w, dy, n, s0=0, ns=None):
    ns = n - s0 if ns is None else ns
    dys = tp_oracle.split_cols(dy, ns)
    partials = [tp_oracle.matmul(dys[j], tp_oracle.transpose(ORIG["col_block"](w, n, (s0 + j + 1) % n)))
                for j in range(ns)]
    dws = [tp_oracle.matmul(tp_oracle.transpose(x), dys[j]) for j in range(ns)]
    return partials, dws


def _mut_row_bwd_dw_block(x, w, dy, n, s0=0, ns=None):
    ns = n - s0 if ns is None else ns
    dxs = [tp_oracle.matmul(dy, tp_oracle.transpose(tp_oracle.row_block(w, n, s))) for s in range(s0, s0 + ns)]
    dws = [tp_oracle.matmul(tp_oracle.transpose(ORIG["x_block"](x, n, (s + 1) % n)), dy) for s in range(s0, s0 + ns)]
    return dxs, dws


def _mut_mlp_bwd_grad_of_h(x, w1, w2, dy, n, act="gelu", s0=0, ns=None):
    # the activation derivative taken at H = act(Z) instead of Z
    ns = n - s0 if ns is None else ns
    partials, dw1, dw2 = [], [], []
    dy = tp_oracle.widen(dy)
    for s in range(s0, s0 + ns):
        w1s, w2s = tp_oracle.col_block(w1, n, s), tp_oracle.row_block(w2, n, s)
        z = tp_oracle.matmul(x, w1s)
        h = tp_oracle.apply_act(z, act)
        dz = tp_oracle.matmul(dy, tp_oracle.transpose(w2s)) * tp_oracle.act_grad(h, act)
        dw2.append(tp_oracle.matmul(tp_oracle.transpose(h), dy))
        dw1.append(tp_oracle.matmul(tp_oracle.transpose(x), dz))
        partials.append(tp_oracle.matmul(dz, tp_oracle.transpose(w1s)))
    return tp_oracle.reduce_sum(partials), tp_oracle.concat_cols(dw1), np.vstack(dw2)


def _mut_reduce_drop_last(partials):
    partials = list(partials)
    return ORIG["reduce_sum"](partials[:-1] if len(partials) > 1 else partials)


def _mut_transpose_square_only(a):
    a = tp_oracle.widen(a)
    return a if a.shape[0] == a.shape[1] else a.T


MUTATIONS = {
    "gelu_grad_sign": ("gelu_grad", _mut_gelu_grad_sign),
    "gelu_grad_cdf_only": ("gelu_grad", _mut_gelu_grad_cdf_only),
    "col_bwd_pairing": ("col_linear_backward", _mut_col_bwd_pairing),
    "row_bwd_dw_block": ("row_linear_backward", _mut_row_bwd_dw_block),
    "mlp_bwd_grad_of_h": ("mlp_backward", _mut_mlp_bwd_grad_of_h),
    "reduce_drop_last": ("reduce_sum", _mut_reduce_drop_last),
    "transpose_square_only": ("transpose", _mut_transpose_square_only),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_backward_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(tp_oracle, attr, fn)
    results = run_pins()
    assert not all(results.values()), f"mutation {name} passed every pin: {results}"
