"""Pins of the oracle's attention per head subset against facts that do not come from it.

Each pin returns True when the oracle agrees with:
  * pure-Python loops (math.exp, no numpy products) on tiny inputs, causal and not;
  * closed forms: with every key identical the softmax is uniform, so each
    output row is the mean of the value rows it may see (all of them, or the
    prefix up to itself when causal); the first token of a causal sequence
    sees only itself, so its output is its own value row;
  * invariants: sequences are independent (a batch equals its sequences run
    alone); adding one vector to every key adds a constant to each query's
    scores and changes nothing; outputs are convex combinations of value rows;
  * the pages' head split: the shards' outputs concatenated equal unsharded
    attention over all heads, for multi-head and for grouped-query attention
    with the key/value heads split or replicated ([TP-topic] figure "Tensor
    Parallelism — Split Layers Across GPUs", panel "Attention Head Parallelism").
Mutation tests plant plausible mistakes and check that a pin fails for each.
"""
import math

import numpy as np
import pytest

from oracle import tp_oracle


def rng(seed):
    return np.random.default_rng([88, seed])


def loops_attention(qkv, hq, hkv, dh, seq_len, causal):
    """Pure-Python reference: explicit loops over sequences, heads, queries and keys."""
    qkv = [[float(v) for v in row] for row in np.asarray(qkv, dtype=np.float64)]
    m = len(qkv)
    out = [[0.0] * (hq * dh) for _ in range(m)]
    group = hq // hkv
    for r0 in range(0, m, seq_len):
        for h in range(hq):
            kv = h // group
            for i in range(seq_len):
                qi = qkv[r0 + i][h * dh:(h + 1) * dh]
                last = i if causal else seq_len - 1
                scores = []
                for j in range(last + 1):
                    kj = qkv[r0 + j][(hq + kv) * dh:(hq + kv + 1) * dh]
                    scores.append(sum(a * b for a, b in zip(qi, kj)) / math.sqrt(dh))
                mx = max(scores)
                ws = [math.exp(sc - mx) for sc in scores]
                tot = sum(ws)
                for c in range(dh):
                    acc = 0.0
                    for j in range(last + 1):
                        acc += ws[j] * qkv[r0 + j][(hq + hkv + kv) * dh + c]
                    out[r0 + i][h * dh + c] = acc / tot
    return np.array(out)


def pin_bruteforce_loops():
    ok = True
    for causal in (True, False):
        g = rng(1 if causal else 2)
        hq, hkv, dh, L = 4, 2, 3, 4
        qkv = g.standard_normal((2 * L, (hq + 2 * hkv) * dh))
        got = tp_oracle.attention_shard(qkv, hq, hkv, dh, L, causal)
        ok &= bool(np.allclose(got, loops_attention(qkv, hq, hkv, dh, L, causal), rtol=1e-12, atol=1e-12))
    return ok


def pin_closed_forms():
    g = rng(3)
    hq, hkv, dh, L = 2, 2, 4, 6
    qkv = g.standard_normal((L, (hq + 2 * hkv) * dh))
    k0 = hq * dh
    qkv[:, k0:k0 + hkv * dh] = qkv[0, k0:k0 + hkv * dh]  # every key identical
    ok = True
    for causal in (False, True):
        got = tp_oracle.attention_shard(qkv, hq, hkv, dh, L, causal)
        for h in range(hq):
            v = qkv[:, (hq + hkv + h) * dh:(hq + hkv + h + 1) * dh]
            want = np.cumsum(v, axis=0) / np.arange(1, L + 1)[:, None] if causal else np.tile(v.mean(0), (L, 1))
            ok &= bool(np.allclose(got[:, h * dh:(h + 1) * dh], want, rtol=1e-13, atol=1e-13))
    # the first token of a causal sequence returns its own value row, exactly
    qkv = g.standard_normal((2 * L, (hq + 2 * hkv) * dh))
    got = tp_oracle.attention_shard(qkv, hq, hkv, dh, L, True)
    for r0 in (0, L):
        for h in range(hq):
            ok &= bool(np.array_equal(got[r0, h * dh:(h + 1) * dh],
                                      qkv[r0, (hq + hkv + h) * dh:(hq + hkv + h + 1) * dh]))
    return ok


def pin_invariants():
    g = rng(4)
    hq, hkv, dh, L = 4, 1, 8, 7
    qkv = g.standard_normal((3 * L, (hq + 2 * hkv) * dh))
    ok = True
    for causal in (True, False):
        whole = tp_oracle.attention_shard(qkv, hq, hkv, dh, L, causal)
        alone = np.vstack([tp_oracle.attention_shard(qkv[r:r + L], hq, hkv, dh, L, causal) for r in range(0, 3 * L, L)])
        ok &= bool(np.array_equal(whole, alone))
        shifted = qkv.copy()
        shifted[:, hq * dh:(hq + hkv) * dh] += g.standard_normal(hkv * dh)  # the same vector added to every key
        ok &= bool(np.allclose(tp_oracle.attention_shard(shifted, hq, hkv, dh, L, causal), whole, rtol=1e-10,
                               atol=1e-10))
        v = qkv[:, (hq + hkv) * dh:]
        ok &= bool(np.all(whole <= np.max(v) + 1e-12) and np.all(whole >= np.min(v) - 1e-12))
    return ok


def pin_head_split():
    ok = True
    for heads, kv_heads, n in ((8, 8, 4), (8, 2, 4), (8, 1, 2), (12, 4, 2)):
        g = rng(10 + heads + kv_heads + n)
        dh, L = 4, 5
        full = g.standard_normal((2 * L, (heads + 2 * kv_heads) * dh))
        ref = tp_oracle.attention_shard(full, heads, kv_heads, dh, L, True)
        blocks = [full[:, tp_oracle.shard_qkv_columns(heads, kv_heads, dh, n, s)] for s in range(n)]
        got = tp_oracle.attention(np.concatenate(blocks, axis=1), n, heads, kv_heads, dh, L, True)
        ok &= bool(np.array_equal(got, ref))
        # a subset of shards gives the matching column blocks
        sub = tp_oracle.attention(np.concatenate(blocks[1:n], axis=1), n, heads, kv_heads, dh, L, True, 1, n - 1)
        ok &= bool(np.array_equal(sub, ref[:, (heads // n) * dh:]))
    return ok


PINS = {
    "bruteforce_loops": pin_bruteforce_loops,
    "closed_forms": pin_closed_forms,
    "invariants": pin_invariants,
    "head_split": pin_head_split,
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
def test_attention_pin(name):
    assert PINS[name](), name


# ----------------------------------------------------------------------------- mutations

ORIG_SHARD = tp_oracle.attention_shard


def _variant(scale=True, diag_masked=False, swap_kv=False, mod_group=False, ignore_seq=False, col_softmax=False):
    def fn(qkv_block, hq, hkv, head_dim, seq_len, causal=True):
        qkv_block = tp_oracle.widen(qkv_block)
        m_rows = qkv_block.shape[0]
        L = m_rows if ignore_seq else seq_len
        group = hq // hkv
        out = np.zeros((m_rows, hq * head_dim))
        koff, voff = hq * head_dim, (hq + hkv) * head_dim
        if swap_kv:
            koff, voff = voff, koff
        for r0 in range(0, m_rows, L):
            rows = slice(r0, r0 + L)
            for h in range(hq):
                kv = h % hkv if mod_group else h // group
                q = qkv_block[rows, h * head_dim:(h + 1) * head_dim]
                k = qkv_block[rows, koff + kv * head_dim:koff + (kv + 1) * head_dim]
                v = qkv_block[rows, voff + kv * head_dim:voff + (kv + 1) * head_dim]
                s = q @ k.T / (np.sqrt(head_dim) if scale else 1.0)
                if causal:
                    s = np.where(np.tril(np.ones((L, L), dtype=bool), -1 if diag_masked else 0), s, -np.inf)
                with np.errstate(invalid="ignore"):  # a planted mask can leave a row with no key
                    if col_softmax:
                        e = np.exp(s - np.max(s, axis=0, keepdims=True))
                        p = e / np.sum(e, axis=0, keepdims=True)
                    else:
                        e = np.exp(s - np.max(s, axis=1, keepdims=True))
                        p = e / np.sum(e, axis=1, keepdims=True)
                out[rows, h * head_dim:(h + 1) * head_dim] = np.nan_to_num(p) @ v
        return out

    return fn


MUTATIONS = {
    "no_scale": _variant(scale=False),
    "diagonal_masked": _variant(diag_masked=True),
    "k_v_swapped": _variant(swap_kv=True),
    "gqa_modulo_group": _variant(mod_group=True),
    "sequence_boundary_ignored": _variant(ignore_seq=True),
    "softmax_over_queries": _variant(col_softmax=True),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_attention_mistake_is_caught(name, monkeypatch):
    monkeypatch.setattr(tp_oracle, "attention_shard", MUTATIONS[name])
    results = run_pins()
    assert not all(results.values()), f"mutation {name} passed every pin: {results}"
