"""Host-side checks of the C interface (no GPU needed, no kernel is launched).

The library must load, export every function include/tp.h declares, and
reject every malformed call with its status before touching HIP. The device
pointers used here are fake: each call is built to fail validation, or is the
workspace-size query of tp_mlp, which enqueues nothing.
"""
import ctypes
import os
import re

import pytest

from tensor_sharded_linear_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tp.h")

F32, BF16 = _lib.TP_F32, _lib.TP_BF16
FAKE = 0x7F0000000000  # never dereferenced: every call below fails validation first


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tp_[a-z_]+)\s*\(", text)))


def m(ptr=FAKE, dtype=BF16, rows=4, cols=8, ld=None, stride=0):
    return _lib.matrix(ptr, dtype, rows, cols, cols if ld is None else ld, stride)


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_library_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(_lib.EXPORTS), names
    for name in names:
        assert hasattr(lib, name), name


def test_version_and_status_strings(lib):
    assert lib.tp_version() >> 16 == 1
    assert lib.tp_version() & 0xffff >= 1  # tp_sp_layernorm and TP_SPLIT_TOKENS
    for code, name in _lib.STATUS_NAMES.items():
        assert lib.tp_status_string(code).decode().startswith(name)
    assert lib.tp_status_string(999).decode() == "unknown tp_status"


def col(lib, X, W, N, s0, ns, act, Y):
    return lib.tp_col_linear(ctypes.byref(X) if X else None, ctypes.byref(W) if W else None, N, s0, ns, act,
                             ctypes.byref(Y) if Y else None, None)


def row(lib, X, W, N, s0, ns, P):
    return lib.tp_row_linear(ctypes.byref(X), ctypes.byref(W), N, s0, ns, ctypes.byref(P), None)


def test_col_linear_validation(lib):
    # X [4, 8], W [8, 16] split in 2 -> Y [4, 16]
    X = m(rows=4, cols=8)
    W = m(FAKE + (1 << 20), rows=8, cols=16)
    Y = m(FAKE + (2 << 20), rows=4, cols=16)
    assert col(lib, None, W, 2, 0, 2, 0, Y) == 1  # NULL descriptor
    assert col(lib, m(dtype=7), W, 2, 0, 2, 0, Y) == 2  # bad dtype
    assert col(lib, m(dtype=F32), W, 2, 0, 2, 0, Y) == 2  # X/W dtype mismatch
    assert col(lib, m(rows=4, cols=6), W, 2, 0, 2, 0, Y) == 3  # X.cols != W.rows
    assert col(lib, X, W, 2, 0, 2, 0, m(FAKE + (2 << 20), rows=4, cols=8)) == 3  # Y.cols != ns*Nout/N
    assert col(lib, X, W, 3, 0, 3, 0, Y) == 4  # 3 does not divide 16
    assert col(lib, X, W, 0, 0, 1, 0, Y) == 4  # N < 1
    assert col(lib, X, W, 2, 1, 2, 0, Y) == 5  # s0 + ns > N
    assert col(lib, X, W, 2, -1, 1, 0, Y) == 5
    assert col(lib, X, W, 2, 0, 0, 0, Y) == 5
    assert col(lib, X, m(FAKE + (1 << 20), rows=8, cols=16, ld=15), 2, 0, 2, 0, Y) == 6  # ld < row
    assert col(lib, m(rows=4, cols=8, stride=64), W, 2, 0, 2, 0, Y) == 6  # X may not be shard-major
    # shard-major W whose blocks overlap: blocks [8, 8] need stride >= 7*8+8 = 64
    assert col(lib, X, m(FAKE + (1 << 20), rows=8, cols=16, ld=8, stride=32), 2, 0, 2, 0, Y) == 6
    assert col(lib, X, W, 2, 0, 2, 0, m(FAKE + 16, rows=4, cols=16)) == 7  # Y overlaps X
    assert col(lib, X, W, 2, 0, 2, 5, Y) == 3  # unknown activation
    assert col(lib, X, m(0, rows=8, cols=16), 2, 0, 2, 0, Y) == 1  # NULL data pointer


def test_row_linear_validation(lib):
    X = m(rows=4, cols=8)
    W = m(FAKE + (1 << 20), rows=8, cols=16)
    P = m(FAKE + (2 << 20), dtype=F32, rows=4, cols=16, stride=64)
    assert row(lib, X, W, 2, 0, 2, m(FAKE + (2 << 20), dtype=BF16, rows=4, cols=16, stride=64)) == 2  # P not fp32
    assert row(lib, X, W, 3, 0, 3, P) == 4  # 3 does not divide K = 8
    assert row(lib, X, m(FAKE + (1 << 20), rows=6, cols=16), 2, 0, 2, P) == 3  # W.rows != K
    assert row(lib, X, W, 2, 0, 2, m(FAKE + (2 << 20), dtype=F32, rows=4, cols=16, stride=0)) == 6  # P overlap
    assert row(lib, X, W, 2, 0, 2, m(FAKE + (2 << 20), dtype=F32, rows=4, cols=16, stride=32)) == 6
    assert row(lib, X, W, 2, 2, 1, P) == 5
    assert row(lib, X, W, 2, 0, 2, m(FAKE + 8, dtype=F32, rows=4, cols=16, stride=64)) == 7  # P over X


def test_reduce_validation(lib):
    P = m(FAKE, dtype=F32, rows=4, cols=16, stride=64)
    Y = m(FAKE + (1 << 20), dtype=F32, rows=4, cols=16)
    red = lib.tp_reduce_partials
    assert red(None, 2, 1, ctypes.byref(Y), None) == 1
    assert red(ctypes.byref(m(FAKE, dtype=BF16, rows=4, cols=16, stride=64)), 2, 1, ctypes.byref(Y), None) == 2
    assert red(ctypes.byref(P), 0, 1, ctypes.byref(Y), None) == 4
    assert red(ctypes.byref(P), 2, 7, ctypes.byref(Y), None) == 3  # bad axis
    assert red(ctypes.byref(P), 2, 0, ctypes.byref(Y), None) == 3  # concat needs Y.cols = 32
    assert red(ctypes.byref(P), 2, 1, ctypes.byref(m(FAKE + (1 << 20), dtype=F32, rows=4, cols=16, stride=8)),
               None) == 6
    assert red(ctypes.byref(m(FAKE, dtype=F32, rows=4, cols=16, stride=16)), 2, 1, ctypes.byref(Y), None) == 6
    assert red(ctypes.byref(P), 2, 1, ctypes.byref(m(FAKE + 64, dtype=F32, rows=4, cols=16)), None) == 7


def mlp_query(lib, X, W1, W2, N, s0, ns, Y):
    size = ctypes.c_size_t(0)
    st = lib.tp_mlp(ctypes.byref(X), ctypes.byref(W1), ctypes.byref(W2), N, s0, ns, 1, None, ctypes.byref(size),
                    ctypes.byref(Y), None)
    return st, size.value


def test_mlp_validation_and_workspace_query(lib):
    M, d, F, N = 64, 32, 128, 4
    X = m(FAKE, rows=M, cols=d)
    W1 = m(FAKE + (1 << 20), rows=d, cols=F)
    W2 = m(FAKE + (2 << 20), rows=F, cols=d)
    Y = m(FAKE + (3 << 20), dtype=F32, rows=M, cols=d)
    st, size = mlp_query(lib, X, W1, W2, N, 0, N, Y)
    assert st == 0
    # H bf16 [64, 128] + fp32 partials [4][64][32], each rounded up to 256 bytes
    assert size == 64 * 128 * 2 + 4 * 64 * 32 * 4
    st, size1 = mlp_query(lib, X, W1, W2, N, 1, 1, Y)
    assert st == 0 and size1 == 64 * 32 * 2  # one shard writes Y directly: only H
    assert mlp_query(lib, X, W1, W2, 3, 0, 3, Y)[0] == 4
    assert mlp_query(lib, X, W1, W2, N, 3, 2, Y)[0] == 5
    assert mlp_query(lib, X, W1, W2, N, 0, N, m(FAKE + (3 << 20), dtype=BF16, rows=M, cols=d))[0] == 2
    assert mlp_query(lib, X, W1, m(FAKE + (2 << 20), rows=F, cols=d + 8), N, 0, N, Y)[0] == 3
    size = ctypes.c_size_t(16)
    st = lib.tp_mlp(ctypes.byref(X), ctypes.byref(W1), ctypes.byref(W2), N, 0, N, 1, ctypes.c_void_p(FAKE + (8 << 20)),
                    ctypes.byref(size), ctypes.byref(Y), None)
    assert st == 8  # workspace too small
    assert lib.tp_mlp(ctypes.byref(X), ctypes.byref(W1), ctypes.byref(W2), N, 0, N, 1, None, None,
                      ctypes.byref(Y), None) == 1


def test_mlp_narrow_decode_workspace_includes_k_chunks(lib):
    # 16 rows and narrow shards (few column tiles): the skinny kernel splits K
    # to fill the GPU, and its chunk sums live in the workspace.
    M, d, F, N = 16, 8192, 2048, 8
    X = m(FAKE, rows=M, cols=d)
    W1 = m(FAKE + (1 << 30), rows=d, cols=F, ld=F // N, stride=d * (F // N))
    W2 = m(FAKE + (4 << 30), rows=F, cols=d, ld=d, stride=(F // N) * d)
    Y = m(FAKE + (8 << 30), dtype=F32, rows=M, cols=d)
    st, size = mlp_query(lib, X, W1, W2, N, 0, N, Y)
    assert st == 0
    base = M * F * 2 + N * M * d * 4
    assert size > base
    assert (size - base) % (M * F * 4) == 0


def test_mlp_decode_workspace_covers_intermediate_and_partials(lib):
    M, d, F, N = 16, 8192, 28672, 8
    X = m(FAKE, rows=M, cols=d)
    W1 = m(FAKE + (1 << 30), rows=d, cols=F, ld=F // N, stride=d * (F // N))
    W2 = m(FAKE + (4 << 30), rows=F, cols=d, ld=d, stride=(F // N) * d)
    Y = m(FAKE + (8 << 30), dtype=F32, rows=M, cols=d)
    st, size = mlp_query(lib, X, W1, W2, N, 0, N, Y)
    assert st == 0
    assert size >= M * F * 2 + N * M * d * 4


# ----------------------------------------------------------------------------- backward entry points


def colb(lib, X, W, dY, N, s0, ns, dXp, dW):
    r = lambda m: ctypes.byref(m) if m is not None else None  # noqa: E731
    return lib.tp_col_linear_backward(r(X), r(W), r(dY), N, s0, ns, r(dXp), r(dW), None)


def rowb(lib, X, W, dY, N, s0, ns, dX, dW):
    r = lambda m: ctypes.byref(m) if m is not None else None  # noqa: E731
    return lib.tp_row_linear_backward(r(X), r(W), r(dY), N, s0, ns, r(dX), r(dW), None)


def test_col_linear_backward_validation(lib):
    # X [4, 8], W [8, 16] split in 2 -> dY [4, 16], partials 2 x [4, 8], dW [8, 16]
    X = m(rows=4, cols=8)
    W = m(FAKE + (1 << 20), rows=8, cols=16)
    dY = m(FAKE + (2 << 20), rows=4, cols=16)
    P = m(FAKE + (3 << 20), dtype=F32, rows=4, cols=8, stride=32)
    G = m(FAKE + (4 << 20), dtype=F32, rows=8, cols=16)
    assert colb(lib, X, W, dY, 2, 0, 2, None, None) == 1  # no output requested
    assert colb(lib, None, W, dY, 2, 0, 2, P, G) == 1
    assert colb(lib, X, W, m(FAKE + (2 << 20), dtype=F32, rows=4, cols=16), 2, 0, 2, P, G) == 2  # dY dtype
    assert colb(lib, X, W, dY, 2, 0, 2, m(FAKE + (3 << 20), rows=4, cols=8, stride=32), G) == 2  # bf16 partials
    assert colb(lib, X, W, m(FAKE + (2 << 20), rows=4, cols=8), 2, 0, 2, P, G) == 3  # dY.cols != ns*width
    assert colb(lib, X, W, dY, 2, 0, 2, P, m(FAKE + (4 << 20), dtype=F32, rows=8, cols=8)) == 3  # dW shape
    assert colb(lib, X, W, dY, 3, 0, 3, P, G) == 4
    assert colb(lib, X, W, dY, 2, 1, 2, P, G) == 5
    assert colb(lib, X, W, dY, 2, 0, 2, m(FAKE + (3 << 20), dtype=F32, rows=4, cols=8, stride=0), G) == 6
    assert colb(lib, X, W, dY, 2, 0, 2, P, m(FAKE + 8, dtype=F32, rows=8, cols=16)) == 7  # dW over X
    assert colb(lib, X, W, dY, 2, 0, 2, m(FAKE + (2 << 20), dtype=F32, rows=4, cols=8, stride=32), G) == 7  # P over dY
    assert colb(lib, X, W, dY, 2, 0, 2, P, m(FAKE + (3 << 20), dtype=F32, rows=8, cols=16)) == 7  # dW over P


def test_row_linear_backward_validation(lib):
    # X [4, 8] split in 2 along K, W [8, 16] -> dY [4, 16], dX [4, 8], dW [8, 16]
    X = m(rows=4, cols=8)
    W = m(FAKE + (1 << 20), rows=8, cols=16)
    dY = m(FAKE + (2 << 20), rows=4, cols=16)
    A = m(FAKE + (3 << 20), dtype=F32, rows=4, cols=8)
    G = m(FAKE + (4 << 20), dtype=F32, rows=8, cols=16)
    assert rowb(lib, X, W, dY, 2, 0, 2, None, None) == 1
    assert rowb(lib, X, W, m(FAKE + (2 << 20), dtype=F32, rows=4, cols=16), 2, 0, 2, A, G) == 2
    assert rowb(lib, X, W, m(FAKE + (2 << 20), rows=4, cols=8), 2, 0, 2, A, G) == 3  # dY.cols != Nout
    assert rowb(lib, X, W, dY, 2, 0, 1, A, G) == 3  # one shard: dX must be [4, 4]
    assert rowb(lib, X, W, dY, 3, 0, 3, A, G) == 4
    assert rowb(lib, X, W, dY, 2, 0, 3, A, G) == 5
    assert rowb(lib, X, W, m(FAKE + (2 << 20), rows=4, cols=16, stride=64), 2, 0, 2, A, G) == 6  # dY shard-major
    assert rowb(lib, X, W, dY, 2, 0, 2, m(FAKE + 16, dtype=F32, rows=4, cols=8), G) == 7  # dX over X
    assert rowb(lib, X, W, dY, 2, 0, 2, A, m(FAKE + (3 << 20), dtype=F32, rows=8, cols=16)) == 7  # dW over dX


def mlpb_query(lib, X, W1, W2, dY, N, s0, ns, act, dX, dW1, dW2):
    size = ctypes.c_size_t(0)
    r = lambda t: ctypes.byref(t) if t is not None else None  # noqa: E731
    st = lib.tp_mlp_backward(r(X), r(W1), r(W2), r(dY), N, s0, ns, act, None, ctypes.byref(size), r(dX), r(dW1),
                             r(dW2), None)
    return st, size.value


def test_mlp_backward_validation_and_workspace(lib):
    M, d, F, N = 64, 32, 128, 4
    X = m(FAKE, rows=M, cols=d)
    W1 = m(FAKE + (1 << 20), rows=d, cols=F)
    W2 = m(FAKE + (2 << 20), rows=F, cols=d)
    dY = m(FAKE + (3 << 20), rows=M, cols=d)
    dX = m(FAKE + (4 << 20), dtype=F32, rows=M, cols=d)
    dW1 = m(FAKE + (5 << 20), dtype=F32, rows=d, cols=F)
    dW2 = m(FAKE + (6 << 20), dtype=F32, rows=F, cols=d)
    hc = M * F * 2  # one [M, ns*width] bf16 buffer (Z, H or dZ)
    st, size = mlpb_query(lib, X, W1, W2, dY, N, 0, N, 1, dX, dW1, dW2)
    assert st == 0 and size == 3 * hc + N * M * d * 4  # Z, H, dZ and the dX partials
    st, size = mlpb_query(lib, X, W1, W2, dY, N, 0, N, 0, dX, dW1, dW2)
    assert st == 0 and size == 2 * hc + N * M * d * 4  # no activation: no Z
    st, size = mlpb_query(lib, X, W1, W2, dY, N, 0, N, 1, None, None, dW2)
    assert st == 0 and size == 2 * hc  # dW2 alone needs Z and H only
    st, size = mlpb_query(lib, X, W1, W2, dY, N, 3, 1, 1, dX, m(FAKE + (5 << 20), dtype=F32, rows=d, cols=F // N),
                          m(FAKE + (6 << 20), dtype=F32, rows=F // N, cols=d))
    assert st == 0 and size == 3 * (M * (F // N) * 2)  # one shard writes dX directly
    assert mlpb_query(lib, X, W1, W2, dY, N, 0, N, 1, None, None, None)[0] == 1
    assert mlpb_query(lib, X, W1, W2, dY, 3, 0, 3, 1, dX, dW1, dW2)[0] == 4
    assert mlpb_query(lib, X, W1, W2, dY, N, 0, N, 5, dX, dW1, dW2)[0] == 3
    assert mlpb_query(lib, X, W1, W2, dY, N, 0, N, 1, m(FAKE + (4 << 20), rows=M, cols=d), dW1, dW2)[0] == 2
    assert mlpb_query(lib, X, W1, W2, m(FAKE + (3 << 20), rows=M, cols=d + 8), N, 0, N, 1, dX, dW1, dW2)[0] == 3
    size = ctypes.c_size_t(16)
    r = ctypes.byref
    st = lib.tp_mlp_backward(r(X), r(W1), r(W2), r(dY), N, 0, N, 1, ctypes.c_void_p(FAKE + (9 << 20)), r(size),
                             r(dX), r(dW1), r(dW2), None)
    assert st == 8  # workspace too small


def test_attention_validation(lib):
    # 8 heads of 16 over N = 2 shards: block = (4 + 2*4) * 16 = 192, output block 64
    def att(qkv, n, s0, ns, heads, kv, dh, L, causal, a):
        r = lambda t: ctypes.byref(t) if t is not None else None  # noqa: E731
        return lib.tp_attention(r(qkv), n, s0, ns, heads, kv, dh, L, causal, r(a), None)

    Q = m(FAKE, rows=20, cols=2 * 192)
    A = m(FAKE + (1 << 20), rows=20, cols=2 * 64)
    assert att(None, 2, 0, 2, 8, 8, 16, 10, 1, A) == 1
    assert att(Q, 2, 0, 2, 8, 8, 16, 10, 1, m(FAKE + (1 << 20), dtype=F32, rows=20, cols=128)) == 2
    assert att(Q, 2, 0, 2, 8, 8, 16, 7, 1, A) == 3       # 20 tokens are not whole sequences of 7
    assert att(Q, 2, 0, 2, 8, 8, 16, 10, 2, A) == 3      # causal must be 0 or 1
    assert att(Q, 2, 0, 2, 8, 3, 16, 10, 1, A) == 3      # heads not a multiple of kv_heads
    assert att(Q, 3, 0, 3, 9, 9, 16, 10, 1, A) == 3      # block widths no longer match Q / A
    assert att(Q, 2, 0, 2, 8, 8, 32, 10, 1, A) == 3      # head_dim 32 needs wider blocks
    assert att(Q, 16, 0, 2, 8, 8, 16, 10, 1, A) == 4     # 16 shards do not split 8 heads
    assert att(Q, 2, 1, 2, 8, 8, 16, 10, 1, A) == 5
    assert att(Q, 2, 0, 2, 8, 8, 16, 10, 1, m(FAKE + 64, rows=20, cols=128)) == 7  # output over QKV
    assert att(Q, 2, 0, 2, 8, 8, 16, 10, 1, m(FAKE + (1 << 20), rows=20, cols=128, ld=100)) == 6


def test_reduce_tokens_axis_validation(lib):
    P = m(FAKE, dtype=BF16, rows=4, cols=16, stride=64)
    red = lib.tp_reduce_partials
    assert red(ctypes.byref(P), 2, 2, ctypes.byref(m(FAKE + (1 << 20), dtype=F32, rows=4, cols=16)), None) == 3
    assert red(ctypes.byref(P), 2, 2, ctypes.byref(m(FAKE + (1 << 20), dtype=F32, rows=8, cols=32)), None) == 3
    assert red(ctypes.byref(P), 2, 2, ctypes.byref(m(FAKE + 16, dtype=BF16, rows=8, cols=16)), None) == 7
    assert red(ctypes.byref(P), 2, 2, ctypes.byref(m(FAKE + (1 << 20), dtype=F32, rows=8, cols=16, ld=8)),
               None) == 6


def test_sp_layernorm_validation(lib):
    # 2 partials of [8 tokens, 16] over N = 4 token shards (2 tokens each); shards 1..2 -> 4 rows
    def ln(P, n, R, keep, p, g, b, eps, N, s0, ns, X1, Y):
        r = lambda t: ctypes.byref(t) if t is not None else None  # noqa: E731
        return lib.tp_sp_layernorm(r(P), n, r(R), keep, p, g, b, eps, N, s0, ns, r(X1), r(Y), None)

    G, B = FAKE + (3 << 20), FAKE + (3 << 20) + 64
    P = m(FAKE, dtype=F32, rows=8, cols=16, stride=128)
    Y = m(FAKE + (1 << 20), dtype=BF16, rows=4, cols=16)
    R = m(FAKE + (2 << 20), dtype=BF16, rows=4, cols=16)
    X1 = m(FAKE + (4 << 20), dtype=F32, rows=4, cols=16)
    assert ln(P, 2, R, None, 0.0, G, B, 1e-5, 4, 1, 2, X1, None) == 1
    assert ln(P, 2, R, None, 0.0, None, B, 1e-5, 4, 1, 2, X1, Y) == 1         # gamma missing
    assert ln(m(FAKE, rows=8, cols=16, stride=128), 2, R, None, 0.0, G, B, 1e-5, 4, 1, 2, X1, Y) == 2
    assert ln(P, 2, R, None, 0.0, G, B, 1e-5, 4, 1, 2, m(FAKE + (4 << 20), rows=4, cols=16), Y) == 2
    assert ln(P, 2, R, None, 0.0, G, B, -1.0, 4, 1, 2, X1, Y) == 3           # eps < 0
    assert ln(P, 2, R, FAKE + (5 << 20), 1.0, G, B, 1e-5, 4, 1, 2, X1, Y) == 3  # p_drop = 1
    assert ln(P, 2, R, None, 0.0, G, B, 1e-5, 4, 1, 4, X1, Y) == 5
    assert ln(P, 2, R, None, 0.0, G, B, 1e-5, 3, 0, 1, X1, Y) == 4           # 3 does not split 8 tokens
    assert ln(P, 2, R, None, 0.0, G, B, 1e-5, 4, 1, 1, X1, Y) == 3           # Y holds 2 shards' rows
    assert ln(P, 2, m(FAKE + (2 << 20), rows=4, cols=8), None, 0.0, G, B, 1e-5, 4, 1, 2, X1, Y) == 3
    assert ln(m(FAKE, dtype=F32, rows=8, cols=16), 2, R, None, 0.0, G, B, 1e-5, 4, 1, 2, X1, Y) == 6
    assert ln(P, 2, R, None, 0.0, G, B, 1e-5, 4, 1, 2, X1, m(FAKE + (1 << 20), dtype=BF16, rows=4, cols=16,
                                                                  ld=8)) == 6
    assert ln(P, 2, R, None, 0.0, G, B, 1e-5, 4, 1, 2, X1, m(FAKE + 64, dtype=F32, rows=4, cols=16)) == 7
    assert ln(P, 2, R, None, 0.0, G, B, 1e-5, 4, 1, 2, m(FAKE + (2 << 20), dtype=F32, rows=4, cols=16), Y) == 7
    assert ln(P, 2, R, None, 0.0, G, B, 1e-5, 4, 1, 2, X1, m(G - 32, dtype=F32, rows=4, cols=16)) == 7
    assert ln(P, 2, R, None, 0.0, G, B, 1e-5, 4, 1, 2, X1, m(FAKE + (4 << 20) + 64, dtype=F32, rows=4,
                                                               cols=16)) == 7  # Y over X1
    # nothing to do: zero tokens
    assert ln(m(FAKE, dtype=F32, rows=0, cols=16, stride=128), 2, None, None, 0.0, None, None, 1e-5, 4, 1, 2,
              None, m(FAKE + (1 << 20), dtype=BF16, rows=0, cols=16)) == 0


def test_size_limits(lib):
    """Sizes past the kernels' 32-bit tile, grid and row limits return TP_ERR_TOO_LARGE."""
    big = (1 << 31)  # one past the largest row or column count a matrix may have
    r = lambda t: ctypes.byref(t) if t is not None else None  # noqa: E731
    # column-parallel product with 2^31 token rows (the stride keeps the address range plausible)
    X = m(FAKE, rows=big, cols=8)
    W = m(FAKE + (1 << 40), rows=8, cols=16)
    Y = m(FAKE + (2 << 40), rows=big, cols=16)
    assert col(lib, X, W, 2, 0, 2, 0, Y) == 10
    assert col(lib, m(FAKE, rows=big - 1, cols=8), W, 2, 0, 2, 0, m(FAKE + 64, rows=big - 1, cols=16)) == 7
    # sequence-parallel LayerNorm over 2^24 executed token rows (one workgroup per row)
    rows = 1 << 24
    P = m(FAKE, dtype=F32, rows=rows, cols=4)
    Yl = m(FAKE + (1 << 40), dtype=F32, rows=rows, cols=4)
    G, B = FAKE + (2 << 40), FAKE + (2 << 40) + 64
    assert lib.tp_sp_layernorm(r(P), 1, None, None, 0.0, G, B, 1e-5, 1, 0, 1, None, r(Yl), None) == 10
    # one row fewer passes the size check and stops at the next one (an output over the partials)
    assert lib.tp_sp_layernorm(r(m(FAKE, dtype=F32, rows=rows - 1, cols=4)), 1, None, None, 0.0, G, B, 1e-5, 1,
                               0, 1, None, r(m(FAKE + 64, dtype=F32, rows=rows - 1, cols=4)), None) == 7
    # attention without a matrix-core path (fp32) over a sequence longer than the element-wise kernel holds
    L = 8193
    Q = m(FAKE, dtype=F32, rows=L, cols=3 * 16)
    A = m(FAKE + (1 << 40), dtype=F32, rows=L, cols=16)
    assert lib.tp_attention(r(Q), 1, 0, 1, 1, 1, 16, L, 1, r(A), None) == 10
    # more executed heads, or more sequences, than the launch grid holds
    Qh = m(FAKE, dtype=BF16, rows=4, cols=3 * 65536 * 16)
    Ah = m(FAKE + (1 << 40), dtype=BF16, rows=4, cols=65536 * 16)
    assert lib.tp_attention(r(Qh), 1, 0, 1, 65536, 65536, 16, 4, 1, r(Ah), None) == 10
    Qs = m(FAKE, dtype=BF16, rows=65536, cols=3 * 16)
    As = m(FAKE + (1 << 40), dtype=BF16, rows=65536, cols=16)
    assert lib.tp_attention(r(Qs), 1, 0, 1, 1, 1, 16, 1, 1, r(As), None) == 10


def test_mlp_noalloc_rejects_oversized_shapes_before_any_hip_call(lib):
    # the Megatron block's workspace (H 67 MB + partials 268 MB) exceeds the built-in scratch
    assert lib.tp_mlp_noalloc_max_scratch() == 64 << 20
    X, W1, W2 = m(rows=2048, cols=4096), m(rows=4096, cols=16384), m(rows=16384, cols=4096)
    Y = m(dtype=F32, rows=2048, cols=4096)
    st = lib.tp_mlp_noalloc(ctypes.byref(X), ctypes.byref(W1), ctypes.byref(W2), 8, 0, 8, 1, ctypes.byref(Y), None)
    assert st == 10  # TP_ERR_TOO_LARGE
    # shape errors are reported as by tp_mlp
    bad = m(rows=2048, cols=4095)
    st = lib.tp_mlp_noalloc(ctypes.byref(bad), ctypes.byref(W1), ctypes.byref(W2), 8, 0, 8, 1, ctypes.byref(Y), None)
    assert st == 3  # TP_ERR_SHAPE
