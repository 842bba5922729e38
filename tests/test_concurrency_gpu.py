"""Concurrent use: the library keeps no mutable global state, so calls from several host
threads, each enqueuing on its own stream, give the same bits as the same calls made one
after another on one stream.
"""
import threading

import pytest
import torch

import tensor_sharded_linear_amd as tp
from synthetic import normal_bf16
from parity import bf16_tensor, dev, note

pytestmark = pytest.mark.gpu

THREADS = 4
ROUNDS = 5


def make_case(i):
    M, d, F, N = 128 + 32 * i, 256, 1024, 4
    x = bf16_tensor(normal_bf16((M, d), 1.0, 9800 + i, 0)[0])
    w1 = bf16_tensor(normal_bf16((d, F), 0.02, 9800 + i, 1)[0])
    w2 = bf16_tensor(normal_bf16((F, d), 0.02, 9800 + i, 2)[0])
    return x, w1, w2, N


def run_case(case):
    x, w1, w2, N = case
    h = tp.col_linear(x, w1, N, act="gelu")
    y = tp.reduce_partials(tp.row_linear(h, w2, N))
    return h, y, tp.mlp(x, w1, w2, N)


def test_threads_on_their_own_streams_match_sequential_calls():
    cases = [make_case(i) for i in range(THREADS)]
    expected = [run_case(c) for c in cases]
    torch.cuda.synchronize()
    results = [[None] * ROUNDS for _ in range(THREADS)]
    errors = []

    def worker(i):
        try:
            s = torch.cuda.Stream(device=dev())
            with torch.cuda.stream(s):
                for r in range(ROUNDS):
                    results[i][r] = run_case(cases[i])
            s.synchronize()
        except Exception as e:  # reported by the main thread
            errors.append(e)

    note(f"{THREADS} threads x {ROUNDS} rounds")
    threads = [threading.Thread(target=worker, args=(i,)) for i in range(THREADS)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for i in range(THREADS):
        for r in range(ROUNDS):
            for got, want in zip(results[i][r], expected[i]):
                assert torch.equal(got, want), f"thread {i} round {r} differs from the sequential result"
