"""tp_mlp_noalloc (the MLP pair with the library's built-in scratch, no workspace) against tp_mlp.

Two calls in a row through the C interface, the second with a smaller input,
each compared bitwise with tp_mlp on the same inputs (the same kernels run in
the same order, so the results must be identical) and with the float64 oracle
under the parity bars. A third call repeats the first shape, so stale scratch
contents from a different shape cannot leak into a result.
"""
import numpy as np
import pytest
import torch

import oracle
import tensor_sharded_linear_amd as tp
from synthetic import normal_bf16
from parity import assert_close, bf16_tensor, host, note

pytestmark = pytest.mark.gpu


def _case(wid, M, d, F, N, shard_major):
    xb, x = normal_bf16((M, d), 1.0, wid, 0)
    if shard_major:
        w1b, w1 = normal_bf16((N, d, F // N), 0.02, wid, 1)
        w2b, w2 = normal_bf16((N, F // N, d), 0.02, wid, 2)
        w1f, w2f = np.concatenate(list(w1), axis=1), np.concatenate(list(w2), axis=0)
    else:
        w1b, w1f = normal_bf16((d, F), 0.02, wid, 1)
        w2b, w2f = normal_bf16((F, d), 0.02, wid, 2)
    return (bf16_tensor(xb), bf16_tensor(w1b), bf16_tensor(w2b)), (x, w1f, w2f)


def _check(name, dev_in, host_in, N):
    X, W1, W2 = dev_in
    note(f"tp_mlp_noalloc {name}: X {tuple(X.shape)} N={N}")
    got = tp.mlp_noalloc(X, W1, W2, N)
    want = tp.mlp(X, W1, W2, N)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int32), want.view(torch.int32)), f"{name}: differs from tp_mlp"
    x, w1, w2 = host_in
    assert_close(host(got), oracle.mlp(x, w1, w2, N, "gelu"), f"{name} vs oracle")


def test_mlp_noalloc_matches_mlp_on_two_calls():
    assert tp.mlp_noalloc_max_scratch() == 64 << 20
    big = _case(5100, 16, 8192, 28672, 8, True)      # the decode-shaped MLP (skinny path, K-split)
    small = _case(5101, 200, 512, 2048, 4, False)    # a smaller input on the tiled path
    _check("decode shape", *big, 8)
    _check("smaller input", *small, 4)
    _check("decode shape again", *big, 8)


def test_mlp_noalloc_rejects_shapes_beyond_scratch():
    # the Megatron block needs 67 MB for H and 268 MB for the partials: more than the scratch holds
    X = torch.zeros((2048, 4096), dtype=torch.bfloat16, device="cuda:0")
    W1 = torch.zeros((4096, 16384), dtype=torch.bfloat16, device="cuda:0")
    W2 = torch.zeros((16384, 4096), dtype=torch.bfloat16, device="cuda:0")
    note("tp_mlp_noalloc rejects the Megatron block (scratch too small)")
    with pytest.raises(tp.TpError) as e:
        tp.mlp_noalloc(X, W1, W2, 8)
    assert e.value.status == 10  # TP_ERR_TOO_LARGE
