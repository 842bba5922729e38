#!/usr/bin/env python3
"""Benchmark of the tensor-parallel sharded linear layer on one MI355X.

One step is one pass of the whole sharded MLP hot path over one batch of
seeded synthetic input already resident in HBM. The headline workload is one
GPU's share of a GPT-3-width MLP, the largest configuration that fits one GPU
(shard 0 of N = 8: X [16384, 12288], W1_0 [12288, 6144], W2_0 [6144, 12288]):
the column-parallel product with the GeLU epilogue, then the row-parallel
product into the shard's fp32 partial (one shard, so there is no sum). The
calls are exactly the ones tp_mlp issues for this shape; calling them one by
one lets HIP events on the launch stream time each kernel inside the timed
region.

Prints one JSON line. Further workloads are measured too and listed under
"secondary": the Megatron MLP block with all 8 shards and the partial-sum
reduce (also as one tp_mlp call), the attention projections, the
decode-shaped MLP (reported in HBM GB/s, as three timed calls and as one
tp_mlp call), the MLP backward pass, the
attention block (projections with attention between them), the MLP followed
by the sequence-parallel LayerNorm boundary, and the explicit all-gather of
the QKV column blocks from shard-major buffers (HBM GB/s); --workload picks
one. Every workload is timed over at least 20 steps, the Megatron-block and
decode shapes (well under a millisecond per step) over at least 100. Only one
GPU is used:
--gpus above 1 exits with a message.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6  # MI355X dense bf16 matrix-core peak (256 CU x 4096 flop/clk x 2.4 GHz)
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E bandwidth
LEAD_CYCLES = 40_000_000  # ~20 ms of GPU spin at the ~2 GHz shader clock
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")
# Workloads that reuse the shapes of another one.
BASE_WORKLOAD = {"megatron_mlp_bwd": "megatron_mlp", "attn_block": "attn_proj", "mlp_sp_block": "megatron_mlp",
                 "megatron_mlp_call": "megatron_mlp", "qkv_all_gather": "attn_proj", "decode_mlp_call": "decode_mlp"}
# Workloads reported in HBM GB/s rather than TFLOP/s.
HBM_WORKLOADS = ("decode_mlp", "decode_mlp_call", "qkv_all_gather")
SP_P_DROP = 0.1
MIN_STEPS = 20  # timed steps of every workload, whatever --steps asks for
# the Megatron-block and decode shapes run well under a millisecond per step: at least 100 of them
MIN_STEPS_SHORT = 100
SHORT_WORKLOADS = ("megatron_mlp", "megatron_mlp_call", "megatron_mlp_bwd", "mlp_sp_block", "decode_mlp",
                   "decode_mlp_call")
ATTN_HEADS, ATTN_HEAD_DIM = 64, 128  # the attention-projection workload: d = 8192 = 64 heads x 128
# The headline metric: TFLOP/s of the sharded MLP (its fraction of the bf16
# peak under "roofline"), with the decode-shaped MLP's HBM GB/s beside it.
METRIC = "sharded-linear TFLOP/s (% of bf16 MFMA peak); decode-shape HBM GB/s"
# Kernel sources each workload's kernels are built from: the HBM traffic recorded
# for a workload is reported only while these files are unchanged.
WORKLOAD_SOURCES = {
    "gpt3_mlp_shard": ["gemm_mfma.hip"],
    "megatron_mlp": ["gemm_mfma.hip", "combine.hip"],
    "megatron_mlp_call": ["gemm_mfma.hip", "combine.hip"],
    "attn_proj": ["gemm_mfma.hip", "combine.hip"],
    "decode_mlp": ["gemm_skinny.hip", "combine.hip"],
    "decode_mlp_call": ["gemm_skinny.hip", "combine.hip"],
    "megatron_mlp_bwd": ["gemm_mfma.hip", "combine.hip"],
    "attn_block": ["gemm_mfma.hip", "attention.hip", "combine.hip"],
    "mlp_sp_block": ["gemm_mfma.hip", "sp_layernorm.hip"],
    "qkv_all_gather": ["combine.hip"],
}


def kernel_source_hash(workload: str) -> str:
    h = hashlib.sha256()
    for name in WORKLOAD_SOURCES[workload]:
        with open(os.path.join(ROOT, "tensor_sharded_linear_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, kernel: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None if stale/absent."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    entry = t.get("workloads", {}).get(workload, {})
    if entry.get("source_hash") != kernel_source_hash(workload):
        return None
    return entry.get("kernels", {}).get(kernel)


# ----------------------------------------------------------------------------- workloads


def make_inputs(name, torch, dev):
    """Seeded synthetic inputs of one workload, uploaded as bf16 bit patterns."""
    from synthetic import WORKLOADS, normal_bf16

    wl = WORKLOADS[BASE_WORKLOAD.get(name, name)]

    def up(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    t = {"wl": wl}
    if name in ("megatron_mlp", "gpt3_mlp_shard", "megatron_mlp_call"):
        width = wl.F // wl.N
        t["x"] = up(normal_bf16((wl.M, wl.d), 1.0, wl.wid, 0)[0])
        if wl.ns == wl.N:
            t["w1"] = up(normal_bf16((wl.d, wl.F), 0.02, wl.wid, 1)[0])
            t["w2"] = up(normal_bf16((wl.F, wl.d), 0.02, wl.wid, 2)[0])
        else:  # one GPU's share: only the executed shard's blocks are stored
            t["w1"] = up(normal_bf16((wl.ns, wl.d, width), 0.02, wl.wid, 1)[0])
            t["w2"] = up(normal_bf16((wl.ns, width, wl.d), 0.02, wl.wid, 2)[0])
    elif name == "attn_proj":
        t["x"] = up(normal_bf16((wl.M, wl.d), 1.0, wl.wid, 0)[0])
        t["wqkv"] = up(normal_bf16((wl.d, wl.F), 0.02, wl.wid, 1)[0])
        t["wo"] = up(normal_bf16((wl.d, wl.out), 0.02, wl.wid, 2)[0])
        t["a"] = up(normal_bf16((wl.M, wl.d), 1.0, wl.wid, 3)[0])
    elif name == "megatron_mlp_bwd":
        wl = WORKLOADS["megatron_mlp"]
        t["wl"] = wl
        t["x"] = up(normal_bf16((wl.M, wl.d), 1.0, wl.wid, 0)[0])
        t["w1"] = up(normal_bf16((wl.d, wl.F), 0.02, wl.wid, 1)[0])
        t["w2"] = up(normal_bf16((wl.F, wl.d), 0.02, wl.wid, 2)[0])
        t["dy"] = up(normal_bf16((wl.M, wl.d), 1.0, wl.wid, 4)[0])
    elif name == "mlp_sp_block":
        from synthetic import keep_mask, normal_f32
        t["x"] = up(normal_bf16((wl.M, wl.d), 1.0, wl.wid, 0)[0])
        t["w1"] = up(normal_bf16((wl.d, wl.F), 0.02, wl.wid, 1)[0])
        t["w2"] = up(normal_bf16((wl.F, wl.d), 0.02, wl.wid, 2)[0])
        t["keep"] = torch.from_numpy(keep_mask((wl.M, wl.d), SP_P_DROP, wl.wid, 5)).to(dev)
        t["gamma"] = torch.from_numpy(normal_f32((wl.d,), 1.0, 0.1, wl.wid, 6)).to(dev)
        t["beta"] = torch.from_numpy(normal_f32((wl.d,), 0.0, 0.1, wl.wid, 7)).to(dev)
    elif name == "attn_block":
        t["x"] = up(normal_bf16((wl.M, wl.d), 1.0, wl.wid, 0)[0])
        t["wqkv"] = up(normal_bf16((wl.d, wl.F), 0.02, wl.wid, 1)[0])
        t["wo"] = up(normal_bf16((wl.d, wl.out), 0.02, wl.wid, 2)[0])
    elif name == "qkv_all_gather":
        # the column-parallel QKV outputs of the 8 shards, each in its own buffer (shard-major)
        t["x"] = up(normal_bf16((wl.N, wl.M, wl.F // wl.N), 1.0, wl.wid, 8)[0])
    elif name in ("decode_mlp", "decode_mlp_call"):
        width = wl.F // wl.N
        t["x"] = up(normal_bf16((wl.M, wl.d), 1.0, wl.wid, 0)[0])
        # two weight sets used alternately, so no step finds the previous step's weights in cache
        t["w1s"] = [up(normal_bf16((wl.N, wl.d, width), 0.02, wl.wid + 100 * r, 1)[0]) for r in range(2)]
        t["w2s"] = [up(normal_bf16((wl.N, width, wl.d), 0.02, wl.wid + 100 * r, 2)[0]) for r in range(2)]
    else:
        raise ValueError(name)
    return t


def plan(name, t, torch, tp):
    """Returns (kernels, step) where step(i, rec) issues one step and calls rec() between kernels."""
    wl = t["wl"]
    dev = t["x"].device
    flop = lambda m, k, n: 2.0 * m * k * n  # noqa: E731
    if name in ("megatron_mlp", "gpt3_mlp_shard"):
        width = wl.F // wl.N
        h = torch.empty((wl.M, wl.ns * width), dtype=torch.bfloat16, device=dev)
        y = torch.empty((wl.M, wl.d), dtype=torch.float32, device=dev)
        p = torch.empty((wl.ns, wl.M, wl.d), dtype=torch.float32, device=dev) if wl.ns > 1 else None
        kernels = [
            {"name": "col_gemm_gelu", "flop": flop(wl.M, wl.d, wl.ns * width), "bound": "mfma",
             "bytes": 2.0 * (wl.M * wl.d + wl.d * wl.ns * width + wl.M * wl.ns * width)},
            {"name": "row_gemm_partials", "flop": flop(wl.M, wl.ns * width, wl.d), "bound": "mfma",
             "bytes": 2.0 * (wl.M * wl.ns * width + wl.ns * width * wl.d) + 4.0 * wl.ns * wl.M * wl.d},
        ]
        if wl.ns > 1:
            kernels.append({"name": "reduce_partials", "flop": 0.0, "bound": "hbm",
                            "bytes": 4.0 * (wl.ns + 1) * wl.M * wl.d})

        def step(i, rec):
            tp.col_linear(t["x"], t["w1"], wl.N, 0, wl.ns, act="gelu", out=h)
            rec()
            if wl.ns > 1:
                tp.row_linear(h, t["w2"] if t["w2"].dim() == 3 else t["w2"][: wl.ns * width], wl.ns, out=p)
                rec()
                tp.reduce_partials(p, "rows", out=y)
            else:
                tp.row_linear(h, t["w2"], 1, out=y.view(1, wl.M, wl.d))
            rec()

        return kernels, step
    if name == "attn_proj":
        width = wl.F // wl.N
        qkv = torch.empty((wl.M, wl.F), dtype=torch.bfloat16, device=dev)
        p = torch.empty((wl.N, wl.M, wl.out), dtype=torch.float32, device=dev)
        y = torch.empty((wl.M, wl.out), dtype=torch.float32, device=dev)
        kb = wl.d // wl.N
        kernels = [
            {"name": "qkv_col_gemm", "flop": flop(wl.M, wl.d, wl.F), "bound": "mfma",
             "bytes": 2.0 * (wl.M * wl.d + wl.d * wl.F + wl.M * wl.F)},
            {"name": "wo_row_gemm_partials", "flop": flop(wl.M, wl.d, wl.out), "bound": "mfma",
             "bytes": 2.0 * (wl.M * wl.d + wl.d * wl.out) + 4.0 * wl.N * wl.M * wl.out},
            {"name": "reduce_partials", "flop": 0.0, "bound": "hbm", "bytes": 4.0 * (wl.N + 1) * wl.M * wl.out},
        ]
        del width, kb

        def step(i, rec):
            tp.col_linear(t["x"], t["wqkv"], wl.N, out=qkv)
            rec()
            tp.row_linear(t["a"], t["wo"], wl.N, out=p)
            rec()
            tp.reduce_partials(p, "rows", out=y)
            rec()

        return kernels, step
    if name == "attn_block":
        # QKV projection -> attention (the 4096 tokens as one causal sequence) -> W_o partials -> sum
        qkv = torch.empty((wl.M, wl.F), dtype=torch.bfloat16, device=dev)
        a = torch.empty((wl.M, wl.d), dtype=torch.bfloat16, device=dev)
        p = torch.empty((wl.N, wl.M, wl.out), dtype=torch.float32, device=dev)
        y = torch.empty((wl.M, wl.out), dtype=torch.float32, device=dev)
        pairs = wl.M * (wl.M + 1) / 2  # visible (query, key) pairs of one causal sequence
        kernels = [
            {"name": "qkv_col_gemm", "flop": flop(wl.M, wl.d, wl.F), "bound": "mfma",
             "bytes": 2.0 * (wl.M * wl.d + wl.d * wl.F + wl.M * wl.F)},
            {"name": "attention", "flop": 4.0 * ATTN_HEADS * ATTN_HEAD_DIM * pairs, "bound": "mfma",
             "bytes": 2.0 * (wl.M * wl.F + wl.M * wl.d)},
            {"name": "wo_row_gemm_partials", "flop": flop(wl.M, wl.d, wl.out), "bound": "mfma",
             "bytes": 2.0 * (wl.M * wl.d + wl.d * wl.out) + 4.0 * wl.N * wl.M * wl.out},
            {"name": "reduce_partials", "flop": 0.0, "bound": "hbm", "bytes": 4.0 * (wl.N + 1) * wl.M * wl.out},
        ]

        def step(i, rec):
            tp.col_linear(t["x"], t["wqkv"], wl.N, out=qkv)
            rec()
            tp.attention(qkv, wl.N, ATTN_HEADS, ATTN_HEADS, ATTN_HEAD_DIM, wl.M, True, out=a)
            rec()
            tp.row_linear(a, t["wo"], wl.N, out=p)
            rec()
            tp.reduce_partials(p, "rows", out=y)
            rec()

        return kernels, step
    if name == "megatron_mlp_call":
        # the same MLP pair issued as one tp_mlp call (its workspace holds H and the partials)
        y = torch.empty((wl.M, wl.d), dtype=torch.float32, device=dev)
        ws = torch.empty(tp.mlp_workspace_bytes(t["x"], t["w1"], t["w2"], wl.N), dtype=torch.uint8, device=dev)
        kernels = [{"name": "tp_mlp", "flop": 2 * flop(wl.M, wl.d, wl.F), "bound": "mfma",
                    "bytes": 2.0 * (wl.M * wl.d + 2 * wl.d * wl.F) + 4.0 * wl.M * wl.d}]

        def step(i, rec):
            tp.mlp(t["x"], t["w1"], t["w2"], wl.N, out=y, workspace=ws)
            rec()

        return kernels, step
    if name == "mlp_sp_block":
        # the MLP pair, then the sequence-parallel boundary: reduce-scatter of the partials over the 8
        # token shards, dropout, residual add, LayerNorm (the token shards' outputs land in one matrix,
        # so the all-gather that follows is the identity in memory)
        width = wl.F // wl.N
        h = torch.empty((wl.N, wl.M, width), dtype=torch.bfloat16, device=dev)
        p = torch.empty((wl.N, wl.M, wl.d), dtype=torch.float32, device=dev)
        y = torch.empty((wl.M, wl.d), dtype=torch.bfloat16, device=dev)
        x1 = torch.empty((wl.M, wl.d), dtype=torch.float32, device=dev)
        kernels = [
            {"name": "col_gemm_gelu", "flop": flop(wl.M, wl.d, wl.F), "bound": "mfma",
             "bytes": 2.0 * (wl.M * wl.d + wl.d * wl.F + wl.M * wl.F)},
            {"name": "row_gemm_partials", "flop": flop(wl.M, wl.F, wl.d), "bound": "mfma",
             "bytes": 2.0 * (wl.M * wl.F + wl.F * wl.d) + 4.0 * wl.N * wl.M * wl.d},
            # partials in, keep bytes, bf16 residual, fp32 pre-norm sum and bf16 output out
            {"name": "sp_layernorm", "flop": 0.0, "bound": "hbm",
             "bytes": (4.0 * wl.N + 1 + 2 + 4 + 2) * wl.M * wl.d + 8.0 * wl.d},
        ]

        def step(i, rec):
            tp.col_linear(t["x"], t["w1"], wl.N, act="gelu", out=h, partitioned=True)
            rec()
            tp.row_linear(h, t["w2"], wl.N, out=p)
            rec()
            tp.sp_layernorm(p, t["gamma"], t["beta"], wl.N, residual=t["x"], keep=t["keep"], p_drop=SP_P_DROP,
                            out=y, residual_out=x1)
            rec()

        return kernels, step
    if name == "megatron_mlp_bwd":
        dx = torch.empty((wl.M, wl.d), dtype=torch.float32, device=dev)
        dw1 = torch.empty((wl.d, wl.F), dtype=torch.float32, device=dev)
        dw2 = torch.empty((wl.F, wl.d), dtype=torch.float32, device=dev)
        ws = torch.empty(tp.mlp_backward_workspace_bytes(t["x"], t["w1"], t["w2"], t["dy"], wl.N), dtype=torch.uint8,
                         device=dev)
        # recompute Z and H, dZ = (dY W2^T) * GeLU'(Z), dW2 = H^T dY, dX partials + sum, dW1 = X^T dZ
        kernels = [{"name": "mlp_backward", "flop": 5 * flop(wl.M, wl.d, wl.F), "bound": "mfma",
                    "bytes": 2.0 * (wl.M * wl.d * 2 + 2 * wl.d * wl.F) + 4.0 * (wl.M * wl.d + 2 * wl.d * wl.F)}]

        def step(i, rec):
            tp.mlp_backward(t["x"], t["w1"], t["w2"], t["dy"], wl.N, dx=dx, dw1=dw1, dw2=dw2, workspace=ws)
            rec()

        return kernels, step
    if name == "qkv_all_gather":
        # the explicit all-gather of column blocks: [8][4096, 3072] -> [4096, 24576], bf16
        y = torch.empty((wl.M, wl.F), dtype=torch.bfloat16, device=dev)
        kernels = [{"name": "all_gather_cols", "flop": 0.0, "bound": "hbm", "bytes": 2.0 * 2 * wl.M * wl.F}]

        def step(i, rec):
            tp.reduce_partials(t["x"], "cols", out=y)
            rec()

        return kernels, step
    if name == "decode_mlp_call":
        # the decode MLP as one tp_mlp call (the same three kernels, launched back to back)
        y = torch.empty((wl.M, wl.d), dtype=torch.float32, device=dev)
        ws = torch.empty(tp.mlp_workspace_bytes(t["x"], t["w1s"][0], t["w2s"][0], wl.N), dtype=torch.uint8,
                         device=dev)
        kernels = [{"name": "tp_mlp", "flop": 2 * flop(wl.M, wl.d, wl.F), "bound": "hbm",
                    "bytes": 2.0 * (wl.M * wl.d + 2 * wl.d * wl.F) + 4.0 * wl.M * wl.d}]

        def step(i, rec):
            r = i % 2
            tp.mlp(t["x"], t["w1s"][r], t["w2s"][r], wl.N, out=y, workspace=ws)
            rec()

        return kernels, step
    if name == "decode_mlp":
        width = wl.F // wl.N
        h = torch.empty((wl.M, wl.F), dtype=torch.bfloat16, device=dev)
        p = torch.empty((wl.N, wl.M, wl.d), dtype=torch.float32, device=dev)
        y = torch.empty((wl.M, wl.d), dtype=torch.float32, device=dev)
        kernels = [
            {"name": "decode_col_gemm_gelu", "flop": flop(wl.M, wl.d, wl.F), "bound": "hbm",
             "bytes": 2.0 * (wl.M * wl.d + wl.d * wl.F + wl.M * wl.F)},
            {"name": "decode_row_gemm_partials", "flop": flop(wl.M, wl.F, wl.d), "bound": "hbm",
             "bytes": 2.0 * (wl.M * wl.F + wl.F * wl.d) + 4.0 * wl.N * wl.M * wl.d},
            {"name": "reduce_partials", "flop": 0.0, "bound": "hbm", "bytes": 4.0 * (wl.N + 1) * wl.M * wl.d},
        ]

        def step(i, rec):
            # the three public calls tp_mlp stands for, with events between them
            # (tp_mlp itself splits the first product's K in two and its second
            # product reads the chunk sums: decode_mlp_call); the two weight sets alternate
            r = i % 2
            tp.col_linear(t["x"], t["w1s"][r], wl.N, act="gelu", out=h)
            rec()
            tp.row_linear(h, t["w2s"][r], wl.N, out=p)
            rec()
            tp.reduce_partials(p, "rows", out=y)
            rec()

        return kernels, step
    raise ValueError(name)


def time_workload(name, steps, warmup, torch, tp):
    dev = torch.device("cuda:0")
    t = make_inputs(name, torch, dev)
    kernels, step = plan(name, t, torch, tp)
    stream = torch.cuda.current_stream(dev)
    for i in range(warmup):
        step(i, lambda: None)
    torch.cuda.synchronize()
    nk = len(kernels)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(nk + 1)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    # A short spin on the stream first lets the host enqueue the steps ahead of
    # the GPU, so the events between kernels time the kernels and not the
    # host's launch overhead (which would show as idle gaps on short kernels).
    torch.cuda._sleep(LEAD_CYCLES)
    for i in range(steps):
        marks = ev[i]
        marks[0].record(stream)
        k = [1]

        def rec(marks=marks, k=k):
            marks[k[0]].record(stream)
            k[0] += 1

        step(i, rec)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_kernel = np.array([[ev[i][j].elapsed_time(ev[i][j + 1]) for j in range(nk)] for i in range(steps)])
    step_ms = np.array([ev[i][0].elapsed_time(ev[i][nk]) for i in range(steps)])
    res = {"workload": name, "steps": steps, "ms_per_step": float(step_ms.mean()),
           "ms_per_step_median": float(np.median(step_ms)), "ms_per_step_min": float(step_ms.min()),
           "wall_s": wall, "kernels": []}
    total_flop = sum(k["flop"] for k in kernels)
    for j, k in enumerate(kernels):
        ms = float(per_kernel[:, j].mean())
        entry = {"name": k["name"], "ms": ms, "ms_median": float(np.median(per_kernel[:, j])),
                 "ms_min": float(per_kernel[:, j].min()), "bound": k["bound"]}
        if k["flop"]:
            entry["tflops"] = k["flop"] / (ms * 1e-3) / 1e12
            entry["frac_mfma_peak"] = entry["tflops"] / PEAK_BF16_TFLOPS
        entry["alg_gbs"] = k["bytes"] / (ms * 1e-3) / 1e9
        entry["frac_hbm_peak"] = entry["alg_gbs"] / PEAK_HBM_GBS
        res["kernels"].append(entry)
    res["tflops"] = total_flop / (res["ms_per_step"] * 1e-3) / 1e12
    if name in HBM_WORKLOADS:
        res["alg_bytes"] = sum(k["bytes"] for k in kernels)
        res["gbs"] = res["alg_bytes"] / (res["ms_per_step"] * 1e-3) / 1e9
    res["_kernels_def"] = kernels
    return res


def engine_clock_mhz():
    """The current engine clock level the driver reports (sysfs, read-only), or None."""
    import glob
    for path in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
        try:
            for line in open(path):
                if line.rstrip().endswith("*"):
                    return float(line.split(":")[1].strip().split("Mhz")[0].split("MHz")[0])
        except (OSError, ValueError, IndexError):
            continue
    return None


def roofline_for(res):
    """The dominant kernel of a workload against its bound."""
    ks = res["kernels"]
    j = int(np.argmax([k["ms"] for k in ks]))
    k, kd = ks[j], res["_kernels_def"][j]
    traffic = measured_traffic(res["workload"], k["name"])
    if kd["bound"] == "mfma":
        achieved = kd["flop"] / (k["ms"] * 1e-3) / 1e12
        return {"kernel": k["name"], "bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS, "traffic": traffic,
                "alg_per_launch": kd["flop"], "ms_per_launch": k["ms"]}
    achieved = kd["bytes"] / (k["ms"] * 1e-3) / 1e9
    return {"kernel": k["name"], "bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": achieved / PEAK_HBM_GBS, "traffic": traffic, "alg_per_launch": kd["bytes"],
            "ms_per_launch": k["ms"]}


def host_cpu_model() -> str:
    """The host CPU's model name as the kernel reports it (read-only), or "unknown"."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(seconds_target: float = 12.0, sample_rows_count: int = 1024):
    """The float64 oracle timed on the host cores on a bounded sample of the headline workload.

    The sample is `sample_rows_count` seeded token rows of the GPT-3-width MLP shard: every
    output row depends only on its own input row, so the oracle's time per row is the same on
    the sample as on all 16384 rows, and the rate (TFLOP/s) extrapolates unchanged.
    """
    import oracle
    from synthetic import WORKLOADS, normal_bf16, sample_rows

    wl = WORKLOADS["gpt3_mlp_shard"]
    width = wl.F // wl.N
    rows = sample_rows(wl.M, sample_rows_count, seed=4242)
    _, x = normal_bf16((wl.M, wl.d), 1.0, wl.wid, 0)
    x = np.ascontiguousarray(x[rows])
    _, w1 = normal_bf16((1, wl.d, width), 0.02, wl.wid, 1)
    _, w2 = normal_bf16((1, width, wl.d), 0.02, wl.wid, 2)
    w1, w2 = w1[0], w2[0]
    try:
        from threadpoolctl import threadpool_info

        threads = max((i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"),
                      default=1)
    except Exception:  # pragma: no cover - threadpoolctl is optional
        threads = os.cpu_count() or 1
    run = lambda: oracle.mlp_shard_partials(x, w1, w2, 1, "gelu")  # noqa: E731
    # one pass first, then as many more as fit the time target
    t0 = time.perf_counter()
    run()
    first = time.perf_counter() - t0
    passes = int(max(1, min(50, round(seconds_target / max(first, 1e-3)))))
    t0 = time.perf_counter()
    for _ in range(passes):
        run()
    dt = time.perf_counter() - t0
    flops = passes * 2 * 2.0 * len(rows) * wl.d * width
    rate = flops / dt / 1e12
    full_step_s = dt / passes * wl.M / len(rows)
    return {"value": rate, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{passes} passes over {len(rows)} seeded token rows of gpt3_mlp_shard (X rows "
                      f"[{len(rows)},{wl.d}], W1_0 [{wl.d},{width}], GeLU, W2_0 [{width},{wl.d}]), float64 "
                      f"numpy oracle, {dt:.1f} s; extrapolated to all {wl.M} rows by M/{len(rows)} "
                      f"(rows are independent): {full_step_s:.1f} s per step",
            "extrapolated": True, "seconds": dt, "full_step_s_extrapolated": full_step_s,
            "host_cpus": os.cpu_count(), "cpu_model": host_cpu_model()}


def copy_calibration(torch, gib: float = 1.0):
    """A plain device copy of known size, for scaling the HBM byte counters."""
    n = int(gib * (1 << 30)) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda:0")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_each_way": n * 4, "launches": 3}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="all",
                    choices=["all", "megatron_mlp", "attn_proj", "gpt3_mlp_shard", "decode_mlp",
                             "decode_mlp_call", "megatron_mlp_bwd", "attn_block", "mlp_sp_block",
                             "megatron_mlp_call", "qkv_all_gather"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a 1 GiB device copy (for HBM counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the sharded layer runs all N logical shards on a single "
              "MI355X; no multi-GPU figure is produced. Use --gpus 1.", file=sys.stderr)
        sys.exit(1)

    import torch

    if args.copy_calibration:
        copy_calibration(torch)
        return
    import tensor_sharded_linear_amd as tp

    tp.library()  # fails loudly if the HIP library is missing
    main_name = "gpt3_mlp_shard" if args.workload == "all" else args.workload
    # the one-call form of the Megatron MLP runs right after its three-call form, in the same thermal state
    names = [main_name] if args.workload != "all" else ["gpt3_mlp_shard", "megatron_mlp", "megatron_mlp_call",
                                                        "attn_proj", "decode_mlp", "decode_mlp_call",
                                                        "megatron_mlp_bwd", "attn_block", "mlp_sp_block",
                                                        "qkv_all_gather"]
    results = {}
    for name in names:
        steps = max(MIN_STEPS_SHORT if name in SHORT_WORKLOADS else MIN_STEPS, args.steps)
        print(f"[bench] {name}: warmup {args.warmup}, steps {steps}", file=sys.stderr, flush=True)
        results[name] = time_workload(name, steps, args.warmup, torch, tp)
        results[name]["sclk_mhz_after"] = engine_clock_mhz()
        torch.cuda.empty_cache()
        print(f"[bench] {name}: {results[name]['ms_per_step']:.3f} ms/step", file=sys.stderr, flush=True)

    main = results[main_name]
    from synthetic import WORKLOADS

    wl = WORKLOADS[BASE_WORKLOAD.get(main_name, main_name)]
    metric = METRIC
    if main_name in HBM_WORKLOADS:
        unit, value = "GB/s", main["gbs"]
    else:
        unit, value = "TFLOP/s", main["tflops"]
    line = {
        "metric": metric,
        "value": value,
        "unit": unit,
        "n_gpus": 1,
        "steps": main["steps"],
        "warmup": args.warmup,
        "ms_per_step": main["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) activations, N(0,0.02) weights, rounded to bf16)",
        "config": {"workload": main_name, "M": wl.M, "d": wl.d, "F": wl.F, "N": wl.N, "shards_run": wl.ns,
                   "parallelism": f"tp{wl.N} shards executed on 1 GPU"},
        "frac_of_bf16_peak": (main["tflops"] / PEAK_BF16_TFLOPS) if main_name not in HBM_WORKLOADS else None,
        "roofline": roofline_for(main),
        "ms_per_step_median": main["ms_per_step_median"],
        "sclk_mhz_after": main["sclk_mhz_after"],
        # the same rate against the peak at the engine clock read right after the workload
        # (the spec peak assumes 2.4 GHz; under sustained MFMA load the clock sits lower)
        "frac_of_bf16_peak_at_sclk": ((main["tflops"] / (PEAK_BF16_TFLOPS * main["sclk_mhz_after"] / 2400.0))
                                      if main_name not in HBM_WORKLOADS and main["sclk_mhz_after"] else None),
        "kernels": main["kernels"],
    }
    secondary = []
    for name in names:
        if name == main_name:
            continue
        r = results[name]
        entry = {"workload": name, "ms_per_step": r["ms_per_step"], "kernels": r["kernels"],
                 "roofline": roofline_for(r)}
        if name in HBM_WORKLOADS:
            label = "decode-shape HBM GB/s" if name.startswith("decode_mlp") else "all-gather HBM GB/s"
            entry.update({"metric": label, "value": r["gbs"], "unit": "GB/s",
                          "frac_of_hbm_peak": r["gbs"] / PEAK_HBM_GBS})
        else:
            entry.update({"metric": "sharded-linear TFLOP/s", "value": r["tflops"], "unit": "TFLOP/s",
                          "frac_of_bf16_peak": r["tflops"] / PEAK_BF16_TFLOPS})
        secondary.append(entry)
    if secondary:
        line["secondary"] = secondary
    if "decode_mlp_call" in results and main_name != "decode_mlp_call":
        # the decode MLP as the library offers it: one tp_mlp call
        line["decode_shape_hbm_gbs"] = results["decode_mlp_call"]["gbs"]
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle on host cores)", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
