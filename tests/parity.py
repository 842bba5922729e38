"""Shared helpers of the GPU parity tests: device upload and the comparison bars.

Bars (the same for every floating-point comparison in the suite):
  * relative Frobenius error  ||Y_gpu - Y_ref||_F / ||Y_ref||_F <= 5e-3
  * elementwise error         max |Y_gpu - Y_ref| <= 2e-2 * rms(Y_ref)
Integer-valued inputs must match exactly (compared by value, so -0 == +0).
An output stored in bfloat16 carries its own rounding on top of the
computation's error: at most half a bf16 ulp, which is <= 2^-8 * |y|. For such
outputs the elementwise bar is 2e-2 * rms(Y_ref) + 2^-8 * |Y_ref| per element
(the Frobenius bar is unchanged). No other allowance exists: whatever a kernel
rounds internally has to fit inside the bars above.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

REL_F_TOL = 5e-3
MAX_ERR_RMS_FACTOR = 2e-2


def note(msg: str) -> None:
    """Name the case before a GPU step (flushed, so a crash still shows it)."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def dev():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a visible GPU")
    return torch.device("cuda:0")


def bf16_tensor(bits: np.ndarray) -> torch.Tensor:
    """uint16 bfloat16 bit patterns -> a bfloat16 device tensor holding those exact bits."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).to(dev())


def f32_tensor(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dev())


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.detach().float().cpu().numpy().astype(np.float64)


def errors(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    diff = got - ref
    nref = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(diff)) / nref if nref > 0 else float(np.linalg.norm(diff))
    rms = nref / np.sqrt(max(ref.size, 1))
    mx = float(np.max(np.abs(diff))) if diff.size else 0.0
    return rel, mx, rms


BF16_HALF_ULP_REL = 2.0 ** -8


def assert_close(got, ref, what: str, stored_bf16: bool = False) -> None:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    rel, mx, rms = errors(got, ref)
    assert rel <= REL_F_TOL, f"{what}: relative Frobenius error {rel:.3e} > {REL_F_TOL}"
    if not stored_bf16:
        assert mx <= MAX_ERR_RMS_FACTOR * rms, f"{what}: max error {mx:.3e} > {MAX_ERR_RMS_FACTOR} * rms {rms:.3e}"
    else:
        allow = MAX_ERR_RMS_FACTOR * rms + BF16_HALF_ULP_REL * np.abs(ref)
        excess = np.abs(got - ref) - allow
        worst = int(np.argmax(excess))
        assert excess.flat[worst] <= 0, (
            f"{what}: error {abs(got.flat[worst] - ref.flat[worst]):.3e} at {worst} exceeds "
            f"{MAX_ERR_RMS_FACTOR} * rms + 2^-8 * |ref| = {allow.flat[worst]:.3e}")


def assert_exact(got, ref, what: str) -> None:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    bad = np.argwhere(got != ref)
    assert bad.size == 0, f"{what}: {len(bad)} mismatches, first at {bad[0].tolist()}: {got[tuple(bad[0])]} vs {ref[tuple(bad[0])]}"
