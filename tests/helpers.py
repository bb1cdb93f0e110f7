"""Test helpers: move synthetic inputs to the device and compare with the oracle."""
from __future__ import annotations

import json
import os

import numpy as np
import torch

import synth


def dev_codes(a: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int32)).to(device)


def dev_half(bits: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device).view(torch.float16)


def dev_bf16(bits: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device).view(torch.bfloat16)


def dev_weights(w: synth.AffineWeights, device="cuda"):
    return dev_codes(w.wq, device), dev_half(w.scales, device), dev_half(w.biases, device)


def dev_moe(mw: synth.MoEWeights, act: int = 0, device="cuda"):
    from affine_quantized_gemv_qgemv_amd import MoeWeights
    return MoeWeights(
        mw.E, mw.H, mw.I, mw.Is,
        dev_codes(mw.router.wq, device), dev_half(mw.router.scales, device),
        dev_half(mw.router.biases, device),
        dev_codes(mw.gu_wq, device), dev_half(mw.gu_s, device), dev_half(mw.gu_b, device),
        dev_codes(mw.dn_wq, device), dev_half(mw.dn_s, device), dev_half(mw.dn_b, device),
        dev_codes(mw.sgu.wq, device), dev_half(mw.sgu.scales, device), dev_half(mw.sgu.biases, device),
        dev_codes(mw.sdn.wq, device), dev_half(mw.sdn.scales, device), dev_half(mw.sdn.biases, device),
        act)


def host_bits(t: torch.Tensor) -> np.ndarray:
    """Raw 16-bit patterns of a float16/bfloat16 device tensor."""
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def _log_margin(what: str, worst: float) -> None:
    """Append the worst err/tol of one comparison to the JSON-lines file named by
    QD_MARGIN_LOG (if set), keyed by the running test, so margins per test
    family can be tabulated after a run."""
    path = os.environ.get("QD_MARGIN_LOG")
    if not path:
        return
    test = os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0]
    with open(path, "a") as f:
        f.write(json.dumps({"test": test, "what": what, "worst": worst}) + "\n")


def assert_within(y_gpu, y_ref, a_ref, what=""):
    """|y_gpu - y_ref| <= 1e-4 * A + 1e-6 element by element."""
    y = np.asarray(y_gpu, dtype=np.float64)
    err = np.abs(y - y_ref)
    tol = 1e-4 * a_ref + 1e-6
    bad = err > tol
    worst = float((err / tol).max()) if err.size else 0.0
    _log_margin(what, worst)
    if bad.any():
        i = np.unravel_index(np.argmax(err / tol), err.shape)
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outside tolerance; worst at {i}: "
                             f"gpu {y[i]!r} ref {y_ref[i]!r} err {err[i]:.3e} tol {tol[i]:.3e}")
    return worst
