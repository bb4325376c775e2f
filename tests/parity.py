"""Comparison helpers for GPU-vs-oracle parity (test code only).

Acceptance bar (per element):
  * integer / index / byte work, and padding: bit-exact;
  * fp32 master, exp_avg, exp_avg_sq: e = |x_gpu - x_orc| / max(|x_orc|, kappa)
    <= 2e-6, where kappa guards against a 1-ulp difference after an exact
    cancellation: for exp_avg kappa = beta1|m_prev| + (1-beta1)|g|, for the
    master kappa = |p_prev (1 - lr wd)| + |update|, for exp_avg_sq kappa = 0;
  * bf16 parameters: <= 1 ulp (sign-magnitude integer distance);
  * squared norm: relative error of the norm <= 1e-5.
The bit-identical fraction is reported beside every float comparison.
"""
from __future__ import annotations

import numpy as np
import torch

F32_TOL = 2e-6
NORM_TOL = 1e-5


def to_np(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    return t.numpy().copy()


def from_np(a: np.ndarray, device="cuda", bf16: bool = False) -> torch.Tensor:
    if bf16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def bits_equal(a: np.ndarray, b: np.ndarray) -> bool:
    if a.dtype == np.float32:
        a, b = a.view(np.uint32), b.view(np.uint32)
    return a.shape == b.shape and np.array_equal(a, b)


def rel_err(gpu: np.ndarray, orc: np.ndarray, kappa=None) -> float:
    g = gpu.astype(np.float64)
    o = orc.astype(np.float64)
    den = np.abs(o)
    if kappa is not None:
        den = np.maximum(den, kappa)
    diff = np.abs(g - o)
    with np.errstate(invalid="ignore", divide="ignore"):
        e = np.where(diff == 0, 0.0, diff / den)
    return float(e.max()) if e.size else 0.0


def bf16_ulps(a: np.ndarray, b: np.ndarray) -> int:
    def sm(x):
        x = x.astype(np.int32)
        return np.where(x & 0x8000, -(x & 0x7FFF), x & 0x7FFF)
    return int(np.abs(sm(a) - sm(b)).max()) if a.size else 0


def identical_fraction(a: np.ndarray, b: np.ndarray) -> float:
    if a.size == 0:
        return 1.0
    if a.dtype == np.float32:
        a, b = a.view(np.uint32), b.view(np.uint32)
    return float(np.mean(a == b))


class StateCheck:
    """Compare one AdamW step's outputs with the bar above."""

    def __init__(self, beta1: float, lr: float, wd: float, step_size: float):
        self.b1, self.lr, self.wd, self.step_size = beta1, lr, wd, step_size

    def check(self, gpu: dict, orc: dict, prev: dict, g2: np.ndarray, label: str = "") -> dict:
        d = 1.0 - self.lr * self.wd
        k_m = self.b1 * np.abs(prev["m"].astype(np.float64)) + (1 - self.b1) * np.abs(g2.astype(np.float64))
        pd = np.abs(prev["p"].astype(np.float64) * d)
        k_p = pd + np.abs(prev["p"].astype(np.float64) * d - orc["p"].astype(np.float64))
        out = {
            "p": rel_err(gpu["p"], orc["p"], k_p),
            "m": rel_err(gpu["m"], orc["m"], k_m),
            "v": rel_err(gpu["v"], orc["v"]),
            "identical_p": identical_fraction(gpu["p"], orc["p"]),
            "identical_m": identical_fraction(gpu["m"], orc["m"]),
            "identical_v": identical_fraction(gpu["v"], orc["v"]),
        }
        assert out["p"] <= F32_TOL, (label, "master", out)
        assert out["m"] <= F32_TOL, (label, "exp_avg", out)
        assert out["v"] <= F32_TOL, (label, "exp_avg_sq", out)
        if "b" in gpu and gpu["b"] is not None:
            out["bf16_ulps"] = bf16_ulps(gpu["b"], orc["b"])
            assert out["bf16_ulps"] <= 1, (label, "bf16", out)
        return out
