"""Helpers shared by the GPU parity tests: device transfer and the parity criteria.

Parity criteria (written out in each test's assertion):
  * fp32: max |gpu - oracle| <= 1e-5 (the course page's 1e-5 agreement with torch's
    scaled_dot_product_attention, "Week 7. Attention", code section);
  * bf16: max |gpu - oracle| <= 2e-2 AND max |gpu - oracle| / max |oracle| <= 1e-2.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import workloads

F32_ATOL = 1e-5
BF16_ATOL = 2e-2
BF16_REL = 1e-2


def say(msg: str) -> None:
    """Name the case before each GPU step, flushed, so a failing run still says what it ran."""
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


def to_dev(t):
    if isinstance(t, np.ndarray):
        t = torch.from_numpy(t)
    return t.contiguous().cuda()


def host_view(t: torch.Tensor) -> np.ndarray:
    """A CPU tensor as the oracle's input array: float32 values, or bf16 bit patterns."""
    t = t.cpu()
    if t.dtype == torch.bfloat16:
        return workloads.bf16_bits(t)
    return t.numpy()


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def errors(got: np.ndarray, ref: np.ndarray):
    err = float(np.max(np.abs(got - ref))) if got.size else 0.0
    scale = float(np.max(np.abs(ref))) if ref.size else 1.0
    return err, err / scale if scale > 0 else err


def assert_bf16_close(got: np.ndarray, ref: np.ndarray, what: str = ""):
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err, rel = errors(got, ref)
    assert err <= BF16_ATOL and rel <= BF16_REL, f"{what}: max-abs {err:.3e}, rel-to-max {rel:.3e}"
    return err, rel


def assert_f32_close(got: np.ndarray, ref: np.ndarray, atol: float = F32_ATOL, what: str = ""):
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err, rel = errors(got, ref)
    assert err <= atol, f"{what}: max-abs {err:.3e} > {atol:.1e}"
    return err, rel
