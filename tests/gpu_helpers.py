"""Helpers for GPU tests: moving seeded inputs to the device and reading results back.

Only data movement lives here (no step of the method): bfloat16 bit patterns
become torch bfloat16 tensors, coefficient rows become the value cache's
octet layout and back, and errors are measured against the oracle's float64.
"""
import math

import numpy as np
import torch

import lrkv_synth as synth

DEV = "cuda:0"


def to_dev(s, dtype: str) -> torch.Tensor:
    """Stored (or raw storage array) -> device tensor of the storage dtype."""
    a = s.store if isinstance(s, synth.Stored) else s
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").to(torch.float64).numpy()


def bits(t: torch.Tensor) -> np.ndarray:
    """Raw storage of a device tensor (uint16 bf16 patterns, or float32)."""
    t = t.detach().to("cpu").contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def round_store(x: np.ndarray, dtype: str) -> np.ndarray:
    """float64 -> storage array (bf16 bits via the generator's rounding, or float32)."""
    if dtype == "bf16":
        return synth.f32_to_bf16_bits(np.asarray(x, dtype=np.float64).astype(np.float32))
    return np.asarray(x, dtype=np.float32)


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    """Spacing of bfloat16 numbers at |x| (8 significant bits)."""
    ax = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.where(ax > 0, ax, 2.0 ** -126)))
    return np.ldexp(1.0, (e - 7).astype(int))


def row_errors(o_gpu: np.ndarray, o_ref: np.ndarray, mode: str) -> np.ndarray:
    """Per-row normalised max error.

    mode "max": max|o_gpu - o_ref| / max|o_ref|   (the float32 gate)
    mode "rms": max|o_gpu - o_ref| / rms(o_ref)   (the bfloat16 unit-scale gate)
    """
    err = np.max(np.abs(o_gpu - o_ref), axis=-1)
    if mode == "max":
        den = np.max(np.abs(o_ref), axis=-1)
    else:
        den = np.sqrt(np.mean(o_ref ** 2, axis=-1))
    return err / np.maximum(den, 1e-30)


# Gates (per output row): float32 workloads 1e-4 of the row's max, bfloat16
# workloads 2e-2 of the row's RMS ("unit scale"); lse 1e-5 relative (fp32) or
# 1e-3 absolute (bf16).
GATE = {"f32": 1e-4, "bf16": 2e-2}
LSE_GATE = {"f32": 1e-5, "bf16": 1e-3}


def check_decode(o_gpu, lse_gpu, o_ref, lse_ref, dtype: str, what: str = "", storage_rounding: bool = False):
    """Decode gate per output row (see GATE).  storage_rounding=True (latent
    outputs, whose elements scale with the coefficient spectrum instead of
    being unit scale) also allows each element the half bfloat16 ulp that
    storing the exact result itself costs: |o_gpu - o_ref| <= 2e-2 rms(o_ref)
    + ulp(o_ref) / 2.  On the latent rows of the batched workload that rounding
    alone reaches 2.0e-2 of the row RMS (a row's largest element is up to 7x
    its RMS), so no bfloat16 output could meet the plain gate there."""
    mode = "max" if dtype == "f32" else "rms"
    if storage_rounding and dtype == "bf16":
        den = np.maximum(np.sqrt(np.mean(o_ref ** 2, axis=-1)), 1e-30)
        excess = np.abs(o_gpu - o_ref) - 0.5 * bf16_ulp(o_ref)
        e = np.max(excess, axis=-1) / den
    else:
        e = row_errors(o_gpu, o_ref, mode)
    assert np.all(np.isfinite(o_gpu)), f"{what}: non-finite output"
    assert e.max() <= GATE[dtype], f"{what}: worst row error {e.max():.3e} > {GATE[dtype]}"
    if lse_gpu is not None:
        d = np.abs(lse_gpu - lse_ref)
        tol = LSE_GATE[dtype] * (np.maximum(1.0, np.abs(lse_ref)) if dtype == "f32" else 1.0)
        assert np.all(d <= tol), f"{what}: lse error {d.max():.3e}"
    return float(e.max())
