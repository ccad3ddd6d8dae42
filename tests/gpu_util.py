"""Shared helpers for the GPU parity tests (not a test module)."""
import numpy as np
import pytest
import torch

import synth
from oracle import dflash_oracle as O


def have_gpu() -> bool:
    return torch.cuda.is_available()


def rel_rows(gpu: np.ndarray, ref: np.ndarray) -> float:
    """max over rows of (max_c |gpu - ref| / max_c |ref|): the per-row
    infinity-norm relative error the tolerances are stated in."""
    gpu = np.asarray(gpu, dtype=np.float64).reshape(ref.shape[0], -1)
    ref = np.asarray(ref, dtype=np.float64).reshape(ref.shape[0], -1)
    den = np.maximum(np.abs(ref).max(axis=1), 1e-300)
    return float((np.abs(gpu - ref).max(axis=1) / den).max())


def tol_for(cfg) -> float:
    """f32 arm: 1e-4; bf16 / fp8 weights with f32 accumulation: 2e-2."""
    return 1e-4 if cfg.weight_dtype == "f32" else 2e-2


def dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def kv_rows_f64(kv, layer: int, start: int, stop: int):
    k, v = kv.rows(layer, start, stop)
    return host(k), host(v)


def check(name, gpu, ref, tol, drafter=None):
    if drafter is not None:
        drafter.status()
    err = rel_rows(gpu, ref)
    print(f"[parity] {name}: rel={err:.3e} tol={tol:.1e}", flush=True)
    assert np.all(np.isfinite(gpu)), f"{name}: non-finite GPU output"
    assert err <= tol, f"{name}: relative error {err:.3e} > {tol:.1e}"
    return err


gpu_only = pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")
