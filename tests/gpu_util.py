"""Shared helpers for the GPU parity tests (not a test module).

Every comparison goes through :func:`check` or :func:`argmax_check`.  Both
print their measured figure, and both append one JSON line to the file named
by the environment variable ``DFLASH_PARITY_LOG`` when it is set.  The
committed parity record is written from that log.
"""
import json
import os

import numpy as np
import pytest
import torch

# A row's lm_head argmax may differ from the oracle's only when the oracle's
# own two best logits are closer than this (logit units; the stand-in lm_head
# gives logits of magnitude <= ~5, so this is ~0.5% of the largest).  Such
# rows are logged as exempt; every other row must match exactly.
ARGMAX_TIE_GAP = 0.025


def have_gpu() -> bool:
    return torch.cuda.is_available()


def parity_log(kind: str, name: str, **fields) -> None:
    path = os.environ.get("DFLASH_PARITY_LOG")
    if not path:
        return
    rec = {"kind": kind, "name": name, **fields}
    os.makedirs(os.path.dirname(os.path.abspath(path)), exist_ok=True)
    with open(path, "a") as fh:
        fh.write(json.dumps(rec) + "\n")


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
    parity_log("rel", name, rel=err, tol=tol, finite=bool(np.all(np.isfinite(gpu))))
    assert np.all(np.isfinite(gpu)), f"{name}: non-finite GPU output"
    assert err <= tol, f"{name}: relative error {err:.3e} > {tol:.1e}"
    return err


def argmax_verdict(out: np.ndarray, ref: np.ndarray, lm: np.ndarray):
    """Compares the argmax over a stand-in lm_head of two sets of hidden
    states.  Returns (mismatched rows, exempt rows, max logit difference),
    where exempt rows are those whose reference top-2 logit gap is below
    ARGMAX_TIE_GAP.  Pure host code: the CPU tests use it to show that a
    planted attention mistake fails the check."""
    from oracle import dflash_oracle as O
    am_o, lo_o = O.lm_argmax(ref, lm)
    am_g, lo_g = O.lm_argmax(out, lm)
    top2 = np.sort(lo_o, axis=1)[:, -2:]
    gap = top2[:, 1] - top2[:, 0]
    exempt = [int(r) for r in np.nonzero(gap < ARGMAX_TIE_GAP)[0]]
    bad = [int(r) for r in range(ref.shape[0]) if am_g[r] != am_o[r] and r not in exempt]
    return bad, exempt, float(np.abs(lo_g - lo_o).max())


def argmax_check(name, out, ref, lm):
    """Identical argmax in every row, near-ties of the reference aside."""
    bad, exempt, pert = argmax_verdict(out, ref, lm)
    from oracle import dflash_oracle as O
    am_o, _ = O.lm_argmax(ref, lm)
    am_g, _ = O.lm_argmax(out, lm)
    n_mis = int(np.sum(am_o != am_g))
    print(f"[argmax] {name}: mismatches={n_mis} outside near-ties={len(bad)} exempt rows={exempt} "
          f"max logit diff={pert:.3e}", flush=True)
    parity_log("argmax", name, mismatches=n_mis, bad=bad, exempt=exempt, max_logit_diff=pert,
               rows=int(ref.shape[0]), tie_gap=ARGMAX_TIE_GAP)
    assert not bad, f"{name}: argmax differs in rows {bad}"


gpu_only = pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")
