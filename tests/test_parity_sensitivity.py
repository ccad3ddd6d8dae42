"""The full-size parity checks fail on planted attention mistakes (CPU only).

The GPU tests at c3/c4/c5 compare the round's output with the oracle at
2e-2 and check the argmax over a stand-in lm_head.  This module plants
mistakes in a copy of the oracle's attention, on the CPU, at the c3 shape
(8 layers, 4096 cached rows + 16 block rows), and runs the very comparison
functions the GPU tests use:

* one 64-key split of the cache dropped (the round kernel splits the 4096
  keys of c3 into 64 splits of 64 keys);
* the block's own 16 keys dropped;
* the splits merged without their softmax weights (a plain mean of the
  per-split normalised outputs);
* attention over the last 512 keys only.

With N(0, 1) block embeddings the first two hide inside 2e-2 (attention
carries little of the output there); with the embeddings scaled by 0.1, as
the GPU tests' second case does, every mistake moves the output at least
four times the tolerance, while the kernel's bf16 rounding moves it by
~1.1e-2.  The cache is prefilled directly with seeded bf16 K/V (as the
c4/c5 tests do), then 16 rows are ingested as in a round.
"""
import numpy as np
import pytest

import synth
from oracle import dflash_oracle as O
from tests.gpu_util import argmax_verdict, rel_rows

TOL = 2e-2
SPLIT = 64
_ATT = O.attention          # the oracle's own attention, which the mutants call


def _drop_split(q, K, V):
    keep = np.ones(K.shape[0], bool)
    keep[SPLIT:2 * SPLIT] = False
    return _ATT(q, K[keep], V[keep])


def _drop_block(q, K, V):
    return _ATT(q, K[:-q.shape[0]], V[:-q.shape[0]])


def _unweighted_merge(q, K, V):
    parts = [_ATT(q, K[s:s + SPLIT], V[s:s + SPLIT]) for s in range(0, K.shape[0], SPLIT)]
    return np.mean(parts, axis=0)


def _last512(q, K, V):
    return _ATT(q, K[-512 - q.shape[0]:], V[-512 - q.shape[0]:])


MUTANTS = {"drop_split": _drop_split, "drop_block": _drop_block, "unweighted_merge": _unweighted_merge,
           "last512": _last512}


@pytest.fixture(scope="module")
def c3_round():
    cfg = synth.ROUND8_BF16
    m = O.OracleModel(synth.make_weights(cfg))
    ctx, t, b = cfg.ctx, cfg.new_rows, cfg.block
    base = ctx - t
    kv = O.OracleKV(cfg)
    ks, vs = synth.make_prefill_kv(cfg, base)
    kv.prefill(ks, vs)
    taps = synth.make_taps(cfg, t, stream=1)
    O.ingest_ctx(m, kv, O.ctx_features(m, taps), synth.positions(base, t))
    return cfg, m, kv, synth.positions(ctx, b), synth.make_lm_head(cfg).astype(np.float64)


def _run(m, kv, noise, pos, name, monkeypatch):
    """The oracle's round with its attention replaced by a mutant."""
    with monkeypatch.context() as mp:
        mp.setattr(O, "attention", MUTANTS[name])
        return O.forward_round(m, kv, noise, pos)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_attention_sensitive_round_catches_mistake(c3_round, name, monkeypatch):
    cfg, m, kv, pos, lm = c3_round
    noise = synth.make_noise(cfg) * np.float32(0.1)
    ref = O.forward_round(m, kv, noise, pos)
    bad = _run(m, kv, noise, pos, name, monkeypatch)
    err = rel_rows(bad, ref)
    print(f"[sensitivity] emb x0.1 {name}: rel={err:.3e}")
    assert err > 4 * TOL, f"{name} moves the output by only {err:.3e}"


def test_plain_scale_blind_spot_is_real(c3_round, monkeypatch):
    """Why the x0.1 case exists: at the plain scale a dropped split or
    dropped block keys stay inside the tolerance."""
    cfg, m, kv, pos, lm = c3_round
    noise = synth.make_noise(cfg)
    ref = O.forward_round(m, kv, noise, pos)
    for name in ("drop_split", "drop_block"):
        err = rel_rows(_run(m, kv, noise, pos, name, monkeypatch), ref)
        print(f"[sensitivity] emb x1 {name}: rel={err:.3e}")
        assert err < TOL


@pytest.mark.parametrize("emb_scale", [1.0, 0.1])
def test_argmax_check_catches_truncated_attention(c3_round, emb_scale, monkeypatch):
    cfg, m, kv, pos, lm = c3_round
    noise = synth.make_noise(cfg) * np.float32(emb_scale)
    ref = O.forward_round(m, kv, noise, pos)
    bad_rows, exempt, _ = argmax_verdict(_run(m, kv, noise, pos, "last512", monkeypatch), ref, lm)
    print(f"[sensitivity] emb x{emb_scale:g} last512: argmax differs in {len(bad_rows)} rows, exempt {exempt}")
    assert len(bad_rows) >= 4
    # and the unmutated round passes the same check
    bad0, _, _ = argmax_verdict(ref.copy(), ref, lm)
    assert not bad0
