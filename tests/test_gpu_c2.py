"""GPU parity for the fresh full-context forward of the 5-layer bf16 drafter
(6 taps, fc K = 12288) over n = 1024 ctx rows plus a 16-token block:
ctx_features(1024) -> scratch cache -> ingest(1024) -> forward_round, against
the oracle's independent forward_full, every output element, plus the argmax
check and a bitwise repeat."""
import numpy as np
import pytest
import torch

import synth
from oracle import dflash_oracle as O
from tests.gpu_util import argmax_check, check, dev, host, tol_for

pytestmark = pytest.mark.gpu


def test_c2_forward_full_matches_oracle():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    from block_diffusion_drafter_round_amd import dflash as D
    cfg = synth.FULL5_BF16
    sw = synth.make_weights(cfg)
    m = O.OracleModel(sw)
    n, b = cfg.ctx, cfg.block
    dr = D.Drafter(sw, max_rows=n)
    taps, noise, pos = synth.make_taps(cfg, n), synth.make_noise(cfg), synth.positions(0, n + b)
    t_taps, t_noise, t_pos = dev(taps), dev(noise), dev(pos)
    out = host(dr.forward_full(t_taps, t_noise, t_pos))
    out2 = host(dr.forward_full(t_taps, t_noise, t_pos))
    dr.status()
    assert np.array_equal(out, out2), "forward_full is not bitwise deterministic"
    feats = host(dr.ctx_features(t_taps))
    check("c2 ctx_features(1024)", feats, O.ctx_features(m, taps), 2e-3)
    ref = O.forward_full(m, taps, noise, pos, n)
    check(f"c2 forward_full n={n}", out, ref, tol_for(cfg))
    argmax_check(f"c2 forward_full n={n}", out, ref, synth.make_lm_head(cfg).astype(np.float64))
