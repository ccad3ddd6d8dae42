"""GPU parity at the benchmark's full size: the 8-layer bf16 drafter, one
cached round at ctx 4096 (ctx_features 16 + ingest 16 + forward_round b=16),
in the same launch configuration bench.py times.

The oracle computes every output element at this size in a few seconds, so
the comparison is complete.  Each round is checked twice over:
* every output element against the oracle (2e-2, per-row relative);
* the argmax over a seeded 151,936-row stand-in lm_head, identical in every
  row whose oracle top-2 gap is not a near-tie.

With N(0, 0.02) weights and N(0, 1) block embeddings, attention contributes
little to the output: dropping a whole 64-key split moves it by only
~1.5e-2.  The second round therefore scales the block embeddings by 0.1, so
that attention shapes the residual stream.  There the planted mistakes move
the output by 0.08 to 0.27 while the kernel's bf16 rounding moves it by
~1.1e-2 (a CPU emulation of its rounding points, and this test on the GPU);
tests/test_parity_sensitivity.py pins the mistakes' effect on the CPU.  A
smaller scale makes the layers amplify every rounding as much as the
mistakes (x0.01: 1.8e-2 from rounding alone), so 0.1 is the balance.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import dflash_oracle as O
from tests.gpu_util import argmax_check, check, dev, host, tol_for

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def c3():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    from block_diffusion_drafter_round_amd import dflash as D
    cfg = synth.ROUND8_BF16
    sw = synth.make_weights(cfg)
    m = O.OracleModel(sw)
    dr = D.Drafter(sw, max_rows=1024)
    ctx, t, b = cfg.ctx, cfg.new_rows, cfg.block
    base = ctx - t
    kv = D.KVCache(cfg, (ctx + b + 63) // 64 * 64)
    okv = O.OracleKV(cfg)
    for lo in range(0, base, 1020):
        hi = min(base, lo + 1020)
        taps = synth.make_taps(cfg, hi - lo, stream=1000 + lo)
        pos = synth.positions(lo, hi - lo)
        dr.ingest_ctx(kv, dr.ctx_features(dev(taps)), dev(pos))
        O.ingest_ctx(m, okv, O.ctx_features(m, taps), pos)
    print(f"[c3] prefilled {base} rows", flush=True)
    lm = synth.make_lm_head(cfg).astype(np.float64)
    return cfg, m, dr, kv, okv, D, lm


@pytest.mark.parametrize("emb_scale", [1.0, 0.1])
def test_c3_round_matches_oracle(c3, emb_scale):
    cfg, m, dr, kv, okv, D, lm = c3
    ctx, t, b = cfg.ctx, cfg.new_rows, cfg.block
    base = ctx - t
    kv.len = base
    okv.truncate(base)
    taps = synth.make_taps(cfg, t, stream=1)
    noise = synth.make_noise(cfg) * np.float32(emb_scale)
    pos_new, pos_blk = synth.positions(base, t), synth.positions(ctx, b)
    tag = f"c3 emb x{emb_scale:g}"

    feats = dr.ctx_features(dev(taps))
    check(f"{tag} ctx_features(16)", host(feats), O.ctx_features(m, taps), 2e-3)
    dr.ingest_ctx(kv, feats, dev(pos_new))
    out = host(dr.forward_round(kv, dev(noise), dev(pos_blk)))
    dr.status()
    assert kv.len == ctx

    O.ingest_ctx(m, okv, O.ctx_features(m, taps), pos_new)
    ref = O.forward_round(m, okv, noise, pos_blk)
    check(f"{tag} forward_round ctx 4096", out, ref, tol_for(cfg))
    argmax_check(f"{tag} forward_round ctx 4096", out, ref, lm)

    # rewind and repeat: deterministic, and len-only rewind is a valid state
    kv.len = base
    dr.ingest_ctx(kv, dr.ctx_features(dev(taps)), dev(pos_new))
    out2 = host(dr.forward_round(kv, dev(noise), dev(pos_blk)))
    assert np.array_equal(out, out2), "round is not bitwise deterministic"
