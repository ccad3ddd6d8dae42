"""GPU parity at long context.

* The 8-layer bf16 drafter with YaRN rope (factor 32), one cached round at
  ctx 32768 per sequence, in the launch configuration of the multi-sequence
  benchmark (one forward_round call per sequence, each on its own cache,
  back to back).
* The 8-layer fp8 e4m3fn drafter (per-row f32 scales) with the DFlash2 conv
  wrap (G = 16) around every sublayer, one cached round at ctx 65536.

The oracle cannot ingest 32,752 rows per sequence in reasonable time, so each
cache is prefilled directly with the same seeded bf16 K/V on both sides; the
round itself (ctx_features 16 + ingest 16 + forward_round b=16) runs in full
through the library and the oracle, and every output element is compared.
Three of the eight sequences are checked against the oracle; all eight must be
bitwise reproducible.  One c4 sequence and the c5 round are also run with
the block embeddings scaled by 0.1, which lets attention shape the output,
so a mistake in the key splits or their merge cannot hide inside the
tolerance (tests/test_parity_sensitivity.py pins that on the CPU).  Every
argmax must match the oracle's outside near-ties.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import dflash_oracle as O
from tests.gpu_util import argmax_check, check, dev, host, kv_rows_f64, tol_for

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def c4():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    from block_diffusion_drafter_round_amd import dflash as D
    cfg = synth.ROUND8_YARN
    sw = synth.make_weights(cfg)
    return cfg, O.OracleModel(sw), D.Drafter(sw, max_rows=64), D


def _round_inputs(cfg, seq, emb_scale=1.0):
    ctx, t, b = cfg.ctx, cfg.new_rows, cfg.block
    base = ctx - t
    return (synth.make_taps(cfg, t, stream=100 + seq), synth.make_noise(cfg, stream=seq) * np.float32(emb_scale),
            synth.positions(base, t), synth.positions(ctx, b))


def _gpu_round(cfg, dr, D, ks, vs, seq, emb_scale=1.0):
    ctx, b = cfg.ctx, cfg.block
    kv = D.KVCache(cfg, (ctx + b + 63) // 64 * 64)
    kv.prefill(ks, vs)
    taps, noise, pos_new, pos_blk = _round_inputs(cfg, seq, emb_scale)
    dr.ingest_ctx(kv, dr.ctx_features(dev(taps)), dev(pos_new))
    out = dr.forward_round(kv, dev(noise), dev(pos_blk))
    assert kv.len == ctx
    return kv, host(out)


@pytest.mark.parametrize("seq,emb_scale", [(0, 1.0), (3, 1.0), (7, 1.0), (0, 0.1)])
def test_c4_round_matches_oracle(c4, seq, emb_scale):
    cfg, m, dr, D = c4
    ctx, t, b = cfg.ctx, cfg.new_rows, cfg.block
    base = ctx - t
    ks, vs = synth.make_prefill_kv(cfg, base, stream=seq)
    print(f"[c4] seq {seq} emb x{emb_scale:g}: prefilled {base} rows", flush=True)
    kv, out = _gpu_round(cfg, dr, D, ks, vs, seq, emb_scale)
    dr.status()

    okv = O.OracleKV(cfg)
    okv.prefill(ks, vs)
    del ks, vs
    taps, noise, pos_new, pos_blk = _round_inputs(cfg, seq, emb_scale)
    O.ingest_ctx(m, okv, O.ctx_features(m, taps), pos_new)
    for l in (0, cfg.n_layers - 1):
        k, v = kv_rows_f64(kv, l, base, ctx)
        check(f"c4 seq {seq} layer {l} ingested K (YaRN)", k, okv.k[l][base:], 1e-2)
        check(f"c4 seq {seq} layer {l} ingested V", v, okv.v[l][base:], 1e-2)
    ref = O.forward_round(m, okv, noise, pos_blk)
    tag = f"c4 seq {seq} emb x{emb_scale:g} forward_round ctx {ctx}"
    check(tag, out, ref, tol_for(cfg))
    argmax_check(tag, out, ref, synth.make_lm_head(cfg).astype(np.float64))


def test_c4_eight_sequences_reproducible(c4):
    """All eight sequences back to back, twice: every output is bitwise equal
    across the two sweeps, and the sequences differ from one another."""
    cfg, m, dr, D = c4
    base = cfg.ctx - cfg.new_rows
    outs = []
    for seq in range(cfg.n_seqs):
        ks, vs = synth.make_prefill_kv(cfg, base, stream=seq)
        kv, o1 = _gpu_round(cfg, dr, D, ks, vs, seq)
        kv.len = base
        _, noise, pos_new, pos_blk = _round_inputs(cfg, seq)
        taps = _round_inputs(cfg, seq)[0]
        dr.ingest_ctx(kv, dr.ctx_features(dev(taps)), dev(pos_new))
        o2 = host(dr.forward_round(kv, dev(noise), dev(pos_blk)))
        dr.status()
        assert np.array_equal(o1, o2), f"sequence {seq} not reproducible"
        outs.append(o1)
        del kv
        torch.cuda.empty_cache()
        print(f"[c4] sweep seq {seq} ok", flush=True)
    for s in range(1, len(outs)):
        assert not np.array_equal(outs[0], outs[s])


def test_c5_fp8_d2conv_round_matches_oracle():
    """fp8 weights + DFlash2 conv at ctx 65536: the full round against the
    oracle on a directly prefilled cache, plus the argmax check and a bitwise
    repeat."""
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    from block_diffusion_drafter_round_amd import dflash as D
    cfg = synth.ROUND8_FP8_D2
    sw = synth.make_weights(cfg)
    m = O.OracleModel(sw)
    dr = D.Drafter(sw, max_rows=64)
    ctx, t, b = cfg.ctx, cfg.new_rows, cfg.block
    base = ctx - t
    ks, vs = synth.make_prefill_kv(cfg, base)
    print(f"[c5] prefilled {base} rows", flush=True)
    kv, out = _gpu_round(cfg, dr, D, ks, vs, 0)
    dr.status()
    kv.len = base
    taps, noise, pos_new, pos_blk = _round_inputs(cfg, 0)
    dr.ingest_ctx(kv, dr.ctx_features(dev(taps)), dev(pos_new))
    out2 = host(dr.forward_round(kv, dev(noise), dev(pos_blk)))
    assert np.array_equal(out, out2), "c5 round is not bitwise deterministic"

    okv = O.OracleKV(cfg)
    okv.prefill(ks, vs)
    del ks, vs
    O.ingest_ctx(m, okv, O.ctx_features(m, taps), pos_new)
    k, v = kv_rows_f64(kv, cfg.n_layers - 1, base, ctx)
    check("c5 last layer ingested K", k, okv.k[cfg.n_layers - 1][base:], 1e-2)
    check("c5 last layer ingested V", v, okv.v[cfg.n_layers - 1][base:], 1e-2)
    ref = O.forward_round(m, okv, noise, pos_blk)
    lm = synth.make_lm_head(cfg).astype(np.float64)
    check(f"c5 fp8 + DFlash2 conv forward_round ctx {ctx}", out, ref, tol_for(cfg))
    argmax_check(f"c5 fp8 + DFlash2 conv forward_round ctx {ctx}", out, ref, lm)

    # attention-sensitive variant: block embeddings x0.1, same cache
    noise_s = noise * np.float32(0.1)
    kv.len = base
    dr.ingest_ctx(kv, dr.ctx_features(dev(taps)), dev(pos_new))
    out_s = host(dr.forward_round(kv, dev(noise_s), dev(pos_blk)))
    dr.status()
    ref_s = O.forward_round(m, okv, noise_s, pos_blk)
    check(f"c5 emb x0.1 forward_round ctx {ctx}", out_s, ref_s, tol_for(cfg))
    argmax_check(f"c5 emb x0.1 forward_round ctx {ctx}", out_s, ref_s, lm)
