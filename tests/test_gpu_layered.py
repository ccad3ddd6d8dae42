"""GPU parity of the layered round path: batched sequences
(dflash_forward_round_batch; [atlas dflash_head] DflashProposerState, one
cache per sequence), paged caches with a block table shared by all layers,
and the context window ([atlas dflash_head] dflash_ctx_cap).

* Batched: every sequence against the oracle's own round on its cache, with
  different cache lengths per sequence and ragged b.
* Paged: ingest and round through a paged cache whose block table is a
  seeded permutation of the pool; the cache rows equal the oracle's, and the
  round is bitwise equal to the same round on contiguous storage.
* Window: smaller than, equal to and larger than the cache, unaligned
  window starts; against the oracle's windowed round.
* Full size: c3 with a 1024-row window on a paged cache, and the c4 sweep
  (8 YaRN sequences at ctx 32768) in one batched call, with the x0.1
  block-embedding case that lets attention shape the output.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import dflash_oracle as O
from tests.gpu_util import argmax_check, check, dev, host, kv_rows_f64, tol_for

pytestmark = pytest.mark.gpu

SMALL_BF16 = synth.DraftConfig(
    name="small_bf16", n_layers=2, hidden=512, n_q_heads=8, n_kv_heads=2, head_dim=64,
    intermediate=768, n_taps=2, weight_dtype="bf16", kv_dtype="bf16", path="round",
    ctx=100, block=16, seed=21)
SMALL_D128_FP8 = SMALL_BF16.replace(name="small_fp8_d128", hidden=1024, n_q_heads=8, n_kv_heads=1,
                                    head_dim=128, weight_dtype="fp8", seed=24)
SMALL_YARN = SMALL_BF16.replace(name="small_yarn_d128", hidden=1024, n_q_heads=8, n_kv_heads=1,
                                head_dim=128, rope_type="yarn", seed=25)
# DFlash2 conv wrap around every sublayer: bf16 with G = 4, fp8 head_dim 128 with G = 16
SMALL_D2 = SMALL_BF16.replace(name="small_bf16_d2", d2_groups=4, seed=27)
SMALL_FP8_D2 = SMALL_D128_FP8.replace(name="small_fp8_d128_d2", d2_groups=16, seed=28)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def _setup(cfg, max_rows=64):
    from block_diffusion_drafter_round_amd import dflash as D
    sw = synth.make_weights(cfg)
    return O.OracleModel(sw), D.Drafter(sw, max_rows=max_rows), D


def _ingest_both(cfg, m, dr, kv, okv, n, stream, pos0=0):
    """n ctx rows through ctx_features + ingest, on the GPU and in the oracle."""
    taps = synth.make_taps(cfg, n, stream=stream)
    pos = synth.positions(pos0, n)
    dr.ingest_ctx(kv, dr.ctx_features(dev(taps)), dev(pos))
    O.ingest_ctx(m, okv, O.ctx_features(m, taps), pos)


@pytest.mark.parametrize("cfg", [SMALL_BF16, SMALL_D128_FP8, SMALL_YARN, SMALL_D2, SMALL_FP8_D2], ids=lambda c: c.name)
@pytest.mark.parametrize("b", [16, 5])
def test_batched_round_matches_oracle(cfg, b):
    m, dr, D = _setup(cfg)
    lens = [0, 37, 100, 64, 129]
    S = len(lens)
    caches, okvs = [], []
    for s, n in enumerate(lens):
        kv = D.KVCache(cfg, 256)
        okv = O.OracleKV(cfg)
        if n:
            _ingest_both(cfg, m, dr, kv, okv, n, stream=s, pos0=30000 if cfg.rope_type == "yarn" else 0)
        caches.append(kv)
        okvs.append(okv)
    base = 30000 if cfg.rope_type == "yarn" else 0
    noise = np.stack([synth.make_noise(cfg, b, stream=s) for s in range(S)])
    pos = np.stack([synth.positions(base + n, b) for n in lens])
    out = host(dr.forward_round_batch(caches, dev(noise), dev(pos)))
    ref = O.forward_round_batch(m, okvs, noise, pos)
    for s in range(S):
        check(f"{cfg.name} batched seq {s} (len {lens[s]}) b={b}", out[s], ref[s], tol_for(cfg))
    assert [c.len for c in caches] == lens
    # the same sequences one call each: the layered path is deterministic per sequence
    out1 = host(dr.forward_round_batch(caches[1:2], dev(noise[1:2]), dev(pos[1:2])))
    check(f"{cfg.name} single-sequence batch", out1[0], ref[1], tol_for(cfg))


@pytest.mark.parametrize("cfg", [SMALL_BF16, SMALL_D128_FP8], ids=lambda c: c.name)
def test_paged_cache_matches_contiguous_and_oracle(cfg):
    m, dr, D = _setup(cfg)
    cap, n, b = 512, 300, 16
    paged = D.PagedKVCache(cfg, cap, page_rows=64, pool_pages=11, seed=3)   # pool larger than the table
    flat = D.KVCache(cfg, cap)
    okv = O.OracleKV(cfg)
    for lo, hi in ((0, 70), (70, 200), (200, 300)):                         # ingest across page borders
        taps = synth.make_taps(cfg, hi - lo, stream=lo)
        pos = synth.positions(lo, hi - lo)
        feats = dr.ctx_features(dev(taps))
        dr.ingest_ctx(paged, feats, dev(pos))
        dr.ingest_ctx(flat, feats, dev(pos))
        O.ingest_ctx(m, okv, O.ctx_features(m, taps), pos)
    for l in (0, cfg.n_layers - 1):
        k, v = kv_rows_f64(paged, l, 0, n)
        check(f"{cfg.name} paged layer {l} K rows", k, okv.k[l], 1e-2)
        check(f"{cfg.name} paged layer {l} V rows", v, okv.v[l], 1e-2)
        kf, vf = kv_rows_f64(flat, l, 0, n)
        assert np.array_equal(k, kf) and np.array_equal(v, vf), "paged and contiguous ingest differ"
    noise, pos_b = synth.make_noise(cfg), synth.positions(n, b)
    out_p = host(dr.forward_round(paged, dev(noise), dev(pos_b)))
    out_f = host(dr.forward_round_batch([flat], dev(noise[None]), dev(pos_b[None])))[0]
    assert np.array_equal(out_p, out_f), "paged round differs from the contiguous layered round"
    check(f"{cfg.name} paged round", out_p, O.forward_round(m, okv, noise, pos_b), tol_for(cfg))
    # the persistent kernel on the contiguous cache agrees within tolerance
    check(f"{cfg.name} persistent vs layered", host(dr.forward_round(flat, dev(noise), dev(pos_b))), out_p, tol_for(cfg))


@pytest.mark.parametrize("cap_rows", [1, 31, 33, 128, 200, 300, 1000])
def test_window_matches_oracle(cap_rows):
    cfg = SMALL_BF16
    m, dr, D = _setup(cfg)
    n, b = 300, 16
    for paged in (False, True):
        kv = D.PagedKVCache(cfg, 512, page_rows=128, seed=9) if paged else D.KVCache(cfg, 512)
        okv = O.OracleKV(cfg)
        _ingest_both(cfg, m, dr, kv, okv, n, stream=1)
        kv.c.ctx_cap = cap_rows
        noise, pos_b = synth.make_noise(cfg), synth.positions(n, b)
        out = host(dr.forward_round(kv, dev(noise), dev(pos_b)))
        ref = O.forward_round(m, okv, noise, pos_b, ctx_cap=cap_rows)
        check(f"window {cap_rows} over {n} rows ({'paged' if paged else 'contiguous'})", out, ref, tol_for(cfg))
        if cap_rows < n:      # the window matters: the unwindowed oracle is measurably different
            assert np.abs(O.forward_round(m, okv, noise, pos_b) - ref).max() > 1e-3


def test_forward_full_with_paged_scratch():
    cfg = SMALL_BF16
    m, dr, D = _setup(cfg, max_rows=100)
    n, b = 100, 16
    taps, noise, pos = synth.make_taps(cfg, n), synth.make_noise(cfg), synth.positions(0, n + b)
    scratch = D.PagedKVCache(cfg, 128, page_rows=64, seed=2)
    out = host(dr.forward_full(dev(taps), dev(noise), dev(pos), scratch))
    check("forward_full, paged scratch", out, O.forward_full(m, taps, noise, pos, n), tol_for(cfg))


def test_layered_path_argument_errors():
    from block_diffusion_drafter_round_amd import dflash as D
    cfg = SMALL_BF16
    m, dr, _ = _setup(cfg)
    kv = D.KVCache(cfg, 128)
    noise, pos = dev(synth.make_noise(cfg)), dev(synth.positions(0, 16))
    dr.ensure_batch(2)
    out = torch.empty((2, 16, cfg.hidden), device="cuda")
    with pytest.raises(D.DflashError) as ei:                     # two sequences on one storage
        D.dflash_forward_round_batch(dr.model, D.kv_array([kv, kv]), torch.stack([noise, noise]),
                                     torch.stack([pos, pos]), 16, out, dr.ws, dr.ws_bytes)
    assert ei.value.code == D.DFLASH_E_INVAL
    kv.c.ctx_cap = -1
    with pytest.raises(D.DflashError):
        dr.forward_round(kv, noise, pos)
    f32 = synth.TINY_F32
    dr32 = D.Drafter(synth.make_weights(f32), max_rows=16)
    kv32 = D.PagedKVCache(f32, 128, page_rows=64)
    with pytest.raises(D.DflashError) as ei:                     # f32 KV: persistent kernel only
        dr32.forward_round(kv32, dev(synth.make_noise(f32)), dev(synth.positions(0, 16)))
    assert ei.value.code == D.DFLASH_E_UNSUPPORTED


# ------------------------------------------------------------------ full size --
def test_c3_window_1024_paged():
    """The c3 drafter (8 layers, bf16) at ctx 4096 on a paged cache with a
    1024-row window: the ctx prefill through the library, one round with
    N(0,1) and with x0.1 block embeddings, against the oracle."""
    cfg = synth.ROUND8_BF16
    m, dr, D = _setup(cfg, max_rows=1020)
    ctx, b = cfg.ctx, cfg.block
    kv = D.PagedKVCache(cfg, (ctx + b + 255) // 256 * 256, page_rows=256, seed=5)
    okv = O.OracleKV(cfg)
    for lo in range(0, ctx, 1020):
        _ingest_both(cfg, m, dr, kv, okv, min(ctx, lo + 1020) - lo, stream=1000 + lo, pos0=lo)
    kv.c.ctx_cap = 1024
    lm = synth.make_lm_head(cfg).astype(np.float64)
    for scale in (1.0, 0.1):
        noise, pos_b = synth.make_noise(cfg) * np.float32(scale), synth.positions(ctx, b)
        out = host(dr.forward_round(kv, dev(noise), dev(pos_b)))
        ref = O.forward_round(m, okv, noise, pos_b, ctx_cap=1024)
        tag = f"c3 paged window 1024 emb x{scale:g}"
        check(tag, out, ref, tol_for(cfg))
        argmax_check(tag, out, ref, lm)


def test_c4_sweep_batched():
    """The c4 sweep in one batched call: 8 YaRN sequences at ctx 32768, each
    cache prefilled directly with its own seeded bf16 rows; three sequences
    against the oracle (also at x0.1 embeddings), all eight finite and
    bitwise reproducible."""
    cfg = synth.ROUND8_YARN
    m, dr, D = _setup(cfg, max_rows=16)
    ctx, b, S = cfg.ctx, cfg.block, cfg.n_seqs
    caches, prefills = [], []
    for s in range(S):
        kv = D.KVCache(cfg, (ctx + b + 63) // 64 * 64)
        ks, vs = synth.make_prefill_kv(cfg, ctx, stream=s)
        kv.prefill(ks, vs)
        caches.append(kv)
        prefills.append((ks, vs) if s in (0, 3, 7) else None)
    lm = synth.make_lm_head(cfg).astype(np.float64)
    pos = np.stack([synth.positions(ctx, b)] * S)
    for scale in (1.0, 0.1):
        noise = np.stack([synth.make_noise(cfg, stream=s) for s in range(S)]) * np.float32(scale)
        out = host(dr.forward_round_batch(caches, dev(noise), dev(pos)))
        out2 = host(dr.forward_round_batch(caches, dev(noise), dev(pos)))
        assert np.array_equal(out, out2), "batched sweep not reproducible"
        assert np.all(np.isfinite(out))
        for s in (0, 3, 7):
            okv = O.OracleKV(cfg)
            okv.prefill(*prefills[s])
            ref = O.forward_round(m, okv, noise[s], pos[s])
            tag = f"c4 batched seq {s} emb x{scale:g} ctx {ctx}"
            check(tag, out[s], ref, tol_for(cfg))
            argmax_check(tag, out[s], ref, lm)


def test_c5_fp8_d2conv_layered():
    """The c5 drafter (fp8 weights, DFlash2 conv, ctx 65536) on the layered
    path (one sequence through the batched call), N(0,1) and x0.1 block
    embeddings, against the oracle on the same directly prefilled cache."""
    cfg = synth.ROUND8_FP8_D2
    m, dr, D = _setup(cfg, max_rows=16)
    ctx, b = cfg.ctx, cfg.block
    kv = D.KVCache(cfg, (ctx + b + 63) // 64 * 64)
    ks, vs = synth.make_prefill_kv(cfg, ctx)
    kv.prefill(ks, vs)
    okv = O.OracleKV(cfg)
    okv.prefill(ks, vs)
    del ks, vs
    lm = synth.make_lm_head(cfg).astype(np.float64)
    pos = synth.positions(ctx, b)
    for scale in (1.0, 0.1):
        noise = synth.make_noise(cfg) * np.float32(scale)
        out = host(dr.forward_round_batch([kv], dev(noise[None]), dev(pos[None])))[0]
        ref = O.forward_round(m, okv, noise, pos)
        tag = f"c5 layered emb x{scale:g} ctx {ctx}"
        check(tag, out, ref, tol_for(cfg))
        argmax_check(tag, out, ref, lm)


def test_batched_ingest_matches_oracle():
    """dflash_ingest_ctx_batch: t rows into each of three caches (two
    contiguous, one paged) in one k|v pass; every cache row against the
    oracle's per-sequence ingest, and bitwise equal to one ingest per cache."""
    cfg = SMALL_BF16
    m, dr, D = _setup(cfg, max_rows=128)
    S, t, lens = 3, 21, (0, 40, 77)
    caches = [D.KVCache(cfg, 256), D.PagedKVCache(cfg, 256, page_rows=64, seed=4), D.KVCache(cfg, 256)]
    singles = [D.KVCache(cfg, 256), D.PagedKVCache(cfg, 256, page_rows=64, seed=4), D.KVCache(cfg, 256)]
    okvs = []
    for q, n in enumerate(lens):
        okv = O.OracleKV(cfg)
        if n:
            taps = synth.make_taps(cfg, n, stream=50 + q)
            pos = synth.positions(0, n)
            for c in (caches[q], singles[q]):
                dr.ingest_ctx(c, dr.ctx_features(dev(taps)), dev(pos))
            O.ingest_ctx(m, okv, O.ctx_features(m, taps), pos)
        okvs.append(okv)
    taps = np.stack([synth.make_taps(cfg, t, stream=60 + q) for q in range(S)])
    pos = np.stack([synth.positions(n, t) for n in lens])
    feats = dr.ctx_features(dev(taps.reshape(S * t, -1))).reshape(S, t, cfg.hidden)
    dr.ingest_ctx_batch(caches, feats, dev(pos))
    assert [c.len for c in caches] == [n + t for n in lens]
    for q in range(S):
        dr.ingest_ctx(singles[q], feats[q].contiguous(), dev(pos[q]))
        O.ingest_ctx(m, okvs[q], O.ctx_features(m, taps[q]), pos[q])
        for l in range(cfg.n_layers):
            k, v = kv_rows_f64(caches[q], l, 0, lens[q] + t)
            check(f"batched ingest seq {q} layer {l} K", k, okvs[q].k[l], 1e-2)
            check(f"batched ingest seq {q} layer {l} V", v, okvs[q].v[l], 1e-2)
            k1, v1 = kv_rows_f64(singles[q], l, 0, lens[q] + t)
            assert np.array_equal(k, k1) and np.array_equal(v, v1), "batched and single ingest differ"
