"""GPU parity: libdflash (HIP, gfx950) against the fp64 CPU oracle.

Every call goes through the C ABI via the ctypes binding.  Tolerances
(per-row infinity-norm relative error): 1e-4 for the f32 arm, 2e-2 for bf16
weights with f32 accumulation.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import dflash_oracle as O
from tests.gpu_util import check, dev, host, kv_rows_f64, rel_rows, tol_for

pytestmark = pytest.mark.gpu

# A small bf16 drafter with GQA 8:2, head_dim 64 and ragged ctx sizes.
SMALL_BF16 = synth.DraftConfig(
    name="small_bf16", n_layers=2, hidden=512, n_q_heads=8, n_kv_heads=2, head_dim=64,
    intermediate=768, n_taps=2, weight_dtype="bf16", kv_dtype="bf16", path="round",
    ctx=100, block=16, seed=21)
# head_dim 128 with 8 q heads on one kv head (128 queries per kv head)
SMALL_BF16_D128 = SMALL_BF16.replace(name="small_bf16_d128", hidden=1024, n_q_heads=8, n_kv_heads=1,
                                     head_dim=128, seed=22)
# fp8 e4m3fn weights with per-row f32 scales
SMALL_FP8 = SMALL_BF16.replace(name="small_fp8", weight_dtype="fp8", seed=23)
SMALL_FP8_D128 = SMALL_BF16_D128.replace(name="small_fp8_d128", weight_dtype="fp8", seed=24)
# YaRN rope (factor 32 over an original context of 8192), exercised at positions past 30000
SMALL_YARN = SMALL_BF16_D128.replace(name="small_yarn_d128", rope_type="yarn", seed=25)
# DFlash2 conv wrap around every sublayer: f32 (G = 2), bf16 (G = 4), fp8 head_dim 128 (G = 16)
TINY_F32_D2 = synth.TINY_F32.replace(name="tiny_f32_d2", d2_groups=2, seed=26)
SMALL_D2 = SMALL_BF16.replace(name="small_bf16_d2", d2_groups=4, seed=27)
SMALL_FP8_D2 = SMALL_FP8_D128.replace(name="small_fp8_d128_d2", d2_groups=16, seed=28)
D2_CFGS = [TINY_F32_D2, SMALL_D2, SMALL_FP8_D2]


def _setup(cfg, max_rows=16):
    from block_diffusion_drafter_round_amd import dflash as D
    sw = synth.make_weights(cfg)
    return sw, O.OracleModel(sw), D.Drafter(sw, max_rows=max_rows), D


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    torch.cuda.init()


def test_zero_layers_final_norm():
    cfg = synth.TINY_F32.replace(n_layers=0)
    sw, m, dr, D = _setup(cfg)
    noise = synth.make_noise(cfg)
    kv = D.KVCache(cfg, 64)
    out = host(dr.forward_round(kv, dev(noise), dev(synth.positions(0, 16))))
    ref = O.forward_round(m, O.OracleKV(cfg), noise, synth.positions(0, 16))
    check("L=0 final norm", out, ref, 1e-6)


@pytest.mark.parametrize("cfg", [synth.TINY_F32, SMALL_BF16, SMALL_BF16_D128, SMALL_FP8], ids=lambda c: c.name)
@pytest.mark.parametrize("t", [1, 5, 64])
def test_ctx_features(cfg, t):
    sw, m, dr, D = _setup(cfg, max_rows=t)
    taps = synth.make_taps(cfg, t, stream=t)
    out = host(dr.ctx_features(dev(taps)))
    check(f"{cfg.name} ctx_features t={t}", out, O.ctx_features(m, taps), tol_for(cfg) / 10)


@pytest.mark.parametrize("cfg,t", [(SMALL_BF16_D128, 4100), (SMALL_BF16_D128, 2020), (SMALL_BF16, 4096)],
                         ids=["d128_t4100", "d128_t2020", "bf16_t4096"])
def test_ctx_features_tall(cfg, t):
    """Tall activations with bf16 weights take the tiled GEMM (128 x 128
    tiles).  4100 rows of hidden 1024: 33 x 8 tiles over the whole K, the
    last row tile holding 4 rows.  2020 rows: 16 x 8 tiles, so K is split
    into two halves that meet in Y; the last row tile holds 100 rows, so one
    wave's 16 rows end inside it (4 in, 12 past M) and the waves above lie
    wholly past M.  4096 rows of hidden 512: 32 x 4 tiles, K halves."""
    sw, m, dr, D = _setup(cfg, max_rows=t)
    taps = synth.make_taps(cfg, t, stream=7)
    out = host(dr.ctx_features(dev(taps)))
    check(f"{cfg.name} ctx_features t={t} (tiled)", out, O.ctx_features(m, taps), tol_for(cfg) / 10)


def test_ctx_features_tall_halves_deterministic():
    """The tiled GEMM's two K halves meet in Y in whichever order they finish;
    a sum of two f32 terms does not depend on that order, so repeated calls
    give the same bits (2020 rows of hidden 1024: 16 x 8 tiles, K halves)."""
    cfg, t = SMALL_BF16_D128, 2020
    sw, m, dr, D = _setup(cfg, max_rows=t)
    taps = dev(synth.make_taps(cfg, t, stream=9))
    first = host(dr.ctx_features(taps)).copy()
    for _ in range(4):
        again = host(dr.ctx_features(taps))
        assert np.array_equal(first.view(np.uint64), again.view(np.uint64))


def test_ingest_tall():
    """8208 ctx rows in one ingest call: the k|v projection (two weight
    segments of 128 columns, k and v) runs as the tiled GEMM, 65 x 2 tiles
    with K split into two halves; the last row tile holds 16 rows."""
    cfg = SMALL_BF16_D128
    n = 8208
    sw, m, dr, D = _setup(cfg, max_rows=n)
    taps = synth.make_taps(cfg, n, stream=8)
    pos = synth.positions(2000, n)
    kv = D.KVCache(cfg, 8256)
    dr.ingest_ctx(kv, dr.ctx_features(dev(taps)), dev(pos))
    assert kv.len == n
    okv = O.OracleKV(cfg)
    O.ingest_ctx(m, okv, O.ctx_features(m, taps), pos)
    for l in range(cfg.n_layers):
        k, v = kv_rows_f64(kv, l, 0, n)
        check(f"{cfg.name} layer {l} cached K, {n} rows (tiled)", k, okv.k[l], 1e-2)
        check(f"{cfg.name} layer {l} cached V, {n} rows (tiled)", v, okv.v[l], 1e-2)


@pytest.mark.parametrize("cfg", [synth.TINY_F32, SMALL_BF16, SMALL_BF16_D128, SMALL_FP8, SMALL_YARN],
                         ids=lambda c: c.name)
def test_ingest_cache_rows(cfg):
    """Cache rows after ingesting in uneven chunks: K normed+roped, V raw, at
    the right rows and positions.  len advances by t per call."""
    sw, m, dr, D = _setup(cfg, max_rows=64)
    n = 37
    taps = synth.make_taps(cfg, n)
    pos = synth.positions(31000 if cfg.rope_type == "yarn" else 1000, n)
    kv = D.KVCache(cfg, 128)
    feats = dr.ctx_features(dev(taps))
    for lo, hi in ((0, 1), (1, 17), (17, 37)):
        dr.ingest_ctx(kv, feats[lo:hi].contiguous(), dev(pos[lo:hi]))
        assert kv.len == hi
    okv = O.OracleKV(cfg)
    O.ingest_ctx(m, okv, O.ctx_features(m, taps), pos)
    tol = 1e-5 if cfg.kv_dtype == "f32" else 1e-2
    for l in range(cfg.n_layers):
        k, v = kv_rows_f64(kv, l, 0, n)
        check(f"{cfg.name} layer {l} cached K", k, okv.k[l], tol)
        check(f"{cfg.name} layer {l} cached V", v, okv.v[l], tol)


@pytest.mark.parametrize("n_layers", [5, 10])
def test_ingest_layer_groups(n_layers):
    """ingest_ctx projects several layers' k|v in one launch (up to 8, fewer
    once rows x layers would pass 8192), with a ragged last group when the
    layer count does not divide: every layer's cache rows must still match
    the oracle."""
    cfg = SMALL_BF16.replace(name=f"small_bf16_l{n_layers}", n_layers=n_layers, seed=40 + n_layers)
    sw, m, dr, D = _setup(cfg, max_rows=129)
    sizes = (1, 16, 40, 64, 129)
    n = sum(sizes)
    taps = synth.make_taps(cfg, n)
    pos = synth.positions(500, n)
    kv = D.KVCache(cfg, 256)
    lo = 0
    for t in sizes:
        feats = dr.ctx_features(dev(taps[lo:lo + t]))
        dr.ingest_ctx(kv, feats, dev(pos[lo:lo + t]))
        lo += t
        assert kv.len == lo
    okv = O.OracleKV(cfg)
    O.ingest_ctx(m, okv, O.ctx_features(m, taps), pos)
    for l in range(cfg.n_layers):
        k, v = kv_rows_f64(kv, l, 0, n)
        check(f"{cfg.name} layer {l} cached K", k, okv.k[l], 1e-2)
        check(f"{cfg.name} layer {l} cached V", v, okv.v[l], 1e-2)


@pytest.mark.parametrize("cfg", [synth.TINY_F32, SMALL_BF16, SMALL_BF16_D128, SMALL_FP8, SMALL_FP8_D128] + D2_CFGS,
                         ids=lambda c: c.name)
@pytest.mark.parametrize("b", [16, 5, 1])
def test_forward_full_vs_oracle(cfg, b):
    sw, m, dr, D = _setup(cfg, max_rows=cfg.ctx)
    n = cfg.ctx
    taps = synth.make_taps(cfg, n)
    noise = synth.make_noise(cfg, rows=b)
    pos = synth.positions(0, n + b)
    out = host(dr.forward_full(dev(taps), dev(noise), dev(pos)))
    ref = O.forward_full(m, taps, noise, pos, n)
    check(f"{cfg.name} forward_full n={n} b={b}", out, ref, tol_for(cfg))


@pytest.mark.parametrize("cfg", [synth.TINY_F32, SMALL_BF16, SMALL_FP8, SMALL_D2], ids=lambda c: c.name)
def test_round_equals_full_bitwise(cfg):
    """[DflashDraft] forward_round: bit-class-identical to the fresh forward.
    On the GPU the two run the same kernels, so they must agree bit for bit,
    also when the cache was filled in several chunks of the same total."""
    sw, m, dr, D = _setup(cfg, max_rows=cfg.ctx)
    n, b = cfg.ctx, cfg.block
    taps = synth.make_taps(cfg, n)
    noise = dev(synth.make_noise(cfg))
    pos = dev(synth.positions(0, n + b))
    full = dr.forward_full(dev(taps), noise, pos)
    kv = D.KVCache(cfg, (n + b + 63) // 64 * 64)
    feats = dr.ctx_features(dev(taps))
    dr.ingest_ctx(kv, feats, pos[:n])
    r1 = dr.forward_round(kv, noise, pos[n:])
    r2 = dr.forward_round(kv, noise, pos[n:])
    assert kv.len == n
    torch.cuda.synchronize()
    assert torch.equal(full, r1), "forward_round != forward_full"
    assert torch.equal(r1, r2), "forward_round is not deterministic"


@pytest.mark.parametrize("cfg", [SMALL_BF16, SMALL_FP8_D128, SMALL_YARN, SMALL_FP8_D2], ids=lambda c: c.name)
def test_multi_round_append_then_round(cfg):
    """Several rounds: each ingests 16 committed rows, then drafts; every
    round matches the oracle's cached path."""
    sw, m, dr, D = _setup(cfg, max_rows=64)
    kv = D.KVCache(cfg, 256)
    okv = O.OracleKV(cfg)
    p = 30000 if cfg.rope_type == "yarn" else 0     # YaRN: positions far past the original context
    for rnd, t in enumerate((40, 16, 16, 3)):
        taps = synth.make_taps(cfg, t, stream=100 + rnd)
        pos = synth.positions(p, t)
        dr.ingest_ctx(kv, dr.ctx_features(dev(taps)), dev(pos))
        O.ingest_ctx(m, okv, O.ctx_features(m, taps), pos)
        p += t
        noise = synth.make_noise(cfg, stream=rnd)
        bpos = synth.positions(p, cfg.block)
        out = host(dr.forward_round(kv, dev(noise), dev(bpos)))
        check(f"{cfg.name} round {rnd} len={p}", out, O.forward_round(m, okv, noise, bpos), tol_for(cfg))


@pytest.mark.parametrize("cfg", [synth.TINY_F32, SMALL_BF16, SMALL_FP8_D128, SMALL_D2], ids=lambda c: c.name)
@pytest.mark.parametrize("n,b", [(37, 16), (40, 5), (41, 7)])
def test_round_writes_block_kv_rows(cfg, n, b):
    """[DflashDraft] forward_round: the block's K (normed + roped) and V land
    transiently at cache rows [len, len + b) while len stays.  Layer 0's
    block rows are checked against the oracle's k/v of the block input
    (with the DFlash2 wrap, of its prepared rows).  len = 37 and 41 are not
    multiples of 4 and b = 5, 7 end inside a row quad, so the kernel's
    partial-quad stores are covered next to the whole-quad ones."""
    sw, m, dr, D = _setup(cfg, max_rows=64)
    kv = D.KVCache(cfg, 128)
    taps = synth.make_taps(cfg, n)
    dr.ingest_ctx(kv, dr.ctx_features(dev(taps)), dev(synth.positions(0, n)))
    noise = synth.make_noise(cfg, rows=b)
    bpos = synth.positions(n, b)
    dr.forward_round(kv, dev(noise), dev(bpos))
    assert kv.len == n
    L = m.layers[0]
    xn = O.rms_norm(noise, L["g_in"], m.eps)
    if cfg.d2_groups:
        xn, _ = O.d2_prepare(xn, L["attn.w_dyn"], L["attn.base"], cfg.d2_groups)
    ok, ov = O.ctx_kv(m, 0, xn, bpos)
    k, v = kv_rows_f64(kv, 0, n, n + b)
    tol = 1e-5 if cfg.kv_dtype == "f32" else 1e-2
    check(f"{cfg.name} block K rows len={n} b={b}", k, ok, tol)
    check(f"{cfg.name} block V rows len={n} b={b}", v, ov, tol)


def test_d2_identity_taps_equal_backbone():
    """DFlash2 special case: with zero dynamic projections and static taps
    [0, 1] the wrap is the identity, so the output equals the same weights
    without the wrap (the conv path and the plain path run different code).
    The two agree to rounding only: GEMM inputs are bf16 (8 significant
    bits, 2^-9 relative), and the conv path rounds the normalised rows
    x*g/rms after the conv while the plain path rounds x*g and applies 1/rms
    to the GEMM output, so they round different values.  Over two layers that
    stays within a few times 2^-9; 2e-3 is the bound used."""
    from block_diffusion_drafter_round_amd import dflash as D
    cfg = SMALL_D2
    sw = synth.make_weights(cfg)
    for l in range(cfg.n_layers):
        for sub in ("attn", "mlp"):
            w = sw.layers[l][f"{sub}.w_dyn"]
            w.data[...] = 0
            base = sw.layers[l][f"{sub}.base"]
            base[..., 0] = 0.0
            base[..., 1] = 1.0
    plain = synth.StoredWeights(cfg.replace(d2_groups=0), sw.fc, sw.g_hidden_norm, sw.g_norm, sw.layers)
    n, b = cfg.ctx, cfg.block
    taps, noise, pos = synth.make_taps(cfg, n), synth.make_noise(cfg), synth.positions(0, n + b)
    o_d2 = host(D.Drafter(sw, max_rows=n).forward_full(dev(taps), dev(noise), dev(pos)))
    o_plain = host(D.Drafter(plain, max_rows=n).forward_full(dev(taps), dev(noise), dev(pos)))
    check("d2 identity taps vs plain backbone", o_d2, o_plain, 2e-3)


def test_errors_leave_state_unchanged():
    cfg = SMALL_BF16
    sw, m, dr, D = _setup(cfg, max_rows=64)
    kv = D.KVCache(cfg, 64)
    feats = dr.ctx_features(dev(synth.make_taps(cfg, 60)))
    dr.ingest_ctx(kv, feats, dev(synth.positions(0, 60)))
    assert kv.len == 60
    with pytest.raises(D.DflashError) as ei:
        dr.forward_round(kv, dev(synth.make_noise(cfg)), dev(synth.positions(60, 16)))
    assert ei.value.code == D.DFLASH_E_CAPACITY
    with pytest.raises(D.DflashError) as ei:
        dr.ingest_ctx(kv, feats[:5].contiguous(), dev(synth.positions(60, 5)))
    assert ei.value.code == D.DFLASH_E_CAPACITY
    assert kv.len == 60
    out = dr.forward_round(kv, dev(synth.make_noise(cfg, rows=4)), dev(synth.positions(60, 4)))
    assert torch.isfinite(out).all()


def test_round_reads_the_packed_copy():
    """dflash_pack_weights copies the layer weights: a change to a layer
    matrix reaches forward_round only after the weights are packed again.
    Flipping the sign bits of layer 0's down projection is exact in bf16."""
    import copy
    cfg = SMALL_BF16
    sw, m, dr, D = _setup(cfg, max_rows=cfg.ctx)
    n, b = cfg.ctx, cfg.block
    taps = synth.make_taps(cfg, n)
    noise = synth.make_noise(cfg, rows=b)
    pos = synth.positions(0, n + b)
    run = lambda: host(dr.forward_full(dev(taps), dev(noise), dev(pos)))
    out_a = run()
    check("small_bf16 packed", out_a, O.forward_full(m, taps, noise, pos, n), tol_for(cfg))

    ptr = dr.weights.layer_arr[0].wd.data
    wd = next(t for t in dr.weights.tensors if t is not None and t.data_ptr() == ptr)
    wd.bitwise_xor_(torch.tensor(-32768, dtype=torch.int16, device=wd.device))
    out_b = run()
    assert np.array_equal(out_a, out_b), "the round read the weights in place, not the packed copy"

    D.dflash_pack_weights(dr.model, dr.packed, dr.packed_bytes)
    out_c = run()
    sw2 = copy.deepcopy(sw)
    sw2.layers[0]["wd"].data = sw2.layers[0]["wd"].data ^ np.uint16(0x8000)
    ref_c = O.forward_full(O.OracleModel(sw2), taps, noise, pos, n)
    check("small_bf16 repacked, layer 0 wd negated", out_c, ref_c, tol_for(cfg))
    assert not np.array_equal(out_a, out_c)


@pytest.mark.parametrize("cfg,b", [
    (SMALL_BF16.replace(name="small_bf16_l10", n_layers=10, seed=50), 16),
    (SMALL_BF16.replace(name="small_bf16_l10", n_layers=10, seed=50), 5),
    (SMALL_FP8_D2.replace(name="small_fp8_d128_d2_l11", n_layers=11, seed=51), 7),
    (synth.TINY_F32.replace(name="tiny_f32_l9", n_layers=9, seed=52), 16),
], ids=lambda x: x.name if hasattr(x, "name") else str(x))
def test_forward_full_more_than_8_layers(cfg, b):
    """A round over more than 8 layers runs as several launches, the residual
    carried between them in the workspace and each launch reading its own
    layers' part of the packed weight stream."""
    sw, m, dr, D = _setup(cfg, max_rows=cfg.ctx)
    n = cfg.ctx
    taps = synth.make_taps(cfg, n)
    noise = synth.make_noise(cfg, rows=b)
    pos = synth.positions(0, n + b)
    out = host(dr.forward_full(dev(taps), dev(noise), dev(pos)))
    ref = O.forward_full(m, taps, noise, pos, n)
    check(f"{cfg.name} forward_full n={n} b={b}", out, ref, tol_for(cfg))


@pytest.mark.parametrize("cfg", [synth.TINY_F32, SMALL_BF16, SMALL_FP8_D2], ids=lambda c: c.name)
@pytest.mark.parametrize("b", [16, 3])
def test_empty_context(cfg, b):
    """No ctx rows: forward_round over an empty cache attends to the block's
    own keys only, and forward_full with n = 0 gives the same rows."""
    sw, m, dr, D = _setup(cfg, max_rows=16)
    noise = synth.make_noise(cfg, rows=b)
    pos = synth.positions(7, b)
    kv = D.KVCache(cfg, 64)
    out = host(dr.forward_round(kv, dev(noise), dev(pos)))
    assert kv.len == 0
    ref = O.forward_round(m, O.OracleKV(cfg), noise, pos)
    check(f"{cfg.name} empty-cache round b={b}", out, ref, tol_for(cfg))
    taps = synth.make_taps(cfg, 0)
    full = host(dr.forward_full(dev(taps), dev(noise), dev(pos)))
    assert np.array_equal(out, full), "forward_full(n = 0) != forward_round on an empty cache"
