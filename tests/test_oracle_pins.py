"""Pins of the CPU oracle to things other than itself.

Each test ties one part of ``oracle/dflash_oracle.py`` to one of:
* a closed form;
* a library routine (transformers' Qwen3 decoder layer and YaRN init, torch's
  fp8 decoder and rms_norm);
* brute force on tiny inputs;
* an invariant the pages state (cached round == fresh forward, non-causal
  equivariance, relative rope).

Mistakes these catch: a dropped term, a wrong sign or index, a transposed
operand, a causal mask, a mis-paired rope, a wrong GQA head map.
"""
import math

import numpy as np
import pytest
import torch

import synth
from oracle import dflash_oracle as O

# A small drafter that still has GQA (4 q heads on 2 kv heads), several layers
# and ctx rows.
SMALL = synth.DraftConfig(
    name="small", n_layers=2, hidden=64, n_q_heads=4, n_kv_heads=2, head_dim=16,
    intermediate=96, n_taps=3, weight_dtype="f32", kv_dtype="f32", path="full",
    ctx=12, block=5, seed=7, init_std=0.2, gain_offset=1.0)


def small_model(cfg=SMALL):
    return O.OracleModel(synth.make_weights(cfg))


def rel(a, b):
    return np.abs(a - b).max() / max(np.abs(b).max(), 1e-300)


# ---------------------------------------------------------------- P1 -------
@pytest.mark.parametrize("cfg", [SMALL, SMALL.replace(rope_type="yarn", yarn_orig_ctx=64, seed=8),
                                 SMALL.replace(d2_groups=4, seed=9)])
def test_p1_cached_round_equals_fresh_forward(cfg):
    """[DflashDraft, forward_round]: the cached round is "bit-class-identical"
    to the block forward over freshly computed ctx features.  Uneven ingest
    chunks (5 + 1 + 6 rows) exercise the append order and ``len``."""
    m = small_model(cfg)
    n, b = cfg.ctx, cfg.block
    taps = synth.make_taps(cfg, n)
    noise = synth.make_noise(cfg)
    pos = synth.positions(3, n + b)
    fresh = O.forward_full(m, taps, noise, pos, n)
    kv = O.OracleKV(cfg)
    for lo, hi in ((0, 5), (5, 6), (6, n)):
        O.ingest_ctx(m, kv, O.ctx_features(m, taps[lo:hi]), pos[lo:hi])
    assert kv.len == n
    cached = O.forward_round(m, kv, noise, pos[n:])
    assert kv.len == n
    assert rel(cached, fresh) <= 1e-12


# ---------------------------------------------------------------- P2 -------
def test_p2_noncausal_equivariance():
    """[DflashDraft, forward]: full non-causal attention.  Permuting the block
    rows together with their positions permutes the outputs.  A causal mask,
    or positions tied to row order, breaks this."""
    m = small_model()
    n, b = SMALL.ctx, SMALL.block
    taps = synth.make_taps(SMALL, n)
    noise = synth.make_noise(SMALL)
    pos = synth.positions(0, n + b)
    out = O.forward_full(m, taps, noise, pos, n)
    perm = np.array([3, 0, 4, 1, 2])
    pos_p = np.concatenate([pos[:n], pos[n:][perm]])
    out_p = O.forward_full(m, taps, noise[perm], pos_p, n)
    assert rel(out_p, out[perm]) <= 1e-12
    # ... and a swap of two rows' positions alone does change the outputs.
    pos_s = pos.copy()
    pos_s[n], pos_s[n + 1] = pos[n + 1], pos[n]
    assert rel(O.forward_full(m, taps, noise, pos_s, n), out) > 1e-6


# ---------------------------------------------------------------- P3 -------
@pytest.mark.parametrize("rope_type", ["plain", "yarn"])
def test_p3_position_shift_invariance(rope_type):
    """Rope makes q.k depend only on position differences.  Shifting every
    position by the same amount leaves the output unchanged.  A rope that is
    not a rotation, or q and k rotated by different rules, breaks this."""
    cfg = SMALL.replace(rope_type=rope_type, yarn_orig_ctx=64)
    m = small_model(cfg)
    n = cfg.ctx
    taps = synth.make_taps(cfg, n)
    noise = synth.make_noise(cfg)
    pos = synth.positions(0, n + cfg.block)
    a = O.forward_full(m, taps, noise, pos, n)
    b = O.forward_full(m, taps, noise, pos + 1000, n)
    assert rel(b, a) <= 1e-10


# ---------------------------------------------------------------- P4 -------
def _brute_attention(q, K, V):
    """Naive attention with exact sums (math.fsum) over explicit loops."""
    b, nq, d = q.shape
    n, nkv, _ = K.shape
    out = np.zeros((b, nq, d))
    for r in range(b):
        for hq in range(nq):
            h = hq // (nq // nkv)
            s = [math.fsum(q[r, hq, i] * K[j, h, i] for i in range(d)) / math.sqrt(d) for j in range(n)]
            mx = max(s)
            e = [math.exp(x - mx) for x in s]
            z = math.fsum(e)
            for i in range(d):
                out[r, hq, i] = math.fsum(e[j] * V[j, h, i] for j in range(n)) / z
    return out


@pytest.mark.parametrize("n,b,nq,nkv", [(1, 1, 2, 1), (5, 3, 2, 1), (4, 2, 4, 2), (3, 3, 6, 3)])
def test_p4_attention_brute_force(n, b, nq, nkv):
    rng = np.random.default_rng(n * 100 + b)
    d = 4
    q = rng.standard_normal((b, nq, d))
    K = rng.standard_normal((n, nkv, d))
    V = rng.standard_normal((n, nkv, d))
    assert rel(O.attention(q, K, V), _brute_attention(q, K, V)) <= 1e-13


def test_p4_attention_special_cases():
    rng = np.random.default_rng(5)
    d, n = 8, 6
    K = rng.standard_normal((n, 1, d))
    V = rng.standard_normal((n, 1, d))
    # q = 0: uniform weights, the mean of V
    out = O.attention(np.zeros((1, 2, d)), K, V)
    assert np.allclose(out[0, 0], V[:, 0].mean(axis=0), atol=1e-14, rtol=0)
    # a single key: exactly its value
    out = O.attention(rng.standard_normal((2, 1, d)), K[:1], V[:1])
    assert np.allclose(out[:, 0], V[0, 0], atol=1e-14, rtol=0)
    # one dominant logit picks that key's value
    q = (K[2, 0] * 1e3)[None, None, :]
    K2 = K.copy()
    K2[:, 0] *= 1e-3
    K2[2, 0] = K[2, 0]
    out = O.attention(q, K2, V)
    assert np.allclose(out[0, 0], V[2, 0], atol=1e-9, rtol=0)


# ---------------------------------------------------------------- P5 -------
def test_p5_plain_rope_closed_form():
    cfg = synth.ROUND8_BF16
    inv, ff, ms = O.rope_tables(cfg)
    j = np.arange(64)
    assert np.array_equal(ff, np.ones(64)) and ms == 1.0
    assert np.allclose(inv, 1e6 ** (-(2 * j) / 128), rtol=1e-15, atol=0)
    assert inv[0] == 1.0


def test_p5_yarn_table_values_and_library():
    """[DflashDraft, rope_yarn]: factor 32, original 8192, beta 32/1, ff =
    the HF-yarn remap (the pages report agreement to 1.6e-7), and mscale =
    0.1 ln(factor) + 1.  Checked against the closed-form values and against
    transformers' own yarn init (f32)."""
    cfg = synth.ROUND8_YARN
    inv, ff, ms = O.rope_tables(cfg)
    assert np.array_equal(ff[:18], np.ones(18))
    assert ff[18] == pytest.approx(1.0 / ((1 / 17) / 32 + 16 / 17), rel=1e-15)
    assert ff[33] == pytest.approx(1.0 / ((16 / 17) / 32 + 1 / 17), rel=1e-15)
    assert ff[33] == pytest.approx(11.333333333333, rel=1e-12)
    assert np.array_equal(ff[34:], np.full(30, 32.0))
    assert ms == pytest.approx(0.1 * math.log(32) + 1, rel=1e-16)
    assert ms == pytest.approx(1.3465735902799727, rel=1e-16)

    from transformers import Qwen3Config
    from transformers.modeling_rope_utils import ROPE_INIT_FUNCTIONS
    hc = Qwen3Config(hidden_size=2048, num_attention_heads=32, num_key_value_heads=4, head_dim=128,
                     max_position_embeddings=262144,
                     rope_parameters={"rope_type": "yarn", "rope_theta": 1e6, "factor": 32.0,
                                      "original_max_position_embeddings": 8192,
                                      "beta_fast": 32.0, "beta_slow": 1.0})
    hf_inv, hf_att = ROPE_INIT_FUNCTIONS["yarn"](hc, "cpu")
    assert np.abs(hf_inv.double().numpy() / inv - 1).max() < 1e-6
    assert hf_att == pytest.approx(ms, rel=1e-12)


def test_p5_rope_is_rotation_and_matches_direct_angles():
    rng = np.random.default_rng(3)
    cfg = SMALL.replace(rope_type="yarn", yarn_orig_ctx=64)
    inv, ff, ms = O.rope_tables(cfg)
    x = rng.standard_normal((7, 3, 16))
    pos = np.array([0, 1, 2, 100, 5000, 65551, 123456])
    y = O.apply_rope(x, pos, inv, ms)
    # norm preserved (up to the q/k scale)
    assert np.allclose(np.linalg.norm(y, axis=-1), ms * np.linalg.norm(x, axis=-1), rtol=1e-13)
    # position 0 is the identity (times ms)
    assert np.allclose(y[0], ms * x[0], rtol=0, atol=1e-15)
    # one pair checked as a complex rotation: (a + ib) e^{i theta}
    r, h, jj = 4, 1, 5
    z = complex(x[r, h, jj], x[r, h, jj + 8]) * complex(math.cos(pos[r] * inv[jj]), math.sin(pos[r] * inv[jj]))
    assert y[r, h, jj] == pytest.approx(ms * z.real, rel=1e-13)
    assert y[r, h, jj + 8] == pytest.approx(ms * z.imag, rel=1e-13)


# ---------------------------------------------------------------- P6 -------
def _hf_layer(cfg, L):
    from transformers import Qwen3Config
    from transformers.models.qwen3.modeling_qwen3 import Qwen3DecoderLayer
    hc = Qwen3Config(hidden_size=cfg.hidden, num_attention_heads=cfg.n_q_heads,
                     num_key_value_heads=cfg.n_kv_heads, head_dim=cfg.head_dim,
                     intermediate_size=cfg.intermediate, rms_norm_eps=cfg.rms_eps,
                     attention_bias=False, hidden_act="silu")
    hc._attn_implementation = "eager"
    layer = Qwen3DecoderLayer(hc, layer_idx=0).double().eval()
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))
    with torch.no_grad():
        sa, mlp = layer.self_attn, layer.mlp
        sa.q_proj.weight.copy_(t(L["wq"])); sa.k_proj.weight.copy_(t(L["wk"]))
        sa.v_proj.weight.copy_(t(L["wv"])); sa.o_proj.weight.copy_(t(L["wo"]))
        sa.q_norm.weight.copy_(t(L["g_q"])); sa.k_norm.weight.copy_(t(L["g_k"]))
        mlp.gate_proj.weight.copy_(t(L["wg"])); mlp.up_proj.weight.copy_(t(L["wu"]))
        mlp.down_proj.weight.copy_(t(L["wd"]))
        layer.input_layernorm.weight.copy_(t(L["g_in"]))
        layer.post_attention_layernorm.weight.copy_(t(L["g_post"]))
    return layer


@pytest.mark.parametrize("rope_type", ["plain", "yarn"])
def test_p6_no_ctx_equals_library_qwen3_layers(rope_type):
    """With no ctx rows, the drafter's block layers are Qwen3 decoder layers
    with full (unmasked) attention.  Compared against transformers'
    Qwen3DecoderLayer in float64, eager attention, attention_mask=None.  The
    cos/sin come from the oracle's inv_freq, with the YaRN scale folded into
    both, as transformers does.  This pins head norm before rope, the NeoX
    pairing, the GQA map, SwiGLU, the residuals and the 1/sqrt(d) scale.  The
    library's eager softmax runs in float32, hence the 1e-6 tolerance."""
    cfg = SMALL.replace(rope_type=rope_type, yarn_orig_ctx=64)
    m = small_model(cfg)
    noise = synth.make_noise(cfg)
    pos = synth.positions(40, cfg.block)
    ours = O.forward_round(m, O.OracleKV(cfg), noise, pos)

    X = torch.from_numpy(noise.astype(np.float64))[None]
    theta = torch.from_numpy(pos.astype(np.float64)[:, None] * m.inv_freq[None, :])
    emb = torch.cat([theta, theta], dim=-1)[None]
    cos, sin = emb.cos() * m.mscale, emb.sin() * m.mscale
    with torch.no_grad():
        for l in range(cfg.n_layers):
            X = _hf_layer(cfg, m.layers[l])(X, attention_mask=None, position_embeddings=(cos, sin))
            X = X[0] if isinstance(X, tuple) else X
        ref = torch.nn.functional.rms_norm(X, (cfg.hidden,), torch.from_numpy(m.g_norm), cfg.rms_eps)
    assert rel(ours, ref[0].numpy()) <= 1e-6


def test_p6_ctx_rows_are_keys_from_features():
    """A ctx row with feature f at position p gives the same K/V as a block
    row whose normed input is f: one layer sees the same keys either way.
    * Model A: n ctx rows with f = rms_norm(x; g_in), plus the block X.
    * Model B: no ctx, and a block of the n + b rows [x; X].
    One layer of A must equal B's last b rows.  With P6 above, this pins the
    ctx path: fc output -> k/v projections with no per-layer input norm,
    then the same head norm and rope as block rows."""
    cfg = SMALL.replace(n_layers=1)
    m = small_model(cfg)
    n, b = cfg.ctx, cfg.block
    rng = np.random.default_rng(11)
    x = rng.standard_normal((n, cfg.hidden))
    feats = O.rms_norm(x, m.layers[0]["g_in"], m.eps)
    noise = synth.make_noise(cfg)
    pos = synth.positions(0, n + b)[::-1].copy()
    kv = O.OracleKV(cfg)
    O.ingest_ctx(m, kv, feats, pos[:n])
    a = O.forward_round(m, kv, noise, pos[n:])
    bb = O.forward_round(m, O.OracleKV(cfg), np.concatenate([x, noise]), pos)
    assert rel(a, bb[n:]) <= 1e-12


def test_p6_ctx_features_fc_then_norm():
    """ctx features = hidden_norm(fc(concat taps)) against a closed form.

    With fc = [0 | I | 0] (it selects tap 1 of the concatenation), fc(taps)
    is tap 1 itself, so the features must be g_hn * tap1 / rms(tap1).  The
    hidden_norm gain is 2 + N(0, 0.02) per channel and the final-norm gain
    is set to 3, so using the wrong gain or the wrong tap changes every
    value; the features' RMS must be ~2 (the gain), not ~3 or ~1."""
    cfg = SMALL
    m = small_model(cfg)
    H, T = cfg.hidden, cfg.n_taps
    m.fc = np.zeros((H, T * H))
    m.fc[:, H:2 * H] = np.eye(H)
    m.g_hidden_norm = 2.0 + 0.02 * np.random.default_rng(3).standard_normal(H)
    m.g_norm = np.full(H, 3.0)
    taps = synth.make_taps(cfg, 9).astype(np.float64)
    tap1 = taps[:, H:2 * H]
    expect = np.empty_like(tap1)
    for r in range(tap1.shape[0]):                       # written out per row and channel
        rms = math.sqrt(sum(v * v for v in tap1[r]) / H + cfg.rms_eps)
        for c in range(H):
            expect[r, c] = m.g_hidden_norm[c] * tap1[r, c] / rms
    got = O.ctx_features(m, taps)
    assert rel(got, expect) <= 1e-13
    assert np.allclose(np.sqrt(np.mean(got ** 2, axis=1)), 2.0, atol=0.02)


# ---------------------------------------------------------------- P7 -------
def test_p7_zero_layers_and_zero_output_projections():
    cfg0 = SMALL.replace(n_layers=0)
    m0 = small_model(cfg0)
    noise = synth.make_noise(cfg0)
    out = O.forward_round(m0, O.OracleKV(cfg0), noise, synth.positions(0, cfg0.block))
    ref = torch.nn.functional.rms_norm(torch.from_numpy(noise.astype(np.float64)), (cfg0.hidden,),
                                       torch.from_numpy(m0.g_norm), cfg0.rms_eps).numpy()
    assert rel(out, ref) <= 1e-14
    # W_o = W_d = 0: every layer leaves the residual stream unchanged
    m = small_model()
    for L in m.layers:
        L["wo"][:] = 0
        L["wd"][:] = 0
    m_ref = O.OracleModel(synth.make_weights(SMALL.replace(n_layers=0)))
    m_ref.g_norm = m.g_norm
    out = O.forward_full(m, synth.make_taps(SMALL, SMALL.ctx), noise, synth.positions(0, SMALL.ctx + 5), SMALL.ctx)
    out_ref = O.forward_round(m_ref, O.OracleKV(cfg0), noise, synth.positions(0, 5))
    assert rel(out, out_ref) <= 1e-14


# ---------------------------------------------------------------- P8 -------
def test_p8_fp8_decode_all_codes_vs_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = O.decode_e4m3fn(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9 and ours[0x08] == 2.0 ** -6


def test_p8_fp8_weight_decode_and_quantiser():
    """W = scale[n] * e4m3fn(q[n,k]).  The stored rows hit +-448 at their
    amax, and the decoded weights lie within half an e4m3 step (relative
    2^-4) of the drawn values."""
    rng = np.random.default_rng(0)
    w = (rng.standard_normal((32, 64)) * 0.02).astype(np.float32)
    sm = synth.store_matrix(w, "fp8")
    W = O.decode_matrix(sm)
    assert np.all(np.abs(O.decode_e4m3fn(sm.data)).max(axis=1) == 448.0)
    big = np.abs(w) > np.abs(w).max(axis=1, keepdims=True) * 2.0 ** -6
    assert np.all(np.abs(W - w)[big] <= np.abs(w)[big] * 2.0 ** -4 + 1e-12)
    # bf16 decode is exact widening
    bits = synth.encode_bf16(w)
    assert np.array_equal(O.decode_bf16(bits), torch.from_numpy(w).to(torch.bfloat16).double().numpy())


# ---------------------------------------------------------------- P9 -------
def _brute_conv(x, Dh, base_h, G):
    rows, H = x.shape
    out = np.zeros_like(x)
    for r in range(rows):
        for c in range(H):
            g = c * G // H
            prev = x[r - 1, c] if r > 0 else 0.0
            out[r, c] = (base_h[c, 0] + Dh[r, g, 0]) * prev + (base_h[c, 1] + Dh[r, g, 1]) * x[r, c]
    return out


def test_p9_d2_conv_brute_force():
    rng = np.random.default_rng(2)
    rows, H, G = 3, 4, 2
    xn = rng.standard_normal((rows, H))
    w_dyn = rng.standard_normal((2 * G * 2, H))
    base = rng.standard_normal((2, H, 2))
    xc, D = O.d2_prepare(xn, w_dyn, base, G)
    Dref = np.array([[math.fsum(xn[r, k] * w_dyn[o, k] for k in range(H)) for o in range(8)] for r in range(rows)])
    assert np.allclose(D.reshape(rows, 8), Dref, rtol=1e-14, atol=1e-15)
    assert np.allclose(xc, _brute_conv(xn, Dref.reshape(rows, 2, G, 2)[:, 0], base[0], G), rtol=1e-14, atol=1e-15)
    y = rng.standard_normal((rows, H))
    assert np.allclose(O.d2_finish(y, D, base, G), _brute_conv(y, Dref.reshape(rows, 2, G, 2)[:, 1], base[1], G),
                       rtol=1e-14, atol=1e-15)


def test_p9_d2_identity_and_shift():
    """With the dynamic projection zero: base taps [0, 1] make both convs the
    identity, so the wrapped model equals the plain backbone exactly.  Base
    taps [1, 0] shift rows down by one, and row 0 becomes zero."""
    cfg = SMALL.replace(d2_groups=4)
    sw = synth.make_weights(cfg)
    m = O.OracleModel(sw)
    for L in m.layers:
        for s in ("attn", "mlp"):
            L[f"{s}.w_dyn"][:] = 0
            L[f"{s}.base"][:] = [0.0, 1.0]
    m_plain = O.OracleModel(synth.make_weights(SMALL.replace(d2_groups=4)))
    m_plain.cfg = SMALL
    n = cfg.ctx
    taps, noise, pos = synth.make_taps(cfg, n), synth.make_noise(cfg), synth.positions(0, n + cfg.block)
    assert rel(O.forward_full(m, taps, noise, pos, n), O.forward_full(m_plain, taps, noise, pos, n)) <= 1e-14
    x = np.random.default_rng(1).standard_normal((4, 8))
    shifted, _ = O.d2_prepare(x, np.zeros((8, 8)), np.tile([1.0, 0.0], (2, 8, 1)), 2)
    assert np.array_equal(shifted[0], np.zeros(8)) and np.array_equal(shifted[1:], x[:-1])


# ---------------------------------------------------------------- P10 ------
def test_p10_rmsnorm():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((5, 33)) * 3
    y = O.rms_norm(x, np.ones(33), 1e-6)
    assert np.allclose(np.sqrt((y * y).mean(axis=1)), 1.0, atol=1e-6)
    g = rng.standard_normal(33)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (33,), torch.from_numpy(g), 1e-6).numpy()
    assert rel(O.rms_norm(x, g, 1e-6), ref) <= 1e-14


# ---------------------------------------------------------------- P11 ------
def test_p11_argmax_ties_lowest_index():
    h = np.array([[1.0, 0.0], [0.0, 1.0]])
    lm = np.array([[0.5, 0.5], [1.0, 0.0], [1.0, 0.0], [0.0, 1.0]])
    am, logits = O.lm_argmax(h, lm)
    assert list(am) == [1, 3]
    assert logits.shape == (2, 4)


# ---------------------------------------------------------- context window --
@pytest.mark.parametrize("cap", [1, 5, 7])
def test_window_equals_round_over_the_last_rows(cap):
    """[atlas dflash_head, dflash_ctx_cap]: a window of N rows gives the same
    result as a plain round over a cache that holds only the last N
    committed rows (built separately, at their own positions)."""
    cfg = SMALL
    m = small_model(cfg)
    n, b = cfg.ctx, cfg.block
    taps, noise, pos = synth.make_taps(cfg, n), synth.make_noise(cfg), synth.positions(0, n + b)
    feats = O.ctx_features(m, taps)
    full = O.OracleKV(cfg)
    O.ingest_ctx(m, full, feats, pos[:n])
    last = O.OracleKV(cfg)
    O.ingest_ctx(m, last, feats[n - cap:], pos[n - cap:n])
    win = O.forward_round(m, full, noise, pos[n:], ctx_cap=cap)
    assert rel(win, O.forward_round(m, last, noise, pos[n:])) <= 1e-13
    # a window that covers everything changes nothing; a smaller one does
    assert rel(O.forward_round(m, full, noise, pos[n:], ctx_cap=n), O.forward_round(m, full, noise, pos[n:])) == 0
    assert rel(win, O.forward_round(m, full, noise, pos[n:])) > 1e-6


def test_window_attention_brute_force():
    """Windowed attention of one query over explicit loops (tiny shapes)."""
    rng = np.random.default_rng(4)
    d, nq, nkv, n, b, cap = 4, 2, 1, 6, 2, 3
    q = rng.standard_normal((b, nq, d))
    K = rng.standard_normal((n + b, nkv, d))
    V = rng.standard_normal((n + b, nkv, d))
    keys = list(range(n - cap, n + b))               # the last cap ctx rows, then the block
    got = O.attention(q, K[keys], V[keys])
    for r in range(b):
        for hq in range(nq):
            s = [sum(q[r, hq, i] * K[j, 0, i] for i in range(d)) / math.sqrt(d) for j in keys]
            w = [math.exp(x - max(s)) for x in s]
            ref = [sum(w[t] * V[j, 0, i] for t, j in enumerate(keys)) / sum(w) for i in range(d)]
            assert np.allclose(got[r, hq], ref, atol=1e-13)


def test_batch_is_independent_rounds():
    """The batched round is each sequence's own round: permuting the
    sequences permutes the outputs, and sequence 0 does not depend on the
    others' caches."""
    cfg = SMALL
    m = small_model(cfg)
    b = cfg.block
    kvs = []
    for sidx, n in enumerate((3, 12, 7)):
        kv = O.OracleKV(cfg)
        O.ingest_ctx(m, kv, O.ctx_features(m, synth.make_taps(cfg, n, stream=sidx)), synth.positions(0, n))
        kvs.append(kv)
    noise = np.stack([synth.make_noise(cfg, stream=s) for s in range(3)])
    pos = np.stack([synth.positions(n, b) for n in (3, 12, 7)])
    out = O.forward_round_batch(m, kvs, noise, pos)
    perm = [2, 0, 1]
    out_p = O.forward_round_batch(m, [kvs[i] for i in perm], noise[perm], pos[perm])
    assert np.array_equal(out_p, out[perm])
    assert np.array_equal(O.forward_round_batch(m, kvs[:1], noise[:1], pos[:1])[0], out[0])
