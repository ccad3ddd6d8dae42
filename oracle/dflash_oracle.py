"""Plain fp64 CPU oracle of the DFlash block-diffusion drafter forward.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  The product path
(the HIP library and its Python binding) never does, and this module imports
nothing from it.  Everything is plain numpy in float64, with no blocking or
fusion beyond what each definition states.  It is meant to be checked by eye
against the pages:

* [memra dflash module] docs.rs, memra_engine::dflash (module index);
* [DflashDraft] docs.rs, memra_engine::dflash::DflashDraft (struct page);
* [atlas dflash_head] spark_model::layers::dflash_head (module page).

Stored inputs are decoded exactly: f32 as is, bf16 by widening the bit
pattern, fp8 e4m3fn by its format definition times the row's f32 scale.
Intermediates are never rounded to a storage type: the oracle keeps the exact
fp64 value of what the method computes.  The one exception is a directly
prefilled KV cache, which *is* the given stored data.

Readings of the pages that the oracle fixes, where the pages leave a step open:

* R-1: the ctx features go straight into the per-layer k/v projections, with
  no per-layer norm in between.  [DflashDraft, ``ingest_ctx``] lists
  "k/v projections + k head-norm + rope" and nothing else.
* R-2: a block row's q, k and v all come from the same normed block row
  (Qwen3 decoder layer).
* R-3: no mask: every block query attends every attended ctx key and every
  block key.  [DflashDraft, ``ctx_features``/``forward``] says "full
  non-causal attention"; [atlas dflash_head, overview] says "bidirectional
  in-block attention".  No window unless a round is given one
  ([atlas dflash_head, ``dflash_ctx_cap``]): then only the most recent
  ctx_cap committed rows are attended; first light has none.
* R-4: the softmax scale is 1/sqrt(head_dim).  The YaRN mscale multiplies q
  and k after rope ([DflashDraft, ``rope_yarn``]).
* R-5: q/k head RMSNorm (gain [head_dim], same eps) comes before rope
  ([memra dflash module, ``DflashKv``]: cached K is "normed+roped").
* R-6: rope rotates pairs (j, j + d/2) over the full head_dim (NeoX halves,
  ``rope_neox_ff``), with angles p * inv_freq[j] in exact fp64.
* R-7/R-8: the RMSNorm gain is plain g * x / rms.  The block layer is a
  pre-norm residual Qwen3 layer: attention, then a SwiGLU MLP.
* R-9: no biases anywhere.
* R-10: the taps are concatenated in input order along the feature axis.
* R-11: q head hq reads kv head floor(hq * n_kv / n_q).
* R-20: for the DFlash2 conv, tap 0 multiplies row r-1 and tap 1 multiplies
  row r.  The dyn projection is laid out [half][group][tap].  Channel c is in
  group floor(c * G / H).  The conv input is the post-norm row ``xn``.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "decode_bf16", "decode_e4m3fn", "decode_matrix", "rope_tables", "rms_norm",
    "apply_rope", "OracleModel", "OracleKV", "ctx_features", "ctx_kv",
    "ingest_ctx", "attention", "block_layer", "forward_round", "forward_round_batch", "forward_full",
    "d2_prepare", "d2_finish", "lm_argmax",
]


# --------------------------------------------------------------------------
# decoding the stored inputs
# --------------------------------------------------------------------------

def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64.  A bf16 value is the top half of
    the f32 with the same bits, so widening is exact."""
    u32 = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u32.view(np.float32).astype(np.float64)


def _e4m3fn_value(code: int) -> float:
    """OCP FP8 e4m3fn: 1 sign, 4 exponent (bias 7), 3 mantissa bits; no
    infinities; S.1111.111 is NaN; max finite 448; subnormals m * 2^-9."""
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return s * m * 2.0 ** -9
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


_E4M3FN_TABLE = np.array([_e4m3fn_value(c) for c in range(256)], dtype=np.float64)


def decode_e4m3fn(codes: np.ndarray) -> np.ndarray:
    """fp8 e4m3fn codes (uint8) -> float64 ([atlas dflash_head,
    ``DflashQuantization``]: weight-only FP8 with per-row scales)."""
    return _E4M3FN_TABLE[np.asarray(codes, dtype=np.uint8)]


def decode_matrix(sm) -> np.ndarray:
    """A stored projection matrix [N, K] -> float64 W[N, K].

    For fp8, W[n, k] = scale[n] * e4m3fn(q[n, k]) (one f32 scale per output
    row)."""
    if sm.dtype == "f32":
        return np.asarray(sm.data, dtype=np.float64)
    if sm.dtype == "bf16":
        return decode_bf16(sm.data)
    if sm.dtype == "fp8":
        return decode_e4m3fn(sm.data) * np.asarray(sm.scale, dtype=np.float64)[:, None]
    raise ValueError(sm.dtype)


def decode_kv(data: np.ndarray, kv_dtype: str) -> np.ndarray:
    return decode_bf16(data) if kv_dtype == "bf16" else np.asarray(data, dtype=np.float64)


# --------------------------------------------------------------------------
# O1-O3: rope tables, RMSNorm, rope
# --------------------------------------------------------------------------

def rope_tables(cfg):
    """Per-dimension rope inverse frequencies and the q/k scale (O1).

    [DflashDraft, ``rope_yarn``]: the effective inverse frequency is
    inv_freq[j] = base^(-2j/d) / ff[j].  For plain rope ff = 1 and the scale
    is 1.  For YaRN, ff is the YaRN frequency remap and the scale is
    0.1 * ln(factor) + 1, applied to q and k after rope.

    YaRN remap, as published by Peng et al., "YaRN: Efficient Context Window
    Extension of Large Language Models" (2023):
    * A dimension pair that turns r times over the original context L0 sits
      at index dim(r) = d * ln(L0 / (2 pi r)) / (2 ln base).
    * Pairs below lo = floor(dim(beta_fast)) keep their frequency.  Pairs at
      or above hi = ceil(dim(beta_slow)) are divided by the factor.  Pairs
      in between blend linearly:
      ramp = clamp((j - lo) / (hi - lo), 0, 1),
      ff = 1 / (ramp / factor + 1 - ramp).
    * lo is clamped to >= 0 and hi to <= d - 1.  If lo == hi, hi is nudged by
      0.001 so the ramp stays defined.
    """
    d = cfg.head_dim
    base = float(cfg.rope_base)
    j = np.arange(d // 2, dtype=np.float64)
    plain = base ** (-2.0 * j / d)
    if cfg.rope_type == "plain":
        return plain, np.ones(d // 2), 1.0
    if cfg.rope_type != "yarn":
        raise ValueError(cfg.rope_type)
    factor = float(cfg.yarn_factor)
    L0 = float(cfg.yarn_orig_ctx)

    def dim_of(r):
        return d * math.log(L0 / (2.0 * math.pi * r)) / (2.0 * math.log(base))

    lo = max(math.floor(dim_of(cfg.yarn_beta_fast)), 0)
    hi = min(math.ceil(dim_of(cfg.yarn_beta_slow)), d - 1)
    if hi == lo:
        hi = lo + 0.001
    ramp = np.clip((j - lo) / (hi - lo), 0.0, 1.0)
    ff = 1.0 / (ramp / factor + 1.0 - ramp)
    mscale = 0.1 * math.log(factor) + 1.0
    return plain / ff, ff, mscale


def rms_norm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm over the last axis (O2): g * x / sqrt(mean(x^2) + eps)."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return np.asarray(g, dtype=np.float64) * x / np.sqrt(ms + eps)


def apply_rope(x: np.ndarray, pos: np.ndarray, inv_freq: np.ndarray, mscale: float) -> np.ndarray:
    """NeoX rotate-half rope, then the q/k scale (O3).

    x: [rows, heads, d]; pos: [rows] absolute positions.  With half = d/2 and
    theta = pos * inv_freq[j] (fp64):
      x'[j]        = x[j] cos(theta) - x[j+half] sin(theta)
      x'[j + half] = x[j+half] cos(theta) + x[j] sin(theta)
    ([DflashDraft, ``rope_yarn``]: ``rope_neox_ff``, mscale applied post-rope.)
    """
    half = x.shape[-1] // 2
    theta = np.asarray(pos, dtype=np.float64)[:, None] * inv_freq[None, :]   # [rows, half]
    c = np.cos(theta)[:, None, :]
    s = np.sin(theta)[:, None, :]
    a, b = x[..., :half], x[..., half:]
    return mscale * np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def silu(z: np.ndarray) -> np.ndarray:
    return z / (1.0 + np.exp(-z))


# --------------------------------------------------------------------------
# the model
# --------------------------------------------------------------------------

class OracleModel:
    """The drafter's weights decoded to float64.

    [DflashDraft, struct fields]: ``fc``, ``hidden_norm``, ``norm``,
    ``layers``, ``rope_yarn``, ``dflash2``.  [atlas dflash_head,
    ``DflashLayer``]: per-layer Qwen3-style weights."""

    def __init__(self, stored):
        cfg = stored.cfg
        self.cfg = cfg
        self.eps = float(cfg.rms_eps)
        self.fc = decode_matrix(stored.fc)
        self.g_hidden_norm = np.asarray(stored.g_hidden_norm, dtype=np.float64)
        self.g_norm = np.asarray(stored.g_norm, dtype=np.float64)
        self.layers = []
        for ls in stored.layers:
            L = {}
            for k, v in ls.items():
                if k.endswith("base") or k.startswith("g_"):
                    L[k] = np.asarray(v, dtype=np.float64)
                else:
                    L[k] = decode_matrix(v)
            self.layers.append(L)
        self.inv_freq, self.ff, self.mscale = rope_tables(cfg)


def ctx_features(m: OracleModel, taps: np.ndarray) -> np.ndarray:
    """Context features (O4): hidden_norm(fc(taps)).

    [DflashDraft, ``ctx_features``]: ctx features for t tapped rows are
    hidden_norm(fc(taps)).  The taps are the raw tapped states
    [t, n_taps * hidden], concatenated in tap order.  [atlas dflash_head,
    overview]: one fc at model entry."""
    taps = np.asarray(taps, dtype=np.float64)
    return rms_norm(taps @ m.fc.T, m.g_hidden_norm, m.eps)


def _heads(x: np.ndarray, n_heads: int, d: int) -> np.ndarray:
    return x.reshape(x.shape[0], n_heads, d)


def ctx_kv(m: OracleModel, layer: int, feats: np.ndarray, pos: np.ndarray):
    """One layer's ctx K and V for rows of ctx features (O5).

    [DflashDraft, ``ingest_ctx``]: per-layer k/v projections, k head-norm,
    rope.  [memra dflash module, ``DflashKv``]: K is normed+roped, V is raw.
    Returns K, V, each [t, n_kv, d]."""
    cfg, L = m.cfg, m.layers[layer]
    d = cfg.head_dim
    k = _heads(feats @ L["wk"].T, cfg.n_kv_heads, d)
    v = _heads(feats @ L["wv"].T, cfg.n_kv_heads, d)
    k = apply_rope(rms_norm(k, L["g_k"], m.eps), pos, m.inv_freq, m.mscale)
    return k, v


class OracleKV:
    """Append-only draft KV cache ([memra dflash module, ``DflashKv``]).

    Per layer, the ctx K (normed+roped) and raw ctx V rows in committed order,
    each kept as [rows, n_kv, d] float64, plus ``len``."""

    def __init__(self, cfg):
        self.cfg = cfg
        self.k = [np.zeros((0, cfg.n_kv_heads, cfg.head_dim)) for _ in range(cfg.n_layers)]
        self.v = [np.zeros((0, cfg.n_kv_heads, cfg.head_dim)) for _ in range(cfg.n_layers)]

    @property
    def len(self) -> int:
        return self.k[0].shape[0]

    def append(self, layer: int, k: np.ndarray, v: np.ndarray) -> None:
        self.k[layer] = np.concatenate([self.k[layer], k], axis=0)
        self.v[layer] = np.concatenate([self.v[layer], v], axis=0)

    def prefill(self, k_stored: np.ndarray, v_stored: np.ndarray) -> None:
        """Fill directly from stored data [n_layers, n_kv, rows, d].  These
        rows are the given (already normed+roped) cache contents."""
        kd = decode_kv(k_stored, self.cfg.kv_dtype)
        vd = decode_kv(v_stored, self.cfg.kv_dtype)
        for l in range(self.cfg.n_layers):
            self.append(l, kd[l].transpose(1, 0, 2), vd[l].transpose(1, 0, 2))

    def truncate(self, rows: int) -> None:
        for l in range(self.cfg.n_layers):
            self.k[l] = self.k[l][:rows]
            self.v[l] = self.v[l][:rows]


def ingest_ctx(m: OracleModel, kv: OracleKV, feats: np.ndarray, pos_new: np.ndarray) -> None:
    """Ingest t new ctx-feature rows at ``kv.len`` (O5, O8).

    [DflashDraft, ``ingest_ctx``]: the rows come in committed order at
    absolute positions ``pos_new``.  Per layer: k/v projections, k head-norm,
    rope, appended at kv.len."""
    feats = np.asarray(feats, dtype=np.float64)
    for l in range(m.cfg.n_layers):
        k, v = ctx_kv(m, l, feats, pos_new)
        kv.append(l, k, v)


def attention(q: np.ndarray, K: np.ndarray, V: np.ndarray) -> np.ndarray:
    """Non-causal grouped-query attention (O6; readings R-3, R-4, R-11).

    q: [b, nq, d]; K, V: [n, nkv, d].  Every query attends all n keys:
      s[r, hq, j] = q[r, hq] . K[j, h] / sqrt(d),  h = floor(hq * nkv / nq)
      O[r, hq]    = sum_j softmax_j(s[r, hq, :])[j] * V[j, h]
    """
    b, nq, d = q.shape
    nkv = K.shape[1]
    out = np.empty((b, nq, d))
    for hq in range(nq):
        h = (hq * nkv) // nq
        s = (q[:, hq, :] @ K[:, h, :].T) / math.sqrt(d)          # [b, n]
        s = s - s.max(axis=1, keepdims=True)
        a = np.exp(s)
        a /= a.sum(axis=1, keepdims=True)
        out[:, hq, :] = a @ V[:, h, :]
    return out


def d2_prepare(xn: np.ndarray, w_dyn: np.ndarray, base: np.ndarray, G: int):
    """DFlash2 conv prepare (O9).

    [memra dflash module, ``Dflash2Conv``; DflashDraft, ``d2_conv_prepare``]:
    * One projection of the pre-conv rows gives both dynamic kernels:
      D = xn . w_dyn^T, read as [rows, half, group, tap].
    * The rows then go through a causal 2-tap depthwise conv over the block
      rows.  Row 0's missing predecessor is zero.
    * The coefficients are base[0][c, tap] + D[r, 0, g(c), tap], with
      g(c) = floor(c * G / H).
    * Tap 0 multiplies row r-1 and tap 1 multiplies row r.
    Returns (convolved rows, D)."""
    rows, H = xn.shape
    D = (xn @ w_dyn.T).reshape(rows, 2, G, 2)
    return _d2_conv(xn, D[:, 0], base[0], G), D


def d2_finish(y: np.ndarray, D: np.ndarray, base: np.ndarray, G: int) -> np.ndarray:
    """DFlash2 conv finish (O9): the same causal 2-tap conv of the sublayer
    OUTPUT rows with base[1] + dyn half 1 of the matching prepare's projection
    ([DflashDraft, ``d2_conv_finish``])."""
    return _d2_conv(y, D[:, 1], base[1], G)


def _d2_conv(x: np.ndarray, Dh: np.ndarray, base_h: np.ndarray, G: int) -> np.ndarray:
    rows, H = x.shape
    grp = (np.arange(H) * G) // H                       # channel -> group
    prev = np.zeros_like(x)
    prev[1:] = x[:-1]
    c0 = base_h[None, :, 0] + Dh[:, grp, 0]             # [rows, H], tap on row r-1
    c1 = base_h[None, :, 1] + Dh[:, grp, 1]             # tap on row r
    return c0 * prev + c1 * x


def block_layer(m: OracleModel, layer: int, X: np.ndarray, pos_block: np.ndarray,
                ctx_K: np.ndarray, ctx_V: np.ndarray) -> np.ndarray:
    """One drafter layer over the b block rows (O6, O9).

    * ctx_K, ctx_V: this layer's ctx keys and values [n, nkv, d], already
      normed+roped / raw.
    * The block rows add their own keys at the end: the block K/V sit at
      rows [n, n + b).
    * Attention sees all n + b keys ([DflashDraft, ``forward_round``]).
    * With a DFlash2 head, each sublayer is wrapped in prepare/finish convs
      ([DflashDraft, ``dflash2`` field]: "around EVERY sublayer").
    """
    cfg, L = m.cfg, m.layers[layer]
    d, nq, nkv, G = cfg.head_dim, cfg.n_q_heads, cfg.n_kv_heads, cfg.d2_groups

    # attention sublayer
    xn = rms_norm(X, L["g_in"], m.eps)
    if G:
        xn, D = d2_prepare(xn, L["attn.w_dyn"], L["attn.base"], G)
    q = apply_rope(rms_norm(_heads(xn @ L["wq"].T, nq, d), L["g_q"], m.eps),
                   pos_block, m.inv_freq, m.mscale)
    k = apply_rope(rms_norm(_heads(xn @ L["wk"].T, nkv, d), L["g_k"], m.eps),
                   pos_block, m.inv_freq, m.mscale)
    v = _heads(xn @ L["wv"].T, nkv, d)
    K = np.concatenate([ctx_K, k], axis=0)
    V = np.concatenate([ctx_V, v], axis=0)
    o = attention(q, K, V).reshape(X.shape[0], nq * d)
    y = o @ L["wo"].T
    if G:
        y = d2_finish(y, D, L["attn.base"], G)
    X = X + y

    # MLP sublayer (SwiGLU)
    xn2 = rms_norm(X, L["g_post"], m.eps)
    if G:
        xn2, D2 = d2_prepare(xn2, L["mlp.w_dyn"], L["mlp.base"], G)
    z = silu(xn2 @ L["wg"].T) * (xn2 @ L["wu"].T)
    y = z @ L["wd"].T
    if G:
        y = d2_finish(y, D2, L["mlp.base"], G)
    return X + y


def forward_round(m: OracleModel, kv: OracleKV, noise_emb: np.ndarray, pos_block: np.ndarray,
                  ctx_cap: int = 0) -> np.ndarray:
    """Block forward over the cached ctx K/V (O8, O7).

    [DflashDraft, ``forward_round``]: only the block rows are projected per
    layer.  The block K/V land transiently after the cache's ``len`` rows and
    are never committed, so ``kv`` is left unchanged.  Returns the final
    normed hidden states [b, hidden] for all b rows.

    ctx_cap > 0 is the context window of [atlas dflash_head,
    ``dflash_ctx_cap``]: the block attends only the most recent ctx_cap
    committed rows, [max(0, len - ctx_cap), len), plus its own rows."""
    lo = max(0, kv.len - ctx_cap) if ctx_cap > 0 else 0
    X = np.asarray(noise_emb, dtype=np.float64)
    for l in range(m.cfg.n_layers):
        X = block_layer(m, l, X, pos_block, kv.k[l][lo:], kv.v[l][lo:])
    return rms_norm(X, m.g_norm, m.eps)


def forward_round_batch(m: OracleModel, kvs, noise_emb, pos_block) -> np.ndarray:
    """Several sequences' rounds ([atlas dflash_head, ``DflashProposerState``]:
    per-sequence drafter state): each sequence's round on its own cache, one
    after another.  noise_emb [S, b, hidden], pos_block [S, b]; returns
    [S, b, hidden]."""
    return np.stack([forward_round(m, kv, noise_emb[s], pos_block[s]) for s, kv in enumerate(kvs)])


def forward_full(m: OracleModel, taps: np.ndarray, noise_emb: np.ndarray,
                 pos: np.ndarray, n: int) -> np.ndarray:
    """First-light forward (O4-O7), written without any cache.

    [DflashDraft, ``forward``]: full non-causal attention over
    [ctx_features ; block], with no draft KV cache and no window.
    * taps: [n, n_taps*hidden]; noise_emb: [b, hidden].
    * pos: the n ctx positions, then the b block positions.
    * Per layer, every ctx row's K/V is recomputed from the features, in
      one pass.
    """
    pos = np.asarray(pos)
    feats = ctx_features(m, taps)
    X = np.asarray(noise_emb, dtype=np.float64)
    for l in range(m.cfg.n_layers):
        ck, cv = ctx_kv(m, l, feats, pos[:n])
        X = block_layer(m, l, X, pos[n:], ck, cv)
    return rms_norm(X, m.g_norm, m.eps)


# --------------------------------------------------------------------------
# O11: argmax over a seeded lm_head (test-only check of the hidden states)
# --------------------------------------------------------------------------

def lm_argmax(hidden: np.ndarray, lm_head: np.ndarray):
    """Logits = hidden . lm_head^T in float64, then the argmax of each row.
    Ties go to the lowest index ([memra dflash module, ``dflash2_walk_greedy``]:
    the torch argmax convention).  Returns (argmax [rows], logits)."""
    logits = np.asarray(hidden, dtype=np.float64) @ np.asarray(lm_head, dtype=np.float64).T
    return np.argmax(logits, axis=1), logits
