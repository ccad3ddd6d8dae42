"""Seeded synthetic inputs for the DFlash drafter forward.

This module is the only code that the CPU oracle (``oracle/``) and the HIP
path share.  It holds no step of the drafter's arithmetic.  It only draws
random numbers and encodes them into the stored formats that both sides
consume:

* f32 values as drawn;
* bf16 bit patterns (uint16, round-to-nearest-even from f32);
* fp8 e4m3fn codes (uint8) with one f32 scale per weight row, where
  ``scale = amax(row) / 448`` and the codes are round-to-nearest-even of
  ``w / scale``.

Each side decodes the stored bytes with its own code.

Workloads
---------
The presets follow the drafter shapes on the memra ``dflash`` module page
(5 layers, 6 taps), the atlas ``dflash_head`` page (8 layers, hidden 2048,
GQA 32:4, head_dim 128, 5 taps, 16-token blocks) and the ``DflashDraft``
``rope_yarn`` field (YaRN factor 32, original context 8192, betas 32/1).

Seeds: ``numpy.random.default_rng([cfg.seed, tensor_id])`` with a fixed
tensor-id enumeration (:func:`tensor_id`).  Projection matrices are drawn
``N(0, 0.02)``.  RMSNorm gains are ``1 + N(0, 0.02)``, so a gain applied to the
wrong channel shows up.  DFlash2 base taps are ``[N(0,.02), 1 + N(0,.02)]``.
Tapped target states and noise embeddings are ``N(0, 1)``.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass, field

import numpy as np

try:  # torch is used only for its bf16 / fp8 encoders (round-to-nearest-even)
    import torch
except ImportError:  # pragma: no cover
    torch = None


# --------------------------------------------------------------------------
# configurations
# --------------------------------------------------------------------------

@dataclass(frozen=True)
class DraftConfig:
    name: str
    n_layers: int
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    intermediate: int
    n_taps: int
    weight_dtype: str          # "f32" | "bf16" | "fp8"
    kv_dtype: str              # "f32" | "bf16"
    rms_eps: float = 1e-6
    rope_base: float = 1e6
    rope_type: str = "plain"   # "plain" | "yarn"
    yarn_factor: float = 32.0
    yarn_orig_ctx: int = 8192
    yarn_beta_fast: float = 32.0
    yarn_beta_slow: float = 1.0
    d2_groups: int = 0         # 0: no DFlash2 conv wrap
    # workload
    path: str = "round"        # "full" | "round"
    ctx: int = 0               # committed ctx rows attended by the round
    block: int = 16
    new_rows: int = 16         # ctx rows ingested per round (round path)
    n_seqs: int = 1
    seed: int = 1000
    init_std: float = 0.02
    gain_offset: float = 1.0   # gains are gain_offset + N(0, init_std)

    @property
    def q_dim(self) -> int:
        return self.n_q_heads * self.head_dim

    @property
    def kv_dim(self) -> int:
        return self.n_kv_heads * self.head_dim

    def replace(self, **kw) -> "DraftConfig":
        return dataclasses.replace(self, **kw)


# Tiny f32 drafter, fresh full-context forward.
TINY_F32 = DraftConfig(
    name="tiny_f32_full", n_layers=2, hidden=256, n_q_heads=4, n_kv_heads=1,
    head_dim=64, intermediate=768, n_taps=3, weight_dtype="f32", kv_dtype="f32",
    path="full", ctx=64, block=16, new_rows=64, seed=1001)

# 5-layer drafter (memra shape: 5 layers, 6 taps), full-context forward.
FULL5_BF16 = DraftConfig(
    name="l5_bf16_full_ctx1024", n_layers=5, hidden=2048, n_q_heads=32,
    n_kv_heads=4, head_dim=128, intermediate=6144, n_taps=6, weight_dtype="bf16",
    kv_dtype="bf16", path="full", ctx=1024, block=16, new_rows=1024, seed=1002)

# 8-layer drafter (atlas shape: 8 layers, 5 taps) on the cached round path.
ROUND8_BF16 = DraftConfig(
    name="l8_bf16_round_ctx4096", n_layers=8, hidden=2048, n_q_heads=32,
    n_kv_heads=4, head_dim=128, intermediate=6144, n_taps=5, weight_dtype="bf16",
    kv_dtype="bf16", path="round", ctx=4096, block=16, new_rows=16, seed=1003)

# Same drafter with YaRN rope at ctx 32768, 8 independent sequences.
ROUND8_YARN = ROUND8_BF16.replace(
    name="l8_bf16_yarn_round_ctx32768_x8", rope_type="yarn", ctx=32768,
    n_seqs=8, seed=1004)

# fp8 e4m3fn weights (per-row f32 scales) + DFlash2 conv wrap, ctx 65536.
ROUND8_FP8_D2 = ROUND8_BF16.replace(
    name="l8_fp8_d2conv_round_ctx65536", weight_dtype="fp8", ctx=65536,
    d2_groups=16, seed=1005)

PRESETS = {c.name: c for c in (TINY_F32, FULL5_BF16, ROUND8_BF16, ROUND8_YARN, ROUND8_FP8_D2)}


# --------------------------------------------------------------------------
# seeded draws and encoders
# --------------------------------------------------------------------------

# per-layer tensors, in a fixed order (their ids are 100 + 32*layer + index)
LAYER_MATS = ("wq", "wk", "wv", "wo", "wg", "wu", "wd")
LAYER_GAINS = ("g_in", "g_post", "g_q", "g_k")
D2_SUBLAYERS = ("attn", "mlp")


def tensor_id(name: str, layer: int = -1) -> int:
    """Fixed enumeration of tensor names used to derive per-tensor seeds."""
    globals_ = {"fc": 1, "g_hidden_norm": 2, "g_norm": 3,
                "taps": 10, "noise": 11, "prefill_k": 12, "prefill_v": 13, "lm_head": 14}
    if layer < 0:
        return globals_[name]
    names = LAYER_MATS + LAYER_GAINS + tuple(
        f"{s}.{t}" for s in D2_SUBLAYERS for t in ("w_dyn", "base"))
    return 100 + 32 * layer + names.index(name)


def rng_for(cfg: DraftConfig, tid: int, stream: int = 0) -> np.random.Generator:
    return np.random.default_rng([cfg.seed, tid, stream])


def normal_f32(rng: np.random.Generator, shape, std: float = 1.0, mean: float = 0.0) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    if mean != 0.0:
        x += np.float32(mean)
    return x


def encode_bf16(x: np.ndarray) -> np.ndarray:
    """f32 -> bf16 bit patterns (uint16), round-to-nearest-even (torch's cast)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def encode_fp8_rows(w: np.ndarray):
    """f32 [N, K] -> (e4m3fn codes uint8 [N, K], f32 scale [N]).

    scale[n] = amax(|w[n, :]|) / 448 (1.0 for an all-zero row); codes are the
    round-to-nearest-even e4m3fn encoding of w / scale (torch's cast), clamped
    to the finite range first."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    amax = np.abs(w).max(axis=1)
    scale = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    y = np.clip(w / scale[:, None], -448.0, 448.0).astype(np.float32)
    codes = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return codes, scale


@dataclass
class StoredMatrix:
    """One projection matrix [N, K] (torch Linear layout) as stored."""
    dtype: str                  # "f32" | "bf16" | "fp8"
    data: np.ndarray            # f32 [N,K] | uint16 [N,K] | uint8 [N,K]
    scale: np.ndarray | None = None  # f32 [N] for fp8

    @property
    def shape(self):
        return self.data.shape


def store_matrix(w: np.ndarray, dtype: str) -> StoredMatrix:
    if dtype == "f32":
        return StoredMatrix("f32", np.ascontiguousarray(w, dtype=np.float32))
    if dtype == "bf16":
        return StoredMatrix("bf16", encode_bf16(w))
    if dtype == "fp8":
        codes, scale = encode_fp8_rows(w)
        return StoredMatrix("fp8", codes, scale)
    raise ValueError(f"unknown weight dtype {dtype!r}")


@dataclass
class StoredWeights:
    cfg: DraftConfig
    fc: StoredMatrix
    g_hidden_norm: np.ndarray
    g_norm: np.ndarray
    layers: list = field(default_factory=list)   # list of dicts


def make_weights(cfg: DraftConfig) -> StoredWeights:
    """All drafter weights for ``cfg`` in their stored form."""
    H, T, I = cfg.hidden, cfg.n_taps, cfg.intermediate
    std, g0 = cfg.init_std, cfg.gain_offset
    wd = cfg.weight_dtype

    def mat(name, shape, layer=-1):
        return store_matrix(normal_f32(rng_for(cfg, tensor_id(name, layer)), shape, std), wd)

    def gain(name, n, layer=-1):
        return normal_f32(rng_for(cfg, tensor_id(name, layer)), (n,), std, g0)

    sw = StoredWeights(cfg, mat("fc", (H, T * H)), gain("g_hidden_norm", H), gain("g_norm", H))
    shapes = {"wq": (cfg.q_dim, H), "wk": (cfg.kv_dim, H), "wv": (cfg.kv_dim, H),
              "wo": (H, cfg.q_dim), "wg": (I, H), "wu": (I, H), "wd": (H, I)}
    for l in range(cfg.n_layers):
        d = {k: mat(k, s, l) for k, s in shapes.items()}
        d["g_in"] = gain("g_in", H, l)
        d["g_post"] = gain("g_post", H, l)
        d["g_q"] = gain("g_q", cfg.head_dim, l)
        d["g_k"] = gain("g_k", cfg.head_dim, l)
        if cfg.d2_groups:
            G = cfg.d2_groups
            for s in D2_SUBLAYERS:
                d[f"{s}.w_dyn"] = mat(f"{s}.w_dyn", (2 * G * 2, H), l)
                b = normal_f32(rng_for(cfg, tensor_id(f"{s}.base", l)), (2, H, 2), std)
                b[:, :, 1] += np.float32(1.0)
                d[f"{s}.base"] = b
        sw.layers.append(d)
    return sw


def make_taps(cfg: DraftConfig, rows: int, stream: int = 0) -> np.ndarray:
    """Tapped target hidden states [rows, n_taps*hidden] f32, N(0,1)."""
    return normal_f32(rng_for(cfg, tensor_id("taps"), stream), (rows, cfg.n_taps * cfg.hidden))


def make_noise(cfg: DraftConfig, rows: int | None = None, stream: int = 0) -> np.ndarray:
    """Block input embeddings [block, hidden] f32, N(0,1)."""
    rows = cfg.block if rows is None else rows
    return normal_f32(rng_for(cfg, tensor_id("noise"), stream), (rows, cfg.hidden))


def positions(start: int, count: int) -> np.ndarray:
    return np.arange(start, start + count, dtype=np.int32)


def make_prefill_kv(cfg: DraftConfig, rows: int, stream: int = 0):
    """Directly prefilled draft-KV contents for long-context workloads.

    Returns (K, V), each [n_layers, n_kv_heads, rows, head_dim] in the KV
    storage format (f32, or bf16 bit patterns as uint16), drawn N(0, 1): the
    cached keys are RMS-normalised per head, so unit-variance entries have the
    same scale."""
    shape = (cfg.n_layers, cfg.n_kv_heads, rows, cfg.head_dim)
    k = normal_f32(rng_for(cfg, tensor_id("prefill_k"), stream), shape)
    v = normal_f32(rng_for(cfg, tensor_id("prefill_v"), stream), shape)
    if cfg.kv_dtype == "bf16":
        return encode_bf16(k), encode_bf16(v)
    return k, v


def make_lm_head(cfg: DraftConfig, vocab: int = 151936) -> np.ndarray:
    """A seeded stand-in for the target's lm_head, [vocab, hidden] f32 N(0, 0.02)."""
    return normal_f32(rng_for(cfg, tensor_id("lm_head")), (vocab, cfg.hidden), 0.02)
