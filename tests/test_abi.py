"""CPU tests of the C ABI: the library loads, exports every function that
include/*.h declares, validates configs and weights without touching the GPU,
and its host-side rope / YaRN tables agree with the oracle's (written
independently, in numpy)."""
import ctypes as C
import os
import re

import numpy as np
import pytest

import synth
from oracle import dflash_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def D():
    from block_diffusion_drafter_round_amd import dflash
    if not os.path.exists(dflash.LIB_PATH):
        from block_diffusion_drafter_round_amd.build import build
        build()
    dflash.lib()
    return dflash


def declared_functions():
    names = []
    for h in ("dflash.h", "dflash_prof.h", "dflash_policy.h"):
        src = open(os.path.join(ROOT, "include", h)).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        names += re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(dflash2?_[a-z_0-9]+)\s*\(", src, flags=re.M)
    return sorted(set(names))


def test_every_declared_function_is_exported(D):
    names = declared_functions()
    assert "dflash_forward_round" in names and "dflash_ingest_ctx" in names and "dflash_prof_start" in names
    L = C.CDLL(D.LIB_PATH)
    missing = [n for n in names if not hasattr(L, n)]
    assert not missing, missing
    assert set(D.EXPORTS) <= set(names)


class FakeWeights:
    """A dflash_weights struct whose pointers are distinct aligned integers:
    load_weights only validates and stores them, it never dereferences."""

    def __init__(self, D, cfg, misalign=None, null=None):
        addr = [0x100000]

        def ptr(name):
            addr[0] += 0x1000
            if name == null:
                return None
            return addr[0] + (4 if name == misalign else 0)

        def mat(name):
            return D.dflash_matrix(ptr(name), ptr(name + ".scale") if cfg.weight_dtype == "fp8" else None)

        self.layers = (D.dflash_layer_weights * max(1, cfg.n_layers))()
        for l in range(cfg.n_layers):
            lw = self.layers[l]
            for n in ("wq", "wk", "wv", "wo", "wg", "wu", "wd"):
                setattr(lw, n, mat(f"{n}"))
            for n in ("g_in", "g_post", "g_q", "g_k"):
                setattr(lw, n, ptr(n))
            if cfg.d2_groups:
                lw.attn_w_dyn, lw.mlp_w_dyn = mat("attn_w_dyn"), mat("mlp_w_dyn")
                lw.attn_base, lw.mlp_base = ptr("attn_base"), ptr("mlp_base")
        self.struct = D.dflash_weights(fc=mat("fc"), g_hidden_norm=ptr("g_hidden_norm"), g_norm=ptr("g_norm"),
                                       layers=self.layers)


@pytest.mark.parametrize("cfg", [synth.TINY_F32, synth.FULL5_BF16, synth.ROUND8_BF16, synth.ROUND8_YARN,
                                 synth.ROUND8_FP8_D2], ids=lambda c: c.name)
def test_load_weights_and_rope_tables_match_oracle(D, cfg):
    fw = FakeWeights(D, cfg)
    m = D.dflash_load_weights(D.make_cfg(cfg), fw.struct)
    try:
        inv, ms = D.dflash_rope_table(m, cfg.head_dim // 2)
        inv_o, _, ms_o = O.rope_tables(cfg)
        assert np.allclose(inv, inv_o, rtol=1e-14, atol=0)
        assert ms == pytest.approx(ms_o, rel=1e-15)
        assert D.dflash_workspace_bytes(m, 16) > 0
        assert D.dflash_workspace_bytes(m, 4096) > D.dflash_workspace_bytes(m, 16)
        assert D.dflash_workspace_bytes(m, -1) == 0
    finally:
        D.dflash_free(m)


@pytest.mark.parametrize("change,code", [
    (dict(hidden=300), 3), (dict(head_dim=96), 3), (dict(n_q_heads=6, n_kv_heads=4), 1),
    (dict(n_q_heads=64, n_kv_heads=2), 3), (dict(rms_eps=0.0), 1), (dict(rope_base=1.0), 1),
    (dict(weight_dtype="fp8", kv_dtype="f32"), 3), (dict(weight_dtype="f32", kv_dtype="bf16"), 3),
    (dict(n_layers=-1), 1), (dict(d2_groups=-1), 1), (dict(d2_groups=3), 3), (dict(d2_groups=128), 3),
    (dict(d2_groups=512), 3),
])
def test_bad_configs_rejected(D, change, code):
    cfg = synth.ROUND8_BF16.replace(**change)
    fw = FakeWeights(D, synth.ROUND8_BF16.replace(n_layers=max(0, cfg.n_layers)))
    with pytest.raises(D.DflashError) as ei:
        D.dflash_load_weights(D.make_cfg(cfg), fw.struct)
    assert ei.value.code == code
    assert D.dflash_last_error()


@pytest.mark.parametrize("misalign,null", [("wq", None), (None, "g_k"), (None, "fc"), ("g_norm", None)])
def test_bad_weight_pointers_rejected(D, misalign, null):
    cfg = synth.TINY_F32
    fw = FakeWeights(D, cfg, misalign=misalign, null=null)
    with pytest.raises(D.DflashError) as ei:
        D.dflash_load_weights(D.make_cfg(cfg), fw.struct)
    assert ei.value.code == D.DFLASH_E_INVAL


@pytest.mark.parametrize("null", ["attn_base", "mlp_w_dyn"])
def test_d2_weights_required(D, null):
    cfg = synth.ROUND8_FP8_D2
    fw = FakeWeights(D, cfg, null=null)
    with pytest.raises(D.DflashError) as ei:
        D.dflash_load_weights(D.make_cfg(cfg), fw.struct)
    assert ei.value.code == D.DFLASH_E_INVAL


def test_fp8_needs_scales(D):
    cfg = synth.ROUND8_BF16.replace(weight_dtype="fp8")
    fw = FakeWeights(D, cfg, null="wo.scale")
    with pytest.raises(D.DflashError) as ei:
        D.dflash_load_weights(D.make_cfg(cfg), fw.struct)
    assert ei.value.code == D.DFLASH_E_INVAL


def test_round_needs_packed_weights(D):
    """forward_round and pack_weights reject their arguments before any HIP call."""
    cfg = synth.TINY_F32
    fw = FakeWeights(D, cfg)
    m = D.dflash_load_weights(D.make_cfg(cfg), fw.struct)
    try:
        with pytest.raises(D.DflashError) as ei:
            D.dflash_pack_weights(m, None, 1 << 20, 0)
        assert ei.value.code == D.DFLASH_E_INVAL
        with pytest.raises(D.DflashError) as ei:
            D.dflash_pack_weights(m, 0x10010, 1 << 20, 0)        # not 256-byte aligned
        assert ei.value.code == D.DFLASH_E_INVAL
        kv = D.dflash_kv(0x100000, 0x200000, 128, 0)
        ws_bytes = D.dflash_workspace_bytes(m, 16)
        rc = D.lib().dflash_forward_round(m, C.byref(kv), 0x300000, 0x400000, 16, 0x500000, 0x600000, ws_bytes, None)
        assert rc == D.DFLASH_E_INVAL
        assert "not packed" in D.dflash_last_error()
        assert kv.len == 0
    finally:
        D.dflash_free(m)


def test_packed_bytes_needs_a_device(D):
    """The packed layout depends on the device's CU count: with no usable
    device the size query reports an error instead of a size."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a device is present")
    cfg = synth.TINY_F32
    fw = FakeWeights(D, cfg)
    m = D.dflash_load_weights(D.make_cfg(cfg), fw.struct)
    try:
        with pytest.raises(D.DflashError) as ei:
            D.dflash_packed_bytes(m)
        assert ei.value.code == D.DFLASH_E_HIP
    finally:
        D.dflash_free(m)
