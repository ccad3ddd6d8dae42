"""ctypes binding of libdflash (include/dflash.h).

The functions keep the C names and only marshal arguments: torch tensors
become device pointers, and the current torch stream becomes the hipStream_t.
Every step of the drafter runs in libdflash's HIP kernels.  If the library is
missing, loading fails with an error; there is no fallback path.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdflash.so")

DFLASH_OK, DFLASH_E_INVAL, DFLASH_E_CAPACITY, DFLASH_E_UNSUPPORTED, DFLASH_E_HIP = range(5)
DFLASH_F32, DFLASH_BF16, DFLASH_FP8_E4M3 = 0, 1, 2
DFLASH_ROPE_PLAIN, DFLASH_ROPE_YARN = 0, 1
DTYPE_CODES = {"f32": DFLASH_F32, "bf16": DFLASH_BF16, "fp8": DFLASH_FP8_E4M3}
ROPE_CODES = {"plain": DFLASH_ROPE_PLAIN, "yarn": DFLASH_ROPE_YARN}


class DflashError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"dflash error {code}: {msg}")
        self.code = code


class dflash_cfg(C.Structure):
    _fields_ = [("n_layers", C.c_int32), ("hidden", C.c_int32), ("n_q_heads", C.c_int32),
                ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32), ("intermediate", C.c_int32),
                ("n_taps", C.c_int32), ("rms_eps", C.c_float), ("rope_base", C.c_double),
                ("rope_type", C.c_int32), ("yarn_factor", C.c_double), ("yarn_orig_ctx", C.c_int32),
                ("yarn_beta_fast", C.c_double), ("yarn_beta_slow", C.c_double),
                ("weight_dtype", C.c_int32), ("kv_dtype", C.c_int32), ("d2_groups", C.c_int32)]


class dflash_matrix(C.Structure):
    _fields_ = [("data", C.c_void_p), ("scale", C.c_void_p)]


class dflash_layer_weights(C.Structure):
    _fields_ = [(n, dflash_matrix) for n in ("wq", "wk", "wv", "wo", "wg", "wu", "wd")] + \
               [(n, C.c_void_p) for n in ("g_in", "g_post", "g_q", "g_k")] + \
               [("attn_w_dyn", dflash_matrix), ("attn_base", C.c_void_p),
                ("mlp_w_dyn", dflash_matrix), ("mlp_base", C.c_void_p)]


class dflash_weights(C.Structure):
    _fields_ = [("fc", dflash_matrix), ("g_hidden_norm", C.c_void_p), ("g_norm", C.c_void_p),
                ("layers", C.POINTER(dflash_layer_weights))]


class dflash2_selector(C.Structure):
    _fields_ = [("vocab", C.c_int32), ("rank", C.c_int32), ("top_k", C.c_int32),
                ("pred_codebook", C.c_void_p), ("succ_codebook", C.c_void_p), ("w_hidden_proj", C.c_void_p)]


class dflash_kv(C.Structure):
    _fields_ = [("k", C.c_void_p), ("v", C.c_void_p), ("capacity", C.c_int32), ("len", C.c_int32),
                ("page_rows", C.c_int32), ("pool_pages", C.c_int32), ("block_table", C.c_void_p),
                ("ctx_cap", C.c_int32)]


_lib = None
EXPORTS = ("dflash_load_weights", "dflash_free", "dflash_workspace_bytes", "dflash_ctx_features",
           "dflash_ingest_ctx", "dflash_forward_round", "dflash_forward_full", "dflash_last_error",
           "dflash_rope_table", "dflash_prof_start", "dflash_prof_stop", "dflash_workspace_status",
           "dflash_prof_trace", "dflash_prof_trace_read", "dflash_packed_bytes", "dflash_pack_weights",
           "dflash_ctx_features_noalloc", "dflash_accept_prefix", "dflash_rejection_accept_len",
           "dflash_confidence_vt", "dflash_slot_confidence_vt", "dflash2_walk_greedy", "dflash2_walk_sampled",
           "dflash2_propose_prepare", "dflash2_propose_greedy", "dflash_batch_workspace_bytes",
           "dflash_forward_round_batch", "dflash_ingest_ctx_batch")

# kernel classes of the measurement hook (include/dflash_prof.h)
K_GEMM_FC, K_GEMM_KV, K_GEMM_QKV, K_GEMM_O, K_GEMM_GATEUP, K_GEMM_DOWN, K_ATTN, K_ROPE, K_NORM, K_ROUND = range(1, 11)


def lib():
    """Load libdflash.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
    L = C.CDLL(LIB_PATH)
    vp, i32, sz = C.c_void_p, C.c_int32, C.c_size_t
    L.dflash_load_weights.argtypes = [C.POINTER(dflash_cfg), C.POINTER(dflash_weights), C.POINTER(vp)]
    L.dflash_free.argtypes = [vp]
    L.dflash_free.restype = None
    L.dflash_workspace_bytes.argtypes = [vp, i32]
    L.dflash_workspace_bytes.restype = sz
    L.dflash_packed_bytes.argtypes = [vp]
    L.dflash_batch_workspace_bytes.argtypes = [vp, i32, i32]
    L.dflash_batch_workspace_bytes.restype = sz
    L.dflash_forward_round_batch.argtypes = [vp, C.POINTER(dflash_kv), i32, vp, vp, i32, vp, vp, sz, vp]
    L.dflash_ingest_ctx_batch.argtypes = [vp, C.POINTER(dflash_kv), i32, vp, vp, i32, vp, sz, vp]
    L.dflash_packed_bytes.restype = sz
    L.dflash_pack_weights.argtypes = [vp, vp, sz, vp]
    L.dflash_ctx_features.argtypes = [vp, vp, i32, vp, vp, sz, vp]
    L.dflash_ctx_features_noalloc.argtypes = [vp, vp, i32, vp, vp]
    L.dflash_ingest_ctx.argtypes = [vp, C.POINTER(dflash_kv), vp, vp, i32, vp, sz, vp]
    L.dflash_forward_round.argtypes = [vp, C.POINTER(dflash_kv), vp, vp, i32, vp, vp, sz, vp]
    L.dflash_forward_full.argtypes = [vp, vp, vp, vp, i32, i32, vp, C.POINTER(dflash_kv), vp, sz, vp]
    L.dflash_last_error.restype = C.c_char_p
    L.dflash_rope_table.argtypes = [vp, C.POINTER(C.c_double), i32, C.POINTER(C.c_double)]
    L.dflash_prof_start.argtypes = [i32, i32]
    L.dflash_prof_stop.argtypes = [C.POINTER(C.c_double), C.POINTER(i32)]
    L.dflash_workspace_status.argtypes = [vp, vp, sz, vp]
    L.dflash_prof_trace.argtypes = [i32]
    pi32, pf32, pf64 = C.POINTER(i32), C.POINTER(C.c_float), C.POINTER(C.c_double)
    L.dflash_accept_prefix.argtypes = [pi32, i32, pi32, i32, pi32]
    L.dflash_rejection_accept_len.argtypes = [pf64, pf64, pf64, i32, pi32]
    L.dflash_confidence_vt.argtypes = [pf32, i32, C.c_double, i32, pi32]
    L.dflash_slot_confidence_vt.argtypes = [pf32, i32, C.c_double, i32, pi32]
    L.dflash2_walk_greedy.argtypes = [C.POINTER(dflash2_selector), pf32, pi32, pf32, i32, i32, pi32]
    L.dflash2_walk_sampled.argtypes = [C.POINTER(dflash2_selector), pf32, pi32, pf32, i32, i32, C.c_double, pf64,
                                       pi32, pf64, pf64]
    L.dflash2_propose_prepare.argtypes = [vp, C.POINTER(dflash2_selector), vp, vp, i32, vp, vp, sz, vp]
    L.dflash2_propose_greedy.argtypes = [vp, C.POINTER(dflash2_selector), vp, vp, i32, i32, pi32, vp, sz, vp]
    L.dflash_prof_trace_read.argtypes = [vp, vp, sz, C.POINTER(C.c_uint64), i32, vp]
    for name in EXPORTS:
        if name not in ("dflash_free", "dflash_workspace_bytes", "dflash_last_error", "dflash_packed_bytes",
                        "dflash_batch_workspace_bytes"):
            getattr(L, name).restype = C.c_int
    _lib = L
    return L


def _check(rc: int):
    if rc != DFLASH_OK:
        raise DflashError(rc, lib().dflash_last_error().decode())


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


# --------------------------------------------------------------------------
# C calls, same names
# --------------------------------------------------------------------------

def dflash_load_weights(cfg: dflash_cfg, weights: dflash_weights) -> int:
    h = C.c_void_p()
    _check(lib().dflash_load_weights(C.byref(cfg), C.byref(weights), C.byref(h)))
    return h.value


def dflash_free(model: int) -> None:
    lib().dflash_free(model)


def dflash_packed_bytes(model: int) -> int:
    n = int(lib().dflash_packed_bytes(model))
    if n == 0 and lib().dflash_last_error():
        raise DflashError(DFLASH_E_HIP, lib().dflash_last_error().decode())
    return n


def dflash_pack_weights(model: int, dst, nbytes: int, stream=None) -> None:
    _check(lib().dflash_pack_weights(model, _ptr(dst), nbytes, _stream(stream)))


def dflash_workspace_bytes(model: int, max_rows: int) -> int:
    return int(lib().dflash_workspace_bytes(model, max_rows))


def dflash_ctx_features(model, taps, t, feats, ws, ws_bytes, stream=None) -> None:
    _check(lib().dflash_ctx_features(model, _ptr(taps), t, _ptr(feats), _ptr(ws), ws_bytes, _stream(stream)))


def dflash_ctx_features_noalloc(model, taps, t, feats, stream=None) -> None:
    _check(lib().dflash_ctx_features_noalloc(model, _ptr(taps), t, _ptr(feats), _stream(stream)))


def dflash_ingest_ctx(model, kv: dflash_kv, feats, pos_new, t, ws, ws_bytes, stream=None) -> None:
    _check(lib().dflash_ingest_ctx(model, C.byref(kv), _ptr(feats), _ptr(pos_new), t, _ptr(ws), ws_bytes,
                                   _stream(stream)))


def dflash_forward_round(model, kv: dflash_kv, noise_emb, pos_block, b, out, ws, ws_bytes, stream=None) -> None:
    _check(lib().dflash_forward_round(model, C.byref(kv), _ptr(noise_emb), _ptr(pos_block), b, _ptr(out),
                                      _ptr(ws), ws_bytes, _stream(stream)))


def dflash_batch_workspace_bytes(model: int, n_seqs: int, max_rows: int = 0) -> int:
    return int(lib().dflash_batch_workspace_bytes(model, n_seqs, max_rows))


def dflash_forward_round_batch(model, kvs, noise_emb, pos_block, b, out, ws, ws_bytes, stream=None) -> None:
    """kvs: a ctypes array of dflash_kv (see kv_array)."""
    _check(lib().dflash_forward_round_batch(model, kvs, len(kvs), _ptr(noise_emb), _ptr(pos_block), b, _ptr(out),
                                            _ptr(ws), ws_bytes, _stream(stream)))


def dflash_ingest_ctx_batch(model, kvs, feats, pos_new, t, ws, ws_bytes, stream=None) -> None:
    """kvs: a ctypes array of dflash_kv (see kv_array); their lens advance by t."""
    _check(lib().dflash_ingest_ctx_batch(model, kvs, len(kvs), _ptr(feats), _ptr(pos_new), t, _ptr(ws), ws_bytes,
                                         _stream(stream)))


def kv_array(caches):
    """A ctypes array of the caches' dflash_kv structs (copies; write the
    lens back with sync_lens if a call changes them)."""
    arr = (dflash_kv * len(caches))()
    for i, c in enumerate(caches):
        arr[i] = c.c
    return arr


def dflash_forward_full(model, taps, noise_emb, pos, n, b, out, scratch: dflash_kv, ws, ws_bytes,
                        stream=None) -> None:
    _check(lib().dflash_forward_full(model, _ptr(taps), _ptr(noise_emb), _ptr(pos), n, b, _ptr(out),
                                     C.byref(scratch), _ptr(ws), ws_bytes, _stream(stream)))


# ---- host policy functions (include/dflash_policy.h) ------------------------

def _arr(ctype, values):
    values = list(values)
    return (ctype * max(len(values), 1))(*values), len(values)


def _policy_check(rc: int, name: str):
    if rc != DFLASH_OK:
        raise DflashError(rc, f"{name}: invalid argument")


def dflash_accept_prefix(cand, vam) -> int:
    c, nc = _arr(C.c_int32, cand)
    v, nv = _arr(C.c_int32, vam)
    m = C.c_int32()
    _policy_check(lib().dflash_accept_prefix(c, nc, v, nv, C.byref(m)), "accept_prefix")
    return m.value


def dflash_rejection_accept_len(p, q, u) -> int:
    n = len(p)
    pa, _ = _arr(C.c_double, p)
    qa, _ = _arr(C.c_double, q)
    ua, _ = _arr(C.c_double, u)
    out = C.c_int32()
    _policy_check(lib().dflash_rejection_accept_len(pa, qa, ua, n, C.byref(out)), "rejection_accept_len")
    return out.value


def dflash_confidence_vt(raws, tau: float, vt_cap: int) -> int:
    r, n = _arr(C.c_float, raws)
    out = C.c_int32()
    _policy_check(lib().dflash_confidence_vt(r, n, tau, vt_cap, C.byref(out)), "confidence_vt")
    return out.value


def dflash_slot_confidence_vt(raws, tau: float, vt_cap: int) -> int:
    r, n = _arr(C.c_float, raws)
    out = C.c_int32()
    _policy_check(lib().dflash_slot_confidence_vt(r, n, tau, vt_cap, C.byref(out)), "slot_confidence_vt")
    return out.value


def make_selector(pred_codebook, succ_codebook, top_k: int, w_hidden_proj=None):
    """A dflash2_selector over host bf16 codebooks (uint16 numpy arrays
    [vocab, rank], kept alive by the caller) and an optional device
    projection matrix."""
    import numpy as np
    assert pred_codebook.dtype == np.uint16 and pred_codebook.flags.c_contiguous
    assert succ_codebook.shape == pred_codebook.shape and succ_codebook.flags.c_contiguous
    return dflash2_selector(vocab=pred_codebook.shape[0], rank=pred_codebook.shape[1], top_k=top_k,
                            pred_codebook=pred_codebook.ctypes.data, succ_codebook=succ_codebook.ctypes.data,
                            w_hidden_proj=_ptr(w_hidden_proj))


def _np_ptr(a, ctype):
    return a.ctypes.data_as(C.POINTER(ctype))


def dflash2_walk_greedy(sel: dflash2_selector, unary, cand, hproj, anchor: int):
    import numpy as np
    unary = np.ascontiguousarray(unary, dtype=np.float32)
    cand = np.ascontiguousarray(cand, dtype=np.int32)
    hproj = np.ascontiguousarray(hproj, dtype=np.float32)
    nd = unary.shape[0]
    path = np.zeros(max(nd, 1), dtype=np.int32)
    _policy_check(lib().dflash2_walk_greedy(C.byref(sel), _np_ptr(unary, C.c_float), _np_ptr(cand, C.c_int32),
                                            _np_ptr(hproj, C.c_float), nd, anchor, _np_ptr(path, C.c_int32)),
                  "walk_greedy")
    return path[:nd].tolist()


def dflash2_walk_sampled(sel: dflash2_selector, unary, cand, hproj, anchor: int, temperature: float, uniforms):
    import numpy as np
    unary = np.ascontiguousarray(unary, dtype=np.float32)
    cand = np.ascontiguousarray(cand, dtype=np.int32)
    hproj = np.ascontiguousarray(hproj, dtype=np.float32)
    uni = np.ascontiguousarray(uniforms, dtype=np.float64)
    nd, k = unary.shape
    path = np.zeros(max(nd, 1), dtype=np.int32)
    qc = np.zeros(max(nd, 1), dtype=np.float64)
    qr = np.zeros(max(nd * k, 1), dtype=np.float64)
    _policy_check(lib().dflash2_walk_sampled(C.byref(sel), _np_ptr(unary, C.c_float), _np_ptr(cand, C.c_int32),
                                             _np_ptr(hproj, C.c_float), nd, anchor, temperature,
                                             _np_ptr(uni, C.c_double), _np_ptr(path, C.c_int32),
                                             _np_ptr(qc, C.c_double), _np_ptr(qr, C.c_double)), "walk_sampled")
    return path[:nd].tolist(), qc[:nd].tolist(), qr[:nd * k].tolist()


def dflash2_propose_prepare(model, sel: dflash2_selector, draft_logits, hidden, b: int, packed, ws, ws_bytes,
                            stream=None) -> None:
    _check(lib().dflash2_propose_prepare(model, C.byref(sel), _ptr(draft_logits), _ptr(hidden), b, _ptr(packed),
                                         _ptr(ws), ws_bytes, _stream(stream)))


def dflash2_propose_greedy(model, sel: dflash2_selector, draft_logits, hidden, b: int, anchor: int, ws, ws_bytes,
                           stream=None):
    out = (C.c_int32 * max(b - 1, 1))()
    _check(lib().dflash2_propose_greedy(model, C.byref(sel), _ptr(draft_logits), _ptr(hidden), b, anchor, out,
                                        _ptr(ws), ws_bytes, _stream(stream)))
    return list(out)[:b - 1]


def dflash_last_error() -> str:
    return lib().dflash_last_error().decode()


def dflash_rope_table(model, half: int):
    buf = (C.c_double * half)()
    ms = C.c_double()
    _check(lib().dflash_rope_table(model, buf, half, C.byref(ms)))
    return list(buf), ms.value


def dflash_workspace_status(model, ws, ws_bytes, stream=None) -> None:
    _check(lib().dflash_workspace_status(model, _ptr(ws), ws_bytes, _stream(stream)))


def dflash_prof_trace(enable: bool) -> None:
    _check(lib().dflash_prof_trace(1 if enable else 0))


def dflash_prof_trace_read(model, ws, ws_bytes, n: int, stream=None):
    buf = (C.c_uint64 * n)()
    _check(lib().dflash_prof_trace_read(model, _ptr(ws), ws_bytes, buf, n, _stream(stream)))
    return list(buf)


def dflash_prof_start(kernel_class: int, max_launches: int) -> None:
    _check(lib().dflash_prof_start(kernel_class, max_launches))


def dflash_prof_stop():
    """-> (total_ms, launches)"""
    ms = C.c_double()
    n = C.c_int32()
    _check(lib().dflash_prof_stop(C.byref(ms), C.byref(n)))
    return ms.value, n.value


# --------------------------------------------------------------------------
# marshalling helpers: configs, device weights, KV storage, workspace
# --------------------------------------------------------------------------

def make_cfg(c) -> dflash_cfg:
    """A dflash_cfg from any object with the drafter config attribute names."""
    return dflash_cfg(
        n_layers=c.n_layers, hidden=c.hidden, n_q_heads=c.n_q_heads, n_kv_heads=c.n_kv_heads,
        head_dim=c.head_dim, intermediate=c.intermediate, n_taps=c.n_taps, rms_eps=c.rms_eps,
        rope_base=c.rope_base, rope_type=ROPE_CODES[c.rope_type], yarn_factor=c.yarn_factor,
        yarn_orig_ctx=c.yarn_orig_ctx, yarn_beta_fast=c.yarn_beta_fast, yarn_beta_slow=c.yarn_beta_slow,
        weight_dtype=DTYPE_CODES[c.weight_dtype], kv_dtype=DTYPE_CODES[c.kv_dtype], d2_groups=c.d2_groups)


def _to_device(arr, device):
    t = torch.from_numpy(arr)
    if t.dtype == torch.uint16:
        t = t.view(torch.int16)
    return t.to(device).contiguous()


class DeviceWeights:
    """Uploads stored weights (objects with ``.dtype``, ``.data`` and ``.scale``
    per matrix) to the GPU and builds the dflash_weights struct over them.
    The tensors live as long as this object does."""

    MATS = ("wq", "wk", "wv", "wo", "wg", "wu", "wd")

    def __init__(self, stored, device="cuda"):
        self.tensors = []
        self.cfg = stored.cfg

        def mat(sm):
            d = _to_device(sm.data, device)
            s = _to_device(sm.scale, device) if sm.scale is not None else None
            self.tensors += [d, s]
            return dflash_matrix(d.data_ptr(), s.data_ptr() if s is not None else None)

        def vec(a):
            t = _to_device(a, device)
            self.tensors.append(t)
            return t.data_ptr()

        L = len(stored.layers)
        self.layer_arr = (dflash_layer_weights * max(L, 1))()
        for l, ls in enumerate(stored.layers):
            lw = self.layer_arr[l]
            for n in self.MATS:
                setattr(lw, n, mat(ls[n]))
            for n in ("g_in", "g_post", "g_q", "g_k"):
                setattr(lw, n, vec(ls[n]))
            if "attn.w_dyn" in ls:
                lw.attn_w_dyn = mat(ls["attn.w_dyn"])
                lw.attn_base = vec(ls["attn.base"])
                lw.mlp_w_dyn = mat(ls["mlp.w_dyn"])
                lw.mlp_base = vec(ls["mlp.base"])
        self.struct = dflash_weights(fc=mat(stored.fc), g_hidden_norm=vec(stored.g_hidden_norm),
                                     g_norm=vec(stored.g_norm), layers=self.layer_arr)


class KVCache:
    """Device storage for one dflash_kv: K [L][nkv][cap][d], V
    [L][nkv][cap/32][d][32] (transposed per tile of 32 rows)."""

    def __init__(self, cfg, capacity: int, device="cuda"):
        dt = torch.float32 if cfg.kv_dtype == "f32" else torch.bfloat16
        L, h, d = cfg.n_layers, cfg.n_kv_heads, cfg.head_dim
        if capacity % 64:
            raise ValueError("capacity must be a multiple of 64")
        self.k = torch.zeros((max(L, 1), h, capacity, d), dtype=dt, device=device)
        self.v = torch.zeros((max(L, 1), h, capacity // 32, d, 32), dtype=dt, device=device)
        self.c = dflash_kv(self.k.data_ptr(), self.v.data_ptr(), capacity, 0)

    @property
    def len(self) -> int:
        return self.c.len

    @len.setter
    def len(self, n: int):
        self.c.len = n

    def prefill(self, k_stored, v_stored) -> None:
        """Write stored rows [L][nkv][rows][d] (f32, or bf16 bits as uint16)
        into rows [0, rows) and set len = rows."""
        rows = k_stored.shape[2]
        k = _to_device(k_stored, self.k.device).view(self.k.dtype)
        v = _to_device(v_stored, self.k.device).view(self.v.dtype)
        self.k[:, :, :rows] = k
        r = torch.arange(rows, device=self.k.device)
        # [L][h][rows][d] -> V[l][h][r / 32][d][r % 32]
        self.v[:, :, r // 32, :, r % 32] = v.permute(2, 0, 1, 3)
        self.c.len = rows

    def rows(self, layer: int, start: int, stop: int):
        """(K, V) of rows [start, stop) of one layer as [rows, nkv, d] tensors."""
        r = torch.arange(start, stop, device=self.k.device)
        return (self.k[layer, :, start:stop].transpose(0, 1),
                self.v[layer][:, r // 32, :, r % 32])


class PagedKVCache(KVCache):
    """Paged storage for one dflash_kv: K [L][pages][nkv][P][d], V
    [L][pages][nkv][P/32][d][32], a device block table mapping logical page i to
    physical page table[i] (by default a fixed seeded permutation of the
    pool, so logical order and storage order differ)."""

    def __init__(self, cfg, capacity: int, page_rows: int = 64, pool_pages: int | None = None, device="cuda",
                 table=None, seed: int = 0):
        import numpy as np
        dt = torch.float32 if cfg.kv_dtype == "f32" else torch.bfloat16
        L, h, d = cfg.n_layers, cfg.n_kv_heads, cfg.head_dim
        npg = capacity // page_rows
        pool = pool_pages if pool_pages is not None else npg
        self.page_rows, self.pool_pages = page_rows, pool
        self.k = torch.zeros((max(L, 1), pool, h, page_rows, d), dtype=dt, device=device)
        self.v = torch.zeros((max(L, 1), pool, h, page_rows // 32, d, 32), dtype=dt, device=device)
        if table is None:
            table = np.random.default_rng(seed).permutation(pool)[:npg]
        self.table_host = np.asarray(table, dtype=np.int32)
        self.table = torch.from_numpy(self.table_host.copy()).to(device)
        self.c = dflash_kv(self.k.data_ptr(), self.v.data_ptr(), capacity, 0, page_rows, pool, self.table.data_ptr(), 0)

    def _locate(self, start: int, stop: int):
        rows = np.arange(start, stop)
        return self.table_host[rows // self.page_rows], rows % self.page_rows

    def prefill(self, k_stored, v_stored) -> None:
        rows = k_stored.shape[2]
        k = _to_device(k_stored, self.k.device).view(self.k.dtype)
        v = _to_device(v_stored, self.k.device).view(self.v.dtype)
        pg, off = self._locate(0, rows)
        pg_t = torch.from_numpy(pg).to(self.k.device)
        off_t = torch.from_numpy(off).to(self.k.device)
        # [L][h][rows][d] -> K[l][page][h][off][d], V[l][page][h][off / 32][d][off % 32]
        self.k[:, pg_t, :, off_t, :] = k.permute(2, 0, 1, 3)
        self.v[:, pg_t, :, off_t // 32, :, off_t % 32] = v.permute(2, 0, 1, 3)
        self.c.len = rows

    def rows(self, layer: int, start: int, stop: int):
        pg, off = self._locate(start, stop)
        pg_t = torch.from_numpy(pg).to(self.k.device)
        off_t = torch.from_numpy(off).to(self.k.device)
        return self.k[layer, pg_t, :, off_t, :], self.v[layer][pg_t, :, off_t // 32, :, off_t % 32]


class Drafter:
    """A loaded model plus one workspace; wraps the five calls with torch
    tensors.  The caller supplies KV storage (:class:`KVCache`)."""

    def __init__(self, stored, device="cuda", max_rows: int = 16):
        self.cfg = stored.cfg
        self.device = torch.device(device)
        self.weights = DeviceWeights(stored, device)
        self.ccfg = make_cfg(self.cfg)
        self.model = dflash_load_weights(self.ccfg, self.weights.struct)
        self.packed_bytes = dflash_packed_bytes(self.model)
        self.packed = torch.empty(max(self.packed_bytes, 256), dtype=torch.uint8, device=self.device)
        dflash_pack_weights(self.model, self.packed, self.packed_bytes)
        self.max_rows = 0
        self.batch_seqs = 0
        self.ws = None
        self.ensure_rows(max_rows)

    def _realloc(self, rows: int, seqs: int):
        """A fresh zero-filled workspace for `rows` ctx rows and, with
        seqs > 0, the layered path for `seqs` sequences."""
        self.max_rows, self.batch_seqs = rows, seqs
        self.ws_bytes = (dflash_batch_workspace_bytes(self.model, seqs, rows) if seqs
                         else dflash_workspace_bytes(self.model, rows))
        self.ws = torch.zeros(self.ws_bytes, dtype=torch.uint8, device=self.device)

    def ensure_rows(self, rows: int):
        if rows > self.max_rows or self.ws is None:
            self._realloc(rows, self.batch_seqs)

    def __del__(self):
        try:
            if getattr(self, "model", None):
                dflash_free(self.model)
                self.model = None
        except Exception:
            pass

    def status(self) -> None:
        """Raise if a kernel that used this workspace timed out at a grid barrier."""
        dflash_workspace_status(self.model, self.ws, self.ws_bytes)

    def ctx_features(self, taps: torch.Tensor) -> torch.Tensor:
        t = taps.shape[0]
        self.ensure_rows(t)
        feats = torch.empty((t, self.cfg.hidden), dtype=torch.float32, device=self.device)
        dflash_ctx_features(self.model, taps, t, feats, self.ws, self.ws_bytes)
        return feats

    def ingest_ctx(self, kv: KVCache, feats: torch.Tensor, pos_new: torch.Tensor) -> None:
        t = feats.shape[0]
        self.ensure_rows(t)
        dflash_ingest_ctx(self.model, kv.c, feats, pos_new, t, self.ws, self.ws_bytes)

    def forward_round(self, kv: KVCache, noise_emb: torch.Tensor, pos_block: torch.Tensor,
                      out: torch.Tensor | None = None) -> torch.Tensor:
        b = noise_emb.shape[0]
        if kv.c.page_rows or kv.c.ctx_cap:
            self.ensure_batch(1)
        if out is None:
            out = torch.empty((b, self.cfg.hidden), dtype=torch.float32, device=self.device)
        dflash_forward_round(self.model, kv.c, noise_emb, pos_block, b, out, self.ws, self.ws_bytes)
        return out

    def ensure_batch(self, n_seqs: int):
        """Grow the workspace to serve the layered path (batched rounds,
        paged or windowed caches) for up to n_seqs sequences."""
        if n_seqs > self.batch_seqs:
            self._realloc(self.max_rows, n_seqs)

    def ingest_ctx_batch(self, caches, feats: torch.Tensor, pos_new: torch.Tensor) -> None:
        """feats [S, t, H], pos_new [S, t]: t new rows into each cache."""
        S, t = feats.shape[0], feats.shape[1]
        self.ensure_rows(S * t)
        arr = kv_array(caches)
        dflash_ingest_ctx_batch(self.model, arr, feats, pos_new, t, self.ws, self.ws_bytes)
        for c, k in zip(caches, arr):
            c.c.len = k.len

    def forward_round_batch(self, caches, noise_emb: torch.Tensor, pos_block: torch.Tensor) -> torch.Tensor:
        """noise_emb [S, b, H], pos_block [S, b] -> out [S, b, H]."""
        S, b = noise_emb.shape[0], noise_emb.shape[1]
        self.ensure_batch(S)
        out = torch.empty((S, b, self.cfg.hidden), dtype=torch.float32, device=self.device)
        dflash_forward_round_batch(self.model, kv_array(caches), noise_emb, pos_block, b, out, self.ws, self.ws_bytes)
        return out

    def forward_full(self, taps: torch.Tensor, noise_emb: torch.Tensor, pos: torch.Tensor,
                     scratch: KVCache | None = None) -> torch.Tensor:
        n, b = taps.shape[0], noise_emb.shape[0]
        self.ensure_rows(n)
        if scratch is not None and scratch.c.page_rows:
            self.ensure_batch(1)
        if scratch is None:
            scratch = KVCache(self.cfg, max(64, (n + b + 63) // 64 * 64), self.device)
        out = torch.empty((b, self.cfg.hidden), dtype=torch.float32, device=self.device)
        dflash_forward_full(self.model, taps, noise_emb, pos, n, b, out, scratch.c, self.ws, self.ws_bytes)
        return out
