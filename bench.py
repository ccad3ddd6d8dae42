#!/usr/bin/env python3
"""Benchmark: DFlash drafter rounds per second at ctx 4096 on one MI355X.

Workload: the 8-layer drafter (hidden 2048, GQA 32:4, head_dim 128, SwiGLU
6144, 5 taps, bf16 weights, bf16 KV), random-initialised, on the cached round
path.  One step (one round) is:
  1. ctx_features of 16 new tapped rows;
  2. ingest_ctx of those 16 rows at positions 4080..4095 (len 4080 -> 4096);
  3. forward_round of a 16-token block at positions 4096..4111, which
     attends 4112 keys;
  4. a rewind of len to 4080 on the host (no GPU work).

The KV cache is prefilled once, untimed, through the same calls.  All inputs
are resident in HBM before the timed region starts.

Printed as one JSON line:
* value: rounds per second;
* roofline: the persistent forward_round kernel's algorithmic bytes per
  launch over its average launch time, timed live with HIP events on its
  stream;
* roofline.traffic: the kernel's measured HBM bytes per launch, from the
  rocprofv3 FETCH_SIZE / WRITE_SIZE record committed under profiles/
  (each counter scaled by what it reads for a plain device copy of known
  size); null when the kernel's sources no longer match that record;
* roofline.copy_gbs / frac_of_copy: the rate of a plain 1 GiB device copy
  measured in the same run, and the kernel's achieved rate against it;
* spread: p10 / p50 / p90 of 100 rounds timed one by one;
* cpu_baseline: the fp64 CPU oracle running the same round on a bounded
  sample, on all host threads and on one (value_1thread).

``python bench.py --copy-calibration`` only copies 256 MiB on the device five
times: run under ``rocprofv3 --pmc FETCH_SIZE`` (then WRITE_SIZE) it gives the
counters' scale factors.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402

METRIC = "drafter 16-token rounds/sec at ctx 4096 + achieved HBM GB/s fraction"
HBM_PEAK_GBS = 8000.0     # MI355X HBM3E, vendor figure
TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "sround_kernel_c3_ctx4096_traffic.md")
KERNEL_SOURCES = [os.path.join(ROOT, "block_diffusion_drafter_round_amd", "csrc", f) for f in ("sround.hip", "sround.h")]


def kernel_sources_sha256() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic() -> dict | None:
    """HBM bytes per launch of the round kernel from the committed counter
    record, or None if the record is missing or was taken on other sources.
    The record holds one line ``traffic-record: key=value; ...``."""
    try:
        with open(TRAFFIC_RECORD) as fh:
            line = next(l for l in fh if l.startswith("traffic-record:"))
    except (OSError, StopIteration):
        return None
    kv = dict(x.strip().split("=", 1) for x in line.split(":", 1)[1].split(";") if "=" in x)
    if kv.get("sources_sha256") != kernel_sources_sha256():
        return None
    fetch = float(kv["fetch_kib"]) * 1024 * float(kv["fetch_scale"])
    write = float(kv["write_kib"]) * 1024 * float(kv["write_scale"])
    return {"fetch": int(fetch), "write": int(write), "total": int(fetch + write)}


def copy_calibration() -> int:
    """256 MiB device-to-device copy, five times (counter calibration)."""
    import torch
    n = 256 << 20
    a = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(f"copied {n} bytes 5 times", flush=True)
    return 0


def round_bytes(cfg, ctx: int, t: int = 16, b: int = 16) -> dict:
    """Algorithmic HBM bytes of one round: every weight read once, the
    attended K/V read once per layer, the new K/V rows written, the taps read.
    Activations that stay in L2 (<1 MB) are not counted."""
    wb = {"f32": 4, "bf16": 2, "fp8": 1}[cfg.weight_dtype]
    kvb = 4 if cfg.kv_dtype == "f32" else 2
    H, I, qd, kvd, L = cfg.hidden, cfg.intermediate, cfg.q_dim, cfg.kv_dim, cfg.n_layers
    layer_w = ((qd + 2 * kvd) * H + H * qd + 3 * I * H) * wb * L
    fc_w = H * cfg.n_taps * H * wb
    ingest_w = 2 * kvd * H * wb * L
    kv_read = (ctx + b) * kvd * 2 * kvb * L
    kv_write = (t + b) * kvd * 2 * kvb * L
    taps = t * cfg.n_taps * H * 4
    scales = 0
    if cfg.weight_dtype == "fp8":
        scales = ((qd + 2 * kvd) + H + 3 * I + 2 * kvd) * 4 * L + H * 4
    if cfg.d2_groups:      # DFlash2: dynamic-coefficient projections [4G][H] (+ fp8 scales) and static taps
        G4 = 4 * cfg.d2_groups
        scales += (2 * G4 * H * wb + (2 * G4 * 4 if cfg.weight_dtype == "fp8" else 0) + 2 * 2 * H * 2 * 4) * L
    tot = layer_w + fc_w + ingest_w + kv_read + kv_write + taps + scales
    return dict(layer_weights=layer_w, fc_weights=fc_w, ingest_weights=ingest_w, kv_read=kv_read,
                kv_write=kv_write, taps=taps, scales=scales, total=tot)


def round_kernel_bytes(cfg, ctx: int, b: int = 16) -> int:
    """One launch of the persistent forward_round kernel: every layer's
    weights once, each layer's K/V over all ctx + b keys once, the block K/V
    rows written, the block embeddings read and the output written."""
    wb = {"f32": 4, "bf16": 2, "fp8": 1}[cfg.weight_dtype]
    kvb = 4 if cfg.kv_dtype == "f32" else 2
    H, I, qd, kvd, L = cfg.hidden, cfg.intermediate, cfg.q_dim, cfg.kv_dim, cfg.n_layers
    layer_w = ((qd + 2 * kvd) * H + H * qd + 3 * I * H) * wb * L
    kv_read = (ctx + b) * kvd * 2 * kvb * L
    kv_write = b * kvd * 2 * kvb * L
    io = 2 * b * H * 4
    return layer_w + kv_read + kv_write + io


def cpu_baseline(cfg, ctx: int, seconds: float) -> dict:
    """The fp64 CPU oracle on the same round: ctx_features(16) + ingest(16)
    + forward_round(16) over a cache of ctx - 16 committed rows.  The cache is
    prefilled directly with seeded bf16 K/V, untimed.  Rounds repeat until
    `seconds` of CPU time have passed."""
    from oracle import dflash_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    m = O.OracleModel(synth.make_weights(cfg))
    base = ctx - 16
    kv = O.OracleKV(cfg)
    kst, vst = synth.make_prefill_kv(cfg, base)
    kv.prefill(kst, vst)
    taps = synth.make_taps(cfg, 16, stream=1)
    noise = synth.make_noise(cfg)
    pos_new = synth.positions(base, 16)
    pos_blk = synth.positions(ctx, 16)
    def rounds(budget: float):
        n, t0 = 0, time.perf_counter()
        while True:
            feats = O.ctx_features(m, taps)
            O.ingest_ctx(m, kv, feats, pos_new)
            O.forward_round(m, kv, noise, pos_blk)
            kv.truncate(base)
            n += 1
            el = time.perf_counter() - t0
            if el >= budget:
                return n, el

    n, el = rounds(seconds)
    rec = {"value": n / el, "unit": "rounds/s", "cores": int(threads), "kind": "oracle",
           "sample": f"{n} full rounds (ctx_features 16 + ingest 16 + forward_round b=16 at ctx {ctx}, "
                     f"cache prefilled directly to {base} rows), {el:.1f} s, numpy fp64"}
    try:  # the same rounds on one host thread (BLAS limited to 1)
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            n1, el1 = rounds(seconds / 2)
        rec["value_1thread"] = n1 / el1
        rec["sample_1thread"] = f"{n1} rounds, {el1:.1f} s, BLAS limited to 1 thread"
    except Exception:  # pragma: no cover
        pass
    return rec


def full_bytes(cfg, n: int, b: int = 16) -> int:
    """Algorithmic HBM bytes of one first-light forward over n ctx rows:
    every weight once (W_k/W_v counted once though ingest and the round both
    read them), the taps, and the n + b K/V rows written and read back."""
    wb = {"f32": 4, "bf16": 2, "fp8": 1}[cfg.weight_dtype]
    kvb = 4 if cfg.kv_dtype == "f32" else 2
    H, I, qd, kvd, L = cfg.hidden, cfg.intermediate, cfg.q_dim, cfg.kv_dim, cfg.n_layers
    w = ((qd + 2 * kvd) * H + H * qd + 3 * I * H) * wb * L + H * cfg.n_taps * H * wb
    return w + n * cfg.n_taps * H * 4 + 2 * (n + b) * kvd * 2 * kvb * L


def batched_sweep_bytes(cfg, ctx: int, S: int, t: int = 16, b: int = 16) -> int:
    """Algorithmic HBM bytes of one batched sweep over S sequences: every
    weight read once for all S (layer weights, fc, ingest W_k/W_v), and per
    sequence its K/V read over ctx + b keys per layer, its new K/V rows
    written and its taps read."""
    r = round_bytes(cfg, ctx, t, b)
    return (r["layer_weights"] + r["fc_weights"] + r["ingest_weights"] + r["scales"]
            + S * (r["kv_read"] + r["kv_write"] + r["taps"]))


def window_round_bytes(cfg, window: int, t: int = 16, b: int = 16) -> int:
    """One round with a context window: as round_bytes, with the K/V read
    over the window's rows plus the block."""
    return round_bytes(cfg, window, t, b)["total"]


def propose_bytes(vocab: int, hidden: int, rank: int, b: int) -> int:
    """The proposal's device step: the draft rows' logits and hidden rows
    read once, the bf16 projection matrix, the packed result written."""
    nd = b - 1
    return nd * vocab * 4 + nd * hidden * 4 + rank * hidden * 2


def other_config(name: str, args) -> int:
    """Times one of the parity configurations with the same library calls
    and prints one JSON line for it (these are not the headline metric).
    c1 / c2: first-light forward_full latency.  c4 / c5: the cached round
    (ctx_features 16 + ingest_ctx 16 + forward_round b = 16) over caches set
    to their committed length directly (zero-filled rows move the same bytes
    as a real prefill), c4 over 8 sequences back to back."""
    import torch
    import synth
    from block_diffusion_drafter_round_amd import dflash as D
    cfg = {"c1": synth.TINY_F32, "c2": synth.FULL5_BF16, "c4": synth.ROUND8_YARN, "c5": synth.ROUND8_FP8_D2,
           "c4b": synth.ROUND8_YARN, "c3w": synth.ROUND8_BF16, "propose": synth.ROUND8_BF16}[name]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"[bench] loading {cfg.name}", file=sys.stderr, flush=True)
    sw = synth.make_weights(cfg)
    b = cfg.block
    stream = torch.cuda.current_stream(dev)
    if name == "propose":
        # DFlash2 proposal over a 151,936-token vocabulary: top-32 of 15 draft
        # rows, rank-64 projection, one small copy, host greedy walk
        V, k, rank = 151936, 32, 64
        dr = D.Drafter(synth.make_weights(cfg.replace(n_layers=1)), device=dev, max_rows=16)
        rng = np.random.default_rng(7)
        logits = torch.from_numpy(rng.standard_normal((b, V)).astype(np.float32)).to(dev)
        hidden = torch.from_numpy(rng.standard_normal((b, cfg.hidden)).astype(np.float32)).to(dev)
        w_hp = torch.from_numpy(synth.encode_bf16((rng.standard_normal((rank, cfg.hidden)) * 0.02)
                                                  .astype(np.float32)).view(np.int16)).to(dev)
        pred = synth.encode_bf16(rng.standard_normal((V, rank)).astype(np.float32))
        succ = synth.encode_bf16(rng.standard_normal((V, rank)).astype(np.float32))
        sel = D.make_selector(pred, succ, k, w_hp)
        packed = torch.empty((b - 1) * (2 * k + rank), dtype=torch.int32, device=dev)
        step = lambda: D.dflash2_propose_greedy(dr.model, sel, logits, hidden, b, 1, dr.ws, dr.ws_bytes, stream)
        units, unit, nbytes = 1, "proposals/s", propose_bytes(V, cfg.hidden, rank, b)
        workload = (f"DFlash2 greedy proposal: top-{k} of {b - 1} draft rows over a {V}-token vocabulary, rank-{rank} "
                    f"projection, one device-to-host copy, host walk (synchronous)")
        prof_cls = None
        # the device step alone, timed with events on its stream
        for _ in range(10):
            D.dflash2_propose_prepare(dr.model, sel, logits, hidden, b, packed, dr.ws, dr.ws_bytes, stream)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(100):
            D.dflash2_propose_prepare(dr.model, sel, logits, hidden, b, packed, dr.ws, dr.ws_bytes, stream)
        e1.record(stream)
        torch.cuda.synchronize()
        prep_us = e0.elapsed_time(e1) / 100 * 1e3
        extra = {"device_step_us": round(prep_us, 2),
                 "device_step_gbs": round(nbytes / (prep_us * 1e-6) / 1e9, 1),
                 "device_step_hbm_frac": round(nbytes / (prep_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
    elif name == "c4b":
        # the c4 sweep as one batched step: ctx_features of the 8 sequences' 16
        # new rows in one call, one batched ingest, one batched round
        ctx, t, S = cfg.ctx, cfg.new_rows, cfg.n_seqs
        base = ctx - t
        dr = D.Drafter(sw, device=dev, max_rows=S * t)
        dr.ensure_batch(S)
        kvs = [D.KVCache(cfg, (ctx + b + 63) // 64 * 64, dev) for _ in range(S)]
        taps = torch.from_numpy(synth.make_taps(cfg, S * t, stream=1)).to(dev)
        noise = torch.from_numpy(np.stack([synth.make_noise(cfg, stream=q) for q in range(S)])).to(dev)
        pos_new = torch.from_numpy(np.stack([synth.positions(base, t)] * S)).to(dev)
        pos_blk = torch.from_numpy(np.stack([synth.positions(ctx, b)] * S)).to(dev)
        feats = torch.empty((S * t, cfg.hidden), dtype=torch.float32, device=dev)
        out = torch.empty((S, b, cfg.hidden), dtype=torch.float32, device=dev)
        arr = D.kv_array(kvs)

        def step():
            for q in range(S):
                arr[q].len = base
            D.dflash_ctx_features(dr.model, taps, S * t, feats, dr.ws, dr.ws_bytes, stream)
            D.dflash_ingest_ctx_batch(dr.model, arr, feats, pos_new, t, dr.ws, dr.ws_bytes, stream)
            D.dflash_forward_round_batch(dr.model, arr, noise, pos_blk, b, out, dr.ws, dr.ws_bytes, stream)
        units, unit, nbytes = S, "sequence-rounds/s", batched_sweep_bytes(cfg, ctx, S, t, b) / S
        workload = (f"{cfg.n_layers}-layer bf16 drafter (YaRN), {S} sequences at ctx {ctx} in one batched step: "
                    f"ctx_features of {S}x{t} rows, batched ingest, batched round (weights read once per step)")
        prof_cls, extra = D.K_ATTN, {"bytes_per_step": batched_sweep_bytes(cfg, ctx, S, t, b)}
    elif name == "c3w":
        # c3 on a paged cache (256-row pages, permuted block table) with a
        # 1024-row context window: ctx_features 16 + ingest 16 + round
        ctx, t, W = cfg.ctx, cfg.new_rows, 1024
        base = ctx - t
        dr = D.Drafter(sw, device=dev, max_rows=16)
        dr.ensure_batch(1)
        kv = D.PagedKVCache(cfg, (ctx + b + 255) // 256 * 256, page_rows=256, device=dev, seed=5)
        kv.c.ctx_cap = W
        taps = torch.from_numpy(synth.make_taps(cfg, t, stream=1)).to(dev)
        noise = torch.from_numpy(synth.make_noise(cfg)).to(dev)
        pos_new = torch.from_numpy(synth.positions(base, t)).to(dev)
        pos_blk = torch.from_numpy(synth.positions(ctx, b)).to(dev)
        feats = torch.empty((t, cfg.hidden), dtype=torch.float32, device=dev)
        out = torch.empty((b, cfg.hidden), dtype=torch.float32, device=dev)

        def step():
            kv.c.len = base
            D.dflash_ctx_features(dr.model, taps, t, feats, dr.ws, dr.ws_bytes, stream)
            D.dflash_ingest_ctx(dr.model, kv.c, feats, pos_new, t, dr.ws, dr.ws_bytes, stream)
            D.dflash_forward_round(dr.model, kv.c, noise, pos_blk, b, out, dr.ws, dr.ws_bytes, stream)
        units, unit, nbytes = 1, "rounds/s", window_round_bytes(cfg, W, t, b)
        workload = (f"{cfg.n_layers}-layer bf16 drafter cached round at ctx {ctx} on a paged cache (256-row pages) "
                    f"with a {W}-row context window (layered path)")
        prof_cls, extra = D.K_ATTN, {}
    elif name in ("c1", "c2"):
        n = cfg.ctx
        dr = D.Drafter(sw, device=dev, max_rows=n)
        scratch = D.KVCache(cfg, (n + b + 63) // 64 * 64, dev)
        taps = torch.from_numpy(synth.make_taps(cfg, n)).to(dev)
        noise = torch.from_numpy(synth.make_noise(cfg)).to(dev)
        pos = torch.from_numpy(synth.positions(0, n + b)).to(dev)
        step = lambda: dr.forward_full(taps, noise, pos, scratch)
        units, unit, nbytes = 1, "forwards/s", full_bytes(cfg, n, b)
        workload = f"{cfg.n_layers}-layer {cfg.weight_dtype} drafter first-light forward_full, n={n} ctx rows, block {b}"
        prof_cls, extra = D.K_GEMM_FC, {}
    else:
        ctx, t = cfg.ctx, cfg.new_rows
        base = ctx - t
        dr = D.Drafter(sw, device=dev, max_rows=64)
        nseq = cfg.n_seqs
        kvs = [D.KVCache(cfg, (ctx + b + 63) // 64 * 64, dev) for _ in range(nseq)]
        taps = torch.from_numpy(synth.make_taps(cfg, t, stream=1)).to(dev)
        noise = torch.from_numpy(synth.make_noise(cfg)).to(dev)
        pos_new = torch.from_numpy(synth.positions(base, t)).to(dev)
        pos_blk = torch.from_numpy(synth.positions(ctx, b)).to(dev)
        feats = torch.empty((t, cfg.hidden), dtype=torch.float32, device=dev)
        out = torch.empty((b, cfg.hidden), dtype=torch.float32, device=dev)

        def step():
            for kv in kvs:
                kv.c.len = base
                D.dflash_ctx_features(dr.model, taps, t, feats, dr.ws, dr.ws_bytes, stream)
                D.dflash_ingest_ctx(dr.model, kv.c, feats, pos_new, t, dr.ws, dr.ws_bytes, stream)
                D.dflash_forward_round(dr.model, kv.c, noise, pos_blk, b, out, dr.ws, dr.ws_bytes, stream)
        units, unit, nbytes = nseq, "sequence-rounds/s", round_bytes(cfg, ctx, t, b)["total"]
        workload = (f"{cfg.n_layers}-layer {cfg.weight_dtype} drafter cached round at ctx {ctx}"
                    f"{' (YaRN)' if cfg.rope_type == 'yarn' else ''}{' with the DFlash2 conv' if cfg.d2_groups else ''}"
                    f", {nseq} sequence(s) back to back")
        prof_cls, extra = D.K_ROUND, {}
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for a, z in evs:
        a.record(stream)
        step()
        z.record(stream)
    torch.cuda.synchronize()
    dr.status()
    per = np.sort(np.array([a.elapsed_time(z) for a, z in evs])) / 1e3      # s per step
    med = float(np.median(per))
    if prof_cls is not None:
        # the dominant kernel class's average launch time, events on its stream
        D.dflash_prof_start(prof_cls, 4096)
        for _ in range(min(args.steps, 20)):
            step()
        tot_ms, nl = D.dflash_prof_stop()
        extra["dominant_kernel_class"] = {D.K_ATTN: "attention (splits + merge)", D.K_ROUND: "persistent round kernel",
                                          D.K_GEMM_FC: "fc GEMM"}[prof_cls]
        extra["dominant_kernel_avg_us"] = round(tot_ms * 1e3 / max(nl, 1), 2)
        extra["dominant_kernel_launches_per_step"] = round(nl / min(args.steps, 20), 2)
    rec = {"metric": f"{cfg.name}: {unit}", "value": round(units / med, 2), "unit": unit, "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(med * 1e3, 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": cfg.weight_dtype,
           "data": "synthetic (seeded N(0,0.02) weights, N(0,1) taps/noise, random init)",
           "config": {"workload": workload},
           "step_ms_p10_p50_p90": [round(float(np.percentile(per, q)) * 1e3, 4) for q in (10, 50, 90)],
           "algorithmic_bytes_per_unit": nbytes,
           "hbm_gbs": round(nbytes * units / med / 1e9, 1),
           "hbm_frac": round(nbytes * units / med / 1e9 / HBM_PEAK_GBS, 4), **extra}
    print(json.dumps(rec), flush=True)
    return 0


def copy_reference(torch, dev, nbytes: int = 1 << 30, reps: int = 10) -> dict:
    """Device-to-device copy of `nbytes`: the HBM rate a plain streaming
    kernel reaches on this GPU (it reads and writes nbytes per copy)."""
    a = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    sec = e0.elapsed_time(e1) / 1e3 / reps
    del a, b
    torch.cuda.empty_cache()
    return {"gbs": round(2 * nbytes / sec / 1e9, 1), "bytes_per_copy": 2 * nbytes,
            "what": f"torch device copy of {nbytes >> 20} MiB (read + write), mean of {reps}"}


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=300)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-prof", action="store_true", help="skip the live per-kernel timing")
    ap.add_argument("--copy-calibration", action="store_true", help="only run the 256 MiB copy used to scale counters")
    ap.add_argument("--config", choices=("c1", "c2", "c4", "c5", "c4b", "c3w", "propose"),
                    help="time one of the other workloads instead (c1 tiny f32 forward_full, c2 5-layer forward_full "
                         "n=1024, c4 YaRN ctx 32768 x 8 sequences back to back, c5 fp8 + DFlash2 ctx 65536, "
                         "c4b the c4 sweep as one batched step, c3w c3 on a paged cache with a 1024-row window, "
                         "propose the DFlash2 greedy proposal)")
    args = ap.parse_args(argv)
    if args.copy_calibration:
        return copy_calibration()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported (the drafter path has no "
              f"cross-GPU work; sequences shard by data parallelism).", file=sys.stderr)
        return 2
    if args.config:
        return other_config(args.config, args)

    import torch
    from block_diffusion_drafter_round_amd import dflash as D

    cfg = synth.ROUND8_BF16
    ctx, t, b = cfg.ctx, cfg.new_rows, cfg.block
    base = ctx - t
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    print(f"[bench] loading {cfg.name}", file=sys.stderr, flush=True)
    sw = synth.make_weights(cfg)
    dr = D.Drafter(sw, device=dev, max_rows=1024)
    cap = (ctx + b + 63) // 64 * 64
    kv = D.KVCache(cfg, cap, dev)
    # untimed prefill of `base` committed rows through the library itself
    for lo in range(0, base, 1020):
        hi = min(base, lo + 1020)
        taps = torch.from_numpy(synth.make_taps(cfg, hi - lo, stream=1000 + lo)).to(dev)
        dr.ingest_ctx(kv, dr.ctx_features(taps), torch.from_numpy(synth.positions(lo, hi - lo)).to(dev))
    assert kv.len == base
    taps = torch.from_numpy(synth.make_taps(cfg, t, stream=1)).to(dev)
    noise = torch.from_numpy(synth.make_noise(cfg)).to(dev)
    pos_new = torch.from_numpy(synth.positions(base, t)).to(dev)
    pos_blk = torch.from_numpy(synth.positions(ctx, b)).to(dev)
    feats = torch.empty((t, cfg.hidden), dtype=torch.float32, device=dev)
    out = torch.empty((b, cfg.hidden), dtype=torch.float32, device=dev)
    model, ws, wsb = dr.model, dr.ws, dr.ws_bytes
    stream = torch.cuda.current_stream(dev)

    def step():
        D.dflash_ctx_features(model, taps, t, feats, ws, wsb, stream)
        D.dflash_ingest_ctx(model, kv.c, feats, pos_new, t, ws, wsb, stream)
        D.dflash_forward_round(model, kv.c, noise, pos_blk, b, out, ws, wsb, stream)
        kv.c.len = base

    def timed(k: int) -> float:
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record(stream)
        for _ in range(k):
            step()
        e1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        return max(e0.elapsed_time(e1) / 1e3, 0.0), wall

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"[bench] timing {args.steps} rounds", file=sys.stderr, flush=True)
    gpu_s, wall_s = timed(args.steps)
    dr.status()     # raises if a round kernel's barrier wait expired (its output would be NaN)
    sec = max(gpu_s, wall_s)
    ms_per_step = sec * 1e3 / args.steps
    rounds_per_s = args.steps / sec
    rb = round_bytes(cfg, ctx, t, b)
    hbm_gbs = rb["total"] / (sec / args.steps) / 1e9

    roofline = None
    if not args.no_prof:
        # live timing of the dominant kernel: the persistent forward_round kernel (1 launch per round)
        D.dflash_prof_start(D.K_ROUND, args.steps)
        gpu_p, wall_p = timed(args.steps)
        tot_ms, nl = D.dflash_prof_stop()
        avg_s = tot_ms / 1e3 / max(nl, 1)
        gb = round_kernel_bytes(cfg, ctx, b)
        ach = gb / avg_s / 1e9
        tr = measured_traffic()
        roofline = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": tr["total"] if tr else None,
                    "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
                    "traffic_fetch": tr["fetch"] if tr else None, "traffic_write": tr["write"] if tr else None,
                    "kernel": "persistent forward_round kernel (8 layers, b=16, 4112 keys)",
                    "bytes_per_launch": gb, "avg_launch_us": round(avg_s * 1e6, 2), "launches": nl,
                    "ms_per_step_while_timed": round(max(gpu_p, wall_p) * 1e3 / args.steps, 4)}

    # per-round spread: each of 100 rounds between its own pair of events
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(100)]
    torch.cuda.synchronize()
    for a, z in evs:
        a.record(stream)
        step()
        z.record(stream)
    torch.cuda.synchronize()
    per = np.sort(np.array([a.elapsed_time(z) for a, z in evs]))
    spread = {"round_ms_p10": round(float(np.percentile(per, 10)), 4), "round_ms_p50": round(float(np.median(per)), 4),
              "round_ms_p90": round(float(np.percentile(per, 90)), 4), "rounds": len(per)}
    copy = copy_reference(torch, dev)
    if roofline is not None:
        roofline["copy_gbs"] = copy["gbs"]
        roofline["frac_of_copy"] = round(roofline["achieved"] / copy["gbs"], 4)

    cpu = None
    if not args.no_cpu:
        print(f"[bench] cpu oracle baseline (~{args.cpu_seconds:.0f} s)", file=sys.stderr, flush=True)
        cpu = cpu_baseline(cfg, ctx, args.cpu_seconds)

    rec = {
        "metric": METRIC, "value": round(rounds_per_s, 2), "unit": "rounds/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,0.02) weights, N(0,1) taps/noise, random init)",
        "config": {"workload": "8-layer drafter cached round: ctx_features 16 + ingest_ctx 16 + forward_round "
                               "b=16 over a ctx-4096 bf16 KV cache (4112 keys)",
                   "layers": cfg.n_layers, "hidden": cfg.hidden, "heads": f"{cfg.n_q_heads}:{cfg.n_kv_heads}",
                   "head_dim": cfg.head_dim, "intermediate": cfg.intermediate, "taps": cfg.n_taps,
                   "ctx": ctx, "block": b, "weights": "bf16", "kv": "bf16"},
        "hbm_gbs": round(hbm_gbs, 1), "hbm_frac": round(hbm_gbs / HBM_PEAK_GBS, 4),
        "round_bytes": rb["total"],
        "spread": spread,
        "copy_reference": copy,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
