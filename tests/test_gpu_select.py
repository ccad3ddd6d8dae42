"""GPU parity of the DFlash2 proposal ([DflashDraft] dflash2_propose_greedy):
device top-k over the draft logits, the rank-r hidden projection, one
device-to-host copy and the host greedy walk, against the oracle
(oracle/dflash_policy.py).

* top-k values and ids: bit-exact (integer decisions on the same f32
  logits; logits quantised to 1/8 so that ties occur and must go to the
  lower id);
* hproj: f32 accumulation against the oracle's f64, 1e-5 relative;
* drafts: identical to the oracle walk fed the device's own top-k and hproj
  (both walks decide in f64 on the same values), and identical to the
  oracle's end-to-end proposal on every slot whose score margin is not a
  near-tie of the hproj rounding.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import dflash_policy as P
from oracle.dflash_oracle import decode_bf16
from tests.gpu_util import dev, parity_log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def drafter():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    from block_diffusion_drafter_round_amd import dflash as D
    cfg = synth.ROUND8_BF16.replace(n_layers=1)
    return cfg, D.Drafter(synth.make_weights(cfg), max_rows=16), D


# (151936, 32): first stage + merge of 149 sorted lists (three per lane at
# most); (151936, 64): lists past the merge's LDS, so three stages; (1025,
# 64): a merge whose second list is one entry and 63 "taken" ones;
# (70000, 17): 69 lists, two on lanes 0-4; 1000 and 100: one stage
@pytest.mark.parametrize("vocab,k,rank,b", [(151936, 32, 64, 16), (151936, 64, 128, 3), (1000, 8, 16, 16),
                                             (100, 64, 8, 2), (4097, 5, 64, 9), (1025, 64, 8, 2), (70000, 17, 16, 5)])
def test_propose_greedy_matches_oracle(drafter, vocab, k, rank, b):
    cfg, dr, D = drafter
    H = cfg.hidden
    rng = np.random.default_rng(vocab + k + rank + b)
    logits = np.round(rng.standard_normal((b, vocab)).astype(np.float32) * 8) / 8      # many ties
    hidden = rng.standard_normal((b, H)).astype(np.float32)
    w_hp = synth.encode_bf16((rng.standard_normal((rank, H)) * 0.02).astype(np.float32))
    pred = synth.encode_bf16(rng.standard_normal((vocab, rank)).astype(np.float32))
    succ = synth.encode_bf16(rng.standard_normal((vocab, rank)).astype(np.float32))
    w_dev = torch.from_numpy(w_hp.view(np.int16)).cuda()
    sel = D.make_selector(pred, succ, k, w_dev)
    nd = b - 1
    t_logits, t_hidden = dev(logits), dev(hidden)
    packed = torch.zeros(nd * (2 * k + rank), dtype=torch.int32, device="cuda")
    D.dflash2_propose_prepare(dr.model, sel, t_logits, t_hidden, b, packed, dr.ws, dr.ws_bytes)
    torch.cuda.synchronize()
    pk = packed.cpu().numpy()
    g_vals = pk[:nd * k].view(np.float32).reshape(nd, k)
    g_idx = pk[nd * k:2 * nd * k].reshape(nd, k)
    g_hp = pk[2 * nd * k:].view(np.float32).reshape(nd, rank)

    o_vals, o_idx = P.topk_rows(logits[1:], k)
    assert np.array_equal(g_idx, o_idx), "top-k ids differ"
    assert np.array_equal(g_vals, o_vals), "top-k values differ"
    o_hp = hidden[1:].astype(np.float64) @ decode_bf16(w_hp).T
    err = float(np.abs(g_hp - o_hp).max() / np.abs(o_hp).max())
    print(f"[select] V={vocab} k={k} r={rank} b={b}: hproj rel {err:.2e}", flush=True)
    parity_log("rel", f"dflash2 hproj V={vocab} k={k} rank={rank} b={b}", rel=err, tol=1e-5, finite=True)
    assert err <= 1e-5

    anchor = int(rng.integers(0, vocab))
    drafts = D.dflash2_propose_greedy(dr.model, sel, t_logits, t_hidden, b, anchor, dr.ws, dr.ws_bytes)
    P_, S_ = decode_bf16(pred), decode_bf16(succ)
    same_inputs = P.walk_greedy(g_vals, g_idx, g_hp, P_, S_, anchor)
    assert drafts == same_inputs, "walk on the device's own top-k / hproj differs"
    ref = P.walk_greedy(o_vals, o_idx, o_hp, P_, S_, anchor)
    # where they differ, the oracle's choice at the first differing slot must be a near-tie
    for p in range(nd):
        if drafts[p] != ref[p]:
            prev = anchor if p == 0 else ref[p - 1]
            sc = np.sort(P.walk_scores(o_vals[p], o_idx[p], prev, o_hp[p], P_, S_))
            assert sc[-1] - sc[-2] < 1e-4, f"slot {p}: drafts differ at a clear margin"
            break
    parity_log("argmax", f"dflash2 drafts V={vocab} k={k} rank={rank} b={b}", mismatches=int(drafts != ref),
               bad=[], exempt=[], max_logit_diff=0.0, rows=nd, tie_gap=1e-4)


def test_propose_rejects_bad_arguments(drafter):
    cfg, dr, D = drafter
    pred = np.zeros((10, 4), np.uint16)
    w = torch.zeros((4, cfg.hidden), dtype=torch.int16, device="cuda")
    logits = torch.zeros((16, 10), device="cuda")
    hidden = torch.zeros((16, cfg.hidden), device="cuda")
    for sel, b in ((D.make_selector(pred, pred, 11, w), 16),      # top_k > vocab
                   (D.make_selector(pred, pred, 4, w), 1),       # no draft row
                   (D.make_selector(pred, pred, 4, None), 16)):  # no projection matrix
        with pytest.raises(D.DflashError) as ei:
            D.dflash2_propose_greedy(dr.model, sel, logits, hidden, b, 0, dr.ws, dr.ws_bytes)
        assert ei.value.code == D.DFLASH_E_INVAL


@pytest.mark.parametrize("hot", [(7,), (7, 100), (0, 148)])
def test_propose_topk_concentrated(drafter, hot):
    """The row's k best packed into one or two 1024-entry chunks (more than
    the 8 per chunk the first stage keeps before the merge), with ties:
    the device top-k must still equal the oracle's bit for bit."""
    cfg, dr, D = drafter
    vocab, k, rank, b = 151936, 32, 16, 4
    rng = np.random.default_rng(1000 + sum(hot))
    logits = (np.round(rng.standard_normal((b, vocab)) * 8) / 8).astype(np.float32)
    for r in range(b):
        for c in hot:
            lo, hi = c * 1024, min(vocab, c * 1024 + 1024)
            pick = rng.choice(hi - lo, size=min(40, hi - lo), replace=False) + lo
            logits[r, pick] = 100.0 + np.round(rng.standard_normal(len(pick)) * 2) / 2    # ties among them too
    hidden = rng.standard_normal((b, cfg.hidden)).astype(np.float32)
    w_hp = synth.encode_bf16((rng.standard_normal((rank, cfg.hidden)) * 0.02).astype(np.float32))
    tab = synth.encode_bf16(rng.standard_normal((vocab, rank)).astype(np.float32))
    sel = D.make_selector(tab, tab, k, torch.from_numpy(w_hp.view(np.int16)).cuda())
    nd = b - 1
    packed = torch.zeros(nd * (2 * k + rank), dtype=torch.int32, device="cuda")
    D.dflash2_propose_prepare(dr.model, sel, dev(logits), dev(hidden), b, packed, dr.ws, dr.ws_bytes)
    torch.cuda.synchronize()
    pk = packed.cpu().numpy()
    g_vals = pk[:nd * k].view(np.float32).reshape(nd, k)
    g_idx = pk[nd * k:2 * nd * k].reshape(nd, k)
    o_vals, o_idx = P.topk_rows(logits[1:], k)
    print(f"[select] concentrated top-k, hot chunks {hot}", flush=True)
    assert np.array_equal(g_idx, o_idx), "top-k ids differ"
    assert np.array_equal(g_vals, o_vals), "top-k values differ"
    # the k best do come from the hot chunks, more than 8 from some chunk
    assert np.all(np.isin(o_idx // 1024, hot))
    assert max(np.bincount(o_idx[r] // 1024).max() for r in range(nd)) > 8
