"""Plain CPU oracle of the drafter's host-side policy functions.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module; the product
library never does, and this module imports nothing from it.  Pure Python
loops over small arrays, written from the function descriptions on
[memra dflash module] (docs.rs memra_engine::dflash, module index), sections
``dspark_accept_prefix``, ``rejection_accept_len``, ``dspark_confidence_vt``,
``dspark_slot_confidence_vt``, ``dflash2_walk_greedy`` and
``dflash2_walk_sampled``, and [DflashDraft] ``dflash2_propose_greedy``.

Readings where the pages leave a step open:

* P-1: in the accepted prefix, draft j (1-based) is accepted when it equals
  the target's argmax for its position, vam[j-1]; the walk stops at the
  first miss and may not accept more drafts than there are verify argmaxes
  beyond the one that becomes the next anchor (m <= len(vam) - 1).
* P-2: sigmoid and the survival product of the confidence windows are
  computed in float64 on the given float scores; a slot is kept when its
  statistic is >= tau.  The window vt = 1 + kept is clamped to [2, vt_cap]
  (vt_cap >= 2).
* P-3: the selector's unary term for slot p, candidate k is the draft logit
  of that candidate (the k-th largest logit of the slot's row); the pair
  term is the sum over the rank r of pred[prev][r] * hproj[p][r] *
  succ[cand][r], all in float64 over the stored values; the first slot's
  predecessor is the round's anchor token.
* P-4: the sampled walk's softmax is over score / temperature; the uniform
  u picks the first candidate whose cumulative probability exceeds u, and
  the last candidate if rounding leaves u at or above the total.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = ["accept_prefix", "rejection_accept_len", "confidence_vt", "slot_confidence_vt", "sigmoid",
           "topk_rows", "walk_scores", "walk_greedy", "walk_sampled", "propose_greedy"]


def accept_prefix(cand, vam) -> int:
    """[memra dflash module, dspark_accept_prefix]: cand[0] is the round's
    anchor, cand[1:] the drafts; vam[j] is the target's argmax for the
    position after anchor + j.  Returns m, the number of leading drafts
    that match (cand[1..m] are committed and vam[m] is the next anchor)."""
    if len(vam) < 1 or len(cand) < 1:
        raise ValueError("need the anchor and at least one verify argmax")
    m = 0
    while m + 1 < len(cand) and m + 1 < len(vam) and cand[m + 1] == vam[m]:
        m += 1
    return m


def rejection_accept_len(p, q, u) -> int:
    """[memra dflash module, rejection_accept_len]: accept draft j while
    u[j] * q[j] < p[j], strictly, in float64; p and q are the target's and
    the proposal's (filtered) probabilities of the drafted tokens, u the
    slots' uniforms.  Returns the number of leading accepted drafts."""
    n = 0
    for pj, qj, uj in zip(p, q, u):
        if not (float(uj) * float(qj) < float(pj)):
            break
        n += 1
    return n


def sigmoid(x: float) -> float:
    x = float(x)
    if x >= 0:
        return 1.0 / (1.0 + math.exp(-x))
    e = math.exp(x)
    return e / (1.0 + e)


def _clamp_vt(kept: int, vt_cap: int) -> int:
    if vt_cap < 2:
        raise ValueError("vt_cap must be >= 2")
    return max(2, min(1 + kept, vt_cap))


def confidence_vt(raws, tau: float, vt_cap: int) -> int:
    """[memra dflash module, dspark_confidence_vt]: raws[k] is the accept
    head's pre-sigmoid score of draft slot k+1.  The survival
    S_k = prod_{j<=k} sigmoid(raws[j]); leading slots are kept while
    S_k >= tau.  Returns vt = 1 + kept, clamped to [2, vt_cap]."""
    s, kept = 1.0, 0
    for r in raws:
        s *= sigmoid(r)
        if not (s >= tau):
            break
        kept += 1
    return _clamp_vt(kept, vt_cap)


def slot_confidence_vt(raws, tau: float, vt_cap: int) -> int:
    """[memra dflash module, dspark_slot_confidence_vt]: the longest prefix
    of slots whose own sigmoid(raws[k]) is >= tau; the first slot below tau
    ends it.  Returns vt = 1 + kept, clamped to [2, vt_cap]."""
    kept = 0
    for r in raws:
        if not (sigmoid(r) >= tau):
            break
        kept += 1
    return _clamp_vt(kept, vt_cap)


# --------------------------------------------------------------------------
# DFlash2 candidate selector
# --------------------------------------------------------------------------

def topk_rows(logits: np.ndarray, k: int):
    """The k largest entries of each row, largest first; equal values in
    increasing index order.  Returns (values [rows, k], indices [rows, k])."""
    logits = np.asarray(logits)
    idx = np.empty((logits.shape[0], k), dtype=np.int64)
    for r in range(logits.shape[0]):
        # primary key: value, descending; secondary: index, ascending
        order = np.lexsort((np.arange(logits.shape[1]), -logits[r].astype(np.float64)))
        idx[r] = order[:k]
    vals = np.take_along_axis(logits, idx, axis=1)
    return vals, idx


def walk_scores(unary_p, cand_p, prev: int, hproj_p, pred_cb, succ_cb):
    """Pair scores of one slot ([memra dflash module, dflash2_walk_greedy]):
    score(k) = unary[k] + sum_r pred[prev][r] * hproj[r] * succ[cand[k]][r]."""
    pv = np.asarray(pred_cb[prev], dtype=np.float64)
    hp = np.asarray(hproj_p, dtype=np.float64)
    out = []
    for k, c in enumerate(cand_p):
        sv = np.asarray(succ_cb[int(c)], dtype=np.float64)
        pair = 0.0
        for r in range(len(pv)):
            pair += pv[r] * hp[r] * sv[r]
        out.append(float(unary_p[k]) + pair)
    return out


def walk_greedy(unary, cand, hproj, pred_cb, succ_cb, anchor: int):
    """[memra dflash module, dflash2_walk_greedy]: per draft slot, the
    candidate of highest pair score (ties to the lowest k); the chosen
    token is the next slot's predecessor.  Returns the drafted tokens."""
    path, prev = [], int(anchor)
    for p in range(len(cand)):
        sc = walk_scores(unary[p], cand[p], prev, hproj[p], pred_cb, succ_cb)
        best = 0
        for k in range(1, len(sc)):
            if sc[k] > sc[best]:
                best = k
        prev = int(cand[p][best])
        path.append(prev)
    return path


def walk_sampled(unary, cand, hproj, pred_cb, succ_cb, anchor: int, temperature: float, uniforms):
    """[memra dflash module, dflash2_walk_sampled]: per draft slot, a
    softmax at `temperature` over the pair scores, one uniform per slot
    drawing the candidate by a cumulative walk in candidate order; the
    chosen token seeds the next slot.  Returns (path, q_chosen, q_rows) with
    q_rows the per-slot candidate probabilities, flattened [slot][k]."""
    path, q_chosen, q_rows, prev = [], [], [], int(anchor)
    for p in range(len(cand)):
        sc = walk_scores(unary[p], cand[p], prev, hproj[p], pred_cb, succ_cb)
        mx = max(sc)
        w = [math.exp((s - mx) / temperature) for s in sc]
        tot = sum(w)
        q = [x / tot for x in w]
        u = float(uniforms[p])
        pick, acc = len(q) - 1, 0.0
        for k, qk in enumerate(q):
            acc += qk
            if u < acc:
                pick = k
                break
        prev = int(cand[p][pick])
        path.append(prev)
        q_chosen.append(q[pick])
        q_rows.extend(q)
    return path, q_chosen, q_rows


def propose_greedy(logits: np.ndarray, hidden: np.ndarray, w_hproj: np.ndarray, pred_cb, succ_cb,
                   anchor: int, top_k: int):
    """[DflashDraft, dflash2_propose_greedy]: the drafts of rows 1..b-1 (row
    0 is the anchor row, not a draft): top-k of each row's draft logits,
    the rank-r projection hproj = hidden . w_hproj^T, then the greedy walk.
    Returns (drafts, top-k values, top-k indices, hproj)."""
    rows = slice(1, logits.shape[0])
    vals, idx = topk_rows(logits[rows], top_k)
    hp = np.asarray(hidden[rows], dtype=np.float64) @ np.asarray(w_hproj, dtype=np.float64).T
    return walk_greedy(vals, idx, hp, pred_cb, succ_cb, anchor), vals, idx, hp
