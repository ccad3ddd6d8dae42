"""Host policy functions: the oracle pinned to closed forms and brute force,
and the library's C versions equal to the oracle (CPU only).

Covers [memra dflash module] dspark_accept_prefix, rejection_accept_len,
dspark_confidence_vt, dspark_slot_confidence_vt, dflash2_walk_greedy and
dflash2_walk_sampled.
"""
import itertools
import math

import numpy as np
import pytest

import synth
from oracle import dflash_policy as P


@pytest.fixture(scope="module")
def D():
    import os
    from block_diffusion_drafter_round_amd import dflash
    if not os.path.exists(dflash.LIB_PATH):
        from block_diffusion_drafter_round_amd.build import build
        build()
    dflash.lib()
    return dflash


# ------------------------------------------------------------ accept prefix --
def test_accept_prefix_pins():
    # cand[0] is the anchor; drafts 1.. are compared with vam[0..]
    assert P.accept_prefix([7, 1, 2, 3], [1, 2, 3, 9]) == 3          # all accepted; vam[3] = 9 is the bonus
    assert P.accept_prefix([7, 1, 2, 3], [5, 2, 3, 9]) == 0          # first draft missed
    assert P.accept_prefix([7, 1, 2, 3], [1, 2, 4, 9]) == 2          # stops at the first miss
    assert P.accept_prefix([7, 1, 2, 3], [1, 9, 3, 9]) == 1          # a later match after a miss never counts
    assert P.accept_prefix([7, 1, 2, 3], [1, 2]) == 1                # vam[m] must exist: m <= len(vam) - 1
    assert P.accept_prefix([7], [4]) == 0                            # no drafts


def test_accept_prefix_brute_force():
    """m is the largest k whose drafts 1..k all equal vam[0..k-1] (every
    candidate/argmax pair over a 3-token alphabet, up to 3 drafts)."""
    for nd in range(4):
        for cand in itertools.product(range(3), repeat=nd + 1):
            for nv in range(1, nd + 2):
                for vam in itertools.product(range(3), repeat=nv):
                    ok = [k for k in range(0, min(nd, nv - 1) + 1)
                          if all(cand[j] == vam[j - 1] for j in range(1, k + 1))]
                    assert P.accept_prefix(list(cand), list(vam)) == max(ok)


# ------------------------------------------------------- rejection accept --
def test_rejection_accept_pins():
    assert P.rejection_accept_len([0.5], [1.0], [0.5]) == 0           # u*q == p: strict, rejected
    assert P.rejection_accept_len([0.5], [1.0], [0.4999999999]) == 1
    assert P.rejection_accept_len([0.0, 1.0], [0.5, 0.5], [0.0, 0.0]) == 0   # p = 0 is never accepted
    assert P.rejection_accept_len([0.3, 0.2, 0.9], [0.3, 0.1, 0.95], [0.99, 0.5, 0.5]) == 3
    assert P.rejection_accept_len([0.3, 0.2, 0.9], [0.3, 0.9, 0.95], [0.2, 0.5, 0.0]) == 1


def test_rejection_accept_probability_is_min_one_p_over_q():
    """The rule accepts a draft with probability min(1, p/q) over uniform u
    (the rejection-sampling identity), checked on a fine uniform grid."""
    u = (np.arange(100000) + 0.5) / 100000
    for p, q in ((0.2, 0.5), (0.5, 0.2), (0.3, 0.3), (0.01, 0.9)):
        rate = np.mean([P.rejection_accept_len([p], [q], [x]) for x in u])
        assert abs(rate - min(1.0, p / q)) < 2e-5


# ------------------------------------------------------ confidence windows --
def test_confidence_vt_closed_form():
    """Equal scores: S_k = s^(k+1), so kept = floor(ln tau / ln s)."""
    for x, tau in ((2.0, 0.5), (0.5, 0.3), (3.0, 0.9), (-1.0, 0.05)):
        s = P.sigmoid(x)
        kept = min(15, math.floor(math.log(tau) / math.log(s) + 1e-12))
        assert P.confidence_vt([x] * 15, tau, 16) == max(2, min(1 + kept, 16))
    assert P.confidence_vt([9.0] * 15, 0.0, 8) == 8                   # clamped to vt_cap
    assert P.confidence_vt([-9.0] * 15, 0.5, 16) == 2                 # floor of 2: one draft always rides
    assert P.confidence_vt([], 0.5, 16) == 2


def test_slot_confidence_vt_stops_at_first_low_slot():
    hi, lo = 3.0, -3.0
    assert P.slot_confidence_vt([hi, hi, lo, hi, hi], 0.5, 16) == 3   # 2 kept: the high tail after a low slot is dropped
    assert P.slot_confidence_vt([hi] * 5, 0.5, 16) == 6
    assert P.slot_confidence_vt([lo, hi], 0.5, 16) == 2
    # per-slot marginal vs cumulative survival: survival drops below tau first
    raws = [1.0] * 10                                                  # sigmoid 0.731
    assert P.slot_confidence_vt(raws, 0.5, 16) == 11
    assert P.confidence_vt(raws, 0.5, 16) == 1 + 2                     # 0.731^2 = 0.534 >= 0.5 > 0.731^3


def test_sigmoid_matches_definition():
    for x in (-40.0, -3.0, 0.0, 0.7, 25.0):
        assert abs(P.sigmoid(x) - 1.0 / (1.0 + math.exp(-x))) < 1e-15


# -------------------------------------------------------- selector walks --
def _selector_inputs(seed=5, vocab=50, rank=8, k=6, nd=7):
    rng = np.random.default_rng(seed)
    pred = synth.encode_bf16(rng.standard_normal((vocab, rank)).astype(np.float32))
    succ = synth.encode_bf16(rng.standard_normal((vocab, rank)).astype(np.float32))
    cand = np.stack([rng.choice(vocab, k, replace=False) for _ in range(nd)]).astype(np.int32)
    unary = np.sort(rng.standard_normal((nd, k)).astype(np.float32), axis=1)[:, ::-1].copy()
    hproj = rng.standard_normal((nd, rank)).astype(np.float32)
    return pred, succ, cand, unary, hproj


def _dec(cb):
    from oracle.dflash_oracle import decode_bf16
    return decode_bf16(cb)


def test_topk_rows_brute_force():
    rng = np.random.default_rng(1)
    x = rng.integers(-3, 4, size=(5, 12)).astype(np.float32)      # many ties
    vals, idx = P.topk_rows(x, 5)
    for r in range(5):
        want = sorted(range(12), key=lambda i: (-x[r, i], i))[:5]
        assert list(idx[r]) == want
        assert list(vals[r]) == [x[r, i] for i in want]


def test_walk_greedy_pins():
    pred, succ, cand, unary, hproj = _selector_inputs()
    P_, S_ = _dec(pred), _dec(succ)
    # zero pair term (hproj = 0): every slot takes its best unary, i.e. k = 0
    assert P.walk_greedy(unary, cand, np.zeros_like(hproj), P_, S_, 3) == list(cand[:, 0])
    # equal unary and zero pair term: a tie everywhere resolves to the lowest k
    assert P.walk_greedy(np.zeros_like(unary), cand, np.zeros_like(hproj), P_, S_, 3) == list(cand[:, 0])
    # the chain: slot p's scores use the token chosen at slot p-1
    path = P.walk_greedy(unary, cand, hproj, P_, S_, 3)
    prev = 3
    for p in range(len(path)):
        sc = [float(unary[p, k]) + float(np.dot(P_[prev] * hproj[p], S_[cand[p, k]])) for k in range(cand.shape[1])]
        assert path[p] == cand[p, int(np.argmax(sc))]
        prev = path[p]


def test_walk_sampled_pins():
    pred, succ, cand, unary, hproj = _selector_inputs()
    P_, S_ = _dec(pred), _dec(succ)
    nd, k = cand.shape
    u = np.random.default_rng(2).random(nd)
    path, qc, qr = P.walk_sampled(unary, cand, hproj, P_, S_, 3, 0.7, u)
    qr = np.asarray(qr).reshape(nd, k)
    assert np.allclose(qr.sum(axis=1), 1.0, atol=1e-12)
    for p in range(nd):
        chosen = list(cand[p]).index(path[p])
        assert qc[p] == qr[p, chosen]
    # T -> 0 gives the greedy walk; u = 0 picks the first candidate with any mass
    assert P.walk_sampled(unary, cand, hproj, P_, S_, 3, 1e-9, u)[0] == P.walk_greedy(unary, cand, hproj, P_, S_, 3)
    path0 = P.walk_sampled(unary, cand, hproj, P_, S_, 3, 1e9, np.zeros(nd))[0]
    assert path0 == list(cand[:, 0])
    # frequencies over a uniform grid of u reproduce q for the first slot
    grid = (np.arange(20000) + 0.5) / 20000
    first = [P.walk_sampled(unary[:1], cand[:1], hproj[:1], P_, S_, 3, 0.7, [x])[0][0] for x in grid]
    freq = np.array([np.mean(np.array(first) == c) for c in cand[0]])
    assert np.abs(freq - qr[0]).max() < 1e-3


# --------------------------------------------- library == oracle (C ABI) --
def test_library_accept_and_windows_match_oracle(D):
    rng = np.random.default_rng(9)
    for _ in range(300):
        nd = int(rng.integers(0, 16))
        cand = rng.integers(0, 3, nd + 1).tolist()
        vam = rng.integers(0, 3, int(rng.integers(1, 18))).tolist()
        assert D.dflash_accept_prefix(cand, vam) == P.accept_prefix(cand, vam)
        p, q, u = rng.random(nd), rng.random(nd), rng.random(nd)
        assert D.dflash_rejection_accept_len(p, q, u) == P.rejection_accept_len(p, q, u)
        raws = (rng.standard_normal(nd) * 3).astype(np.float32)
        tau, cap = float(rng.random()), int(rng.integers(2, 20))
        assert D.dflash_confidence_vt(raws, tau, cap) == P.confidence_vt(raws, tau, cap)
        assert D.dflash_slot_confidence_vt(raws, tau, cap) == P.slot_confidence_vt(raws, tau, cap)
    assert D.dflash_rejection_accept_len([0.5], [1.0], [0.5]) == 0


def test_library_rejects_bad_arguments(D):
    with pytest.raises(D.DflashError):
        D.dflash_confidence_vt([1.0], 0.5, 1)
    with pytest.raises(D.DflashError):
        D.dflash_accept_prefix([1], [])


def test_library_walks_match_oracle(D):
    for seed in range(6):
        pred, succ, cand, unary, hproj = _selector_inputs(seed=seed, k=8 if seed % 2 else 5)
        P_, S_ = _dec(pred), _dec(succ)
        sel = D.make_selector(pred, succ, cand.shape[1])
        anchor = seed + 1
        assert D.dflash2_walk_greedy(sel, unary, cand, hproj, anchor) == \
            P.walk_greedy(unary, cand, hproj, P_, S_, anchor)
        u = np.random.default_rng(seed + 100).random(cand.shape[0])
        g = D.dflash2_walk_sampled(sel, unary, cand, hproj, anchor, 0.8, u)
        o = P.walk_sampled(unary, cand, hproj, P_, S_, anchor, 0.8, u)
        assert g[0] == o[0]
        assert np.array_equal(np.asarray(g[1]), np.asarray(o[1]))
        assert np.array_equal(np.asarray(g[2]), np.asarray(o[2]))
    # an out-of-vocabulary candidate is an argument error
    cand[0, 0] = 10 ** 6
    with pytest.raises(D.DflashError):
        D.dflash2_walk_greedy(sel, unary, cand, hproj, 1)
