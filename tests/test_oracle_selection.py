"""Pins of the oracle's selection and dispatch steps against brute force, library
routines and the invariants the source pages fix. CPU only.

- Token choice picks top-k (dongbusteel page, TopK(G(x), k); hrletsgo page, basic
  MoE structure: Mixtral always picks 2 of 8).
- Expert choice: every expert takes exactly c = k*T/N tokens and a token may get
  0..N experts (hrletsgo page, Mixture-of-Tokens section).
- Capacity drop: no expert keeps more than C = gamma*N-bar tokens and the dropped
  ones are those with the lowest gating score (Capacity-Aware Inference summary,
  Methodology, Token Drop).
"""
import itertools
import json
import os

import numpy as np
import pytest
import scipy.special

import moe_inputs as mi
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _dominates(key_a, idx_a, key_b, idx_b):
    """(key desc, index asc) order: a strictly before b."""
    return key_a > key_b or (key_a == key_b and idx_a < idx_b)


def _brute_best_subset(keys, size):
    """The unique subset of `size` indices such that every member precedes every
    non-member under (key desc, index asc), found by enumerating all subsets."""
    n = len(keys)
    found = []
    for S in itertools.combinations(range(n), size):
        rest = [j for j in range(n) if j not in S]
        if all(_dominates(keys[a], a, keys[b], b) for a in S for b in rest):
            found.append(set(S))
    assert len(found) == 1
    return found[0]


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("E,k", [(4, 1), (5, 2), (6, 3), (6, 6)])
def test_topk_matches_brute_force(seed, E, k):
    l = mi.quantised_logits(12, E, levels=3, seed=seed)
    ids = oracle.topk_select(l, k)
    for t in range(l.shape[0]):
        best = _brute_best_subset(list(l[t]), k)
        assert set(ids[t].tolist()) == best
        # slots in descending key order, ties by lower index
        for j in range(k - 1):
            a, b = ids[t, j], ids[t, j + 1]
            assert _dominates(l[t, a], a, l[t, b], b)


@pytest.mark.parametrize("seed", range(5))
@pytest.mark.parametrize("T,E,k", [(8, 2, 1), (9, 3, 2), (10, 4, 2), (6, 3, 3)])
def test_expert_choice_matches_brute_force(seed, T, E, k):
    l = mi.quantised_logits(T, E, levels=3, seed=seed + 10)
    sel, w = oracle.expert_choice_select(l, k)
    c = (k * T) // E
    for e in range(E):
        best = _brute_best_subset(list(l[:, e]), c)
        assert set(np.nonzero(sel[:, e])[0].tolist()) == best
    # weights: softmax over the tokens of each column (library softmax), zero elsewhere
    s = scipy.special.softmax(l.astype(np.float64), axis=0)
    np.testing.assert_allclose(w, np.where(sel, s, 0.0), rtol=1e-13, atol=0)


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("T,E,k,gamma", [(9, 2, 1, 1.0), (10, 3, 2, 1.0), (10, 4, 2, 0.75),
                                         (8, 3, 2, 1.25)])
def test_capacity_drop_matches_brute_force(seed, T, E, k, gamma):
    l = mi.quantised_logits(T, E, levels=3, seed=seed + 20)
    # skew the router so that some experts overflow
    l = (l + np.array([1.5] + [0.0] * (E - 1), dtype=np.float32)[None, :]).astype(np.float32)
    ids = oracle.topk_select(l, k)
    p32 = oracle.routing_score32(l)
    C = oracle.capacity(T, k, E, gamma)
    kept = oracle.capacity_drop(ids, p32, C, E)
    for e in range(E):
        cand = [t for t in range(T) if e in ids[t]]
        keys = [p32[t, e] for t in cand]
        kept_e = {i for i, t in enumerate(cand) if kept[t, list(ids[t]).index(e)]}
        if len(cand) <= C:
            assert kept_e == set(range(len(cand)))
        else:
            assert kept_e == _brute_best_subset(keys, C)


@pytest.mark.parametrize("seed", range(8))
def test_selection_invariants_random_shapes(seed):
    rng = np.random.default_rng(seed)
    T = int(rng.integers(1, 300))
    E = int(rng.integers(1, 17))
    k = int(rng.integers(1, E + 1))
    l = mi.quantised_logits(T, E, levels=4, seed=seed + 30)
    ids = oracle.topk_select(l, k)
    # exactly k distinct experts per token
    assert ids.shape == (T, k)
    assert all(len(set(r.tolist())) == k for r in ids)
    # expert choice: exactly c per expert, sum = E*c, a token gets 0..E experts
    if k * T >= E:
        sel, _ = oracle.expert_choice_select(l, k)
        c = (k * T) // E
        assert (sel.sum(axis=0) == c).all() and sel.sum() == E * c
        per_tok = sel.sum(axis=1)
        assert per_tok.min() >= 0 and per_tok.max() <= E
    # capacity: counts <= C, dominance (min kept key >= max dropped key, ties to lower token)
    gamma = float(rng.choice([0.5, 1.0, 1.25]))
    C = oracle.capacity(T, k, E, gamma)
    p32 = oracle.routing_score32(l)
    kept = oracle.capacity_drop(ids, p32, C, E)
    for e in range(E):
        tt, jj = np.nonzero(ids == e)
        kk = kept[tt, jj] == 1
        assert kk.sum() == min(len(tt), C)
        if kk.any() and (~kk).any():
            kmin = p32[tt[kk], e].min()
            dmax = p32[tt[~kk], e].max()
            assert kmin >= dmax
            if kmin == dmax:     # equal keys: every kept one at that key precedes every dropped one
                assert tt[kk][p32[tt[kk], e] == kmin].max() < tt[~kk][p32[tt[~kk], e] == dmax].min()


def _dispatch_by_loop(pairs, T, E):
    """Counting sort written as plain loops: per expert, the pairs in the given order."""
    counts = [0] * E
    for _, e, _ in pairs:
        counts[e] += 1
    offsets = [0]
    for e in range(E):
        offsets.append(offsets[-1] + counts[e])
    fill = offsets[:-1].copy()
    perm_token = [0] * len(pairs)
    pos = [0] * len(pairs)
    for i, (t, e, _) in enumerate(pairs):
        perm_token[fill[e]] = t
        pos[i] = fill[e]
        fill[e] += 1
    return counts, offsets, perm_token, pos


@pytest.mark.parametrize("overrides", [{}, dict(gamma=0.75), dict(routing="expert"),
                                       dict(E=5, k=3, T=37, gamma=1.0)])
def test_dispatch_is_stable_counting_sort(overrides):
    cfg = mi.TINY.with_(**overrides)
    l = mi.quantised_logits(cfg.T, cfg.E, levels=5, seed=7)
    r = oracle.route(cfg, logits=l)
    if cfg.routing == "expert":
        tt, ee = np.nonzero(r["sel"])
    else:
        tt, jj = np.nonzero(r["kept"])
        ee = r["ids"][tt, jj]
    pairs = list(zip(tt.tolist(), ee.tolist(), [0] * len(tt)))
    counts, offsets, perm_token, pos = _dispatch_by_loop(pairs, cfg.T, cfg.E)
    assert r["counts"].tolist() == counts
    assert r["offsets"].tolist() == offsets
    assert r["perm_token"].tolist() == perm_token
    assert r["tok_pos"].tolist() == pos
    # CSR: token t's rows, in pair order; a bijection onto the rows
    assert sorted(r["tok_pos"].tolist()) == list(range(len(pairs)))
    for t in range(cfg.T):
        rows = r["tok_pos"][r["tok_ptr"][t]:r["tok_ptr"][t + 1]]
        assert all(r["perm_token"][p] == t for p in rows)


def test_gates_closed_forms():
    l = mi.normal_logits(50, 6, seed=3)
    # k = E with renormalisation: the gates are the dense softmax
    ids = oracle.topk_select(l, 6)
    g = oracle.topk_gates(l, ids, renorm=True)
    p = scipy.special.softmax(l.astype(np.float64), axis=1)
    np.testing.assert_allclose(g, np.take_along_axis(p, ids.astype(np.int64), 1), rtol=1e-13)
    # renormalised gates sum to 1; they equal the softmax over the selected logits
    ids2 = oracle.topk_select(l, 2)
    g2 = oracle.topk_gates(l, ids2, renorm=True)
    np.testing.assert_allclose(g2.sum(1), 1.0, rtol=1e-14)
    sel = np.take_along_axis(l.astype(np.float64), ids2.astype(np.int64), 1)
    np.testing.assert_allclose(g2, scipy.special.softmax(sel, axis=1), rtol=1e-13)
    # without renormalisation: the full-softmax probabilities
    g3 = oracle.topk_gates(l, ids2, renorm=False)
    np.testing.assert_allclose(g3, np.take_along_axis(p, ids2.astype(np.int64), 1), rtol=1e-13)


def test_capacity_special_cases():
    cfg = mi.TINY.with_(gamma=0.0)
    l = mi.normal_logits(cfg.T, cfg.E, seed=4, bias=np.linspace(2, -2, cfg.E).astype(np.float32))
    nodrop = oracle.route(cfg, logits=l)
    # gamma >= E/k: C >= T, identical to no drop
    big = oracle.route(cfg.with_(gamma=cfg.E / cfg.k), logits=l)
    for key in ("counts", "offsets", "perm_token", "tok_ptr", "tok_pos"):
        assert (big[key] == nodrop[key]).all()
    assert big["kept"].all()
    # C = 0: everything dropped
    tiny = oracle.route(cfg.with_(gamma=1e-6), logits=l)
    assert tiny["C"] == 0 and tiny["kept"].sum() == 0 and tiny["offsets"][-1] == 0
    assert (tiny["tok_ptr"] == 0).all()


def test_expert_choice_c_equals_T():
    l = mi.normal_logits(20, 4, seed=5)
    sel, w = oracle.expert_choice_select(l, 4)          # k = E: c = T
    assert sel.all()
    np.testing.assert_allclose(w.sum(axis=0), 1.0, rtol=1e-14)


def test_golden_hand_examples():
    with open(os.path.join(GOLDEN, "hand_routing_examples.json")) as f:
        gold = json.load(f)
    for case in gold["token_choice"]:
        l = np.array(case["logits"], dtype=np.float32)
        ids = oracle.topk_select(l, case["k"])
        assert ids.tolist() == case["ids"]
        np.testing.assert_allclose(oracle.topk_gates(l, ids, True), case["gates"], rtol=1e-9)
    for case in gold["expert_choice"]:
        l = np.array(case["logits"], dtype=np.float32)
        sel, w = oracle.expert_choice_select(l, case["k"])
        got = [sorted(np.nonzero(sel[:, e])[0].tolist()) for e in range(l.shape[1])]
        assert got == case["selected_tokens_per_expert"]
        np.testing.assert_allclose(w, case["weights"], rtol=1e-9, atol=1e-12)
    for case in gold["capacity_drop"]:
        l = np.array(case["logits"], dtype=np.float32)
        T, E = l.shape
        C = oracle.capacity(T, case["k"], E, case["gamma"])
        assert C == case["C"]
        ids = oracle.topk_select(l, case["k"])
        kept = oracle.capacity_drop(ids, oracle.routing_score32(l), C, E)
        assert kept.tolist() == case["kept"]
