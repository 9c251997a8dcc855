"""Pins of the oracle's two capacity variants (Capacity-Aware Inference summary, Methodology:
Expanded Drop and the device-level variant), independent of the oracle's own code paths:
hand-derived examples, reductions to the token drop, brute-force subset dominance on tiny
inputs, and invariants."""
import itertools
import json
import os

import numpy as np
import pytest

import oracle
import moe_inputs as mi

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_expanded_group_examples.json")


def _p32(logits):
    return oracle.routing_score32(np.asarray(logits, dtype=np.float32))


@pytest.mark.parametrize("ex", json.load(open(GOLDEN))["expanded_drop"])
def test_expanded_drop_hand_examples(ex):
    l = np.asarray(ex["logits"], dtype=np.float32)
    k, m = ex["k"], ex["m"]
    T, E = l.shape
    assert oracle.capacity(T, k, E, ex["gamma"]) == ex["C"]
    ids = oracle.topk_select(l, k + m)
    assert ids.tolist() == ex["ids_ext"]
    kept = oracle.expanded_drop(ids, _p32(l), ex["C"], k)
    assert kept.tolist() == ex["kept"]
    g = oracle.expanded_gates(l, ids, k)
    for key, w in ex.get("weights_of_kept", {}).items():
        t, j = map(int, key.split(","))
        assert abs(g[t, j] - w) < 1e-12


@pytest.mark.parametrize("ex", json.load(open(GOLDEN))["group_capacity"])
def test_group_capacity_hand_examples(ex):
    l = np.asarray(ex["logits"], dtype=np.float32)
    T, E = l.shape
    assert oracle.group_capacity(T, ex["k"], ex["D"], ex["gamma"]) == ex["C_D"]
    ids = oracle.topk_select(l, ex["k"])
    assert ids.tolist() == ex["ids"]
    kept = oracle.group_capacity_drop(ids, _p32(l), ex["C_D"], E, ex["D"])
    assert kept.tolist() == ex["kept"]


def _random_logits(rng, T, E, levels=None):
    if levels:
        return mi.quantised_logits(T, E, levels, int(rng.integers(1 << 30)))
    return rng.normal(size=(T, E)).astype(np.float32)


@pytest.mark.parametrize("seed,levels", [(0, None), (1, 3), (2, 2)])
def test_expanded_with_no_extra_candidates_is_the_token_drop(seed, levels):
    rng = np.random.default_rng(seed)
    l = _random_logits(rng, 200, 8, levels)
    ids = oracle.topk_select(l, 2)
    p = _p32(l)
    for C in (0, 10, 37, 50, 400):
        assert (oracle.expanded_drop(ids, p, C, 2) == oracle.capacity_drop(ids, p, C, 8)).all()


@pytest.mark.parametrize("seed,levels", [(0, None), (3, 3)])
def test_groups_of_one_expert_are_the_token_drop(seed, levels):
    rng = np.random.default_rng(seed)
    T, E, k, gamma = 300, 16, 4, 0.8
    l = _random_logits(rng, T, E, levels)
    ids = oracle.topk_select(l, k)
    p = _p32(l)
    C = oracle.capacity(T, k, E, gamma)
    assert oracle.group_capacity(T, k, E, gamma) == C
    assert (oracle.group_capacity_drop(ids, p, C, E, E) == oracle.capacity_drop(ids, p, C, E)).all()


def _rank_key(p, t, j, e):
    # strict priority of a pair: higher p32, then lower token, then lower slot
    return (-float(p[t, e]), t, j)


@pytest.mark.parametrize("seed", range(6))
def test_group_capacity_brute_force(seed):
    """Per group, the kept set is the one subset of size min(n, C_D) whose every member
    outranks every non-member; found by enumerating all subsets."""
    rng = np.random.default_rng(100 + seed)
    T, E, k, D = 5, 4, 2, 2
    l = _random_logits(rng, T, E, 2 if seed % 2 else None)
    ids = oracle.topk_select(l, k)
    p = _p32(l)
    C_D = int(rng.integers(0, 4))
    kept = oracle.group_capacity_drop(ids, p, C_D, E, D)
    gs = E // D
    for g in range(D):
        pairs = [(t, j) for t in range(T) for j in range(k) if ids[t, j] // gs == g]
        want = min(len(pairs), C_D)
        ok = []
        for sub in itertools.combinations(pairs, want):
            rest = [q for q in pairs if q not in sub]
            if all(_rank_key(p, *a, ids[a]) < _rank_key(p, *b, ids[b]) for a in sub for b in rest):
                ok.append(set(sub))
        assert len(ok) == 1
        got = {(t, j) for (t, j) in pairs if kept[t, j]}
        assert got == ok[0]


@pytest.mark.parametrize("seed,levels", [(0, None), (1, 3), (2, None), (4, 2)])
def test_expanded_drop_invariants(seed, levels):
    rng = np.random.default_rng(seed)
    T, E, k, m, gamma = 400, 8, 2, 2, 0.9
    l = _random_logits(rng, T, E, levels)
    # a skewed router: the straggler case the variant is for
    l = (l + np.array([-1.2 * np.log(e + 1.0) for e in range(E)], dtype=np.float32)).astype(np.float32)
    ids = oracle.topk_select(l, k + m)
    p = _p32(l)
    C = oracle.capacity(T, k, E, gamma)
    kept = oracle.expanded_drop(ids, p, C, k)
    base = oracle.capacity_drop(ids[:, :k], p, C, E)
    # the top-k decisions are those of the token drop
    assert (kept[:, :k] == base).all()
    lost = k - base.sum(axis=1)
    extra = kept[:, k:].sum(axis=1)
    # a token takes extra experts only in place of lost picks, never more than k in all
    assert (extra <= lost).all()
    assert (kept.sum(axis=1) <= k).all()
    # no expert goes past its capacity
    for e in range(E):
        assert np.count_nonzero((ids == e) & (kept == 1)) <= C
    # the variant re-homes at least some dropped pairs on this skewed router
    assert extra.sum() > 0
    # an extra pair kept at expert e outranks every pair offered to e and not admitted
    # while e still had room at the end (room left means nobody was turned away)
    for e in range(E):
        used = np.count_nonzero((ids == e) & (kept == 1))
        offered = [(t, j) for t, j in zip(*np.nonzero(ids[:, k:] == e)) if lost[t] > 0]
        refused = [(t, j + k) for (t, j) in offered if not kept[t, j + k]]
        taken = [(t, j + k) for (t, j) in offered if kept[t, j + k]]
        for (t, j) in refused:
            fully_served = extra[t] == lost[t]
            if not fully_served:
                # refused although the token still needed a place: e had no room for it
                assert used == C or all(
                    _rank_key(p, a, b, e) < _rank_key(p, t, j, e) for (a, b) in taken)


def test_expanded_gates_scale():
    l = np.array([[2.0, 1.0, 0.5, -1.0]], dtype=np.float32)
    ids = oracle.topk_select(l, 3)
    g = oracle.expanded_gates(l, ids, 2)
    # top-k gates sum to 1, the extra candidate is its probability over the same mass
    assert abs(g[0, :2].sum() - 1.0) < 1e-12
    assert abs(g[0, 2] - np.exp(0.5 - 2.0) / (1.0 + np.exp(-1.0))) < 1e-12
    g0 = oracle.expanded_gates(l, ids, 2, renorm=False)
    assert abs(g0[0].sum() - oracle.softmax_rows(l)[0, ids[0]].sum()) < 1e-12


def test_route_with_variants_keeps_at_most_k_rows_per_token():
    rng = np.random.default_rng(7)
    T, E, k = 256, 16, 2
    l = (rng.normal(size=(T, E)) + np.linspace(2, -2, E)).astype(np.float32)
    for kw in (dict(expand_m=2, gamma=0.8), dict(cap_groups=4, gamma=0.8), dict(cap_groups=1, gamma=0.5)):
        cfg = mi.TINY.with_(T=T, E=E, k=k, **kw)
        r = oracle.route(cfg, logits=l)
        per_tok = np.diff(r["tok_ptr"])
        assert per_tok.max() <= k
        assert r["offsets"][-1] == per_tok.sum() == r["kept"].sum()
        # each row's weight is the gate of its (token, slot)
        tt, jj = np.nonzero(r["kept"])
        w = {(int(t), int(r["ids"][t, j])): r["gates"][t, j] for t, j in zip(tt, jj)}
        for p in range(int(r["offsets"][-1])):
            e = int(np.searchsorted(r["offsets"], p, side="right") - 1)
            assert abs(r["perm_w"][p] - w[(int(r["perm_token"][p]), e)]) == 0.0


def test_route_rejects_inconsistent_variants():
    l = np.zeros((8, 4), dtype=np.float32)
    base = mi.TINY.with_(T=8, E=4, k=2)
    for kw in (dict(expand_m=1), dict(cap_groups=2), dict(expand_m=1, cap_groups=2, gamma=1.0),
               dict(expand_m=3, gamma=1.0), dict(cap_groups=3, gamma=1.0)):
        with pytest.raises(ValueError):
            oracle.route(base.with_(**kw), logits=l)
