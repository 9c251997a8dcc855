"""Hand-derived pins of the oracle functions that the selection goldens do not reach:
router_logits (including the bfloat16 widening and the one rounding of the exact sum),
routing_stats, combine, expert_rows_ffn and shared_expert. CPU only.

Expected values live in tests/golden/hand_oracle_pins.json, each worked out by hand from
the definitions the pages give (see that file's citation). A plausible slip in any of
these functions (a dropped bias, a float32 running sum, a transposed weight, a row mapped
to the neighbouring expert, a balance term scaled by E, a shared row added twice, a
dropped pair counted as kept) changes at least one expected value.
"""
import json
import math
import os
from fractions import Fraction
from types import SimpleNamespace

import numpy as np
import pytest

import oracle

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                     "hand_oracle_pins.json")))
LN3 = np.float32(math.log(3.0))


def _frac(s):
    return float(Fraction(s))


def _silu(z):
    return z / (1.0 + math.exp(-z))


@pytest.mark.parametrize("i", range(len(GOLDEN["router"])))
def test_router_logits_hand_examples(i):
    g = GOLDEN["router"][i]
    if "x_bf16_bits" in g:
        x = np.array(g["x_bf16_bits"], dtype=np.uint16)
    else:
        x = np.array(g["x"], dtype=np.float32)
    w = np.array(g["w_router"], dtype=np.float32)
    b = None if g["bias"] is None else np.array(g["bias"], dtype=np.float32)
    l = oracle.router_logits(x, w, b)
    assert l.dtype == np.float32
    assert (l == np.array(g["logits"], dtype=np.float32)).all(), (l, g["logits"])


def test_widen_bf16_bit_patterns():
    bits = np.array([0x3F80, 0xC000, 0x3E20, 0x4140, 0x0000, 0x8000, 0x7F7F], dtype=np.uint16)
    got = oracle.widen(bits)
    want = [1.0, -2.0, 0.15625, 12.0, 0.0, -0.0, 3.3895313892515355e38]   # 0x7F7F: largest bf16
    assert got.dtype == np.float64
    assert got.tolist() == want


def _routing_for(g):
    T, E, k = g["T"], g["E"], g["k"]
    l = np.array([[LN3 if v == "ln3" else np.float32(v) for v in row] for row in g["logits"]],
                 dtype=np.float32)
    cfg = SimpleNamespace(T=T, E=E, k=k, routing=g["routing"], gamma=g["gamma"], renorm_topk=True,
                          expand_m=0, cap_groups=0)
    return oracle.route(cfg, logits=l)


@pytest.mark.parametrize("i", range(len(GOLDEN["routing_stats"])))
def test_routing_stats_hand_examples(i):
    g = GOLDEN["routing_stats"][i]
    r = _routing_for(g)
    assert r["counts"].tolist() == g["counts"]
    s = oracle.routing_stats(r, g["E"], g["T"], g["k"])
    np.testing.assert_allclose(s["f"], [_frac(v) for v in g["f"]], rtol=0, atol=1e-15)
    # 'ln3' is the float32 nearest ln 3: softmax values hold to ~1e-7
    np.testing.assert_allclose(s["P"], [_frac(v) for v in g["P"]], rtol=0, atol=2e-7)
    assert abs(s["balance"] - _frac(g["balance"])) <= 2e-7
    assert abs(s["max_over_mean"] - _frac(g["max_over_mean"])) <= 1e-15
    assert s["dropped"] == g["dropped"]
    assert s["empty"] == g["empty"]


def test_routing_stats_balance_is_unscaled_sum():
    """The page's term is sum_i f_i P_i; for a perfectly uniform router and uniform loads it
    is 1/E (the Switch paper's extra factor E, which would make it 1, is not applied)."""
    E = 8
    l = np.zeros((E, E), dtype=np.float32)
    l[np.arange(E), np.arange(E)] = 0.0            # all logits equal: P_i = 1/E
    r = {"counts": np.full(E, 3, dtype=np.int32), "logits": l}
    s = oracle.routing_stats(r, E, E, 3)
    assert abs(s["balance"] - 1.0 / E) <= 1e-15


def test_combine_hand_example():
    g = GOLDEN["combine"]
    r = {"tok_ptr": np.array(g["tok_ptr"]), "tok_pos": np.array(g["tok_pos"]),
         "perm_w": np.array(g["perm_w"], dtype=np.float64)}
    o = np.array(g["o_rows"], dtype=np.float32)
    y = oracle.combine(o, r, g["T"])
    assert y.tolist() == g["y"]
    ys = oracle.combine(o, r, g["T"], o_shared=np.array(g["o_shared"], dtype=np.float32))
    assert ys.tolist() == g["y_shared"]


def _expert_inputs(g):
    cfg = SimpleNamespace(d_model=len(g["x_rows"][0]))
    return SimpleNamespace(cfg=cfg, w_gate=np.array(g["w_gate"], dtype=np.float32),
                           w_up=np.array(g["w_up"], dtype=np.float32),
                           w_down=np.array(g["w_down"], dtype=np.float32))


def _expected_rows(g):
    return np.array([[sum(c * _silu(z) for c, z in col) for col in row]
                     for row in g["o_silu_terms"]])


def test_expert_rows_ffn_hand_example():
    g = GOLDEN["expert_rows"]
    inp = _expert_inputs(g)
    r = {"offsets": np.array(g["offsets"])}
    x = np.array(g["x_rows"], dtype=np.float32)
    want = _expected_rows(g)
    got = oracle.expert_rows_ffn(x, r, inp, np.arange(3))
    np.testing.assert_allclose(got, want, rtol=1e-14, atol=1e-15)
    # a subset of rows, out of order: each row still goes through its own expert
    sub = oracle.expert_rows_ffn(x, r, inp, np.array([2, 0]))
    np.testing.assert_allclose(sub, want[[2, 0]], rtol=1e-14, atol=1e-15)


def test_shared_expert_hand_example():
    """The shared expert is the same SwiGLU map over every token (weight 1): with expert 0's
    weights of the hand example as the shared weights, token rows give expert 0's rows."""
    g = GOLDEN["expert_rows"]
    x = np.array(g["x_rows"][:2], dtype=np.float32)
    inp = SimpleNamespace(cfg=SimpleNamespace(T=2), x=x,
                          ws_gate=np.array(g["w_gate"][0], dtype=np.float32),
                          ws_up=np.array(g["w_up"][0], dtype=np.float32),
                          ws_down=np.array(g["w_down"][0], dtype=np.float32))
    np.testing.assert_allclose(oracle.shared_expert(inp), _expected_rows(g)[:2], rtol=1e-14,
                               atol=1e-15)
    np.testing.assert_allclose(oracle.shared_expert(inp, tokens=np.array([1])),
                               _expected_rows(g)[1:2], rtol=1e-14, atol=1e-15)


def test_combine_of_expert_rows_equals_layer():
    """Two separate oracle routes to y agree: the per-row expert outputs (expert_rows_ffn)
    combined with the routing weights (combine) equal layer_forward's per-token evaluation."""
    import moe_inputs as mi
    for cfg in (mi.TINY.with_(gamma=0.75, bias=("zipf", 1.2), d_ff_shared=64),
                mi.TINY.with_(routing="expert", T=40)):
        inp = mi.make_inputs(cfg)
        y, r = oracle.layer_forward(inp)
        N = int(r["offsets"][-1])
        o = oracle.expert_rows_ffn(inp.x[r["perm_token"]], r, inp, np.arange(N))
        o_sh = oracle.shared_expert(inp) if cfg.d_ff_shared else None
        y2 = oracle.combine(o, r, cfg.T, o_shared=o_sh)
        np.testing.assert_allclose(y2, y, rtol=1e-12, atol=1e-13)
