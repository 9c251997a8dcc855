"""Pins of the oracle's layer output y = sum_i G(x)_i E_i(x) (dongbusteel page, the
gate-weighted expert sum) against independent evaluations. CPU only.

- a dense evaluation of the definition through torch.nn.functional (every expert
  on every token, gate matrix with zeros for unselected pairs), not through the
  oracle's dispatch;
- E = k = 1 reduces to a textbook SwiGLU FFN;
- linearity in W_down, expert relabelling and token-permutation symmetries;
- the shared expert adds a weight-1 path for every token (routing/active-parameter
  page, routing section).
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import moe_inputs as mi
import oracle


def _t(a):
    return torch.from_numpy(np.asarray(mi.bf16_to_f32(a) if a.dtype == np.uint16 else a,
                                       dtype=np.float64))


def _dense_gate(cfg, r):
    G = np.zeros((cfg.T, cfg.E))
    if cfg.routing == "expert":
        G[r["sel"]] = r["sel_w"][r["sel"]]
    else:
        for t in range(cfg.T):
            for j in range(cfg.k):
                if r["kept"][t, j]:
                    G[t, r["ids"][t, j]] = r["gates"][t, j]
    return torch.from_numpy(G)


def _dense_y(inp, r):
    cfg = inp.cfg
    X = _t(inp.x)
    G = _dense_gate(cfg, r)
    y = torch.zeros(cfg.T, cfg.d_model, dtype=torch.float64)
    for e in range(cfg.E):
        h = F.silu(F.linear(X, _t(inp.w_gate[e]))) * F.linear(X, _t(inp.w_up[e]))
        y += G[:, e:e + 1] * F.linear(h, _t(inp.w_down[e]))
    if cfg.d_ff_shared:
        h = F.silu(F.linear(X, _t(inp.ws_gate))) * F.linear(X, _t(inp.ws_up))
        y += F.linear(h, _t(inp.ws_down))
    return y.numpy()


SMALL = [
    mi.TINY,
    mi.TINY.with_(gamma=0.75, bias=("zipf", 1.2)),
    mi.TINY.with_(routing="expert", T=40),
    mi.TINY.with_(dtype="bf16", E=16, k=4, T=48, d_model=64, d_ff=96, d_ff_shared=32,
                        gamma=1.25, bias=("normal", 1.0)),
    mi.TINY.with_(renorm_topk=False, k=3),
]


@pytest.mark.parametrize("cfg", SMALL, ids=lambda c: f"{c.routing}-g{c.gamma}-E{c.E}k{c.k}-{c.dtype}")
def test_layer_equals_dense_definition(cfg):
    inp = mi.make_inputs(cfg)
    y, r = oracle.layer_forward(inp)
    yd = _dense_y(inp, r)
    np.testing.assert_allclose(y, yd, rtol=1e-10, atol=1e-12)


def test_single_expert_is_textbook_swiglu():
    cfg = mi.TINY.with_(E=1, k=1)
    inp = mi.make_inputs(cfg)
    y, r = oracle.layer_forward(inp)
    X = _t(inp.x)
    ref = F.linear(F.silu(F.linear(X, _t(inp.w_gate[0]))) * F.linear(X, _t(inp.w_up[0])),
                   _t(inp.w_down[0]))
    assert (r["counts"] == [cfg.T]).all()
    np.testing.assert_allclose(y, ref.numpy(), rtol=1e-12, atol=1e-13)


def test_linearity_in_w_down_and_zero():
    cfg = mi.TINY.with_(gamma=1.0)
    inp = mi.make_inputs(cfg)
    y, _ = oracle.layer_forward(inp)
    inp.w_down = inp.w_down * np.float32(2.0)
    y2, _ = oracle.layer_forward(inp)
    np.testing.assert_allclose(y2, 2.0 * y, rtol=1e-13, atol=1e-14)
    inp.w_down = np.zeros_like(inp.w_down)
    y0, _ = oracle.layer_forward(inp)
    assert np.abs(y0).max() == 0.0


def test_expert_relabelling_invariance():
    cfg = mi.TINY
    inp = mi.make_inputs(cfg)
    y, _ = oracle.layer_forward(inp)
    perm = np.random.default_rng(0).permutation(cfg.E)
    inp.w_router = inp.w_router[:, perm].copy()
    inp.w_gate, inp.w_up, inp.w_down = inp.w_gate[perm], inp.w_up[perm], inp.w_down[perm]
    y2, _ = oracle.layer_forward(inp)
    np.testing.assert_allclose(y2, y, rtol=1e-12, atol=1e-13)


def test_token_permutation_equivariance():
    cfg = mi.TINY
    inp = mi.make_inputs(cfg)
    y, _ = oracle.layer_forward(inp)
    perm = np.random.default_rng(1).permutation(cfg.T)
    inp.x = inp.x[perm].copy()
    y2, _ = oracle.layer_forward(inp)
    np.testing.assert_allclose(y2, y[perm], rtol=1e-12, atol=1e-13)


def test_sampled_tokens_equal_full_rows():
    cfg = mi.TINY.with_(gamma=0.75, bias=("zipf", 1.2), d_ff_shared=64)
    inp = mi.make_inputs(cfg)
    y, r = oracle.layer_forward(inp)
    toks = np.array([0, 5, 17, 63, 31])
    ys, _ = oracle.layer_forward(inp, tokens=toks, routing=r)
    np.testing.assert_allclose(ys, y[toks], rtol=1e-12, atol=1e-14)   # BLAS blocking may differ


def test_dropped_everywhere_gives_shared_only():
    cfg = mi.TINY.with_(gamma=1e-6, d_ff_shared=64)
    inp = mi.make_inputs(cfg)
    y, r = oracle.layer_forward(inp)
    assert r["C"] == 0
    np.testing.assert_allclose(y, oracle.shared_expert(inp), rtol=1e-12, atol=1e-14)


def test_logits_closed_form():
    """l = x W_r + b, one rounding of the exact product (bf16 x times fp32 W is exact in
    fp64 per term; sum of d terms in fp64 is far inside fp32 rounding)."""
    cfg = mi.MIXTRAL.with_(T=16, d_model=256, d_ff=64)
    inp = mi.make_inputs(cfg)
    l = oracle.router_logits(inp.x, inp.w_router, inp.bias)
    X = torch.from_numpy(mi.bf16_to_f32(inp.x).astype(np.float64))
    ref = (X @ torch.from_numpy(inp.w_router.astype(np.float64))
           + torch.from_numpy(inp.bias.astype(np.float64))).to(torch.float32).numpy()
    assert (l == ref).all()
