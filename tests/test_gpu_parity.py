"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Bars (written here, applied below):
  - float32 logits within 1e-5 absolute of the oracle's (one rounding of the exact sum);
  - with the oracle's logits fed in (MOE_ROUTE_LOGITS_IN): every routing decision,
    count, offset, permutation index and CSR entry bit-identical; gates and combine
    weights within 1e-6 relative (float32 exp and division);
  - layer output: max|dy| <= 2e-2 * RMS for bf16 arithmetic (1e-4 for float32 arithmetic),
    per token (each token's output RMS) always and over the whole output for token choice
    with a float32 output; a bf16 output is additionally allowed its own rounding (half an
    ulp per element) and must equal the rounding of the float32 output bit for bit;
  - dispatch gather: bit-identical rows.
Sizes: small shapes that span several tiles with ragged tails and the degenerate cases
of each selection form; capacity buckets past each of the selection kernel's size paths;
the named workloads at full size, every token compared.
"""
import numpy as np
import pytest

import moe_inputs as mi
import oracle
from gpu_support import (check_y, dev_weights, host_f32, inputs_for, rel_err, run_layer,
                         run_route, run_steps, say, tol_for)

pytestmark = pytest.mark.gpu

C0 = mi.TINY
SMALL = {
    "cfg0-fp32": C0,
    "ragged-bf16": C0.with_(dtype="bf16", T=300, d_model=256, d_ff=320, bias=("normal", 0.5)),
    "drop-E16-bf16": C0.with_(dtype="bf16", T=200, d_model=128, E=16, k=4, d_ff=192, gamma=1.0,
                              bias=("zipf", 1.2)),
    "fine-shared-bf16": C0.with_(dtype="bf16", T=333, d_model=192, E=128, k=8, d_ff=128,
                                 d_ff_shared=64, gamma=1.25, bias=("normal", 1.0)),
    # 200 experts (padded to 256): the 128-token x 64-expert router on four expert groups, with
    # enough K steps (d_model 1024) for its steady-state copy waits
    "wide-E200-bf16": C0.with_(dtype="bf16", T=333, d_model=1024, E=200, k=6, d_ff=64,
                               gamma=1.25, bias=("normal", 1.0)),
    "expert-choice-bf16": C0.with_(dtype="bf16", T=1000, routing="expert"),
    "expert-choice-bf16-yf32": C0.with_(dtype="bf16", y_dtype="f32", T=1000, routing="expert"),
    "ragged-bf16-yf32": C0.with_(dtype="bf16", y_dtype="f32", T=300, d_model=256, d_ff=320,
                                 bias=("normal", 0.5)),
    "expert-choice-fp32": C0.with_(T=100, d_model=64, E=6, k=3, d_ff=96, routing="expert"),
    "single-expert-bf16": C0.with_(dtype="bf16", T=257, d_model=64, E=1, k=1, d_ff=64),
    "one-token-bf16": C0.with_(dtype="bf16", T=1, d_model=64, d_ff=64),
    "all-dropped-shared-bf16": C0.with_(dtype="bf16", T=96, d_model=64, d_ff=64, d_ff_shared=64,
                                        gamma=1e-6),
    # routing collapse onto one expert: few tiles on a wide grid, so the grouped GEMMs cut
    # each tile's K range into 2 to 8 parts summed in order by a second kernel
    "collapse-ksplit-bf16": C0.with_(dtype="bf16", T=300, d_model=2048, E=32, k=1, d_ff=256,
                                     bias=("onehot", 30.0)),
    "collapse-ksplit-shared-bf16": C0.with_(dtype="bf16", T=200, d_model=1024, E=32, k=1,
                                            d_ff=512, d_ff_shared=512, bias=("onehot", 30.0)),
    # decode-shaped batches (at most 64 rows per expert): the skinny GEMM path, its K
    # parts summed by the reduction kernel; 32-row and 64-row tiles, with a shared expert
    # whose K differs from the routed experts'
    "decode-T8-bf16": C0.with_(dtype="bf16", T=8, d_model=512, E=8, k=2, d_ff=1024),
    "decode-T48-shared-bf16": C0.with_(dtype="bf16", T=48, d_model=256, E=16, k=1, d_ff=512,
                                       d_ff_shared=256, gamma=1.0, bias=("zipf", 1.2)),
    "decode-T1-E64-bf16": C0.with_(dtype="bf16", T=1, d_model=1024, E=64, k=4, d_ff=512),
    # up to 128 rows per group: the skinny path's 128-row units, with a shared expert of 120 rows
    "small-T120-shared-bf16": C0.with_(dtype="bf16", T=120, d_model=256, E=4, k=2, d_ff=512,
                                       d_ff_shared=256, bias=("normal", 0.5)),
    # 200 rows per group: the down GEMM's skinny units in two 128-row blocks per group
    "small-T200-E2-shared-bf16": C0.with_(dtype="bf16", T=200, d_model=256, E=2, k=2, d_ff=512,
                                          d_ff_shared=256),
    # capacity variants: Expanded Drop (m extra candidates re-home dropped pairs) and
    # capacity per group of experts, under skewed routers
    "expanded-drop-bf16": C0.with_(dtype="bf16", T=500, d_model=128, E=8, k=2, d_ff=192,
                                   gamma=0.75, expand_m=2, bias=("zipf", 1.2)),
    "expanded-drop-E64-fp32": C0.with_(T=300, E=64, k=4, expand_m=4, gamma=1.0,
                                       bias=("normal", 1.0)),
    "group-capacity-bf16": C0.with_(dtype="bf16", T=400, E=16, k=4, d_ff=192, cap_groups=4,
                                    gamma=0.75, bias=("zipf", 1.2)),
    "group-capacity-one-group-fp32": C0.with_(T=200, cap_groups=1, gamma=0.5,
                                              bias=("normal", 0.5)),
    "no-renorm-fp32": C0.with_(k=3, renorm_topk=False),
    "k-equals-E-fp32": C0.with_(E=4, k=4, T=50),
    "zipf-drop-fp32": C0.with_(gamma=0.75, bias=("zipf", 1.2), T=160),
}


def _bits(a):
    """raw bit patterns of a device tensor or host array (bf16 as uint16, fp32 as uint32)"""
    import torch
    if isinstance(a, torch.Tensor):
        a = a.contiguous()
        a = (a.view(torch.int16) if a.element_size() == 2 else a.view(torch.int32)).cpu().numpy()
    if a.dtype.itemsize == 1:
        return a.view(np.uint8)
    return a.view(np.uint16) if a.dtype.itemsize == 2 else a.view(np.uint32)


def _meaningful(cfg, h):
    """the routing arrays a call defines (rows past offsets[E] are unspecified)"""
    N = int(h["offsets"][-1])
    out = dict(logits=h["logits"], counts=h["counts"], offsets=h["offsets"],
               perm_token=h["perm_token"][:N], perm_w=h["perm_w"][:N], tok_ptr=h["tok_ptr"],
               tok_pos=h["tok_pos"][:N])
    if cfg.routing == "token":
        out.update(topk_ids=h["topk_ids"], topk_w=h["topk_w"], kept=h["kept"])
    return out


def _compare_routing(cfg, rb, ro, exact_logits=None):
    g = rb.host()
    N = int(ro["offsets"][-1])
    assert g["offsets"].tolist() == ro["offsets"].tolist()
    assert g["counts"].tolist() == ro["counts"].tolist()
    assert (g["perm_token"][:N] == ro["perm_token"]).all()
    assert (g["tok_ptr"] == ro["tok_ptr"]).all()
    assert (g["tok_pos"][:N] == ro["tok_pos"]).all()
    np.testing.assert_allclose(g["perm_w"][:N], ro["perm_w"], rtol=1e-6, atol=1e-7)
    if cfg.routing == "token":
        assert (g["topk_ids"] == ro["ids"]).all()
        assert (g["kept"] == ro["kept"]).all()
        np.testing.assert_allclose(g["topk_w"], ro["gates"], rtol=1e-6, atol=1e-7)
    if exact_logits is not None:
        assert (g["logits"] == exact_logits).all()


@pytest.mark.parametrize("name", list(SMALL))
def test_router_logits(name):
    cfg = SMALL[name]
    inp = inputs_for(cfg)
    dev = dev_weights(inp)
    rb, _, _ = run_route(cfg, dev)
    ref = oracle.router_logits(inp.x, inp.w_router, inp.bias)
    assert np.abs(rb.logits.cpu().numpy() - ref).max() <= 1e-5


@pytest.mark.parametrize("name", list(SMALL))
def test_selection_bit_exact(name):
    cfg = SMALL[name]
    inp = inputs_for(cfg)
    dev = dev_weights(inp)
    l = oracle.router_logits(inp.x, inp.w_router, inp.bias)
    ro = oracle.route(cfg, logits=l)
    rb, _, _ = run_route(cfg, dev, logits_in=l)
    _compare_routing(cfg, rb, ro, exact_logits=l)


# bf16 layers with E <= 10: the matrix-core router also runs the top-k of its tokens
FUSED_TOPK = {
    "ragged-bf16": SMALL["ragged-bf16"],
    "expanded-drop-bf16": SMALL["expanded-drop-bf16"],
    "no-renorm-bf16": C0.with_(dtype="bf16", k=3, renorm_topk=False, T=200, bias=("normal", 0.5)),
    "E10-drop-bf16": C0.with_(dtype="bf16", T=333, d_model=192, E=10, k=3, d_ff=128, gamma=0.9,
                              bias=("zipf", 1.2)),
    "E9-nodrop-bf16": C0.with_(dtype="bf16", T=50, d_model=64, E=9, k=9, d_ff=64),
    # at most 16 tokens: the router's one workgroup also writes the dispatch (compared with the
    # dispatch kernel run on the same logits)
    "T16-E10-bf16": C0.with_(dtype="bf16", T=16, d_model=192, E=10, k=3, d_ff=64),
    "T5-E9-k9-bf16": C0.with_(dtype="bf16", T=5, d_model=64, E=9, k=9, d_ff=64),
    "T16-E8-k8-bf16": C0.with_(dtype="bf16", T=16, d_model=128, E=8, k=8, d_ff=64,
                               bias=("normal", 0.5)),
    "T17-E8-bf16": C0.with_(dtype="bf16", T=17, d_model=128, E=8, k=2, d_ff=64),
    # expert choice: the router also writes the logits transposed, which the selection then
    # reads instead of the token-major logits
    "EC-T300-E8-bf16": C0.with_(dtype="bf16", routing="expert", T=300, d_model=128, E=8, k=2,
                                d_ff=64),
    "EC-T2500-E10-bf16": C0.with_(dtype="bf16", routing="expert", T=2500, d_model=192, E=10,
                                  k=3, d_ff=64),
}


@pytest.mark.parametrize("name", list(FUSED_TOPK))
def test_fused_topk_equals_topk_kernel(name):
    """moe_route with the router computing logits (and, for these shapes, the top-k inside the
    same kernel, the dispatch too for at most 16 tokens, or for expert choice the transposed
    logits the selection reads) against moe_route fed those very logits (the separate kernels):
    every routing array bit-identical; and the selection against the oracle on the same
    logits."""
    cfg = FUSED_TOPK[name]
    inp = inputs_for(cfg)
    dev = dev_weights(inp)
    ra, _, _ = run_route(cfg, dev)
    ha = ra.host()
    rb, _, _ = run_route(cfg, dev, logits_in=ha["logits"])
    hb = rb.host()
    ma, mb = _meaningful(cfg, ha), _meaningful(cfg, hb)
    for key in ma:
        assert (_bits(np.asarray(ma[key])) == _bits(np.asarray(mb[key]))).all(), key
    ro = oracle.route(cfg, logits=ha["logits"])
    _compare_routing(cfg, ra, ro, exact_logits=ha["logits"])


TIE_CASES = [
    dict(T=517, E=8, k=2), dict(T=300, E=5, k=3), dict(T=129, E=16, k=4), dict(T=700, E=128, k=8),
    dict(T=64, E=33, k=7), dict(T=1, E=8, k=8), dict(T=2049, E=8, k=2, gamma=1.0),
    dict(T=1000, E=8, k=2, gamma=0.5), dict(T=999, E=128, k=8, gamma=1.25),
    dict(T=300, E=16, k=4, gamma=0.1), dict(T=257, E=8, k=1, gamma=1e-6),
    dict(T=300, E=8, k=2, gamma=8.0), dict(T=2500, E=8, k=2, routing="expert"),
    dict(T=77, E=6, k=5, routing="expert"), dict(T=300, E=128, k=8, routing="expert"),
    dict(T=64, E=64, k=64, routing="expert"),
    dict(T=999, E=16, k=2, gamma=0.75, expand_m=3), dict(T=300, E=32, k=4, gamma=0.5, expand_m=8),
    dict(T=1000, E=8, k=2, gamma=0.5, cap_groups=2), dict(T=500, E=64, k=8, gamma=1.25, cap_groups=8),
    dict(T=333, E=16, k=4, gamma=0.25, cap_groups=1),
    # at most 256 tokens: the single-block histogram + scan + scatter
    dict(T=200, E=16, k=2, gamma=0.75, expand_m=3), dict(T=150, E=16, k=4, gamma=0.5, cap_groups=4),
    dict(T=256, E=1024, k=8, gamma=1.0), dict(T=256, E=8, k=2),
    # a huge capacity factor ("no limit"): the capacity is clamped to T*k, nothing is dropped
    dict(T=300, E=8, k=2, gamma=1e12), dict(T=300, E=8, k=2, gamma=1e12, expand_m=2),
    dict(T=300, E=8, k=2, gamma=1e12, cap_groups=2),
    # more than 8 slots per token in the histogram + scatter (slot loads go in batches of 8):
    # every pair kept, a capacity, the extra candidates of Expanded Drop, group capacity
    dict(T=700, E=32, k=12), dict(T=700, E=32, k=12, gamma=0.8),
    dict(T=600, E=32, k=4, gamma=0.5, expand_m=12), dict(T=500, E=32, k=12, gamma=1.25, cap_groups=4),
]


@pytest.mark.parametrize("levels", [3, 40])
@pytest.mark.parametrize("case", range(len(TIE_CASES)))
def test_selection_ties_bit_exact(case, levels):
    """Logits drawn from a few values (ties everywhere): decisions must follow the tie rules
    (lower expert / lower token first) exactly as the oracle takes them."""
    kw = dict(TIE_CASES[case])
    cfg = C0.with_(d_model=64, d_ff=64, **kw)
    l = mi.quantised_logits(cfg.T, cfg.E, levels=levels, seed=case)
    ro = oracle.route(cfg, logits=l)
    dev = dict(x=None, w_router=None, bias=None)
    rb, _, _ = run_route(cfg, dev, logits_in=l)
    _compare_routing(cfg, rb, ro, exact_logits=l)


@pytest.mark.parametrize("name", list(SMALL))
def test_steps_with_oracle_routing(name):
    """dispatch gather, expert FFN and combine, each against the oracle, on oracle routing."""
    cfg = SMALL[name]
    inp = inputs_for(cfg)
    dev = dev_weights(inp)
    l = oracle.router_logits(inp.x, inp.w_router, inp.bias)
    ro = oracle.route(cfg, logits=l)
    out = run_steps(cfg, dev, logits_in=l)
    N = int(ro["offsets"][-1])
    # gather: bit-identical rows
    assert (_bits(out["x_perm"][:N]) == _bits(inp.x[ro["perm_token"]])).all()
    tol = tol_for(cfg)
    # expert FFN per dispatched row
    if N:
        rows = np.arange(N)
        o_ref = oracle.expert_rows_ffn(inp.x[ro["perm_token"]], ro, inp, rows)
        assert rel_err(host_f32(out["o_perm"][:N]), o_ref) <= tol
    # whole layer
    y_ref, _ = oracle.layer_forward(inp, routing=ro)
    check_y(cfg, host_f32(out["y"]), y_ref)


@pytest.mark.parametrize("name", list(SMALL))
def test_layer_forward_small(name):
    """moe_layer_forward end to end (its own logits); at these sizes no decision is close
    enough to a tie for the 1e-5 logit error to flip it, so routing must equal the oracle's."""
    cfg = SMALL[name]
    inp = inputs_for(cfg)
    dev = dev_weights(inp)
    y, rb = run_layer(cfg, dev)
    y_ref, ro = oracle.layer_forward(inp)
    _compare_routing(cfg, rb, ro)
    check_y(cfg, host_f32(y), y_ref)


@pytest.mark.parametrize("name", ["ragged-bf16", "fine-shared-bf16", "expert-choice-bf16",
                                  "decode-T8-bf16", "decode-T48-shared-bf16", "small-T120-shared-bf16",
                                  "small-T200-E2-shared-bf16",
                                  "decode-T1-E64-bf16"])
def test_layer_forward_deterministic_and_equal_to_steps(name):
    """Two runs give bit-identical routing and output; the one-call layer equals the four
    separate entry points bit for bit (the same arithmetic in the same order, no atomics in
    any decision or sum; for decode shapes the layer sums the down GEMM's K parts inside the
    combine, the separate entry points in their own kernel)."""
    import torch
    cfg = SMALL[name]
    inp = inputs_for(cfg)
    dev = dev_weights(inp)
    y1, rb1 = run_layer(cfg, dev)
    y2, rb2 = run_layer(cfg, dev)
    assert torch.equal(y1, y2)
    h1, h2 = _meaningful(cfg, rb1.host()), _meaningful(cfg, rb2.host())
    for k, v in h1.items():
        assert (_bits(v) == _bits(h2[k])).all() if v.dtype.itemsize in (2, 4) else (v == h2[k]).all(), k
    steps = run_steps(cfg, dev)
    assert torch.equal(y1, steps["y"])


def test_routing_stats():
    import torch
    import mixture_experts_layer_42_amd as moe
    cfg = SMALL["drop-E16-bf16"]
    inp = inputs_for(cfg)
    dev = dev_weights(inp)
    l = oracle.router_logits(inp.x, inp.w_router, inp.bias)
    ro = oracle.route(cfg, logits=l)
    rb, ws, n = run_route(cfg, dev, logits_in=l)
    out = torch.empty(2 * cfg.E + 4, dtype=torch.float32, device="cuda")
    moe.moe_routing_stats(moe.problem_of(cfg), rb.struct, out, ws, n)
    got = out.cpu().numpy()
    ref = oracle.routing_stats(ro, cfg.E, cfg.T, cfg.k)
    E = cfg.E
    np.testing.assert_allclose(got[:E], ref["f"], rtol=1e-6, atol=1e-7)
    np.testing.assert_allclose(got[E:2 * E], ref["P"], rtol=1e-5, atol=1e-6)
    assert abs(got[2 * E] - ref["balance"]) <= 1e-5 * max(1.0, ref["balance"])
    assert abs(got[2 * E + 1] - ref["max_over_mean"]) <= 1e-5 * ref["max_over_mean"]
    assert got[2 * E + 2] == ref["dropped"]
    assert got[2 * E + 3] == ref["empty"]


def test_routing_stats_hand_examples():
    """moe_routing_stats on the hand-derived examples of tests/golden/hand_oracle_pins.json,
    the routing computed by moe_route from the given logits: every statistic equals the value
    worked out by hand (the balance term is the unscaled sum of f_i P_i)."""
    import json
    import os
    from fractions import Fraction
    import torch
    import mixture_experts_layer_42_amd as moe
    gold = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_oracle_pins.json")))
    ln3 = np.float32(np.log(3.0))
    for gc in gold["routing_stats"]:
        T, E, k = gc["T"], gc["E"], gc["k"]
        cfg = C0.with_(T=T, E=E, k=k, d_model=64, d_ff=64, routing=gc["routing"], gamma=gc["gamma"])
        l = np.array([[ln3 if v == "ln3" else np.float32(v) for v in row] for row in gc["logits"]],
                     dtype=np.float32)
        rb, ws, n = run_route(cfg, dict(x=None, w_router=None, bias=None), logits_in=l)
        out = torch.empty(2 * E + 4, dtype=torch.float32, device="cuda")
        moe.moe_routing_stats(moe.problem_of(cfg), rb.struct, out, ws, n)
        got = out.cpu().numpy().astype(np.float64)
        fr = lambda v: float(Fraction(v))   # noqa: E731
        assert rb.counts.cpu().numpy().tolist() == gc["counts"]
        np.testing.assert_allclose(got[:E], [fr(v) for v in gc["f"]], rtol=0, atol=1e-7)
        np.testing.assert_allclose(got[E:2 * E], [fr(v) for v in gc["P"]], rtol=0, atol=1e-6)
        assert abs(got[2 * E] - fr(gc["balance"])) <= 1e-6
        assert abs(got[2 * E + 1] - fr(gc["max_over_mean"])) <= 1e-6
        assert got[2 * E + 2] == gc["dropped"] and got[2 * E + 3] == gc["empty"]


@pytest.mark.parametrize("name", ["fine-shared-bf16", "expert-choice-bf16", "all-dropped-shared-bf16"])
def test_combine_against_oracle_combine(name):
    """moe_combine alone: the GPU's own expert outputs (o_perm, o_shared) and routing, combined
    on the GPU and by oracle.combine (float64): within float32 summation error."""
    cfg = SMALL[name]
    inp = inputs_for(cfg)
    dev = dev_weights(inp)
    l = oracle.router_logits(inp.x, inp.w_router, inp.bias)
    out = run_steps(cfg.with_(y_dtype="f32"), dev, logits_in=l)
    g = out["rb"].host()
    N = int(g["offsets"][-1])
    o = out["o_perm"].cpu().numpy()
    o_sh = out["o_shared"].cpu().numpy() if out["o_shared"] is not None else None
    r = dict(tok_ptr=g["tok_ptr"], tok_pos=g["tok_pos"][:N], perm_w=g["perm_w"][:N].astype(np.float64))
    y_ref = oracle.combine(o[:max(N, 1)], r, cfg.T, o_shared=o_sh)
    # float32 summation bound: n terms summed with n roundings of at most 2^-24 each, relative
    # to the sum of the terms' magnitudes (the same combine over |w| and |o|)
    mag = oracle.combine(np.abs(o[:max(N, 1)]), dict(r, perm_w=np.abs(r["perm_w"])), cfg.T,
                         o_shared=None if o_sh is None else np.abs(o_sh))
    n = int(np.diff(g["tok_ptr"]).max()) + 2
    y = out["y"].cpu().numpy().astype(np.float64)
    assert (np.abs(y - y_ref) <= n * 2.0 ** -24 * mag + 1e-37).all()


# capacity buckets past each size path of the selection kernel: up to 2048 and 4096 keys per
# bucket in registers, 4097..16384 in registers at 16 keys per thread, beyond that re-read
# from memory; a router bias sends most pairs to expert 0 (and many to expert 1)
BIG_BUCKETS = [
    dict(T=10000, levels=0), dict(T=12000, levels=3), dict(T=40000, levels=0),
    dict(T=40000, levels=5), dict(T=20000, levels=0, expand_m=1), dict(T=20000, levels=4, cap_groups=1),
]


@pytest.mark.parametrize("case", range(len(BIG_BUCKETS)))
def test_capacity_large_buckets_bit_exact(case):
    kw = dict(BIG_BUCKETS[case])
    levels = kw.pop("levels")
    cfg = C0.with_(d_model=64, d_ff=64, E=4, k=2, gamma=0.5, **kw)
    bias = np.array([3.0, 1.5, 0.0, 0.0], dtype=np.float32)
    if levels:
        l = (mi.quantised_logits(cfg.T, cfg.E, levels=levels, seed=case) + bias).astype(np.float32)
    else:
        l = mi.normal_logits(cfg.T, cfg.E, seed=case, bias=bias)
    ro = oracle.route(cfg, logits=l)
    cand = np.bincount(ro["ids"][:, :cfg.k].ravel(), minlength=cfg.E)
    say(f"[big-bucket] {kw} levels={levels}: candidates per expert {cand.tolist()}, kept "
        f"{ro['counts'].tolist()}")
    assert cand.max() > 4096
    rb, _, _ = run_route(cfg, dict(x=None, w_router=None, bias=None), logits_in=l)
    _compare_routing(cfg, rb, ro, exact_logits=l)


@pytest.mark.parametrize("name", ["collapse-ksplit-bf16", "fine-shared-bf16", "expert-choice-bf16",
                                  "decode-T48-shared-bf16", "group-capacity-bf16"])
def test_deterministic_across_launch_shapes(name, monkeypatch):
    """Runs under different launch shapes (the persistent grids capped at 256, 120, 37 and 8
    workgroups through MOE_GRID_CUS) give bit-identical routing and output: no result
    depends on how work is spread over the CUs (the K-split plan is fixed independently of the
    grid, every sum runs in a fixed order, no decision depends on timing)."""
    import torch
    cfg = SMALL[name]
    inp = inputs_for(cfg)
    dev = dev_weights(inp)
    ref_y, ref_rb = None, None
    for cus in ("", "120", "37", "8"):
        monkeypatch.setenv("MOE_GRID_CUS", cus)
        y, rb = run_layer(cfg, dev)
        h = _meaningful(cfg, rb.host())
        if ref_y is None:
            ref_y, ref_h = y, h
            continue
        assert torch.equal(_bits_t(y), _bits_t(ref_y)), f"output differs with MOE_GRID_CUS={cus}"
        for k, v in ref_h.items():
            assert (_bits(np.asarray(h[k])) == _bits(np.asarray(v))).all(), (k, cus)


# groups whose last row tile holds at most 64 rows: the grouped GEMMs run that tile across two
# column panels (64 x 512 B-columns); routing collapse puts such tiles into the K-split tail,
# and an odd panel count leaves one panel with its own 64-row tile
WIDE_CASES = {
    "collapse-ksplit-bf16": SMALL["collapse-ksplit-bf16"].with_(y_dtype="f32"),
    "wide-even-panels-bf16": C0.with_(dtype="bf16", y_dtype="f32", T=1536, d_model=1024, E=8,
                                      k=2, d_ff=1024, bias=("normal", 0.5)),
    "wide-odd-panels-bf16": C0.with_(dtype="bf16", y_dtype="f32", T=1536, d_model=768, E=8,
                                     k=2, d_ff=384, bias=("normal", 0.5)),
}


@pytest.mark.parametrize("name", list(WIDE_CASES))
def test_wide_last_row_tiles(name, monkeypatch):
    """The grouped GEMMs without wide last row tiles (MOE_GEMM_WIDE=0), with them in the down
    GEMM (the default), in both GEMMs (MOE_GEMM_WIDE=all), and with panel-by-panel instead of
    banded tile order (MOE_GEMM_BAND=1) give the same float32 output bit for bit (every output
    element sums its K products in the same MFMA order whatever tile holds it and whenever it
    runs), and that output meets the bar against the oracle."""
    import torch
    cfg = WIDE_CASES[name]
    inp = inputs_for(cfg)
    dev = dev_weights(inp)
    y_ref, ro = oracle.layer_forward(inp)
    counts = ro["counts"]
    short = [int(e) for e in range(cfg.E) if 0 < counts[e] % 256 <= 64]
    say(f"[wide] {name}: rows per expert {counts.tolist()}, last tile <= 64 rows: {short}")
    assert short, "no group ends in a 64-row tile: the case would not exercise wide tiles"
    monkeypatch.setenv("MOE_GEMM_WIDE", "0")
    y0, _ = run_layer(cfg, dev)
    monkeypatch.setenv("MOE_GEMM_WIDE", "all")
    y2, _ = run_layer(cfg, dev)
    monkeypatch.setenv("MOE_GEMM_BAND", "1")   # the other tile order as well
    y3, _ = run_layer(cfg, dev)
    monkeypatch.delenv("MOE_GEMM_BAND")
    monkeypatch.delenv("MOE_GEMM_WIDE")
    y1, rb = run_layer(cfg, dev)
    assert torch.equal(_bits_t(y0), _bits_t(y1)), "wide tiles in the down GEMM changed the output"
    assert torch.equal(_bits_t(y0), _bits_t(y2)), "wide tiles in both GEMMs changed the output"
    assert torch.equal(_bits_t(y0), _bits_t(y3)), "banded tile order changed the output"
    _compare_routing(cfg, rb, ro)
    check_y(cfg, host_f32(y1), y_ref)


def _bits_t(t):
    import torch
    return t.contiguous().view(torch.int16 if t.element_size() == 2 else torch.int32)


# ------------------------------------------------------------------------------ full size

def _decisions(r, T):
    offs = r["offsets"]
    N = int(offs[-1])
    e_of = np.searchsorted(offs, np.arange(N), side="right") - 1
    ptr, pos = r["tok_ptr"], r["tok_pos"]
    return [tuple(e_of[pos[ptr[t]:ptr[t + 1]]].tolist()) for t in range(T)]


def _explained(cfg, t, l, ro, ndiff):
    """True if token t's routing may legitimately differ: its decision sits within the
    float32 logit tolerance of a tie in the oracle's own scores."""
    tol = 3e-5
    if cfg.routing == "expert":
        c = ro["c"]
        for e in range(cfg.E):
            col = l[:, e]
            tau = np.sort(col)[::-1][c - 1]
            if abs(col[t] - tau) <= tol:
                return True
        return False
    srt = np.sort(l[t])[::-1]
    if cfg.k < cfg.E and srt[cfg.k - 1] - srt[cfg.k] <= tol:
        return True
    if cfg.gamma > 0:
        C = ro["C"]
        for e in set(ro["ids"][t].tolist()) | set(np.argsort(-l[t])[:cfg.k + 1].tolist()):
            cand = np.nonzero((ro["ids"] == e).any(axis=1))[0]
            if cand.size <= C - ndiff:
                continue
            keys = ro["p32"][cand, e]
            order = cand[np.argsort(-keys, kind="stable")]
            rank = int(np.nonzero(order == t)[0][0]) if t in order else C
            if abs(rank - C) <= ndiff + 1:
                return True
    return False


FULL = ["mixtral-token-choice-bf16", "expert-choice-bf16", "capacity-drop-zipf-bf16",
        "fine-grained-shared-bf16"]


@pytest.mark.parametrize("name", FULL)
def test_full_size_layer(name):
    """The named workload at full size, in the launch configuration the bench times
    (moe_layer_forward), every token compared. Checks: logits within 1e-5; with the
    oracle's logits fed in, every routing array bit-identical and y of every token within
    the bar; through moe_layer_forward, decisions equal the oracle's except tokens whose
    decision sits within the logit tolerance of a tie (listed, explained, rare), and y of
    every other token within the bar, on a float32 output of the same launch (the arithmetic)
    and on the bf16 output (its exact rounding). Over the whole output the float32 output is
    held to 2e-2 of the RMS for token choice; under expert choice, where bf16 rounding alone
    misses that global figure (tests/test_bar_reading.py), it is held to 2e-2 of the RMS
    against the oracle's routing evaluated with h rounded to bf16, and the global figures are
    printed."""
    import torch
    from bf16_emulation import h_bf16_layer
    cfg = mi.workload(name)
    say(f"[full] {name}: generating inputs")
    inp = inputs_for(cfg)
    dev = dev_weights(inp)
    say(f"[full] {name}: oracle routing")
    l = oracle.router_logits(inp.x, inp.w_router, inp.bias)
    ro = oracle.route(cfg, logits=l)
    say(f"[full] {name}: rows kept {int(ro['offsets'][-1])} of {cfg.T * cfg.k}")
    # 1) selection with the oracle's logits, and the rest of the layer on that routing
    steps = run_steps(cfg, dev, logits_in=l)
    _compare_routing(cfg, steps["rb"], ro, exact_logits=l)
    y_steps = host_f32(steps["y"])
    del steps
    # 2) the bench's launch configuration
    y_layer, rb = run_layer(cfg, dev)
    g = rb.host()
    assert np.abs(g["logits"] - l).max() <= 1e-5
    d_o, d_g = _decisions(ro, cfg.T), _decisions(g, cfg.T)
    diff = [t for t in range(cfg.T) if d_o[t] != d_g[t]]
    say(f"[full] {name}: tokens whose routing moved across a near-tie: {len(diff)}")
    assert len(diff) <= max(3, cfg.T // 500)
    for t in diff:
        assert _explained(cfg, t, l, ro, len(diff)), f"token {t} routing differs without a tie"
    ok = np.ones(cfg.T, dtype=bool)
    ok[diff] = False
    cfg32 = cfg.with_(y_dtype="f32")
    y32, _ = run_layer(cfg32, dev, with_routing=False)
    y32 = y32.cpu().numpy()
    # bf16 output: exactly the rounding of the float32 output
    assert (y_layer.view(torch.int16).cpu().numpy().view(np.uint16) == mi.f32_to_bf16_bits(y32)).all()
    y16 = host_f32(y_layer)
    del y_layer
    say(f"[full] {name}: oracle FFN on all {cfg.T} tokens")
    y_ref, _ = oracle.layer_forward(inp, routing=ro)
    # float32 output of the same launch: the arithmetic against the bar, every token
    p32, g32 = check_y(cfg32, y32[ok], y_ref[ok])
    ps, gs = check_y(cfg, y_steps, y_ref)
    pl, gl = check_y(cfg, y16[ok], y_ref[ok])
    e_round = rel_err(mi.bf16_to_f32(mi.f32_to_bf16_bits(y_ref.astype(np.float32))), y_ref)
    msg = (f"[full] {name}: max|dy|/RMS per-token/global over all tokens: float32 y "
           f"{p32:.4f}/{g32:.4f}  bf16 y {pl:.4f}/{gl:.4f} (oracle-logit path {ps:.4f}/{gs:.4f}); "
           f"exact answer rounded to bf16: global {e_round:.4f}; max|y|/RMS "
           f"{np.abs(y_ref).max() / np.sqrt(np.mean(y_ref ** 2)):.1f}")
    if cfg.routing == "expert":
        y_h = h_bf16_layer(inp, ro)
        e_h = rel_err(y_h, y_ref)
        g_vs_h = rel_err(y32[ok], y_h[ok])
        msg += f"; h rounded to bf16: global {e_h:.4f}; float32 y against it: global {g_vs_h:.4f}"
        assert g_vs_h <= tol_for(cfg), ("global bar against the bf16-h evaluation", g_vs_h)
    say(msg)


def test_operand_offsets_past_2gib():
    """A layer whose down-GEMM activation panel (h: T k = 524288 rows x d_ff = 3072 bf16,
    3.2 GB) reaches past 2 GiB, so the GEMM's 32-bit operand offsets exceed 2^31 and must be
    taken as unsigned. Logits within 1e-5; y (float32 output) on sampled tokens, which include
    rows beyond the 2 GiB mark, within the bar; tokens whose decisions moved across a near-tie
    are excluded and must be rare."""
    cfg = C0.with_(name="offsets-past-2gib", dtype="bf16", y_dtype="f32", T=65536, d_model=64,
                   E=16, k=8, d_ff=3072, d_ff_shared=0, bias=("none",), seed=7)
    say("[big] generating inputs")
    inp = inputs_for(cfg)
    dev = dev_weights(inp)
    l = oracle.router_logits(inp.x, inp.w_router, inp.bias)
    ro = oracle.route(cfg, logits=l)
    say("[big] moe_layer_forward")
    y32, rb = run_layer(cfg, dev)
    g = rb.host()
    assert np.abs(g["logits"] - l).max() <= 1e-5
    d_o, d_g = _decisions(ro, cfg.T), _decisions(g, cfg.T)
    diff = {t for t in range(cfg.T) if d_o[t] != d_g[t]}
    assert len(diff) <= cfg.T // 500
    rng = np.random.default_rng(11)
    sample = np.array(sorted({0, cfg.T - 1} | set(rng.choice(cfg.T, 30, replace=False).tolist())
                             - diff))
    # rows past 2 GiB of h: some sampled token must own one
    first_far = (1 << 31) // (cfg.d_ff * 2) + 1
    pos = ro["tok_pos"]
    owned = [pos[ro["tok_ptr"][t]:ro["tok_ptr"][t + 1]] for t in sample]
    assert any((p >= first_far).any() for p in owned)
    say(f"[big] oracle FFN on {sample.size} sampled tokens")
    y_ref, _ = oracle.layer_forward(inp, tokens=sample, routing=ro)
    p32, g32 = check_y(cfg, host_f32(y32)[sample], y_ref)
    say(f"[big] max|dy|/RMS per-token/global {p32:.4f}/{g32:.4f}")


@pytest.mark.parametrize("T", [1, 8, 64, 128, 256, 384, 768])
def test_decode_shaped_layer(T):
    """The Mixtral-shaped layer with a decode-sized batch (T tokens, every expert's rows fit
    the skinny GEMM path, units of 32, 64 or 128 rows): y of every token against the oracle,
    through moe_layer_forward
    (row gather folded into the GEMM) and through the separate steps (x_perm copied)."""
    cfg = mi.MIXTRAL.with_(T=T)
    say(f"[decode] T={T}: generating inputs")
    inp = inputs_for(cfg)
    dev = dev_weights(inp)
    l = oracle.router_logits(inp.x, inp.w_router, inp.bias)
    ro = oracle.route(cfg, logits=l)
    say(f"[decode] T={T}: oracle FFN on all tokens")
    y_ref, _ = oracle.layer_forward(inp, routing=ro)
    steps = run_steps(cfg, dev, logits_in=l)
    _compare_routing(cfg, steps["rb"], ro, exact_logits=l)
    check_y(cfg, host_f32(steps["y"]), y_ref)
    cfg32 = cfg.with_(y_dtype="f32")
    y32, rb = run_layer(cfg32, dev)
    g = rb.host()
    d_o, d_g = _decisions(ro, T), _decisions(g, T)
    ok = np.array([d_o[t] == d_g[t] for t in range(T)])
    assert ok.sum() >= T - 1
    p32, g32 = check_y(cfg32, host_f32(y32)[ok], y_ref[ok])
    say(f"[decode] T={T}: max|dy|/RMS per-token/global {p32:.4f}/{g32:.4f}")


# ------------------------------------------------------------------------------ random shapes

def _random_problem(seed):
    """A valid small problem drawn from every option the ABI has (seeded)."""
    r = np.random.default_rng(1000 + seed)
    bf16 = r.random() < 0.8
    E = int(r.choice([1, 2, 5, 8, 9, 10, 16, 24, 33, 64, 100, 128]))
    k = int(r.integers(1, min(E, 8) + 1))
    T = int(r.choice([1, 2, 7, 31, 64, 65, 129, 256, 257, 333, 600]))
    kw = dict(dtype="bf16" if bf16 else "f32", T=T, E=E, k=k,
              d_model=int(r.choice([64, 128, 192, 256, 512])),
              d_ff=int(r.choice([64, 128, 192, 256, 320, 384])),
              d_ff_shared=int(r.choice([0, 0, 64])), renorm_topk=bool(r.random() < 0.8),
              bias=[("none",), ("normal", 1.0), ("zipf", 1.2)][int(r.integers(0, 3))], seed=seed)
    form = r.random()
    if form < 0.2 and k * T >= E:
        kw.update(routing="expert")
    elif form < 0.6:
        kw.update(gamma=float(r.choice([0.25, 0.5, 1.0, 1.25])))
        extra = r.random()
        if extra < 0.2 and k + 2 <= E:
            kw.update(expand_m=int(r.integers(1, min(4, E - k) + 1)))
        elif extra < 0.4:
            divs = [D for D in (1, 2, 4, 8) if E % D == 0]
            kw.update(cap_groups=int(r.choice(divs)))
    if not bf16:
        kw.update(y_dtype="f32")
    return C0.with_(name=f"random-{seed}", **kw)


_RANDOM_START = int(__import__("os").environ.get("MOE_RANDOM_START", "0"))
_RANDOM_CASES = int(__import__("os").environ.get("MOE_RANDOM_CASES", "48"))


@pytest.mark.parametrize("seed", range(_RANDOM_START, _RANDOM_START + _RANDOM_CASES))
def test_random_shapes(seed):
    """Seeded random problems over the ABI's options (dtype, ragged T, 1..128 experts, k,
    shared expert, renormalisation, biases, every selection form): routing with the oracle's
    logits bit-identical, then the dispatch, expert FFN and combine on that routing against
    the oracle's layer output."""
    cfg = _random_problem(seed)
    say(f"[random] seed {seed}: {cfg}")
    inp = inputs_for(cfg)
    dev = dev_weights(inp)
    l = oracle.router_logits(inp.x, inp.w_router, inp.bias)
    ro = oracle.route(cfg, logits=l)
    rb, _, _ = run_route(cfg, dev, logits_in=l)
    _compare_routing(cfg, rb, ro, exact_logits=l)
    out = run_steps(cfg, dev, logits_in=l)
    y_ref, _ = oracle.layer_forward(inp, routing=ro)
    check_y(cfg, host_f32(out["y"]), y_ref)
