"""Debug mode (MOE_DEBUG): non-finite inputs become MOE_ERR_INVALID_ARG before any work is
enqueued, at every entry point; without it the hot path checks nothing."""
import numpy as np
import pytest

import moe_inputs as mi
from gpu_support import dev_weights, inputs_for, run_steps, workspace

pytestmark = pytest.mark.gpu

CFG = mi.TINY.with_(dtype="bf16", T=96, d_model=128, d_ff=192, d_ff_shared=64,
                          bias=("normal", 0.5))


def _route(moe, prob, dev, x, ws, n):
    rb = moe.RoutingBuffers(prob)
    rb.logits.fill_(-7.0)
    moe.moe_route(prob, x, dev["w_router"], dev["bias"], 0, rb.struct, ws, n)
    return rb


def test_debug_mode_rejects_nonfinite(monkeypatch):
    import torch
    import mixture_experts_layer_42_amd as moe
    inp = inputs_for(CFG)
    dev = dev_weights(inp)
    prob = moe.problem_of(CFG)
    ws, n = workspace(prob)
    monkeypatch.setenv("MOE_DEBUG", "1")
    # finite inputs pass every entry point
    out = run_steps(CFG, dev)
    torch.cuda.synchronize()
    # a NaN in x: moe_route refuses, logits untouched
    bad_x = dev["x"].clone()
    bad_x.view(-1)[12345 % bad_x.numel()] = float("nan")
    rb = moe.RoutingBuffers(prob)
    rb.logits.fill_(-7.0)
    with pytest.raises(moe.MoEError) as ei:
        moe.moe_route(prob, bad_x, dev["w_router"], dev["bias"], 0, rb.struct, ws, n)
    assert ei.value.status == moe.MOE_ERR_INVALID_ARG
    torch.cuda.synchronize()
    assert (rb.logits == -7.0).all()
    # an infinity in the router bias
    bad_b = dev["bias"].clone() if dev["bias"] is not None else None
    if bad_b is not None:
        bad_b[3] = float("inf")
        with pytest.raises(moe.MoEError):
            moe.moe_route(prob, dev["x"], dev["w_router"], bad_b, 0, rb.struct, ws, n)
    # a NaN in one expert weight: moe_expert_ffn refuses, o untouched
    rb2 = out["rb"]
    R, d = CFG.T * CFG.k, CFG.d_model
    o = torch.full((R, d), 3.0, dtype=torch.float32, device="cuda")
    o_sh = torch.full((CFG.T, d), 3.0, dtype=torch.float32, device="cuda")
    w_down = dev["w_down"].clone()
    w_down.view(-1)[-1] = float("nan")
    with pytest.raises(moe.MoEError):
        moe.moe_expert_ffn(prob, out["x_perm"], rb2.struct, dev["w_gate"], dev["w_up"], w_down,
                           dev["x"], dev["ws_gate"], dev["ws_up"], dev["ws_down"], o, o_sh, ws, n)
    torch.cuda.synchronize()
    assert (o == 3.0).all() and (o_sh == 3.0).all()
    # a NaN in a kept expert-output row: moe_combine refuses, y untouched
    o_bad = out["o_perm"].clone()
    o_bad[0, 0] = float("nan")
    y = torch.full((CFG.T, d), 5.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(moe.MoEError):
        moe.moe_combine(prob, o_bad, out["o_shared"], rb2.struct, y)
    torch.cuda.synchronize()
    assert (y == 5.0).all()
    # the whole layer
    with pytest.raises(moe.MoEError):
        moe.moe_layer_forward(prob, bad_x, dev["w_router"], dev["bias"], dev["w_gate"],
                              dev["w_up"], dev["w_down"], dev["ws_gate"], dev["ws_up"],
                              dev["ws_down"], y, None, ws, n)
    torch.cuda.synchronize()
    assert (y == 5.0).all()
    # rows past the kept count are not inspected (they are unspecified by contract)
    N = int(rb2.host()["offsets"][-1])
    if N < R:
        o_tail = out["o_perm"].clone()
        o_tail[N:] = float("nan")
        moe.moe_combine(prob, o_tail, out["o_shared"], rb2.struct, y)
        torch.cuda.synchronize()


def test_without_debug_mode_nothing_is_checked(monkeypatch):
    """The hot path does not look at values: a NaN in a kept expert-output row reaches y.
    (Only arithmetic is fed a NaN here: non-finite router inputs would make the selection
    indices themselves meaningless, which is why the contract requires finite inputs.)"""
    import torch
    import mixture_experts_layer_42_amd as moe
    inp = inputs_for(CFG)
    dev = dev_weights(inp)
    prob = moe.problem_of(CFG)
    monkeypatch.delenv("MOE_DEBUG", raising=False)
    out = run_steps(CFG, dev)
    rb = out["rb"]
    h = rb.host()
    assert int(h["offsets"][-1]) > 0
    p0 = int(h["tok_pos"][0])   # a row of token 0
    o_bad = out["o_perm"].clone()
    o_bad[p0, 0] = float("nan")
    y = torch.zeros(CFG.T, CFG.d_model, dtype=torch.bfloat16, device="cuda")
    moe.moe_combine(prob, o_bad, out["o_shared"], rb.struct, y)   # no raise
    torch.cuda.synchronize()
    yh = y.float().cpu().numpy()
    assert np.isnan(yh[0, 0]) and np.isfinite(yh[1:]).all()
