"""Test-side emulation of the one rounding every bf16 expert pipeline must make: the hidden
activation h, the bf16 operand of the down projection, rounded to bf16 with everything else in
float64. It is not part of the oracle (which computes the exact definition) and shares nothing
with the HIP path; the tests use it to show which part of an output error that rounding alone
explains."""
import numpy as np

import moe_inputs as mi
import oracle


def bf16_round(a):
    return mi.bf16_to_f32(mi.f32_to_bf16_bits(np.asarray(a, dtype=np.float32))).astype(np.float64)


def h_bf16_layer(inp, r):
    """y [T, d_model] float64 with every routed expert's h (and the shared expert's) rounded to
    bf16; routing r as oracle.route returns it."""
    cfg = inp.cfg
    X = oracle.widen(inp.x)
    y = np.zeros((cfg.T, cfg.d_model))
    for e in range(cfg.E):
        rows = np.arange(r["offsets"][e], r["offsets"][e + 1])
        if rows.size == 0:
            continue
        toks = r["perm_token"][rows]
        v = X[toks]
        h = bf16_round(oracle.silu(v @ oracle.widen(inp.w_gate[e]).T)
                       * (v @ oracle.widen(inp.w_up[e]).T))
        np.add.at(y, toks, r["perm_w"][rows][:, None] * (h @ oracle.widen(inp.w_down[e]).T))
    if cfg.d_ff_shared:
        h = bf16_round(oracle.silu(X @ oracle.widen(inp.ws_gate).T) * (X @ oracle.widen(inp.ws_up).T))
        y += h @ oracle.widen(inp.ws_down).T
    return y
