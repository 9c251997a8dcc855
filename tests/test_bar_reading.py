"""Why the layer-output bar is read per token for expert choice (CPU only).

The bar for bf16 layer outputs is a maximum error relative to "the output's RMS". Under
expert choice (hrletsgo page, Mixture-of-Tokens section: each expert takes its c best
tokens) the combine weight is a softmax over the tokens of an expert's column, so output
scales differ between tokens by a factor of tens and the output is heavy-tailed: its
largest element is about 40 times its RMS at T = 8192. Any bf16 pipeline makes relative
errors of about 2^-9 per rounding, and the largest elements' errors, divided by the whole
output's RMS, then exceed 2e-2 even when the arithmetic is exact:

  - the exact answer rounded once to bf16 (the best any bf16 output can be),
  - the exact answer computed with only the hidden activation h rounded to bf16 (what any
    bf16 down-projection GEMM must do, since h is its bf16 operand).

Measured here on the expert-choice workload at T = 8192 with narrower experts (d_model 256,
d_ff 512, so that the float64 evaluation takes about a second): both miss the global bar by
a wide margin while each token's error relative to that token's own RMS stays below it.
Under token choice the same two emulations stay within 2e-2 globally. So the bar is checked
per token for every workload, and over the whole output for token choice; the GPU tests
apply exactly that. The emulations (tests/bf16_emulation.py) are test code, numpy float64
with explicit bf16 roundings, not part of the oracle and not of the HIP path.
"""
import numpy as np
import pytest

import moe_inputs as mi
import oracle
from bf16_emulation import bf16_round as _bf16, h_bf16_layer as _h_bf16_layer

BAR = 2e-2


def _ratios(z, y):
    """(global, per-token) max |z - y| / RMS: over the whole output, and per token against
    that token's own RMS (tokens with an exactly zero output excluded)."""
    err = np.abs(z - y)
    rms_t = np.sqrt(np.mean(y ** 2, axis=1))
    nz = rms_t > 0
    return float(err.max() / np.sqrt(np.mean(y ** 2))), float((err[nz] / rms_t[nz, None]).max())


CASES = {
    "expert-choice": mi.EXPERT_CHOICE.with_(T=8192, d_model=256, d_ff=512),
    "token-choice": mi.MIXTRAL.with_(T=4096, d_model=256, d_ff=512),
}


@pytest.mark.parametrize("name", list(CASES))
def test_bf16_rounding_against_the_output_bar(name):
    cfg = CASES[name]
    inp = mi.make_inputs(cfg)
    y, r = oracle.layer_forward(inp)
    tail = float(np.abs(y).max() / np.sqrt(np.mean(y ** 2)))
    g_round, t_round = _ratios(_bf16(y), y)
    g_h, t_h = _ratios(_h_bf16_layer(inp, r), y)
    print(f"{name}: max|y|/RMS {tail:.1f}; exact answer rounded to bf16: global {g_round:.4f} "
          f"per-token {t_round:.4f}; h rounded to bf16: global {g_h:.4f} per-token {t_h:.4f}")
    # per token, both emulations hold the bar
    assert t_round <= BAR and t_h <= BAR
    if name == "expert-choice":
        assert tail > 25.0
        # over the whole output neither can: the global reading is unattainable in bf16
        assert g_round > 2 * BAR and g_h > 2 * BAR
    else:
        assert tail < 10.0
        assert g_round <= BAR and g_h <= BAR
