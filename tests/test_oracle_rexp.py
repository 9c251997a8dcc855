"""Pins of the float32 routing-score encoding (Cody & Waite exponential + fixed
left-to-right sum + IEEE division) that ranks the capacity drop. CPU only.

The score must order pairs like the exact softmax probability (the gating score
of the Capacity-Aware Inference summary, Token Drop); these tests bound how far
it is from the float64 exponential and softmax.
"""
import math

import numpy as np
import pytest
import scipy.special

import moe_inputs as mi
import oracle

REXP_MAX_ULP = 1.05    # measured bound over every float32 in [-87, 0]: 1.028 ulp


def _ulp_err(got32, ref64):
    ref32 = ref64.astype(np.float32)
    ulp = np.spacing(np.abs(ref32)).astype(np.float64)
    return np.abs(got32.astype(np.float64) - ref64) / ulp


def test_rexp_special_values():
    assert oracle.rexp(np.array([0.0], np.float32))[0] == np.float32(1.0)
    assert oracle.rexp(np.array([-0.0], np.float32))[0] == np.float32(1.0)
    assert oracle.rexp(np.array([-87.5, -100.0, -1e30], np.float32)).tolist() == [0.0, 0.0, 0.0]
    # exact powers of two: x = -n ln2 (rounded) lands within an ulp of 2^-n
    for n in (1, 2, 10, 60, 120):
        x = np.float32(-n * math.log(2.0))
        v = oracle.rexp(np.array([x]))[0]
        assert abs(float(v) - math.exp(float(x))) <= 2 * float(np.spacing(np.float32(math.exp(float(x)))))


@pytest.mark.slow
def test_rexp_exhaustive_error_bound_and_monotone():
    """Every float32 in [-87, 0]: error <= REXP_MAX_ULP ulp of the float64 exponential,
    and non-decreasing in x."""
    lo_bits = np.uint32(0x80000000)          # -0.0
    hi_bits = np.float32(-87.0).view(np.uint32)
    chunk = 1 << 24
    worst = 0.0
    prev_last = None
    start = int(lo_bits)
    while start <= int(hi_bits):
        stop = min(start + chunk, int(hi_bits) + 1)
        bits = np.arange(start, stop, dtype=np.uint32)
        x = bits.view(np.float32)            # descending: -0, -tiny, ..., -87
        v = oracle.rexp(x)
        ref = np.exp(x.astype(np.float64))
        worst = max(worst, float(_ulp_err(v, ref).max()))
        # monotone: x decreases along the array, so v must not increase
        assert (np.diff(v) <= 0).all()
        if prev_last is not None:
            assert v[0] <= prev_last
        prev_last = v[-1]
        start = stop
    assert worst <= REXP_MAX_ULP, worst


def test_rexp_error_bound_sample():
    """Fast version of the exhaustive sweep: 2M evenly spread float32s in [-87, 0]."""
    bits = np.linspace(0x80000000, int(np.float32(-87.0).view(np.uint32)), 2_000_000).astype(np.uint32)
    x = bits.view(np.float32)
    err = _ulp_err(oracle.rexp(x), np.exp(x.astype(np.float64)))
    assert err.max() <= REXP_MAX_ULP


@pytest.mark.parametrize("E", [2, 8, 128])
def test_routing_score_close_to_softmax(E):
    l = mi.normal_logits(512, E, seed=E, bias=np.linspace(1, -1, E).astype(np.float32))
    p32 = oracle.routing_score32(l)
    p = scipy.special.softmax(l.astype(np.float64), axis=1)
    rel = np.abs(p32 - p) / p
    # each q within 2 ulp, the E-term float32 sum within (E-1)/2 ulp, one division: loose bound
    assert rel.max() <= (4 + E) * 2.0 ** -24
    assert (p32 > 0).all() and p32.dtype == np.float32


def test_routing_score_orders_like_softmax_when_gaps_exceed_error():
    """For pairs whose exact probabilities differ by more than the encoding's error, the
    encoding orders them the same way (it is a faithful ranking key)."""
    l = mi.normal_logits(2000, 8, seed=11)
    p32 = oracle.routing_score32(l)[:, 3].astype(np.float64)
    p = scipy.special.softmax(l.astype(np.float64), axis=1)[:, 3]
    i, j = np.triu_indices(300, 1)
    gap = np.abs(p[i] - p[j]) / np.maximum(p[i], p[j])
    far = gap > 1e-5
    assert (np.sign(p32[i] - p32[j])[far] == np.sign(p[i] - p[j])[far]).all()


def test_capacity_formula():
    """C = gamma * N-bar with N-bar = T*k/E, floored (Capacity-Aware Inference summary)."""
    assert oracle.capacity(4096, 2, 8, 1.0) == 1024
    assert oracle.capacity(16384, 8, 128, 1.25) == 1280
    assert oracle.capacity(5, 1, 2, 1.0) == 2
    assert oracle.capacity(100, 1, 8, 1.0) == 12
    assert oracle.expert_choice_capacity(8192, 2, 8) == 2048
    assert oracle.expert_choice_capacity(7, 2, 4) == 3
