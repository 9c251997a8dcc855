"""The seeded input recipe against what the workloads state (CPU only).

The skewed capacity-drop workload gives its router a Zipf(1.2) bias over the experts and
states that expert 0 then draws about 40% of the top-2 assignments; the recipe reads the
bias as b_e = -1.2 ln(e + 1) (the log of the Zipf weights). The plain Zipf weights used
directly as the bias would give expert 0 well under 20%, so the statement separates the two.
"""
import math

import numpy as np

import moe_inputs as mi
import oracle


def _share_of_expert0(cfg):
    x = mi._store(mi._normal(cfg.seed, mi.TID_X, 0, (cfg.T, cfg.d_model), 1.0), cfg.dtype)
    wr = mi._normal(cfg.seed, mi.TID_WR, 0, (cfg.d_model, cfg.E), 1.0 / math.sqrt(cfg.d_model))
    l = oracle.router_logits(x, wr, mi.router_bias(cfg))
    ids = oracle.topk_select(l, cfg.k)
    return float(np.mean(ids == 0))   # of all T k assignments


def test_zipf_workload_gives_expert0_about_40_percent():
    cfg = mi.CONFIGS[3]
    assert cfg.bias == ("zipf", 1.2) and cfg.k == 2
    share = _share_of_expert0(cfg)
    assert 0.35 <= share <= 0.45, share


def test_zipf_weights_as_the_bias_would_not():
    # the other reading, the Zipf weights themselves as the bias, misses the stated share
    cfg = mi.CONFIGS[3]
    w = np.array([(e + 1.0) ** -1.2 for e in range(cfg.E)], dtype=np.float64)
    x = mi._store(mi._normal(cfg.seed, mi.TID_X, 0, (cfg.T, cfg.d_model), 1.0), cfg.dtype)
    wr = mi._normal(cfg.seed, mi.TID_WR, 0, (cfg.d_model, cfg.E), 1.0 / math.sqrt(cfg.d_model))
    l = oracle.router_logits(x, wr, (w / w.sum()).astype(np.float32))
    ids = oracle.topk_select(l, cfg.k)
    assert float(np.mean(ids == 0)) < 0.25
