"""Seeded synthetic inputs for the sparse MoE layer forward.

This module is shared by the tests, the bench and the oracle's callers. It holds
no arithmetic of the layer itself: it only draws random tensors, rounds them to
the storage type, and names the workloads.

Recipe (one independent stream per tensor and per expert, so that any expert can
be regenerated alone and generation order never matters):

  stream(tensor_id, expert) = numpy.random.default_rng(SeedSequence([seed, tensor_id, expert]))

  x            ~ N(0, 1)                         [T, d_model]
  w_router     ~ N(0, 1/d_model)  (fp32 always)  [d_model, E]
  w_gate, w_up ~ N(0, 1/d_model)                 [E, d_ff, d_model]   (nn.Linear [out, in])
  w_down       ~ N(0, 1/d_ff)                    [E, d_model, d_ff]
  shared expert: same scalings with d_ff_shared  [d_ff_s, d_model], [d_ff_s, d_model], [d_model, d_ff_s]
  router bias  : per workload (normal with a stated *variance*, or b_e = -s*ln(e+1))

Normals are drawn in float32, scaled by a float32 standard deviation, and, for
bf16 workloads, rounded to bfloat16 with round-to-nearest-even. bf16 tensors are
held as numpy uint16 bit patterns (numpy has no bfloat16); ``bf16_to_f32``
widens them exactly.

The five named workloads follow the MoE-layer shapes that the source pages
discuss: a Mixtral-8x7B-shaped layer (top-2 of 8, page "moe-vs-mot-routing-
inference-cost", section on the basic MoE structure), expert-choice routing with
c = k*T/N (same page, Mixture-of-Tokens section), capacity-aware token drop
C = gamma * N-bar under a skewed router (Capacity-Aware Inference summary,
Methodology, Token Drop), and a fine-grained layer with a shared expert (the
routing/active-parameter page, section on how routing allocates the compute
budget).
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace
from typing import Optional

import numpy as np

# tensor ids of the per-tensor random streams
TID_X, TID_WR, TID_BIAS, TID_WG, TID_WU, TID_WD, TID_SG, TID_SU, TID_SD = range(1, 10)


@dataclass(frozen=True)
class MoEConfig:
    name: str
    T: int
    d_model: int
    E: int
    k: int
    d_ff: int
    d_ff_shared: int = 0
    routing: str = "token"          # "token" (token choice) or "expert" (expert choice)
    gamma: float = 0.0              # capacity factor; <= 0 means no capacity limit
    expand_m: int = 0               # expanded drop: m extra candidate experts per token
    cap_groups: int = 0             # capacity per group of E/cap_groups experts (0: per expert)
    renorm_topk: bool = True
    dtype: str = "bf16"             # "bf16" or "f32": x, expert weights, hidden activation
    y_dtype: str = ""               # layer output type; "" = same as dtype
    bias: tuple = ("none",)         # ("none",) | ("normal", variance) | ("zipf", s)
    seed: int = 0

    def with_(self, **kw) -> "MoEConfig":
        return replace(self, **kw)


CONFIGS = {
    0: MoEConfig("tiny-token-choice-fp32", T=64, d_model=128, E=8, k=2, d_ff=256, dtype="f32"),
    1: MoEConfig("mixtral-token-choice-bf16", T=4096, d_model=4096, E=8, k=2, d_ff=14336,
                 bias=("normal", 0.5)),
    2: MoEConfig("expert-choice-bf16", T=8192, d_model=4096, E=8, k=2, d_ff=14336,
                 routing="expert"),
    3: MoEConfig("capacity-drop-zipf-bf16", T=4096, d_model=4096, E=8, k=2, d_ff=14336,
                 gamma=1.0, bias=("zipf", 1.2)),
    4: MoEConfig("fine-grained-shared-bf16", T=16384, d_model=2048, E=128, k=8, d_ff=768,
                 d_ff_shared=768, gamma=1.25, bias=("normal", 1.0)),
}


def workload(name: str) -> MoEConfig:
    """The workload of that name (see CONFIGS)."""
    for c in CONFIGS.values():
        if c.name == name:
            return c
    raise KeyError(name)


TINY = workload("tiny-token-choice-fp32")
MIXTRAL = workload("mixtral-token-choice-bf16")
EXPERT_CHOICE = workload("expert-choice-bf16")
CAPACITY_ZIPF = workload("capacity-drop-zipf-bf16")
FINE_GRAINED = workload("fine-grained-shared-bf16")


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns uint16 bit patterns.
    Inputs are finite by construction."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns (uint16) to float32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _rng(seed: int, tid: int, expert: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, tid, expert]))


def _normal(seed, tid, expert, shape, std) -> np.ndarray:
    a = _rng(seed, tid, expert).standard_normal(shape, dtype=np.float32)
    a *= np.float32(std)
    return a


@dataclass
class MoEInputs:
    """Host copies of one workload's tensors. bf16 tensors are uint16 bit patterns."""
    cfg: MoEConfig
    x: np.ndarray
    w_router: np.ndarray
    bias: Optional[np.ndarray]
    w_gate: np.ndarray
    w_up: np.ndarray
    w_down: np.ndarray
    ws_gate: Optional[np.ndarray] = None
    ws_up: Optional[np.ndarray] = None
    ws_down: Optional[np.ndarray] = None
    extra: dict = field(default_factory=dict)

    def as_f32(self, name: str) -> Optional[np.ndarray]:
        """Exact float32 view of a tensor (widens bf16 bit patterns)."""
        a = getattr(self, name)
        if a is None:
            return None
        return bf16_to_f32(a) if a.dtype == np.uint16 else a


def _store(a: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(a) if dtype == "bf16" else a


def router_bias(cfg: MoEConfig) -> Optional[np.ndarray]:
    kind = cfg.bias[0]
    if kind == "none":
        return None
    if kind == "normal":
        var = float(cfg.bias[1])
        return _normal(cfg.seed, TID_BIAS, 0, (cfg.E,), math.sqrt(var))
    if kind == "zipf":
        s = float(cfg.bias[1])
        return np.array([-s * math.log(e + 1.0) for e in range(cfg.E)], dtype=np.float32)
    if kind == "onehot":   # routing-collapse shape: one expert gets a large constant bias
        b = np.zeros(cfg.E, dtype=np.float32)
        b[int(cfg.bias[2]) if len(cfg.bias) > 2 else 0] = np.float32(cfg.bias[1])
        return b
    raise ValueError(f"unknown bias kind {kind!r}")


def _expert_stack(cfg, tid, shape, std, threads):
    E = cfg.E
    out = np.empty((E,) + shape, dtype=np.uint16 if cfg.dtype == "bf16" else np.float32)

    def one(e):
        out[e] = _store(_normal(cfg.seed, tid, e, shape, std), cfg.dtype)

    if threads > 1 and E > 1:
        with ThreadPoolExecutor(max_workers=min(threads, E)) as ex:
            list(ex.map(one, range(E)))
    else:
        for e in range(E):
            one(e)
    return out


def make_inputs(cfg: MoEConfig, threads: int = 8, cache: Optional[dict] = None) -> MoEInputs:
    """Generate every tensor of the workload ``cfg`` (deterministic in cfg.seed).
    ``cache`` (a dict) lets workloads with equal shapes share the expert weight stacks."""
    d, E, dff = cfg.d_model, cfg.E, cfg.d_ff
    s = cfg.seed
    x = _store(_normal(s, TID_X, 0, (cfg.T, d), 1.0), cfg.dtype)
    w_router = _normal(s, TID_WR, 0, (d, E), 1.0 / math.sqrt(d))
    bias = router_bias(cfg)
    key = (s, E, d, dff, cfg.dtype)
    if cache is not None and key in cache:
        w_gate, w_up, w_down = cache[key]
    else:
        w_gate = _expert_stack(cfg, TID_WG, (dff, d), 1.0 / math.sqrt(d), threads)
        w_up = _expert_stack(cfg, TID_WU, (dff, d), 1.0 / math.sqrt(d), threads)
        w_down = _expert_stack(cfg, TID_WD, (d, dff), 1.0 / math.sqrt(dff), threads)
        if cache is not None:
            cache[key] = (w_gate, w_up, w_down)
    ws = [None, None, None]
    if cfg.d_ff_shared > 0:
        fs = cfg.d_ff_shared
        ws = [_store(_normal(s, TID_SG, 0, (fs, d), 1.0 / math.sqrt(d)), cfg.dtype),
              _store(_normal(s, TID_SU, 0, (fs, d), 1.0 / math.sqrt(d)), cfg.dtype),
              _store(_normal(s, TID_SD, 0, (d, fs), 1.0 / math.sqrt(fs)), cfg.dtype)]
    return MoEInputs(cfg, x, w_router, bias, w_gate, w_up, w_down, *ws)


def quantised_logits(T: int, E: int, levels: int, seed: int) -> np.ndarray:
    """fp32 logits drawn from a few distinct values, so that ties are common
    (used to exercise the tie rules of every selection form)."""
    r = _rng(seed, 100, 0).integers(0, levels, size=(T, E))
    return (r.astype(np.float32) * np.float32(0.25) - np.float32(1.0)).astype(np.float32)


def normal_logits(T: int, E: int, seed: int, bias: Optional[np.ndarray] = None) -> np.ndarray:
    """fp32 logits ~ N(0,1) (+ bias), for selection-only tests."""
    l = _rng(seed, 101, 0).standard_normal((T, E), dtype=np.float32)
    if bias is not None:
        l = (l + bias[None, :].astype(np.float32)).astype(np.float32)
    return l
