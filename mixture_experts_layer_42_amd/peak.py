"""ctypes binding of libmoe_peak.so, the achievable-peak microbenchmarks (include/moe_peak.h).

Marshalling and timing only: each function launches one microbenchmark kernel on torch's
current stream, times it with HIP events on that stream, and converts the known work of the
launch into a rate. The layer never calls this module; bench.py reports its figures next to
the datasheet peaks.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
PEAK_LIB_PATH = os.path.join(_PKG, "libmoe_peak.so")
MFMA_FLOP = 2 * 32 * 32 * 16        # one v_mfma_f32_32x32x16_bf16
WAVES_PER_WG = 8

_lib = None


def load(path: str = PEAK_LIB_PATH) -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m mixture_experts_layer_42_amd.build`")
    import torch  # noqa: F401  (bind to torch's HIP runtime, as the layer's binding does)
    lib = ctypes.CDLL(path)
    V, I, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    for name, args in {"moe_peak_mfma": [V, V, V, I, I, V], "moe_peak_lds": [V, I, I, V],
                       "moe_peak_copy": [V, V, SZ, I, V]}.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = I
    _lib = lib
    return lib


def _timed(launch, reps=1):
    import torch
    st = torch.cuda.current_stream()
    launch(st.cuda_stream)                      # warm-up (clocks, code load)
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(st)
    for _ in range(reps):
        launch(st.cuda_stream)
    t1.record(st)
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) * 1e-3 / reps


def _check(rc, name):
    if rc != 0:
        raise RuntimeError(f"{name} failed with hipError {rc}")


def mfma(num_cu: int, iters: int = 200000, wg_per_cu: int = 2) -> dict:
    """Sustained bf16 matrix-core rate of a full grid (no memory traffic) and the shader
    clock it ran at (cycle counter over the 100 MHz real-time counter, median workgroup)."""
    import numpy as np
    import torch
    lib = load()
    grid = num_cu * wg_per_cu
    g = torch.Generator().manual_seed(0)
    seed = torch.randn(256 * 8, generator=g).to(torch.bfloat16).cuda()
    out = torch.empty(grid * WAVES_PER_WG * 64, dtype=torch.float32, device="cuda")
    clk = torch.zeros(2 * grid, dtype=torch.int64, device="cuda")
    dt = _timed(lambda s: _check(lib.moe_peak_mfma(seed.data_ptr(), out.data_ptr(), clk.data_ptr(),
                                                   grid, iters, s), "moe_peak_mfma"))
    c = clk.view(grid, 2).cpu().numpy().astype(np.float64)
    ghz = float(np.median(c[:, 0] / c[:, 1]) * 0.1)
    flop = float(grid) * WAVES_PER_WG * 4 * iters * MFMA_FLOP
    return {"tflops": round(flop / dt / 1e12, 1), "clock_ghz": round(ghz, 3),
            "ms": round(dt * 1e3, 2), "how": f"{grid} workgroups x 8 waves, 4 * {iters} "
            "v_mfma_f32_32x32x16_bf16 per wave on register operands"}


def lds(num_cu: int, iters: int = 20000, wg_per_cu: int = 2) -> dict:
    """LDS read bandwidth per CU with 16-byte reads spread over all banks."""
    import torch
    lib = load()
    grid = num_cu * wg_per_cu
    out = torch.empty(grid * WAVES_PER_WG * 64, dtype=torch.float32, device="cuda")
    dt = _timed(lambda s: _check(lib.moe_peak_lds(out.data_ptr(), grid, iters, s), "moe_peak_lds"))
    total = float(grid) * WAVES_PER_WG * 8 * iters * 1024
    return {"tb_s": round(total / dt / 1e12, 2), "per_cu_gb_s": round(total / dt / 1e9 / num_cu, 1),
            "ms": round(dt * 1e3, 2)}


def copy(num_cu: int, nbytes: int = 1 << 30, wg_per_cu: int = 8) -> dict:
    """HBM stream copy with 16-byte loads and stores: (read + write bytes) / time."""
    import torch
    lib = load()
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dt = _timed(lambda s: _check(lib.moe_peak_copy(src.data_ptr(), dst.data_ptr(), nbytes,
                                                   num_cu * wg_per_cu, s), "moe_peak_copy"), reps=5)
    return {"gb_s": round(2.0 * nbytes / dt / 1e9, 1), "bytes": nbytes}
