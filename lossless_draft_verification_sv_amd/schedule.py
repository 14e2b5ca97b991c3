"""Step-time tables for the hardware-aware prefix scheduler (sv_schedule_prefix).

The scheduler of the DSpark paper review (4.2.2) looks up the time of a target step that
verifies n tokens in a table measured when the engine starts. Here a step is the verify call of
this library plus a target forward pass. The verify part is measured on this device: the
flattened verify call (sv_verify_ragged) is timed at a few token counts between B (no drafts)
and B*(K+1) (every draft) and interpolated. The target part has no model in this library, so it
is a roofline model of a dense decoder on this GPU: the weights are read once per step and the
matrix work is 2 * params * n flops, done in tiles of `tile` tokens:

    t_target(n) = max(weight_bytes / hbm, 2 * params * ceil(n / tile) * tile / mfma)

which is flat while the step is bound by the weight read and rises in jumps of one tile once
the matrix work dominates, the shape the pages describe. Its parameters are inputs, not
measurements.
"""
from __future__ import annotations

import numpy as np
import torch

from ._binding import load_library


def synthetic_target_step_us(n, params: float = 8.0e9, bytes_per_param: float = 2.0,
                             hbm_gbps: float = 8000.0, mfma_tflops: float = 2500.0,
                             tile: int = 256) -> np.ndarray:
    """Roofline time (us) of a dense decoder step over n tokens (see the module docstring)."""
    n = np.asarray(n, dtype=np.float64)
    read = params * bytes_per_param / (hbm_gbps * 1e9) * 1e6
    work = 2.0 * params * np.ceil(n / tile) * tile / (mfma_tflops * 1e12) * 1e6
    return np.maximum(read, work)


def measure_verify_step_us(B: int, K: int, V: int, dtype: str = "bf16", points: int = 9,
                           reps: int = 20, device: str = "cuda:0") -> np.ndarray:
    """Time (us) of sv_verify_ragged for every total token count n = B .. B*(K+1), measured
    at `points` counts (drafts spread evenly over the requests, all sampling at temperature
    1) and interpolated linearly; entries below B are set to the value at B."""
    import lossless_draft_verification_sv_amd as sv

    lib = load_library()
    dev = torch.device(device)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    gen = torch.Generator(device=dev).manual_seed(0)
    target = torch.randn(B * (K + 1), V, device=dev, dtype=torch.float32, generator=gen).to(tdt)
    draft = torch.randn(B * K, V, device=dev, dtype=torch.float32, generator=gen).to(tdt)
    tokens = torch.randint(0, V, (B, K), device=dev, dtype=torch.int32, generator=gen)
    uni = torch.rand(B, K, device=dev, generator=gen)
    res = torch.rand(B, device=dev, generator=gen)
    temps = torch.ones(B, device=dev)
    ns = np.unique(np.linspace(0, B * K, points).round().astype(int))
    times = []
    for total in ns:
        k = np.full(B, total // B, np.int32)
        k[: total % B] += 1
        ts = np.concatenate([[0], np.cumsum(k + 1)[:-1]]).astype(np.int32)
        ds = np.concatenate([[0], np.cumsum(k)[:-1]]).astype(np.int32)
        args = [torch.from_numpy(a).to(dev) for a in (k, ts, ds)]
        for _ in range(3):
            sv.sv_verify_ragged(target, draft, tokens, uni, res, temps, *args)
        torch.cuda.synchronize(dev)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            sv.sv_verify_ragged(target, draft, tokens, uni, res, temps, *args)
        e1.record()
        torch.cuda.synchronize(dev)
        times.append(e0.elapsed_time(e1) * 1e3 / reps)
    del lib
    n_all = np.arange(B + B * K + 1)
    return np.interp(n_all - B, ns, np.asarray(times))


def step_time_table(B: int, K: int, V: int, dtype: str = "bf16", **target_model) -> np.ndarray:
    """step_time[n] (us) for n = 0 .. B + B*K: measured verify time plus the synthetic target
    step, float32, ready for sv_schedule_prefix."""
    n = np.arange(B + B * K + 1)
    verify = measure_verify_step_us(B, K, V, dtype)
    return (verify + synthetic_target_step_us(n, **target_model)).astype(np.float32)
