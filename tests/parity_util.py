"""Shared helpers of the GPU parity tests: run the HIP path, run the oracle, compare."""
from __future__ import annotations

import numpy as np
import torch

from exact_attention_32_amd import inputs as I

# Tolerances (max abs error against the fp64 oracle).
TOL_O = {"f16": 1e-2, "bf16": 1e-2, "fp8": 5e-2, "e5m2": 5e-2}
TOL_LSE = 1e-3

_OUT_DT = {"f16": torch.float16, "bf16": torch.bfloat16, "fp8": torch.bfloat16, "e5m2": torch.bfloat16}


def say(msg: str):
    print(msg, flush=True)


def oracle_inputs(x: I.Inputs, oracle):
    """Exact fp64 values of the inputs (fp8: decoded codes times descales)."""
    if I.is_fp8(x.work.dtype):
        fmt = "e5m2" if x.work.dtype == "e5m2" else "e4m3"
        return tuple(oracle.decode_fp8_blocks(c.numpy(), ds.numpy(), fmt)
                     for c, ds in ((x.q, x.q_descale), (x.k, x.k_descale), (x.v, x.v_descale)))
    return x.q.double().numpy(), x.k.double().numpy(), x.v.double().numpy()


def run_gpu(x: I.Inputs, dev="cuda:0"):
    import exact_attention_32_amd as ea

    w = x.work
    if I.is_fp8(w.dtype):
        o, lse = ea.fwd_fp8(x.q.to(dev), x.k.to(dev), x.v.to(dev), x.q_descale.to(dev), x.k_descale.to(dev),
                            x.v_descale.to(dev), causal=w.causal, scale=w.scale,
                            fmt="e5m2" if w.dtype == "e5m2" else "e4m3")
    else:
        o, lse = ea.fwd(x.q.to(dev), x.k.to(dev), x.v.to(dev), causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    return o, lse


def rounding_floor(o_ref: np.ndarray, dtype: str) -> np.ndarray:
    """|round(O_ref) - O_ref| elementwise: the error of a correctly rounded output."""
    t = torch.from_numpy(np.ascontiguousarray(o_ref)).to(_OUT_DT[dtype]).double().numpy()
    return np.abs(t - o_ref)


def compare(o_gpu: np.ndarray, lse_gpu: np.ndarray, o_ref: np.ndarray, lse_ref: np.ndarray, dtype: str):
    """Error statistics and the pass decision.

    Gate: every element |O - O_ref| <= tol + |round(O_ref) - O_ref| (the stated
    tolerance on top of the output's own rounding), and max |LSE - LSE_ref| <= 1e-3.
    """
    err = np.abs(o_gpu - o_ref)
    floor = rounding_floor(o_ref, dtype)
    excess = err - floor
    lerr = np.abs(lse_gpu - lse_ref)
    stats = {
        "max_abs_err_O": float(err.max()),
        "rms_err_O": float(np.sqrt(np.mean(err ** 2))),
        "floor_O": float(floor.max()),
        "max_err_over_floor_O": float(excess.max()),
        "max_abs_err_LSE": float(lerr.max()),
        "finite": bool(np.all(np.isfinite(o_gpu)) and np.all(np.isfinite(lse_gpu))),
    }
    stats["pass"] = bool(stats["finite"] and excess.max() <= TOL_O[dtype] and lerr.max() <= TOL_LSE)
    return stats


def sample_rows(w: I.Workload, n_random: int, seed: int):
    """(b*H + h, i) rows: first/last rows, tile edges, and random rows, over several heads."""
    rng = np.random.Generator(np.random.PCG64(seed))
    BH = w.B * w.H
    fixed = [0, 1, 2, 31, 32, 63, 64, 127, 128, 129, 255, 256, w.S_q // 2, w.S_q - 2, w.S_q - 1]
    fixed = sorted({i for i in fixed if 0 <= i < w.S_q})
    rows = []
    for j, i in enumerate(fixed):
        rows.append((int((j * 7919) % BH), i))
        rows.append((BH - 1, i))
    for _ in range(n_random):
        rows.append((int(rng.integers(BH)), int(rng.integers(w.S_q))))
    return np.array(sorted(set(rows)), dtype=np.int64)
