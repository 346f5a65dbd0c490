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


def ulp_distance(a: np.ndarray, b: np.ndarray, dtype: str) -> np.ndarray:
    """Distance in units in the last place between two arrays of values representable in the output
    type (bf16 or f16), counted along the ordered bit patterns (a step across a binade boundary is
    one ulp; +0 and -0 are the same point)."""
    dt = _OUT_DT[dtype]
    ia = torch.from_numpy(np.ascontiguousarray(a)).to(dt).view(torch.int16).numpy().astype(np.int64)
    ib = torch.from_numpy(np.ascontiguousarray(b)).to(dt).view(torch.int16).numpy().astype(np.int64)
    # sign-magnitude -> ordered integers
    oa = np.where(ia < 0, -(ia & 0x7FFF), ia)
    ob = np.where(ib < 0, -(ib & 0x7FFF), ib)
    return np.abs(oa - ob)


# E4M3 round-to-nearest: relative error at most 2^-4 for normal values (3 mantissa bits); a
# subnormal (below 2^-6) is off by at most 2^-10 in absolute terms
E4M3_REL = 2.0 ** -4
E4M3_SUB_ABS = 2.0 ** -10
FEW_KEYS = 16


def fp8_few_key_tolerance(oracle, q, k, v, o_ref, causal: bool, scale: float):
    """Per-element tolerance on O for the fp8 path's rows with fewer than FEW_KEYS visible keys,
    from the rounding of the probabilities to E4M3 alone; NaN elsewhere (and None when no row is
    that short).

    With weights p_j (the exact softmax row, from the oracle) rounded to p_j (1 + e_j), |e_j| <= u,
    the normalised result moves by sum_j p_j e_j (v_j - O) / sum_j p_j (1 + e_j), at most
    u / (1 - u) * sum_j p_j |v_j - O| per output element; a subnormal probability adds at most
    2^-10 over the row's probability mass, which the first key tile puts at 2^5 or more, per key.
    Over many keys these errors average out; over a handful they do not, and the literal fp8
    tolerance is then below what any E4M3 rounding of P allows.  The bf16 rounding of O itself
    (2^-9 relative) and 1e-4 of accumulation slack are added."""
    B, H, Sq, d = q.shape
    Sk = k.shape[2]
    nvis = np.array([min(i + 1, Sk) if causal else Sk for i in range(Sq)])
    short = np.nonzero(nvis < FEW_KEYS)[0]
    if short.size == 0:
        return None
    tol = np.full(o_ref.shape, np.nan)
    i0, nr = int(short.min()), int(short.max() - short.min() + 1)
    u = E4M3_REL
    for bh in range(B * H):
        b, h = divmod(bh, H)
        P = oracle.softmax_block(q, k, causal, scale, bh, i0, nr)
        for i in short:
            n = int(nvis[i])
            dev = np.abs(v[b, h, :n] - o_ref[b, h, i][None, :])
            rounding = u / (1.0 - u) * (P[i - i0, :n, None] * dev).sum(0)
            sub = n * (E4M3_SUB_ABS / 32.0) * dev.max(0)
            tol[b, h, i] = rounding + sub + 2.0 ** -9 * np.abs(o_ref[b, h, i]) + 1e-4
    return tol


def compare(o_gpu: np.ndarray, lse_gpu: np.ndarray, o_ref: np.ndarray, lse_ref: np.ndarray, dtype: str,
            few_key_tol: np.ndarray | None = None):
    """Error statistics and the pass decision.

    Gate, per element of O: |O - O_ref| <= tol (1e-2 for f16/bf16, 5e-2 for fp8), or else O is
    within one ulp of the correctly rounded value RN(O_ref).  The second case is counted, in two
    classes: RN(O_ref) itself misses tol (bf16 spacing is 2^-6 in [2, 4) and 2^-5 in [4, 8), so no
    output of the type meets tol there), or RN(O_ref) meets tol and O is its neighbour.
    few_key_tol (fp8 only, see fp8_few_key_tolerance): where finite and above tol, the tolerance of
    that element; elements that pass only by it are counted.
    LSE: max |LSE - LSE_ref| <= 1e-3.  The raw max |O - O_ref| (and where it is: the (b, h, i, t) index),
    the mean and RMS error and the rounding floor are reported.
    """
    tol = TOL_O[dtype]
    err = np.abs(o_gpu - o_ref)
    floor = rounding_floor(o_ref, dtype)
    lerr = np.abs(lse_gpu - lse_ref)
    over = err > tol
    few_key = np.zeros_like(over)
    if few_key_tol is not None:
        few_key = over & np.isfinite(few_key_tol) & (err <= np.where(np.isfinite(few_key_tol), few_key_tol, 0.0))
        over = over & ~few_key
    rounded = torch.from_numpy(np.ascontiguousarray(o_ref)).to(_OUT_DT[dtype]).double().numpy()
    one_ulp = over & (ulp_distance(o_gpu, rounded, dtype) <= 1)
    failed = over & ~one_ulp
    stats = {
        "max_abs_err_O": float(err.max()) if err.size else 0.0,
        "worst_O_at": tuple(int(i) for i in np.unravel_index(int(np.argmax(err)), err.shape)) if err.size else None,
        "mean_abs_err_O": float(err.mean()) if err.size else 0.0,
        "rms_err_O": float(np.sqrt(np.mean(err ** 2))) if err.size else 0.0,
        "floor_O": float(floor.max()) if floor.size else 0.0,
        "n_elements": int(err.size),
        "n_over_tol": int(over.sum()),
        "n_one_ulp_rn_misses_tol": int((one_ulp & (floor > tol)).sum()),
        "n_one_ulp_neighbour": int((one_ulp & (floor <= tol)).sum()),
        "n_failed": int(failed.sum()),
        "n_fp8_few_key_rounding": int(few_key.sum()),
        "max_abs_err_LSE": float(lerr.max()) if lerr.size else 0.0,
        "finite": bool(np.all(np.isfinite(o_gpu)) and np.all(np.isfinite(lse_gpu))),
    }
    stats["pass"] = bool(stats["finite"] and stats["n_failed"] == 0 and stats["max_abs_err_LSE"] <= TOL_LSE)
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
