"""MI355X (gfx950) fused exact-attention forward.

A thin binding over the C-ABI library ``libattn_fwd.so`` (declared in
``include/attn.h``): argument checks, output allocation and marshalling only;
every step of the computation runs in the library's HIP kernels.  PyTorch
provides device memory and the current stream.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libattn_fwd.so")

ATTN_F16, ATTN_BF16, ATTN_FP8_E4M3, ATTN_F32, ATTN_FP8_E5M2 = 0, 1, 2, 3, 4
ATTN_SCHED_DEFAULT, ATTN_SCHED_CLASSIC, ATTN_SCHED_PINGPONG, ATTN_SCHED_DEPHASED = 0, 1, 2, 3

_lib = None


class AttnError(RuntimeError):
    pass


def load_library(path: str | None = None) -> ctypes.CDLL:
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    path = path or LIB_PATH
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise AttnError(f"HIP library not built: {path} (run exact_attention_32_amd.build.build())")
    L = ctypes.CDLL(path)
    vp, ci, cf = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    L.attn_fwd.restype = ci
    L.attn_fwd.argtypes = [vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, cf, ci, vp]
    L.attn_fwd_fp8.restype = ci
    L.attn_fwd_fp8.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, cf, vp]
    L.attn_fwd_fp8_e5m2.restype = ci
    L.attn_fwd_fp8_e5m2.argtypes = L.attn_fwd_fp8.argtypes
    L.attn_status_string.restype = ctypes.c_char_p
    L.attn_status_string.argtypes = [ci]
    L.attn_fwd_plan.restype = ci
    L.attn_fwd_plan.argtypes = [ci, ci, ci, ci, ci, ci, ci] + [ctypes.POINTER(ci)] * 4
    L.attn_quantize_e4m3.restype = ci
    L.attn_quantize_e4m3.argtypes = [vp, ci, vp, vp, ci, ci, ci, ci, vp]
    L.attn_quantize_e5m2.restype = ci
    L.attn_quantize_e5m2.argtypes = L.attn_quantize_e4m3.argtypes
    L.attn_fwd_set_policy.restype = ci
    L.attn_fwd_set_policy.argtypes = [ci, ci, ci, ci, ci]
    L.attn_fwd_schedule.restype = ci
    L.attn_fwd_schedule.argtypes = [ci, ci, ci]
    L.attn_quantize_qkv.restype = ci
    L.attn_quantize_qkv.argtypes = [vp, vp, vp, ci, ci] + [vp] * 6 + [ci] * 5 + [vp]
    L.attn_qk_rmsnorm.restype = ci
    L.attn_qk_rmsnorm.argtypes = [vp] * 6 + [ci] * 5 + [cf, ci, vp]
    L.attn_qk_rmsnorm_split.restype = ci
    L.attn_qk_rmsnorm_split.argtypes = [vp] * 5 + [ci] * 5 + [cf, ci, vp]
    L.attn_fwd_qnorm.restype = ci
    L.attn_fwd_qnorm.argtypes = [vp] * 7 + [ci] * 6 + [cf, ci, vp]
    if path == LIB_PATH:
        _lib = L
    return L


def status_string(code: int) -> str:
    return load_library().attn_status_string(int(code)).decode()


def _check(rc: int):
    if rc != 0:
        raise AttnError(f"attn: {status_string(rc)} (status {rc})")


def plan(B, H, S_q, S_k, d, causal=False, dtype=ATTN_BF16):
    """(queries per workgroup, keys per tile, waves per workgroup, workgroups) the library launches."""
    out = [ctypes.c_int() for _ in range(4)]
    _check(load_library().attn_fwd_plan(B, H, S_q, S_k, d, int(bool(causal)), dtype, *[ctypes.byref(x) for x in out]))
    return tuple(x.value for x in out)


def set_policy(schedule: int = ATTN_SCHED_DEFAULT, qb: int = 1, nw: int = 8, ns: int = 4, bk: int = 64):
    """Process-wide choice of the f16/bf16 schedule and tile shape: qb 32-query blocks per wave,
    nw waves, ns LDS stages, bk keys per tile (tuning and tests); ATTN_SCHED_DEFAULT restores the
    measured policy table."""
    _check(load_library().attn_fwd_set_policy(int(schedule), int(qb), int(nw), int(ns), int(bk)))


KERNEL_NAMES = {ATTN_SCHED_CLASSIC: "attn_fwd_kernel", ATTN_SCHED_PINGPONG: "attn_fwd_pp_kernel",
                ATTN_SCHED_DEPHASED: "attn_fwd_dp_kernel"}


def kernel_name(d: int, causal: bool, dtype: int) -> str:
    """Name of the HIP kernel that fwd / fwd_fp8 launch for these arguments under the current policy."""
    if dtype in (ATTN_FP8_E4M3, ATTN_FP8_E5M2):
        return "attn_fwd_fp8_kernel"
    r = load_library().attn_fwd_schedule(int(d), int(bool(causal)), int(dtype))
    if r < 0:
        _check(-r)
    return KERNEL_NAMES[r]


def _shapes(q, k, v):
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, H, S, d]")
    B, H, S_q, d = q.shape
    if k.shape[0] != B or k.shape[1] != H or k.shape[3] != d or v.shape != k.shape:
        raise ValueError(f"shape mismatch: q {tuple(q.shape)} k {tuple(k.shape)} v {tuple(v.shape)}")
    for t in (q, k, v):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("q, k, v must be contiguous device tensors")
        if t.device != q.device:
            raise ValueError("q, k, v must be on one device")
    return B, H, S_q, k.shape[2], d


def _stream(dev):
    """dev's current stream as the library's stream argument."""
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _call(dev, fn, *args):
    """Run a library entry point on dev's current stream with dev the current device: the library
    launches on the current device, whatever device the stream belongs to."""
    if dev.index is None or dev.index == torch.cuda.current_device():
        return fn(*args, _stream(dev))
    with torch.cuda.device(dev):
        return fn(*args, _stream(dev))


def _check_buffer(t, name: str, shape, dtype, device):
    """A caller-supplied output must be exactly what the kernel writes: its shape, type, device and
    a dense layout (the library writes through the raw pointer)."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, not {tuple(t.shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, not {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, not {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = False, scale: float | None = None,
        out: torch.Tensor | None = None, lse: torch.Tensor | None = None, want_lse: bool = True):
    """Exact attention forward for tensors [B, H, S, d] -> (O, LSE).

    fp16 / bf16: O has q's dtype.  float8_e4m3fn / float8_e5m2 (fp8 codes with unit descales; see
    fwd_fp8 for block-scaled codes): O is bf16.  LSE is fp32 [B, H, S_q] (natural log), or None if
    want_lse is False.
    """
    B, H, S_q, S_k, d = _shapes(q, k, v)
    if q.dtype != k.dtype or q.dtype != v.dtype:
        raise ValueError("q, k, v must share a dtype")
    dt = {torch.bfloat16: ATTN_BF16, torch.float16: ATTN_F16, torch.float8_e4m3fn: ATTN_FP8_E4M3,
          torch.float8_e5m2: ATTN_FP8_E5M2}.get(q.dtype)
    if dt is None:
        raise ValueError(f"unsupported dtype {q.dtype}")
    if scale is None:
        scale = d ** -0.5
    out_dt = torch.bfloat16 if dt in (ATTN_FP8_E4M3, ATTN_FP8_E5M2) else q.dtype
    if out is None:
        out = torch.empty(q.shape, dtype=out_dt, device=q.device)
    _check_buffer(out, "out", (B, H, S_q, d), out_dt, q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, H, S_q), dtype=torch.float32, device=q.device)
    if lse is not None:
        _check_buffer(lse, "lse", (B, H, S_q), torch.float32, q.device)
    rc = _call(q.device, load_library().attn_fwd, q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
               lse.data_ptr() if lse is not None else None, B, H, S_q, S_k, d,
               int(bool(causal)), float(scale), dt)
    _check(rc)
    return out, lse


def fwd_qnorm(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, q_rstd: torch.Tensor, w_q: torch.Tensor,
              causal: bool = False, scale: float | None = None, out: torch.Tensor | None = None,
              lse: torch.Tensor | None = None, want_lse: bool = True):
    """fwd of RMSNorm(q) with k and v, the norm folded into the kernel's Q loads: q raw, q_rstd
    [B, S_q] fp32 from qk_rmsnorm_split, w_q [H*d] in q's dtype, k already normalised.  The same
    bits as fwd(qk_rmsnorm(q, k, w_q, w_k)[0], k_norm, v).  bf16 / fp16 only."""
    B, H, S_q, S_k, d = _shapes(q, k, v)
    if q.dtype != k.dtype or q.dtype != v.dtype:
        raise ValueError("q, k, v must share a dtype")
    dt = {torch.bfloat16: ATTN_BF16, torch.float16: ATTN_F16}.get(q.dtype)
    if dt is None:
        raise ValueError(f"unsupported dtype {q.dtype}")
    _check_buffer(q_rstd, "q_rstd", (B, S_q), torch.float32, q.device)
    _check_buffer(w_q, "w_q", (H * d,), q.dtype, q.device)
    if scale is None:
        scale = d ** -0.5
    if out is None:
        out = torch.empty(q.shape, dtype=q.dtype, device=q.device)
    _check_buffer(out, "out", (B, H, S_q, d), q.dtype, q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, H, S_q), dtype=torch.float32, device=q.device)
    if lse is not None:
        _check_buffer(lse, "lse", (B, H, S_q), torch.float32, q.device)
    rc = _call(q.device, load_library().attn_fwd_qnorm, q.data_ptr(), k.data_ptr(), v.data_ptr(), q_rstd.data_ptr(),
               w_q.data_ptr(), out.data_ptr(), lse.data_ptr() if lse is not None else None, B, H, S_q,
               S_k, d, int(bool(causal)), float(scale), dt)
    _check(rc)
    return out, lse


_FP8_TORCH = {"e4m3": torch.float8_e4m3fn, "e5m2": torch.float8_e5m2}


def fwd_fp8(q, k, v, q_descale, k_descale, v_descale, causal: bool = False, scale: float | None = None,
            out: torch.Tensor | None = None, lse: torch.Tensor | None = None, want_lse: bool = True,
            fmt: str = "e4m3"):
    """Block-scaled fp8 attention -> (O bf16, LSE fp32).

    q, k, v hold OCP codes of the format ``fmt`` ("e4m3" or "e5m2") as uint8 or as the matching
    torch float8 dtype; descales are fp32 [B, H, ceil(S/128)].
    """
    if fmt not in _FP8_TORCH:
        raise ValueError(f"fmt must be 'e4m3' or 'e5m2', not {fmt!r}")
    B, H, S_q, S_k, d = _shapes(q, k, v)
    for t in (q, k, v):
        if t.dtype not in (torch.uint8, _FP8_TORCH[fmt]):
            raise ValueError(f"fp8 inputs must be uint8 codes or {_FP8_TORCH[fmt]}")
    for t, n, s in ((q_descale, "q_descale", S_q), (k_descale, "k_descale", S_k), (v_descale, "v_descale", S_k)):
        _check_buffer(t, n, (B, H, (s + 127) // 128), torch.float32, q.device)
    if scale is None:
        scale = d ** -0.5
    if out is None:
        out = torch.empty((B, H, S_q, d), dtype=torch.bfloat16, device=q.device)
    _check_buffer(out, "out", (B, H, S_q, d), torch.bfloat16, q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, H, S_q), dtype=torch.float32, device=q.device)
    if lse is not None:
        _check_buffer(lse, "lse", (B, H, S_q), torch.float32, q.device)
    L = load_library()
    entry = L.attn_fwd_fp8 if fmt == "e4m3" else L.attn_fwd_fp8_e5m2
    rc = _call(q.device, entry, q.data_ptr(), k.data_ptr(), v.data_ptr(), q_descale.data_ptr(), k_descale.data_ptr(),
               v_descale.data_ptr(), out.data_ptr(), lse.data_ptr() if lse is not None else None, B, H, S_q, S_k,
               d, int(bool(causal)), float(scale))
    _check(rc)
    return out, lse


def quantize_fp8(x: torch.Tensor, fmt: str = "e4m3", codes: torch.Tensor | None = None,
                 descale: torch.Tensor | None = None):
    """Per-(b, h, 128-row block) fp8 quantisation of x [B, H, S, d] (fp32, bf16 or fp16) on the GPU.

    fmt is "e4m3" or "e5m2".  Returns (codes uint8 [B, H, S, d], descale fp32 [B, H, ceil(S/128)]),
    the inputs of fwd_fp8 with the same fmt.
    """
    if fmt not in _FP8_TORCH:
        raise ValueError(f"fmt must be 'e4m3' or 'e5m2', not {fmt!r}")
    if x.dim() != 4 or not x.is_cuda or not x.is_contiguous():
        raise ValueError("x must be a contiguous [B, H, S, d] device tensor")
    dt = {torch.float32: ATTN_F32, torch.bfloat16: ATTN_BF16, torch.float16: ATTN_F16}.get(x.dtype)
    if dt is None:
        raise ValueError(f"unsupported dtype {x.dtype}")
    B, H, S, d = x.shape
    if codes is None:
        codes = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    if descale is None:
        descale = torch.empty((B, H, (S + 127) // 128), dtype=torch.float32, device=x.device)
    _check_buffer(codes, "codes", tuple(x.shape), torch.uint8, x.device)
    _check_buffer(descale, "descale", (B, H, (S + 127) // 128), torch.float32, x.device)
    L = load_library()
    entry = L.attn_quantize_e4m3 if fmt == "e4m3" else L.attn_quantize_e5m2
    rc = _call(x.device, entry, x.data_ptr(), dt, codes.data_ptr(), descale.data_ptr(), B, H, S, d)
    _check(rc)
    return codes, descale


def quantize_qkv(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, fmt: str = "e4m3"):
    """Per-block fp8 quantisation of q [B, H, S_q, d], k and v [B, H, S_k, d] in one launch.

    Returns ((q_codes, k_codes, v_codes), (q_descale, k_descale, v_descale)), bit-identical to three
    quantize_fp8 calls: the inputs of fwd_fp8 with the same fmt.
    """
    if fmt not in _FP8_TORCH:
        raise ValueError(f"fmt must be 'e4m3' or 'e5m2', not {fmt!r}")
    B, H, S_q, S_k, d = _shapes(q, k, v)
    if q.dtype != k.dtype or q.dtype != v.dtype:
        raise ValueError("q, k, v must share a dtype")
    dt = {torch.float32: ATTN_F32, torch.bfloat16: ATTN_BF16, torch.float16: ATTN_F16}.get(q.dtype)
    if dt is None:
        raise ValueError(f"unsupported dtype {q.dtype}")
    codes = tuple(torch.empty(t.shape, dtype=torch.uint8, device=t.device) for t in (q, k, v))
    descales = tuple(torch.empty((B, H, (s + 127) // 128), dtype=torch.float32, device=q.device)
                     for s in (S_q, S_k, S_k))
    rc = _call(q.device, load_library().attn_quantize_qkv, q.data_ptr(), k.data_ptr(), v.data_ptr(), dt,
               ATTN_FP8_E4M3 if fmt == "e4m3" else ATTN_FP8_E5M2,
               *[c.data_ptr() for c in codes], *[x.data_ptr() for x in descales],
               B, H, S_q, S_k, d)
    _check(rc)
    return codes, descales


def quantize_e4m3(x: torch.Tensor, codes: torch.Tensor | None = None, descale: torch.Tensor | None = None):
    """quantize_fp8 with fmt="e4m3"."""
    return quantize_fp8(x, "e4m3", codes, descale)


def quantize_e5m2(x: torch.Tensor, codes: torch.Tensor | None = None, descale: torch.Tensor | None = None):
    """quantize_fp8 with fmt="e5m2"."""
    return quantize_fp8(x, "e5m2", codes, descale)


def qk_rmsnorm(q: torch.Tensor, k: torch.Tensor, w_q: torch.Tensor, w_k: torch.Tensor, eps: float = 1e-6,
               q_out: torch.Tensor | None = None, k_out: torch.Tensor | None = None, inplace: bool = False):
    """RMSNorm of q [B, H, S_q, d] and k [B, H, S_k, d] across heads (one RMS per token over all
    H*d channels), times the per-channel weights w_q, w_k [H*d]; bf16 or fp16 throughout.

    Returns (q_norm, k_norm); with inplace=True they are q and k themselves.
    """
    B, H, S_q, S_k, d = _shapes(q, k, k)
    for t in (q, k, w_q, w_k):
        if t.dtype != q.dtype or not t.is_cuda or not t.is_contiguous() or t.device != q.device:
            raise ValueError("q, k, w_q, w_k must be contiguous device tensors of one dtype")
    if w_q.numel() != H * d or w_k.numel() != H * d:
        raise ValueError("w_q and w_k must have H*d entries")
    dt = {torch.bfloat16: ATTN_BF16, torch.float16: ATTN_F16}.get(q.dtype)
    if dt is None:
        raise ValueError(f"unsupported dtype {q.dtype}")
    if inplace:
        q_out, k_out = q, k
    q_out = torch.empty_like(q) if q_out is None else q_out
    k_out = torch.empty_like(k) if k_out is None else k_out
    for t, ref in ((q_out, q), (k_out, k)):
        if t.shape != ref.shape or t.dtype != ref.dtype or not t.is_contiguous() or t.device != ref.device:
            raise ValueError("outputs must be contiguous tensors of the inputs' shape and dtype")
    rc = _call(q.device, load_library().attn_qk_rmsnorm, q.data_ptr(), k.data_ptr(), w_q.data_ptr(), w_k.data_ptr(),
               q_out.data_ptr(), k_out.data_ptr(), B, H, S_q, S_k, d, float(eps), dt)
    _check(rc)
    return q_out, k_out


def qk_rmsnorm_split(q: torch.Tensor, k: torch.Tensor, w_k: torch.Tensor, eps: float = 1e-6,
                     q_rstd: torch.Tensor | None = None, k_out: torch.Tensor | None = None, inplace: bool = False):
    """K normalised as qk_rmsnorm does it; for Q only the per-token factor r [B, S_q] (fp32), which
    fwd_qnorm folds into its Q loads.  Returns (q_rstd, k_norm); with inplace=True k_norm is k."""
    B, H, S_q, S_k, d = _shapes(q, k, k)
    for t in (q, k, w_k):
        if t.dtype != q.dtype or not t.is_cuda or not t.is_contiguous() or t.device != q.device:
            raise ValueError("q, k, w_k must be contiguous device tensors of one dtype")
    if w_k.numel() != H * d:
        raise ValueError("w_k must have H*d entries")
    dt = {torch.bfloat16: ATTN_BF16, torch.float16: ATTN_F16}.get(q.dtype)
    if dt is None:
        raise ValueError(f"unsupported dtype {q.dtype}")
    if q_rstd is None:
        q_rstd = torch.empty((B, S_q), dtype=torch.float32, device=q.device)
    _check_buffer(q_rstd, "q_rstd", (B, S_q), torch.float32, q.device)
    if inplace:
        k_out = k
    k_out = torch.empty_like(k) if k_out is None else k_out
    _check_buffer(k_out, "k_out", tuple(k.shape), k.dtype, k.device)
    rc = _call(q.device, load_library().attn_qk_rmsnorm_split, q.data_ptr(), k.data_ptr(), w_k.data_ptr(),
               q_rstd.data_ptr(), k_out.data_ptr(), B, H, S_q, S_k, d, float(eps), dt)
    _check(rc)
    return q_rstd, k_out
