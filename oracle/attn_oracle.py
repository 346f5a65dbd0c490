"""ctypes wrapper around the fp64 CPU oracle (``attn_oracle.c``).

TEST INFRASTRUCTURE ONLY: tests, the smoke check and the benchmark's
CPU-baseline leg use this to check the GPU path; the product path never
imports it.  It shares no code with the GPU library.

The oracle computes plain softmax attention (the "standard attention" that the
FlashAttention-3 deep dive (techknowgenie) opens with) in fp64 with an explicit
softmax matrix, plus the key-block online-softmax loop of that page's section 2
for the two-pass = online check.  See the header of ``attn_oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "attn_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(src: str = SRC, out: str = LIB) -> str:
    """Compile the oracle with gcc into a shared library; returns its path."""
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-shared", "-fPIC", src, "-o", out,
           "-lpthread", "-lm"]
    subprocess.run(cmd, check=True)
    return out


_dptr = ctypes.POINTER(ctypes.c_double)
_FMT = {"e4m3": 0, "e5m2": 1}


def default_threads() -> int:
    """Worker threads for the oracle: this process's CPUs, at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _p(a: np.ndarray):
    return a.ctypes.data_as(_dptr)


def _f64(a) -> np.ndarray:
    a = np.asarray(a, dtype=np.float64)
    return np.ascontiguousarray(a)


class Oracle:
    """fp64 attention oracle.  Arrays are numpy, layout [B, H, S, d]."""

    def __init__(self, lib_path: str | None = None):
        path = lib_path or LIB
        if lib_path is None and not os.path.exists(path):
            build()
        self.path = path
        L = ctypes.CDLL(path)
        ci, cd = ctypes.c_int, ctypes.c_double
        L.oracle_attn_explicit.restype = ci
        L.oracle_attn_explicit.argtypes = [_dptr] * 5 + [ci] * 6 + [cd, ci]
        L.oracle_attn_online.restype = ci
        L.oracle_attn_online.argtypes = [_dptr] * 5 + [ci] * 6 + [cd, ci, ci]
        L.oracle_attn_rows.restype = ci
        L.oracle_attn_rows.argtypes = [_dptr] * 5 + [ci] * 6 + [cd, ctypes.c_void_p, ctypes.c_int64, ci]
        L.oracle_softmax_block.restype = ci
        L.oracle_softmax_block.argtypes = [_dptr] * 3 + [ci] * 6 + [cd, ctypes.c_int64, ci, ci]
        L.oracle_e4m3_value.restype = cd
        L.oracle_e4m3_value.argtypes = [ctypes.c_uint8]
        L.oracle_decode_e4m3_blocks.restype = ci
        L.oracle_decode_e4m3_blocks.argtypes = [ctypes.c_void_p, ctypes.c_void_p] + [ci] * 5 + [_dptr]
        L.oracle_e4m3_encode.restype = ctypes.c_uint8
        L.oracle_e4m3_encode.argtypes = [ctypes.c_double]
        L.oracle_quantize_e4m3_blocks.restype = ci
        L.oracle_quantize_e4m3_blocks.argtypes = [ctypes.c_void_p] + [ci] * 5 + [ctypes.c_void_p, ctypes.c_void_p]
        L.oracle_e5m2_value.restype = cd
        L.oracle_e5m2_value.argtypes = [ctypes.c_uint8]
        L.oracle_fp8_encode.restype = ctypes.c_uint8
        L.oracle_fp8_encode.argtypes = [ctypes.c_double, ci]
        L.oracle_quantize_fp8_blocks.restype = ci
        L.oracle_quantize_fp8_blocks.argtypes = [ctypes.c_void_p] + [ci] * 6 + [ctypes.c_void_p, ctypes.c_void_p]
        L.oracle_decode_fp8_blocks.restype = ci
        L.oracle_decode_fp8_blocks.argtypes = [ctypes.c_void_p, ctypes.c_void_p] + [ci] * 6 + [_dptr]
        L.oracle_rmsnorm_across_heads.restype = ci
        L.oracle_rmsnorm_across_heads.argtypes = [_dptr, _dptr] + [ci] * 4 + [cd, _dptr]
        self.L = L
        self.last_threads = 0

    @staticmethod
    def _shapes(q, k, v):
        if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
            raise ValueError("q, k, v must be [B, H, S, d]")
        B, H, Sq, d = q.shape
        if k.shape[:2] != (B, H) or v.shape != k.shape or k.shape[3] != d:
            raise ValueError("shape mismatch")
        return B, H, Sq, k.shape[2], d

    def attention(self, q, k, v, causal: bool, scale: float, nthreads: int = 0):
        """Two-pass fp64 attention with an explicit softmax matrix -> (O, LSE)."""
        q, k, v = _f64(q), _f64(k), _f64(v)
        B, H, Sq, Sk, d = self._shapes(q, k, v)
        o = np.empty((B, H, Sq, d), np.float64)
        lse = np.empty((B, H, Sq), np.float64)
        n = self.L.oracle_attn_explicit(_p(q), _p(k), _p(v), _p(o), _p(lse), B, H, Sq, Sk, d, int(causal),
                                        float(scale), int(nthreads) if nthreads > 0 else default_threads())
        if n < 0:
            raise ValueError("oracle rejected arguments")
        self.last_threads = n
        return o, lse

    def attention_online(self, q, k, v, causal: bool, scale: float, bc: int, nthreads: int = 0):
        """Online-softmax fp64 attention over key blocks of size ``bc`` -> (O, LSE)."""
        q, k, v = _f64(q), _f64(k), _f64(v)
        B, H, Sq, Sk, d = self._shapes(q, k, v)
        o = np.empty((B, H, Sq, d), np.float64)
        lse = np.empty((B, H, Sq), np.float64)
        n = self.L.oracle_attn_online(_p(q), _p(k), _p(v), _p(o), _p(lse), B, H, Sq, Sk, d, int(causal),
                                      float(scale), int(bc), int(nthreads) if nthreads > 0 else default_threads())
        if n < 0:
            raise ValueError("oracle rejected arguments")
        self.last_threads = n
        return o, lse

    def attention_rows(self, q, k, v, causal: bool, scale: float, rows, nthreads: int = 0):
        """O and LSE for selected query rows.  ``rows`` is an (n, 2) array of (b*H + h, i)."""
        q, k, v = _f64(q), _f64(k), _f64(v)
        B, H, Sq, Sk, d = self._shapes(q, k, v)
        rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1, 2))
        n = rows.shape[0]
        o = np.empty((n, d), np.float64)
        lse = np.empty((n,), np.float64)
        r = self.L.oracle_attn_rows(_p(q), _p(k), _p(v), _p(o), _p(lse), B, H, Sq, Sk, d, int(causal),
                                    float(scale), rows.ctypes.data, n, int(nthreads) if nthreads > 0 else default_threads())
        if r < 0:
            raise ValueError("oracle rejected arguments")
        self.last_threads = r
        return o, lse

    def softmax_block(self, q, k, causal: bool, scale: float, bh: int, i0: int, nr: int):
        """Explicit softmax rows [i0, i0+nr) of head bh, shape (nr, S_k)."""
        q, k = _f64(q), _f64(k)
        B, H, Sq, d = q.shape
        Sk = k.shape[2]
        P = np.empty((nr, Sk), np.float64)
        r = self.L.oracle_softmax_block(_p(q), _p(k), _p(P), B, H, Sq, Sk, d, int(causal), float(scale),
                                        int(bh), int(i0), int(nr))
        if r < 0:
            raise ValueError("oracle rejected arguments")
        return P

    def e4m3_table(self) -> np.ndarray:
        """Value of each of the 256 OCP E4M3 codes (NaN for the NaN codes)."""
        return np.array([self.L.oracle_e4m3_value(c) for c in range(256)], dtype=np.float64)

    def decode_e4m3_blocks(self, codes, descale, blk: int = 128) -> np.ndarray:
        """Exact fp64 values of block-scaled e4m3 data: codes [B,H,S,d] uint8, descale [B,H,ceil(S/blk)] fp32."""
        codes = np.ascontiguousarray(np.asarray(codes, dtype=np.uint8))
        descale = np.ascontiguousarray(np.asarray(descale, dtype=np.float32))
        B, H, S, d = codes.shape
        if descale.shape != (B, H, (S + blk - 1) // blk):
            raise ValueError("descale shape must be [B, H, ceil(S/blk)]")
        out = np.empty(codes.shape, np.float64)
        r = self.L.oracle_decode_e4m3_blocks(codes.ctypes.data, descale.ctypes.data, B, H, S, d, blk, _p(out))
        if r < 0:
            raise ValueError("oracle rejected arguments")
        return out


    def e5m2_table(self) -> np.ndarray:
        """Value of each of the 256 OCP E5M2 codes (+-inf, NaN for the specials)."""
        return np.array([self.L.oracle_e5m2_value(c) for c in range(256)], dtype=np.float64)

    def fp8_encode(self, x, fmt: str) -> np.ndarray:
        """Nearest finite code (ties to even, saturating) of format "e4m3" or "e5m2" for each value of x."""
        f = _FMT[fmt]
        x = np.asarray(x, dtype=np.float64)
        return np.array([self.L.oracle_fp8_encode(float(v), f) for v in x.reshape(-1)], dtype=np.uint8).reshape(x.shape)

    def quantize_fp8_blocks(self, x, fmt: str, blk: int = 128):
        """Block quantisation of fp32 x [B,H,S,d] to "e4m3" / "e5m2" -> (codes, descale [B,H,ceil(S/blk)])."""
        x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
        B, H, S, d = x.shape
        codes = np.empty(x.shape, np.uint8)
        descale = np.empty((B, H, (S + blk - 1) // blk), np.float32)
        r = self.L.oracle_quantize_fp8_blocks(x.ctypes.data, B, H, S, d, blk, _FMT[fmt], codes.ctypes.data,
                                              descale.ctypes.data)
        if r < 0:
            raise ValueError("oracle rejected arguments")
        return codes, descale

    def decode_fp8_blocks(self, codes, descale, fmt: str, blk: int = 128) -> np.ndarray:
        """Exact fp64 values of block-scaled "e4m3" / "e5m2" data."""
        codes = np.ascontiguousarray(np.asarray(codes, dtype=np.uint8))
        descale = np.ascontiguousarray(np.asarray(descale, dtype=np.float32))
        B, H, S, d = codes.shape
        if descale.shape != (B, H, (S + blk - 1) // blk):
            raise ValueError("descale shape must be [B, H, ceil(S/blk)]")
        out = np.empty(codes.shape, np.float64)
        r = self.L.oracle_decode_fp8_blocks(codes.ctypes.data, descale.ctypes.data, B, H, S, d, blk, _FMT[fmt], _p(out))
        if r < 0:
            raise ValueError("oracle rejected arguments")
        return out

    def rmsnorm_across_heads(self, x, w, eps: float) -> np.ndarray:
        """fp64 RMSNorm of every token's hidden vector (all heads) of x [B,H,S,d], weight w [H*d]."""
        x = _f64(x)
        w = _f64(w).reshape(-1)
        B, H, S, d = x.shape
        if w.size != H * d:
            raise ValueError("w must have H*d entries")
        out = np.empty_like(x)
        if self.L.oracle_rmsnorm_across_heads(_p(x), _p(w), B, H, S, d, float(eps), _p(out)) < 0:
            raise ValueError("oracle rejected arguments")
        return out

    def e4m3_encode(self, x) -> np.ndarray:
        """Nearest finite E4M3 code (ties to even, saturating) of each value of x (any shape)."""
        x = np.asarray(x, dtype=np.float64)
        return np.array([self.L.oracle_e4m3_encode(float(v)) for v in x.reshape(-1)], dtype=np.uint8).reshape(x.shape)

    def quantize_e4m3_blocks(self, x, blk: int = 128):
        """Block quantisation of fp32 x [B,H,S,d] -> (codes uint8 [B,H,S,d], descale fp32 [B,H,ceil(S/blk)])."""
        x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
        B, H, S, d = x.shape
        codes = np.empty(x.shape, np.uint8)
        descale = np.empty((B, H, (S + blk - 1) // blk), np.float32)
        r = self.L.oracle_quantize_e4m3_blocks(x.ctypes.data, B, H, S, d, blk, codes.ctypes.data, descale.ctypes.data)
        if r < 0:
            raise ValueError("oracle rejected arguments")
        return codes, descale


_default: Oracle | None = None


def get() -> Oracle:
    """The oracle built from this directory's source (built on first use)."""
    global _default
    if _default is None:
        _default = Oracle()
    return _default
