"""Seeded synthetic inputs for the attention forward pass.

This module holds no attention arithmetic: it draws Q, K, V, casts them to the
storage dtype and, for the fp8 path, block-quantises them to OCP E4M3 codes with
per-(batch, head, 128-row block) fp32 descales.  The same bytes feed the GPU
kernels and the fp64 CPU oracle.

Recipe (the pages state no distributions or seeds, so these are choices):
  * numpy ``Generator(PCG64(seed))``; ``standard_normal(float32)`` drawn in the
    order Q, K, V, each of shape [B, H, S, d];
  * outliers (long-context workload): exactly floor(0.01 * N) distinct entries
    of Q, then independently of K, chosen uniformly without replacement, are
    multiplied by 10 in fp32 before the cast;
  * fp16/bf16: round-to-nearest-even cast (torch ``.to``);
  * fp8: block quantisation in the spirit of the FlashAttention-3 deep dive
    (techknowgenie), section 4 "Block quantization and dynamic scaling": one
    scale per 128-row block of each (b, h) -- at d = 128 that block is a
    128 x 128 tile -- taken from the block's local |max|:
    descale = amax / 448 (448 = largest finite E4M3), 1 if amax == 0;
    code = E4M3(x / descale), round-to-nearest-even, saturating at +-448.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

FP8_BLOCK = 128
E4M3_MAX = 448.0


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    S_q: int
    S_k: int
    d: int
    dtype: str          # "f16", "bf16", "fp8" (OCP E4M3) or "e5m2" (OCP E5M2)
    causal: bool
    seed: int
    outliers: bool = False

    @property
    def scale(self) -> float:
        """1/sqrt(d) rounded to fp32 (the value both sides receive)."""
        return float(np.float32(1.0 / math.sqrt(self.d)))

    def visible_pairs(self) -> int:
        """Number of (query, key) pairs that take part in the softmax, over all (b, h)."""
        if not self.causal:
            per = self.S_q * self.S_k
        else:
            # key j visible to query i iff j <= i: rows i < S_k see i + 1 keys, the rest all S_k
            n = min(self.S_q, self.S_k)
            per = n * (n + 1) // 2 + (self.S_q - n) * self.S_k
        return per * self.B * self.H

    def flops(self) -> int:
        """Algorithmic FLOP: 2*d for Q.K^T plus 2*d for P.V per visible pair."""
        return 4 * self.d * self.visible_pairs()

    def hbm_bytes(self) -> int:
        """Algorithmic HBM bytes: Q, K, V read once, O and LSE written once, descales read once."""
        elt = 1 if is_fp8(self.dtype) else 2
        out_elt = 2
        n_q = self.B * self.H * self.S_q * self.d
        n_k = self.B * self.H * self.S_k * self.d
        total = n_q * elt + 2 * n_k * elt + n_q * out_elt + self.B * self.H * self.S_q * 4
        if is_fp8(self.dtype):
            total += 4 * self.B * self.H * (_nblk(self.S_q) + 2 * _nblk(self.S_k))
        return total


def is_fp8(dtype: str) -> bool:
    """Block-scaled 8-bit inputs: "fp8" (E4M3) or "e5m2"."""
    return dtype in ("fp8", "e5m2")


def _nblk(s: int) -> int:
    return (s + FP8_BLOCK - 1) // FP8_BLOCK


# The workloads the benchmark and the parity tests use.  Names state the sizes.
WORKLOADS = {
    w.name: w
    for w in [
        Workload("f16_b1_h2_s128_d64", 1, 2, 128, 128, 64, "f16", False, 1),
        Workload("bf16_b4_h16_s2048_d128", 4, 16, 2048, 2048, 128, "bf16", False, 2),
        Workload("bf16_causal_b1_h32_s8192_d128", 1, 32, 8192, 8192, 128, "bf16", True, 3),
        Workload("fp8_b2_h16_s4096_d128", 2, 16, 4096, 4096, 128, "fp8", False, 4),
        Workload("bf16_causal_outliers_b1_h16_s16384_d64", 1, 16, 16384, 16384, 64, "bf16", True, 5, True),
        Workload("bf16_b2_h16_s4096_d128", 2, 16, 4096, 4096, 128, "bf16", False, 6),
        Workload("e5m2_b2_h16_s4096_d128", 2, 16, 4096, 4096, 128, "e5m2", False, 7),
    ]
}


@dataclasses.dataclass
class Inputs:
    work: Workload
    q: torch.Tensor            # [B,H,S_q,d] f16/bf16, or uint8 E4M3 codes
    k: torch.Tensor
    v: torch.Tensor
    q_descale: torch.Tensor | None = None   # [B,H,ceil(S_q/128)] fp32 (fp8 only)
    k_descale: torch.Tensor | None = None
    v_descale: torch.Tensor | None = None
    q32: np.ndarray | None = None           # the fp32 draws before quantisation (fp8 only)
    k32: np.ndarray | None = None
    v32: np.ndarray | None = None


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """OCP E4M3 ("fn") codes of float values: round-to-nearest-even, saturating to +-448.

    Format: sign, 4 exponent bits (bias 7), 3 mantissa bits; exponent field 0 is
    subnormal (2^-6 * m/8); code 0x7f / 0xff is NaN and never produced here.
    """
    x = np.asarray(x, dtype=np.float64)
    sign = (np.signbit(x)).astype(np.uint8) << 7
    a = np.abs(x)
    a = np.minimum(a, E4M3_MAX)
    code = np.zeros(a.shape, dtype=np.int64)
    sub = a < 2.0 ** -6
    # subnormals (and the rounding of the top subnormals up to 2^-6): quantum 2^-9
    code[sub] = np.rint(a[sub] * 2.0 ** 9).astype(np.int64)
    nrm = ~sub
    if np.any(nrm):
        an = a[nrm]
        _, e2 = np.frexp(an)            # an = f * 2^e2, f in [0.5, 1)
        e = e2.astype(np.int64) - 1     # an in [2^e, 2^(e+1))
        mant = np.rint(an / np.ldexp(1.0, e) * 8.0).astype(np.int64) - 8   # 0..8
        carry = mant == 8
        e = np.where(carry, e + 1, e)
        mant = np.where(carry, 0, mant)
        field = e + 7
        c = (field << 3) | mant
        c = np.minimum(c, 0x7E)         # saturate (RNE above 448 would leave the format)
        code[nrm] = c
    return (code.astype(np.uint8) | sign).astype(np.uint8)


E5M2_MAX = 57344.0


def e5m2_encode(x: np.ndarray) -> np.ndarray:
    """OCP E5M2 codes of float values: round-to-nearest-even, saturating to +-57344.

    Format: sign, 5 exponent bits (bias 15), 2 mantissa bits; exponent field 0
    is subnormal (2^-14 * m/4); exponent field 31 holds inf / NaN, never produced here.
    """
    x = np.asarray(x, dtype=np.float64)
    sign = (np.signbit(x)).astype(np.uint8) << 7
    a = np.minimum(np.abs(x), E5M2_MAX)
    code = np.zeros(a.shape, dtype=np.int64)
    sub = a < 2.0 ** -14
    code[sub] = np.rint(a[sub] * 2.0 ** 16).astype(np.int64)   # quantum 2^-16
    nrm = ~sub
    if np.any(nrm):
        an = a[nrm]
        _, e2 = np.frexp(an)
        e = e2.astype(np.int64) - 1
        mant = np.rint(an / np.ldexp(1.0, e) * 4.0).astype(np.int64) - 4   # 0..4
        carry = mant == 4
        e = np.where(carry, e + 1, e)
        mant = np.where(carry, 0, mant)
        c = ((e + 15) << 2) | mant
        code[nrm] = np.minimum(c, 0x7B)
    return (code.astype(np.uint8) | sign).astype(np.uint8)


def quantize_fp8_blocks(x: np.ndarray, fmt: str = "e4m3", blk: int = FP8_BLOCK):
    """Per-(b, h, blk-row block) scaling of x [B,H,S,d] fp32 to E4M3 or E5M2 codes -> (codes, descale [B,H,nblk])."""
    enc, fmax = {"e4m3": (e4m3_encode, E4M3_MAX), "e5m2": (e5m2_encode, E5M2_MAX)}[fmt]
    B, H, S, d = x.shape
    nb = (S + blk - 1) // blk
    codes = np.empty(x.shape, dtype=np.uint8)
    desc = np.empty((B, H, nb), dtype=np.float32)
    for j in range(nb):
        r0, r1 = j * blk, min(S, (j + 1) * blk)
        xb = x[:, :, r0:r1, :]
        amax = np.abs(xb).max(axis=(2, 3)).astype(np.float32)
        ds = np.where(amax > 0, amax / np.float32(fmax), np.float32(1.0)).astype(np.float32)
        desc[:, :, j] = ds
        codes[:, :, r0:r1, :] = enc(xb.astype(np.float64) / ds.astype(np.float64)[:, :, None, None])
    return codes, desc


def quantize_e4m3_blocks(x: np.ndarray, blk: int = FP8_BLOCK):
    """Per-(b, h, blk-row block) scaling of x [B,H,S,d] fp32 -> (codes uint8, descale fp32 [B,H,nblk])."""
    return quantize_fp8_blocks(x, "e4m3", blk)


_TORCH_DT = {"f16": torch.float16, "bf16": torch.bfloat16}


def make_inputs(work: Workload) -> Inputs:
    rng = np.random.Generator(np.random.PCG64(work.seed))
    q = rng.standard_normal((work.B, work.H, work.S_q, work.d), dtype=np.float32)
    k = rng.standard_normal((work.B, work.H, work.S_k, work.d), dtype=np.float32)
    v = rng.standard_normal((work.B, work.H, work.S_k, work.d), dtype=np.float32)
    if work.outliers:
        for t in (q, k):
            flat = t.reshape(-1)
            n = int(0.01 * flat.size)
            idx = rng.choice(flat.size, size=n, replace=False)
            flat[idx] *= np.float32(10.0)
    if is_fp8(work.dtype):
        fmt = "e5m2" if work.dtype == "e5m2" else "e4m3"
        qc, qd = quantize_fp8_blocks(q, fmt)
        kc, kd = quantize_fp8_blocks(k, fmt)
        vc, vd = quantize_fp8_blocks(v, fmt)
        return Inputs(work, torch.from_numpy(qc), torch.from_numpy(kc), torch.from_numpy(vc),
                      torch.from_numpy(qd), torch.from_numpy(kd), torch.from_numpy(vd), q, k, v)
    dt = _TORCH_DT[work.dtype]
    return Inputs(work, torch.from_numpy(q).to(dt), torch.from_numpy(k).to(dt), torch.from_numpy(v).to(dt))


def random_workload(B: int, H: int, S_q: int, S_k: int, d: int, dtype: str, causal: bool, seed: int,
                    outliers: bool = False) -> Workload:
    return Workload(f"{dtype}{'_causal' if causal else ''}_b{B}_h{H}_sq{S_q}_sk{S_k}_d{d}", B, H, S_q, S_k, d,
                    dtype, causal, seed, outliers)


def make_device_inputs(B: int, H: int, S: int, d: int, dtype: str, seed: int, device="cuda:0"):
    """Seeded inputs generated directly in device memory, for sizes whose host-side draw would be
    slow (beyond 2^31 elements per tensor): torch's generator on the device, ``randn`` in fp32
    in the order Q, K, V, then the RNE cast to bf16/f16.  For "fp8"/"e5m2" the tensors are
    uniformly random finite codes of that format (no NaN or infinity codes) with per-(b, h,
    128-row block) descales uniform in [0.5, 2): synthetic quantised data, not a quantisation
    of anything.  The codes are those of magnitude below 2 (0x00-0x3f and 0x80-0xbf in both
    formats, subnormals included), so that scores stay in the range of N(0, 1) data.
    Returns (q, k, v, descales or None); descales are (q_ds, k_ds, v_ds)."""
    g = torch.Generator(device=device).manual_seed(seed)
    shape = (B, H, S, d)
    if not is_fp8(dtype):
        tdt = torch.bfloat16 if dtype == "bf16" else torch.float16
        out = [torch.randn(shape, generator=g, device=device, dtype=torch.float32).to(tdt) for _ in range(3)]
        return out[0], out[1], out[2], None
    out = []
    for _ in range(3):
        mag = torch.randint(0, 0x40, shape, generator=g, device=device, dtype=torch.int32)
        sign = torch.randint(0, 2, shape, generator=g, device=device, dtype=torch.int32) * 0x80
        out.append((mag + sign).to(torch.uint8))
    ds = tuple(torch.rand((B, H, _nblk(S)), generator=g, device=device, dtype=torch.float32) * 1.5 + 0.5
               for _ in range(3))
    return out[0], out[1], out[2], ds
