"""The C-ABI library: it loads, exports what include/attn.h declares, and rejects bad arguments on the host.

No compute call is made here: every call below fails validation before the
library touches the HIP runtime (the pointers are fake integers and are never
dereferenced).
"""
import ctypes
import os
import re

import pytest

import exact_attention_32_amd as ea

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")

OK, NULL, SHAPE, UNSUP, ALIGN, OVERFLOW, LAUNCH, VALUE, DESCALE = range(9)
P = 0x10000   # a fake, 16-byte aligned "device pointer" (never dereferenced)


@pytest.fixture(scope="module")
def lib():
    return ea.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_\w+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) >= {"attn_fwd", "attn_fwd_fp8", "attn_fwd_fp8_e5m2", "attn_status_string", "attn_fwd_plan",
                          "attn_quantize_e4m3", "attn_quantize_e5m2", "attn_fwd_set_policy", "attn_qk_rmsnorm",
                          "attn_quantize_qkv", "attn_qk_rmsnorm_split", "attn_fwd_qnorm"}
    for n in names:
        assert hasattr(lib, n), f"library does not export {n}"


def test_rate_library_exports_its_header():
    """The matrix-core calibration library exports what include/mfma_rate.h declares, and rejects
    bad arguments before any launch."""
    from exact_attention_32_amd import build as B

    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "mfma_rate.h")).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(attn_\w+)\s*\(", text)))
    assert names == ["attn_mfma_rate", "attn_mfma_rate_fp8", "attn_mfma_rate_fp8_regs", "attn_mfma_rate_regs"]
    L = ctypes.CDLL(B.RATE_LIB)
    for n in names:
        f = getattr(L, n)
        f.restype = ctypes.c_int
        f.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
        assert f(None, 1, 1, P, None) == 1 and f(P, 1, 1, None, None) == 1
        assert f(P, 0, 1, P, None) == 1 and f(P, 1, 0, P, None) == 1


def test_status_strings(lib):
    for code in range(9):
        s = lib.attn_status_string(code)
        assert s and s.decode() != "unknown status"
    assert lib.attn_status_string(99).decode() == "unknown status"


def call(lib, q=P, k=P, v=P, o=P, lse=P, B=1, H=1, Sq=16, Sk=16, d=128, causal=0, scale=0.125, dtype=1):
    return lib.attn_fwd(q, k, v, o, lse, B, H, Sq, Sk, d, causal, scale, dtype, None)


FP8_ENTRIES = ("attn_fwd_fp8", "attn_fwd_fp8_e5m2")


def call8(lib, q=P, k=P, v=P, qd=P, kd=P, vd=P, o=P, lse=P, B=1, H=1, Sq=16, Sk=16, d=128, causal=0, scale=0.125):
    """Both fp8 entry points must return the same status; that status."""
    rcs = {getattr(lib, n)(q, k, v, qd, kd, vd, o, lse, B, H, Sq, Sk, d, causal, scale, None) for n in FP8_ENTRIES}
    assert len(rcs) == 1, rcs
    return rcs.pop()


def test_null_pointers(lib):
    for kw in ("q", "k", "v", "o"):
        assert call(lib, **{kw: None}) == NULL
        assert call8(lib, **{kw: None}) == NULL
    for kw in ("qd", "kd", "vd"):
        assert call8(lib, **{kw: None}) == DESCALE


def test_shapes(lib):
    for kw in ("B", "H", "Sq", "Sk"):
        assert call(lib, **{kw: -3}) == SHAPE
        assert call8(lib, **{kw: -1}) == SHAPE
    # no keys while there are queries: the softmax is undefined
    assert call(lib, Sk=0) == SHAPE and call8(lib, Sk=0) == SHAPE


def test_empty_inputs(lib):
    """No query rows: ATTN_OK with nothing launched, read or written (so NULL pointers are fine and
    no GPU is needed); d, dtype and scale are still checked."""
    none = dict(q=None, k=None, v=None, o=None, lse=None)
    for kw in ("B", "H", "Sq"):
        assert call(lib, **{kw: 0}) == OK
        assert call(lib, **{kw: 0}, **none) == OK
        assert call(lib, **{kw: 0}, Sk=0, **none) == OK
        assert call8(lib, **{kw: 0}, qd=None, kd=None, vd=None, **none) == OK
        for dt in (0, 1, 2, 4):
            assert call(lib, **{kw: 0}, dtype=dt, **none) == OK
        assert call(lib, **{kw: 0}, d=96) == UNSUP and call(lib, **{kw: 0}, dtype=7) == UNSUP
        assert call(lib, **{kw: 0}, scale=0.0) == VALUE and call8(lib, **{kw: 0}, scale=float("nan")) == VALUE
    bq, bk, w, n = ea.plan(0, 16, 4096, 4096, 128, False)
    assert n == 0 and (bq, bk, w) == ea.plan(1, 1, 1, 1, 128, False)[:3]
    assert ea.plan(2, 16, 0, 0, 64, True, dtype=ea.ATTN_FP8_E4M3)[3] == 0
    with pytest.raises(ea.AttnError):
        ea.plan(1, 1, 16, 0, 128)
    # quantisers: a tensor with no rows is skipped
    for kw in ("B", "H", "S"):
        assert callq(lib, **{kw: 0}, x=None, codes=None, ds=None) == OK
        assert callq(lib, **{kw: 0}, d=96) == UNSUP
    assert callqkv(lib, B=0, q=None, k=None, v=None, cq=None, ck=None, cv=None, dq=None, dk=None, dv=None) == OK
    assert callqkv(lib, Sq=0, Sk=0, dtype=2) == UNSUP
    assert callqkv(lib, Sq=0, Sk=0, q=None, cq=None, dq=None) == OK
    # QK-RMSNorm: no tokens, nothing to do
    assert callqn(lib, B=0, q=None, k=None, wq=None, wk=None, qo=None, ko=None) == OK
    assert callqn(lib, Sq=0, Sk=0, q=None, k=None, wq=None, wk=None, qo=None, ko=None) == OK
    assert callqn(lib, B=0, eps=-1.0) == VALUE and callqn(lib, B=0, d=96) == UNSUP


def test_unsupported(lib):
    for d in (0, 32, 96, 256, 127):
        assert call(lib, d=d) == UNSUP
    assert call(lib, dtype=7) == UNSUP
    assert call(lib, dtype=-1) == UNSUP


def test_alignment(lib):
    for kw in ("q", "k", "v", "o"):
        assert call(lib, **{kw: P + 8}) == ALIGN
        assert call8(lib, **{kw: P + 2}) == ALIGN
    assert call(lib, lse=P + 2) == ALIGN
    assert call8(lib, qd=P + 2) == DESCALE


def test_overflow(lib):
    assert call(lib, Sq=(2 ** 31 - 1) // 64, d=128) == OVERFLOW
    assert call(lib, Sk=2 ** 25, d=64) == OVERFLOW
    # grid size: ceil(S_q / block_q) * B * H must fit in an int
    assert call(lib, B=2 ** 16, H=2 ** 16, Sq=16) == OVERFLOW


def test_scale(lib):
    for s in (0.0, -1.0, float("inf"), float("nan")):
        assert call(lib, scale=s) == VALUE
        assert call8(lib, scale=s) == VALUE


def test_plan(lib):
    bq, bk, w, n = ea.plan(2, 16, 4096, 4096, 128, False)
    assert bq >= 32 and bq % 32 == 0 and bk % 32 == 0 and w >= 1
    assert n == -(-4096 // bq) * 32
    with pytest.raises(ea.AttnError):
        ea.plan(1, 1, 16, 16, 96)
    # fp8: one 128-key tile per descale block
    for dt in (ea.ATTN_FP8_E4M3, ea.ATTN_FP8_E5M2):
        bq, bk, w, n = ea.plan(2, 16, 4096, 4096, 128, False, dtype=dt)
        assert bk == 128 and bq % 128 == 0 and n == -(-4096 // bq) * 32


def test_binding_rejects_host_tensors():
    import torch

    q = torch.zeros(1, 1, 4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        ea.fwd(q, q, q)


def callq(lib, x=P, dtype=3, codes=P, ds=P, B=1, H=1, S=16, d=128):
    """Both quantisers must return the same status; that status."""
    rcs = {getattr(lib, n)(x, dtype, codes, ds, B, H, S, d, None) for n in ("attn_quantize_e4m3", "attn_quantize_e5m2")}
    assert len(rcs) == 1, rcs
    return rcs.pop()


def test_quantize_validation(lib):
    assert callq(lib, x=None) == NULL and callq(lib, codes=None) == NULL
    assert callq(lib, ds=None) == DESCALE and callq(lib, ds=P + 2) == DESCALE
    for kw in ("B", "H", "S"):
        assert callq(lib, **{kw: -1}) == SHAPE
    assert callq(lib, d=96) == UNSUP and callq(lib, dtype=2) == UNSUP and callq(lib, dtype=4) == UNSUP
    assert callq(lib, dtype=7) == UNSUP
    assert callq(lib, x=P + 4) == ALIGN and callq(lib, codes=P + 8) == ALIGN
    assert callq(lib, B=2 ** 16, H=2 ** 16, S=2 ** 10) == OVERFLOW


C, PP, DP = ea.ATTN_SCHED_CLASSIC, ea.ATTN_SCHED_PINGPONG, ea.ATTN_SCHED_DEPHASED
COMPILED = [(C, 1, 8, 3, 64), (C, 1, 8, 4, 64), (C, 2, 4, 3, 64), (C, 2, 4, 4, 64), (C, 1, 4, 2, 64),
            (C, 1, 4, 3, 64), (C, 1, 8, 2, 128), (PP, 1, 8, 3, 64), (DP, 1, 8, 4, 64)]
D64_ONLY = [(C, 2, 8, 3, 64), (C, 2, 8, 4, 64), (C, 1, 4, 3, 192), (C, 1, 4, 2, 256)]


def test_set_policy(lib):
    try:
        for bad in ((C, 3, 8, 4, 64), (PP, 1, 8, 4, 64), (9, 1, 8, 4, 64), (DP, 1, 8, 3, 64), (C, 1, 8, 4, 128),
                    (C, 1, 8, 2, 64), (C, 1, 8, 4, 192)):
            assert lib.attn_fwd_set_policy(*bad) == UNSUP
        for sched, qb, nw, ns, bkk in COMPILED:
            assert lib.attn_fwd_set_policy(sched, qb, nw, ns, bkk) == OK
            bq, bk, w, n = ea.plan(2, 16, 4096, 4096, 128, False)
            assert (bq, bk, w) == (qb * nw * 32, bkk, nw) and n == -(-4096 // bq) * 32
            # fp8 plans do not follow the f16/bf16 override
            assert ea.plan(2, 16, 4096, 4096, 128, False, dtype=ea.ATTN_FP8_E4M3)[:3] == (256, 128, 8)
        for sched, qb, nw, ns, bkk in D64_ONLY:
            assert lib.attn_fwd_set_policy(sched, qb, nw, ns, bkk) == OK
            assert ea.plan(1, 16, 4096, 4096, 64, False)[:3] == (qb * nw * 32, bkk, nw)
            with pytest.raises(ea.AttnError):
                ea.plan(1, 16, 4096, 4096, 128, False)
    finally:
        assert lib.attn_fwd_set_policy(ea.ATTN_SCHED_DEFAULT, 0, 0, 0, 0) == OK
    # the measured table: d = 128 takes 128-key tiles
    assert ea.plan(2, 16, 4096, 4096, 128, False)[:3] == (256, 128, 8)
    assert ea.kernel_name(128, False, ea.ATTN_BF16) == "attn_fwd_kernel"
    # d = 64: 64 queries per wave where their 512-query workgroups come out in rounds at least as
    # full as those of 256-query ones (non-causal) or pair into full rounds on long sequences
    # (causal); else 128-key tiles with 32 queries per wave
    assert ea.plan(1, 16, 16384, 16384, 64, False)[:3] == (512, 64, 8)   # 2 rounds against 4
    assert ea.plan(2, 16, 4096, 4096, 64, False)[:3] == (512, 64, 8)     # 1 round against 2
    assert ea.plan(1, 20, 8192, 8192, 64, False)[:3] == (256, 128, 8)    # 2 rounds against 3
    assert ea.plan(1, 8, 8192, 8192, 64, False)[:3] == (256, 128, 8)     # 1 round either way
    assert ea.plan(1, 16, 16384, 16384, 64, True)[:3] == (512, 64, 8)
    assert ea.plan(4, 32, 2048, 2048, 64, True)[:3] == (256, 128, 8)
    assert ea.plan(1, 8, 8192, 8192, 64, True)[:3] == (256, 128, 8)
    # at most 128 query rows: 128-query workgroups (no clamped rows computed)
    assert ea.plan(1, 2, 128, 128, 64, False)[:3] == (128, 64, 4)
    assert ea.plan(1, 2, 129, 128, 64, False)[:3] == (256, 128, 8)


def test_plan_causal_pairs(lib):
    """Causal problems whose tile pairs fill the CUs in whole rounds launch one workgroup per pair
    of query tiles (n-1-j, j); others, non-causal ones and fp8 one per tile.  (Here, without a
    device, the CU count is the 256 the table was measured on.)"""
    assert ea.plan(1, 32, 8192, 8192, 128, True) == (256, 128, 8, 32 * 16)   # 512 pairs: 2 rounds
    assert ea.plan(1, 16, 16384, 16384, 64, True) == (512, 64, 8, 16 * 16)   # 256 pairs: 1 round
    assert ea.plan(2, 43, 1200, 1200, 128, True)[3] == 2 * 43 * 3   # 5 tiles: 2 pairs and 1 alone
    assert ea.plan(2, 256, 1300, 900, 64, True) == (256, 128, 8, 2 * 256 * 3)   # 6 tiles: 3 pairs
    assert ea.plan(1, 32, 8192, 8192, 128, False)[3] == 32 * 32
    assert ea.plan(1, 2, 1024, 1024, 128, True)[3] == 2 * 4   # 4 pairs would leave CUs idle
    # 300 pairs would take two rounds where 600 single tiles balance in about 1.2
    assert ea.plan(1, 20, 7680, 7680, 128, True)[3] == 20 * 30
    # d = 64: 30 tiles of 512 queries do not pair into full rounds, nor do 60 of 256
    assert ea.plan(1, 20, 15360, 15360, 64, True) == (256, 128, 8, 20 * 60)
    assert ea.plan(1, 32, 8192, 8192, 128, True, dtype=ea.ATTN_FP8_E4M3)[3] == 32 * 32


def callqn(lib, q=P, k=P, wq=P, wk=P, qo=P, ko=P, B=1, H=2, Sq=16, Sk=16, d=128, eps=1e-6, dtype=1):
    return lib.attn_qk_rmsnorm(q, k, wq, wk, qo, ko, B, H, Sq, Sk, d, eps, dtype, None)


def test_qk_rmsnorm_validation(lib):
    for kw in ("q", "k", "wq", "wk", "qo", "ko"):
        assert callqn(lib, **{kw: None}) == NULL
        assert callqn(lib, **{kw: P + 8}) == ALIGN
    for kw in ("B", "H", "Sq", "Sk"):
        assert callqn(lib, **{kw: -1}) == SHAPE
    # a tensor with no tokens is not touched, so its pointers are not needed, but the other's are
    assert callqn(lib, Sq=0, k=None) == NULL and callqn(lib, Sk=0, q=None) == NULL
    assert callqn(lib, d=96) == UNSUP and callqn(lib, dtype=2) == UNSUP and callqn(lib, dtype=3) == UNSUP
    assert callqn(lib, H=65, d=128) == UNSUP and callqn(lib, H=129, d=64) == UNSUP
    for e in (-1e-6, float("nan"), float("inf")):
        assert callqn(lib, eps=e) == VALUE
    assert callqn(lib, B=2 ** 16, Sq=2 ** 16) == OVERFLOW


def callqs(lib, q=P, k=P, wk=P, r=P, ko=P, B=1, H=2, Sq=16, Sk=16, d=128, eps=1e-6, dtype=1):
    return lib.attn_qk_rmsnorm_split(q, k, wk, r, ko, B, H, Sq, Sk, d, eps, dtype, None)


def test_qk_rmsnorm_split_validation(lib):
    for kw in ("q", "k", "wk", "r", "ko"):
        assert callqs(lib, **{kw: None}) == NULL
    for kw in ("q", "k", "wk", "ko"):
        assert callqs(lib, **{kw: P + 8}) == ALIGN
    assert callqs(lib, r=P + 2) == ALIGN   # the factors are floats: 4-byte alignment
    for kw in ("B", "H", "Sq", "Sk"):
        assert callqs(lib, **{kw: -1}) == SHAPE
    assert callqs(lib, Sq=0, r=None, k=None) == NULL and callqs(lib, Sk=0, q=P, r=None) == NULL
    assert callqs(lib, d=96) == UNSUP and callqs(lib, dtype=2) == UNSUP
    assert callqs(lib, eps=float("nan")) == VALUE
    assert callqs(lib, B=0) == OK and callqs(lib, Sq=0, Sk=0) == OK


def callfq(lib, q=P, k=P, v=P, r=P, wq=P, o=P, lse=P, B=1, H=2, Sq=16, Sk=16, d=128, causal=0, scale=0.125, dtype=1):
    return lib.attn_fwd_qnorm(q, k, v, r, wq, o, lse, B, H, Sq, Sk, d, causal, scale, dtype, None)


def test_fwd_qnorm_validation(lib):
    for kw in ("q", "k", "v", "o", "r", "wq"):
        assert callfq(lib, **{kw: None}) == NULL
    for kw in ("q", "k", "v", "o", "wq"):
        assert callfq(lib, **{kw: P + 8}) == ALIGN
    assert callfq(lib, r=P + 2) == ALIGN and callfq(lib, lse=P + 2) == ALIGN
    for kw in ("B", "H", "Sq", "Sk"):
        assert callfq(lib, **{kw: -1}) == SHAPE
    assert callfq(lib, Sk=0) == SHAPE
    for dt in (0, 1):
        assert callfq(lib, d=96, dtype=dt) == UNSUP
    assert callfq(lib, dtype=2) == UNSUP and callfq(lib, dtype=4) == UNSUP and callfq(lib, dtype=3) == UNSUP
    assert callfq(lib, scale=float("inf")) == VALUE
    # no query rows: nothing to do, and the factor and weight pointers are not needed
    assert callfq(lib, Sq=0, r=None, wq=None) == OK and callfq(lib, B=0) == OK


def callqkv(lib, q=P, k=P, v=P, dtype=3, fmt=2, cq=P, ck=P, cv=P, dq=P, dk=P, dv=P, B=1, H=1, Sq=16, Sk=16, d=128):
    return lib.attn_quantize_qkv(q, k, v, dtype, fmt, cq, ck, cv, dq, dk, dv, B, H, Sq, Sk, d, None)


def test_quantize_qkv_validation(lib):
    for kw in ("q", "k", "v", "cq", "ck", "cv"):
        assert callqkv(lib, **{kw: None}) == NULL
    for kw in ("dq", "dk", "dv"):
        assert callqkv(lib, **{kw: None}) == DESCALE and callqkv(lib, **{kw: P + 2}) == DESCALE
    for kw in ("q", "k", "v", "cq", "ck", "cv"):
        assert callqkv(lib, **{kw: P + 4}) == ALIGN
    for kw in ("B", "H", "Sq", "Sk"):
        assert callqkv(lib, **{kw: -1}) == SHAPE
    # an empty tensor is skipped, but the others' pointers are still checked
    assert callqkv(lib, Sq=0, k=None) == NULL and callqkv(lib, Sk=0, q=None) == NULL
    assert callqkv(lib, fmt=0) == UNSUP and callqkv(lib, fmt=1) == UNSUP and callqkv(lib, fmt=3) == UNSUP
    assert callqkv(lib, d=96) == UNSUP and callqkv(lib, dtype=2) == UNSUP
    assert callqkv(lib, B=2 ** 16, H=2 ** 16, Sk=2 ** 10) == OVERFLOW


def test_output_buffer_checks():
    """The binding refuses a caller-supplied output the kernel would write past or into the wrong
    memory: wrong shape, type, device or layout (checked before any library call)."""
    import torch

    import exact_attention_32_amd as ea

    dev = torch.device("cpu")
    good = torch.empty(2, 3, 5, 64, dtype=torch.bfloat16)
    ea._check_buffer(good, "out", (2, 3, 5, 64), torch.bfloat16, dev)
    bad = [
        torch.empty(2, 3, 4, 64, dtype=torch.bfloat16),                       # too few rows
        torch.empty(2, 3, 5, 64, dtype=torch.float16),                        # wrong type
        torch.empty(2, 3, 64, 5, dtype=torch.bfloat16).transpose(2, 3),       # not dense
        torch.empty(2, 3, 5, 64, dtype=torch.bfloat16, device="meta"),        # another device
        None,
    ]
    for t in bad:
        with pytest.raises(ValueError):
            ea._check_buffer(t, "out", (2, 3, 5, 64), torch.bfloat16, dev)
