"""GPU parity of the QK-RMSNorm across heads (attn_qk_rmsnorm) and of norm -> attention.

The oracle normalises in fp64 and rounds to the tensor's type (the reading of the norm's output:
the sglang write-up's kernel stores its result in the input type, in place).  The kernel takes the
per-token statistic in fp32, so its result may land on the other side of a rounding boundary of
the 16-bit type where the exact value is within fp32 error of it: the bar is at most one unit in
the last place of the 16-bit type everywhere, and at most 0.1% of the elements not bit-equal.
"""
import numpy as np
import pytest
import torch

from exact_attention_32_amd import inputs as I
from oracle import attn_oracle
from tests import parity_util as U

pytestmark = pytest.mark.gpu

TDT = {"bf16": torch.bfloat16, "f16": torch.float16}


@pytest.fixture(scope="module")
def oracle():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import exact_attention_32_amd as ea

    ea.load_library()
    return attn_oracle.get()


def _draw(B, H, S, d, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(B, H, S, d, generator=g)
    # tokens of very different magnitude, and one all-zero token
    scale = torch.exp2(torch.randint(-10, 8, (B, 1, S, 1), generator=g).float())
    x = x * scale
    x[0, :, S // 2, :] = 0.0
    w = torch.empty(H * d).uniform_(0.5, 1.5, generator=g)
    return x.to(TDT[dtype]), w.to(TDT[dtype])


def _ulp_close(got: torch.Tensor, ref64: np.ndarray, dtype: str):
    """(max distance in units in the last place of the 16-bit type, fraction not bit-equal)."""
    ref = torch.from_numpy(ref64).to(TDT[dtype])
    gb = got.cpu().view(torch.int16).to(torch.int32)
    rb = ref.view(torch.int16).to(torch.int32)
    # map sign-magnitude bit patterns onto a monotone integer line
    gi = torch.where(gb < 0, -(gb & 0x7FFF), gb)
    ri = torch.where(rb < 0, -(rb & 0x7FFF), rb)
    dist = (gi - ri).abs()
    return int(dist.max()), float((dist != 0).float().mean())


SHAPES = [(1, 1, 1, 1, 64), (1, 3, 17, 5, 64), (2, 16, 130, 257, 128), (1, 24, 300, 300, 128),
          (2, 64, 33, 40, 128), (1, 128, 9, 9, 64)]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_qknorm_matches_oracle(oracle, shape, dtype):
    import exact_attention_32_amd as ea

    B, H, Sq, Sk, d = shape
    U.say(f"[gpu] qk_rmsnorm {shape} {dtype}")
    q, wq = _draw(B, H, Sq, d, dtype, 10 + Sq)
    k, wk = _draw(B, H, Sk, d, dtype, 20 + Sk)
    eps = 1e-6
    dev = "cuda:0"
    qn, kn = ea.qk_rmsnorm(q.to(dev), k.to(dev), wq.to(dev), wk.to(dev), eps=eps)
    torch.cuda.synchronize()
    for got, x, w in ((qn, q, wq), (kn, k, wk)):
        ref = oracle.rmsnorm_across_heads(x.double().numpy(), w.double().numpy(), eps)
        dist, frac = _ulp_close(got, ref, dtype)
        assert dist <= 1 and frac <= 1e-3, (dist, frac)
    assert torch.all(qn[0, :, Sq // 2] == 0) and torch.all(kn[0, :, Sk // 2] == 0)


def test_qknorm_in_place(oracle):
    import exact_attention_32_amd as ea

    dev = "cuda:0"
    q, wq = _draw(2, 16, 200, 128, "bf16", 5)
    k, wk = _draw(2, 16, 300, 128, "bf16", 6)
    U.say("[gpu] qk_rmsnorm in place")
    q1, k1 = ea.qk_rmsnorm(q.to(dev), k.to(dev), wq.to(dev), wk.to(dev))
    q2, k2 = q.to(dev), k.to(dev)
    r = ea.qk_rmsnorm(q2, k2, wq.to(dev), wk.to(dev), inplace=True)
    torch.cuda.synchronize()
    assert r[0].data_ptr() == q2.data_ptr() and r[1].data_ptr() == k2.data_ptr()
    assert torch.equal(q1, q2) and torch.equal(k1, k2)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(1, 4, 300, 333, 128), (2, 8, 257, 257, 64)], ids=lambda s: "x".join(map(str, s)))
def test_qknorm_then_attention(oracle, shape, causal):
    """RMSNorm then attention on the GPU against RMSNorm (fp64, rounded to bf16) then attention (fp64)."""
    import exact_attention_32_amd as ea

    B, H, Sq, Sk, d = shape
    dev = "cuda:0"
    q, wq = _draw(B, H, Sq, d, "bf16", 40 + Sq)
    k, wk = _draw(B, H, Sk, d, "bf16", 50 + Sk)
    v = torch.randn(B, H, Sk, d, generator=torch.Generator().manual_seed(60)).to(torch.bfloat16)
    eps, scale = 1e-6, d ** -0.5
    U.say(f"[gpu] qk_rmsnorm -> attention {shape} causal={causal}")
    qn, kn = ea.qk_rmsnorm(q.to(dev), k.to(dev), wq.to(dev), wk.to(dev), eps=eps)
    o, lse = ea.fwd(qn, kn, v.to(dev), causal=causal, scale=scale)
    torch.cuda.synchronize()
    qr = torch.from_numpy(oracle.rmsnorm_across_heads(q.double().numpy(), wq.double().numpy(), eps)).to(torch.bfloat16)
    kr = torch.from_numpy(oracle.rmsnorm_across_heads(k.double().numpy(), wk.double().numpy(), eps)).to(torch.bfloat16)
    ro, rl = oracle.attention(qr.double().numpy(), kr.double().numpy(), v.double().numpy(), causal, scale)
    st = U.compare(o.double().cpu().numpy(), lse.double().cpu().numpy(), ro, rl, "bf16")
    U.say(f"   {st}")
    assert st["pass"], st


FOLD = [(1, 4, 300, 333, 128, False), (2, 8, 257, 257, 64, True), (1, 16, 1000, 1000, 128, True),
        (1, 128, 2048, 2048, 64, True), (2, 64, 1024, 1024, 128, True), (2, 3, 17, 5, 64, False)]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("shape", FOLD, ids=lambda s: "x".join(map(str, s)))
def test_qnorm_fold_equals_separate(oracle, shape, dtype):
    """Q's RMSNorm folded into attention's Q loads: K and the attention output are bit for bit those
    of the separate norm followed by attention, and the per-token factor is the norm's."""
    import exact_attention_32_amd as ea

    B, H, Sq, Sk, d, causal = shape
    dev = "cuda:0"
    q, wq = _draw(B, H, Sq, d, dtype, 70 + Sq)
    k, wk = _draw(B, H, Sk, d, dtype, 80 + Sk)
    v = torch.randn(B, H, Sk, d, generator=torch.Generator().manual_seed(90)).to(TDT[dtype])
    q, k, v, wq, wk = q.to(dev), k.to(dev), v.to(dev), wq.to(dev), wk.to(dev)
    eps = 1e-6
    U.say(f"[gpu] qnorm fold {shape} {dtype}")
    qn, kn = ea.qk_rmsnorm(q, k, wq, wk, eps=eps)
    o1, l1 = ea.fwd(qn, kn, v, causal=causal)
    r, kn2 = ea.qk_rmsnorm_split(q, k, wk, eps=eps)
    o2, l2 = ea.fwd_qnorm(q, kn2, v, r, wq, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(kn, kn2)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    # the factor against the oracle's norm: q * r * w reproduces the fp64 RMSNorm to fp32 accuracy
    ref = oracle.rmsnorm_across_heads(q.double().cpu().numpy(), wq.double().cpu().numpy(), eps)
    recon = (q.double().cpu() * r.double().cpu()[:, None, :, None] * wq.double().cpu().view(H, 1, d)).numpy()
    err = np.abs(recon - ref) / np.maximum(np.abs(ref), 1e-30)
    # (fp32 sums over up to H*d = 8192 squares: a few parts in 10^6 at most)
    assert float(err[np.abs(ref) > 0].max(initial=0.0)) < 2e-5


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(1, 4, 300, 333, 128), (2, 8, 257, 257, 64)], ids=lambda s: "x".join(map(str, s)))
def test_qnorm_fold_oracle(oracle, shape, causal):
    """Folded norm -> attention against RMSNorm (fp64, rounded to bf16) then attention (fp64), at the
    shapes of the separate path's oracle test.  (The reference rounds the fp64 norm, the kernel an
    fp32 one, so a few normalised values sit one bf16 ulp apart; through a large score one such
    value moves a row's LSE by up to ~1e-2, and at large hidden sizes (H*d = 8192) some row meets
    one.  The pairing shapes are covered by bit equality with the separate path above.)"""
    import exact_attention_32_amd as ea

    B, H, Sq, Sk, d = shape
    dev = "cuda:0"
    q, wq = _draw(B, H, Sq, d, "bf16", 40 + Sq)   # the separate path's test draws
    k, wk = _draw(B, H, Sk, d, "bf16", 50 + Sk)
    v = torch.randn(B, H, Sk, d, generator=torch.Generator().manual_seed(60)).to(torch.bfloat16)
    eps, scale = 1e-6, d ** -0.5
    U.say(f"[gpu] qnorm fold vs oracle {shape} causal={causal}")
    r, kn = ea.qk_rmsnorm_split(q.to(dev), k.to(dev), wk.to(dev), eps=eps)
    o, lse = ea.fwd_qnorm(q.to(dev), kn, v.to(dev), r, wq.to(dev), causal=causal, scale=scale)
    torch.cuda.synchronize()
    qr = torch.from_numpy(oracle.rmsnorm_across_heads(q.double().numpy(), wq.double().numpy(), eps)).to(torch.bfloat16)
    kr = torch.from_numpy(oracle.rmsnorm_across_heads(k.double().numpy(), wk.double().numpy(), eps)).to(torch.bfloat16)
    ro, rl = oracle.attention(qr.double().numpy(), kr.double().numpy(), v.double().numpy(), causal, scale)
    st = U.compare(o.double().cpu().numpy(), lse.double().cpu().numpy(), ro, rl, "bf16")
    U.say(f"   {st}")
    assert st["pass"], st


def test_qnorm_fold_every_schedule(oracle):
    """The fold in every kernel that f16/bf16 attention can launch."""
    import exact_attention_32_amd as ea

    dev = "cuda:0"
    q, wq = _draw(1, 4, 300, 128, "bf16", 61)
    k, wk = _draw(1, 4, 333, 128, "bf16", 62)
    v = torch.randn(1, 4, 333, 128, generator=torch.Generator().manual_seed(63)).to(torch.bfloat16)
    q, k, v, wq, wk = q.to(dev), k.to(dev), v.to(dev), wq.to(dev), wk.to(dev)
    qn, kn = ea.qk_rmsnorm(q, k, wq, wk)
    r, _ = ea.qk_rmsnorm_split(q, k, wk)
    try:
        for sched in ((1, 1, 8, 2, 128), (1, 1, 8, 4, 64), (2, 1, 8, 3, 64), (3, 1, 8, 4, 64)):
            ea.set_policy(*sched)
            for causal in (False, True):
                U.say(f"[gpu] qnorm fold sched={sched} causal={causal}")
                o1, l1 = ea.fwd(qn, kn, v, causal=causal)
                o2, l2 = ea.fwd_qnorm(q, kn, v, r, wq, causal=causal)
                torch.cuda.synchronize()
                assert torch.equal(o1, o2) and torch.equal(l1, l2), (sched, causal)
    finally:
        ea.set_policy(ea.ATTN_SCHED_DEFAULT)


def test_qknorm_empty(oracle):
    """A tensor with no tokens is not touched; the other one is normalised as usual."""
    import exact_attention_32_amd as ea

    dev = "cuda:0"
    U.say("[gpu] qk_rmsnorm empty")
    k, wk = _draw(1, 4, 37, 128, "bf16", 5)
    q = torch.zeros(1, 4, 0, 128, dtype=torch.bfloat16, device=dev)
    qn, kn = ea.qk_rmsnorm(q, k.to(dev), wk.to(dev), wk.to(dev), eps=1e-6)
    torch.cuda.synchronize()
    assert qn.shape == q.shape
    ref = oracle.rmsnorm_across_heads(k.double().numpy(), wk.double().numpy(), 1e-6)
    dist, frac = _ulp_close(kn, ref, "bf16")
    assert dist <= 1 and frac <= 1e-3, (dist, frac)
    e = torch.zeros(0, 4, 5, 128, dtype=torch.bfloat16, device=dev)
    ea.qk_rmsnorm(e, e, wk.to(dev), wk.to(dev))
