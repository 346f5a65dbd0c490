"""GPU parity of the per-block fp8 (E4M3, E5M2) quantisers: bit-exact against the oracle's quantiser.

Codes and descales are integer / exactly specified outputs, so the bar is
equality: fp32 inputs are compared with the oracle run on the same fp32
values; bf16 and fp16 inputs with the oracle run on their exact fp32 values.
"""
import numpy as np
import pytest
import torch

from oracle import attn_oracle
from tests import parity_util as U

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def oracle():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import exact_attention_32_amd as ea

    ea.load_library()
    return attn_oracle.get()


def _draw(shape, seed, spread=True):
    rng = np.random.Generator(np.random.PCG64(seed))
    x = rng.standard_normal(shape, dtype=np.float32)
    if spread:
        # blocks of very different magnitude, a few large and tiny entries, exact ties
        B, H, S, d = shape
        for j in range(0, S, 128):
            x[:, :, j:j + 128] *= np.float32(2.0 ** rng.integers(-20, 20))
        x.reshape(-1)[rng.choice(x.size, size=min(64, x.size), replace=False)] *= np.float32(1e3)
    return x


def _check(oracle, x32: np.ndarray, dtype: torch.dtype, fmt: str = "e4m3"):
    import exact_attention_32_amd as ea

    xt = torch.from_numpy(x32).to(dtype)
    exact32 = xt.float().numpy()          # the exact values the kernel sees
    codes, ds = ea.quantize_fp8(xt.to("cuda:0"), fmt)
    torch.cuda.synchronize()
    rc, rd = oracle.quantize_fp8_blocks(exact32, fmt)
    gc, gd = codes.cpu().numpy(), ds.cpu().numpy()
    assert np.array_equal(gd, rd), np.argwhere(gd != rd)[:5]
    bad = np.argwhere(gc != rc)
    assert bad.size == 0, [(tuple(i), float(exact32[tuple(i)]), int(gc[tuple(i)]), int(rc[tuple(i)])) for i in bad[:5]]


SHAPES = [(1, 1, 1, 64), (1, 2, 127, 128), (2, 3, 300, 64), (1, 2, 513, 128), (2, 2, 1024, 128)]


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.float16], ids=["f32", "bf16", "f16"])
def test_quantize_matches_oracle(oracle, shape, dtype, fmt):
    x = _draw(shape, 3000 + sum(shape))
    if dtype == torch.float16:
        x = np.clip(x, -6e4, 6e4)
    U.say(f"[gpu] quantize {fmt} {shape} {dtype}")
    _check(oracle, x, dtype, fmt)


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_quantize_special_blocks(oracle, fmt):
    """All-zero block (descale 1), negative zero, exact midpoints of the code grid after scaling
    (normal and subnormal), saturation edge."""
    x = np.zeros((1, 1, 384, 64), np.float32)
    # block 1: values that are exact midpoints of the scaled grid (amax = fmax -> descale 1)
    tdt, ncode, fmax = ((torch.float8_e4m3fn, 127, 448.0) if fmt == "e4m3" else (torch.float8_e5m2, 124, 57344.0))
    tab = torch.arange(ncode, dtype=torch.uint8).view(tdt).to(torch.float64).numpy()
    mids = ((tab[:-1] + tab[1:]) / 2).astype(np.float32)
    blk = x[0, 0, 128:256].reshape(-1)
    blk[:mids.size] = mids
    blk[mids.size:2 * mids.size] = -mids
    blk[-1] = fmax
    # block 2: -0.0 entries and values around the largest code
    b2 = x[0, 0, 256:384].reshape(-1)
    b2[:] = np.float32(-0.0)
    b2[0:4] = [1.0, -1.0, 0.999, 1.0001]
    U.say(f"[gpu] quantize special blocks {fmt}")
    _check(oracle, x, torch.float32, fmt)


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_quantized_inputs_drive_fp8_attention(oracle, fmt):
    """quantize_fp8 -> fwd_fp8 reproduces the fp8 path of the input generator (same codes)."""
    import exact_attention_32_amd as ea
    from exact_attention_32_amd import inputs as I

    w = I.random_workload(1, 2, 200, 200, 128, "fp8" if fmt == "e4m3" else "e5m2", False, seed=77)
    x = I.make_inputs(w)
    dev = "cuda:0"
    U.say(f"[gpu] quantize -> fwd_fp8 {fmt}")
    qc, qd = ea.quantize_fp8(torch.from_numpy(x.q32).to(dev), fmt)
    assert torch.equal(qc.cpu(), x.q) and torch.equal(qd.cpu(), x.q_descale)
    o1, l1 = ea.fwd_fp8(qc, x.k.to(dev), x.v.to(dev), qd, x.k_descale.to(dev), x.v_descale.to(dev), scale=w.scale,
                        fmt=fmt)
    o2, l2 = U.run_gpu(x)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_quantize_qkv_equals_single_calls(oracle, fmt, dtype):
    """One launch for Q, K, V (S_q != S_k) gives the bytes of three single-tensor calls."""
    import exact_attention_32_amd as ea

    dev = "cuda:0"
    U.say(f"[gpu] quantize_qkv {fmt} {dtype}")
    q = torch.from_numpy(_draw((2, 3, 300, 128), 11)).to(dtype).to(dev)
    k = torch.from_numpy(_draw((2, 3, 513, 128), 12)).to(dtype).to(dev)
    v = torch.from_numpy(_draw((2, 3, 513, 128), 13)).to(dtype).to(dev)
    codes, ds = ea.quantize_qkv(q, k, v, fmt)
    for t, c, d in zip((q, k, v), codes, ds):
        c1, d1 = ea.quantize_fp8(t, fmt)
        assert torch.equal(c, c1) and torch.equal(d, d1)


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_quantize_empty(oracle, fmt):
    """A tensor with no rows is skipped: empty outputs alone, and the other tensors of a Q, K, V
    launch are quantised as by single calls."""
    import exact_attention_32_amd as ea

    dev = "cuda:0"
    U.say(f"[gpu] quantize empty {fmt}")
    for shape in ((2, 3, 0, 128), (0, 3, 50, 64), (2, 0, 50, 128)):
        codes, ds = ea.quantize_fp8(torch.zeros(shape, device=dev), fmt)
        assert codes.shape == shape and ds.shape == (shape[0], shape[1], (shape[2] + 127) // 128)
    q = torch.zeros(2, 3, 0, 128, device=dev)
    k = torch.from_numpy(_draw((2, 3, 300, 128), 14)).to(dev)
    v = torch.from_numpy(_draw((2, 3, 300, 128), 15)).to(dev)
    (qc, kc, vc), (qd, kd, vd) = ea.quantize_qkv(q, k, v, fmt)
    assert qc.shape == q.shape and qd.shape == (2, 3, 0)
    for t, c, d in ((k, kc, kd), (v, vc, vd)):
        c1, d1 = ea.quantize_fp8(t, fmt)
        assert torch.equal(c, c1) and torch.equal(d, d1)
