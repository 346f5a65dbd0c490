"""GPU parity beyond 2^31 elements per tensor (64-bit element offsets in every kernel).

B=1, H=136, S=131072, d=128: Q, K, V and O hold 2.28e9 elements each, so the offsets of the
last heads exceed 2^31.  The inputs are drawn on the device (seeded, exact_attention_32_amd.inputs);
three heads (the first, a middle one, the last) are copied to the host, and the oracle computes
sampled rows of them, which are compared with the GPU output under the usual gates.
"""
import numpy as np
import pytest
import torch

from exact_attention_32_amd import inputs as I
from oracle import attn_oracle
from tests import parity_util as U

pytestmark = pytest.mark.gpu

B, H, S, D = 1, 136, 131072, 128
HEADS = [0, 68, 135]


@pytest.fixture(scope="module")
def oracle():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import exact_attention_32_amd as ea

    ea.load_library()
    return attn_oracle.get()


def _rows(seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    fixed = [0, 1, 255, 256, S // 2, S - 2, S - 1]
    rows = [(h, i) for h in range(len(HEADS)) for i in fixed]
    rows += [(int(rng.integers(len(HEADS))), int(rng.integers(S))) for _ in range(24)]
    return np.array(sorted(set(rows)), dtype=np.int64)


@pytest.mark.parametrize("dtype,causal", [("bf16", False), ("bf16", True), ("fp8", True)])
def test_beyond_2g_elements(oracle, dtype, causal):
    import exact_attention_32_amd as ea

    assert B * H * S * D > 2 ** 31
    U.say(f"[gpu] large B={B} H={H} S={S} d={D} {dtype} causal={causal}")
    q, k, v, ds = I.make_device_inputs(B, H, S, D, dtype, seed=77)
    scale = float(np.float32(D ** -0.5))
    if ds is None:
        o, lse = ea.fwd(q, k, v, causal=causal, scale=scale)
    else:
        o, lse = ea.fwd_fp8(q, k, v, *ds, causal=causal, scale=scale)
    torch.cuda.synchronize()
    U.say("   kernel done")
    sel = torch.tensor(HEADS, device=q.device)

    def host(t, d_s=None):
        t = t[:, sel].cpu()
        if d_s is None:
            return t.double().numpy()
        codes = t.numpy()
        return oracle.decode_fp8_blocks(codes, d_s[:, sel].cpu().numpy(), "e4m3")

    if ds is None:
        qh, kh, vh = host(q), host(k), host(v)
    else:
        qh, kh, vh = host(q, ds[0]), host(k, ds[1]), host(v, ds[2])
    rows = _rows(5)
    ro, rl = oracle.attention_rows(qh, kh, vh, causal, scale, rows)
    oh = o[:, sel].reshape(len(HEADS), S, D)
    lh = lse[:, sel].reshape(len(HEADS), S)
    og = oh[rows[:, 0], rows[:, 1]].double().cpu().numpy()
    lg = lh[rows[:, 0], rows[:, 1]].double().cpu().numpy()
    st = U.compare(og, lg, ro, rl, dtype)
    U.say(f"   {st}")
    assert st["pass"], st
