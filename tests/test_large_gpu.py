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


# The longest key sequence the library accepts at d = 128 (S_k * d must stay within the 32-bit
# element range of one head): every key-tile offset, the clamped S_k tail (127 keys) and the row
# sums over 16.7 million keys, against the softmax definition written out in closed form for a
# structured input.  The keys of a head repeat seven score classes (key k has score q0 * A[k % 7])
# and the values repeat with them (V[k] = BASE[k % 7]), except one key k* with score q0 * B_STAR
# and value V_STAR: then, per query row, with n_r keys in class r,
#   Z = sum_r n_r e^(s_r - m) + e^(s* - m),  O = (sum_r n_r e^(s_r - m) BASE[r] + e^(s* - m) V_STAR) / Z,
#   LSE = m + ln Z   (m any shift; the max is taken).
# k* jumps the scores 11.5 above the classes, so the running max moves inside the row: in the
# middle of the keys (head 0) and in the last, ragged tile (head 1).  Query rows alternate
# q0 = 1 and q0 = 1/2.  All values are exact in bf16 and in E4M3.
N_MAX = (2 ** 31 - 1) // 128
A_CLS = [0.0, 0.25, -0.5, 0.75, -1.0, 1.5, -2.0]
B_STAR = 13.0
SQ_LONG = 64


def _long_inputs(dev):
    k_star = [2 ** 23 + 5, N_MAX - 1]
    r = torch.arange(N_MAX, device=dev) % 7
    jj = torch.arange(D, device=dev, dtype=torch.float32)
    base = torch.stack([((jj + 3 * c) % 7 - 3) / 4 for c in range(7)])            # [7, D], multiples of 1/4
    v_star = ((jj % 5) - 2) / 2                                                   # [D], multiples of 1/2
    k = torch.zeros((1, 2, N_MAX, D), dtype=torch.bfloat16, device=dev)
    v = torch.empty((1, 2, N_MAX, D), dtype=torch.bfloat16, device=dev)
    a = torch.tensor(A_CLS, device=dev)
    for h in range(2):
        k[0, h, :, 0] = a[r].to(torch.bfloat16)
        k[0, h, k_star[h], 0] = B_STAR
        v[0, h] = base.to(torch.bfloat16)[r]
        v[0, h, k_star[h]] = v_star.to(torch.bfloat16)
    q = torch.zeros((1, 2, SQ_LONG, D), dtype=torch.bfloat16, device=dev)
    q[0, :, 0::2, 0] = 1.0
    q[0, :, 1::2, 0] = 0.5
    return q, k, v, k_star, base.double().cpu().numpy(), v_star.double().cpu().numpy()


def long_reference(k_star, base, v_star, n_keys=N_MAX, sq=SQ_LONG):
    """The closed form above, per head h with its special key k_star[h]."""
    o = np.zeros((len(k_star), sq, base.shape[1]))
    lse = np.zeros((len(k_star), sq))
    for h in range(len(k_star)):
        n = np.array([(n_keys - c + 6) // 7 for c in range(7)], dtype=np.float64)   # keys k < N with k % 7 == c
        n[k_star[h] % 7] -= 1
        for i in range(sq):
            q0 = 1.0 if i % 2 == 0 else 0.5
            s = q0 * np.array(A_CLS)
            s_star = q0 * B_STAR
            m = max(s.max(), s_star)
            w = n * np.exp(s - m)
            w_star = np.exp(s_star - m)
            z = w.sum() + w_star
            o[h, i] = (w @ base + w_star * v_star) / z
            lse[h, i] = m + np.log(z)
    return o, lse


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_longest_key_sequence(dtype):
    import exact_attention_32_amd as ea

    dev = torch.device("cuda:0")
    assert N_MAX * D <= 2 ** 31 - 1 < (N_MAX + 1) * D
    U.say(f"[gpu] longest key sequence S_k={N_MAX} d={D} {dtype}")
    q, k, v, k_star, base, v_star = _long_inputs(dev)
    if dtype == "bf16":
        o, lse = ea.fwd(q, k, v, causal=False, scale=1.0)
        tol = 1e-2
    else:
        f8 = torch.float8_e4m3fn
        q8, k8, v8 = q.to(f8), k.to(f8), v.to(f8)
        del k, v
        ones = [torch.ones((1, 2, (s + 127) // 128), dtype=torch.float32, device=dev) for s in (SQ_LONG, N_MAX, N_MAX)]
        o, lse = ea.fwd_fp8(q8, k8, v8, *ones, causal=False, scale=1.0)
        tol = 5e-2
    torch.cuda.synchronize()
    U.say("   kernel done")
    ro, rl = long_reference(k_star, base, v_star)
    og = o[0].double().cpu().numpy()
    lg = lse[0].double().cpu().numpy()
    d_o = float(np.abs(og - ro).max())
    d_l = float(np.abs(lg - rl).max())
    U.say(f"   max|dO| {d_o:.3e}  max|dLSE| {d_l:.3e}")
    assert d_o <= tol and d_l <= 1e-3, (d_o, d_l)
