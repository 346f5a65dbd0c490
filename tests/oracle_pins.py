"""Checks that pin the fp64 oracle to facts outside itself.

Each check takes an ``Oracle`` object and raises AssertionError on failure.
They are written so that a plausible slip anywhere in the oracle -- a dropped
scale, a wrong mask direction, a transposed or reversed index, a missing max
term in the LSE, a wrong normalisation, a wrong rescale in the online loop, a
wrong E4M3 bias -- fails at least one of them (``test_oracle_mutants.py``
plants such slips and checks that).

What pins what:
  * torch's scaled_dot_product_attention in float64 on the CPU (an independent
    library implementation of softmax attention; its ``is_causal`` mask is the
    lower-triangular, top-left one, i.e. key j visible to query i iff j <= i);
  * scipy's logsumexp on independently computed scores (the LSE);
  * brute force by a different route: O_i = sum_j v_j / sum_k exp(s_ik - s_ij);
  * closed forms (one key, causal row 0, two keys: the logistic function,
    Q = 0: the mean of the visible V rows, V = 1: ones);
  * invariants (linearity and shift in V, key/query permutations, head
    independence, scale/Q trade);
  * the OCP E4M3 definition (values in tests/golden) and torch's float8 cast.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

TINY_SHAPES = [
    (1, 1, 1, 1, 1),
    (1, 1, 3, 5, 2),
    (2, 3, 7, 7, 4),
    (1, 2, 17, 17, 8),
    (1, 2, 33, 70, 16),
    (2, 1, 70, 33, 16),
]


def _rand(shape, seed, scale=1.0):
    return np.random.Generator(np.random.PCG64(seed)).standard_normal(shape) * scale


def _case(shape, seed):
    B, H, Sq, Sk, d = shape
    q = _rand((B, H, Sq, d), seed)
    k = _rand((B, H, Sk, d), seed + 1)
    v = _rand((B, H, Sk, d), seed + 2)
    return q, k, v


def check_sdpa_fp64(oracle):
    for n, shape in enumerate(TINY_SHAPES):
        q, k, v = _case(shape, 100 + 3 * n)
        for causal in (False, True):
            scale = 0.37 + 0.1 * n
            o, _ = oracle.attention(q, k, v, causal, scale)
            ref = torch.nn.functional.scaled_dot_product_attention(
                torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), is_causal=causal, scale=scale
            ).numpy()
            err = np.abs(o - ref).max()
            assert err <= 1e-12, f"O vs SDPA fp64 {shape} causal={causal}: {err}"


def check_lse_logsumexp(oracle):
    from scipy.special import logsumexp

    for n, shape in enumerate(TINY_SHAPES):
        q, k, v = _case(shape, 200 + 3 * n)
        B, H, Sq, Sk, d = shape
        for causal in (False, True):
            scale = 0.5 + 0.05 * n
            _, lse = oracle.attention(q, k, v, causal, scale)
            s = scale * np.einsum("bhid,bhjd->bhij", q, k)
            if causal:
                mask = np.arange(Sk)[None, :] > np.arange(Sq)[:, None]
                s = np.where(mask[None, None], -np.inf, s)
            ref = logsumexp(s, axis=-1)
            err = np.abs(lse - ref).max()
            assert err <= 1e-12, f"LSE vs logsumexp {shape} causal={causal}: {err}"


def check_brute_force(oracle):
    """O_i = sum_j v_j / sum_k exp(s_ik - s_ij), LSE_i = log sum_j exp(s_ij), pure Python."""
    for n, shape in enumerate(TINY_SHAPES[:4]):
        q, k, v = _case(shape, 300 + 3 * n)
        B, H, Sq, Sk, d = shape
        for causal in (False, True):
            scale = 0.8
            o, lse = oracle.attention(q, k, v, causal, scale)
            for b in range(B):
                for h in range(H):
                    for i in range(Sq):
                        vis = [j for j in range(Sk) if (not causal) or j <= i]
                        s = {j: scale * math.fsum(float(q[b, h, i, t]) * float(k[b, h, j, t]) for t in range(d))
                             for j in vis}
                        w = {j: 1.0 / math.fsum(math.exp(s[kk] - s[j]) for kk in vis) for j in vis}
                        for t in range(d):
                            ref = math.fsum(w[j] * float(v[b, h, j, t]) for j in vis)
                            assert abs(o[b, h, i, t] - ref) <= 1e-12, ("brute O", shape, causal, b, h, i, t)
                        ref_lse = math.log(math.fsum(math.exp(s[j]) for j in vis))
                        assert abs(lse[b, h, i] - ref_lse) <= 1e-12, ("brute LSE", shape, causal, b, h, i)


def check_softmax_rows(oracle):
    q, k, _ = _case((1, 2, 40, 50, 8), 400)
    for causal in (False, True):
        P = oracle.softmax_block(q, k, causal, 0.9, bh=1, i0=3, nr=30)
        assert np.all(P >= 0.0)
        sums = P.sum(axis=1)
        assert np.abs(sums - 1.0).max() <= 1e-14 * 50, f"rows do not sum to 1: {sums}"
        if causal:
            for r in range(30):
                i = 3 + r
                assert np.all(P[r, i + 1:] == 0.0), "masked entries must be exactly zero"
                assert np.all(P[r, : i + 1] > 0.0)


def check_v_ones(oracle):
    for causal in (False, True):
        q, k, _ = _case((2, 2, 19, 23, 8), 500)
        v = np.ones((2, 2, 23, 8))
        o, _ = oracle.attention(q, k, v, causal, 1.3)
        assert np.abs(o - 1.0).max() <= 1e-14, "V = 1 must give O = 1"


def check_q_zero(oracle):
    for causal in (False, True):
        _, k, v = _case((1, 2, 21, 17, 8), 600)
        q = np.zeros((1, 2, 21, 8))
        o, lse = oracle.attention(q, k, v, causal, 0.7)
        for i in range(21):
            n = min(i + 1, 17) if causal else 17
            ref = v[:, :, :n, :].mean(axis=2)
            assert np.abs(o[:, :, i, :] - ref).max() <= 1e-13, ("Q = 0 mean", causal, i)
            assert np.abs(lse[:, :, i] - math.log(n)).max() <= 1e-13, ("Q = 0 LSE", causal, i)


def check_closed_forms(oracle):
    # one key: O_i = v_0, LSE_i = scale * q_i . k_0
    q, k, v = _case((1, 1, 6, 1, 4), 700)
    for causal in (False, True):
        o, lse = oracle.attention(q, k, v, causal, 0.6)
        assert np.abs(o - v[:, :, :1, :]).max() <= 1e-15
        ref = 0.6 * np.array([math.fsum(q[0, 0, i] * k[0, 0, 0]) for i in range(6)])
        assert np.abs(lse[0, 0] - ref).max() <= 1e-14
    # causal row 0 sees only key 0
    q, k, v = _case((1, 2, 9, 9, 4), 710)
    o, lse = oracle.attention(q, k, v, True, 0.45)
    assert np.abs(o[:, :, 0, :] - v[:, :, 0, :]).max() == 0.0
    ref = 0.45 * np.array([[math.fsum(q[0, h, 0] * k[0, h, 0]) for h in range(2)]])
    assert np.abs(lse[:, :, 0] - ref).max() <= 1e-14
    # causal row 1: two keys, weights are logistic functions of the score gap
    s0 = 0.45 * math.fsum(q[0, 0, 1] * k[0, 0, 0])
    s1 = 0.45 * math.fsum(q[0, 0, 1] * k[0, 0, 1])
    w0 = 1.0 / (1.0 + math.exp(s1 - s0))
    w1 = 1.0 / (1.0 + math.exp(s0 - s1))
    assert np.abs(o[0, 0, 1] - (w0 * v[0, 0, 0] + w1 * v[0, 0, 1])).max() <= 1e-14
    hi, lo = max(s0, s1), min(s0, s1)
    assert abs(lse[0, 0, 1] - (hi + math.log1p(math.exp(lo - hi)))) <= 1e-14
    # hand-derived two-key example: q = (1, 0), k = I, v = [[1, 2], [3, 4]], scale 1
    with open(os.path.join(GOLDEN, "two_key_example.json")) as f:
        g = json.load(f)
    o, lse = oracle.attention(np.array(g["q"], float)[None, None], np.array(g["k"], float)[None, None],
                              np.array(g["v"], float)[None, None], False, g["scale"])
    e = math.e
    ref_o = [(e * 1 + 3) / (e + 1), (e * 2 + 4) / (e + 1)]   # softmax(1, 0) = (e, 1)/(e + 1)
    assert np.abs(o[0, 0, 0] - ref_o).max() <= 1e-15
    assert abs(lse[0, 0, 0] - math.log(e + 1)) <= 1e-15


def check_invariants(oracle):
    B, H, Sq, Sk, d = 1, 2, 13, 29, 8
    q, k, v = _case((B, H, Sq, Sk, d), 800)
    v2 = _rand(v.shape, 803)
    for causal in (False, True):
        o1, l1 = oracle.attention(q, k, v, causal, 0.55)
        o2, _ = oracle.attention(q, k, v2, causal, 0.55)
        o12, l12 = oracle.attention(q, k, 2.0 * v - 3.0 * v2, causal, 0.55)
        assert np.abs(o12 - (2.0 * o1 - 3.0 * o2)).max() <= 1e-13, "linearity in V"
        assert np.abs(l12 - l1).max() == 0.0, "LSE does not depend on V"
        os_, _ = oracle.attention(q, k, v + 1.75, causal, 0.55)
        assert np.abs(os_ - (o1 + 1.75)).max() <= 1e-13, "shift in V"
        # scale and Q trade: (2q, s/2) == (q, s) up to rounding
        oq, lq = oracle.attention(2.0 * q, k, v, causal, 0.275)
        assert np.abs(oq - o1).max() <= 1e-13 and np.abs(lq - l1).max() <= 1e-13
        # head independence
        q3 = q.copy()
        q3[:, 1] = _rand(q3[:, 1].shape, 805)
        o3, l3 = oracle.attention(q3, k, v, causal, 0.55)
        assert np.array_equal(o3[:, 0], o1[:, 0]) and np.array_equal(l3[:, 0], l1[:, 0])
        assert np.abs(o3[:, 1] - o1[:, 1]).max() > 1e-3
    # non-causal: permuting keys together with values leaves O unchanged; permuting queries permutes O
    perm = np.random.Generator(np.random.PCG64(9)).permutation(Sk)
    o1, l1 = oracle.attention(q, k, v, False, 0.55)
    op, lp = oracle.attention(q, k[:, :, perm], v[:, :, perm], False, 0.55)
    assert np.abs(op - o1).max() <= 1e-13 and np.abs(lp - l1).max() <= 1e-13
    qperm = np.random.Generator(np.random.PCG64(10)).permutation(Sq)
    oqp, lqp = oracle.attention(q[:, :, qperm], k, v, False, 0.55)
    assert np.abs(oqp - o1[:, :, qperm]).max() <= 1e-13 and np.abs(lqp - l1[:, :, qperm]).max() <= 1e-13
    # causal: changing a key that query i cannot see does not change row i
    k4, v4 = k.copy(), v.copy()
    k4[:, :, 7:] = _rand(k4[:, :, 7:].shape, 811)
    v4[:, :, 7:] = _rand(v4[:, :, 7:].shape, 812)
    oc, lc = oracle.attention(q, k, v, True, 0.55)
    oc4, lc4 = oracle.attention(q, k4, v4, True, 0.55)
    assert np.array_equal(oc4[:, :, :7], oc[:, :, :7]) and np.array_equal(lc4[:, :, :7], lc[:, :, :7])
    assert np.abs(oc4[:, :, 7:] - oc[:, :, 7:]).max() > 1e-3


def check_online_equals_two_pass(oracle):
    for shape in [(1, 2, 37, 37, 8), (2, 1, 50, 300, 16), (1, 1, 300, 50, 4)]:
        q, k, v = _case(shape, 900)
        for causal in (False, True):
            o, lse = oracle.attention(q, k, v, causal, 0.66)
            for bc in (1, 16, 37, 64, 256):
                oo, lo = oracle.attention_online(q, k, v, causal, 0.66, bc)
                assert np.abs(oo - o).max() <= 1e-12, ("online O", shape, causal, bc)
                assert np.abs(lo - lse).max() <= 1e-12, ("online LSE", shape, causal, bc)


def check_rows_mode(oracle):
    q, k, v = _case((2, 3, 40, 45, 8), 1000)
    rows = np.array([[0, 0], [5, 39], [3, 17], [1, 1], [4, 44 - 5]])
    for causal in (False, True):
        o, lse = oracle.attention(q, k, v, causal, 0.4)
        orow, lrow = oracle.attention_rows(q, k, v, causal, 0.4, rows)
        for n, (bh, i) in enumerate(rows):
            b, h = divmod(int(bh), 3)
            assert np.array_equal(orow[n], o[b, h, i]) and lrow[n] == lse[b, h, i]


def check_e4m3_decode(oracle):
    table = oracle.e4m3_table()
    with open(os.path.join(GOLDEN, "e4m3_ocp_values.json")) as f:
        g = json.load(f)
    for hexcode, val in g["values"].items():
        c = int(hexcode, 16)
        if val == "nan":
            assert math.isnan(table[c]), hexcode
        else:
            assert table[c] == float(val), (hexcode, table[c], val)
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(table), nan)
    assert np.array_equal(table[~nan], ref[~nan])


def check_decode_blocks(oracle):
    rng = np.random.Generator(np.random.PCG64(1100))
    B, H, S, d = 2, 3, 300, 8
    codes = rng.integers(0, 256, size=(B, H, S, d), dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x42   # no NaN codes in data
    desc = rng.uniform(0.01, 2.0, size=(B, H, 3)).astype(np.float32)
    out = oracle.decode_e4m3_blocks(codes, desc)
    vals = codes.view(np.uint8)
    ref_tab = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ref = ref_tab[vals] * np.repeat(desc.astype(np.float64), 128, axis=2)[:, :, :S, None]
    assert np.array_equal(out, ref)


def check_large_scores(oracle):
    """Scores near 1000 (no overflow allowed): two keys with s = (1000, 999.5) -> logistic weights."""
    q = np.array([[[[1.0, 0.0]]]])
    k = np.array([[[[1000.0, 0.0], [999.5, 0.0]]]])
    v = np.array([[[[1.0, -2.0], [5.0, 3.0]]]])
    o, lse = oracle.attention(q, k, v, False, 1.0)
    w0 = 1.0 / (1.0 + math.exp(-0.5))
    w1 = 1.0 / (1.0 + math.exp(0.5))
    assert np.all(np.isfinite(o)) and np.isfinite(lse[0, 0, 0])
    assert np.abs(o[0, 0, 0] - (w0 * v[0, 0, 0] + w1 * v[0, 0, 1])).max() <= 1e-14
    assert abs(lse[0, 0, 0] - (1000.0 + math.log1p(math.exp(-0.5)))) <= 1e-12
    oo, lo = oracle.attention_online(q, k, v, False, 1.0, 1)
    assert np.abs(oo - o).max() <= 1e-14 and abs(lo[0, 0, 0] - lse[0, 0, 0]) <= 1e-12
    # and against the library on a random case with large scores of both signs
    qq, kk, vv = _case((1, 2, 20, 30, 8), 1200)
    for causal in (False, True):
        o, _ = oracle.attention(qq, kk, vv, causal, 150.0)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(qq), torch.from_numpy(kk), torch.from_numpy(vv), is_causal=causal, scale=150.0
        ).numpy()
        assert np.all(np.isfinite(o)) and np.abs(o - ref).max() <= 1e-12


def check_e4m3_encode(oracle):
    """Nearest-even E4M3 encoding against torch's float8_e4m3fn cast (round to nearest even from
    fp32): every finite value, every midpoint between neighbours (exact ties), the floats next to
    each midpoint, random floats in range, both signs; saturation above 448; code round trip."""
    tab = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    vals = tab[[c for c in range(127)]]                      # 0 .. 448, code order
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)   # exact in fp32
    up = np.nextafter(mids, np.float32(np.inf))
    dn = np.nextafter(mids, np.float32(0))
    rng = np.random.Generator(np.random.PCG64(1300))
    rnd = np.concatenate([rng.uniform(0, 448, 4000), np.exp2(rng.uniform(-12, 8.8, 4000))]).astype(np.float32)
    pos = np.concatenate([vals.astype(np.float32), mids, up, dn, rnd])
    pos = pos[pos <= 448]
    x = np.concatenate([pos, -pos]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = oracle.e4m3_encode(x.astype(np.float64))
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(float(x[i]), int(got[i]), int(ref[i])) for i in bad[:5]]
    big = np.array([448.001, 449.0, 463.99, 464.0, 500.0, 1e4, 3e38])
    assert np.all(oracle.e4m3_encode(big) == 0x7E) and np.all(oracle.e4m3_encode(-big) == 0xFE)
    finite = [c for c in range(256) if (c & 0x7F) != 0x7F]
    assert np.array_equal(oracle.e4m3_encode(tab[finite]), np.array(finite, dtype=np.uint8))


def check_quantize_blocks(oracle):
    """Block quantisation against the input generator's independent quantiser, and its defining
    relations: descale = fp32(amax) / fp32(448) (1 for an all-zero block), the element of largest
    |x| gets the largest code (448), the ragged last block has its own scale, and every decoded
    value is within half a code step of x."""
    from exact_attention_32_amd import inputs as I

    rng = np.random.Generator(np.random.PCG64(1400))
    B, H, S, d = 2, 3, 300, 16
    x = rng.standard_normal((B, H, S, d), dtype=np.float32)
    x[:, :, 128:256] *= np.float32(37.5)          # blocks of different scales
    x[1, 2, 0:128] = 0.0                          # an all-zero block
    x[0, 1, 130, 3] = -1000.0                     # a block whose |max| is negative
    codes, ds = oracle.quantize_e4m3_blocks(x)
    rc, rd = I.quantize_e4m3_blocks(x)
    assert np.array_equal(codes, rc) and np.array_equal(ds, rd)
    tab = oracle.e4m3_table()
    for b in range(B):
        for h in range(H):
            for j in range(3):
                xb = x[b, h, j * 128:(j + 1) * 128]
                amax = np.float32(np.abs(xb).max())
                want = np.float32(amax / np.float32(448.0)) if amax > 0 else np.float32(1.0)
                assert ds[b, h, j] == want
                cb = codes[b, h, j * 128:(j + 1) * 128]
                if amax > 0:
                    assert (cb.reshape(-1)[np.argmax(np.abs(xb))] & 0x7F) == 0x7E
                dec = tab[cb] * np.float64(ds[b, h, j])
                step = np.maximum(np.abs(xb.astype(np.float64)) * 2.0 ** -3, 2.0 ** -9 * np.float64(ds[b, h, j]))
                assert np.all(np.abs(dec - xb) <= step / 2 * (1 + 1e-12))
    assert np.all(codes[1, 2, 0:128] == 0) and ds[1, 2, 0] == 1.0


def check_e5m2(oracle):
    """E5M2 values against torch's float8_e5m2 view of all 256 codes; nearest-even encoding against
    torch's cast on finite values, midpoints and their neighbouring floats; saturation at 57344;
    block quantisation against the input generator's E5M2 quantiser."""
    from exact_attention_32_amd import inputs as I

    table = oracle.e5m2_table()
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e5m2).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(table), nan) and np.array_equal(table[~nan], ref[~nan])
    vals = ref[:0x7C]                                   # 0 .. 57344, code order
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    rng = np.random.Generator(np.random.PCG64(1500))
    pos = np.concatenate([vals.astype(np.float32), mids, np.nextafter(mids, np.float32(np.inf)),
                          np.nextafter(mids, np.float32(0)), np.exp2(rng.uniform(-18, 15.8, 3000)).astype(np.float32)])
    pos = pos[pos <= 57344]
    x = np.concatenate([pos, -pos]).astype(np.float32)
    want = torch.from_numpy(x).to(torch.float8_e5m2).view(torch.uint8).numpy()
    got = oracle.fp8_encode(x.astype(np.float64), "e5m2")
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(x[i]), int(got[i]), int(want[i])) for i in bad[:5]]
    big = np.array([57345.0, 61439.0, 61440.0, 1e6])
    assert np.all(oracle.fp8_encode(big, "e5m2") == 0x7B) and np.all(oracle.fp8_encode(-big, "e5m2") == 0xFB)
    xq = rng.standard_normal((2, 2, 200, 8), dtype=np.float32)
    xq[:, :, 128:] *= np.float32(1e-3)
    c, d = oracle.quantize_fp8_blocks(xq, "e5m2")
    rc, rd = I.quantize_fp8_blocks(xq, "e5m2")
    assert np.array_equal(c, rc) and np.array_equal(d, rd)
    amax = np.abs(xq[:, :, :128]).max(axis=(2, 3)).astype(np.float32)
    assert np.array_equal(d[:, :, 0], (amax / np.float32(57344.0)).astype(np.float32))
    dec = oracle.decode_fp8_blocks(c, d, "e5m2")
    assert np.array_equal(dec, table[c] * np.repeat(d.astype(np.float64), 128, axis=2)[:, :, :200, None])


def check_rmsnorm(oracle):
    """RMSNorm across heads against closed forms and invariants: a constant token gives
    c / sqrt(eps + c^2) * w; with eps = 0 and unit weights every token's hidden vector (all heads)
    has mean square 1, the ratio between heads of one token is kept (one RMS per token, not per
    head), the map is invariant under positive scaling and odd; a one-hot weight selects exactly
    its channel (h * d + t); tokens are independent; an all-zero token stays zero."""
    rng = np.random.Generator(np.random.PCG64(4100))
    B, H, S, d = 2, 3, 5, 4
    # constant tokens: closed form
    for c, eps in ((0.5, 0.0), (0.5, 1e-6), (-3.0, 0.25), (1e-4, 1e-6)):
        x = np.full((B, H, S, d), c)
        w = rng.uniform(0.5, 2.0, H * d)
        out = oracle.rmsnorm_across_heads(x, w, eps)
        want = c / math.sqrt(eps + c * c) * w.reshape(1, H, 1, d)
        assert np.allclose(out, np.broadcast_to(want, out.shape), rtol=1e-14, atol=0)
    # unit mean square per token over all heads; heads of different scale keep their ratio
    x = rng.standard_normal((B, H, S, d))
    x[:, 1] *= 10.0
    x[:, 2] *= 0.01
    ones = np.ones(H * d)
    out = oracle.rmsnorm_across_heads(x, ones, 0.0)
    ms = (out ** 2).mean(axis=(1, 3))
    assert np.allclose(ms, 1.0, rtol=0, atol=1e-12)
    ratio = out / x
    assert np.allclose(ratio, ratio[:, :1, :, :1], rtol=1e-13, atol=0)
    # positive scaling invariance and oddness (eps = 0)
    assert np.allclose(oracle.rmsnorm_across_heads(3.7 * x, ones, 0.0), out, rtol=1e-13, atol=0)
    assert np.array_equal(oracle.rmsnorm_across_heads(-x, ones, 0.0), -out)
    # one-hot weight: only channel (h, t) survives, with the token's factor
    for h, t in ((0, 0), (2, 3), (1, 2)):
        w = np.zeros(H * d)
        w[h * d + t] = 1.0
        o1 = oracle.rmsnorm_across_heads(x, w, 0.0)
        mask = np.zeros((H, d), bool)
        mask[h, t] = True
        assert np.all(o1.transpose(0, 2, 1, 3)[:, :, ~mask] == 0.0)
        assert np.allclose(o1[:, h, :, t], out[:, h, :, t], rtol=1e-14, atol=0)
    # tokens are independent; a zero token stays zero (eps > 0)
    x2 = x.copy()
    x2[1, :, 3, :] = 0.0
    x2[0, :, 2, :] *= 5.0
    o2 = oracle.rmsnorm_across_heads(x2, ones, 1e-6)
    o_ref = oracle.rmsnorm_across_heads(x, ones, 1e-6)
    keep = np.ones((B, S), bool)
    keep[1, 3] = keep[0, 2] = False
    assert np.array_equal(o2.transpose(0, 2, 1, 3)[keep], o_ref.transpose(0, 2, 1, 3)[keep])
    assert np.all(o2[1, :, 3, :] == 0.0)
    # eps enters under the square root, added to the mean square
    xs = np.full((1, 2, 1, 2), 1e-3)
    o3 = oracle.rmsnorm_across_heads(xs, np.ones(4), 1e-6)
    assert np.allclose(o3, 1e-3 / math.sqrt(1e-6 + 1e-6), rtol=1e-14, atol=0)


ALL_CHECKS = [
    check_sdpa_fp64,
    check_lse_logsumexp,
    check_brute_force,
    check_softmax_rows,
    check_v_ones,
    check_q_zero,
    check_closed_forms,
    check_invariants,
    check_online_equals_two_pass,
    check_rows_mode,
    check_e4m3_decode,
    check_e4m3_encode,
    check_quantize_blocks,
    check_e5m2,
    check_rmsnorm,
    check_decode_blocks,
    check_large_scores,
]
