"""GPU parity: the HIP kernels against the fp64 oracle, element by element.

Gate, per element: |O - O_ref| <= 1e-2 for f16/bf16 and 5e-2 for fp8 (E4M3 and E5M2), or else O
within one ulp of the correctly rounded RN(O_ref) (bf16 spacing is 2^-6 in [2, 4) and 2^-5 in
[4, 8), so there a correctly rounded output alone can miss 1e-2); such elements are counted and
reported, split by whether RN(O_ref) itself misses the tolerance; max |LSE - LSE_ref| <= 1e-3.
"""
import numpy as np
import pytest
import torch

from exact_attention_32_amd import inputs as I
from oracle import attn_oracle
from tests import parity_util as U

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def oracle():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import exact_attention_32_amd as ea

    ea.load_library()
    return attn_oracle.get()


# (B, H, S_q, S_k, d): several tiles plus ragged tails, S_q != S_k, tiny and single-row cases
SMALL = [
    (1, 1, 1, 1, 64),
    (1, 1, 1, 1, 128),
    (1, 2, 3, 17, 128),
    (1, 2, 17, 3, 64),
    (1, 1, 17, 17, 128),
    (2, 3, 130, 130, 64),
    (1, 2, 130, 200, 128),
    (2, 2, 300, 333, 128),
    (1, 3, 333, 300, 64),
    (1, 2, 513, 257, 128),
    (2, 1, 640, 640, 64),
    (1, 2, 1000, 1000, 128),
    # at most 128 query rows (the small-problem workgroup shape) against many key tiles
    (1, 2, 128, 700, 128),
    (2, 2, 96, 1000, 64),
]


def _run_full(oracle, w):
    x = I.make_inputs(w)
    U.say(f"[gpu] {w.name} causal={w.causal}")
    o, lse = U.run_gpu(x)
    q, k, v = U.oracle_inputs(x, oracle)
    ro, rl = oracle.attention(q, k, v, w.causal, w.scale)
    few = U.fp8_few_key_tolerance(oracle, q, k, v, ro, w.causal, w.scale) if I.is_fp8(w.dtype) else None
    st = U.compare(o.double().cpu().numpy(), lse.double().cpu().numpy(), ro, rl, w.dtype, few_key_tol=few)
    U.say(f"   {st}")
    return st


@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("causal", [False, True])
def test_small_full(oracle, shape, dtype, causal):
    B, H, Sq, Sk, d = shape
    w = I.random_workload(B, H, Sq, Sk, d, dtype, causal, seed=1000 + Sq + 7 * Sk + d)
    st = _run_full(oracle, w)
    assert st["pass"], st


@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("causal", [False, True])
def test_small_full_fp8(oracle, shape, causal):
    B, H, Sq, Sk, d = shape
    w = I.random_workload(B, H, Sq, Sk, d, "fp8", causal, seed=2000 + Sq + 7 * Sk + d)
    st = _run_full(oracle, w)
    assert st["pass"], st


@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("causal", [False, True])
def test_small_full_e5m2(oracle, shape, causal):
    B, H, Sq, Sk, d = shape
    w = I.random_workload(B, H, Sq, Sk, d, "e5m2", causal, seed=2500 + Sq + 7 * Sk + d)
    st = _run_full(oracle, w)
    assert st["pass"], st


SCHEDULES = [(1, 1, 8, 3, 64), (1, 1, 8, 4, 64), (1, 2, 4, 3, 64), (1, 2, 4, 4, 64), (1, 1, 4, 2, 64),
             (1, 1, 4, 3, 64), (1, 1, 8, 2, 128), (2, 1, 8, 3, 64), (3, 1, 8, 4, 64), (1, 2, 8, 3, 64),
             (1, 2, 8, 4, 64), (1, 1, 4, 3, 192), (1, 1, 4, 2, 256)]
D64_ONLY = {(1, 2, 8, 3, 64), (1, 2, 8, 4, 64), (1, 1, 4, 3, 192), (1, 1, 4, 2, 256)}
SCHED_SHAPES = [(1, 1, 1, 1, 64), (1, 2, 17, 3, 128), (2, 3, 130, 130, 64), (1, 2, 300, 333, 128),
                (1, 2, 513, 257, 128), (1, 2, 1000, 1000, 64)]


@pytest.mark.parametrize("sched", SCHEDULES, ids=lambda s: "s%d_%d_%d_%d_%d" % s)
def test_every_schedule(oracle, sched):
    """Every compiled schedule and tile shape (not only the policy table's choice), bf16 and f16,
    causal and not, on ragged shapes at both head dimensions."""
    import exact_attention_32_amd as ea

    ea.set_policy(*sched)
    try:
        for i, (B, H, Sq, Sk, d) in enumerate(SCHED_SHAPES):
            if sched in D64_ONLY and d != 64:
                x = I.make_inputs(I.random_workload(B, H, Sq, Sk, d, "bf16", False, seed=1))
                with pytest.raises(ea.AttnError):
                    U.run_gpu(x)
                continue
            for dtype in ("bf16", "f16"):
                for causal in (False, True):
                    w = I.random_workload(B, H, Sq, Sk, d, dtype, causal, seed=3000 + 17 * i + sched[0])
                    st = _run_full(oracle, w)
                    assert st["pass"], (sched, w.name, st)
    finally:
        ea.set_policy(ea.ATTN_SCHED_DEFAULT)


# causal shapes whose (batch, head) count makes the library pair query tiles (n-1-j, j) in one
# workgroup, the light tile with its keys in reverse order: even and odd tile counts (an odd one
# leaves the middle tile alone), S_q < S_k and S_q > S_k, both head dimensions and tile shapes
PAIRED = [(1, 128, 2048, 2048, 64), (2, 43, 1200, 1200, 128), (1, 128, 1000, 1100, 128), (2, 256, 1300, 900, 64)]


@pytest.mark.parametrize("shape", PAIRED, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_causal_pairs(oracle, shape, dtype):
    import exact_attention_32_amd as ea

    B, H, Sq, Sk, d = shape
    bq, bk, w_, n = ea.plan(B, H, Sq, Sk, d, True)
    nqt = -(-Sq // bq)
    assert n == B * H * ((nqt + 1) // 2), (shape, bq, n)   # paired
    w = I.random_workload(B, H, Sq, Sk, d, dtype, True, seed=4000 + Sq + 7 * Sk + d + H)
    st = _run_full(oracle, w)
    assert st["pass"], st


@pytest.mark.parametrize("shape", [s for s in PAIRED if s[4] == 64], ids=lambda s: "x".join(map(str, s)))
def test_causal_pairs_wide(oracle, shape):
    """The d = 64 tiles of 64 queries per wave and 64 keys, paired: 4 query tiles a head (even)
    and 3 (odd, the middle one alone)."""
    import exact_attention_32_amd as ea

    B, H, Sq, Sk, d = shape
    ea.set_policy(ea.ATTN_SCHED_CLASSIC, 2, 8, 4, 64)
    try:
        bq, bk, w_, n = ea.plan(B, H, Sq, Sk, d, True)
        nqt = -(-Sq // bq)
        assert bq == 512 and n == B * H * ((nqt + 1) // 2), (shape, bq, n)
        for dtype in ("bf16", "f16"):
            w = I.random_workload(B, H, Sq, Sk, d, dtype, True, seed=4100 + Sq + 7 * Sk + H)
            st = _run_full(oracle, w)
            assert st["pass"], (dtype, st)
    finally:
        ea.set_policy(ea.ATTN_SCHED_DEFAULT)


@pytest.mark.parametrize("kind", ["ramp12", "step40", "step150"])
def test_causal_pairs_rising(oracle, kind):
    """Rising scores through paired causal tiles: the heavy tile raises its running max as the
    keys go up, the light tile (keys in reverse order) starts from its largest scores."""
    import exact_attention_32_amd as ea

    dev = "cuda:0"
    for d, dtype, S in ((64, "bf16", 1024), (128, "f16", 1024)):
        q, k, v = _rising_inputs(kind, 1, 128, S, d, dtype, seed=d + 11)
        bq, _, _, n = ea.plan(1, 128, S, S, d, True)
        assert S // bq == 4 and n == 128 * 2   # four query tiles a head, in two pairs
        U.say(f"[gpu] pairs rising {kind} d={d} {dtype}")
        o, lse = ea.fwd(q.to(dev), k.to(dev), v.to(dev), causal=True, scale=d ** -0.5)
        torch.cuda.synchronize()
        ro, rl = oracle.attention(q.double().numpy(), k.double().numpy(), v.double().numpy(), True, d ** -0.5)
        st = U.compare(o.double().cpu().numpy(), lse.double().cpu().numpy(), ro, rl, dtype)
        assert st["pass"], (kind, d, dtype, st)


def _random_shapes(n, seed):
    """Seeded random problem shapes: ragged S_q and S_k (equal, shorter or longer), both head dims,
    all four input types, causal or not, and head counts up to 300 so that a share of the causal
    f16/bf16 ones reach the paired-tile launch (B*H*ceil(n/2) >= 256)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out = []
    for i in range(n):
        d = int(rng.choice([64, 128]))
        dtype = str(rng.choice(["bf16", "f16", "fp8", "e5m2"]))
        causal = bool(rng.integers(0, 2))
        B = int(rng.integers(1, 3))
        H = int(rng.choice([1, 3, 17, 130, 300]))
        if d == 128 and H == 300:
            H = 260
        S_q = int(rng.integers(1, 1400 if H < 100 else 700))
        S_k = int(max(1, S_q + rng.integers(-S_q // 2, S_q // 2 + 2)))
        out.append((B, H, S_q, S_k, d, dtype, causal, 6000 + i))
    return out


@pytest.mark.parametrize("case", _random_shapes(96, 2024), ids=lambda c: "%s_b%d_h%d_%dx%d_d%d%s" % (
    c[5], c[0], c[1], c[2], c[3], c[4], "_causal" if c[6] else ""))
def test_random_shapes(oracle, case):
    """Every element against the oracle on seeded random shapes (the default policy)."""
    B, H, Sq, Sk, d, dtype, causal, seed = case
    w = I.random_workload(B, H, Sq, Sk, d, dtype, causal, seed=seed)
    st = _run_full(oracle, w)
    assert st["pass"], (case, st)


@pytest.mark.parametrize("causal", [False, True])
def test_outliers_small(oracle, causal):
    w = I.random_workload(1, 2, 700, 700, 64, "bf16", causal, seed=55, outliers=True)
    st = _run_full(oracle, w)
    assert st["pass"], st


def test_tiny_workload_full(oracle):
    w = I.WORKLOADS["f16_b1_h2_s128_d64"]
    st = _run_full(oracle, w)
    assert st["pass"], st


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_invariant_inputs(oracle, d, causal):
    """V = 1 gives O = 1; Q = 0 gives the mean of the visible V rows and LSE = log(count)."""
    dev = "cuda:0"
    import exact_attention_32_amd as ea

    B, H, S = 1, 2, 300
    U.say(f"[gpu] invariants d={d} causal={causal}")
    g = torch.Generator().manual_seed(d + causal)
    q = torch.randn(B, H, S, d, generator=g).to(torch.bfloat16)
    k = torch.randn(B, H, S, d, generator=g).to(torch.bfloat16)
    v = torch.randn(B, H, S, d, generator=g).to(torch.bfloat16)
    ones = torch.ones_like(v)
    o, _ = ea.fwd(q.to(dev), k.to(dev), ones.to(dev), causal=causal, scale=d ** -0.5)
    assert torch.all(o.cpu().float() == 1.0)
    z = torch.zeros_like(q)
    o, lse = ea.fwd(z.to(dev), k.to(dev), v.to(dev), causal=causal, scale=d ** -0.5)
    torch.cuda.synchronize()
    vv = v.double()
    n = torch.arange(1, S + 1, dtype=torch.float64)
    ref = (vv.cumsum(2) / n[None, None, :, None]) if causal else vv.mean(2, keepdim=True).expand_as(vv)
    ref_lse = torch.log(n) if causal else torch.full((S,), float(np.log(S)), dtype=torch.float64)
    st = U.compare(o.cpu().double().numpy(), lse.cpu().double().numpy(), ref.numpy(),
                   ref_lse[None, None, :].expand(B, H, S).numpy(), "bf16")
    assert st["pass"], st


def _rising_inputs(kind, B, H, S, d, dtype, seed, knoise=0.5):
    """Scores that grow along the keys, so the running max keeps moving: every query and key
    share a component along u = (1, ..., 1), with a key weight r_j.  In base-2 units the score
    is about r_j * sqrt(d) * log2(e) above the noise: 'ramp3' and 'ramp12' raise it by 3 and 12
    per 128 keys; 'step20', 'step40', 'step90' and 'step150' jump by that much at key 256 (past
    2^15 a probability does not fit f16, past 2^64 the kernel forms P again for bf16 too, and
    2^150 overflows fp32, so p = exp2 of the score over a stale max is infinite there)."""
    g = torch.Generator().manual_seed(seed)
    j = torch.arange(S, dtype=torch.float64)
    unit = float(np.sqrt(d) * np.log2(np.e))
    if kind == "ramp3":
        r = j * (3.0 / 128) / unit
    elif kind == "ramp12":
        r = j * (12.0 / 128) / unit
    else:
        r = (j >= 256).double() * (float(kind[4:]) / unit)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float16
    q = (0.5 * torch.randn(B, H, S, d, generator=g, dtype=torch.float64) + 1.0).to(dt)
    k = (knoise * torch.randn(B, H, S, d, generator=g, dtype=torch.float64) + r[None, None, :, None]).to(dt)
    v = torch.randn(B, H, S, d, generator=g, dtype=torch.float64).to(dt)
    return q, k, v


CLASSIC = [s for s in SCHEDULES if s[0] == 1]


@pytest.mark.parametrize("kind", ["ramp3", "ramp12", "step20", "step40", "step90", "step150"])
@pytest.mark.parametrize("sched", [None] + CLASSIC, ids=lambda s: "default" if s is None else "s%d_%d_%d_%d_%d" % s)
def test_rising_scores(oracle, kind, sched):
    """Running max raised inside the key loop, by small and by overflowing steps, on every
    classic schedule: the row-sum bound must catch it and the update must keep O and LSE exact."""
    import exact_attention_32_amd as ea

    dev = "cuda:0"
    if sched is not None:
        ea.set_policy(*sched)
    try:
        for d in (64, 128):
            if sched is not None and sched in D64_ONLY and d != 64:
                continue
            for dtype in ("bf16", "f16"):
                for causal in (False, True):
                    q, k, v = _rising_inputs(kind, 1, 2, 700, d, dtype, seed=d + 2 * causal)
                    U.say(f"[gpu] rising {kind} sched={sched} d={d} {dtype} causal={causal}")
                    o, lse = ea.fwd(q.to(dev), k.to(dev), v.to(dev), causal=causal, scale=d ** -0.5)
                    torch.cuda.synchronize()
                    ro, rl = oracle.attention(q.double().numpy(), k.double().numpy(), v.double().numpy(), causal,
                                              d ** -0.5)
                    st = U.compare(o.double().cpu().numpy(), lse.double().cpu().numpy(), ro, rl, dtype)
                    assert st["pass"], (kind, sched, d, dtype, causal, st)
    finally:
        ea.set_policy(ea.ATTN_SCHED_DEFAULT)


@pytest.mark.parametrize("scale_log2", [20, 40])
def test_rising_scores_large_values(oracle, scale_log2):
    """bf16: a step of 60 in base 2 (P up to 2^60 on the tile that moves the max: the deferred
    factor, not a second pass) with V, then V scaled by 2^20 or 2^40, so that this tile's products
    reach 2^106.  O is linear in V and every step of the kernel commutes with scaling V by a power
    of two while nothing overflows, so the scaled output must be finite and exactly 2^s times the
    unscaled one, which passes the gate against the oracle."""
    import exact_attention_32_amd as ea

    dev = "cuda:0"
    for d in (64, 128):
        for causal in (False, True):
            q, k, v = _rising_inputs("step60", 1, 2, 700, d, "bf16", seed=d + 2 * causal + scale_log2)
            vs = (v.double() * 2.0 ** scale_log2).to(torch.bfloat16)
            U.say(f"[gpu] rising step60 V x 2^{scale_log2} d={d} causal={causal}")
            o, lse = ea.fwd(q.to(dev), k.to(dev), v.to(dev), causal=causal, scale=d ** -0.5)
            o_s, lse_s = ea.fwd(q.to(dev), k.to(dev), vs.to(dev), causal=causal, scale=d ** -0.5)
            torch.cuda.synchronize()
            assert torch.isfinite(o_s).all()
            assert torch.equal(o_s.double(), o.double() * 2.0 ** scale_log2) and torch.equal(lse_s, lse)
            ro, rl = oracle.attention(q.double().numpy(), k.double().numpy(), v.double().numpy(), causal, d ** -0.5)
            st = U.compare(o.double().cpu().numpy(), lse.double().cpu().numpy(), ro, rl, "bf16")
            assert st["pass"], (scale_log2, d, causal, st)


@pytest.mark.parametrize("kind", ["ramp3", "ramp12", "step20", "step150"])
@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_rising_scores_fp8(oracle, kind, fmt):
    """The same rising scores through the fp8 kernel (block-quantised from the fp32 values).  The
    keys' own noise is small here, so that a row's weight spreads over many keys: P in E4M3 has
    4 significant bits, and a row dominated by two or three keys would test that rounding (a
    property of the fp8 path), not the running max."""
    import exact_attention_32_amd as ea

    dev = "cuda:0"
    for d in (64, 128):
        for causal in (False, True):
            q, k, v = (t.float().numpy() for t in _rising_inputs(kind, 1, 2, 700, d, "bf16", seed=d + 2 * causal,
                                                                  knoise=0.05))
            codes = [I.quantize_fp8_blocks(t, fmt) for t in (q, k, v)]
            U.say(f"[gpu] rising fp8 {kind} {fmt} d={d} causal={causal}")
            o, lse = ea.fwd_fp8(*(torch.from_numpy(c).to(dev) for c, _ in codes),
                                *(torch.from_numpy(ds).to(dev) for _, ds in codes),
                                causal=causal, scale=d ** -0.5, fmt=fmt)
            torch.cuda.synchronize()
            qx, kx, vx = (oracle.decode_fp8_blocks(c, ds, fmt) for c, ds in codes)
            ro, rl = oracle.attention(qx, kx, vx, causal, d ** -0.5)
            st = U.compare(o.double().cpu().numpy(), lse.double().cpu().numpy(), ro, rl, "fp8")
            assert st["pass"], (kind, fmt, d, causal, st)


def test_deterministic(oracle):
    w = I.random_workload(2, 4, 777, 777, 128, "bf16", True, seed=77)
    x = I.make_inputs(w)
    U.say(f"[gpu] determinism {w.name}")
    o1, l1 = U.run_gpu(x)
    o2, l2 = U.run_gpu(x)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("name", sorted(I.WORKLOADS))
def test_workload_full(oracle, name):
    """Every full-size workload in the benchmark's launch configuration, every element of O and LSE
    against the oracle (the fp64 oracle takes a few seconds per workload on the host's cores)."""
    w = I.WORKLOADS[name]
    x = I.make_inputs(w)
    U.say(f"[gpu] full {name}")
    o, lse = U.run_gpu(x)
    og, lg = o.double().cpu().numpy(), lse.double().cpu().numpy()
    del o, lse
    q, k, v = U.oracle_inputs(x, oracle)
    ro, rl = oracle.attention(q, k, v, w.causal, w.scale)
    st = U.compare(og, lg, ro, rl, w.dtype)
    U.say(f"   {name}: {st}")
    assert st["pass"], st


@pytest.mark.parametrize("name", ["fp8_b2_h16_s4096_d128", "e5m2_b2_h16_s4096_d128"])
def test_fp8_quantisation_error_report(oracle, name):
    """Reported, not gated: the fp8 path against attention on the unquantised fp32 draws (the
    error that block quantisation itself adds), on sampled rows of the full-size workload."""
    w = I.WORKLOADS[name]
    x = I.make_inputs(w)
    U.say(f"[gpu] quantisation error report {name}")
    o, lse = U.run_gpu(x)
    o = o.view(w.B * w.H, w.S_q, w.d)
    lse = lse.view(w.B * w.H, w.S_q)
    rows = U.sample_rows(w, n_random=100, seed=w.seed + 100)
    og = o[rows[:, 0], rows[:, 1]].double().cpu().numpy()
    lg = lse[rows[:, 0], rows[:, 1]].double().cpu().numpy()
    ro, rl = oracle.attention_rows(x.q32.astype(np.float64), x.k32.astype(np.float64), x.v32.astype(np.float64),
                                   w.causal, w.scale, rows)
    err_o, err_l = np.abs(og - ro), np.abs(lg - rl)
    U.say(f"   vs unquantised fp32 inputs: max|dO| {err_o.max():.3e} rms {np.sqrt((err_o ** 2).mean()):.3e}, "
          f"max|dLSE| {err_l.max():.3e}")
    assert np.all(np.isfinite(og)) and np.all(np.isfinite(lg))


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("causal", [False, True])
def test_fp8_unit_descales(oracle, fmt, causal):
    """fp8 codes through attn_fwd (unit descales) equal fwd_fp8 with all-one descales, bit for bit,
    and match the oracle on the decoded codes."""
    import exact_attention_32_amd as ea

    dev = "cuda:0"
    B, H, S, d = 1, 2, 333, 128
    U.say(f"[gpu] fp8 unit descales {fmt} causal={causal}")
    q, k, v, _ = I.make_device_inputs(B, H, S, d, "fp8" if fmt == "e4m3" else "e5m2", seed=21 + causal)
    tdt = torch.float8_e4m3fn if fmt == "e4m3" else torch.float8_e5m2
    o1, l1 = ea.fwd(q.view(tdt), k.view(tdt), v.view(tdt), causal=causal)
    ones = torch.ones((B, H, (S + 127) // 128), dtype=torch.float32, device=dev)
    o2, l2 = ea.fwd_fp8(q, k, v, ones, ones, ones, causal=causal, fmt=fmt)
    torch.cuda.synchronize()
    assert o1.dtype == torch.bfloat16 and torch.equal(o1, o2) and torch.equal(l1, l2)
    dec = [oracle.decode_fp8_blocks(t.cpu().numpy(), ones.cpu().numpy(), fmt) for t in (q, k, v)]
    ro, rl = oracle.attention(*dec, causal, d ** -0.5)
    st = U.compare(o1.double().cpu().numpy(), l1.double().cpu().numpy(), ro, rl, "fp8")
    U.say(f"   {st}")
    assert st["pass"], st


def test_empty_queries(oracle):
    """No query rows (B, H or S_q = 0): empty O and LSE, nothing launched; keys without queries are
    fine, queries without keys are an error.  The sizes around the empty call stay correct."""
    import exact_attention_32_amd as ea

    dev = "cuda:0"
    U.say("[gpu] empty inputs")
    for B, H, S_q, S_k in ((1, 2, 0, 64), (0, 2, 16, 16), (1, 0, 16, 16), (1, 2, 0, 0)):
        for dt in (torch.bfloat16, torch.float16):
            q = torch.zeros(B, H, S_q, 128, dtype=dt, device=dev)
            k = torch.zeros(B, H, S_k, 128, dtype=dt, device=dev)
            o, lse = ea.fwd(q, k, k, causal=True)
            assert o.shape == (B, H, S_q, 128) and lse.shape == (B, H, S_q)
        q8 = torch.zeros(B, H, S_q, 64, dtype=torch.uint8, device=dev)
        k8 = torch.zeros(B, H, S_k, 64, dtype=torch.uint8, device=dev)
        ds = [torch.ones(B, H, (s + 127) // 128, device=dev) for s in (S_q, S_k, S_k)]
        for fmt in ("e4m3", "e5m2"):
            o, lse = ea.fwd_fp8(q8, k8, k8, *ds, fmt=fmt)
            assert o.shape == (B, H, S_q, 64) and o.dtype == torch.bfloat16
    with pytest.raises(ea.AttnError):
        ea.fwd(torch.zeros(1, 1, 4, 64, dtype=torch.bfloat16, device=dev),
               torch.zeros(1, 1, 0, 64, dtype=torch.bfloat16, device=dev),
               torch.zeros(1, 1, 0, 64, dtype=torch.bfloat16, device=dev))
    # a normal call right after still matches the oracle
    st = _run_full(oracle, I.random_workload(1, 2, 70, 90, 64, "bf16", True, seed=8))
    assert st["pass"], st


@pytest.mark.parametrize("dtype", ["bf16", "fp8", "qnorm"])
def test_graph_replay_equals_eager(oracle, dtype):
    """The attention launch captured in a HIP graph (the library allocates nothing and records no
    memset): three replays, with eager work and synchronisations between them, each bit-equal to
    the eager result.  'qnorm': the split QK-RMSNorm and the attention with the Q fold, two
    launches in one graph."""
    import exact_attention_32_amd as ea

    dev = "cuda:0"
    U.say(f"[gpu] graph replay {dtype}")
    w = I.random_workload(1, 4, 700, 900, 128, "bf16" if dtype == "qnorm" else dtype, True, seed=31)
    x = I.make_inputs(w)
    q, k, v = x.q.to(dev), x.k.to(dev), x.v.to(dev)
    o = torch.empty((w.B, w.H, w.S_q, w.d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.B, w.H, w.S_q), dtype=torch.float32, device=dev)
    scratch = []   # intermediate tensors the graph must rewrite on every replay
    if dtype == "fp8":
        qd, kd, vd = x.q_descale.to(dev), x.k_descale.to(dev), x.v_descale.to(dev)

        def run():
            ea.fwd_fp8(q, k, v, qd, kd, vd, causal=True, scale=w.scale, out=o, lse=lse)
    elif dtype == "qnorm":
        g = torch.Generator().manual_seed(32)
        wq = (torch.rand(w.H * w.d, generator=g) + 0.5).to(torch.bfloat16).to(dev)
        wk = (torch.rand(w.H * w.d, generator=g) + 0.5).to(torch.bfloat16).to(dev)
        r = torch.empty((w.B, w.S_q), dtype=torch.float32, device=dev)
        kn = torch.empty_like(k)
        scratch = [r, kn]

        def run():
            ea.qk_rmsnorm_split(q, k, wk, q_rstd=r, k_out=kn)
            ea.fwd_qnorm(q, kn, v, r, wq, causal=True, scale=w.scale, out=o, lse=lse)
    else:
        def run():
            ea.fwd(q, k, v, causal=True, scale=w.scale, out=o, lse=lse)
    run()
    torch.cuda.synchronize()
    o_ref, l_ref = o.clone(), lse.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run()   # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    for rep in range(3):
        o.fill_(7.0)
        lse.fill_(7.0)
        for t in scratch:
            t.fill_(7.0)
        junk = torch.randn(1024, 1024, device=dev) @ torch.randn(1024, 1024, device=dev)   # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(lse, l_ref), f"replay {rep} differs from the eager result"
        del junk


def _fp8_range_inputs(kind, S, d, seed):
    """fp32 Q, K, V [1, 1, S, d] whose fp8 probabilities or V descales reach the ends of their range:
    'sink0' / 'sinkmid': key 0 (or key S/2) eleven binades above S-1 keys of nearly equal score, V
    N(0,1); 'sink_vsmall': the same sink at key 0 with the other V blocks scaled by 2^-10..2^-8 (V
    descales spread over ten binades, the largest first); 'vspread0' / 'vspreadmid': V blocks scaled
    by 2^-10..2^10 (the largest first, or in the middle), N(0,1) queries and keys."""
    rng = np.random.Generator(np.random.PCG64(seed))
    scale = d ** -0.5
    nb = (S + 127) // 128
    u = np.ones(d) / np.sqrt(d)
    if kind.startswith("sink"):
        q = np.tile(4.0 * u, (S, 1))
        k = 1e-3 * rng.standard_normal((S, d))
        j = S // 2 + 5 if kind == "sinkmid" else 0
        k[j] += u * (11.0 / (scale * 4.0 * np.log2(np.e)))
        v = rng.standard_normal((S, d))
        if kind == "sink_vsmall":
            for b in range(1, nb):
                v[128 * b:128 * (b + 1)] *= 2.0 ** rng.uniform(-10.0, -8.0)
    else:
        q = rng.standard_normal((S, d))
        k = rng.standard_normal((S, d))
        v = rng.standard_normal((S, d))
        ex = rng.uniform(-10.0, 10.0, nb)
        ex[0 if kind == "vspread0" else nb // 2] = 10.0
        for b in range(nb):
            v[128 * b:128 * (b + 1)] *= 2.0 ** ex[b]
    return tuple(a.astype(np.float32)[None, None] for a in (q, k, v))


@pytest.mark.parametrize("kind", ["sink0", "sinkmid", "sink_vsmall", "vspread0", "vspreadmid"])
@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_fp8_range(oracle, kind, fmt):
    """The fp8 path where its probabilities span many binades (an attention sink over 4K flat keys)
    and where V's block descales differ by up to 2^20.  The sink cases keep V at N(0,1) and are gated
    at 5e-2.  Where V itself reaches 2^10 in magnitude, an E4M3 probability's own rounding (up to
    2^-4 of its value) moves O by far more than 5e-2 in absolute terms, so those cases are gated at
    5e-2 relative to the largest |O|; the descale must not shift the probabilities out of E4M3's
    range either way."""
    import exact_attention_32_amd as ea

    dev = "cuda:0"
    S = 4200
    for d in (64, 128):
        for causal in (False, True):
            q, k, v = _fp8_range_inputs(kind, S, d, seed=d + 3 * causal)
            codes = [I.quantize_fp8_blocks(t, fmt) for t in (q, k, v)]
            U.say(f"[gpu] fp8 range {kind} {fmt} d={d} causal={causal}")
            o, lse = ea.fwd_fp8(*(torch.from_numpy(c).to(dev) for c, _ in codes),
                                *(torch.from_numpy(ds).to(dev) for _, ds in codes),
                                causal=causal, scale=d ** -0.5, fmt=fmt)
            torch.cuda.synchronize()
            qx, kx, vx = (oracle.decode_fp8_blocks(c, ds, fmt) for c, ds in codes)
            ro, rl = oracle.attention(qx, kx, vx, causal, d ** -0.5)
            og, lg = o.double().cpu().numpy(), lse.double().cpu().numpy()
            err_o, err_l = float(np.abs(og - ro).max()), float(np.abs(lg - rl).max())
            gate = 5e-2 * (max(1.0, float(np.abs(ro).max())) if kind.startswith("vspread") else 1.0)
            U.say(f"   max|dO| {err_o:.3e} (gate {gate:.3e}, max|O| {np.abs(ro).max():.3e}), max|dLSE| {err_l:.3e}")
            assert np.all(np.isfinite(og)) and err_o <= gate and err_l <= U.TOL_LSE, (kind, fmt, d, causal)


def test_binding_rejects_bad_outputs(oracle):
    """fwd / fwd_fp8 / quantize_fp8 refuse outputs of the wrong size, type, device or layout (before
    any launch), and the same call with correct outputs then runs."""
    import exact_attention_32_amd as ea

    dev = "cuda:0"
    U.say("[gpu] binding output checks")
    q = torch.randn(1, 2, 70, 64, device=dev).to(torch.bfloat16)
    for out, lse in ((torch.empty(1, 2, 69, 64, dtype=torch.bfloat16, device=dev), None),
                     (torch.empty(1, 2, 70, 64, dtype=torch.float16, device=dev), None),
                     (torch.empty(1, 2, 70, 64, dtype=torch.bfloat16), None),
                     (None, torch.empty(1, 2, 69, dtype=torch.float32, device=dev)),
                     (None, torch.empty(1, 2, 70, dtype=torch.float32))):
        with pytest.raises(ValueError):
            ea.fwd(q, q, q, out=out, lse=lse)
    c = torch.zeros(1, 2, 70, 64, dtype=torch.uint8, device=dev)
    ds = torch.ones(1, 2, 1, device=dev)
    with pytest.raises(ValueError):
        ea.fwd_fp8(c, c, c, ds, ds, ds.cpu())
    with pytest.raises(ValueError):
        ea.fwd_fp8(c, c, c, ds, ds, ds, out=torch.empty(1, 2, 70, 64, dtype=torch.float16, device=dev))
    with pytest.raises(ValueError):
        ea.quantize_fp8(q.float(), codes=torch.empty(1, 2, 70, 64, dtype=torch.uint8))
    o, lse = ea.fwd(q, q, q, out=torch.empty(1, 2, 70, 64, dtype=torch.bfloat16, device=dev))
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
