"""The seeded input recipe: reproducibility, the E4M3 encoder, block descales, outliers."""
import numpy as np
import pytest
import torch

from exact_attention_32_amd import inputs as I


def test_seeded_reproducible():
    w = I.random_workload(1, 2, 33, 40, 64, "bf16", False, seed=7)
    a, b = I.make_inputs(w), I.make_inputs(w)
    for x, y in ((a.q, b.q), (a.k, b.k), (a.v, b.v)):
        assert torch.equal(x, y)
    c = I.make_inputs(I.random_workload(1, 2, 33, 40, 64, "bf16", False, seed=8))
    assert not torch.equal(a.q, c.q)


def test_bf16_cast_is_rne_of_fp32_draws():
    w = I.random_workload(1, 1, 16, 16, 64, "bf16", False, seed=3)
    x = I.make_inputs(w)
    rng = np.random.Generator(np.random.PCG64(3))
    q32 = rng.standard_normal((1, 1, 16, 64), dtype=np.float32)
    assert torch.equal(x.q, torch.from_numpy(q32).to(torch.bfloat16))


def test_e4m3_encoder_matches_torch_cast_in_range():
    rng = np.random.Generator(np.random.PCG64(11))
    x = np.concatenate([
        rng.standard_normal(200000).astype(np.float32) * 50,
        rng.uniform(-448, 448, 100000).astype(np.float32),
        (rng.standard_normal(100000) * 2.0 ** -8).astype(np.float32),   # subnormal range
        np.array([0.0, -0.0, 448.0, -448.0, 2.0 ** -6, 2.0 ** -9, 2.0 ** -10, 1.5 * 2.0 ** -10, 464.0 - 1e-3],
                 np.float32),
    ])
    x = np.clip(x, -448, 448)
    mine = I.e4m3_encode(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(mine, ref)


def test_e4m3_encoder_saturates():
    codes = I.e4m3_encode(np.array([448.0, 449.0, 470.0, 1e6, -1e6]))
    assert list(codes) == [0x7E, 0x7E, 0x7E, 0x7E, 0xFE]


def test_block_quantisation():
    w = I.random_workload(2, 3, 300, 300, 128, "fp8", False, seed=5)
    x = I.make_inputs(w)
    assert x.q_descale.shape == (2, 3, 3)
    tab = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for t32, codes, desc in ((x.q32, x.q, x.q_descale), (x.v32, x.v, x.v_descale)):
        for j in range(3):
            blk = t32[:, :, j * 128:(j + 1) * 128]
            amax = np.abs(blk).max(axis=(2, 3))
            assert np.array_equal(desc[:, :, j].numpy(), (amax / np.float32(448)).astype(np.float32))
            cb = codes[:, :, j * 128:(j + 1) * 128].numpy()
            # the block's largest magnitude lands on +-448 (code 0x7e / 0xfe)
            assert np.all(np.abs(tab[cb]).max(axis=(2, 3)) == 448.0)
        # decoded values are within half an E4M3 step of the fp32 draws
        dec = tab[codes.numpy()] * np.repeat(desc.numpy().astype(np.float64), 128, axis=2)[:, :, :300, None]
        rel = np.abs(dec - t32) / np.maximum(np.abs(t32), 2.0 ** -6 * np.repeat(desc.numpy(), 128, axis=2)[:, :, :300, None])
        assert rel.max() <= 2.0 ** -4 + 1e-6


def test_outliers_exactly_one_percent():
    w = I.random_workload(1, 2, 64, 64, 64, "bf16", True, seed=9, outliers=True)
    rng = np.random.Generator(np.random.PCG64(9))
    q = rng.standard_normal((1, 2, 64, 64), dtype=np.float32)
    x = I.make_inputs(w)
    ratio = x.q.float().numpy() / torch.from_numpy(q).to(torch.bfloat16).float().numpy()
    n_big = int(np.sum(np.abs(ratio) > 5))
    assert n_big == int(0.01 * q.size)


@pytest.mark.parametrize("name", sorted(I.WORKLOADS))
def test_workload_accounting(name):
    w = I.WORKLOADS[name]
    n = w.S_q * (w.S_q + 1) // 2 if w.causal else w.S_q * w.S_k
    assert w.flops() == 4 * w.d * n * w.B * w.H


def test_e5m2_encoder_matches_torch_cast_in_range():
    rng = np.random.Generator(np.random.PCG64(12))
    x = np.concatenate([
        rng.standard_normal(200000).astype(np.float32) * 3000,
        rng.uniform(-57344, 57344, 100000).astype(np.float32),
        np.exp2(rng.uniform(-20, 15.8, 100000)).astype(np.float32),
    ])
    x = x[np.abs(x) <= 57344]
    ref = torch.from_numpy(x).to(torch.float8_e5m2).view(torch.uint8).numpy()
    assert np.array_equal(I.e5m2_encode(x), ref)


def test_e5m2_encoder_saturates():
    big = np.array([57344.0, 57345.0, 61439.0, 61440.0, 1e9])
    assert np.all(I.e5m2_encode(big) == 0x7B) and np.all(I.e5m2_encode(-big) == 0xFB)


def test_e5m2_block_quantisation():
    w = I.random_workload(1, 2, 260, 260, 64, "e5m2", False, seed=6)
    x = I.make_inputs(w)
    tab = torch.arange(256, dtype=torch.uint8).view(torch.float8_e5m2).to(torch.float64).numpy()
    for codes, ds, raw in ((x.q, x.q_descale, x.q32), (x.k, x.k_descale, x.k32)):
        assert ds.shape == (1, 2, 3)
        dec = tab[codes.numpy()] * np.repeat(ds.numpy().astype(np.float64), 128, axis=2)[:, :, :260, None]
        # 2 mantissa bits: relative error at most 2^-3 for normal codes
        assert np.all(np.abs(dec - raw) <= np.abs(raw) * 2.0 ** -3 + 2.0 ** -16 * ds.numpy().max())
        amax = np.abs(raw[:, :, :128]).max(axis=(2, 3)).astype(np.float32)
        assert np.array_equal(ds.numpy()[:, :, 0], amax / np.float32(57344.0))
