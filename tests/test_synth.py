"""The seeded generator: determinism, bf16 rounding, the planted-peak recipe."""
import numpy as np
import pytest

import domino_synth as ds


def test_bf16_round_to_nearest_even():
    # 1 + 2^-8 is halfway between bf16 neighbours 1 and 1 + 2^-7: ties go to even (1.0)
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 65280.0, 1e-40, np.inf, -0.0], np.float32)
    b = ds.round_to_bf16_bits(x)
    back = ds.bf16_bits_to_f32(b)
    assert back[0] == 1.0 and back[1] == 1.0 and back[2] == 1.0 + 2 ** -6
    assert back[3] == -2.5 and back[4] == 65280.0 and back[6] == np.inf
    assert b[7] == 0x8000
    # brute force over random floats: the result is one of the two neighbours and the nearest
    rng = np.random.default_rng(0)
    f = rng.standard_normal(100000).astype(np.float32)
    g = ds.bf16_bits_to_f32(ds.round_to_bf16_bits(f)).astype(np.float64)
    lo = (f.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32).astype(np.float64)
    step = np.abs(ds.bf16_bits_to_f32(ds.round_to_bf16_bits(lo.astype(np.float32)) + 1).astype(np.float64) - lo)
    assert np.all(np.abs(g - f) <= step / 2 + 1e-30)


def test_generation_is_deterministic_and_row_local():
    sh = ds.HeadShape(d=64, h=32, r=16, V=5000, K=16, wdtype="bf16")
    w1 = ds.make_weights(sh, (7, 0))
    w2 = ds.make_weights(sh, (7, 0))
    assert ds.digest(*w1.arrays().values()) == ds.digest(*w2.arrays().values())
    a = ds.make_inputs(sh, 5, (7, 1))
    b = ds.make_inputs(sh, [3, 1], (7, 1))
    np.testing.assert_array_equal(a.L_base[[3, 1]], b.L_base)
    np.testing.assert_array_equal(a.H[[3, 1]], b.H)
    np.testing.assert_array_equal(a.last_tok[[3, 1]], b.last_tok)


def test_chunked_weights_do_not_depend_on_thread_count(monkeypatch):
    sh = ds.HeadShape(d=16, h=8, r=8, V=3 * ds.CHUNK_ROWS + 5, K=16, wdtype="bf16")
    a = ds.make_weights(sh, (7, 2))
    monkeypatch.setattr(ds, "_threads", lambda: 1)
    b = ds.make_weights(sh, (7, 2))
    assert ds.digest(a.W2, a.E) == ds.digest(b.W2, b.E)


def test_planted_peak_sits_above_noise_max():
    sh = ds.HeadShape(d=16, h=8, r=8, V=20000, K=16, wdtype="bf16")
    inp = ds.make_inputs(sh, 3, (7, 3), sigma=3.0, peak="zipf")
    for b in range(3):
        for i in range(16):
            row = inp.L_base[b, i]
            v = inp.peak_ids[b, i]
            others = np.delete(row, v)
            assert row[v] == np.float32(others.max() + np.float32(6.0)) or row[v] >= others.max() + 5.999
            assert np.argmax(row) == v
    # Zipf ranks favour small ids
    big = ds.make_inputs(sh, 40, (7, 4), sigma=3.0, peak="zipf")
    assert np.median(big.peak_ids) < 1000


def test_temperature_and_ranges():
    sh = ds.HeadShape(d=16, h=8, r=8, V=1000, K=16, wdtype="f32")
    inp = ds.make_inputs(sh, 20, (7, 5), temperature=(1.0, 4.0))
    assert np.all((inp.temperature >= 1.0) & (inp.temperature <= 4.0))
    assert np.all((inp.last_tok >= 0) & (inp.last_tok < sh.V))


def test_named_workloads_have_page_shapes():
    for name, wl in ds.WORKLOADS.items():
        if name == "tiny":
            assert (wl.shape.V, wl.shape.d, wl.shape.h, wl.shape.r, wl.shape.wdtype) == (1024, 256, 64, 16, "f32")
        else:
            assert (wl.shape.h, wl.shape.r, wl.shape.V, wl.shape.K) == (1024, 256, 151936, 16)
    assert ds.WORKLOADS["qwen3_8b_b256"].B == 256 and ds.WORKLOADS["qwen3_8b_b32"].B == 32


def test_geometric_targets_construction():
    rng = np.random.default_rng(2)
    draft = rng.integers(0, 50, size=(500, 16)).astype(np.int32)
    tgt, k = ds.geometric_prefix_targets(draft, (4, 3), 50)
    for b in range(500):
        assert np.array_equal(tgt[b, :k[b]], draft[b, :k[b]])
        if k[b] < 16:
            assert tgt[b, k[b]] != draft[b, k[b]]
    assert 5.0 < k.mean() < 8.0  # mean 7 before truncation at 16
