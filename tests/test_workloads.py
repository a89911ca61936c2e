"""The seeded input generators: shapes, dtypes, determinism, injected ties."""
import numpy as np

import workloads as wl


def test_c0_shape_and_mix():
    w = wl.c0()
    assert w.logits.shape == (4, 1024) and w.logits.dtype == np.float32 and w.dtype == "f32"
    assert list(w.temperature) == [0.0, 0.0, np.float32(0.7), np.float32(0.7)]
    assert list(w.top_k[2:]) == [50, 50] and np.allclose(w.top_p[2:], 0.9)
    assert w.pool.shape == (4, 64) and w.pool.dtype == np.int32
    assert np.all((w.cols >= 1) & (w.cols < 64))
    assert np.array_equal(wl.c0().logits, w.logits)


def test_c0_permuted_moves_greedy_rows():
    w = wl.c0_permuted()
    assert list(np.flatnonzero(w.temperature == 0)) == [1, 3]


def test_c1_ties_and_greedy():
    w = wl.c1()
    assert w.temperature is None and w.logits.shape == (64, 32000)
    for b, i_star, j in w.meta["ties"]:
        hits = np.flatnonzero(w.logits[b] == w.logits[b].max())
        assert sorted(hits.tolist()) == sorted([i_star, j])
    assert any(j < i_star for _, i_star, j in w.meta["ties"])
    # spikes: every row's max is well above the N(0,2) bulk
    assert np.all(w.logits.max(axis=1) > 6.0)


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.00390625, 1.005859375, 1.0078125 + 2 ** -9, -2.5, 0.0, -0.0],
                 dtype=np.float32)
    h = wl.to_bf16_bits(x)
    back = wl.bf16_bits_to_f32(h)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: rounds to the even mantissa (1.0)
    assert back[0] == 1.0 and back[1] == 1.0
    assert back[2] == np.float32(1.0078125)
    assert back[4] == -2.5 and h[6] == 0x8000


def test_tiny_generator_covers_edge_parameters():
    w = wl.tiny(np.random.default_rng(0), 64, 300)
    assert w.logits.shape == (64, 300)
    assert np.any(w.temperature == 0) and np.any(w.top_k >= 300) and np.any(w.top_k < 1)
    assert np.any(w.top_p >= 1) and np.any(w.top_p < 1e-6)
    assert np.any(w.cols == -1)
