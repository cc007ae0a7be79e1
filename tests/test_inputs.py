"""The seeded input recipe: determinism, bf16 rounding and span placement."""
import numpy as np

import workloads as W


def test_seeded_generation_is_deterministic():
    a = W.host_normal_bf16((3, 5, 7), W.seed_of(2, 1, W.T_Q))
    b = W.host_normal_bf16((3, 5, 7), W.seed_of(2, 1, W.T_Q))
    c = W.host_normal_bf16((3, 5, 7), W.seed_of(2, 1, W.T_K))
    assert np.array_equal(a, b) and not np.array_equal(a, c)
    assert W.seed_of(3, 5, W.T_CV) == 3056


def test_bf16_round_is_rne():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 1.0 + 2 ** -9, 3.0e38], dtype=np.float32)
    r = W.bf16_round(x)
    assert r.tolist()[:5] == [1.0, 1.0, 1.0 + 4 * 2 ** -8, -2.5, 1.0]
    u = r.view(np.uint32)
    assert np.all(u & 0xFFFF == 0)
    big = W.host_normal_bf16((10000,), 1)
    assert np.all(big.view(np.uint32) & 0xFFFF == 0)
    assert abs(big.std() - 1.0) < 0.03


def test_gamma_recipe():
    g = W.host_gamma(128, 3)
    assert g.dtype == np.float32 and abs(g.mean() - 1.0) < 0.05 and 0.05 < g.std() < 0.15


def test_image_spans_non_overlapping_and_unaligned():
    w = W.WORKLOADS[5]
    spans = W.workload_spans(w)
    assert len(spans) == w.B and len(spans[0]) == 4
    assert 0 <= len(spans[1]) <= 4
    for sp in spans:
        last = -1
        for (s, e) in sp:
            assert e - s == W.IMAGE_TOKENS and s >= last and 0 <= s and e <= w.S
            last = e
    starts = [s for sp in spans for (s, _) in sp]
    assert any(s % 64 for s in starts)
    for seed in range(50):
        sp = W.image_spans(1000, 3, seed)
        assert all(sp[i][1] <= sp[i + 1][0] for i in range(2)) and sp[-1][1] <= 1000
