"""Host logic of the attention-stack schedule (no GPU): the layer plan and
the chunking of a prompt."""
import pytest

import oracle.attention as A
from global_gqa_amd.schedule import chunk_bounds, plan_layers


def test_plan_27b_stack():
    """62 layers: 10 global (every sixth, from layer 5) and 52 local; local
    layers keep a 1024-slot ring with base 10k, global layers a full cache
    with base 1M and the interpolation scale (Gemma 3 Technical Report,
    section 2; 27B module print: 62 decoder layers)."""
    plans = plan_layers(62, 131072, 1024, 8.0)
    kinds = [p.kind for p in plans]
    assert kinds.count(A.GLOBAL) == 10 and kinds.count(A.LOCAL) == 52
    assert [p.index for p in plans if p.kind == A.GLOBAL] == list(range(5, 62, 6))
    assert all(A.layer_kind(p.index) == p.kind for p in plans)
    for p in plans:
        if p.kind == A.LOCAL:
            assert (p.capacity, p.is_ring, p.rope_base, p.interp_scale) == (1024, True, 1e4, 1.0)
        else:
            assert (p.capacity, p.is_ring, p.rope_base, p.interp_scale) == (131072, False, 1e6, 8.0)


def test_plan_short_context():
    """The ring keeps its window length even when the context is shorter
    (the library rejects a ring shorter than the window); the global cache
    is the context length."""
    plans = plan_layers(6, 500)
    assert plans[0].capacity == 1024 and plans[5].capacity == 500


def test_plan_rejects_bad_sizes():
    for args in [(0, 10), (6, 0)]:
        with pytest.raises(ValueError):
            plan_layers(*args)


def test_chunk_bounds():
    assert chunk_bounds(10, 4) == [(0, 4), (4, 8), (8, 10)]
    assert chunk_bounds(8, 4) == [(0, 4), (4, 8)]
    assert chunk_bounds(131072, 4096)[-1] == (126976, 131072)
    with pytest.raises(ValueError):
        chunk_bounds(10, 0)
