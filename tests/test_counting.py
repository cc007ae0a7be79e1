"""The in-window pair counter used for TFLOP/s equals brute-force counting
of the oracle's visibility matrix, and reproduces the workloads' totals."""
import numpy as np
import pytest

import oracle.attention as A
import workloads as W
from global_gqa_amd import counting as C


@pytest.mark.parametrize("S,window,spans,p0", [
    (50, 7, [], 0), (64, 64, [(3, 20)], 0), (100, 10, [(5, 9), (40, 80)], 0), (77, 1, [(10, 30)], 1000),
    (200, 30, [(0, 200)], 0)])
def test_pairs_equal_visibility_count(S, window, spans, p0):
    pos = p0 + np.arange(S)
    for kind in (A.LOCAL, A.GLOBAL):
        vis = A.visibility(pos, pos, kind, window, spans)
        got = C.prefill_pairs(1, S, kind == A.LOCAL, window, pos0=[p0], spans=[spans])
        assert got == int(vis.sum())


def test_chunked_pairs_equal_visibility_count():
    p0, C_, cap, W_ = 300, 90, 64, 50
    qpos = p0 + np.arange(C_)
    for (kind, ring) in ((A.GLOBAL, None), (A.LOCAL, cap)):
        kmin = max(0, p0 - cap) if ring else 0
        kpos = np.arange(kmin, p0 + C_)
        vis = A.visibility(qpos, kpos, kind, W_)
        got = C.prefill_pairs(1, C_, kind == A.LOCAL, W_, pos0=[p0], has_cache=True, ring_capacity=ring)
        assert got == int(vis.sum())


def test_workload_totals():
    w = W.WORKLOADS[2]
    loc = C.prefill_flops(1, w.S, w.Hq, w.D, True, W.WINDOW)
    glo = C.prefill_flops(1, w.S, w.Hq, w.D, False, W.WINDOW)
    assert round(loc / 1e11, 4) == 1.2886 and round(glo / 1e11, 4) == 5.4982
    assert abs((5 * loc + glo) / 1.1941e12 - 1) < 1e-4
    w4 = W.WORKLOADS[4]
    g4 = C.prefill_pairs(1, w4.S, False, W.WINDOW, pos0=[w4.pos0], has_cache=True)
    assert g4 == 528_484_352
    l4 = C.prefill_flops(1, w4.S, w4.Hq, w4.D, True, W.WINDOW, pos0=[w4.pos0], has_cache=True, ring_capacity=1024)
    assert abs(l4 / 6.872e10 - 1) < 1e-3
    w3 = W.WORKLOADS[3]
    pos = [w3.pos0] * w3.B
    glob = C.decode_bytes(w3.B, w3.Hq, w3.Hkv, w3.D, pos, False, W.WINDOW)
    loc = C.decode_bytes(w3.B, w3.Hq, w3.Hkv, w3.D, pos, True, W.WINDOW)
    assert abs((glob + 5 * loc) / 9.9324e9 - 1) < 2e-3
