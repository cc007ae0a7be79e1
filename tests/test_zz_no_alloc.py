"""g3attn_decode_noalloc (the decode entry point for callers that cannot
allocate: its split-K partials live in the library's static per-GPU array)
gives what g3attn_decode gives with a caller workspace, through the C ABI,
on two calls in a row (the second smaller, so it reads an array that still
holds the first call's partials), and both match the oracle."""
import ctypes

import numpy as np
import pytest

import oracle.attention as A
import workloads as W
from tests.gpu_util import assert_parity, assert_rowwise_bf16, dev_bf16, dev_f32, host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import global_gqa_amd as G  # noqa: E402

CONFIG = 12  # seed namespace of this test's inputs


def _case(layer, B, Hq, Hkv, D, cap, is_ring, positions, kind, base, scale):
    sd = lambda t: W.seed_of(CONFIG, layer, t)  # noqa: E731
    ck = W.host_normal_bf16((B, Hkv, cap, D), sd(W.T_CK))
    cv = W.host_normal_bf16((B, Hkv, cap, D), sd(W.T_CV))
    q = W.host_normal_bf16((B, Hq, D), sd(W.T_Q))
    kn = W.host_normal_bf16((B, Hkv, D), sd(W.T_K))
    vn = W.host_normal_bf16((B, Hkv, D), sd(W.T_V))
    gq, gk = W.host_gamma(D, sd(W.T_GQ)), W.host_gamma(D, sd(W.T_GK))
    pos = np.array(positions, dtype=np.int32)
    maxp = int(pos.max())
    outs, caches = [], []
    for noalloc in (False, True):
        cache = G.KVCache(dev_bf16(ck), dev_bf16(cv), is_ring)
        args = (dev_bf16(q), dev_bf16(kn), dev_bf16(vn), torch.from_numpy(pos).cuda(), maxp, cache, kind, W.WINDOW,
                base, scale, dev_f32(gq), dev_f32(gk), W.EPS)
        torch.cuda.synchronize()
        print(f"decode{'_noalloc' if noalloc else ''} B={B} Hq={Hq} Hkv={Hkv} D={D} cap={cap} ring={is_ring}",
              flush=True)
        o = G.decode_noalloc(*args) if noalloc else G.decode(*args)
        torch.cuda.synchronize()
        outs.append(host(o))
        caches.append((host(cache.k), host(cache.v)))
    assert np.array_equal(outs[0], outs[1]), "noalloc decode differs from decode with a workspace"
    assert np.array_equal(caches[0][0], caches[1][0]) and np.array_equal(caches[0][1], caches[1][1])
    ref, rck, rcv = A.decode(q, kn, vn, ck, cv, is_ring, pos, kind, W.WINDOW, base, scale, gq, gk, W.EPS)
    assert_parity(outs[1], ref, "noalloc decode")
    assert np.array_equal(caches[1][1], rcv)
    assert_rowwise_bf16(caches[1][0], rck, "noalloc decode cache k")
    return int(G.lib().g3attn_decode_workspace_size(B, Hq, Hkv, D, maxp, ctypes.byref(G.KVCacheC(0, 0, cap, is_ring))))


def test_noalloc_decode_matches_workspace_decode_twice():
    # first: a global layer over a long linear cache (157 splits of 256 slots, merged by the second kernel)
    big = _case(0, B=3, Hq=8, Hkv=4, D=128, cap=40000, is_ring=False, positions=[1023, 30000, 39999],
                kind=A.GLOBAL, base=1e6, scale=8.0)
    # second, smaller: a 1B-shaped local layer on a ring (fewer partials than the array still holds)
    small = _case(1, B=2, Hq=4, Hkv=1, D=256, cap=1024, is_ring=True, positions=[5, 2000], kind=A.LOCAL,
                  base=1e4, scale=1.0)
    assert 0 < small < big <= G.DECODE_NOALLOC_MAX_BYTES, (small, big)
