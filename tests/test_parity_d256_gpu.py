"""GPU parity at head dimension 256 (the Gemma 3 1B attention shape: 4 query
heads sharing 1 kv head, "Gemma explained: What's new in Gemma 3", 1B module
print): the prologue, self-contained and chunked prefill, and decode through
the C ABI against the fp64 oracle, plus every GQA group size, the mask
shapes and the online-maximum fallback."""
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

D = 256
CONFIG = 8  # seed namespace of this file's inputs


def _inputs(layer, B, S, Hq, Hkv):
    q = W.host_normal_bf16((B, S, Hq, D), W.seed_of(CONFIG, layer, W.T_Q))
    k = W.host_normal_bf16((B, S, Hkv, D), W.seed_of(CONFIG, layer, W.T_K))
    v = W.host_normal_bf16((B, S, Hkv, D), W.seed_of(CONFIG, layer, W.T_V))
    gq = W.host_gamma(D, W.seed_of(CONFIG, layer, W.T_GQ))
    gk = W.host_gamma(D, W.seed_of(CONFIG, layer, W.T_GK))
    return q, k, v, gq, gk


def _params(kind, scale_global=1.0):
    return (W.ROPE_BASE_LOCAL, 1.0) if kind == A.LOCAL else (W.ROPE_BASE_GLOBAL, scale_global)


def test_qknorm_rope_d256():
    T, Hq, Hkv = 300, 4, 1
    pos = np.concatenate([np.arange(150), np.random.default_rng(3).integers(0, 32768, T - 151), [32767]])
    pos = pos.astype(np.int32)
    q = W.host_normal_bf16((T, Hq, D), 1)
    k = W.host_normal_bf16((T, Hkv, D), 2)
    gq, gk = W.host_gamma(D, 3), W.host_gamma(D, 4)
    for base, scale in [(1e4, 1.0), (1e6, 8.0)]:
        qo, ko = G.qknorm_rope(dev_bf16(q), dev_bf16(k), torch.from_numpy(pos).cuda(), dev_f32(gq), dev_f32(gk),
                               W.EPS, base, scale)
        torch.cuda.synchronize()
        assert_rowwise_bf16(host(qo), A.qknorm_rope(q, gq, W.EPS, pos, base, scale), "q_hat")
        assert_rowwise_bf16(host(ko), A.qknorm_rope(k, gk, W.EPS, pos, base, scale), "k_hat")


def _prefill(q, k, v, gq, gk, kind, window, base, scale, spans=None, pos0=None, cache=None, sm=0.0):
    B = q.shape[0]
    flat = [(b, s, e) for b in range(B) for (s, e) in spans[b]] if spans else None
    o = G.prefill(dev_bf16(q), dev_bf16(k), dev_bf16(v), kind, window, base, scale,
                  None if gq is None else dev_f32(gq), None if gk is None else dev_f32(gk), W.EPS, sm, flat, pos0,
                  cache)
    torch.cuda.synchronize()
    return host(o)


@pytest.mark.parametrize("kind", [A.LOCAL, A.GLOBAL])
def test_prefill_1b_shape(kind):
    """1B heads (Hq=4, Hkv=1), S spanning many 32-key tiles and a ragged tail,
    the 1024-token window."""
    B, S, Hq, Hkv = 1, 1500, 4, 1
    q, k, v, gq, gk = _inputs(kind, B, S, Hq, Hkv)
    base, scale = _params(kind, 8.0)
    got = _prefill(q, k, v, gq, gk, kind, W.WINDOW, base, scale)
    ref = A.prefill(q, k, v, kind, W.WINDOW, base, scale, gq, gk, W.EPS)
    assert_parity(got, ref, f"D=256 kind={kind}")


@pytest.mark.parametrize("kind", [A.LOCAL, A.GLOBAL])
@pytest.mark.parametrize("Hq,Hkv", [(2, 2), (4, 2), (8, 1)])
def test_prefill_groups_spans_pos0(kind, Hq, Hkv):
    """Every other GQA group size, B = 2 with per-sequence first positions,
    unaligned image spans and a small window."""
    B, S = 2, 333
    q, k, v, gq, gk = _inputs(10 + Hq + Hkv, B, S, Hq, Hkv)
    pos0 = [0, 90]
    spans = [[(5, 69)], [(100, 130), (300, 400)]]
    base, scale = _params(kind)
    got = _prefill(q, k, v, gq, gk, kind, 100, base, scale, spans=spans, pos0=pos0)
    ref = A.prefill(q, k, v, kind, 100, base, scale, gq, gk, W.EPS, spans=spans, pos0=pos0)
    assert_parity(got, ref, f"D=256 Hq={Hq} Hkv={Hkv} kind={kind}")


@pytest.mark.parametrize("S,window", [(1, 1024), (33, 1), (64, 32), (97, 1024)])
def test_prefill_edge_shapes(S, window):
    q, k, v, gq, gk = _inputs(20 + S, 1, S, 4, 1)
    for kind in (A.LOCAL, A.GLOBAL):
        base, scale = _params(kind)
        got = _prefill(q, k, v, gq, gk, kind, window, base, scale)
        ref = A.prefill(q, k, v, kind, window, base, scale, gq, gk, W.EPS)
        assert_parity(got, ref, f"D=256 S={S} W={window} kind={kind}")


def test_prefill_online_max_fallback():
    """No QK-norm and integer-valued q/k with scale * log2(e) = 4: sequence 1's
    logits leave the fast path's range (online-maximum pass), sequence 0's
    (scaled by 1/64) do not; a huge interpolation scale keeps every rotation
    angle below 1e-6 rad so the logits stay exact."""
    B, S, Hq, Hkv = 2, 300, 4, 1
    rng = np.random.default_rng(31)
    q = np.round(rng.standard_normal((B, S, Hq, D))).astype(np.float32)
    k = np.round(rng.standard_normal((B, S, Hkv, D))).astype(np.float32)
    v = W.host_normal_bf16((B, S, Hkv, D), 32)
    q[0] *= 1.0 / 64
    sm = 4.0 / np.log2(np.e)
    for kind in (A.LOCAL, A.GLOBAL):
        base = W.ROPE_BASE_LOCAL if kind == A.LOCAL else W.ROPE_BASE_GLOBAL
        got = _prefill(q, k, v, None, None, kind, 100, base, 1e9, sm=sm)
        ref = A.prefill(q, k, v, kind, 100, base, 1e9, None, None, W.EPS, sm)
        assert_parity(got[0], ref[0], "sequence 0 (fast path)")
        assert_parity(got[1], ref[1], "sequence 1 (online maximum)")


def _fill_cache(k_raw, v_raw, gk, cap, is_ring, base, scale, n):
    B, S, Hkv, _ = k_raw.shape
    ck = np.zeros((B, Hkv, cap, D), dtype=np.float32)
    cv = np.zeros((B, Hkv, cap, D), dtype=np.float32)
    for b in range(B):
        kh = W.bf16_round(A.qknorm_rope(k_raw[b, :n], gk, W.EPS, np.arange(n), base, scale).astype(np.float32))
        for j in range(n):
            s = j % cap if is_ring else j
            ck[b, :, s] = kh[j]
            cv[b, :, s] = v_raw[b, j]
    return ck, cv


@pytest.mark.parametrize("kind,is_ring,cap,p0", [(A.GLOBAL, False, 2000, 1100), (A.LOCAL, True, 1024, 1100),
                                                 (A.LOCAL, True, 1024, 1024)])
def test_chunked_prefill_against_cache(kind, is_ring, cap, p0):
    B, Stot, Hq, Hkv = 1, 1400, 4, 1
    q, k, v, gq, gk = _inputs(40 + kind, B, Stot, Hq, Hkv)
    base, scale = _params(kind, 8.0)
    ck, cv = _fill_cache(k, v, gk, cap, is_ring, base, scale, p0)
    cache = G.KVCache(dev_bf16(ck), dev_bf16(cv), is_ring)
    o = G.prefill(dev_bf16(q[:, p0:]), dev_bf16(k[:, p0:]), dev_bf16(v[:, p0:]), kind, W.WINDOW, base, scale,
                  dev_f32(gq), dev_f32(gk), W.EPS, 0.0, None, [p0], cache)
    torch.cuda.synchronize()
    ref, rck, rcv = A.prefill_chunk(q[:, p0:], k[:, p0:], v[:, p0:], ck, cv, is_ring, kind, W.WINDOW, base, scale,
                                    gq, gk, W.EPS, pos0=[p0])
    assert_parity(host(o), ref, f"D=256 chunk kind={kind} ring={is_ring}")
    assert np.array_equal(host(cache.v), rcv)
    assert_rowwise_bf16(host(cache.k), rck, "cache k after append")


@pytest.mark.parametrize("kind,is_ring,cap", [(A.GLOBAL, False, 5000), (A.LOCAL, True, 1024)])
@pytest.mark.parametrize("Hq,Hkv", [(4, 1), (2, 2), (8, 1), (4, 2)])  # G = 4, 1, 8, 2
def test_decode_against_cache(kind, is_ring, cap, Hq, Hkv):
    B = 4
    positions = np.array([0, 700, 1023, 4097], dtype=np.int32)
    base, scale = _params(kind, 8.0)
    sd = 500 + 10 * Hq + Hkv
    ck = W.host_normal_bf16((B, Hkv, cap, D), sd)
    cv = W.host_normal_bf16((B, Hkv, cap, D), sd + 1)
    q = W.host_normal_bf16((B, Hq, D), sd + 2)
    kn = W.host_normal_bf16((B, Hkv, D), sd + 3)
    vn = W.host_normal_bf16((B, Hkv, D), sd + 4)
    gq, gk = W.host_gamma(D, sd + 5), W.host_gamma(D, sd + 6)
    cache = G.KVCache(dev_bf16(ck), dev_bf16(cv), is_ring)
    maxp = int(positions.max())
    o = G.decode(dev_bf16(q), dev_bf16(kn), dev_bf16(vn), torch.from_numpy(positions).cuda(), maxp, cache, kind,
                 W.WINDOW, base, scale, dev_f32(gq), dev_f32(gk), W.EPS)
    torch.cuda.synchronize()
    ref, rck, rcv = A.decode(q, kn, vn, ck, cv, is_ring, positions, kind, W.WINDOW, base, scale, gq, gk, W.EPS)
    assert_parity(host(o), ref, f"D=256 decode kind={kind} G={Hq // Hkv}")
    assert np.array_equal(host(cache.v), rcv)
    assert_rowwise_bf16(host(cache.k), rck, "cache k after decode append")
