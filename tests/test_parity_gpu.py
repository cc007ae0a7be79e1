"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on the
same seeded inputs, at sizes the oracle finishes in seconds that still span
several tiles and a ragged tail, plus edge cases and exact mask probes."""
import numpy as np
import pytest

import oracle.attention as A
import workloads as W
from tests.gpu_util import assert_parity, assert_rowwise_bf16, dev_bf16, dev_f32, errors, host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import global_gqa_amd as G  # noqa: E402


def _inputs(config, layer, B, S, Hq, Hkv, D=128):
    q = W.host_normal_bf16((B, S, Hq, D), W.seed_of(config, layer, W.T_Q))
    k = W.host_normal_bf16((B, S, Hkv, D), W.seed_of(config, layer, W.T_K))
    v = W.host_normal_bf16((B, S, Hkv, D), W.seed_of(config, layer, W.T_V))
    gq = W.host_gamma(D, W.seed_of(config, layer, W.T_GQ))
    gk = W.host_gamma(D, W.seed_of(config, layer, W.T_GK))
    return q, k, v, gq, gk


def _kind_params(kind, scale_global=1.0):
    return (W.ROPE_BASE_LOCAL, 1.0) if kind == A.LOCAL else (W.ROPE_BASE_GLOBAL, scale_global)


# ------------------------------------------------------------------ prologue
@pytest.mark.parametrize("base,scale,norm", [(1e4, 1.0, True), (1e6, 8.0, True), (1e4, 1.0, False)])
def test_qknorm_rope_matches_oracle(base, scale, norm):
    T, Hq, Hkv, D = 333, 4, 2, 128
    rng = np.random.default_rng(11)
    q = W.host_normal_bf16((T, Hq, D), 1)
    k = W.host_normal_bf16((T, Hkv, D), 2)
    pos = np.concatenate([np.arange(200), rng.integers(0, 131072, T - 201), [131071]]).astype(np.int32)
    gq, gk = W.host_gamma(D, 3), W.host_gamma(D, 4)
    qo, ko = G.qknorm_rope(dev_bf16(q), dev_bf16(k), torch.from_numpy(pos).cuda(),
                           dev_f32(gq) if norm else None, dev_f32(gk) if norm else None, 1e-6, base, scale)
    torch.cuda.synchronize()
    rq = A.qknorm_rope(q, gq if norm else None, 1e-6, pos, base, scale, norm)
    rk = A.qknorm_rope(k, gk if norm else None, 1e-6, pos, base, scale, norm)
    assert_rowwise_bf16(host(qo), rq, "q_hat")
    assert_rowwise_bf16(host(ko), rk, "k_hat")
    # in place
    qi = dev_bf16(q)
    G.qknorm_rope(qi, None, torch.from_numpy(pos).cuda(), dev_f32(gq) if norm else None, None, 1e-6, base, scale,
                  q_out=qi)
    torch.cuda.synchronize()
    assert bool(torch.equal(qi, qo)), "in-place result differs"



# ------------------------------------------------------------------ prefill
def _run_prefill(q, k, v, gq, gk, kind, base, scale, spans=None, pos0=None, window=W.WINDOW):
    B = q.shape[0]
    flat = None
    if spans:
        flat = [(b, s, e) for b in range(B) for (s, e) in spans[b]]
    o = G.prefill(dev_bf16(q), dev_bf16(k), dev_bf16(v), kind, window, base, scale, dev_f32(gq), dev_f32(gk),
                  W.EPS, 0.0, flat, pos0)
    torch.cuda.synchronize()
    return host(o)


@pytest.mark.parametrize("kind", [A.LOCAL, A.GLOBAL])
def test_prefill_single_layer_2k(kind):
    """The single-layer workload at full size: B=1, S=2048, Hq=4, Hkv=2."""
    w = W.WORKLOADS[1]
    q, k, v, gq, gk = _inputs(1, kind, w.B, w.S, w.Hq, w.Hkv)
    base, scale = _kind_params(kind)
    got = _run_prefill(q, k, v, gq, gk, kind, base, scale)
    ref = A.prefill(q, k, v, kind, W.WINDOW, base, scale, gq, gk, W.EPS)
    assert_parity(got, ref, f"config1 kind={kind}")


@pytest.mark.parametrize("kind", [A.LOCAL, A.GLOBAL])
@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (4, 2), (8, 2), (8, 1)])
def test_prefill_ragged_gqa_groups(kind, Hq, Hkv):
    """Ragged S (not a multiple of any tile), B=2, every GQA group size, a
    small window so local rows cross several key tiles."""
    B, S = 2, 777
    q, k, v, gq, gk = _inputs(9, 10 * Hq + Hkv, B, S, Hq, Hkv)
    base, scale = _kind_params(kind, 8.0)
    got = _run_prefill(q, k, v, gq, gk, kind, base, scale, window=200)
    ref = A.prefill(q, k, v, kind, 200, base, scale, gq, gk, W.EPS)
    assert_parity(got, ref, f"S=777 Hq={Hq} Hkv={Hkv} kind={kind}")


@pytest.mark.parametrize("kind", [A.LOCAL, A.GLOBAL])
def test_prefill_spans_and_pos0(kind):
    """Mixed-mask recipe on a reduced shape: unaligned image spans, B=2,
    per-sequence first positions."""
    B, S, Hq, Hkv = 2, 1500, 4, 2
    q, k, v, gq, gk = _inputs(5, kind, B, S, Hq, Hkv)
    pos0 = [0, 300]
    spans = [W.image_spans(S, 4, 77, base=0), W.image_spans(S, 2, 78, base=300)]
    base, scale = _kind_params(kind)
    got = _run_prefill(q, k, v, gq, gk, kind, base, scale, spans=spans, pos0=pos0, window=500)
    ref = A.prefill(q, k, v, kind, 500, base, scale, gq, gk, W.EPS, spans=spans, pos0=pos0)
    assert_parity(got, ref, f"spans kind={kind}")


@pytest.mark.parametrize("S,window", [(1, 1024), (2, 1), (65, 1), (130, 64), (300, 1024)])
def test_prefill_edge_shapes(S, window):
    B, Hq, Hkv = 1, 2, 1
    q, k, v, gq, gk = _inputs(8, S, B, S, Hq, Hkv)
    for kind in (A.LOCAL, A.GLOBAL):
        base, scale = _kind_params(kind)
        got = _run_prefill(q, k, v, gq, gk, kind, base, scale, window=window)
        ref = A.prefill(q, k, v, kind, window, base, scale, gq, gk, W.EPS)
        assert_parity(got, ref, f"S={S} W={window} kind={kind}")


@pytest.mark.parametrize("D", [128, 256])
def test_local_window_past_any_reach_equals_global(D):
    """A local layer whose window exceeds every position gap has no band
    limit: with the largest int32 window the prefill (self-contained and
    against a linear cache) and the decode give the global layer's bits."""
    B, S, Hq, Hkv = 2, 700, 4, 1
    q, k, v, gq, gk = _inputs(8, 200 + D, B, S, Hq, Hkv, D=D)
    big = 2 ** 31 - 1
    loc = _run_prefill(q, k, v, gq, gk, A.LOCAL, 1e4, 1.0, window=big)
    glo = _run_prefill(q, k, v, gq, gk, A.GLOBAL, 1e4, 1.0, window=big)
    assert np.array_equal(loc, glo), "prefill: local with an unbounded window differs from global"
    assert_parity(loc, A.prefill(q, k, v, A.GLOBAL, W.WINDOW, 1e4, 1.0, gq, gk, W.EPS), "unbounded window")
    cap, p = 900, 800
    ck = W.host_normal_bf16((B, Hkv, cap, D), W.seed_of(8, 210 + D, W.T_CK))
    cv = W.host_normal_bf16((B, Hkv, cap, D), W.seed_of(8, 210 + D, W.T_CV))
    pos = torch.full((B,), p, dtype=torch.int32, device="cuda")
    outs = []
    for kind in (A.LOCAL, A.GLOBAL):
        cache = G.KVCache(dev_bf16(ck), dev_bf16(cv), False)
        outs.append(host(G.decode(dev_bf16(q[:, 0]), dev_bf16(k[:, 0]), dev_bf16(v[:, 0]), pos, p, cache, kind, big,
                                  1e4, 1.0, dev_f32(gq), dev_f32(gk), W.EPS)))
    torch.cuda.synchronize()
    assert np.array_equal(outs[0], outs[1]), "decode: local with an unbounded window differs from global"


def test_prefill_span_covering_whole_sequence_and_edges():
    B, S, Hq, Hkv = 3, 300, 2, 1
    q, k, v, gq, gk = _inputs(8, 99, B, S, Hq, Hkv)
    spans = [[(0, 300)], [(0, 1), (299, 300)], [(0, 64), (64, 128), (290, 300)]]
    for kind in (A.LOCAL, A.GLOBAL):
        base, scale = _kind_params(kind)
        got = _run_prefill(q, k, v, gq, gk, kind, base, scale, spans=spans, window=100)
        ref = A.prefill(q, k, v, kind, 100, base, scale, gq, gk, W.EPS, spans=spans)
        assert_parity(got, ref, f"span edges kind={kind}")


def test_prefill_mask_probe_exact():
    """K = 0 gives uniform weights, V = indicator of a key set gives
    o_i = |A n vis(i)| / |vis(i)| (exact up to the final bf16 rounding)."""
    B, S, Hq, Hkv, D = 1, 2100, 2, 1, 128
    spans = [[(1030, 1286)]]
    key_set = [0, 1, 63, 64, 500, 1023, 1024, 1030, 1100, 1285, 1286, 2047, 2099]
    v = np.zeros((B, S, Hkv, D), dtype=np.float32)
    v[0, key_set, 0, :] = 1.0
    k = np.zeros((B, S, Hkv, D), dtype=np.float32)
    q = W.host_normal_bf16((B, S, Hq, D), 5)
    gq = np.ones(D, dtype=np.float32)
    for kind in (A.LOCAL, A.GLOBAL):
        got = _run_prefill(q, k, v, gq, gq, kind, 1e4, 1.0, spans=spans)
        for i in range(S):
            lo, hi = A.visible_interval(i, kind, W.WINDOW, spans[0])
            want = sum(1 for j in key_set if lo <= j <= hi) / (hi - lo + 1)
            # unit roundoff of bf16 (8 significant bits) is 2^-8
            ok = bool(np.all(np.abs(got[0, i] - want) <= 2.0 ** -8 * want))
            assert ok, (kind, i, float(got[0, i, 0, 0]), want)


@pytest.mark.parametrize("kind", [A.LOCAL, A.GLOBAL])
def test_prefill_online_max_fallback(kind):
    """Sequence 1 has logits far outside the fast path's exponent range, so
    its tiles take the online-maximum pass; sequence 0 stays on the fast path.
    The inputs keep the logits exact on the GPU (so the comparison is well
    conditioned even though the softmax is nearly one-hot): no QK-norm,
    integer-valued q/k, a softmax scale with scale*log2(e) = 4 (a power of
    two), and an interpolation scale so large that every rotation angle is
    below 1e-6 rad."""
    B, S, Hq, Hkv = 2, 600, 4, 2
    rng = np.random.default_rng(21)
    q = np.round(rng.standard_normal((B, S, Hq, 128))).astype(np.float32)
    k = np.round(rng.standard_normal((B, S, Hkv, 128))).astype(np.float32)
    v = W.host_normal_bf16((B, S, Hkv, 128), 22)
    q[0] *= 1.0 / 64  # dyadic: still exact; keeps sequence 0 on the fast path
    sm = 4.0 / np.log2(np.e)
    base = W.ROPE_BASE_LOCAL if kind == A.LOCAL else W.ROPE_BASE_GLOBAL
    o = G.prefill(dev_bf16(q), dev_bf16(k), dev_bf16(v), kind, 200, base, 1e9, None, None, W.EPS, sm)
    torch.cuda.synchronize()
    ref = A.prefill(q, k, v, kind, 200, base, 1e9, None, None, W.EPS, sm)
    assert_parity(host(o)[0], ref[0], "sequence 0 (fast path)")
    assert_parity(host(o)[1], ref[1], "sequence 1 (online maximum)")


def test_prefill_deterministic():
    q, k, v, gq, gk = _inputs(1, 0, 1, 1000, 4, 2)
    a = _run_prefill(q, k, v, gq, gk, A.GLOBAL, 1e6, 1.0)
    b = _run_prefill(q, k, v, gq, gk, A.GLOBAL, 1e6, 1.0)
    assert np.array_equal(a, b)


# ------------------------------------------------------------------ chunked prefill
def _fill_cache_host(k_raw, v_raw, gk, cap, is_ring, base, scale, n):
    """Cache state after positions 0..n-1 (raw k normed+rotated by the oracle,
    rounded to bf16 as the GPU cache stores it)."""
    B, S, Hkv, D = k_raw.shape
    ck = np.zeros((B, Hkv, cap, D), dtype=np.float32)
    cv = np.zeros((B, Hkv, cap, D), dtype=np.float32)
    for b in range(B):
        kh = W.bf16_round(A.qknorm_rope(k_raw[b, :n], gk, W.EPS, np.arange(n), base, scale).astype(np.float32))
        for j in range(n):
            s = j % cap if is_ring else j
            ck[b, :, s] = kh[j]
            cv[b, :, s] = v_raw[b, j]
    return ck, cv


# p0 = 1500 puts the cache/chunk boundary inside a key tile; p0 = 1536 on a tile edge (every cache tile
# whole).  The 48-slot ring (window 40) is smaller than a key tile, so its slots repeat inside one tile.
@pytest.mark.parametrize("kind,is_ring,cap,p0,window", [(A.GLOBAL, False, 3000, 1500, W.WINDOW),
                                                        (A.LOCAL, True, 1024, 1500, W.WINDOW),
                                                        (A.LOCAL, False, 3000, 1500, W.WINDOW),
                                                        (A.GLOBAL, False, 3000, 1536, W.WINDOW),
                                                        (A.LOCAL, True, 1024, 1536, W.WINDOW),
                                                        (A.LOCAL, True, 48, 1536, 40)])
def test_chunked_prefill_against_cache(kind, is_ring, cap, p0, window):
    B, Stot, Hq, Hkv = 1, 2600, 4, 2
    q, k, v, gq, gk = _inputs(4, kind, B, Stot, Hq, Hkv)
    base, scale = _kind_params(kind, 8.0)
    ck, cv = _fill_cache_host(k, v, gk, cap, is_ring, base, scale, p0)
    cache = G.KVCache(dev_bf16(ck), dev_bf16(cv), is_ring)
    spans = [[(1600, 1856)]]
    o = G.prefill(dev_bf16(q[:, p0:]), dev_bf16(k[:, p0:]), dev_bf16(v[:, p0:]), kind, window, base, scale,
                  dev_f32(gq), dev_f32(gk), W.EPS, 0.0, [(0, 1600, 1856)], [p0], cache)
    torch.cuda.synchronize()
    ref, rck, rcv = A.prefill_chunk(q[:, p0:], k[:, p0:], v[:, p0:], ck, cv, is_ring, kind, window, base, scale,
                                    gq, gk, W.EPS, spans=spans, pos0=[p0])
    assert_parity(host(o), ref, f"chunk kind={kind} ring={is_ring}")
    assert np.array_equal(host(cache.v), rcv)
    assert_rowwise_bf16(host(cache.k), rck, "cache k after append")


# ------------------------------------------------------------------ decode
@pytest.mark.parametrize("kind,is_ring,cap", [(A.GLOBAL, False, 5000), (A.LOCAL, True, 1024), (A.LOCAL, False, 5000)])
@pytest.mark.parametrize("Hq,Hkv", [(4, 2), (8, 1), (2, 2)])
def test_decode_against_cache(kind, is_ring, cap, Hq, Hkv):
    B, D = 5, 128
    positions = np.array([0, 7, 1023, 1500, 4097], dtype=np.int32)
    base, scale = _kind_params(kind, 8.0)
    rng_seed = 100 * Hq + Hkv
    ck = W.host_normal_bf16((B, Hkv, cap, D), rng_seed)
    cv = W.host_normal_bf16((B, Hkv, cap, D), rng_seed + 1)
    q = W.host_normal_bf16((B, Hq, D), rng_seed + 2)
    kn = W.host_normal_bf16((B, Hkv, D), rng_seed + 3)
    vn = W.host_normal_bf16((B, Hkv, D), rng_seed + 4)
    gq, gk = W.host_gamma(D, 5), W.host_gamma(D, 6)
    cache = G.KVCache(dev_bf16(ck), dev_bf16(cv), is_ring)
    maxp = int(positions.max())
    o = G.decode(dev_bf16(q), dev_bf16(kn), dev_bf16(vn), torch.from_numpy(positions).cuda(), maxp, cache, kind,
                 W.WINDOW, base, scale, dev_f32(gq), dev_f32(gk), W.EPS)
    torch.cuda.synchronize()
    ref, rck, rcv = A.decode(q, kn, vn, ck, cv, is_ring, positions, kind, W.WINDOW, base, scale, gq, gk, W.EPS)
    assert_parity(host(o), ref, f"decode kind={kind} ring={is_ring} G={Hq // Hkv}")
    assert np.array_equal(host(cache.v), rcv)
    assert_rowwise_bf16(host(cache.k), rck, "cache k after decode append")


# Split shapes where the halving of short-cache splits lands on one workgroup
# per CU: the 1B model's 32 sequences on 1024-slot rings (256 splits of 128
# slots, as in its decode step), a short global cache over 8 sequences (256
# splits of 256 slots), and head dimension 128 with 16 sequences of a
# 4096-slot cache (256 splits of 256 slots).
@pytest.mark.parametrize("D,B,Hq,Hkv,kind,is_ring,cap", [(256, 32, 4, 1, A.LOCAL, True, 1024),
                                                         (256, 8, 4, 1, A.GLOBAL, False, 8192),
                                                         (128, 16, 8, 1, A.GLOBAL, False, 4096)])
def test_decode_one_workgroup_per_cu_grid(D, B, Hq, Hkv, kind, is_ring, cap):
    seed = 9100 + D + B
    rng = np.random.default_rng(seed)
    hi = 3 * cap if is_ring else cap
    positions = rng.integers(0, hi, size=B).astype(np.int32)
    positions[:3] = [0, cap - 1, hi - 1]
    if is_ring:
        positions[3] = cap  # the first wrap of the ring
    base, scale = _kind_params(kind, 8.0)
    ck = W.host_normal_bf16((B, Hkv, cap, D), seed)
    cv = W.host_normal_bf16((B, Hkv, cap, D), seed + 1)
    q = W.host_normal_bf16((B, Hq, D), seed + 2)
    kn = W.host_normal_bf16((B, Hkv, D), seed + 3)
    vn = W.host_normal_bf16((B, Hkv, D), seed + 4)
    gq, gk = W.host_gamma(D, seed + 5), W.host_gamma(D, seed + 6)
    cache = G.KVCache(dev_bf16(ck), dev_bf16(cv), is_ring)
    maxp = int(positions.max())
    o = G.decode(dev_bf16(q), dev_bf16(kn), dev_bf16(vn), torch.from_numpy(positions).cuda(), maxp, cache, kind,
                 W.WINDOW, base, scale, dev_f32(gq), dev_f32(gk), W.EPS)
    torch.cuda.synchronize()
    ref, rck, rcv = A.decode(q, kn, vn, ck, cv, is_ring, positions, kind, W.WINDOW, base, scale, gq, gk, W.EPS)
    assert_parity(host(o), ref, f"decode one workgroup per CU D={D} B={B} kind={kind}")
    assert np.array_equal(host(cache.v), rcv)
    assert_rowwise_bf16(host(cache.k), rck, "cache k after decode append")


# A cache slot never written (a fresh allocation past a sequence's end) may hold
# NaN.  Rows the token cannot see get probability 0, and 0 * NaN must not reach
# the sums: the kernels drop such rows' values, not only their weights.
_BF16_NAN = float("nan")


@pytest.mark.parametrize("D,Hq,Hkv", [(128, 4, 2), (256, 4, 1)])
@pytest.mark.parametrize("kind,is_ring,cap", [(A.GLOBAL, False, 5000), (A.LOCAL, True, 1024), (A.LOCAL, False, 5000)])
def test_decode_ignores_nan_in_unwritten_slots(kind, is_ring, cap, D, Hq, Hkv):
    B = 4
    positions = np.array([3, 700, 1500, 4097], dtype=np.int32)
    base, scale = _kind_params(kind, 8.0)
    seed = 7000 + D + 10 * kind + int(is_ring)
    ck = W.host_normal_bf16((B, Hkv, cap, D), seed)
    cv = W.host_normal_bf16((B, Hkv, cap, D), seed + 1)
    for b, p in enumerate(positions):
        if p + 1 < cap:  # slots past p were never written (for a ring only while p < capacity)
            ck[b, :, p + 1:] = _BF16_NAN
            cv[b, :, p + 1:] = _BF16_NAN
    q = W.host_normal_bf16((B, Hq, D), seed + 2)
    kn = W.host_normal_bf16((B, Hkv, D), seed + 3)
    vn = W.host_normal_bf16((B, Hkv, D), seed + 4)
    gq, gk = W.host_gamma(D, 5), W.host_gamma(D, 6)
    cache = G.KVCache(dev_bf16(ck), dev_bf16(cv), is_ring)
    o = G.decode(dev_bf16(q), dev_bf16(kn), dev_bf16(vn), torch.from_numpy(positions).cuda(), int(positions.max()),
                 cache, kind, W.WINDOW, base, scale, dev_f32(gq), dev_f32(gk), W.EPS)
    torch.cuda.synchronize()
    ref, _, _ = A.decode(q, kn, vn, ck, cv, is_ring, positions, kind, W.WINDOW, base, scale, gq, gk, W.EPS)
    assert_parity(host(o), ref, f"decode over NaN-filled unwritten slots kind={kind} ring={is_ring} D={D}")


@pytest.mark.parametrize("kind,is_ring,cap,p0,Stot", [(A.GLOBAL, False, 3000, 1500, 2600),
                                                      (A.LOCAL, True, 1024, 300, 1000),
                                                      (A.LOCAL, False, 3000, 1500, 2600)])
def test_chunked_prefill_ignores_nan_in_unwritten_slots(kind, is_ring, cap, p0, Stot):
    B, Hq, Hkv = 1, 4, 2
    q, k, v, gq, gk = _inputs(4, kind, B, Stot, Hq, Hkv)
    base, scale = _kind_params(kind, 8.0)
    ck, cv = _fill_cache_host(k, v, gk, cap, is_ring, base, scale, p0)
    written = min(p0, cap) if is_ring else p0
    ck[:, :, written:] = _BF16_NAN
    cv[:, :, written:] = _BF16_NAN
    cache = G.KVCache(dev_bf16(ck), dev_bf16(cv), is_ring)
    o = G.prefill(dev_bf16(q[:, p0:]), dev_bf16(k[:, p0:]), dev_bf16(v[:, p0:]), kind, W.WINDOW, base, scale,
                  dev_f32(gq), dev_f32(gk), W.EPS, 0.0, None, [p0], cache)
    torch.cuda.synchronize()
    ref, _, _ = A.prefill_chunk(q[:, p0:], k[:, p0:], v[:, p0:], ck, cv, is_ring, kind, W.WINDOW, base, scale,
                                gq, gk, W.EPS, pos0=[p0])
    assert_parity(host(o), ref, f"chunk over NaN-filled unwritten slots kind={kind} ring={is_ring}")


@pytest.mark.parametrize("D,Hq,Hkv", [(128, 4, 2), (256, 4, 1)])
@pytest.mark.parametrize("kind,is_ring,cap", [(A.GLOBAL, False, 2000), (A.LOCAL, True, 1024)])
def test_decode_online_max_fallback(kind, is_ring, cap, D, Hq, Hkv):
    """Sequence 1's logits leave the fast pass's exponent range, so its splits
    are streamed again with a running maximum; sequence 0 stays on the fast
    pass.  As in the prefill's fallback test the logits are exact on the GPU:
    no QK-norm, integer-valued q and keys, scale * log2(e) = 4, and rotation
    angles below 1e-6 rad."""
    B = 2
    rng = np.random.default_rng(23 + D)
    positions = np.array([1500, 1500], dtype=np.int32)
    ck = np.round(rng.standard_normal((B, Hkv, cap, D))).astype(np.float32)
    cv = W.host_normal_bf16((B, Hkv, cap, D), 24 + D)
    q = np.round(rng.standard_normal((B, Hq, D))).astype(np.float32)
    kn = np.round(rng.standard_normal((B, Hkv, D))).astype(np.float32)
    vn = W.host_normal_bf16((B, Hkv, D), 25 + D)
    q[0] *= 1.0 / 64  # dyadic: still exact; keeps sequence 0 on the fast pass
    sm = 4.0 / np.log2(np.e)
    base = W.ROPE_BASE_LOCAL if kind == A.LOCAL else W.ROPE_BASE_GLOBAL
    cache = G.KVCache(dev_bf16(ck), dev_bf16(cv), is_ring)
    o = G.decode(dev_bf16(q), dev_bf16(kn), dev_bf16(vn), torch.from_numpy(positions).cuda(), int(positions.max()),
                 cache, kind, W.WINDOW, base, 1e9, None, None, W.EPS, sm)
    torch.cuda.synchronize()
    ref, _, _ = A.decode(q, kn, vn, ck, cv, is_ring, positions, kind, W.WINDOW, base, 1e9, None, None, W.EPS, sm)
    assert_parity(host(o)[0], ref[0], "sequence 0 (fast pass)")
    assert_parity(host(o)[1], ref[1], "sequence 1 (running maximum)")


def test_decode_deterministic_and_matches_prefill_last_row():
    """Decode of token p equals row p of a self-contained prefill whose first
    p tokens were written to the cache by a chunked prefill."""
    B, S, Hq, Hkv = 1, 700, 4, 2
    q, k, v, gq, gk = _inputs(3, 0, B, S, Hq, Hkv)
    full = _run_prefill(q, k, v, gq, gk, A.GLOBAL, 1e6, 1.0)
    cache = G.KVCache.empty(B, Hkv, 1024, is_ring=False)
    p = S - 1
    G.prefill(dev_bf16(q[:, :p]), dev_bf16(k[:, :p]), dev_bf16(v[:, :p]), A.GLOBAL, W.WINDOW, 1e6, 1.0,
              dev_f32(gq), dev_f32(gk), W.EPS, 0.0, None, [0], cache)
    pos = torch.tensor([p], dtype=torch.int32, device="cuda")
    outs = []
    for _ in range(2):
        c2 = G.KVCache(cache.k.clone(), cache.v.clone(), False)
        o = G.decode(dev_bf16(q[:, p]), dev_bf16(k[:, p]), dev_bf16(v[:, p]), pos, p, c2, A.GLOBAL, W.WINDOW, 1e6,
                     1.0, dev_f32(gq), dev_f32(gk), W.EPS)
        torch.cuda.synchronize()
        outs.append(host(o))
    assert np.array_equal(outs[0], outs[1])
    e = errors(outs[0], full[:, p])
    assert e["max_abs"] < 1e-2, e
