"""Parity at the full workload sizes, in the launch configuration bench.py
times: the same seeded device-generated inputs, the same calls; the oracle
recomputes sampled rows (one query head at a time, every key it can see).
"""
import numpy as np
import pytest

import oracle.attention as A
import workloads as W
from tests.gpu_util import assert_parity, assert_rowwise_bf16, host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import global_gqa_amd as G  # noqa: E402


def _h(t):
    return host(t)


def _oracle_rows(q_raw, qpos, kh, kpos, v, kind, window, base, scale, gq, eps, spans=()):
    """Oracle output of one query head for selected rows.
    q_raw [R, D] raw queries, kh [K, D] normed+rotated keys, v [K, D]."""
    qh = A.qknorm_rope(q_raw[:, None, :], gq, eps, qpos, base, scale)
    mask = A.visibility(qpos, kpos, kind, window, spans)
    return A.attend(qh, kh[:, None, :], v[:, None, :], mask, float(q_raw.shape[-1]) ** -0.5)[:, 0, :]


ROWS_8K = np.r_[0:32, 1000:1032, 4100:4132, 8160:8192]


@pytest.mark.parametrize("layer", [0, 5])  # a local layer and the global layer of the block
def test_27b_prefill_block_sampled(layer):
    w = W.WORKLOADS[2]
    kind = G.layer_kind(layer)
    base = W.ROPE_BASE_GLOBAL if kind == G.GLOBAL else W.ROPE_BASE_LOCAL
    q = W.device_normal_bf16((w.B, w.S, w.Hq, w.D), W.seed_of(2, layer, W.T_Q))
    k = W.device_normal_bf16((w.B, w.S, w.Hkv, w.D), W.seed_of(2, layer, W.T_K))
    v = W.device_normal_bf16((w.B, w.S, w.Hkv, w.D), W.seed_of(2, layer, W.T_V))
    gq = W.host_gamma(w.D, W.seed_of(2, layer, W.T_GQ))
    gk = W.host_gamma(w.D, W.seed_of(2, layer, W.T_GK))
    o = G.prefill(q, k, v, kind, W.WINDOW, base, 1.0, torch.from_numpy(gq).cuda(), torch.from_numpy(gk).cuda(),
                  W.EPS)
    torch.cuda.synchronize()
    pos = np.arange(w.S)
    for h in (0, 17, 31):
        g = h // (w.Hq // w.Hkv)
        kh = A.qknorm_rope(_h(k[0, :, g:g + 1]), gk, W.EPS, pos, base, 1.0)[:, 0, :]
        ref = _oracle_rows(_h(q[0, ROWS_8K, h]), ROWS_8K, kh, pos, _h(v[0, :, g]), kind, W.WINDOW, base, 1.0, gq,
                           W.EPS)
        assert_parity(_h(o[0, ROWS_8K, h]), ref, f"27B prefill layer {layer} head {h}")


@pytest.mark.parametrize("layer", [0, 5])
def test_27b_decode_block_sampled(layer):
    w = W.WORKLOADS[3]
    kind = G.layer_kind(layer)
    base = W.ROPE_BASE_GLOBAL if kind == G.GLOBAL else W.ROPE_BASE_LOCAL
    p = w.pos0
    cap = W.RING_CAP if kind == G.LOCAL else p + 64
    ck = W.device_normal_bf16((w.B, w.Hkv, cap, w.D), W.seed_of(3, layer, W.T_CK))
    cv = W.device_normal_bf16((w.B, w.Hkv, cap, w.D), W.seed_of(3, layer, W.T_CV))
    q = W.device_normal_bf16((w.B, w.Hq, w.D), W.seed_of(3, layer, W.T_Q))
    kn = W.device_normal_bf16((w.B, w.Hkv, w.D), W.seed_of(3, layer, W.T_K))
    vn = W.device_normal_bf16((w.B, w.Hkv, w.D), W.seed_of(3, layer, W.T_V))
    gq = W.host_gamma(w.D, W.seed_of(3, layer, W.T_GQ))
    gk = W.host_gamma(w.D, W.seed_of(3, layer, W.T_GK))
    sample_b = [0, 13, 31]
    before = {b: (_h(ck[b]), _h(cv[b])) for b in sample_b}
    cache = G.KVCache(ck, cv, is_ring=(kind == G.LOCAL))
    positions = torch.full((w.B,), p, dtype=torch.int32, device="cuda")
    o = G.decode(q, kn, vn, positions, p, cache, kind, W.WINDOW, base, 1.0, torch.from_numpy(gq).cuda(),
                 torch.from_numpy(gk).cuda(), W.EPS)
    torch.cuda.synchronize()
    for b in sample_b:
        ck0, cv0 = before[b]
        ref, rck, rcv = A.decode(_h(q[b:b + 1]), _h(kn[b:b + 1]), _h(vn[b:b + 1]), ck0[None], cv0[None],
                                 kind == G.LOCAL, [p], kind, W.WINDOW, base, 1.0, gq, gk, W.EPS)
        assert_parity(_h(o[b:b + 1]), ref, f"27B decode layer {layer} seq {b}")
        slot = p % cap if kind == G.LOCAL else p
        assert np.array_equal(_h(cv[b, :, slot]), rcv[0, :, slot])
        assert_rowwise_bf16(_h(ck[b, :, slot]), rck[0, :, slot], "appended key")


@pytest.mark.parametrize("layer", [0, 5])
def test_27b_chunked_prefill_128k_sampled(layer):
    w = W.WORKLOADS[4]
    kind = G.layer_kind(layer)
    p0 = w.pos0
    if kind == G.GLOBAL:
        base, scale, cap, ring = W.ROPE_BASE_GLOBAL, w.interp_scale_global, p0 + w.S, False
    else:
        base, scale, cap, ring = W.ROPE_BASE_LOCAL, 1.0, W.RING_CAP, True
    ck = W.device_normal_bf16((w.B, w.Hkv, cap, w.D), W.seed_of(4, layer, W.T_CK))
    cv = W.device_normal_bf16((w.B, w.Hkv, cap, w.D), W.seed_of(4, layer, W.T_CV))
    q = W.device_normal_bf16((w.B, w.S, w.Hq, w.D), W.seed_of(4, layer, W.T_Q))
    k = W.device_normal_bf16((w.B, w.S, w.Hkv, w.D), W.seed_of(4, layer, W.T_K))
    v = W.device_normal_bf16((w.B, w.S, w.Hkv, w.D), W.seed_of(4, layer, W.T_V))
    gq = W.host_gamma(w.D, W.seed_of(4, layer, W.T_GQ))
    gk = W.host_gamma(w.D, W.seed_of(4, layer, W.T_GK))
    heads = (0, 31)
    kvh = sorted({h // (w.Hq // w.Hkv) for h in heads})
    old = {g: (_h(ck[0, g]), _h(cv[0, g])) for g in kvh}
    cache = G.KVCache(ck, cv, is_ring=ring)
    o = G.prefill(q, k, v, kind, W.WINDOW, base, scale, torch.from_numpy(gq).cuda(), torch.from_numpy(gk).cuda(),
                  W.EPS, 0.0, None, [p0], cache)
    torch.cuda.synchronize()
    rows = np.r_[0:32, 2000:2032, 4064:4096]
    chunk_pos = p0 + np.arange(w.S)
    for h in heads:
        g = h // (w.Hq // w.Hkv)
        kh_new = A.qknorm_rope(_h(k[0, :, g:g + 1]), gk, W.EPS, chunk_pos, base, scale)[:, 0, :]
        lo_old = max(0, p0 - cap) if ring else 0
        old_pos = np.arange(lo_old, p0)
        slots = old_pos % cap if ring else old_pos
        kh = np.concatenate([old[g][0][slots], kh_new])
        vv = np.concatenate([old[g][1][slots], _h(v[0, :, g])])
        kpos = np.concatenate([old_pos, chunk_pos])
        ref = _oracle_rows(_h(q[0, rows, h]), chunk_pos[rows], kh, kpos, vv, kind, W.WINDOW, base, scale, gq,
                           W.EPS)
        assert_parity(_h(o[0, rows, h]), ref, f"128K chunk layer {layer} head {h}")
        # the chunk's keys/values were appended (a ring keeps its last 1024 positions)
        tail = chunk_pos[-8:]
        tslot = tail % cap if ring else tail
        assert np.array_equal(_h(cv[0, g, tslot]), _h(v[0, -8:, g]))
        assert_rowwise_bf16(_h(ck[0, g, tslot]), kh_new[-8:], "appended chunk keys")


@pytest.mark.parametrize("kind", [G.LOCAL, G.GLOBAL])
def test_mixed_mask_4k_full_heads(kind):
    """Mixed-mask workload at full size (B=2, S=4096, Hq=16, Hkv=8, image
    spans), every row of three heads per sequence."""
    w = W.WORKLOADS[5]
    layer = 0 if kind == G.LOCAL else 5
    base = W.ROPE_BASE_GLOBAL if kind == G.GLOBAL else W.ROPE_BASE_LOCAL
    inp = W.layer_inputs(w, layer)
    spans = W.workload_spans(w)
    flat = [(b, s, e) for b in range(w.B) for (s, e) in spans[b]]
    dev = {n: torch.from_numpy(x).cuda().to(torch.bfloat16) for n, x in inp.items() if n in ("q", "k", "v")}
    o = G.prefill(dev["q"], dev["k"], dev["v"], kind, W.WINDOW, base, 1.0, torch.from_numpy(inp["q_gamma"]).cuda(),
                  torch.from_numpy(inp["k_gamma"]).cuda(), W.EPS, 0.0, flat)
    torch.cuda.synchronize()
    pos = np.arange(w.S)
    for b in range(w.B):
        for h in (0, 5, 15):
            g = h // (w.Hq // w.Hkv)
            kh = A.qknorm_rope(inp["k"][b, :, g:g + 1], inp["k_gamma"], W.EPS, pos, base, 1.0)[:, 0, :]
            ref = _oracle_rows(inp["q"][b, :, h], pos, kh, pos, inp["v"][b, :, g], kind, W.WINDOW, base, 1.0,
                               inp["q_gamma"], W.EPS, spans[b])
            assert_parity(_h(o[b, :, h]), ref, f"mixed mask b={b} h={h} kind={kind}")


def test_local_uneven_items_per_workgroup():
    """Local layer with 16 kv heads x 33 query tiles = 528 work items: with one
    workgroup per CU some workgroups run one item more than others (and the
    last query tile is ragged).  Every row of four heads against the oracle."""
    B, S, Hq, Hkv, D = 1, 33 * 128 - 40, 32, 16, 128
    rng = np.random.default_rng(77)
    q = W.bf16_round(rng.standard_normal((B, S, Hq, D)).astype(np.float32))
    k = W.bf16_round(rng.standard_normal((B, S, Hkv, D)).astype(np.float32))
    v = W.bf16_round(rng.standard_normal((B, S, Hkv, D)).astype(np.float32))
    gq = W.host_gamma(D, 78)
    gk = W.host_gamma(D, 79)
    dv = lambda x: torch.from_numpy(x).cuda().to(torch.bfloat16)  # noqa: E731
    o = G.prefill(dv(q), dv(k), dv(v), G.LOCAL, W.WINDOW, W.ROPE_BASE_LOCAL, 1.0, torch.from_numpy(gq).cuda(),
                  torch.from_numpy(gk).cuda(), W.EPS)
    torch.cuda.synchronize()
    pos = np.arange(S)
    for h in (0, 9, 22, 31):
        g = h // (Hq // Hkv)
        kh = A.qknorm_rope(k[0, :, g:g + 1], gk, W.EPS, pos, W.ROPE_BASE_LOCAL, 1.0)[:, 0, :]
        ref = _oracle_rows(q[0, :, h], pos, kh, pos, v[0, :, g], G.LOCAL, W.WINDOW, W.ROPE_BASE_LOCAL, 1.0, gq, W.EPS)
        assert_parity(_h(o[0, :, h]), ref, f"uneven local h={h}")
