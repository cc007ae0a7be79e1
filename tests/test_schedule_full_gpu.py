"""GPU parity of the whole 62-layer 27B attention stack at its full size: one
131072-position sequence, the prompt (131040 tokens) through 32 chunked
prefills of up to 4096 tokens over per-layer caches, then 32 decode steps
(positions 131040..131071), the last 16 by replaying a captured graph.

Gemma 3 Technical Report, section 2: 5:1 interleaving (62 layers = 10 global
and 52 local, the first local), local span 1024 with RoPE base 10k, global
layers over the whole 128K context with RoPE base 1M and linear position
interpolation (scale 8 here).  "Gemma explained: What's new in Gemma 3",
27B print: 32 query heads, 16 kv heads of 128.

The oracle cannot run 62 layers x 128K rows, so sampled outputs are
compared: rows of the last prompt chunk and the last decoded token of one
global layer (59, the last global) and one local layer (60), each computed
by the oracle from the raw inputs of every position it sees, for three of
the sixteen kv groups.  Inputs repeat per chunk as in the bench: layer i
reads input set i % 2 (chunk row r of every chunk takes row r of the set;
every decode step takes the set's one decode row)."""
import numpy as np
import pytest

import oracle.attention as A
import workloads as W
from tests.gpu_util import assert_parity, dev_bf16, dev_f32, host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from global_gqa_amd.schedule import AttentionStack, chunk_bounds  # noqa: E402

CONFIG = 11  # seed namespace of this test's inputs
N_LAYERS, HQ, HKV, D = 62, 32, 16, 128
TOTAL, CHUNK, N_DECODE, INTERP = 131072, 4096, 32, 8.0
KV_GROUPS = [0, 7, 15]  # kv heads checked (query heads 2g, 2g + 1)
CHUNK_ROWS = [0, 1, 1023, 2048, 4062, 4063]  # rows of the last prompt chunk checked
CHECK = {59: A.GLOBAL, 60: A.LOCAL}


def _oracle_rows(plan, qpos, qraw, kpos, kraw, vraw, gq, gk):
    """Oracle outputs of query rows qraw [n, Hq', D] at qpos against keys of
    raw kraw / vraw [m, Hkv', D] at kpos, for one layer plan."""
    qh = A.qknorm_rope(qraw, gq, W.EPS, qpos, plan.rope_base, plan.interp_scale, True)
    kh = A.qknorm_rope(kraw, gk, W.EPS, kpos, plan.rope_base, plan.interp_scale, True)
    mask = A.visibility(qpos, kpos, plan.kind, plan.window)
    return A.attend(qh, kh, vraw, mask, D ** -0.5)


def test_62_layer_128k_schedule_sampled_rows():
    print("62-layer 128K schedule: building inputs", flush=True)
    sets = [tuple(W.host_normal_bf16(shape, W.seed_of(CONFIG, s, t)) for shape, t in
                  [((1, CHUNK, HQ, D), W.T_Q), ((1, CHUNK, HKV, D), W.T_K), ((1, CHUNK, HKV, D), W.T_V)])
            for s in range(2)]
    dsets = [tuple(W.host_normal_bf16(shape, W.seed_of(CONFIG, 10 + s, t)) for shape, t in
                   [((1, HQ, D), W.T_Q), ((1, HKV, D), W.T_K), ((1, HKV, D), W.T_V)]) for s in range(2)]
    gq = [W.host_gamma(D, W.seed_of(CONFIG, 20 + l, W.T_GQ)) for l in range(N_LAYERS)]
    gk = [W.host_gamma(D, W.seed_of(CONFIG, 20 + l, W.T_GK)) for l in range(N_LAYERS)]
    stack = AttentionStack(N_LAYERS, 1, HQ, HKV, max_positions=TOTAL, max_chunk=CHUNK, D=D, window=W.WINDOW,
                           global_interp_scale=INTERP, q_gammas=[dev_f32(g) for g in gq],
                           k_gammas=[dev_f32(g) for g in gk], eps=W.EPS)
    assert sum(p.kind == A.GLOBAL for p in stack.plans) == 10
    for l, kind in CHECK.items():
        assert stack.plans[l].kind == kind
    dpre = [tuple(dev_bf16(x) for x in s) for s in sets]
    ddec = [tuple(dev_bf16(x) for x in s) for s in dsets]
    o_pre = torch.empty_like(dpre[0][0])
    o_last = {l: torch.zeros_like(dpre[0][0]) for l in CHECK}  # the last chunk fills 4064 of 4096 rows
    prompt = TOTAL - N_DECODE
    bounds = chunk_bounds(prompt, CHUNK)
    assert len(bounds) == 32 and bounds[-1] == (126976, prompt)
    for ci, (s0, e0) in enumerate(bounds):
        n = e0 - s0
        last = ci == len(bounds) - 1
        for i in range(N_LAYERS):
            q, k, v = dpre[i & 1]
            o = o_last[i][:, :n] if (last and i in CHECK) else o_pre[:, :n]
            stack.prefill_layer(i, q[:, :n], k[:, :n], v[:, :n], o=o)
        stack.advance(n)
        if ci % 8 == 7:
            torch.cuda.synchronize()
            print(f"prefill chunk {ci + 1}/{len(bounds)} done", flush=True)
    n_eager = N_DECODE // 2
    o_dec = torch.empty_like(ddec[0][0])
    for t in range(n_eager):
        for i in range(N_LAYERS):
            q, k, v = ddec[i & 1]
            stack.decode_layer(i, q, k, v, o=o_dec)
        stack.advance(1)
    torch.cuda.synchronize()
    o_bufs = [torch.empty_like(ddec[0][0]) for _ in range(N_LAYERS)]
    step = stack.capture_decode([ddec[i & 1][0] for i in range(N_LAYERS)], [ddec[i & 1][1] for i in range(N_LAYERS)],
                                [ddec[i & 1][2] for i in range(N_LAYERS)], o_bufs)
    for t in range(N_DECODE - n_eager):
        step()
    torch.cuda.synchronize()
    assert stack.pos == TOTAL
    print("62-layer 128K schedule ran; oracle checks", flush=True)

    qh_sel = [h for g in KV_GROUPS for h in (2 * g, 2 * g + 1)]
    s_last, e_last = bounds[-1]
    for l, kind in CHECK.items():
        plan = stack.plans[l]
        qs, ks, vs = sets[l & 1]
        dq, dk, dv = dsets[l & 1]

        ksel, vsel = ks[0][:, KV_GROUPS], vs[0][:, KV_GROUPS]

        def raw_kv(pos):
            """Raw k, v [len(pos), Hkv', D] of the positions (prompt rows repeat per chunk)."""
            pos = np.asarray(pos)
            r = pos % CHUNK
            k = np.where((pos < prompt)[:, None, None], ksel[r], dk[0][KV_GROUPS][None])
            v = np.where((pos < prompt)[:, None, None], vsel[r], dv[0][KV_GROUPS][None])
            return k, v

        # sampled rows of the last prompt chunk
        rows = np.array(CHUNK_ROWS)
        qpos = s_last + rows
        klo = 0 if kind == A.GLOBAL else int(qpos.min()) - plan.window + 1
        kpos = np.arange(klo, int(qpos.max()) + 1)
        kr, vr = raw_kv(kpos)
        ref = _oracle_rows(plan, qpos, qs[0][rows][:, qh_sel], kpos, kr, vr, gq[l], gk[l])
        got = host(o_last[l])[0][rows][:, qh_sel]
        e = assert_parity(got, ref, f"layer {l} last chunk rows")
        print(f"layer {l} chunk rows: {e}", flush=True)
        # the last decoded token (position TOTAL - 1), from the graph replay
        p = TOTAL - 1
        kpos = np.arange(0 if kind == A.GLOBAL else p - plan.window + 1, p + 1)
        kr, vr = raw_kv(kpos)
        ref = _oracle_rows(plan, np.array([p]), dq[0][qh_sel][None], kpos, kr, vr, gq[l], gk[l])[0]
        got = host(o_bufs[l])[0][qh_sel]
        e = assert_parity(got, ref, f"layer {l} last decode token")
        print(f"layer {l} decode token {p}: {e}", flush=True)
