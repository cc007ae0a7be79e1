"""GPU parity of a whole attention stack: a prompt through successive chunked
prefills over per-layer caches (local rings that wrap inside a chunk and
across chunk boundaries, linear global caches with position interpolation),
then decode steps, every output against the oracle's self-contained prefill
of the full sequence of that layer (row p of it is what the token at
position p must produce)."""
import numpy as np
import pytest

import oracle.attention as A
import workloads as W
from tests.gpu_util import assert_parity, assert_rowwise_bf16, dev_bf16, dev_f32, host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from global_gqa_amd.schedule import AttentionStack  # noqa: E402

CONFIG = 7  # seed namespace of this test's inputs


@pytest.mark.parametrize("B,Hq,Hkv,chunks,n_decode", [
    (1, 4, 2, [700, 700, 400], 3),   # ring wraps inside chunk 2, then across the chunk 2/3 boundary
    (2, 8, 1, [1024, 1024, 37], 2),  # chunks of exactly the ring size, a ragged last chunk, G = 8
])
def test_stack_prompt_then_decode(B, Hq, Hkv, chunks, n_decode):
    n_layers, D = 7, 128  # L L L L L G L
    prompt = sum(chunks)
    N = prompt + n_decode
    interp = 8.0
    layers = []
    for l in range(n_layers):
        q = W.host_normal_bf16((B, N, Hq, D), W.seed_of(CONFIG, l, W.T_Q))
        k = W.host_normal_bf16((B, N, Hkv, D), W.seed_of(CONFIG, l, W.T_K))
        v = W.host_normal_bf16((B, N, Hkv, D), W.seed_of(CONFIG, l, W.T_V))
        gq = W.host_gamma(D, W.seed_of(CONFIG, l, W.T_GQ))
        gk = W.host_gamma(D, W.seed_of(CONFIG, l, W.T_GK))
        layers.append((q, k, v, gq, gk))
    stack = AttentionStack(n_layers, B, Hq, Hkv, max_positions=N + 5, max_chunk=max(chunks),
                           global_interp_scale=interp, q_gammas=[dev_f32(x[3]) for x in layers],
                           k_gammas=[dev_f32(x[4]) for x in layers], eps=W.EPS)
    assert [p.kind for p in stack.plans] == [A.LOCAL] * 5 + [A.GLOBAL, A.LOCAL]
    out = [np.zeros((B, N, Hq, D)) for _ in range(n_layers)]
    s = 0
    for c in chunks:
        for l, (q, k, v, _, _) in enumerate(layers):
            o = stack.prefill_layer(l, dev_bf16(q[:, s:s + c]), dev_bf16(k[:, s:s + c]), dev_bf16(v[:, s:s + c]))
            out[l][:, s:s + c] = host(o)
        stack.advance(c)
        s += c
    for t in range(n_decode):
        p = prompt + t
        for l, (q, k, v, _, _) in enumerate(layers):
            o = stack.decode_layer(l, dev_bf16(q[:, p]), dev_bf16(k[:, p]), dev_bf16(v[:, p]))
            out[l][:, p] = host(o)
        stack.advance(1)
    torch.cuda.synchronize()
    assert stack.pos == N
    for l, (q, k, v, gq, gk) in enumerate(layers):
        plan = stack.plans[l]
        ref = A.prefill(q, k, v, plan.kind, plan.window, plan.rope_base, plan.interp_scale, gq, gk, W.EPS)
        assert_parity(out[l][:, :prompt], ref[:, :prompt], f"layer {l} prompt")
        assert_parity(out[l][:, prompt:], ref[:, prompt:], f"layer {l} decode")
        # the cache ends up holding the last `capacity` positions (all, for a linear cache)
        cap = plan.capacity
        pos = np.arange(max(0, N - cap) if plan.is_ring else 0, N)
        slots = A.ring_slot(pos, cap, plan.is_ring)
        ck, cv = host(stack.caches[l].k), host(stack.caches[l].v)
        for b in range(B):
            assert np.array_equal(cv[b][:, slots, :], v[b][pos].transpose(1, 0, 2)), f"layer {l} cache v"
            kh = A.qknorm_rope(k[b][pos], gk, W.EPS, pos, plan.rope_base, plan.interp_scale, True)
            assert_rowwise_bf16(ck[b][:, slots, :], kh.transpose(1, 0, 2), f"layer {l} cache k")


def test_stack_decode_graph_replays():
    """The decode step of every layer captured once in a HIP graph and
    replayed token after token (inputs refilled and outputs read back with
    eager work and synchronisations between replays) gives the oracle's rows,
    like the eager calls."""
    n_layers, B, Hq, Hkv, D = 7, 1, 4, 2, 128
    prompt, n_decode = 1100, 4  # the ring has wrapped before the first decoded token
    N = prompt + n_decode
    layers = []
    for l in range(n_layers):
        layers.append(tuple(W.host_normal_bf16(shape, W.seed_of(CONFIG + 1, l, t)) for shape, t in
                            [((B, N, Hq, D), W.T_Q), ((B, N, Hkv, D), W.T_K), ((B, N, Hkv, D), W.T_V)]) +
                      (W.host_gamma(D, W.seed_of(CONFIG + 1, l, W.T_GQ)), W.host_gamma(D, W.seed_of(CONFIG + 1, l, W.T_GK))))
    stack = AttentionStack(n_layers, B, Hq, Hkv, max_positions=N, max_chunk=prompt, global_interp_scale=8.0,
                           q_gammas=[dev_f32(x[3]) for x in layers], k_gammas=[dev_f32(x[4]) for x in layers],
                           eps=W.EPS)
    for l, (q, k, v, _, _) in enumerate(layers):
        stack.prefill_layer(l, dev_bf16(q[:, :prompt]), dev_bf16(k[:, :prompt]), dev_bf16(v[:, :prompt]))
    stack.advance(prompt)
    qb = [torch.zeros((B, Hq, D), dtype=torch.bfloat16, device="cuda") for _ in range(n_layers)]
    kb = [torch.zeros((B, Hkv, D), dtype=torch.bfloat16, device="cuda") for _ in range(n_layers)]
    vb = [torch.zeros((B, Hkv, D), dtype=torch.bfloat16, device="cuda") for _ in range(n_layers)]
    ob = [torch.zeros((B, Hq, D), dtype=torch.bfloat16, device="cuda") for _ in range(n_layers)]
    torch.cuda.synchronize()
    step = stack.capture_decode(qb, kb, vb, ob)
    torch.cuda.synchronize()
    assert stack.pos == prompt and int(stack.positions[0]) == prompt  # capture ran nothing
    got = np.zeros((n_layers, B, n_decode, Hq, D))
    for t in range(n_decode):
        p = prompt + t
        for l, (q, k, v, _, _) in enumerate(layers):
            qb[l].copy_(dev_bf16(q[:, p]))
            kb[l].copy_(dev_bf16(k[:, p]))
            vb[l].copy_(dev_bf16(v[:, p]))
        torch.cuda.synchronize()
        step()
        torch.cuda.synchronize()
        for l in range(n_layers):
            got[l, :, t] = host(ob[l])
    assert stack.pos == N and int(stack.positions[0]) == N
    for l, (q, k, v, gq, gk) in enumerate(layers):
        plan = stack.plans[l]
        ref = A.prefill(q, k, v, plan.kind, plan.window, plan.rope_base, plan.interp_scale, gq, gk, W.EPS)
        for t in range(n_decode):
            assert_parity(got[l, :, t], ref[:, prompt + t], f"layer {l} graph replay {t}")


def test_stack_rejects_positions_past_capacity():
    stack = AttentionStack(6, 1, 2, 1, max_positions=100, max_chunk=64)
    x = torch.zeros((1, 64, 2, 128), dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros((1, 64, 1, 128), dtype=torch.bfloat16, device="cuda")
    stack.prefill_layer(0, x, kv, kv)
    stack.advance(64)
    with pytest.raises(ValueError):
        stack.prefill_layer(0, x, kv, kv)  # 64 + 64 > 100
    with pytest.raises(ValueError):
        stack.prefill_layer(0, torch.zeros((1, 65, 2, 128), dtype=torch.bfloat16, device="cuda"), kv, kv)
