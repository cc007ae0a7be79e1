#!/usr/bin/env python3
"""Throughput of the Gemma 3 local/global GQA attention stack on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input,
leg after leg:
  * prefill      : the 27B-shaped block [L,L,L,L,L,G], B=1, S=8192, Hq=32,
                   Hkv=16, D=128 (QK-RMSNorm + RoPE prologue, flash attention);
  * decode       : 32 sequences with 32768 cached positions, one new token
                   each, the same six layers (1024-slot rings for local
                   layers, the full cache for the global one);
  * chunked      : a 4096-query chunk at positions 126976..131071 against a
                   131072-position cache (global, RoPE base 1e6 with position
                   interpolation 8) plus the five local layers;
  * mixed        : B=2, S=4096, Hq=16, Hkv=8, one local and one global layer
                   over sequences with seeded 256-token image spans
                   (bidirectional inside a span);
  * single       : the single attention layer B=1, S=2048, Hq=4, Hkv=2, run as
                   a local and as a global layer (launch-dominated);
  * prefill_1b and decode_1b : the prefill and decode blocks at Gemma 3 1B
                   shapes (Hq=4, Hkv=1, D=256): one 32768-token sequence, and
                   32 sequences with 32767 cached positions;
  * qkv / qkv_1b : the prefill blocks as whole attention sublayers from the
                   layer input (27B: x [8192, 5376]; 1B: x [32768, 1152]): per
                   layer input RMSNorm, the fused q/k/v projection (keys
                   normed and rotated in its epilogue), the flash prefill on
                   those keys, o_proj and the post-attention RMSNorm added to
                   the residual; torch's library GEMM of the same q/k/v
                   projection is timed beside it for context.
Beside the steps, once: the whole 62-layer 27B attention stack (52 local,
10 global) over one 128K sequence, the prompt through chunked prefills of
4096 tokens and then a decode loop, on per-layer caches (``schedule``); and
the oracle timed on the host cores on bounded samples of each workload
(``cpu_baseline``).

`value` is the 27B prefill block's in-window TFLOP/s (4*D flops per visible
(query head, key) pair) over the median of the K timed steps' block times on
the GPU (HIP events on the launch stream); mean, min and max are reported
beside it.  Each leg's main kernel is bracketed by events the library records
on its launch stream inside the same timed steps; the per-leg `roofline`
blocks use their mean durations.  Inputs are seeded synthetic N(0,1) bf16
already resident in HBM.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "prefill attn TFLOP/s (in-window) + decode KV GB/s, 27B shapes, 1 MI355X"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E, published
DEFAULT_LEGS = "prefill,decode,chunked,mixed,single,prefill_1b,decode_1b,qkv,qkv_1b"


def _parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--legs", default=DEFAULT_LEGS)
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle-on-host baseline")
    ap.add_argument("--no-schedule", action="store_true", help="skip the 62-layer 128K schedule run")
    ap.add_argument("--no-probes", action="store_true", help="skip the measured MFMA / HBM ceilings")
    ap.add_argument("--kernel-events", choices=("timed", "separate"), default="timed",
                    help="record the per-kernel events inside the timed steps (default) or in steps of their own")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="also run one device copy of this many MiB (HBM counter calibration)")
    return ap.parse_args()


class Leg:
    """Inputs, outputs and workspaces of one leg, all resident in HBM."""

    def __init__(self, name):
        self.name = name
        self.calls = []        # callables, one per layer
        self.work = []         # algorithmic flops or bytes per layer
        self.kinds = []        # layer kind per layer
        self.unit = ""
        self.inputs = []       # per-layer device tensors, for the host baseline
        self.per_kernel = False


def _events(torch, n):
    evs = []
    for _ in range(n):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        b.record()
        evs.append((a, b))
    return evs


def _kind_params(G, W, kind):
    return (W.ROPE_BASE_GLOBAL, 1.0) if kind == G.GLOBAL else (W.ROPE_BASE_LOCAL, 1.0)


def build_prefill_leg(torch, G, W, C, cfg=2, name="prefill"):
    """A self-contained prefill over the workload's layers (config 1: local
    then global; config 2 and the 1B block: L,L,L,L,L,G; config 5: local
    then global over sequences with image spans)."""
    w = W.WORKLOADS[cfg]
    c = w.config
    leg = Leg(name)
    leg.unit = "flop"
    leg.workload = w
    spans = W.workload_spans(w)
    leg.spans = spans
    flat = None if spans is None else [(b, s, e) for b in range(w.B) for (s, e) in spans[b]]
    for l, kname in enumerate(w.kinds):
        kind = G.GLOBAL if kname == "global" else G.LOCAL
        base, scale = _kind_params(G, W, kind)
        q = W.device_normal_bf16((w.B, w.S, w.Hq, w.D), W.seed_of(c, l, W.T_Q))
        k = W.device_normal_bf16((w.B, w.S, w.Hkv, w.D), W.seed_of(c, l, W.T_K))
        v = W.device_normal_bf16((w.B, w.S, w.Hkv, w.D), W.seed_of(c, l, W.T_V))
        gq = torch.from_numpy(W.host_gamma(w.D, W.seed_of(c, l, W.T_GQ))).cuda()
        gk = torch.from_numpy(W.host_gamma(w.D, W.seed_of(c, l, W.T_GK))).cuda()
        o = torch.empty_like(q)
        ws = torch.empty(G.prefill_workspace_size(w.B, w.S, w.Hq, w.Hkv, w.D), dtype=torch.uint8, device="cuda")
        leg.inputs.append(dict(q=q, k=k, v=v, gq=gq, gk=gk, kind=kind, base=base, scale=scale))

        def call(q=q, k=k, v=v, gq=gq, gk=gk, o=o, ws=ws, kind=kind, base=base, scale=scale):
            G.prefill(q, k, v, kind, W.WINDOW, base, scale, gq, gk, W.EPS, 0.0, flat, None, None, o=o, workspace=ws)
        leg.calls.append(call)
        leg.kinds.append(kind)
        leg.work.append(C.prefill_flops(w.B, w.S, w.Hq, w.D, kind == G.LOCAL, W.WINDOW, spans=spans))
    return leg


def build_decode_leg(torch, G, W, C, cfg=3, name="decode"):
    w = W.WORKLOADS[cfg]
    c = w.config
    leg = Leg(name)
    leg.unit = "byte"
    leg.workload = w
    p = w.pos0
    positions = torch.full((w.B,), p, dtype=torch.int32, device="cuda")
    for l in range(len(w.kinds)):
        kind = G.layer_kind(l)
        base, scale = _kind_params(G, W, kind)
        cap = W.RING_CAP if kind == G.LOCAL else p + 64  # global: positions 0..p (p+1 slots), padded
        ck = W.device_normal_bf16((w.B, w.Hkv, cap, w.D), W.seed_of(c, l, W.T_CK))
        cv = W.device_normal_bf16((w.B, w.Hkv, cap, w.D), W.seed_of(c, l, W.T_CV))
        cache = G.KVCache(ck, cv, is_ring=(kind == G.LOCAL))
        q = W.device_normal_bf16((w.B, w.Hq, w.D), W.seed_of(c, l, W.T_Q))
        kn = W.device_normal_bf16((w.B, w.Hkv, w.D), W.seed_of(c, l, W.T_K))
        vn = W.device_normal_bf16((w.B, w.Hkv, w.D), W.seed_of(c, l, W.T_V))
        gq = torch.from_numpy(W.host_gamma(w.D, W.seed_of(c, l, W.T_GQ))).cuda()
        gk = torch.from_numpy(W.host_gamma(w.D, W.seed_of(c, l, W.T_GK))).cuda()
        o = torch.empty_like(q)
        ws = torch.empty(G.decode_workspace_size(w.B, w.Hq, w.Hkv, w.D, p, cache), dtype=torch.uint8, device="cuda")
        leg.inputs.append(dict(q=q, kn=kn, vn=vn, ck=ck, cv=cv, gq=gq, gk=gk, kind=kind, base=base, scale=scale,
                               ring=kind == G.LOCAL, p=p))

        def call(q=q, kn=kn, vn=vn, cache=cache, gq=gq, gk=gk, o=o, ws=ws, kind=kind, base=base):
            G.decode(q, kn, vn, positions, p, cache, kind, W.WINDOW, base, 1.0, gq, gk, W.EPS, 0.0, o=o, workspace=ws)
        leg.calls.append(call)
        leg.kinds.append(kind)
        leg.work.append(C.decode_bytes(w.B, w.Hq, w.Hkv, w.D, [p] * w.B, kind == G.LOCAL, W.WINDOW))
    return leg


def build_chunked_leg(torch, G, W, C):
    w = W.WORKLOADS[4]
    leg = Leg("chunked")
    leg.unit = "flop"
    leg.workload = w
    leg.spans = None
    p0 = w.pos0
    for l in range(len(w.kinds)):
        kind = G.layer_kind(l)
        if kind == G.GLOBAL:
            base, scale, cap, ring = W.ROPE_BASE_GLOBAL, w.interp_scale_global, p0 + w.S, False
        else:
            base, scale, cap, ring = W.ROPE_BASE_LOCAL, 1.0, W.RING_CAP, True
        ck = W.device_normal_bf16((w.B, w.Hkv, cap, w.D), W.seed_of(4, l, W.T_CK))
        cv = W.device_normal_bf16((w.B, w.Hkv, cap, w.D), W.seed_of(4, l, W.T_CV))
        cache = G.KVCache(ck, cv, is_ring=ring)
        q = W.device_normal_bf16((w.B, w.S, w.Hq, w.D), W.seed_of(4, l, W.T_Q))
        k = W.device_normal_bf16((w.B, w.S, w.Hkv, w.D), W.seed_of(4, l, W.T_K))
        v = W.device_normal_bf16((w.B, w.S, w.Hkv, w.D), W.seed_of(4, l, W.T_V))
        gq = torch.from_numpy(W.host_gamma(w.D, W.seed_of(4, l, W.T_GQ))).cuda()
        gk = torch.from_numpy(W.host_gamma(w.D, W.seed_of(4, l, W.T_GK))).cuda()
        o = torch.empty_like(q)
        ws = torch.empty(G.prefill_workspace_size(w.B, w.S, w.Hq, w.Hkv, w.D), dtype=torch.uint8, device="cuda")
        leg.inputs.append(dict(q=q, k=k, v=v, ck=ck, cv=cv, gq=gq, gk=gk, kind=kind, base=base, scale=scale,
                               ring=ring, p0=p0))

        def call(q=q, k=k, v=v, cache=cache, gq=gq, gk=gk, o=o, ws=ws, kind=kind, base=base, scale=scale):
            G.prefill(q, k, v, kind, W.WINDOW, base, scale, gq, gk, W.EPS, 0.0, None, [p0], cache, o=o,
                      workspace=ws)
        leg.calls.append(call)
        leg.kinds.append(kind)
        leg.work.append(C.prefill_flops(w.B, w.S, w.Hq, w.D, kind == G.LOCAL, W.WINDOW, pos0=[p0], has_cache=True,
                                        ring_capacity=W.RING_CAP if ring else None))
    return leg


def build_qkv_leg(torch, G, W, C, cfg=2, name="qkv", dm=None):
    w = W.WORKLOADS[cfg]
    c = w.config
    dm = W.D_MODEL_27B if dm is None else dm
    leg = Leg(name)
    leg.d_model = dm
    leg.unit = "flop"
    leg.workload = w
    leg.gemm = []
    n = len(w.kinds)
    leg.oev = []
    leg.owork = []
    for l in range(n):
        kind = G.layer_kind(l)
        base, _ = _kind_params(G, W, kind)
        x = W.device_normal_bf16((w.B, w.S, dm), W.seed_of(c, l, W.T_X))
        wt = W.device_normal_bf16(((w.Hq + 2 * w.Hkv) * w.D, dm), W.seed_of(c, l, W.T_W), std=dm ** -0.5)
        gq = torch.from_numpy(W.host_gamma(w.D, W.seed_of(c, l, W.T_GQ))).cuda()
        gk = torch.from_numpy(W.host_gamma(w.D, W.seed_of(c, l, W.T_GK))).cuda()
        q = torch.empty((w.B, w.S, w.Hq, w.D), dtype=torch.bfloat16, device="cuda")
        kh = torch.empty((w.B, w.Hkv, w.S, w.D), dtype=torch.bfloat16, device="cuda")
        v = torch.empty((w.B, w.S, w.Hkv, w.D), dtype=torch.bfloat16, device="cuda")
        o = torch.empty_like(q)
        ws = torch.empty(G.prefill_workspace_size(w.B, w.S, w.Hq, w.Hkv, w.D), dtype=torch.uint8, device="cuda")
        y = torch.empty((w.B * w.S, wt.shape[0]), dtype=torch.bfloat16, device="cuda")
        wo = W.device_normal_bf16((dm, w.Hq * w.D), W.seed_of(c, l, W.T_CK), std=(w.Hq * w.D) ** -0.5)
        gi = torch.from_numpy(W.host_gamma(dm, W.seed_of(c, l, W.T_CV))).cuda()
        gp = torch.from_numpy(W.host_gamma(dm, W.seed_of(c, l, W.T_SPANS))).cuda()
        # the input norm's gamma folded into the projection weights once (load time)
        wf = G.fold_norm_weight(wt, gi)
        xs = torch.empty((w.B, w.S), dtype=torch.float32, device="cuda")
        yo = torch.empty_like(x)
        xo = torch.empty_like(x)

        def call(x=x, wf=wf, xs=xs, gq=gq, gk=gk, q=q, kh=kh, v=v, o=o, ws=ws, kind=kind, base=base, wo=wo, gp=gp,
                 yo=yo, xo=xo, l=l):
            G.rms_scale(x, W.EPS, scale=xs)
            G.qkv_project(x, wf, w.Hq, w.Hkv, base, 1.0, gk, W.EPS, None, q=q, khat=kh, v=v, x_scale=xs)
            if leg.per_kernel:
                G.set_timing_events(None, None)  # the projection kernel only
            G.prefill_khat(q, kh, v, kind, W.WINDOW, base, 1.0, gq, W.EPS, 0.0, None, None, None, o=o, workspace=ws)
            if leg.per_kernel:
                G.set_timing_events(*leg.oev[l])
            G.o_project(o, wo, y=yo)
            if leg.per_kernel:
                G.set_timing_events(None, None)
            G.rmsnorm(yo, gp, W.EPS, residual=x, out=xo)

        def gemm(x=x, wt=wt, y=y):
            torch.mm(x.view(w.B * w.S, dm), wt.t(), out=y)  # 2-D GEMM, y = x W^T
        leg.calls.append(call)
        leg.kinds.append(kind)
        leg.gemm.append(gemm)
        leg.work.append(2.0 * w.B * w.S * dm * (w.Hq + 2 * w.Hkv) * w.D)
        leg.owork.append(2.0 * w.B * w.S * w.Hq * w.D * dm)
    return leg


def run_leg(torch, G, leg, step_ev, kernel_ev):
    """Launch the leg's layers.  step_ev: events bracketing the whole leg (or
    None); kernel_ev: per layer, events the library records around the
    layer's main kernel on its launch stream (or None)."""
    if step_ev is not None:
        step_ev[0].record()
    leg.per_kernel = kernel_ev is not None
    for l, call in enumerate(leg.calls):
        if kernel_ev is not None:
            G.set_timing_events(*kernel_ev[l])
        call()
    if kernel_ev is not None:
        G.set_timing_events(None, None)
    if step_ev is not None:
        step_ev[1].record()


def graph_replay_ms(torch, leg, K):
    """The leg's layer calls captured once into a HIP graph (on a side
    stream) and replayed K times: per-replay block times in ms.  This is the
    form a serving loop runs decode in; it leaves out the host's per-call
    argument marshalling, which for short layers takes longer than the GPU
    work and so sets the pace of eager calls."""
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            for call in leg.calls:
                call()
    torch.cuda.current_stream().wait_stream(side)
    g.replay()
    torch.cuda.synchronize()
    ev = _events(torch, K)
    for s in range(K):
        ev[s][0].record()
        g.replay()
        ev[s][1].record()
    torch.cuda.synchronize()
    return [e[0].elapsed_time(e[1]) for e in ev]


def run_schedule(torch, G, W, C, n_layers=62, total=131072, chunk=4096, n_decode=32):
    """One 128K sequence through the whole 27B attention stack: a prompt of
    total - n_decode tokens in chunks, then n_decode decode steps (the last at
    position total - 1).  Synthetic raw q/k/v, two sets alternating by layer;
    each layer's cache is written by its own calls."""
    from global_gqa_amd.schedule import AttentionStack, chunk_bounds

    w = W.WORKLOADS[2]
    Hq, Hkv, D = w.Hq, w.Hkv, w.D
    stack = AttentionStack(n_layers, 1, Hq, Hkv, max_positions=total, max_chunk=chunk, D=D, window=W.WINDOW,
                           global_interp_scale=8.0, eps=W.EPS)
    pre = [(W.device_normal_bf16((1, chunk, Hq, D), W.seed_of(6, i, W.T_Q)),
            W.device_normal_bf16((1, chunk, Hkv, D), W.seed_of(6, i, W.T_K)),
            W.device_normal_bf16((1, chunk, Hkv, D), W.seed_of(6, i, W.T_V))) for i in range(2)]
    dec = [(W.device_normal_bf16((1, Hq, D), W.seed_of(6, 10 + i, W.T_Q)),
            W.device_normal_bf16((1, Hkv, D), W.seed_of(6, 10 + i, W.T_K)),
            W.device_normal_bf16((1, Hkv, D), W.seed_of(6, 10 + i, W.T_V))) for i in range(2)]
    o_pre = torch.empty_like(pre[0][0])
    o_dec = torch.empty_like(dec[0][0])
    prompt = total - n_decode
    bounds = chunk_bounds(prompt, chunk)
    flops = 0.0
    for (s0, e0) in bounds:
        for p in stack.plans:
            flops += C.prefill_flops(1, e0 - s0, Hq, D, p.kind == G.LOCAL, p.window, pos0=[s0], has_cache=True,
                                     ring_capacity=p.capacity if p.is_ring else None)
    nbytes_tok = [sum(C.decode_bytes(1, Hq, Hkv, D, [prompt + t], p.kind == G.LOCAL, p.window) for p in stack.plans)
                  for t in range(n_decode)]
    n_eager = n_decode // 4
    ev = _events(torch, 4)
    torch.cuda.synchronize()
    ev[0][0].record()
    for (s0, e0) in bounds:
        n = e0 - s0
        for i in range(n_layers):
            q, k, v = pre[i & 1]
            stack.prefill_layer(i, q[:, :n], k[:, :n], v[:, :n], o=o_pre[:, :n])
        stack.advance(n)
    ev[0][1].record()
    # decode: the first tokens with eager calls, the rest by replaying one
    # captured graph of the 62 layers' calls (a serving loop's form)
    for t in range(n_eager):
        for i in range(n_layers):
            q, k, v = dec[i & 1]
            stack.decode_layer(i, q, k, v, o=o_dec)
        stack.advance(1)
    ev[1][1].record()
    torch.cuda.synchronize()
    step = stack.capture_decode([dec[i & 1][0] for i in range(n_layers)], [dec[i & 1][1] for i in range(n_layers)],
                                [dec[i & 1][2] for i in range(n_layers)], [o_dec] * n_layers)
    torch.cuda.synchronize()
    ev[2][0].record()
    for t in range(n_decode - n_eager):
        step()
    ev[2][1].record()
    torch.cuda.synchronize()
    ms_pre = ev[0][0].elapsed_time(ev[0][1])
    ms_eager = ev[0][1].elapsed_time(ev[1][1])
    ms_graph = ev[2][0].elapsed_time(ev[2][1])
    b_eager = sum(nbytes_tok[:n_eager])
    b_graph = sum(nbytes_tok[n_eager:])
    return {"workload": f"27b-{n_layers}-layer-128k: prompt {prompt} tokens in chunks of {chunk}, then "
                        f"{n_decode} decode steps (positions {prompt}..{total - 1}), B=1",
            "layers": n_layers, "global_layers": sum(p.kind == G.GLOBAL for p in stack.plans),
            "prompt_ms": ms_pre, "prompt_in_window_flop": flops, "prompt_TFLOPs": flops / (ms_pre * 1e-3) / 1e12,
            "decode_ms_per_token": ms_graph / (n_decode - n_eager),
            "decode_GBs": b_graph / (ms_graph * 1e-3) / 1e9,
            "decode_eager_ms_per_token": ms_eager / n_eager,
            "decode_eager_GBs": b_eager / (ms_eager * 1e-3) / 1e9,
            "decode_bytes_per_token": b_graph / (n_decode - n_eager)}


# ---------------------------------------------------------------- host baseline
def _blas_threads():
    try:
        from threadpoolctl import threadpool_info

        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        return os.cpu_count() or 1


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform

    return platform.processor() or "unknown"


def _h(t):
    """Device tensor slice -> host float32 array."""
    return t.float().cpu().numpy()


def cpu_baseline(torch, G, W, C, by):
    """The oracle as it stands (NumPy float64, BLAS threads as configured),
    timed on the host cores on bounded samples of each workload whose leg
    ran; the same inputs the GPU legs use (copied back from HBM).  Returns
    the 27B prefill block's sample as `value`, and per workload and layer
    wall times with their rates."""
    import oracle.attention as A

    kname = {G.LOCAL: "local", G.GLOBAL: "global"}
    threads = _blas_threads()
    per = {}

    def timed(fn):
        t0 = time.perf_counter()
        fn()
        return time.perf_counter() - t0

    def prefill_sample(leg, hq, hkv, label):
        w = leg.workload
        rows = []
        for x in leg.inputs:
            q, k, v = _h(x["q"][:, :, 0:hq]), _h(x["k"][:, :, 0:hkv]), _h(x["v"][:, :, 0:hkv])
            gq, gk = _h(x["gq"]), _h(x["gk"])
            t = timed(lambda: A.prefill(q, k, v, x["kind"], W.WINDOW, x["base"], x["scale"], gq, gk, W.EPS,
                                        spans=leg.spans))
            fl = C.prefill_flops(w.B, w.S, hq, w.D, x["kind"] == G.LOCAL, W.WINDOW, spans=leg.spans)
            rows.append({"layer": kname[x["kind"]], "s": t, "flop": fl, "TFLOPs": fl / t / 1e12})
        tot_f, tot_t = sum(r["flop"] for r in rows), sum(r["s"] for r in rows)
        return {"unit": "TFLOP/s", "value": tot_f / tot_t / 1e12, "s": tot_t, "sample": label, "layers": rows}

    if "single" in by:
        leg = by["single"]
        w = leg.workload
        per["single"] = prefill_sample(leg, w.Hq, w.Hkv, f"the whole workload (B={w.B}, S={w.S}, Hq={w.Hq}, "
                                       f"Hkv={w.Hkv}), local and global layer")
        try:
            from threadpoolctl import threadpool_limits

            with threadpool_limits(limits=1):
                one = prefill_sample(leg, w.Hq, w.Hkv, "the same, one BLAS thread")
            per["single"]["one_thread"] = one
        except Exception as e:  # pragma: no cover
            per["single"]["one_thread"] = {"error": str(e)}
    if "prefill" in by:
        per["prefill"] = prefill_sample(by["prefill"], 2, 1, "query heads 0-1 / kv head 0 of each of the 6 layers, "
                                                             "all 8192 rows")
    if "mixed" in by:
        per["mixed"] = prefill_sample(by["mixed"], 2, 1, "query heads 0-1 / kv head 0 of both layers, both "
                                                         "sequences (with their image spans), all rows")
    if "decode" in by:
        leg = by["decode"]
        w = leg.workload
        rows = []
        nb = 4
        for x in leg.inputs:
            q, kn, vn = _h(x["q"][0:nb, 0:2]), _h(x["kn"][0:nb, 0:1]), _h(x["vn"][0:nb, 0:1])
            ck, cv = _h(x["ck"][0:nb, 0:1]), _h(x["cv"][0:nb, 0:1])
            gq, gk = _h(x["gq"]), _h(x["gk"])
            pos = [x["p"]] * nb
            t = timed(lambda: A.decode(q, kn, vn, ck, cv, x["ring"], pos, x["kind"], W.WINDOW, x["base"], 1.0, gq, gk,
                                       W.EPS))
            nbytes = C.decode_bytes(nb, 2, 1, w.D, pos, x["kind"] == G.LOCAL, W.WINDOW)
            rows.append({"layer": kname[x["kind"]], "s": t, "bytes": nbytes, "GBs": nbytes / t / 1e9})
        tb, tt = sum(r["bytes"] for r in rows), sum(r["s"] for r in rows)
        per["decode"] = {"unit": "GB/s", "value": tb / tt / 1e9, "s": tt, "layers": rows,
                         "sample": f"sequences 0-{nb - 1}, kv head 0 (query heads 0-1) of each of the 6 layers"}
    if "chunked" in by:
        leg = by["chunked"]
        w = leg.workload
        n_rows = 512
        rows = []
        for l in (0, 5):  # one local layer and the global layer
            x = leg.inputs[l]
            q, k, v = _h(x["q"][:, :n_rows, 0:2]), _h(x["k"][:, :n_rows, 0:1]), _h(x["v"][:, :n_rows, 0:1])
            ck, cv = _h(x["ck"][:, 0:1]), _h(x["cv"][:, 0:1])
            gq, gk = _h(x["gq"]), _h(x["gk"])
            t = timed(lambda: A.prefill_chunk(q, k, v, ck, cv, x["ring"], x["kind"], W.WINDOW, x["base"], x["scale"],
                                              gq, gk, W.EPS, pos0=[x["p0"]]))
            fl = C.prefill_flops(1, n_rows, 2, w.D, x["kind"] == G.LOCAL, W.WINDOW, pos0=[x["p0"]], has_cache=True,
                                 ring_capacity=W.RING_CAP if x["ring"] else None)
            rows.append({"layer": kname[x["kind"]], "s": t, "flop": fl, "TFLOPs": fl / t / 1e12})
        tf, tt = sum(r["flop"] for r in rows), sum(r["s"] for r in rows)
        per["chunked"] = {"unit": "TFLOP/s", "value": tf / tt / 1e12, "s": tt, "layers": rows,
                          "sample": f"the first {n_rows} query rows of the chunk (they see the same keys as in the "
                                    "whole chunk), query heads 0-1 / kv head 0, layer 0 (local) and 5 (global)"}
    head = per.get("prefill")
    return {"value": None if head is None else head["value"], "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": None if head is None else
            f"27B prefill block: {head['sample']} (in-window {sum(r['flop'] for r in head['layers']):.4g} flop in "
            f"{head['s']:.2f} s, NumPy float64)",
            "cpu_model": _cpu_model(), "nproc": os.cpu_count(), "blas_threads": int(threads),
            "per_workload": per}


# ---------------------------------------------------------------- summaries
def _src_hash(name):
    p = os.path.join(ROOT, "global_gqa_amd", "csrc", name)
    return hashlib.sha256(open(p, "rb").read()).hexdigest()[:16]


def _traffic(kernel_src, key):
    """Measured HBM bytes per launch from the committed counter summary, if
    it was taken on the current kernel source; else None."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        t = json.load(open(p))
        e = t[key]
        if e.get("source_sha256_16") != _src_hash(kernel_src):
            return None
        return float(e["hbm_bytes_per_launch"])
    except Exception:
        return None


def _stats(xs):
    return {"median": statistics.median(xs), "mean": statistics.fmean(xs), "min": min(xs), "max": max(xs)}


def measured_ceilings():
    """The roofline probes' measured ceilings on this card: dense bf16 MFMA
    (32x32x16 chains in every wave, 2 waves per SIMD) with the shader clock it
    ran at, and the HBM read rate over 2 GiB."""
    from global_gqa_amd import probes

    m = probes.mfma_ceiling()
    h = probes.hbm_read_ceiling()
    return {"mfma_bf16": {"tflops": m["tflops"], "frac_of_published": m["tflops"] / PEAK_BF16_TFLOPS,
                          "clock_ghz": m["clock_ghz"], "what": "v_mfma_f32_32x32x16_bf16 chains only, "
                          f"{m['workgroups']} workgroups x 4 waves, {m['mfma_per_wave']} MFMAs per wave, best of 5"},
            "hbm_read": {"gbps": h["gbps"], "frac_of_published": h["gbps"] / PEAK_HBM_GBPS,
                         "what": f"16-byte non-temporal loads over {h['bytes'] >> 20} MiB, best of 5 per pattern, "
                                 f"best pattern: {h['best']['pattern']} x {h['best']['workgroups']} workgroups",
                         "runs": h["runs"]}}


def add_ceiling_fractions(node, ceil):
    """Every roofline block also states its rate against the measured
    ceiling of its bound (the published peak stays its `peak`)."""
    if isinstance(node, dict):
        r = node.get("roofline")
        if isinstance(r, dict) and r.get("achieved") is not None:
            c = ceil["mfma_bf16"]["tflops"] if r.get("bound") == "mfma" else ceil["hbm_read"]["gbps"]
            r["ceiling_measured"] = c
            r["frac_of_ceiling"] = r["achieved"] / c
        for k, v in node.items():
            if k != "roofline":
                add_ceiling_fractions(v, ceil)


def main():
    args = _parse()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); "
              "multi-GPU sharding is described in the design notes but not built.", file=sys.stderr)
        sys.exit(2)
    import torch

    import global_gqa_amd as G
    import workloads as W
    from global_gqa_amd import counting as C

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    G.lib()
    torch.cuda.set_device(0)
    legs = []
    names = [s for s in args.legs.split(",") if s]
    builders = {"prefill": build_prefill_leg, "decode": build_decode_leg, "chunked": build_chunked_leg,
                "mixed": lambda *a: build_prefill_leg(*a, cfg=5, name="mixed"),
                "single": lambda *a: build_prefill_leg(*a, cfg=1, name="single"),
                "prefill_1b": lambda *a: build_prefill_leg(*a, cfg=9, name="prefill_1b"),
                "decode_1b": lambda *a: build_decode_leg(*a, cfg=10, name="decode_1b"), "qkv": build_qkv_leg,
                "qkv_1b": lambda *a: build_qkv_leg(*a, cfg=9, name="qkv_1b", dm=W.D_MODEL_1B)}
    for n in names:
        leg = builders[n](torch, G, W, C)
        n_l = len(leg.calls)
        leg.step_ev = [_events(torch, 1)[0] for _ in range(max(args.steps, 1))]
        leg.kern_ev = [_events(torch, n_l) for _ in range(max(args.steps, 3))]
        if hasattr(leg, "oev"):
            leg.oev_steps = [_events(torch, n_l) for _ in range(max(args.steps, 3))]
        legs.append(leg)
        print(f"[bench] built leg {n}", file=sys.stderr, flush=True)
    torch.cuda.synchronize()

    for s in range(args.warmup):
        for leg in legs:
            run_leg(torch, G, leg, None, None)
    torch.cuda.synchronize()
    print(f"[bench] warmup {args.warmup} done", file=sys.stderr, flush=True)

    K = max(args.steps, 1)
    in_steps = args.kernel_events == "timed"
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        for leg in legs:
            if hasattr(leg, "oev_steps"):
                leg.oev = leg.oev_steps[s]
            run_leg(torch, G, leg, leg.step_ev[s], leg.kern_ev[s] if in_steps else None)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    print(f"[bench] timed {args.steps} steps in {wall:.2f} s", file=sys.stderr, flush=True)
    KK = K if in_steps else max(3, args.steps // 2)
    if not in_steps:
        for s in range(KK):
            for leg in legs:
                if hasattr(leg, "oev_steps"):
                    leg.oev = leg.oev_steps[s]
                run_leg(torch, G, leg, None, leg.kern_ev[s])
        torch.cuda.synchronize()
        print(f"[bench] {KK} steps of per-kernel timing done", file=sys.stderr, flush=True)
    step_ms = {leg.name: [leg.step_ev[s][0].elapsed_time(leg.step_ev[s][1]) for s in range(K)] for leg in legs}
    kern_ms = {leg.name: [sum(leg.kern_ev[s][l][0].elapsed_time(leg.kern_ev[s][l][1]) for s in range(KK)) / KK
                          for l in range(len(leg.calls))] for leg in legs}
    o_ms = {leg.name: [sum(leg.oev_steps[s][l][0].elapsed_time(leg.oev_steps[s][l][1]) for s in range(KK)) / KK
                       for l in range(len(leg.calls))] for leg in legs if hasattr(leg, "oev_steps")}
    graph_ms = {}
    for leg in legs:
        if leg.unit == "byte":
            graph_ms[leg.name] = graph_replay_ms(torch, leg, K)
    if graph_ms:
        print(f"[bench] graph replay of {sorted(graph_ms)} done", file=sys.stderr, flush=True)
    gemm_ms = None
    if any(leg.name == "qkv" for leg in legs):  # the library GEMM beside the 27B projection
        leg = [x for x in legs if x.name == "qkv"][0]
        for g in leg.gemm:
            g()
        ev = _events(torch, 1)[0]
        torch.cuda.synchronize()
        ev[0].record()
        for s in range(KK):
            for g in leg.gemm:
                g()
        ev[1].record()
        torch.cuda.synchronize()
        gemm_ms = ev[0].elapsed_time(ev[1]) / (KK * len(leg.gemm))

    if args.calibrate_copy_mib:
        n = args.calibrate_copy_mib << 20
        a = torch.empty(n, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()

    out = {"metric": METRIC, "value": None, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": wall * 1e3 / K, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded N(0,1) bf16, random-init, in HBM)"}
    by = {leg.name: leg for leg in legs}
    kernel_timing = ("events around each main kernel, recorded by the library on its launch stream inside the "
                     "timed steps" if in_steps else "events around each main kernel in separate steps")

    def prefill_summary(leg, traffic_key):
        w = leg.workload
        st = _stats(step_ms[leg.name])
        flops = sum(leg.work)
        kms = kern_ms[leg.name]
        achieved = flops / (sum(kms) * 1e-3) / 1e12
        cfg = {"workload": w.name, "B": w.B, "S": w.S, "Hq": w.Hq, "Hkv": w.Hkv, "D": w.D,
               "layers": "".join("G" if k == G.GLOBAL else "L" for k in leg.kinds), "window": W.WINDOW,
               "rope_base": [W.ROPE_BASE_LOCAL, W.ROPE_BASE_GLOBAL], "in_window_flop": flops,
               "block_ms": st}
        if w.mode == "chunked":
            cfg.update(pos0=w.pos0, cache_positions=w.pos0, interp_scale_global=w.interp_scale_global)
        if leg.spans is not None:
            cfg["image_spans"] = leg.spans
        kern = "prefill_fwd" if w.D == 128 else "prefill_fwd_d256"
        src = "prefill.hip" if w.D == 128 else "prefill_d256.hip"
        roof = {"bound": "mfma", "kernel": kern, "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / PEAK_BF16_TFLOPS, "traffic": _traffic(src, traffic_key),
                "launch_ms": kms, "launch_flop": leg.work, "timing": kernel_timing}
        return flops / (st["median"] * 1e-3) / 1e12, cfg, roof

    def decode_summary(leg, traffic_key):
        w = leg.workload
        st = _stats(step_ms[leg.name])
        nbytes = sum(leg.work)
        kms = kern_ms[leg.name]
        # split-K kernel: KV bytes only (q/o/new rows are handled around it)
        kv_bytes = [b - 2.0 * w.D * (2 * w.B * w.Hq + 2 * w.B * w.Hkv) for b in leg.work]
        ach = sum(kv_bytes) / (sum(kms) * 1e-3) / 1e9
        v = nbytes / (st["median"] * 1e-3) / 1e9
        gst = _stats(graph_ms[leg.name])
        gv = nbytes / (gst["median"] * 1e-3) / 1e9
        return {"value": v, "unit": "GB/s", "workload": w.name, "block_ms": st, "bytes_per_block": nbytes,
                "frac_hbm": v / PEAK_HBM_GBPS,
                "graph_replay": {"value": gv, "unit": "GB/s", "frac_hbm": gv / PEAK_HBM_GBPS, "block_ms": gst,
                                 "what": "the same block's calls captured once into a HIP graph and replayed "
                                         "(median of K replays); value above: eager calls from Python"},
                "roofline": {"bound": "hbm", "kernel": "decode_splitk", "achieved": ach, "peak": PEAK_HBM_GBPS,
                             "unit": "GB/s", "frac": ach / PEAK_HBM_GBPS,
                             "traffic": _traffic("decode.hip", traffic_key), "launch_ms": kms,
                             "launch_kv_bytes": kv_bytes, "timing": kernel_timing}}

    def prefill_leg_entry(name, key):
        v, cfg, roof = prefill_summary(by[name], key)
        return {"value": v, "unit": "TFLOP/s", "config": cfg, "roofline": roof}

    if "prefill" in by:
        out["value"], out["config"], out["roofline"] = prefill_summary(by["prefill"], "prefill")
        out["timing"] = {"value": "in-window flop of the block / median of the K steps' block times (HIP events)",
                         "block_ms": out["config"]["block_ms"]}
    if "decode" in by:
        out["decode"] = decode_summary(by["decode"], "decode")
    if "chunked" in by:
        out["chunked_prefill"] = prefill_leg_entry("chunked", "chunked")
    if "mixed" in by:
        out["mixed_mask"] = prefill_leg_entry("mixed", "mixed")
    if "single" in by:
        out["single_layer"] = prefill_leg_entry("single", "single")
    if "prefill_1b" in by or "decode_1b" in by:
        g1 = {}
        if "prefill_1b" in by:
            g1["prefill"] = prefill_leg_entry("prefill_1b", "prefill_1b")
        if "decode_1b" in by:
            g1["decode"] = decode_summary(by["decode_1b"], "decode_1b")
        out["gemma3_1b"] = g1

    def qkv_summary(leg, tag):
        w = leg.workload
        st = _stats(step_ms[leg.name])
        kms = kern_ms[leg.name]
        ach = sum(leg.work) / (sum(kms) * 1e-3) / 1e12
        oms = o_ms[leg.name]
        o_ach = sum(leg.owork) / (sum(oms) * 1e-3) / 1e12
        return {
            "value": ach, "unit": "TFLOP/s", "workload": w.name + " from the layer input",
            "d_model": leg.d_model, "tokens": w.B * w.S, "heads": [w.Hq, w.Hkv, w.Hkv], "D": w.D,
            "block_ms": st, "block": "per layer: the input RMSNorm's per-token scale (its gamma folded into the "
                                     "projection weights once, before the timed steps), the fused q/k/v "
                                     "projection applying that scale, prefill on the projected keys, o_proj, "
                                     "post-attention RMSNorm added to the residual",
            "projection_flop_per_layer": leg.work[0],
            "roofline": {"bound": "mfma", "kernel": "qkv_proj", "achieved": ach, "peak": PEAK_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": ach / PEAK_BF16_TFLOPS,
                         "traffic": _traffic("qkv_proj.hip", f"{leg.name}/qkv_proj"), "launch_ms": kms},
            "o_proj": {"value": o_ach, "unit": "TFLOP/s", "kernel": "qkv_proj (no key/value heads)",
                       "flop_per_layer": leg.owork[0], "frac": o_ach / PEAK_BF16_TFLOPS,
                       "traffic": _traffic("qkv_proj.hip", f"{leg.name}/o_proj"), "launch_ms": oms}}

    if "qkv" in by:
        leg = by["qkv"]
        out["fused_qkv"] = qkv_summary(leg, "27b")
        out["fused_qkv"]["library_gemm"] = None if gemm_ms is None else {
            "what": "torch.mm (library GEMM) of the same projection into one [tokens, 8192] output, "
                    "without the key norm and rotation",
            "ms": gemm_ms, "TFLOPs": leg.work[0] / (gemm_ms * 1e-3) / 1e12}
    if "qkv_1b" in by:
        out.setdefault("gemma3_1b", {})["fused_qkv"] = qkv_summary(by["qkv_1b"], "1b")
    if out["value"] is None:
        out["value"] = 0.0
    if not args.no_probes:
        print("[bench] roofline probes...", file=sys.stderr, flush=True)
        out["ceilings"] = measured_ceilings()
        add_ceiling_fractions(out, out["ceilings"])
    if not args.no_schedule:
        print("[bench] 62-layer 128K schedule...", file=sys.stderr, flush=True)
        out["schedule_27b_128k"] = run_schedule(torch, G, W, C)
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle on host)...", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(torch, G, W, C, by)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out))


if __name__ == "__main__":
    main()
