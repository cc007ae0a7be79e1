#!/usr/bin/env python3
"""Throughput of the Gemma 3 local/global GQA attention stack on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input:
  * prefill leg  : the 27B-shaped block [L,L,L,L,L,G], B=1, S=8192, Hq=32,
                   Hkv=16, D=128 (QK-RMSNorm + RoPE prologue, flash attention);
  * decode leg   : 32 sequences with 32768 cached positions, one new token
                   each, the same six layers (1024-slot rings for local
                   layers, the full cache for the global one);
  * chunked leg  : a 4096-query chunk at positions 126976..131071 against a
                   131072-position cache (global, RoPE base 1e6 with position
                   interpolation 8) plus the five local layers;
  * prefill_1b and decode_1b : the same two blocks at Gemma 3 1B shapes
                   (Hq=4, Hkv=1, D=256): one 32768-token sequence, and 32
                   sequences with 32767 cached positions;
  * qkv / qkv_1b : the prefill blocks as whole attention sublayers from the
                   layer input (27B: x [8192, 5376]; 1B: x [32768, 1152]): per layer input RMSNorm, the
                   fused q/k/v projection (keys normed and rotated in its
                   epilogue), the flash prefill on those keys, o_proj and the
                   post-attention RMSNorm added to the residual; the same
                   q/k/v projection through torch's library GEMM is timed
                   beside it for context.
Beside the steps, once: the whole 62-layer 27B attention stack (52 local,
10 global) over one 128K sequence, the prompt through chunked prefills of
4096 tokens and then a decode loop, on per-layer caches (``schedule``).
`value` is the prefill leg's in-window TFLOP/s (4*D flops per visible
(query head, key) pair over the leg's wall time on the GPU); the decode
leg's KV GB/s and the chunked leg's TFLOP/s are reported beside it.
Inputs are seeded synthetic N(0,1) bf16 already resident in HBM.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "prefill attn TFLOP/s (in-window) + decode KV GB/s, 27B shapes, 1 MI355X"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E, published
LAYERS = 6                  # one 5:1 block


def _parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--legs", default="prefill,decode,chunked,prefill_1b,decode_1b,qkv,qkv_1b")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle-on-host baseline")
    ap.add_argument("--no-schedule", action="store_true", help="skip the 62-layer 128K schedule run")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="also run one device copy of this many MiB (HBM counter calibration)")
    return ap.parse_args()


class Leg:
    """Inputs, outputs and workspaces of one leg, all resident in HBM."""

    def __init__(self, name):
        self.name = name
        self.calls = []        # callables, one per layer
        self.work = []         # algorithmic flops or bytes per layer
        self.unit = ""
        self.main_ev = []      # (start, stop) events per layer around the main kernel


def _events(torch, n):
    evs = []
    for _ in range(n):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        b.record()
        evs.append((a, b))
    return evs


def build_prefill_leg(torch, G, W, C, cfg=2, name="prefill"):
    w = W.WORKLOADS[cfg]
    c = w.config
    leg = Leg(name)
    leg.unit = "flop"
    leg.workload = w
    leg.inputs = []
    for l in range(LAYERS):
        kind = G.layer_kind(l)
        base = W.ROPE_BASE_GLOBAL if kind == G.GLOBAL else W.ROPE_BASE_LOCAL
        q = W.device_normal_bf16((w.B, w.S, w.Hq, w.D), W.seed_of(c, l, W.T_Q))
        k = W.device_normal_bf16((w.B, w.S, w.Hkv, w.D), W.seed_of(c, l, W.T_K))
        v = W.device_normal_bf16((w.B, w.S, w.Hkv, w.D), W.seed_of(c, l, W.T_V))
        gq = torch.from_numpy(W.host_gamma(w.D, W.seed_of(c, l, W.T_GQ))).cuda()
        gk = torch.from_numpy(W.host_gamma(w.D, W.seed_of(c, l, W.T_GK))).cuda()
        o = torch.empty_like(q)
        ws = torch.empty(G.prefill_workspace_size(w.B, w.S, w.Hq, w.Hkv, w.D), dtype=torch.uint8, device="cuda")
        leg.inputs.append((q, k, v, gq, gk, kind))

        def call(q=q, k=k, v=v, gq=gq, gk=gk, o=o, ws=ws, kind=kind, base=base):
            G.prefill(q, k, v, kind, W.WINDOW, base, 1.0, gq, gk, W.EPS, 0.0, None, None, None, o=o, workspace=ws)
        leg.calls.append(call)
        leg.work.append(C.prefill_flops(w.B, w.S, w.Hq, w.D, kind == G.LOCAL, W.WINDOW))
    return leg


def build_decode_leg(torch, G, W, C, cfg=3, name="decode"):
    w = W.WORKLOADS[cfg]
    c = w.config
    leg = Leg(name)
    leg.unit = "byte"
    leg.workload = w
    p = w.pos0
    positions = torch.full((w.B,), p, dtype=torch.int32, device="cuda")
    for l in range(LAYERS):
        kind = G.layer_kind(l)
        base = W.ROPE_BASE_GLOBAL if kind == G.GLOBAL else W.ROPE_BASE_LOCAL
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

        def call(q=q, kn=kn, vn=vn, cache=cache, gq=gq, gk=gk, o=o, ws=ws, kind=kind, base=base):
            G.decode(q, kn, vn, positions, p, cache, kind, W.WINDOW, base, 1.0, gq, gk, W.EPS, 0.0, o=o, workspace=ws)
        leg.calls.append(call)
        leg.work.append(C.decode_bytes(w.B, w.Hq, w.Hkv, w.D, [p] * w.B, kind == G.LOCAL, W.WINDOW))
    return leg


def build_chunked_leg(torch, G, W, C):
    w = W.WORKLOADS[4]
    leg = Leg("chunked")
    leg.unit = "flop"
    leg.workload = w
    p0 = w.pos0
    for l in range(LAYERS):
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

        def call(q=q, k=k, v=v, cache=cache, gq=gq, gk=gk, o=o, ws=ws, kind=kind, base=base, scale=scale):
            G.prefill(q, k, v, kind, W.WINDOW, base, scale, gq, gk, W.EPS, 0.0, None, [p0], cache, o=o,
                      workspace=ws)
        leg.calls.append(call)
        leg.work.append(C.prefill_flops(w.B, w.S, w.Hq, w.D, kind == G.LOCAL, W.WINDOW, pos0=[p0], has_cache=True,
                                        ring_capacity=W.RING_CAP if ring else None))
    return leg


def build_qkv_leg(torch, G, W, C, cfg=2, name="qkv", dm=None):
    w = W.WORKLOADS[cfg]
    c = w.config
    dm = W.D_MODEL_27B if dm is None else dm
    leg = Leg(name)
    leg.d_model = dm
    leg.o_ms = [0.0] * LAYERS
    leg.unit = "flop"
    leg.workload = w
    leg.per_kernel = False
    leg.gemm = []
    leg.oev = _events(torch, LAYERS)
    leg.owork = []
    for l in range(LAYERS):
        kind = G.layer_kind(l)
        base = W.ROPE_BASE_GLOBAL if kind == G.GLOBAL else W.ROPE_BASE_LOCAL
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
        hn = torch.empty_like(x)
        yo = torch.empty_like(x)
        xo = torch.empty_like(x)

        def call(x=x, wt=wt, gq=gq, gk=gk, q=q, kh=kh, v=v, o=o, ws=ws, kind=kind, base=base, wo=wo, gi=gi, gp=gp,
                 hn=hn, yo=yo, xo=xo, l=l):
            G.rmsnorm(x, gi, W.EPS, out=hn)
            G.qkv_project(hn, wt, w.Hq, w.Hkv, base, 1.0, gk, W.EPS, None, q=q, khat=kh, v=v)
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
        leg.gemm.append(gemm)
        leg.work.append(2.0 * w.B * w.S * dm * (w.Hq + 2 * w.Hkv) * w.D)
        leg.owork.append(2.0 * w.B * w.S * w.Hq * w.D * dm)
    return leg


def run_leg(torch, G, leg, timed, per_kernel=False):
    """Launch the leg's layers.  timed: events bracket the whole leg.
    per_kernel: events bracket each layer's main kernel (recorded by the
    library on the launch stream); kept out of the leg-timed steps because the
    extra event packets between kernels lengthen the leg itself."""
    if timed:
        leg.ev_leg[0].record()
    leg.per_kernel = per_kernel
    for l, call in enumerate(leg.calls):
        if per_kernel:
            G.set_timing_events(*leg.main_ev[l])
        call()
    if per_kernel:
        G.set_timing_events(None, None)
    if timed:
        leg.ev_leg[1].record()


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


def cpu_baseline(torch, W, C, prefill_leg):
    """The oracle as it stands on the host cores: query heads 0-3 (kv heads
    0-1) of each layer of the prefill block, all 8192 query rows."""
    import numpy as np

    import oracle.attention as A

    try:
        from threadpoolctl import threadpool_info

        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    w = prefill_leg.workload
    flops = 0.0
    t_total = 0.0
    for (q, k, v, gq, gk, kind) in prefill_leg.inputs:
        qh = q[:, :, 0:4].float().cpu().numpy()
        kh = k[:, :, 0:2].float().cpu().numpy()
        vh = v[:, :, 0:2].float().cpu().numpy()
        base = W.ROPE_BASE_GLOBAL if kind == A.GLOBAL else W.ROPE_BASE_LOCAL
        t0 = time.perf_counter()
        A.prefill(qh, kh, vh, kind, W.WINDOW, base, 1.0, gq.cpu().numpy(), gk.cpu().numpy(), W.EPS)
        t_total += time.perf_counter() - t0
        flops += C.prefill_flops(1, w.S, 4, w.D, kind == A.LOCAL, W.WINDOW)
    return {"value": flops / t_total / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": "27B prefill block, query heads 0-3 / kv heads 0-1 of each of the 6 layers, all 8192 rows "
                      f"(in-window {flops:.4g} flop in {t_total:.2f} s, NumPy float64)"}


def _src_hash(name):
    p = os.path.join(ROOT, "global_gqa_amd", "csrc", name)
    return hashlib.sha256(open(p, "rb").read()).hexdigest()[:16]


def _model_tag(w):
    return "1b" if w.D == 256 else "27b"


def _traffic(kernel_src, launches_key):
    """Measured HBM bytes per launch from the committed counter summary, if
    it was taken on the current kernel source; else None."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        t = json.load(open(p))
        e = t[launches_key]
        if e.get("source_sha256_16") != _src_hash(kernel_src):
            return None
        return float(e["hbm_bytes_per_launch"])
    except Exception:
        return None


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
                "prefill_1b": lambda *a: build_prefill_leg(*a, cfg=9, name="prefill_1b"),
                "decode_1b": lambda *a: build_decode_leg(*a, cfg=10, name="decode_1b"), "qkv": build_qkv_leg,
                "qkv_1b": lambda *a: build_qkv_leg(*a, cfg=9, name="qkv_1b", dm=W.D_MODEL_1B)}
    for n in names:
        leg = builders[n](torch, G, W, C)
        leg.ev_leg = _events(torch, 1)[0]
        leg.main_ev = _events(torch, LAYERS)
        legs.append(leg)
        print(f"[bench] built leg {n}", file=sys.stderr, flush=True)
    torch.cuda.synchronize()

    for s in range(args.warmup):
        for leg in legs:
            run_leg(torch, G, leg, timed=False)
    torch.cuda.synchronize()
    print(f"[bench] warmup {args.warmup} done", file=sys.stderr, flush=True)

    leg_ms = {leg.name: 0.0 for leg in legs}
    main_ms = {leg.name: [0.0] * LAYERS for leg in legs}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        for leg in legs:
            run_leg(torch, G, leg, timed=True)
        torch.cuda.synchronize()
        for leg in legs:
            leg_ms[leg.name] += leg.ev_leg[0].elapsed_time(leg.ev_leg[1])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    K = max(args.steps, 1)
    print(f"[bench] timed {args.steps} steps in {wall:.2f} s", file=sys.stderr, flush=True)
    # per-kernel durations (roofline), in steps of their own
    KK = max(3, args.steps // 2)
    for s in range(KK):
        for leg in legs:
            run_leg(torch, G, leg, timed=False, per_kernel=True)
        torch.cuda.synchronize()
        for leg in legs:
            for l in range(LAYERS):
                main_ms[leg.name][l] += leg.main_ev[l][0].elapsed_time(leg.main_ev[l][1])
                if hasattr(leg, "oev"):
                    leg.o_ms[l] += leg.oev[l][0].elapsed_time(leg.oev[l][1])
    print(f"[bench] {KK} steps of per-kernel timing done", file=sys.stderr, flush=True)
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
        gemm_ms = ev[0].elapsed_time(ev[1]) / (KK * LAYERS)

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

    def prefill_summary(leg):
        w = leg.workload
        ms = leg_ms[leg.name] / K
        flops = sum(leg.work)
        kms = [x / KK for x in main_ms[leg.name]]
        achieved = flops / (sum(kms) * 1e-3) / 1e12
        cfg = {"workload": w.name, "B": w.B, "S": w.S, "Hq": w.Hq, "Hkv": w.Hkv, "D": w.D, "layers": "LLLLLG",
               "window": W.WINDOW, "rope_base": [W.ROPE_BASE_LOCAL, W.ROPE_BASE_GLOBAL],
               "in_window_flop_per_block": flops, "prefill_block_ms": ms}
        kern = "prefill_fwd" if w.D == 128 else "prefill_fwd_d256"
        src = "prefill.hip" if w.D == 128 else "prefill_d256.hip"
        roof = {"bound": "mfma", "kernel": kern, "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / PEAK_BF16_TFLOPS, "traffic": _traffic(src, f"{kern}_{_model_tag(w)}_block"),
                "launch_ms": kms, "launch_flop": leg.work}
        return flops / (ms * 1e-3) / 1e12, cfg, roof

    def decode_summary(leg):
        w = leg.workload
        ms = leg_ms[leg.name] / K
        nbytes = sum(leg.work)
        kms = [x / KK for x in main_ms[leg.name]]
        # split-K kernel: KV bytes only (q/o/new rows are handled around it)
        kv_bytes = [b - 2.0 * w.D * (2 * w.B * w.Hq + 2 * w.B * w.Hkv) for b in leg.work]
        ach = sum(kv_bytes) / (sum(kms) * 1e-3) / 1e9
        return {"value": nbytes / (ms * 1e-3) / 1e9, "unit": "GB/s", "workload": w.name, "ms": ms,
                "bytes_per_block": nbytes, "frac_hbm": nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS,
                "roofline": {"bound": "hbm", "kernel": "decode_splitk", "achieved": ach, "peak": PEAK_HBM_GBPS,
                             "unit": "GB/s", "frac": ach / PEAK_HBM_GBPS,
                             "traffic": _traffic("decode.hip", f"decode_splitk_{_model_tag(w)}_block"),
                             "launch_ms": kms}}

    if "prefill" in by:
        out["value"], out["config"], out["roofline"] = prefill_summary(by["prefill"])
    if "decode" in by:
        out["decode"] = decode_summary(by["decode"])
    if "chunked" in by:
        leg = by["chunked"]
        ms = leg_ms["chunked"] / K
        flops = sum(leg.work)
        kms = [x / KK for x in main_ms["chunked"]]
        out["chunked_prefill"] = {"value": flops / (ms * 1e-3) / 1e12, "unit": "TFLOP/s",
                                  "workload": leg.workload.name, "ms": ms, "in_window_flop_per_block": flops,
                                  "kernel_TFLOPs": flops / (sum(kms) * 1e-3) / 1e12, "launch_ms": kms}
    if "prefill_1b" in by or "decode_1b" in by:
        g1 = {}
        if "prefill_1b" in by:
            v, cfg, roof = prefill_summary(by["prefill_1b"])
            g1["prefill"] = {"value": v, "unit": "TFLOP/s", "config": cfg, "roofline": roof}
        if "decode_1b" in by:
            g1["decode"] = decode_summary(by["decode_1b"])
        out["gemma3_1b"] = g1
    def qkv_summary(leg, tag):
        w = leg.workload
        ms = leg_ms[leg.name] / K
        kms = [x / KK for x in main_ms[leg.name]]
        ach = sum(leg.work) / (sum(kms) * 1e-3) / 1e12
        o_ach = sum(leg.owork) / (sum(leg.o_ms) / KK * 1e-3) / 1e12
        return {
            "value": ach, "unit": "TFLOP/s", "workload": w.name + " from the layer input",
            "d_model": leg.d_model, "tokens": w.B * w.S, "heads": [w.Hq, w.Hkv, w.Hkv], "D": w.D,
            "block_ms": ms, "block": "per layer: input RMSNorm, fused q/k/v projection, prefill on the projected "
                                     "keys, o_proj, post-attention RMSNorm added to the residual",
            "projection_flop_per_layer": leg.work[0],
            "roofline": {"bound": "mfma", "kernel": "qkv_proj", "achieved": ach, "peak": PEAK_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": ach / PEAK_BF16_TFLOPS,
                         "traffic": _traffic("qkv_proj.hip", f"qkv_proj_{tag}_block"), "launch_ms": kms},
            "o_proj": {"value": o_ach, "unit": "TFLOP/s", "kernel": "qkv_proj (no key/value heads)",
                       "flop_per_layer": leg.owork[0], "frac": o_ach / PEAK_BF16_TFLOPS,
                       "launch_ms": [t / KK for t in leg.o_ms]}}

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
    if not args.no_schedule:
        print("[bench] 62-layer 128K schedule...", file=sys.stderr, flush=True)
        out["schedule_27b_128k"] = run_schedule(torch, G, W, C)
    if not args.no_cpu_baseline and "prefill" in by:
        print("[bench] cpu baseline (oracle on host)...", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(torch, W, C, by["prefill"])
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out))


if __name__ == "__main__":
    main()
