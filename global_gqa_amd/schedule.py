"""A whole Gemma 3 attention stack over its KV caches: a prompt through
successive chunked prefills, then a decode loop.

Host-side sequencing of the library's calls, nothing more: every step runs in
``g3attn_prefill`` / ``g3attn_decode``.  The caches and workspaces are
allocated once, when the stack is built, so the per-layer calls allocate
nothing.

The layer pattern and the per-kind parameters follow the Gemma 3 Technical
Report, section 2: five local layers per global one with a local layer first
(layer i is global iff i % 6 == 5; 62 layers give 10 global and 52 local),
local layers attend to the last 1024 positions with RoPE base 10k, global
layers to all earlier positions with RoPE base 1M and (for the 128K-context
models) linear position interpolation.  A local layer's cache is a ring of
the last ``window`` positions (slot = position mod window); a global layer's
cache holds every position (slot = position).  No weights are involved: the
caller supplies each layer's raw q, k, v (the projections are outside the
attention path).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Optional, Sequence

from . import GLOBAL, LOCAL, WINDOW, KVCache, decode, decode_workspace_size, layer_kind, prefill, \
    prefill_workspace_size

ROPE_BASE_LOCAL = 1.0e4
ROPE_BASE_GLOBAL = 1.0e6


@dataclass(frozen=True)
class LayerPlan:
    """Parameters of one layer's attention calls and its cache."""
    index: int
    kind: int
    window: int
    rope_base: float
    interp_scale: float
    capacity: int  # cache slots per (sequence, kv head)
    is_ring: bool


def plan_layers(n_layers: int, max_positions: int, window: int = WINDOW, global_interp_scale: float = 1.0,
                local_base: float = ROPE_BASE_LOCAL, global_base: float = ROPE_BASE_GLOBAL) -> List[LayerPlan]:
    """Per-layer plan of an ``n_layers`` stack holding up to ``max_positions``
    positions per sequence.  A local layer's ring has ``window`` slots (the
    library requires a ring at least as long as the window)."""
    if n_layers < 1 or max_positions < 1 or window < 1:
        raise ValueError("n_layers, max_positions and window must be positive")
    plans = []
    for i in range(n_layers):
        kind = layer_kind(i)
        if kind == LOCAL:
            plans.append(LayerPlan(i, LOCAL, window, local_base, 1.0, window, True))
        else:
            plans.append(LayerPlan(i, GLOBAL, window, global_base, global_interp_scale, max_positions, False))
    return plans


def chunk_bounds(n_tokens: int, chunk: int) -> List[tuple]:
    """[start, end) of the successive prefill chunks of an ``n_tokens`` prompt."""
    if chunk < 1:
        raise ValueError("chunk must be positive")
    return [(s, min(s + chunk, n_tokens)) for s in range(0, n_tokens, chunk)]


class AttentionStack:
    """Attention state of a model: one KV cache per layer and the number of
    positions already in them (the same for every sequence of the batch)."""

    def __init__(self, n_layers: int, B: int, Hq: int, Hkv: int, max_positions: int, max_chunk: int, D: int = 128,
                 window: int = WINDOW, global_interp_scale: float = 1.0, q_gammas: Optional[Sequence] = None,
                 k_gammas: Optional[Sequence] = None, eps: float = 1e-6, softmax_scale: float = 0.0,
                 device: str = "cuda"):
        import torch

        if max_chunk < 1:
            raise ValueError("max_chunk must be positive")
        self.plans = plan_layers(n_layers, max_positions, window, global_interp_scale)
        self.B, self.Hq, self.Hkv, self.D = B, Hq, Hkv, D
        self.max_positions, self.max_chunk = max_positions, max_chunk
        self.eps, self.softmax_scale = eps, softmax_scale
        ones = torch.ones(D, dtype=torch.float32, device=device)
        self.q_gammas = list(q_gammas) if q_gammas is not None else [ones] * n_layers
        self.k_gammas = list(k_gammas) if k_gammas is not None else [ones] * n_layers
        if len(self.q_gammas) != n_layers or len(self.k_gammas) != n_layers:
            raise ValueError("one q and one k gamma per layer")
        self.caches = [KVCache.empty(B, Hkv, p.capacity, D, is_ring=p.is_ring, device=device) for p in self.plans]
        self.prefill_ws = torch.empty(max(prefill_workspace_size(B, max_chunk, Hq, Hkv, D), 256), dtype=torch.uint8,
                                      device=device)
        dec = max(decode_workspace_size(B, Hq, Hkv, D, max_positions - 1, c) for c in self.caches)
        self.decode_ws = torch.empty(max(dec, 256), dtype=torch.uint8, device=device)
        self.positions = torch.zeros(B, dtype=torch.int32, device=device)
        self.pos = 0

    @property
    def n_layers(self) -> int:
        return len(self.plans)

    def prefill_layer(self, i: int, q, k, v, o=None, spans=None, stream=None):
        """Layer i's prefill of the next chunk: q [B, C, Hq, D], k/v
        [B, C, Hkv, D] raw bf16 at positions pos .. pos + C - 1; appends the
        chunk's keys and values to layer i's cache.  Returns o."""
        C = q.shape[1]
        if C > self.max_chunk:
            raise ValueError(f"chunk of {C} tokens exceeds max_chunk={self.max_chunk}")
        if self.pos + C > self.max_positions:
            raise ValueError(f"positions {self.pos}..{self.pos + C - 1} exceed max_positions={self.max_positions}")
        p = self.plans[i]
        return prefill(q, k, v, p.kind, p.window, p.rope_base, p.interp_scale, self.q_gammas[i], self.k_gammas[i],
                       self.eps, self.softmax_scale, spans, [self.pos] * self.B, self.caches[i], o=o,
                       workspace=self.prefill_ws, stream=stream)

    def decode_layer(self, i: int, q, k_new, v_new, o=None, stream=None):
        """Layer i's decode step for the token at position pos: q [B, Hq, D],
        k_new/v_new [B, Hkv, D] raw bf16.  Returns o."""
        if self.pos >= self.max_positions:
            raise ValueError(f"position {self.pos} exceeds max_positions={self.max_positions}")
        p = self.plans[i]
        return decode(q, k_new, v_new, self.positions, self.max_positions - 1, self.caches[i], p.kind, p.window,
                      p.rope_base, p.interp_scale, self.q_gammas[i], self.k_gammas[i], self.eps,
                      self.softmax_scale, o=o, workspace=self.decode_ws, stream=stream)

    def capture_decode(self, q_bufs, k_bufs, v_bufs, o_bufs):
        """Capture one decode step of every layer (layer i reads q_bufs[i],
        k_bufs[i], v_bufs[i] and writes o_bufs[i]) followed by the position
        increment into a HIP graph, and return a function that replays it for
        the token at the current position.  The library's calls allocate
        nothing and issue no memsets, so the captured launches replay as they
        are; the caller refills the input buffers between replays."""
        import torch

        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                for i in range(self.n_layers):
                    self.decode_layer(i, q_bufs[i], k_bufs[i], v_bufs[i], o=o_bufs[i])
                self.positions.add_(1)
        torch.cuda.current_stream().wait_stream(side)

        def step():
            if self.pos >= self.max_positions:
                raise ValueError(f"position {self.pos} exceeds max_positions={self.max_positions}")
            g.replay()
            self.pos += 1

        step.graph = g  # keeps the graph alive with the function
        return step

    def reset(self):
        """Start a new prompt: position 0 (old cache contents are never read
        again: every later read is of a position written after the reset)."""
        self.pos = 0
        self.positions.fill_(0)

    def advance(self, n: int):
        """Every layer has processed the next n positions."""
        if n < 0 or self.pos + n > self.max_positions:
            raise ValueError("advance past max_positions")
        self.pos += n
        self.positions.fill_(self.pos)
