"""Seeded synthetic inputs for the Gemma 3 attention-stack workloads.

This module is shared by the tests, the bench and the smoke check.  It holds
shapes and random-number recipes only: none of the attention arithmetic
(norm, rotation, masking, softmax) lives here, and it imports neither the
oracle nor the HIP binding.

Recipe (used everywhere):
  * seed = 1000 * config + 10 * layer + tensor_id, with tensor ids
    q 0, k 1, v 2, q-gamma 3, k-gamma 4, cache-K 5, cache-V 6, spans 7,
    layer input x 8, stacked projection weight W 9;
  * tensors are standard-normal float32 rounded to bfloat16 by
    round-to-nearest-even; gamma = 1 + 0.1 * N(0, 1) kept in float32;
    projection weights are N(0, 1) / sqrt(d_model) (fan-in scaling, so that
    the projected q, k, v have unit scale like the other inputs) rounded to
    bfloat16;
  * small tensors come from NumPy's PCG64 on the host; the multi-GB KV caches
    of the decode and long-context workloads come from torch's device
    generator (Philox) so that the bench does not spend minutes on the CPU.
    Tests that need a host copy of such a tensor copy the slice they need
    back from the device.

Shapes follow the 27B module print on "Gemma explained: What's new in
Gemma 3" (32 query heads, 16 KV heads, head_dim 128) and, for the 1B
workloads, that page's 1B print (4 query heads, 1 KV head, head_dim 256),
the 1024-token local span and the 128K (1B: 32K) context of the Technical
Report (sections 1 and 2), and the 256-token image size (Technical Report,
section 1).
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Sequence, Tuple

import numpy as np

T_Q, T_K, T_V, T_GQ, T_GK, T_CK, T_CV, T_SPANS, T_X, T_W = range(10)
D_MODEL_27B = 5376       # hidden size in the 27B print (q_proj 5376 -> 4096)
D_MODEL_1B = 1152        # hidden size in the 1B print (q_proj 1152 -> 1024)

WINDOW = 1024            # local span (Technical Report, section 1)
ROPE_BASE_LOCAL = 1.0e4  # Technical Report, section 2 "Long context"
ROPE_BASE_GLOBAL = 1.0e6
EPS = 1.0e-6             # q_norm / k_norm eps in the 27B module print
IMAGE_TOKENS = 256       # soft tokens per image (Technical Report, section 1)
RING_CAP = 1024          # local-layer cache holds the last 1024 positions


def seed_of(config: int, layer: int, tensor_id: int) -> int:
    return 1000 * int(config) + 10 * int(layer) + int(tensor_id)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 to the nearest bfloat16 (ties to even); returns float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32)


def host_normal_bf16(shape: Sequence[int], seed: int) -> np.ndarray:
    g = np.random.Generator(np.random.PCG64(seed))
    return bf16_round(g.standard_normal(tuple(shape), dtype=np.float32))


def host_weight_bf16(shape: Sequence[int], seed: int) -> np.ndarray:
    """Projection weight [out, in]: N(0, 1) / sqrt(in) rounded to bf16."""
    g = np.random.Generator(np.random.PCG64(seed))
    w = g.standard_normal(tuple(shape), dtype=np.float32) * np.float32(1.0 / np.sqrt(shape[-1]))
    return bf16_round(w)


def host_gamma(D: int, seed: int) -> np.ndarray:
    g = np.random.Generator(np.random.PCG64(seed))
    return (1.0 + 0.1 * g.standard_normal(D, dtype=np.float64)).astype(np.float32)


def device_normal_bf16(shape: Sequence[int], seed: int, device="cuda", std: float = 1.0):
    """Normal bf16 tensor (standard deviation std) drawn on the device
    (torch Philox)."""
    import torch

    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    out = torch.empty(tuple(shape), dtype=torch.bfloat16, device=device)
    # fill in slabs to bound the float32 staging buffer
    flat = out.view(-1)
    step = 1 << 26
    for s in range(0, flat.numel(), step):
        n = min(step, flat.numel() - s)
        r = torch.randn(n, generator=gen, device=device, dtype=torch.float32)
        if std != 1.0:
            r.mul_(float(std))
        flat[s:s + n] = r.to(torch.bfloat16)
    return out


def image_spans(S: int, n: int, seed: int, length: int = IMAGE_TOKENS, base: int = 0) -> List[Tuple[int, int]]:
    """n non-overlapping [start, end) spans of ``length`` tokens in [0, S).

    Starts are at token granularity (not tile aligned): draw n sorted gap
    offsets in [0, S - n*length] and lay the spans out left to right.
    """
    if n == 0:
        return []
    free = S - n * length
    assert free >= 0
    g = np.random.Generator(np.random.PCG64(seed))
    offs = np.sort(g.integers(0, free + 1, size=n))
    return [(base + int(offs[i]) + i * length, base + int(offs[i]) + (i + 1) * length) for i in range(n)]


@dataclasses.dataclass(frozen=True)
class Workload:
    config: int
    name: str
    B: int
    S: int          # tokens per sequence (prefill) / chunk length (chunked) / 1 (decode)
    Hq: int
    Hkv: int
    D: int
    kinds: Tuple[str, ...]          # layer kinds run in order: "local" / "global"
    interp_scale_global: float = 1.0
    pos0: int = 0                   # first query position (chunked prefill / decode)
    cached: int = 0                 # positions already in the global cache
    mode: str = "prefill"           # prefill | decode | chunked
    max_spans: int = 0


# The five 27B-shaped workloads (shapes from the 27B module print; see the
# module docstring) and two of the 1B model.
WORKLOADS = {
    1: Workload(1, "single-layer-2k", B=1, S=2048, Hq=4, Hkv=2, D=128, kinds=("local", "global")),
    2: Workload(2, "27b-prefill-8k-block", B=1, S=8192, Hq=32, Hkv=16, D=128,
                kinds=("local",) * 5 + ("global",)),
    3: Workload(3, "27b-decode-32k-block", B=32, S=1, Hq=32, Hkv=16, D=128,
                kinds=("local",) * 5 + ("global",), pos0=32768, cached=32768, mode="decode"),
    4: Workload(4, "27b-chunked-prefill-128k-block", B=1, S=4096, Hq=32, Hkv=16, D=128,
                kinds=("local",) * 5 + ("global",), interp_scale_global=8.0,
                pos0=126976, cached=126976, mode="chunked"),
    5: Workload(5, "mixed-mask-4k", B=2, S=4096, Hq=16, Hkv=8, D=128, kinds=("local", "global"),
                max_spans=4),
    # Gemma 3 1B shapes (1B module print: 4 query heads, 1 KV head,
    # head_dim 256) at its 32K context (Technical Report, section 2).
    9: Workload(9, "1b-prefill-32k-block", B=1, S=32768, Hq=4, Hkv=1, D=256,
                kinds=("local",) * 5 + ("global",)),
    10: Workload(10, "1b-decode-32k-block", B=32, S=1, Hq=4, Hkv=1, D=256,
                 kinds=("local",) * 5 + ("global",), pos0=32767, cached=32767, mode="decode"),
}


def workload_spans(w: Workload) -> Optional[List[List[Tuple[int, int]]]]:
    """Image spans per sequence: sequence 0 has max_spans, the others a
    seeded count in 0..max_spans."""
    if w.max_spans == 0:
        return None
    out = []
    for b in range(w.B):
        if b == 0:
            n = w.max_spans
        else:
            g = np.random.Generator(np.random.PCG64(seed_of(w.config, 0, T_SPANS) + 100 + b))
            n = int(g.integers(0, w.max_spans + 1))
        out.append(image_spans(w.S, n, seed_of(w.config, 0, T_SPANS) + b, base=w.pos0))
    return out


def layer_inputs(w: Workload, layer: int, shrink: Optional[dict] = None):
    """Host q/k/v and gammas of one layer: dict of float32 arrays.

    ``shrink`` overrides shape fields (B, S, Hq, Hkv) for reduced parity cases
    that keep the recipe but fit the oracle.
    """
    B, S, Hq, Hkv, D = w.B, w.S, w.Hq, w.Hkv, w.D
    if shrink:
        B = shrink.get("B", B)
        S = shrink.get("S", S)
        Hq = shrink.get("Hq", Hq)
        Hkv = shrink.get("Hkv", Hkv)
    c = w.config
    if w.mode == "decode":
        q = host_normal_bf16((B, Hq, D), seed_of(c, layer, T_Q))
        k = host_normal_bf16((B, Hkv, D), seed_of(c, layer, T_K))
        v = host_normal_bf16((B, Hkv, D), seed_of(c, layer, T_V))
    else:
        q = host_normal_bf16((B, S, Hq, D), seed_of(c, layer, T_Q))
        k = host_normal_bf16((B, S, Hkv, D), seed_of(c, layer, T_K))
        v = host_normal_bf16((B, S, Hkv, D), seed_of(c, layer, T_V))
    return dict(q=q, k=k, v=v,
                q_gamma=host_gamma(D, seed_of(c, layer, T_GQ)),
                k_gamma=host_gamma(D, seed_of(c, layer, T_GK)))
