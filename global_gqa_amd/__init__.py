"""Python binding of libg3attn (Gemma 3 local/global GQA attention on MI355X).

Argument marshalling only: every step of the attention runs in the HIP
kernels of ``libg3attn.so``; torch supplies device memory and the current
stream.  There is no fallback: if the library is missing or fails to load,
every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple

LOCAL = 0
GLOBAL = 1
WINDOW = 1024
RING_CAPACITY = 1024

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libg3attn.so")

G3_OK, G3_EINVAL, G3_EUNSUPPORTED, G3_EHIP, G3_EWORKSPACE = 0, -1, -2, -3, -4


class G3Error(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"g3attn error {code}: {msg}")
        self.code = code


class Span(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("start", ctypes.c_int32), ("end", ctypes.c_int32)]


class KVCacheC(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("capacity", ctypes.c_int32),
                ("is_ring", ctypes.c_int32)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libg3attn.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m global_gqa_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    L.g3attn_qknorm_rope.argtypes = [vp, vp, vp, vp, vp, vp, f32, vp, i32, i32, i32, i32, f32, f32, vp]
    L.g3attn_qknorm_rope.restype = ctypes.c_int
    L.g3attn_prefill.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, f32, f32, vp, vp, f32, f32,
                                 ctypes.POINTER(Span), i32, ctypes.POINTER(i32), ctypes.POINTER(KVCacheC), vp, sz, vp]
    L.g3attn_prefill.restype = ctypes.c_int
    L.g3attn_prefill_khat.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, f32, f32, vp, f32, f32,
                                      ctypes.POINTER(Span), i32, ctypes.POINTER(i32), ctypes.POINTER(KVCacheC), vp,
                                      sz, vp]
    L.g3attn_prefill_khat.restype = ctypes.c_int
    L.g3attn_qkv_project.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32, f32, vp, f32,
                                     ctypes.POINTER(i32), vp]
    L.g3attn_qkv_project.restype = ctypes.c_int
    L.g3attn_o_project.argtypes = [vp, vp, vp, i32, i32, i32, vp]
    L.g3attn_o_project.restype = ctypes.c_int
    L.g3attn_rmsnorm.argtypes = [vp, vp, vp, f32, vp, i32, i32, vp]
    L.g3attn_rmsnorm.restype = ctypes.c_int
    L.g3attn_rms_scale.argtypes = [vp, f32, vp, i32, i32, vp]
    L.g3attn_rms_scale.restype = ctypes.c_int
    L.g3attn_fold_norm_weight.argtypes = [vp, vp, vp, i32, i32, vp]
    L.g3attn_fold_norm_weight.restype = ctypes.c_int
    L.g3attn_prefill_workspace_size.argtypes = [i32, i32, i32, i32, i32]
    L.g3attn_prefill_workspace_size.restype = sz
    L.g3attn_decode.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, vp, i32, ctypes.POINTER(KVCacheC), i32, i32, f32,
                                f32, vp, vp, f32, f32, vp, sz, vp]
    L.g3attn_decode.restype = ctypes.c_int
    L.g3attn_decode_noalloc.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, vp, i32, ctypes.POINTER(KVCacheC), i32,
                                        i32, f32, f32, vp, vp, f32, f32, vp]
    L.g3attn_decode_noalloc.restype = ctypes.c_int
    L.g3attn_decode_workspace_size.argtypes = [i32, i32, i32, i32, i32, ctypes.POINTER(KVCacheC)]
    L.g3attn_decode_workspace_size.restype = sz
    L.g3attn_last_error.argtypes = []
    L.g3attn_last_error.restype = ctypes.c_char_p
    L.g3attn_version.argtypes = []
    L.g3attn_version.restype = ctypes.c_int32
    L.g3attn_set_timing_events.argtypes = [vp, vp]
    L.g3attn_set_timing_events.restype = ctypes.c_int
    _lib = L
    return L


def _check(code: int):
    if code != G3_OK:
        raise G3Error(code, lib().g3attn_last_error().decode())


def layer_kind(i: int) -> int:
    """Layer i of the stack is global iff i % 6 == 5: five local layers per
    global one, the first layer local (Gemma 3 Technical Report, section 2)."""
    return GLOBAL if i % 6 == 5 else LOCAL


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int:
    """The HIP stream to launch on: ``stream``, else torch's current stream
    of the current device (read as a raw handle where torch offers it: that
    skips building a Stream object, a few microseconds per call)."""
    import torch

    if stream is not None:
        return stream.cuda_stream
    raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
    if raw is not None:
        return raw(torch._C._cuda_getDevice())
    return torch.cuda.current_stream().cuda_stream


def _check_tensor(name, t, dtype, shape=None):
    import torch

    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


class KVCache:
    """Per-layer KV cache: k, v device bf16 tensors [B, Hkv, capacity, D]."""

    def __init__(self, k, v, is_ring: bool):
        import torch

        _check_tensor("cache.k", k, torch.bfloat16)
        _check_tensor("cache.v", v, torch.bfloat16, k.shape)
        self.k, self.v, self.is_ring = k, v, bool(is_ring)

    @classmethod
    def empty(cls, B, Hkv, capacity, D=128, is_ring=False, device="cuda"):
        import torch

        k = torch.zeros((B, Hkv, capacity, D), dtype=torch.bfloat16, device=device)
        v = torch.zeros_like(k)
        return cls(k, v, is_ring)

    @property
    def capacity(self) -> int:
        return int(self.k.shape[2])

    def c(self) -> KVCacheC:
        return KVCacheC(self.k.data_ptr(), self.v.data_ptr(), self.capacity, int(self.is_ring))


def qknorm_rope(q, k, positions, q_gamma, k_gamma, eps: float, rope_base: float, interp_scale: float = 1.0,
                q_out=None, k_out=None, stream=None):
    """QK-RMSNorm then RoPE of q [T, Hq, D] and/or k [T, Hkv, D] (either may be
    None).  Returns (q_out, k_out)."""
    import torch

    ref = q if q is not None else k
    T, D = ref.shape[0], ref.shape[2]
    Hq = q.shape[1] if q is not None else 0
    Hkv = k.shape[1] if k is not None else 0
    for n, t in (("q", q), ("k", k), ("q_out", q_out), ("k_out", k_out)):
        _check_tensor(n, t, torch.bfloat16)
    _check_tensor("positions", positions, torch.int32, (T,))
    _check_tensor("q_gamma", q_gamma, torch.float32, (D,))
    _check_tensor("k_gamma", k_gamma, torch.float32, (D,))
    if q is not None and q_out is None:
        q_out = torch.empty_like(q)
    if k is not None and k_out is None:
        k_out = torch.empty_like(k)
    _check(lib().g3attn_qknorm_rope(_ptr(q), _ptr(k), _ptr(q_out), _ptr(k_out), _ptr(q_gamma), _ptr(k_gamma),
                                    float(eps), _ptr(positions), T, Hq, Hkv, D, float(rope_base),
                                    float(interp_scale), _stream(stream)))
    return q_out, k_out


def prefill_workspace_size(B, S, Hq, Hkv, D=128) -> int:
    return int(lib().g3attn_prefill_workspace_size(B, S, Hq, Hkv, D))


def decode_workspace_size(B, Hq, Hkv, D, max_position, cache: KVCache) -> int:
    cc = cache.c()
    return int(lib().g3attn_decode_workspace_size(B, Hq, Hkv, D, max_position, ctypes.byref(cc)))


def _workspace(nbytes, device):
    import torch

    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


def _spans_pos0(spans, pos0, B):
    sp = None
    n_sp = 0
    if spans:
        n_sp = len(spans)
        sp = (Span * n_sp)(*[Span(int(b), int(s), int(e)) for (b, s, e) in spans])
    p0 = None
    if pos0 is not None:
        p0 = (ctypes.c_int32 * B)(*[int(x) for x in pos0])
    return sp, n_sp, p0


def prefill(q, k, v, layer_kind: int, window: int, rope_base: float, interp_scale: float, q_gamma, k_gamma,
            eps: float, softmax_scale: float = 0.0, spans: Optional[Sequence[Tuple[int, int, int]]] = None,
            pos0: Optional[Sequence[int]] = None, cache: Optional[KVCache] = None, o=None, workspace=None,
            stream=None):
    """One attention layer's prefill.  q [B, S, Hq, D], k/v [B, S, Hkv, D]
    raw bf16; spans: (batch, start, end) absolute positions; pos0: first
    position per sequence; cache: attend to and append into a KV cache."""
    import torch

    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    _check_tensor("q", q, torch.bfloat16)
    _check_tensor("k", k, torch.bfloat16, (B, S, Hkv, D))
    _check_tensor("v", v, torch.bfloat16, (B, S, Hkv, D))
    _check_tensor("q_gamma", q_gamma, torch.float32, (D,))
    _check_tensor("k_gamma", k_gamma, torch.float32, (D,))
    if o is None:
        o = torch.empty_like(q)
    _check_tensor("o", o, torch.bfloat16, q.shape)
    need = prefill_workspace_size(B, S, Hq, Hkv, D)
    if workspace is None:
        workspace = _workspace(need, q.device)
    sp, n_sp, p0 = _spans_pos0(spans, pos0, B)
    cc = ctypes.byref(cache.c()) if cache is not None else None
    _check(lib().g3attn_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(o), B, S, Hq, Hkv, D, int(layer_kind), int(window),
                                float(rope_base), float(interp_scale), _ptr(q_gamma), _ptr(k_gamma), float(eps),
                                float(softmax_scale), sp, n_sp, p0, cc, workspace.data_ptr(),
                                workspace.numel() * workspace.element_size(), _stream(stream)))
    return o


def prefill_khat(q, khat, v, layer_kind: int, window: int, rope_base: float, interp_scale: float, q_gamma,
                 eps: float, softmax_scale: float = 0.0, spans: Optional[Sequence[Tuple[int, int, int]]] = None,
                 pos0: Optional[Sequence[int]] = None, cache: Optional[KVCache] = None, o=None, workspace=None,
                 stream=None):
    """prefill() with the keys already normed and rotated: khat
    [B, Hkv, S, D] head-major (as qkv_project writes it)."""
    import torch

    B, S, Hq, D = q.shape
    Hkv = khat.shape[1]
    _check_tensor("q", q, torch.bfloat16)
    _check_tensor("khat", khat, torch.bfloat16, (B, Hkv, S, D))
    _check_tensor("v", v, torch.bfloat16, (B, S, Hkv, D))
    _check_tensor("q_gamma", q_gamma, torch.float32, (D,))
    if o is None:
        o = torch.empty_like(q)
    _check_tensor("o", o, torch.bfloat16, q.shape)
    if workspace is None:
        workspace = _workspace(prefill_workspace_size(B, S, Hq, Hkv, D), q.device)
    sp, n_sp, p0 = _spans_pos0(spans, pos0, B)
    cc = ctypes.byref(cache.c()) if cache is not None else None
    _check(lib().g3attn_prefill_khat(_ptr(q), _ptr(khat), _ptr(v), _ptr(o), B, S, Hq, Hkv, D, int(layer_kind),
                                     int(window), float(rope_base), float(interp_scale), _ptr(q_gamma), float(eps),
                                     float(softmax_scale), sp, n_sp, p0, cc, workspace.data_ptr(),
                                     workspace.numel() * workspace.element_size(), _stream(stream)))
    return o


def qkv_project(x, w, Hq: int, Hkv: int, rope_base: float, interp_scale: float, k_gamma, eps: float,
                pos0: Optional[Sequence[int]] = None, q=None, khat=None, v=None, stream=None, x_scale=None):
    """Input projections of one layer with the key prologue fused: x
    [B, S, d_model] bf16, w [(Hq + 2 Hkv) * D, d_model] bf16 (Wq, Wk, Wv
    rows stacked; D = 128 or 256 from its shape).  x_scale: fp32 [B, S] (or
    [B * S]) multiplying each token's projections (the input norm folded in:
    raw x, x_scale = rms_scale(x), w = fold_norm_weight(w, gamma)).  Returns
    (q [B, S, Hq, D] raw, khat [B, Hkv, S, D] normed + rotated, v [B, S, Hkv,
    D] raw)."""
    import torch

    B, S, dm = x.shape
    D = w.shape[0] // (Hq + 2 * Hkv)
    _check_tensor("x", x, torch.bfloat16)
    _check_tensor("x_scale", x_scale, torch.float32)
    if x_scale is not None and x_scale.numel() != B * S:
        raise ValueError(f"x_scale has {x_scale.numel()} elements, expected {B * S}")
    _check_tensor("w", w, torch.bfloat16, ((Hq + 2 * Hkv) * D, dm))
    _check_tensor("k_gamma", k_gamma, torch.float32, (D,))
    if q is None:
        q = torch.empty((B, S, Hq, D), dtype=torch.bfloat16, device=x.device)
    if khat is None:
        khat = torch.empty((B, Hkv, S, D), dtype=torch.bfloat16, device=x.device)
    if v is None:
        v = torch.empty((B, S, Hkv, D), dtype=torch.bfloat16, device=x.device)
    _check_tensor("q", q, torch.bfloat16, (B, S, Hq, D))
    _check_tensor("khat", khat, torch.bfloat16, (B, Hkv, S, D))
    _check_tensor("v", v, torch.bfloat16, (B, S, Hkv, D))
    _, _, p0 = _spans_pos0(None, pos0, B)
    _check(lib().g3attn_qkv_project(_ptr(x), _ptr(x_scale), _ptr(w), _ptr(q), _ptr(khat), _ptr(v), B, S, dm, Hq,
                                    Hkv, D, float(rope_base), float(interp_scale), _ptr(k_gamma), float(eps), p0,
                                    _stream(stream)))
    return q, khat, v


def o_project(attn, w_o, y=None, stream=None):
    """The layer's o_proj: attn [B, S, Hq, D] with Hq * D = in, or [..., in]
    with fewer than four axes (bf16); w_o [out, in] bf16.  Returns y
    [B, S, out] or [..., out]."""
    import torch

    _check_tensor("attn", attn, torch.bfloat16)
    _check_tensor("w_o", w_o, torch.bfloat16)
    n_out, n_in = w_o.shape
    if attn.dim() >= 4 and attn.shape[-2] * attn.shape[-1] == n_in:  # [B, S, Hq, D]
        lead = attn.shape[:-2]
    elif attn.shape[-1] == n_in:
        lead = attn.shape[:-1]
    else:
        raise ValueError(f"attn shape {tuple(attn.shape)} does not end in in_features {n_in} or [Hq, D]")
    T = attn.numel() // n_in
    if y is None:
        y = torch.empty(tuple(lead) + (n_out,), dtype=torch.bfloat16, device=attn.device)
    _check_tensor("y", y, torch.bfloat16)
    if y.numel() != T * n_out:
        raise ValueError(f"y has {y.numel()} elements, expected {T * n_out}")
    _check(lib().g3attn_o_project(_ptr(attn), _ptr(w_o), _ptr(y), T, n_in, n_out, _stream(stream)))
    return y


def rmsnorm(x, gamma, eps: float, residual=None, out=None, stream=None):
    """out = residual + x / sqrt(mean(x^2) + eps) * gamma over the last axis
    (residual and gamma optional); out may be x or residual."""
    import torch

    W = x.shape[-1]
    T = x.numel() // W
    _check_tensor("x", x, torch.bfloat16)
    _check_tensor("residual", residual, torch.bfloat16, x.shape)
    _check_tensor("gamma", gamma, torch.float32, (W,))
    if out is None:
        out = torch.empty_like(x)
    _check_tensor("out", out, torch.bfloat16, x.shape)
    _check(lib().g3attn_rmsnorm(_ptr(x), _ptr(residual), _ptr(gamma), float(eps), _ptr(out), T, W,
                                _stream(stream)))
    return out



def rms_scale(x, eps: float, scale=None, stream=None):
    """scale[t] = 1 / sqrt(mean(x[t]^2) + eps) over the last axis of bf16 x:
    fp32 of shape x.shape[:-1]; the input norm's per-token factor for
    qkv_project(..., x_scale=...)."""
    import torch

    W = x.shape[-1]
    T = x.numel() // W
    _check_tensor("x", x, torch.bfloat16)
    if scale is None:
        scale = torch.empty(tuple(x.shape[:-1]), dtype=torch.float32, device=x.device)
    _check_tensor("scale", scale, torch.float32)
    if scale.numel() != T:
        raise ValueError(f"scale has {scale.numel()} elements, expected {T}")
    _check(lib().g3attn_rms_scale(_ptr(x), float(eps), _ptr(scale), T, W, _stream(stream)))
    return scale


def fold_norm_weight(w, gamma, out=None, stream=None):
    """w [rows, width] bf16 with gamma [width] fp32 folded in:
    out[n, k] = w[n, k] * gamma[k], rounded to bf16 (out may be w)."""
    import torch

    _check_tensor("w", w, torch.bfloat16)
    rows, width = w.shape
    _check_tensor("gamma", gamma, torch.float32, (width,))
    if out is None:
        out = torch.empty_like(w)
    _check_tensor("out", out, torch.bfloat16, w.shape)
    _check(lib().g3attn_fold_norm_weight(_ptr(w), _ptr(gamma), _ptr(out), rows, width, _stream(stream)))
    return out

def decode(q, k_new, v_new, positions, max_position: int, cache: KVCache, layer_kind: int, window: int,
           rope_base: float, interp_scale: float, q_gamma, k_gamma, eps: float, softmax_scale: float = 0.0,
           o=None, workspace=None, stream=None):
    """One decode step: q [B, Hq, D], k_new/v_new [B, Hkv, D] raw bf16,
    positions int32 [B] on the device.  Appends to and reads the cache."""
    import torch

    B, Hq, D = q.shape
    Hkv = k_new.shape[1]
    _check_tensor("q", q, torch.bfloat16)
    _check_tensor("k_new", k_new, torch.bfloat16, (B, Hkv, D))
    _check_tensor("v_new", v_new, torch.bfloat16, (B, Hkv, D))
    _check_tensor("positions", positions, torch.int32, (B,))
    _check_tensor("q_gamma", q_gamma, torch.float32, (D,))
    _check_tensor("k_gamma", k_gamma, torch.float32, (D,))
    if o is None:
        o = torch.empty_like(q)
    _check_tensor("o", o, torch.bfloat16, q.shape)
    if workspace is None:
        workspace = _workspace(decode_workspace_size(B, Hq, Hkv, D, max_position, cache), q.device)
    cc = cache.c()
    _check(lib().g3attn_decode(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(o), B, Hq, Hkv, D, _ptr(positions),
                               int(max_position), ctypes.byref(cc), int(layer_kind), int(window), float(rope_base),
                               float(interp_scale), _ptr(q_gamma), _ptr(k_gamma), float(eps), float(softmax_scale),
                               workspace.data_ptr(), workspace.numel() * workspace.element_size(), _stream(stream)))
    return o


DECODE_NOALLOC_MAX_BYTES = 16 << 20  # G3_DECODE_NOALLOC_MAX_BYTES


def decode_noalloc(q, k_new, v_new, positions, max_position: int, cache: KVCache, layer_kind: int, window: int,
                   rope_base: float, interp_scale: float, q_gamma, k_gamma, eps: float, softmax_scale: float = 0.0,
                   o=None, stream=None):
    """decode() through g3attn_decode_noalloc: no workspace; the split-K
    partials go to the library's static per-GPU array (calls overlapping on
    one GPU race).  With ``o`` given, the call allocates nothing."""
    import torch

    B, Hq, D = q.shape
    Hkv = k_new.shape[1]
    _check_tensor("q", q, torch.bfloat16)
    _check_tensor("k_new", k_new, torch.bfloat16, (B, Hkv, D))
    _check_tensor("v_new", v_new, torch.bfloat16, (B, Hkv, D))
    _check_tensor("positions", positions, torch.int32, (B,))
    _check_tensor("q_gamma", q_gamma, torch.float32, (D,))
    _check_tensor("k_gamma", k_gamma, torch.float32, (D,))
    if o is None:
        o = torch.empty_like(q)
    _check_tensor("o", o, torch.bfloat16, q.shape)
    cc = cache.c()
    _check(lib().g3attn_decode_noalloc(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(o), B, Hq, Hkv, D, _ptr(positions),
                                       int(max_position), ctypes.byref(cc), int(layer_kind), int(window),
                                       float(rope_base), float(interp_scale), _ptr(q_gamma), _ptr(k_gamma),
                                       float(eps), float(softmax_scale), _stream(stream)))
    return o


def set_timing_events(start_event, stop_event):
    """Record torch.cuda.Event pair around the next main-kernel launches
    (None, None to stop).  Events must have been created on the device."""
    if start_event is None:
        _check(lib().g3attn_set_timing_events(None, None))
        return
    _check(lib().g3attn_set_timing_events(ctypes.c_void_p(start_event.cuda_event),
                                          ctypes.c_void_p(stop_event.cuda_event)))
