"""fp64 NumPy definition of the Gemma 3 attention-layer stack.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``; never by the product path.

This is the plain definition, written for a reader to check against the pages
by eye: every array is upcast to float64, nothing is tiled, fused or
reordered, and every step cites the passage it follows.  Where the pages are
silent the reading taken is stated at the step (the list of readings is kept
with the design notes of the repository).

Layout conventions (the same as the library's, so tests can compare arrays
directly):
  q      [B, S, Hq,  D]      raw query vectors after the q projection
  k, v   [B, S, Hkv, D]      raw key / value vectors
  cache  [B, Hkv, cap, D]    K holds normed+rotated keys, V raw values;
                             a linear cache stores position j in slot j, a
                             ring stores it in slot j mod cap.
"""
from __future__ import annotations

import numpy as np

LOCAL = 0
GLOBAL = 1


def layer_kind(i: int) -> int:
    """Kind of decoder layer ``i`` (0-based).

    Gemma 3 Technical Report, section 2, "5:1 interleaving of local/global
    layers": five local sliding-window layers per global layer, and the first
    layer of the model is local.  The plainest schedule with both properties
    is the repeating block L,L,L,L,L,G, i.e. layer i is global iff i % 6 == 5.
    """
    return GLOBAL if i % 6 == 5 else LOCAL


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def rms_norm(x, gamma, eps: float) -> np.ndarray:
    """RMSNorm over the last axis: x / sqrt(mean(x^2) + eps) * gamma.

    Gemma 3 Technical Report, section 2 (QK-norm replaces soft-capping) and
    the 27B module print on "Gemma explained: What's new in Gemma 3", which
    shows q_norm/k_norm as RMSNorm over the head dimension (128,) with
    eps=1e-06.  gamma is the effective per-dimension multiplier, shared by all
    heads of the tensor; ``None`` means no scaling (gamma = 1).
    """
    x = _f64(x)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    y = x / np.sqrt(ms + eps)
    if gamma is not None:
        y = y * _f64(gamma)
    return y


def rope_inv_freq(D: int, base: float) -> np.ndarray:
    """Rotary frequencies theta_k = base^(-2k/D), k = 0 .. D/2-1.

    Gemma 3 Technical Report, section 2 "Long context": RoPE base 10k on local
    layers and 1M on global layers.  The pages do not print the frequency
    formula; this is the standard RoPE definition.
    """
    k = np.arange(D // 2, dtype=np.float64)
    return float(base) ** (-2.0 * k / D)


def rope(x, positions, base: float, interp_scale: float = 1.0) -> np.ndarray:
    """Rotate pairs (x_k, x_{k+D/2}) by phi = (p / s) * theta_k.

    x: [T, H, D]; positions: [T] absolute token positions.
    Gemma 3 Technical Report, section 2 "Long context": global layers use
    position interpolation in the manner of Chen et al. (2023), read here as
    the linear map p -> p / s applied before the angle; s = 1 means none.
    Pairing is half-split (dimension k with k + D/2).
    """
    x = _f64(x)
    T, H, D = x.shape
    half = D // 2
    p = _f64(positions).reshape(T) / float(interp_scale)
    phi = p[:, None] * rope_inv_freq(D, base)[None, :]          # [T, D/2]
    c = np.cos(phi)[:, None, :]
    s = np.sin(phi)[:, None, :]
    x1 = x[..., :half]
    x2 = x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x1 * s + x2 * c], axis=-1)


def qknorm_rope(x, gamma, eps: float, positions, base: float,
                interp_scale: float = 1.0, norm: bool = True) -> np.ndarray:
    """QK-RMSNorm followed by RoPE (the prologue of every attention layer).

    Order: normalise first, then rotate.  The pages put the norm modules in
    the attention block and say RoPE sits inside the dot-product attention
    ("Gemma explained", note under the 27B print), which is read as norm ->
    RoPE.  x: [T, H, D], positions: [T].
    """
    y = rms_norm(x, gamma, eps) if norm else _f64(x)
    return rope(y, positions, base, interp_scale)


def _same_span(qpos, kpos, spans) -> np.ndarray:
    """Boolean [Tq, Tk]: both positions lie in one image span [start, end)."""
    qpos = np.asarray(qpos).reshape(-1)
    kpos = np.asarray(kpos).reshape(-1)
    out = np.zeros((qpos.size, kpos.size), dtype=bool)
    for (s, e) in spans:
        out |= ((qpos >= s) & (qpos < e))[:, None] & ((kpos >= s) & (kpos < e))[None, :]
    return out


def visibility(qpos, kpos, kind: int, window: int, spans=()) -> np.ndarray:
    """Which keys a query may attend to, as a boolean [Tq, Tk] matrix.

    * global: causal, j <= i (Gemma 3 Technical Report, section 2), or both
      tokens in one image span, where attention is bidirectional ("Gemma
      explained", vision section: bidirectional attention on image inputs);
    * local: the global rule intersected with the sliding window of 1024
      tokens (Technical Report, section 1), read as |i - j| < window, i.e.
      1024 keys including the query itself.
    """
    qpos = np.asarray(qpos, dtype=np.int64).reshape(-1)
    kpos = np.asarray(kpos, dtype=np.int64).reshape(-1)
    vis = kpos[None, :] <= qpos[:, None]
    if len(spans):
        vis = vis | _same_span(qpos, kpos, spans)
    if kind == LOCAL:
        vis = vis & (np.abs(qpos[:, None] - kpos[None, :]) < int(window))
    return vis


def visible_interval(i: int, kind: int, window: int, spans=()):
    """The contiguous key range [lo, hi] visible to query position i.

    Derived from ``visibility`` for one row: the causal range [0, i] is
    extended to the end of an image span containing i, and for local layers
    clipped to the window.  Used by tests to build closed-form probes.
    """
    hi = i
    for (s, e) in spans:
        if s <= i < e:
            hi = max(hi, e - 1)
    lo = 0
    if kind == LOCAL:
        lo = max(0, i - int(window) + 1)
        hi = min(hi, i + int(window) - 1)
    return lo, hi


def attend(qh, kh, v, mask, softmax_scale: float) -> np.ndarray:
    """Masked softmax attention with GQA head sharing.

    qh [Tq, Hq, D], kh [Tk, Hkv, D], v [Tk, Hkv, D], mask [Tq, Tk] bool.
    Logits are scale * <q, k> with no soft-cap (the Technical Report,
    section 2, removes Gemma 2's soft-capping).  Query head h reads kv head
    h // (Hq / Hkv): contiguous groups, as GQA shares each K/V head among a
    group of query heads (section 2; 27B print: 32 query heads, 16 KV heads).
    Softmax subtracts the row maximum; every row must see at least one key.
    """
    qh, kh, v = _f64(qh), _f64(kh), _f64(v)
    Tq, Hq, D = qh.shape
    Hkv = kh.shape[1]
    assert Hq % Hkv == 0
    G = Hq // Hkv
    assert mask.any(axis=1).all(), "a query row sees no key"
    out = np.empty((Tq, Hq, v.shape[2]), dtype=np.float64)
    for h in range(Hq):
        g = h // G
        z = softmax_scale * (qh[:, h, :] @ kh[:, g, :].T)      # [Tq, Tk]
        z = np.where(mask, z, -np.inf)
        z = z - z.max(axis=1, keepdims=True)
        p = np.exp(z)
        p = p / p.sum(axis=1, keepdims=True)
        out[:, h, :] = p @ v[:, g, :]
    return out


def qkv_project(x, w_q, w_k, w_v, Hq: int, Hkv: int):
    """Input projections of an attention layer: q = x Wq^T, k = x Wk^T,
    v = x Wv^T, each output split into heads.

    "Gemma explained: What's new in Gemma 3", 27B module print: q_proj,
    k_proj and v_proj are Linear maps without bias, 5376 -> 4096 (32 query
    heads of 128) and 5376 -> 2048 (16 key/value heads of 128).  A Linear map
    with weight W [out, in] sends x to x W^T.  The print does not show how
    the output features split into heads; the reading taken is contiguous
    blocks: feature h * D + d is dimension d of head h.

    x [B, S, d_model]; w_q [Hq * D, d_model]; w_k, w_v [Hkv * D, d_model].
    Returns (q [B, S, Hq, D], k [B, S, Hkv, D], v [B, S, Hkv, D]) in float64,
    raw (the QK-norm and RoPE of ``qknorm_rope`` come after).
    """
    x = _f64(x)
    B, S, _ = x.shape
    D = _f64(w_q).shape[0] // Hq
    q = (x @ _f64(w_q).T).reshape(B, S, Hq, D)
    k = (x @ _f64(w_k).T).reshape(B, S, Hkv, D)
    v = (x @ _f64(w_v).T).reshape(B, S, Hkv, D)
    return q, k, v


def o_project(attn, w_o):
    """The layer's output projection: y = attn W_o^T over the concatenated
    heads.

    "Gemma explained: What's new in Gemma 3", 27B module print: o_proj is a
    Linear map 4096 -> 5376 without bias, i.e. the Hq heads of D values are
    read as one vector of Hq * D (head-major, the same contiguous-block
    reading as the input projections).  attn [..., Hq, D]; w_o [out, Hq * D].
    Returns y [..., out] in float64.
    """
    a = _f64(attn)
    a = a.reshape(a.shape[:-2] + (a.shape[-2] * a.shape[-1],))
    return a @ _f64(w_o).T


def residual_rms_norm(x, gamma, eps: float, residual=None):
    """residual + RMSNorm(x) over the model width.

    Technical Report, section 2: Gemma 3 uses RMSNorm both before (pre-norm)
    and after (post-norm) the attention; the 27B print lists
    input_layernorm and post_attention_layernorm, RMSNorm over 5376 with
    eps 1e-6.  The reading taken for the residual stream: the layer maps x to
    x + post_attention_layernorm(o_proj(attention(input_layernorm(x)))), so
    the post-norm output is added to the residual and the pre-norm has none.
    """
    y = rms_norm(x, gamma, eps)
    return y if residual is None else _f64(residual) + y


def attention_block(x, w_q, w_k, w_v, w_o, Hq: int, Hkv: int, gamma_in, gamma_post, q_gamma, k_gamma,
                    eps: float, kind: int, window: int, rope_base: float, interp_scale: float,
                    softmax_scale=None, spans=None, pos0=None):
    """One attention sublayer from its input: x + post_norm(o_proj(attn(pre_norm(x)))).

    x [B, S, d_model]; the steps are ``residual_rms_norm`` (no residual),
    ``qkv_project``, ``prefill`` and ``o_project``, then
    ``residual_rms_norm`` with x as the residual.  Returns [B, S, d_model].
    """
    h = residual_rms_norm(x, gamma_in, eps)
    q, k, v = qkv_project(h, w_q, w_k, w_v, Hq, Hkv)
    a = prefill(q, k, v, kind, window, rope_base, interp_scale, q_gamma, k_gamma, eps, softmax_scale, spans, pos0)
    y = o_project(a, w_o)
    return residual_rms_norm(y, gamma_post, eps, residual=x)


def _scale(softmax_scale, D):
    return float(D) ** -0.5 if not softmax_scale else float(softmax_scale)


def prefill(q, k, v, kind: int, window: int, rope_base: float, interp_scale: float,
            q_gamma, k_gamma, eps: float, softmax_scale=None, spans=None, pos0=None):
    """Self-contained prefill of one attention layer.

    q [B, S, Hq, D], k/v [B, S, Hkv, D] raw.  Token r of sequence b sits at
    position pos0[b] + r (pos0 defaults to 0).  spans[b] is a list of
    (start, end) absolute positions of that sequence's image spans.
    Returns o [B, S, Hq, D] in float64.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, S, Hq, D = q.shape
    scale = _scale(softmax_scale, D)
    out = np.empty_like(q)
    for b in range(B):
        p0 = 0 if pos0 is None else int(pos0[b])
        pos = p0 + np.arange(S)
        sp = [] if spans is None else list(spans[b])
        qh = qknorm_rope(q[b], q_gamma, eps, pos, rope_base, interp_scale, q_gamma is not None)
        kh = qknorm_rope(k[b], k_gamma, eps, pos, rope_base, interp_scale, k_gamma is not None)
        mask = visibility(pos, pos, kind, window, sp)
        out[b] = attend(qh, kh, v[b], mask, scale)
    return out


def ring_slot(j, cap: int, is_ring: bool):
    """Cache slot of absolute position j: j mod cap in a ring, else j.

    The local layers keep only the last 1024 positions (Technical Report,
    abstract and section 1: the short local span keeps the KV cache small),
    stored here as a ring buffer indexed by position modulo its capacity.
    """
    return (np.asarray(j) % cap) if is_ring else np.asarray(j)


def prefill_chunk(q, k, v, cache_k, cache_v, is_ring: bool, kind: int, window: int,
                  rope_base: float, interp_scale: float, q_gamma, k_gamma, eps: float,
                  softmax_scale=None, spans=None, pos0=None):
    """Chunked prefill against a KV cache.

    Chunk token r of sequence b sits at position p0 = pos0[b] plus r.  The
    cache holds normed+rotated keys and raw values of positions before p0 (a
    linear cache: every position from 0; a ring: the last ``cap`` of them).
    Queries see cached positions through the cache and chunk positions
    through the chunk itself; afterwards the chunk's keys/values are written
    to their slots.  Returns (o [B, C, Hq, D], new_cache_k, new_cache_v).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    ck = _f64(cache_k).copy()
    cv = _f64(cache_v).copy()
    B, C, Hq, D = q.shape
    cap = ck.shape[2]
    scale = _scale(softmax_scale, D)
    out = np.empty_like(q)
    for b in range(B):
        p0 = 0 if pos0 is None else int(pos0[b])
        qpos = p0 + np.arange(C)
        sp = [] if spans is None else list(spans[b])
        qh = qknorm_rope(q[b], q_gamma, eps, qpos, rope_base, interp_scale, q_gamma is not None)
        kh_new = qknorm_rope(k[b], k_gamma, eps, qpos, rope_base, interp_scale, k_gamma is not None)
        lo_old = max(0, p0 - cap) if is_ring else 0
        old_pos = np.arange(lo_old, p0)
        slots = ring_slot(old_pos, cap, is_ring)
        kpos = np.concatenate([old_pos, qpos])
        kh = np.concatenate([ck[b][:, slots, :].transpose(1, 0, 2), kh_new], axis=0)
        vv = np.concatenate([cv[b][:, slots, :].transpose(1, 0, 2), v[b]], axis=0)
        mask = visibility(qpos, kpos, kind, window, sp)
        out[b] = attend(qh, kh, vv, mask, scale)
        new_slots = ring_slot(qpos, cap, is_ring)
        for r in range(C):  # in position order, so later positions win in a ring
            ck[b][:, new_slots[r], :] = kh_new[r]
            cv[b][:, new_slots[r], :] = v[b][r]
    return out, ck, cv


def decode(q, k_new, v_new, cache_k, cache_v, is_ring: bool, positions, kind: int,
           window: int, rope_base: float, interp_scale: float, q_gamma, k_gamma,
           eps: float, softmax_scale=None):
    """One decode step per sequence.

    q [B, Hq, D], k_new/v_new [B, Hkv, D] raw, for the new token of sequence b
    at position p = positions[b]; the cache holds positions before p.  The new
    key is normed, rotated and written to its slot first, then the token
    attends to [0, p] (global) or (p - window, p] (local), itself included.
    Returns (o [B, Hq, D], new_cache_k, new_cache_v).
    """
    q, k_new, v_new = _f64(q), _f64(k_new), _f64(v_new)
    ck = _f64(cache_k).copy()
    cv = _f64(cache_v).copy()
    B, Hq, D = q.shape
    cap = ck.shape[2]
    scale = _scale(softmax_scale, D)
    out = np.empty_like(q)
    for b in range(B):
        p = int(positions[b])
        pos = np.array([p])
        qh = qknorm_rope(q[b][None], q_gamma, eps, pos, rope_base, interp_scale, q_gamma is not None)
        kh = qknorm_rope(k_new[b][None], k_gamma, eps, pos, rope_base, interp_scale, k_gamma is not None)
        s = int(ring_slot(p, cap, is_ring))
        ck[b][:, s, :] = kh[0]
        cv[b][:, s, :] = v_new[b]
        lo = max(0, p - cap + 1) if is_ring else 0
        kpos = np.arange(lo, p + 1)
        mask = visibility(pos, kpos, kind, window)
        slots = ring_slot(kpos, cap, is_ring)
        kk = ck[b][:, slots, :].transpose(1, 0, 2)
        vv = cv[b][:, slots, :].transpose(1, 0, 2)
        out[b] = attend(qh, kk, vv, mask, scale)[0]
    return out, ck, cv
