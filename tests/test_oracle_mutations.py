"""Planted mistakes in the oracle must be caught by its pins.

Each case swaps one oracle function for a plausible wrong variant (on the
CPU, in this process only) and runs the pins that should notice it.  A pin
set that stays green under a planted slip would not be pinning anything.
"""
import numpy as np
import pytest

import oracle.attention as A
import tests.test_oracle_pins as P

_rope_ok = A.rope
_norm_ok = A.rms_norm
_vis_ok = A.visibility
_attend_ok = A.attend
_decode_ok = A.decode
_qkv_ok = A.qkv_project
_oproj_ok = A.o_project
_rres_ok = A.residual_rms_norm
_block_ok = A.attention_block


def rope_wrong_sign(x, positions, base, interp_scale=1.0):
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    h = D // 2
    p = np.asarray(positions, dtype=np.float64).reshape(-1) / interp_scale
    phi = p[:, None] * A.rope_inv_freq(D, base)[None, :]
    c, s = np.cos(phi)[:, None, :], np.sin(phi)[:, None, :]
    return np.concatenate([x[..., :h] * c + x[..., h:] * s, x[..., :h] * s + x[..., h:] * c], axis=-1)


def rope_interleaved(x, positions, base, interp_scale=1.0):
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    p = np.asarray(positions, dtype=np.float64).reshape(-1) / interp_scale
    phi = p[:, None] * A.rope_inv_freq(D, base)[None, :]
    c, s = np.cos(phi)[:, None, :], np.sin(phi)[:, None, :]
    out = np.empty_like(x)
    out[..., 0::2] = x[..., 0::2] * c - x[..., 1::2] * s
    out[..., 1::2] = x[..., 0::2] * s + x[..., 1::2] * c
    return out


def rope_no_interp(x, positions, base, interp_scale=1.0):
    return _rope_ok(x, positions, base, 1.0)


def norm_no_eps(x, gamma, eps):
    return _norm_ok(x, gamma, 0.0)


def norm_no_gamma(x, gamma, eps):
    return _norm_ok(x, None, eps)


def vis_window_inclusive(qpos, kpos, kind, window, spans=()):
    return _vis_ok(qpos, kpos, kind, window + 1, spans)


def vis_no_spans(qpos, kpos, kind, window, spans=()):
    return _vis_ok(qpos, kpos, kind, window, ())


def attend_gqa_modulo(qh, kh, v, mask, softmax_scale):
    qh, kh, v = (np.asarray(t, dtype=np.float64) for t in (qh, kh, v))
    Hq, Hkv = qh.shape[1], kh.shape[1]
    out = np.empty((qh.shape[0], Hq, v.shape[2]))
    for h in range(Hq):
        g = h % Hkv
        z = np.where(mask, softmax_scale * qh[:, h] @ kh[:, g].T, -np.inf)
        p = np.exp(z - z.max(axis=1, keepdims=True))
        out[:, h] = (p / p.sum(axis=1, keepdims=True)) @ v[:, g]
    return out


def attend_no_scale(qh, kh, v, mask, softmax_scale):
    return _attend_ok(qh, kh, v, mask, 1.0)


def attend_softmax_wrong_axis(qh, kh, v, mask, softmax_scale):
    qh, kh, v = (np.asarray(t, dtype=np.float64) for t in (qh, kh, v))
    Hq, Hkv = qh.shape[1], kh.shape[1]
    G = Hq // Hkv
    out = np.empty((qh.shape[0], Hq, v.shape[2]))
    for h in range(Hq):
        z = np.where(mask, softmax_scale * qh[:, h] @ kh[:, h // G].T, -np.inf)
        p = np.exp(z - np.nanmax(np.where(mask, z, np.nan)))
        p = p / np.maximum(p.sum(axis=0, keepdims=True), 1e-300)
        out[:, h] = p @ v[:, h // G]
    return out


def decode_ring_off_by_one(q, k_new, v_new, cache_k, cache_v, is_ring, positions, *a, **kw):
    if is_ring:
        cap = np.asarray(cache_k).shape[2]
        cache_k = np.roll(np.asarray(cache_k, dtype=np.float64), 1, axis=2)
        cache_v = np.roll(np.asarray(cache_v, dtype=np.float64), 1, axis=2)
        assert cap > 1
    return _decode_ok(q, k_new, v_new, cache_k, cache_v, is_ring, positions, *a, **kw)


def qkv_heads_interleaved(x, w_q, w_k, w_v, Hq, Hkv):
    q, k, v = _qkv_ok(x, w_q, w_k, w_v, Hq, Hkv)
    B, S = q.shape[:2]
    fix = lambda t: t.reshape(B, S, -1).reshape(B, S, t.shape[3], t.shape[2]).swapaxes(2, 3)
    return fix(q), fix(k), fix(v)


def qkv_k_v_swapped(x, w_q, w_k, w_v, Hq, Hkv):
    return _qkv_ok(x, w_q, w_v, w_k, Hq, Hkv)


def qkv_row_of_weight(x, w_q, w_k, w_v, Hq, Hkv):
    """Reads a square Wq as [in, out] (x Wq instead of x Wq^T)."""
    q, k, v = _qkv_ok(x, w_q, w_k, w_v, Hq, Hkv)
    x = np.asarray(x, dtype=np.float64)
    if w_q.shape[0] == w_q.shape[1]:
        q = (x @ np.asarray(w_q, dtype=np.float64)).reshape(q.shape)
    return q, k, v


def o_project_heads_interleaved(attn, w_o):
    a = np.asarray(attn, dtype=np.float64)
    return _oproj_ok(np.swapaxes(a, -1, -2).copy().reshape(a.shape), w_o)


def residual_dropped(x, gamma, eps, residual=None):
    return _rres_ok(x, gamma, eps)


def _block_with(x, w_q, w_k, w_v, w_o, Hq, Hkv, gamma_in, gamma_post, q_gamma, k_gamma, eps, kind, window,
                rope_base, interp_scale, softmax_scale=None, spans=None, pos0=None, slip=""):
    """The oracle's sublayer with one step done wrong (``slip``)."""
    h = x if slip == "no_input_norm" else A.residual_rms_norm(x, gamma_in, eps)
    q, k, v = A.qkv_project(h, w_q, w_k, w_v, Hq, Hkv)
    if slip == "k_v_swapped":
        k, v = v, k
    a = A.prefill(q, k, v, kind, window, rope_base, interp_scale, q_gamma, k_gamma, eps, softmax_scale, spans, pos0)
    y = A.o_project(a, w_o)
    res = h if slip == "residual_from_normed_input" else x
    if slip == "no_post_norm":
        return np.asarray(res, dtype=np.float64) + y
    return A.residual_rms_norm(y, gamma_post, eps, residual=res)


def block_no_input_norm(*a, **kw):
    return _block_with(*a, slip="no_input_norm", **kw)


def block_residual_from_normed_input(*a, **kw):
    return _block_with(*a, slip="residual_from_normed_input", **kw)


def block_no_post_norm(*a, **kw):
    return _block_with(*a, slip="no_post_norm", **kw)


def block_k_v_swapped(*a, **kw):
    return _block_with(*a, slip="k_v_swapped", **kw)


def _all_pins():
    out = []
    for name in dir(P):
        if name.startswith("test_"):
            fn = getattr(P, name)
            params = getattr(fn, "pytestmark", [])
            cases = [None]
            for m in params:
                if m.name == "parametrize":
                    argnames = m.args[0]
                    cases = [(argnames, vals) for vals in m.args[1]]
            for c in cases:
                out.append((name, fn, c))
    return out


def _run(fn, case):
    if case is None:
        fn()
        return
    argnames, vals = case
    names = [s.strip() for s in argnames.split(",")]
    if len(names) == 1:
        fn(vals)
    else:
        fn(*vals)


MUTATIONS = [
    ("rope", rope_wrong_sign),
    ("rope", rope_interleaved),
    ("rope", rope_no_interp),
    ("rms_norm", norm_no_eps),
    ("rms_norm", norm_no_gamma),
    ("visibility", vis_window_inclusive),
    ("visibility", vis_no_spans),
    ("attend", attend_gqa_modulo),
    ("attend", attend_no_scale),
    ("attend", attend_softmax_wrong_axis),
    ("decode", decode_ring_off_by_one),
    ("qkv_project", qkv_heads_interleaved),
    ("qkv_project", qkv_k_v_swapped),
    ("qkv_project", qkv_row_of_weight),
    ("o_project", o_project_heads_interleaved),
    ("residual_rms_norm", residual_dropped),
    ("attention_block", block_no_input_norm),
    ("attention_block", block_residual_from_normed_input),
    ("attention_block", block_no_post_norm),
    ("attention_block", block_k_v_swapped),
]


@pytest.mark.parametrize("attr,bad", MUTATIONS, ids=[m[1].__name__ for m in MUTATIONS])
def test_planted_mistake_is_caught(monkeypatch, attr, bad):
    monkeypatch.setattr(A, attr, bad)
    caught = []
    for name, fn, case in _all_pins():
        try:
            with np.errstate(all="ignore"):
                _run(fn, case)
        except (AssertionError, ValueError, FloatingPointError, IndexError):
            caught.append(name)
    assert caught, f"no pin noticed the planted mistake {bad.__name__}"
