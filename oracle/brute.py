"""Loop-only brute force of one attention layer, for tiny inputs.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Written independently
of ``oracle.attention``: plain Python loops over every (sequence, head,
query, key) with the visibility predicate evaluated literally per pair, and
``math`` for every transcendental.  It exists to pin the vectorised oracle on
inputs with S <= ~16 and tiny head dimensions.
"""
from __future__ import annotations

import math


def _norm_vec(x, gamma, eps):
    # RMSNorm over one head vector (Technical Report section 2 QK-norm;
    # "Gemma explained" 27B print: RMSNorm((128,), eps=1e-06)).
    ms = sum(t * t for t in x) / len(x)
    r = 1.0 / math.sqrt(ms + eps)
    return [x[d] * r * (1.0 if gamma is None else float(gamma[d])) for d in range(len(x))]


def _rope_vec(x, p, base, scale):
    # Half-split pairs rotated by (p/scale) * base^(-2k/D) (Technical Report
    # section 2 "Long context": RoPE bases and position interpolation).
    D = len(x)
    h = D // 2
    out = list(x)
    for kk in range(h):
        phi = (p / scale) * base ** (-2.0 * kk / D)
        c, s = math.cos(phi), math.sin(phi)
        out[kk] = x[kk] * c - x[kk + h] * s
        out[kk + h] = x[kk] * s + x[kk + h] * c
    return out


def _visible(i, j, kind, window, spans):
    same = any(s <= i < e and s <= j < e for (s, e) in spans)
    glob = (j <= i) or same
    if kind == 1:
        return glob
    return glob and abs(i - j) < window


def prefill(q, k, v, kind, window, base, scale, q_gamma, k_gamma, eps,
            softmax_scale=None, spans=None, pos0=None):
    """Same contract as ``oracle.attention.prefill``; nested lists or arrays in,
    nested lists [B][S][Hq][D] out."""
    B = len(q)
    S = len(q[0])
    Hq = len(q[0][0])
    D = len(q[0][0][0])
    Hkv = len(k[0][0])
    G = Hq // Hkv
    sm = (D ** -0.5) if not softmax_scale else softmax_scale
    out = []
    for b in range(B):
        p0 = 0 if pos0 is None else int(pos0[b])
        sp = [] if spans is None else list(spans[b])
        qh = [[None] * Hq for _ in range(S)]
        kh = [[None] * Hkv for _ in range(S)]
        for t in range(S):
            for h in range(Hq):
                x = [float(q[b][t][h][d]) for d in range(D)]
                if q_gamma is not None:
                    x = _norm_vec(x, q_gamma, eps)
                qh[t][h] = _rope_vec(x, p0 + t, base, scale)
            for g in range(Hkv):
                x = [float(k[b][t][g][d]) for d in range(D)]
                if k_gamma is not None:
                    x = _norm_vec(x, k_gamma, eps)
                kh[t][g] = _rope_vec(x, p0 + t, base, scale)
        ob = []
        for i in range(S):
            row = []
            for h in range(Hq):
                g = h // G
                logits = []
                for j in range(S):
                    if _visible(p0 + i, p0 + j, kind, window, sp):
                        z = sm * sum(qh[i][h][d] * kh[j][g][d] for d in range(D))
                        logits.append((j, z))
                zmax = max(z for _, z in logits)
                w = [(j, math.exp(z - zmax)) for j, z in logits]
                tot = sum(e for _, e in w)
                o = [sum(e * float(v[b][j][g][d]) for j, e in w) / tot for d in range(D)]
                row.append(o)
            ob.append(row)
        out.append(ob)
    return out
