"""Pins of the fp64 oracle against what the pages and the mathematics fix.

The pages print no worked numeric example, so the oracle is pinned by
closed forms, invariants, brute force on tiny inputs, a library special case
and the constants the pages state.  Each pin is chosen so that a plausible
slip in the oracle (a dropped term, a wrong sign or index, a transposed
operand, an off-by-one window) fails at least one of them;
``test_oracle_mutations.py`` plants such slips and checks that they do.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle.attention as A
from oracle import brute

HERE = os.path.dirname(os.path.abspath(__file__))
RNG = np.random.default_rng(1234)


def _rand(*shape, rng=None):
    rng = RNG if rng is None else rng
    return rng.standard_normal(shape)


# ---------------------------------------------------------------- constants
def test_golden_constants_and_layer_schedule():
    g = json.load(open(os.path.join(HERE, "golden", "gemma3_constants.json")))
    kinds = [A.layer_kind(i) for i in range(g["layers_27b"]["value"])]
    assert kinds[0] == A.LOCAL  # first layer is local
    n_glob = sum(1 for k in kinds if k == A.GLOBAL)
    n_loc = len(kinds) - n_glob
    assert (n_glob, n_loc) == (10, 52)
    # every global layer is preceded by exactly five local ones
    for i, k in enumerate(kinds):
        if k == A.GLOBAL:
            assert kinds[i - 5:i] == [A.LOCAL] * g["local_per_global"]["value"]
    assert g["q_heads_27b"]["value"] * g["head_dim_27b"]["value"] == 4096
    assert g["kv_heads_27b"]["value"] * g["head_dim_27b"]["value"] == 2048
    assert g["image_tokens"]["value"] == 16 * 16  # 64x64 patches pooled 4x4


# ---------------------------------------------------------------- RMSNorm
def test_rmsnorm_closed_form_mean_square():
    x = _rand(50, 3, 128)
    eps = 1e-6
    y = A.rms_norm(x, None, eps)
    ms = np.mean(x * x, axis=-1)
    np.testing.assert_allclose(np.mean(y * y, axis=-1), ms / (ms + eps), rtol=1e-12)


def test_rmsnorm_constant_vector_and_gamma():
    D = 128
    gamma = 1 + 0.1 * _rand(D)
    c = 3.0
    x = np.full((1, 1, D), c)
    y = A.rms_norm(x, gamma, 1e-6)
    np.testing.assert_allclose(y[0, 0], c / math.sqrt(c * c + 1e-6) * gamma, rtol=1e-14)


def test_rmsnorm_scale_invariance_eps0():
    x = _rand(10, 2, 16)
    np.testing.assert_allclose(A.rms_norm(7.5 * x, None, 0.0), A.rms_norm(x, None, 0.0), rtol=1e-13)


# ---------------------------------------------------------------- RoPE
def test_rope_closed_form_unit_vectors():
    D, base = 8, 100.0
    theta = A.rope_inv_freq(D, base)
    np.testing.assert_allclose(theta, [1.0, 100 ** -0.25, 100 ** -0.5, 100 ** -0.75], rtol=1e-15)
    p = 5.0
    for kk in range(D // 2):
        e = np.zeros((1, 1, D))
        e[0, 0, kk] = 1.0
        y = A.rope(e, [p], base)[0, 0]
        want = np.zeros(D)
        want[kk] = math.cos(p * theta[kk])
        want[kk + D // 2] = math.sin(p * theta[kk])
        np.testing.assert_allclose(y, want, atol=1e-15)


def test_rope_identity_at_zero_and_norm_preserved():
    x = _rand(7, 3, 128)
    np.testing.assert_array_equal(A.rope(x, np.zeros(7), 1e4), x)
    pos = np.array([0, 1, 17, 1023, 4096, 65535, 131071])
    for base in (1e4, 1e6):
        y = A.rope(x, pos, base)
        np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-12)


def test_rope_relative_property():
    # <R(q, m), R(k, n)> depends only on m - n
    q = _rand(1, 1, 128)
    k = _rand(1, 1, 128)
    for base in (1e4, 1e6):
        for (m, n, c) in [(10, 3, 100), (5000, 4000, 77777), (0, 0, 131000)]:
            a = np.sum(A.rope(q, [m], base) * A.rope(k, [n], base))
            b = np.sum(A.rope(q, [m + c], base) * A.rope(k, [n + c], base))
            assert abs(a - b) < 1e-9 * max(1.0, abs(a))


def test_rope_position_interpolation_is_position_division():
    x = _rand(4, 2, 128)
    pos = np.array([0, 8, 126976, 131071])
    np.testing.assert_allclose(A.rope(x, pos, 1e6, 8.0), A.rope(x, pos / 8.0, 1e6, 1.0), rtol=1e-13, atol=1e-13)


# ---------------------------------------------------------------- visibility
def test_visibility_window_edges_closed_form():
    S, W = 40, 7
    pos = np.arange(S)
    vis = A.visibility(pos, pos, A.LOCAL, W)
    for i in range(S):
        for j in range(S):
            assert vis[i, j] == (0 <= i - j < W)
    assert vis.sum(axis=1).tolist() == [min(i + 1, W) for i in range(S)]
    glob = A.visibility(pos, pos, A.GLOBAL, W)
    assert np.array_equal(glob, np.tril(np.ones((S, S), dtype=bool)))


def test_visibility_spans_and_interval():
    S, W = 30, 6
    spans = [(3, 8), (12, 16), (20, 29)]
    pos = np.arange(S)
    for kind in (A.LOCAL, A.GLOBAL):
        vis = A.visibility(pos, pos, kind, W, spans)
        for i in range(S):
            lo, hi = A.visible_interval(i, kind, W, spans)
            row = np.zeros(S, dtype=bool)
            row[lo:hi + 1] = True
            assert np.array_equal(vis[i], row), (kind, i)
    # inside a span every token sees every other token of the span
    g = A.visibility(pos, pos, A.GLOBAL, W, spans)
    assert g[3, 7] and g[7, 3] and not g[2, 3] and g[8, 7] and not g[7, 8]


def test_local_with_window_at_least_S_equals_global():
    B, S, Hq, Hkv, D = 2, 24, 4, 2, 16
    q, k, v = _rand(B, S, Hq, D), _rand(B, S, Hkv, D), _rand(B, S, Hkv, D)
    gq, gk = 1 + 0.1 * _rand(D), 1 + 0.1 * _rand(D)
    spans = [[(2, 9)], []]
    for W in (S, S + 5):
        lo = A.prefill(q, k, v, A.LOCAL, W, 1e4, 1.0, gq, gk, 1e-6, spans=spans)
        gl = A.prefill(q, k, v, A.GLOBAL, W, 1e4, 1.0, gq, gk, 1e-6, spans=spans)
        assert np.array_equal(lo, gl)
    lo = A.prefill(q, k, v, A.LOCAL, S - 1, 1e4, 1.0, gq, gk, 1e-6, spans=spans)
    assert not np.allclose(lo, gl)


# ---------------------------------------------------------------- softmax / GQA
def test_rows_sum_to_one_value_ones():
    B, S, Hq, Hkv, D = 1, 33, 4, 2, 16
    q, k = _rand(B, S, Hq, D), _rand(B, S, Hkv, D)
    v = np.ones((B, S, Hkv, D))
    for kind in (A.LOCAL, A.GLOBAL):
        o = A.prefill(q, k, v, kind, 5, 1e4, 1.0, None, None, 1e-6, spans=[[(10, 20)]])
        np.testing.assert_allclose(o, 1.0, rtol=1e-13)


def test_gqa_equals_mha_with_repeated_kv():
    B, S, Hq, Hkv, D = 1, 20, 6, 2, 8
    q, k, v = _rand(B, S, Hq, D), _rand(B, S, Hkv, D), _rand(B, S, Hkv, D)
    G = Hq // Hkv
    a = A.prefill(q, k, v, A.GLOBAL, 4, 1e4, 1.0, None, None, 1e-6)
    b = A.prefill(q, np.repeat(k, G, axis=2), np.repeat(v, G, axis=2), A.GLOBAL, 4, 1e4, 1.0, None, None, 1e-6)
    assert np.array_equal(a, b)


# ---------------------------------------------------------------- brute force
@pytest.mark.parametrize("case", [
    dict(S=9, Hq=2, Hkv=1, D=4, W=3, kind=A.LOCAL, spans=[[(2, 6)]], pos0=None, scale=1.0),
    dict(S=12, Hq=4, Hkv=2, D=8, W=1, kind=A.LOCAL, spans=[[]], pos0=None, scale=1.0),
    dict(S=12, Hq=4, Hkv=2, D=8, W=12, kind=A.LOCAL, spans=[[(0, 3), (7, 11)]], pos0=[5], scale=1.0),
    dict(S=10, Hq=2, Hkv=2, D=4, W=4, kind=A.GLOBAL, spans=[[(4, 9)]], pos0=[1000], scale=8.0),
    dict(S=11, Hq=3, Hkv=1, D=8, W=2, kind=A.LOCAL, spans=[[(1, 4), (5, 10)]], pos0=[3], scale=1.0),
])
def test_brute_force_tiny(case):
    rng = np.random.default_rng(7)
    S, Hq, Hkv, D = case["S"], case["Hq"], case["Hkv"], case["D"]
    q, k, v = rng.standard_normal((1, S, Hq, D)), rng.standard_normal((1, S, Hkv, D)), rng.standard_normal((1, S, Hkv, D))
    gq, gk = 1 + 0.1 * rng.standard_normal(D), 1 + 0.1 * rng.standard_normal(D)
    spans = None
    if case["spans"] is not None and case["pos0"] is not None:
        spans = [[(s + case["pos0"][0], e + case["pos0"][0]) for (s, e) in case["spans"][0]]]
    elif case["spans"] is not None:
        spans = case["spans"]
    base = 1e4 if case["kind"] == A.LOCAL else 1e6
    for sm in (None, 0.3):
        o = A.prefill(q, k, v, case["kind"], case["W"], base, case["scale"], gq, gk, 1e-6, sm, spans, case["pos0"])
        ob = np.array(brute.prefill(q.tolist(), k.tolist(), v.tolist(), case["kind"], case["W"], base, case["scale"],
                                    gq, gk, 1e-6, sm, spans, case["pos0"]))
        np.testing.assert_allclose(o, ob, rtol=1e-11, atol=1e-12)


# ---------------------------------------------------------------- library special case
def test_torch_sdpa_float64_special_case():
    torch = pytest.importorskip("torch")
    B, S, Hq, Hkv, D, W = 1, 64, 4, 2, 32, 9
    spans = [[(5, 17), (40, 47)]]
    q, k, v = _rand(B, S, Hq, D), _rand(B, S, Hkv, D), _rand(B, S, Hkv, D)
    for kind in (A.LOCAL, A.GLOBAL):
        o = A.prefill(q, k, v, kind, W, 1e4, 1.0, None, None, 1e-6, spans=spans)
        # independent construction: no norm (gamma None), RoPE applied with
        # complex multiplication on (x_k + i x_{k+D/2}), mask built by loops
        pos = torch.arange(S, dtype=torch.float64)
        theta = torch.tensor([1e4 ** (-2.0 * j / D) for j in range(D // 2)], dtype=torch.float64)
        rot = torch.polar(torch.ones(S, D // 2, dtype=torch.float64), pos[:, None] * theta[None, :])

        def crope(x):
            x = torch.from_numpy(x[0])
            z = torch.complex(x[..., :D // 2], x[..., D // 2:]) * rot[:, None, :]
            return torch.cat([z.real, z.imag], dim=-1)
        qh, kh = crope(q), crope(k)
        mask = torch.zeros(S, S, dtype=torch.bool)
        for i in range(S):
            for j in range(S):
                ok = j <= i or any(s <= i < e and s <= j < e for (s, e) in spans[0])
                if kind == A.LOCAL:
                    ok = ok and abs(i - j) < W
                mask[i, j] = ok
        G = Hq // Hkv
        kk = kh.repeat_interleave(G, dim=1).transpose(0, 1).contiguous()
        vv = torch.from_numpy(v[0]).repeat_interleave(G, dim=1).transpose(0, 1).contiguous()
        ref = torch.nn.functional.scaled_dot_product_attention(
            qh.transpose(0, 1).contiguous(), kk, vv, attn_mask=mask)
        np.testing.assert_allclose(o[0], ref.transpose(0, 1).numpy(), rtol=1e-10, atol=1e-12)


# ---------------------------------------------------------------- mask probes
def test_mask_probe_zero_keys_uniform_weights():
    # K = 0 makes every logit 0: each row averages V over its visible keys
    B, S, Hq, Hkv, D, W = 1, 50, 2, 1, 8, 7
    spans = [[(10, 19), (30, 34)]]
    q, v = _rand(B, S, Hq, D), _rand(B, S, Hkv, D)
    k = np.zeros((B, S, Hkv, D))
    for kind in (A.LOCAL, A.GLOBAL):
        o = A.prefill(q, k, v, kind, W, 1e4, 1.0, None, None, 1e-6, spans=spans)
        for i in range(S):
            lo, hi = A.visible_interval(i, kind, W, spans[0])
            want = v[0, lo:hi + 1, 0].mean(axis=0)
            np.testing.assert_allclose(o[0, i, 0], want, rtol=1e-12, atol=1e-14)


def test_mask_probe_indicator_values_exact_counts():
    # V = indicator of key set A: o_i = |A n vis(i)| / |vis(i)| (K = 0)
    S, W = 40, 8
    spans = [[(12, 20)]]
    key_set = {0, 5, 11, 12, 19, 20, 33, 39}
    v = np.zeros((1, S, 1, 1))
    for j in key_set:
        v[0, j, 0, 0] = 1.0
    k = np.zeros((1, S, 1, 1))
    q = np.ones((1, S, 1, 1))
    for kind in (A.LOCAL, A.GLOBAL):
        o = A.prefill(q, k, v, kind, W, 1e4, 1.0, None, None, 1e-6, spans=spans)
        for i in range(S):
            lo, hi = A.visible_interval(i, kind, W, spans[0])
            cnt = sum(1 for j in key_set if lo <= j <= hi)
            assert abs(o[0, i, 0, 0] - cnt / (hi - lo + 1)) < 1e-15


def test_mask_probe_full_window_one_key():
    # i >= W-1 in a local layer sees exactly W keys: a one-key probe gives 1/W or 0
    S, W = 1100, 1024
    v = np.zeros((1, S, 1, 1))
    v[0, 50, 0, 0] = 1.0
    o = A.prefill(np.ones((1, S, 1, 2)), np.zeros((1, S, 1, 2)), v, A.LOCAL, W, 1e4, 1.0, None, None, 1e-6)
    for i in (1023, 1073, 1074, 1099):
        want = 1.0 / W if i - 50 < W else 0.0
        assert o[0, i, 0, 0] == want


# ---------------------------------------------------------------- cache consistency
def _layer(B, S, Hq, Hkv, D, rng):
    return (rng.standard_normal((B, S, Hq, D)), rng.standard_normal((B, S, Hkv, D)),
            rng.standard_normal((B, S, Hkv, D)), 1 + 0.1 * rng.standard_normal(D), 1 + 0.1 * rng.standard_normal(D))


def _fill_cache(k, v, gk, cap, is_ring, base, scale, n):
    """Cache holding positions 0..n-1 of the (raw) k/v sequence, built with
    the oracle's own norm+rope (the state a run of chunked prefills leaves)."""
    B, S, Hkv, D = k.shape
    ck = np.zeros((B, Hkv, cap, D))
    cv = np.zeros((B, Hkv, cap, D))
    for b in range(B):
        kh = A.qknorm_rope(k[b, :n], gk, 1e-6, np.arange(n), base, scale)
        for j in range(n):
            s = j % cap if is_ring else j
            ck[b, :, s] = kh[j]
            cv[b, :, s] = v[b, j]
    return ck, cv


@pytest.mark.parametrize("kind,is_ring,cap,W", [(A.GLOBAL, False, 64, 64), (A.LOCAL, True, 8, 8), (A.LOCAL, False, 64, 5)])
def test_decode_equals_last_row_of_prefill(kind, is_ring, cap, W):
    rng = np.random.default_rng(3)
    B, S, Hq, Hkv, D = 2, 30, 4, 2, 8
    q, k, v, gq, gk = _layer(B, S, Hq, Hkv, D, rng)
    base, scale = (1e6, 8.0) if kind == A.GLOBAL else (1e4, 1.0)
    full = A.prefill(q, k, v, kind, W, base, scale, gq, gk, 1e-6)
    p = S - 1
    ck, cv = _fill_cache(k, v, gk, cap, is_ring, base, scale, p)
    o, ck2, cv2 = A.decode(q[:, p], k[:, p], v[:, p], ck, cv, is_ring, [p] * B, kind, W, base, scale, gq, gk, 1e-6)
    np.testing.assert_allclose(o, full[:, p], rtol=1e-12, atol=1e-13)
    ck_ref, cv_ref = _fill_cache(k, v, gk, cap, is_ring, base, scale, S)
    np.testing.assert_allclose(ck2, ck_ref, rtol=1e-13, atol=1e-14)
    np.testing.assert_array_equal(cv2, cv_ref)


@pytest.mark.parametrize("kind,is_ring,cap,W", [(A.GLOBAL, False, 80, 80), (A.LOCAL, True, 16, 16), (A.LOCAL, True, 16, 9)])
def test_chunked_prefill_equals_row_slice(kind, is_ring, cap, W):
    rng = np.random.default_rng(4)
    B, S, Hq, Hkv, D = 1, 70, 4, 2, 8
    q, k, v, gq, gk = _layer(B, S, Hq, Hkv, D, rng)
    base, scale = (1e6, 8.0) if kind == A.GLOBAL else (1e4, 1.0)
    spans = [[(50, 58)]]
    full = A.prefill(q, k, v, kind, W, base, scale, gq, gk, 1e-6, spans=spans)
    p0 = 45
    ck, cv = _fill_cache(k, v, gk, cap, is_ring, base, scale, p0)
    o, ck2, cv2 = A.prefill_chunk(q[:, p0:], k[:, p0:], v[:, p0:], ck, cv, is_ring, kind, W, base, scale, gq, gk,
                                  1e-6, spans=spans, pos0=[p0])
    np.testing.assert_allclose(o, full[:, p0:], rtol=1e-12, atol=1e-13)
    ck_ref, cv_ref = _fill_cache(k, v, gk, cap, is_ring, base, scale, S)
    np.testing.assert_allclose(ck2, ck_ref, rtol=1e-13, atol=1e-14)
    np.testing.assert_array_equal(cv2, cv_ref)


def test_ring_equals_linear_window():
    rng = np.random.default_rng(5)
    B, S, Hq, Hkv, D, W = 1, 40, 2, 1, 8, 10
    q, k, v, gq, gk = _layer(B, S, Hq, Hkv, D, rng)
    p = 37
    ckr, cvr = _fill_cache(k, v, gk, W, True, 1e4, 1.0, p)
    ckl, cvl = _fill_cache(k, v, gk, 64, False, 1e4, 1.0, p)
    a = A.decode(q[:, p], k[:, p], v[:, p], ckr, cvr, True, [p], A.LOCAL, W, 1e4, 1.0, gq, gk, 1e-6)[0]
    b = A.decode(q[:, p], k[:, p], v[:, p], ckl, cvl, False, [p], A.LOCAL, W, 1e4, 1.0, gq, gk, 1e-6)[0]
    np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-14)


def test_global_position_shift_invariance():
    rng = np.random.default_rng(6)
    B, S, Hq, Hkv, D = 1, 30, 2, 1, 16
    q, k, v, gq, gk = _layer(B, S, Hq, Hkv, D, rng)
    for kind in (A.LOCAL, A.GLOBAL):
        a = A.prefill(q, k, v, kind, 7, 1e4, 1.0, gq, gk, 1e-6)
        b = A.prefill(q, k, v, kind, 7, 1e4, 1.0, gq, gk, 1e-6, pos0=[100000])
        np.testing.assert_allclose(a, b, rtol=1e-8, atol=1e-9)


# ---------------------------------------------------------------- projections
def test_qkv_project_identity_blocks():
    """With Wq = I (d_model = Hq D) the queries are the input cut into
    heads of D consecutive features; Wk = Wv = the first Hkv D rows of I
    select the leading features."""
    B, S, Hq, Hkv, D = 2, 3, 4, 2, 8
    dm = Hq * D
    x = _rand(B, S, dm)
    eye = np.eye(dm)
    q, k, v = A.qkv_project(x, eye, eye[: Hkv * D], 2 * eye[: Hkv * D], Hq, Hkv)
    for h in range(Hq):
        np.testing.assert_array_equal(q[:, :, h, :], x[:, :, h * D:(h + 1) * D])
    for g in range(Hkv):
        np.testing.assert_array_equal(k[:, :, g, :], x[:, :, g * D:(g + 1) * D])
        np.testing.assert_array_equal(v[:, :, g, :], 2 * x[:, :, g * D:(g + 1) * D])


def test_qkv_project_one_hot_input_reads_a_weight_column():
    """A token whose input is the unit vector e_i projects to column i of
    each weight matrix (not row i: the map is x W^T; Wq is square here so
    that reading it transposed would go unnoticed by the shapes)."""
    Hq, Hkv, D, dm = 2, 1, 3, 6
    wq, wk, wv = _rand(Hq * D, dm), _rand(Hkv * D, dm), _rand(Hkv * D, dm)
    for i in range(dm):
        x = np.zeros((1, 1, dm))
        x[0, 0, i] = 1.0
        q, k, v = A.qkv_project(x, wq, wk, wv, Hq, Hkv)
        np.testing.assert_array_equal(q.reshape(-1), wq[:, i])
        np.testing.assert_array_equal(k.reshape(-1), wk[:, i])
        np.testing.assert_array_equal(v.reshape(-1), wv[:, i])


def test_qkv_project_brute_force_tiny():
    """Scalar loops over (sequence, token, head, dim, input feature)."""
    rng = np.random.default_rng(7)
    B, S, Hq, Hkv, D, dm = 2, 3, 2, 1, 3, 5
    x = rng.standard_normal((B, S, dm))
    ws = [rng.standard_normal((H * D, dm)) for H in (Hq, Hkv, Hkv)]
    got = A.qkv_project(x, ws[0], ws[1], ws[2], Hq, Hkv)
    for out, w, H in zip(got, ws, (Hq, Hkv, Hkv)):
        for b in range(B):
            for s in range(S):
                for h in range(H):
                    for d in range(D):
                        acc = 0.0
                        for i in range(dm):
                            acc += float(x[b, s, i]) * float(w[h * D + d, i])
                        assert abs(out[b, s, h, d] - acc) <= 1e-12 * (1 + abs(acc))


def test_o_project_identity_one_hot_and_brute_force():
    """o_proj reads the heads as one head-major vector: with W_o = I the output
    is the heads concatenated; a one-hot attention output picks a column of
    W_o; scalar loops agree."""
    rng = np.random.default_rng(8)
    B, S, Hq, D = 2, 3, 2, 4
    a = rng.standard_normal((B, S, Hq, D))
    np.testing.assert_array_equal(A.o_project(a, np.eye(Hq * D)), a.reshape(B, S, Hq * D))
    w = rng.standard_normal((Hq * D, Hq * D))  # square, so a transposed read would not fail on shape
    for h in range(Hq):
        for d in range(D):
            e = np.zeros((1, 1, Hq, D))
            e[0, 0, h, d] = 1.0
            np.testing.assert_array_equal(A.o_project(e, w).reshape(-1), w[:, h * D + d])
    w = rng.standard_normal((5, Hq * D))
    y = A.o_project(a, w)
    for b in range(B):
        for s in range(S):
            for o in range(5):
                acc = 0.0
                for h in range(Hq):
                    for d in range(D):
                        acc += float(a[b, s, h, d]) * float(w[o, h * D + d])
                assert abs(y[b, s, o] - acc) <= 1e-12 * (1 + abs(acc))


def test_residual_rms_norm_closed_forms():
    """Without a residual it is the RMSNorm; with one it adds it; RMSNorm of a
    zero row is zero, so a zero sublayer output leaves the residual stream
    unchanged (the block is then the identity)."""
    x = _rand(3, 16)
    g = 1 + 0.1 * _rand(16)
    r = _rand(3, 16)
    np.testing.assert_array_equal(A.residual_rms_norm(x, g, 1e-6), A.rms_norm(x, g, 1e-6))
    np.testing.assert_allclose(A.residual_rms_norm(x, g, 1e-6, residual=r) - r, A.rms_norm(x, g, 1e-6),
                               rtol=0, atol=1e-12)
    c = np.full((1, 16), -3.0)  # constant row: mean square 9, so every value maps to -1 * gamma
    np.testing.assert_allclose(A.residual_rms_norm(c, g, 0.0, residual=r[:1]), r[:1] - g[None, :], atol=1e-12)
    np.testing.assert_array_equal(A.residual_rms_norm(np.zeros((2, 16)), g, 1e-6, residual=r[:2]), r[:2])


def test_attention_block_zero_output_projection_is_identity_and_matches_steps():
    """W_o = 0 makes the sublayer x -> x + post_norm(0) = x; otherwise the block
    equals its steps composed by hand."""
    rng = np.random.default_rng(9)
    B, S, dm, Hq, Hkv, D = 1, 12, 16, 2, 1, 8
    x = rng.standard_normal((B, S, dm))
    wq, wk, wv = (rng.standard_normal((H * D, dm)) / 4 for H in (Hq, Hkv, Hkv))
    gi, gp, gq, gk = (1 + 0.1 * rng.standard_normal(n) for n in (dm, dm, D, D))
    args = (Hq, Hkv, gi, gp, gq, gk, 1e-6, A.LOCAL, 4, 1e4, 1.0)
    np.testing.assert_array_equal(A.attention_block(x, wq, wk, wv, np.zeros((dm, Hq * D)), *args), x)
    wo = rng.standard_normal((dm, Hq * D)) / 4
    got = A.attention_block(x, wq, wk, wv, wo, *args)
    h = A.rms_norm(x, gi, 1e-6)
    q, k, v = h @ wq.T, h @ wk.T, h @ wv.T
    o = A.prefill(q.reshape(B, S, Hq, D), k.reshape(B, S, Hkv, D), v.reshape(B, S, Hkv, D), A.LOCAL, 4, 1e4, 1.0,
                  gq, gk, 1e-6)
    y = o.reshape(B, S, Hq * D) @ wo.T
    np.testing.assert_allclose(got, x + A.rms_norm(y, gp, 1e-6), rtol=0, atol=1e-12)


def _block_inputs(rng, B, S, dm, Hq, Hkv, D):
    x = rng.standard_normal((B, S, dm))
    wq, wk, wv = (rng.standard_normal((H * D, dm)) / 4 for H in (Hq, Hkv, Hkv))
    wo = rng.standard_normal((dm, Hq * D)) / 4
    gi, gp, gq, gk = (1 + 0.3 * rng.standard_normal(n) for n in (dm, dm, D, D))
    return x, wq, wk, wv, wo, gi, gp, gq, gk


@pytest.mark.parametrize("kind", [A.LOCAL, A.GLOBAL])
def test_attention_block_input_norm_makes_the_sublayer_scale_free(kind):
    """With eps = 0 and no QK-norm, the sublayer sees x only through the input
    RMSNorm, which is blind to the scale of x: block(c x) - c x equals
    block(x) - x for any c > 0.  Without that norm (or with it after the
    projections), the logits would grow like c^2 and the softmax change."""
    rng = np.random.default_rng(21)
    B, S, dm, Hq, Hkv, D = 2, 9, 16, 4, 2, 8
    x, wq, wk, wv, wo, gi, gp, _, _ = _block_inputs(rng, B, S, dm, Hq, Hkv, D)
    args = (Hq, Hkv, gi, gp, None, None, 0.0, kind, 3, 1e4, 1.0)
    base = A.attention_block(x, wq, wk, wv, wo, *args) - x
    for c in (0.25, 3.7):
        got = A.attention_block(c * x, wq, wk, wv, wo, *args) - c * x
        np.testing.assert_allclose(got, base, rtol=0, atol=1e-11)


def test_attention_block_adds_rows_of_unit_rms():
    """The post-attention RMSNorm makes what the sublayer adds to the residual
    a row of mean square exactly 1 before its gamma (eps = 0):
    mean(((block(x) - x) / gamma_post)^2) = 1 for every token."""
    rng = np.random.default_rng(22)
    B, S, dm, Hq, Hkv, D = 2, 7, 16, 2, 1, 8
    x, wq, wk, wv, wo, gi, gp, gq, gk = _block_inputs(rng, B, S, dm, Hq, Hkv, D)
    for kind in (A.LOCAL, A.GLOBAL):
        out = A.attention_block(x, wq, wk, wv, wo, Hq, Hkv, gi, gp, gq, gk, 0.0, kind, 4, 1e6, 8.0)
        ms = np.mean(((out - x) / gp) ** 2, axis=-1)
        np.testing.assert_allclose(ms, 1.0, rtol=0, atol=1e-12)


@pytest.mark.parametrize("Hq,Hkv", [(4, 2), (2, 2)])
def test_attention_block_single_token_is_the_value_path(Hq, Hkv):
    """A one-token sequence attends only to itself, and a softmax over one key
    is 1, so attention returns that token's value vector (query head h gets
    kv head h / G).  The sublayer is then
    x + RMSNorm_post(W_o [v of each head's kv group]), v = W_v RMSNorm_in(x),
    written out here with plain array operations; q, k, the rotation and the
    QK-norm drop out."""
    rng = np.random.default_rng(23)
    dm, D, eps = 16, 8, 1e-6
    x, wq, wk, wv, wo, gi, gp, gq, gk = _block_inputs(rng, 1, 1, dm, Hq, Hkv, D)
    xr = x[0, 0]
    h = xr / np.sqrt(np.mean(xr * xr) + eps) * gi
    v = (wv @ h).reshape(Hkv, D)
    G = Hq // Hkv
    heads = np.concatenate([v[i // G] for i in range(Hq)])
    y = wo @ heads
    want = xr + y / np.sqrt(np.mean(y * y) + eps) * gp
    for kind in (A.LOCAL, A.GLOBAL):
        got = A.attention_block(x, wq, wk, wv, wo, Hq, Hkv, gi, gp, gq, gk, eps, kind, 1, 1e4, 1.0, pos0=[5])
        np.testing.assert_allclose(got[0, 0], want, rtol=0, atol=1e-12)
