"""GPU parity of the fused input projection (q/k/v projections with the key
QK-norm + RoPE in the epilogue) and of the prefill that consumes its keys,
through the C ABI, against the fp64 oracle on the same seeded inputs.

Gate for the projections: each output element is one bf16 rounding of an
fp32 result, so |err| <= 2^-8 |ref| (the rounding, 2^-9 relative, with a
factor 2 of slack) plus a floor of 1e-3 of the row's rms for elements near
zero (fp32 accumulation over d_model products: about sqrt(d_model) * 2^-24
of the sum of |x_i w_i|, a few 1e-5 of the rms at d_model = 5376).
"""
import numpy as np
import pytest

import oracle.attention as A
import workloads as W
from tests.gpu_util import assert_parity, dev_bf16, dev_f32, errors, host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import global_gqa_amd as G  # noqa: E402

D = 128


def assert_proj(got, ref, what=""):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    rms = np.sqrt(np.mean(ref * ref, axis=-1, keepdims=True))
    tol = 2.0 ** -8 * np.abs(ref) + 1e-3 * rms
    bad = np.abs(got - ref) > tol
    assert not bad.any(), f"{what}: {bad.sum()} of {bad.size} out of tolerance; worst {np.abs(got - ref)[bad].max()}"


# Max-abs gate on the attention output inside a sublayer.  The attention's
# own bar is 2e-2 on unit-scale bf16 inputs; here its inputs are the
# projections of the bf16-rounded normed input, each rounded to bf16 once,
# while the oracle projects exactly.  That rounding reaches o undamped where
# a row sees few keys (row 0 sees only itself, so o = v): two roundings of
# 2^-9 relative on values up to |v| ~ 5 add ~2e-2, hence 4e-2.  Mean-abs and
# relative L2 keep the attention bar.
MAX_ABS_SUBLAYER_O = 4e-2


def assert_sublayer(got, ref, x):
    """Gate for a whole sublayer's output x + RMSNorm_post(o_proj(attention)).

    The post-attention RMSNorm rescales the attention's o_proj output (of
    size about 1 / sqrt(visible keys)) to unit RMS, so the attention's error,
    absolute and within the attention bar on o, comes out relative to unit
    scale in what the sublayer adds: relative L2 <= 1e-2 on that contribution
    and on the whole output, mean-abs <= 8e-3 (0.8 of the L2 bound, the ratio
    of mean-abs to RMS for normal errors) and max-abs <= 0.1 against
    outliers."""
    assert np.all(np.isfinite(got)), "non-finite sublayer output"
    xr = np.asarray(x, dtype=np.float64)
    ec, e = errors(got - xr, ref - xr), errors(got, ref)
    assert ec["rel_l2"] <= 1e-2 and e["rel_l2"] <= 1e-2, (ec, e)
    assert ec["mean_abs"] <= 8e-3 and ec["max_abs"] <= 0.1, ec


def _proj_inputs(config, B, S, dm, Hq, Hkv):
    x = W.host_normal_bf16((B, S, dm), W.seed_of(config, 0, W.T_X))
    w = W.host_weight_bf16(((Hq + 2 * Hkv) * D, dm), W.seed_of(config, 0, W.T_W))
    gk = W.host_gamma(D, W.seed_of(config, 0, W.T_GK))
    gq = W.host_gamma(D, W.seed_of(config, 0, W.T_GQ))
    return x, w, gq, gk


def _split(w, Hq, Hkv):
    return w[:Hq * D], w[Hq * D:(Hq + Hkv) * D], w[(Hq + Hkv) * D:]


def _oracle_khat(k, gk, pos0, base, scale):
    """[B, S, Hkv, D] raw keys -> [B, Hkv, S, D] normed and rotated."""
    B, S = k.shape[:2]
    out = np.empty((B, k.shape[2], S, D))
    for b in range(B):
        pos = (0 if pos0 is None else pos0[b]) + np.arange(S)
        kh = A.qknorm_rope(k[b], gk, W.EPS, pos, base, scale, gk is not None)
        out[b] = kh.transpose(1, 0, 2)
    return out


@pytest.mark.parametrize("B,S,dm,Hq,Hkv,pos0,base,scale,norm", [
    (2, 300, 256, 4, 2, [0, 5000], 1e6, 8.0, True),    # ragged token tiles spanning two sequences
    (1, 1, 64, 2, 1, None, 1e4, 1.0, True),            # one token, one input chunk
    (3, 77, 128, 8, 1, [9, 9, 9], 1e4, 1.0, False),    # uniform pos0, no norm, two chunks
    (1, 640, 320, 4, 4, [131000], 1e6, 8.0, True),     # 5 full tiles, odd chunk count, far positions
    (2, 130, 64, 3, 1, [0, 1], 1e4, 1.0, True),        # odd head count: the last head pair has one head
    (1, 1024, 128, 2, 2, None, 1e6, 8.0, True),        # exact token tiles, no tail
])
def test_qkv_project_matches_oracle(B, S, dm, Hq, Hkv, pos0, base, scale, norm):
    x, w, _, gk = _proj_inputs(20, B, S, dm, Hq, Hkv)
    gk = gk if norm else None
    print(f"qkv_project B={B} S={S} d_model={dm} Hq={Hq} Hkv={Hkv}", flush=True)
    q, kh, v = G.qkv_project(dev_bf16(x), dev_bf16(w), Hq, Hkv, base, scale,
                             dev_f32(gk) if norm else None, W.EPS, pos0)
    torch.cuda.synchronize()
    wq, wk, wv = _split(w, Hq, Hkv)
    rq, rk, rv = A.qkv_project(x, wq, wk, wv, Hq, Hkv)
    assert_proj(host(q), rq, "q")
    assert_proj(host(v), rv, "v")
    assert_proj(host(kh), _oracle_khat(rk, gk, pos0, base, scale), "khat")


def test_qkv_project_deterministic_and_writes_every_element():
    B, S, dm, Hq, Hkv = 2, 200, 192, 4, 2
    x, w, _, gk = _proj_inputs(21, B, S, dm, Hq, Hkv)
    xd, wd, gkd = dev_bf16(x), dev_bf16(w), dev_f32(gk)
    outs = []
    for fill in (float("nan"), 7.0):
        q = torch.full((B, S, Hq, D), fill, dtype=torch.bfloat16, device="cuda")
        kh = torch.full((B, Hkv, S, D), fill, dtype=torch.bfloat16, device="cuda")
        v = torch.full((B, S, Hkv, D), fill, dtype=torch.bfloat16, device="cuda")
        G.qkv_project(xd, wd, Hq, Hkv, 1e4, 1.0, gkd, W.EPS, None, q=q, khat=kh, v=v)
        torch.cuda.synchronize()
        outs.append((q, kh, v))
    for a, b in zip(*outs):
        assert bool(torch.isfinite(a.float()).all()), "an output element was left unwritten"
        assert bool(torch.equal(a, b)), "results differ between identical calls"


@pytest.mark.parametrize("kind", [A.LOCAL, A.GLOBAL])
def test_qkv_project_then_prefill_khat_end_to_end(kind):
    """x -> projections (keys normed + rotated in the epilogue) -> flash
    prefill reading those keys, against oracle projections then the oracle
    prefill; image spans, per-sequence first positions, ragged S."""
    B, S, dm, Hq, Hkv = 2, 700, 256, 4, 2
    x, w, gq, gk = _proj_inputs(22, B, S, dm, Hq, Hkv)
    pos0 = [0, 300]
    spans = [W.image_spans(S, 2, 91, base=0), W.image_spans(S, 1, 92, base=300)]
    flat = [(b, s, e) for b in range(B) for (s, e) in spans[b]]
    base, scale = (W.ROPE_BASE_LOCAL, 1.0) if kind == A.LOCAL else (W.ROPE_BASE_GLOBAL, 8.0)
    window = 256
    q, kh, v = G.qkv_project(dev_bf16(x), dev_bf16(w), Hq, Hkv, base, scale, dev_f32(gk), W.EPS, pos0)
    o = G.prefill_khat(q, kh, v, kind, window, base, scale, dev_f32(gq), W.EPS, 0.0, flat, pos0)
    torch.cuda.synchronize()
    wq, wk, wv = _split(w, Hq, Hkv)
    rq, rk, rv = A.qkv_project(x, wq, wk, wv, Hq, Hkv)
    ref = A.prefill(rq, rk, rv, kind, window, base, scale, gq, gk, W.EPS, spans=spans, pos0=pos0)
    assert_parity(host(o), ref, f"qkv -> prefill_khat kind={kind}")


def test_prefill_khat_equals_prefill_on_same_keys():
    """Given the keys that the library's own prologue makes (qknorm_rope in
    head-major order), prefill_khat and prefill launch the same flash kernel
    and must agree bit for bit."""
    B, S, Hq, Hkv = 2, 500, 8, 2
    rng_q = W.host_normal_bf16((B, S, Hq, D), 31)
    rng_k = W.host_normal_bf16((B, S, Hkv, D), 32)
    rng_v = W.host_normal_bf16((B, S, Hkv, D), 33)
    gq, gk = W.host_gamma(D, 34), W.host_gamma(D, 35)
    qd, kd, vd = dev_bf16(rng_q), dev_bf16(rng_k), dev_bf16(rng_v)
    pos0 = [3, 1000]
    for kind, base, scale in ((A.LOCAL, 1e4, 1.0), (A.GLOBAL, 1e6, 8.0)):
        o1 = G.prefill(qd, kd, vd, kind, 300, base, scale, dev_f32(gq), dev_f32(gk), W.EPS, pos0=pos0)
        pos = torch.tensor([p + s for p in pos0 for s in range(S)], dtype=torch.int32, device="cuda")
        _, kr = G.qknorm_rope(None, kd.view(B * S, Hkv, D), pos, None, dev_f32(gk), W.EPS, base, scale)
        kh = kr.view(B, S, Hkv, D).permute(0, 2, 1, 3).contiguous()
        o2 = G.prefill_khat(qd, kh, vd, kind, 300, base, scale, dev_f32(gq), W.EPS, pos0=pos0)
        torch.cuda.synchronize()
        assert bool(torch.equal(o1, o2)), f"kind={kind}: prefill_khat differs from prefill"


@pytest.mark.parametrize("is_ring,cap", [(True, 1024), (False, 2048)])
def test_qkv_project_chunks_into_cache(is_ring, cap):
    """Two 600-token chunks of one local layer: each chunk's keys come from
    the projection, prefill_khat attends to the cache and appends; the
    second chunk's output equals rows [600, 1200) of the oracle prefill of
    the whole 1200 tokens, and the cache holds the oracle's keys."""
    B, C, dm, Hq, Hkv, window = 1, 600, 128, 4, 2, 1024
    x, w, gq, gk = _proj_inputs(23, B, 2 * C, dm, Hq, Hkv)
    base, scale = W.ROPE_BASE_LOCAL, 1.0
    cache = G.KVCache.empty(B, Hkv, cap, D, is_ring=is_ring)
    xd, wd = dev_bf16(x), dev_bf16(w)
    outs = []
    for c in range(2):
        xc = xd[:, c * C:(c + 1) * C].contiguous()
        q, kh, v = G.qkv_project(xc, wd, Hq, Hkv, base, scale, dev_f32(gk), W.EPS, [c * C])
        outs.append(G.prefill_khat(q, kh, v, A.LOCAL, window, base, scale, dev_f32(gq), W.EPS, pos0=[c * C],
                                   cache=cache))
    torch.cuda.synchronize()
    wq, wk, wv = _split(w, Hq, Hkv)
    rq, rk, rv = A.qkv_project(x, wq, wk, wv, Hq, Hkv)
    ref = A.prefill(rq, rk, rv, A.LOCAL, window, base, scale, gq, gk, W.EPS)
    assert_parity(host(outs[1]), ref[:, C:], f"second chunk ring={is_ring}")
    assert_parity(host(outs[0]), ref[:, :C], f"first chunk ring={is_ring}")
    kref = _oracle_khat(rk, gk, None, base, scale)  # [B, Hkv, 2C, D]
    n = 2 * C
    pos = np.arange(max(0, n - cap), n)
    slots = pos % cap if is_ring else pos
    assert_proj(host(cache.k)[:, :, slots], kref[:, :, pos], "cached keys")
    assert_proj(host(cache.v)[:, :, slots], rv[:, pos].transpose(0, 2, 1, 3), "cached values")


def test_qkv_project_27b_sampled_rows():
    """The 27B layer shape at the prefill bench size: x [1, 8192, 5376],
    W [(32 + 2 * 16) * 128, 5376]; the oracle projects 48 sampled tokens
    (first and last of the sequence and of tiles included) for every head."""
    B, S, dm, Hq, Hkv = 1, 8192, W.D_MODEL_27B, 32, 16
    x, w, _, gk = _proj_inputs(24, B, S, dm, Hq, Hkv)
    base, scale = W.ROPE_BASE_GLOBAL, 8.0
    print("qkv_project 27B 8192 x 5376", flush=True)
    q, kh, v = G.qkv_project(dev_bf16(x), dev_bf16(w), Hq, Hkv, base, scale, dev_f32(gk), W.EPS)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    toks = np.unique(np.concatenate([[0, 127, 128, 4095, 8191], rng.integers(0, S, 43)]))
    wq, wk, wv = _split(w, Hq, Hkv)
    rq, rk, rv = A.qkv_project(x[:, toks], wq, wk, wv, Hq, Hkv)
    ti = torch.as_tensor(toks, device="cuda")
    assert_proj(host(q[:, ti]), rq, "q")
    assert_proj(host(v[:, ti]), rv, "v")
    kh_s = host(kh[:, :, ti])  # [B, Hkv, n, D]
    ref = np.empty_like(kh_s)
    kn = A.qknorm_rope(rk[0], gk, W.EPS, toks, base, scale, True)  # positions = token indices
    ref[0] = kn.transpose(1, 0, 2)
    assert_proj(kh_s, ref, "khat")


@pytest.mark.parametrize("T,n_in,n_out", [(300, 256, 384), (1, 64, 128), (1024, 128, 256)])
def test_o_project_matches_oracle(T, n_in, n_out):
    """Ragged token tiles, a single token, an odd number of 128-feature
    blocks (the last tile has one), exact tiles."""
    a = W.host_normal_bf16((1, T, n_in // 64, 64), W.seed_of(25, T, W.T_X))  # heads of 64 values
    w = W.host_weight_bf16((n_out, n_in), W.seed_of(25, T, W.T_W))
    y = G.o_project(dev_bf16(a), dev_bf16(w))
    torch.cuda.synchronize()
    assert tuple(y.shape) == (1, T, n_out)
    assert_proj(host(y), A.o_project(a, w), "y")


def test_o_project_27b_sampled_rows():
    """The 27B o_proj (4096 -> 5376) over 8192 tokens; the oracle projects 40
    sampled tokens."""
    T, Hq = 8192, 32
    a = W.host_normal_bf16((1, T, Hq, D), W.seed_of(26, 0, W.T_X))
    w = W.host_weight_bf16((W.D_MODEL_27B, Hq * D), W.seed_of(26, 0, W.T_W))
    print("o_project 27B 8192 x 4096 -> 5376", flush=True)
    y = G.o_project(dev_bf16(a), dev_bf16(w))
    torch.cuda.synchronize()
    toks = np.unique(np.concatenate([[0, 255, 256, 8191], np.random.default_rng(6).integers(0, T, 36)]))
    ti = torch.as_tensor(toks, device="cuda")
    assert_proj(host(y[:, ti]), A.o_project(a[:, toks], w), "y")


@pytest.mark.parametrize("T,width,residual,gamma", [(300, 5376, True, True), (7, 1152, False, True),
                                                    (64, 64, True, False), (3, 8192, False, False)])
def test_rmsnorm_matches_oracle(T, width, residual, gamma):
    x = W.bf16_round(W.host_normal_bf16((T, width), W.seed_of(27, width, W.T_X)) * 3.0)  # both sides see these bf16 values
    r = W.host_normal_bf16((T, width), W.seed_of(27, width, W.T_Q)) if residual else None
    g = W.host_gamma(width, W.seed_of(27, width, W.T_GK)) if gamma else None
    out = G.rmsnorm(dev_bf16(x), dev_f32(g) if gamma else None, W.EPS, residual=dev_bf16(r) if residual else None)
    torch.cuda.synchronize()
    assert_proj(host(out), A.residual_rms_norm(x, g, W.EPS, residual=r), "rmsnorm")
    if residual:  # in place into the residual stream
        rd = dev_bf16(r)
        G.rmsnorm(dev_bf16(x), dev_f32(g) if gamma else None, W.EPS, residual=rd, out=rd)
        torch.cuda.synchronize()
        assert bool(torch.equal(rd, out)), "in-place result differs"


@pytest.mark.parametrize("kind", [A.LOCAL, A.GLOBAL])
def test_attention_block_from_input_end_to_end(kind):
    """The whole attention sublayer through the library: input RMSNorm, fused
    q/k/v projection, prefill on the projected keys, o_proj, post-attention
    RMSNorm added to the residual; against the oracle's block."""
    B, S, dm, Hq, Hkv = 2, 500, 256, 4, 2
    x = W.host_normal_bf16((B, S, dm), W.seed_of(28, kind, W.T_X))
    w = W.host_weight_bf16(((Hq + 2 * Hkv) * D, dm), W.seed_of(28, kind, W.T_W))
    wo = W.host_weight_bf16((dm, Hq * D), W.seed_of(28, kind, W.T_V))
    gq, gk = W.host_gamma(D, W.seed_of(28, kind, W.T_GQ)), W.host_gamma(D, W.seed_of(28, kind, W.T_GK))
    gi, gp = W.host_gamma(dm, W.seed_of(28, kind, W.T_CK)), W.host_gamma(dm, W.seed_of(28, kind, W.T_CV))
    base, scale = (W.ROPE_BASE_LOCAL, 1.0) if kind == A.LOCAL else (W.ROPE_BASE_GLOBAL, 8.0)
    window = 200
    xd = dev_bf16(x)
    h = G.rmsnorm(xd, dev_f32(gi), W.EPS)
    q, kh, v = G.qkv_project(h, dev_bf16(w), Hq, Hkv, base, scale, dev_f32(gk), W.EPS)
    o = G.prefill_khat(q, kh, v, kind, window, base, scale, dev_f32(gq), W.EPS)
    y = G.o_project(o, dev_bf16(wo))
    out = G.rmsnorm(y, dev_f32(gp), W.EPS, residual=xd)
    torch.cuda.synchronize()
    wq, wk, wv = _split(w, Hq, Hkv)
    ref = A.attention_block(x, wq, wk, wv, wo, Hq, Hkv, gi, gp, gq, gk, W.EPS, kind, window, base, scale)
    # the attention output itself, at the bar every attention output meets
    rq, rk, rv = A.qkv_project(A.residual_rms_norm(x, gi, W.EPS), wq, wk, wv, Hq, Hkv)
    assert_parity(host(o), A.prefill(rq, rk, rv, kind, window, base, scale, gq, gk, W.EPS), "attention output",
                  max_abs=MAX_ABS_SUBLAYER_O)
    assert_sublayer(host(out), ref, x)


# ---------------------------------------------------------------- head dim 256 (Gemma 3 1B)
def _proj_inputs_d(config, B, S, dm, Hq, Hkv, Dh):
    x = W.host_normal_bf16((B, S, dm), W.seed_of(config, 0, W.T_X))
    w = W.host_weight_bf16(((Hq + 2 * Hkv) * Dh, dm), W.seed_of(config, 0, W.T_W))
    gq, gk = W.host_gamma(Dh, W.seed_of(config, 0, W.T_GQ)), W.host_gamma(Dh, W.seed_of(config, 0, W.T_GK))
    return x, w, gq, gk


@pytest.mark.parametrize("B,S,dm,Hq,Hkv,pos0,norm", [
    (2, 300, 256, 4, 1, [0, 7000], True),      # ragged tiles over two sequences, per-sequence positions
    (1, 1, 64, 2, 2, None, True),              # one token, one input chunk
    (1, 513, 1152, 4, 1, None, False),         # the 1B width (1152 = 36 chunks), no norm
])
def test_qkv_project_d256_matches_oracle(B, S, dm, Hq, Hkv, pos0, norm):
    """Head dimension 256: the key's RMSNorm and its RoPE pairs (d, d + 128)
    span the two waves that hold the head's halves."""
    Dh = 256
    x, w, _, gk = _proj_inputs_d(29, B, S, dm, Hq, Hkv, Dh)
    gk = gk if norm else None
    print(f"qkv_project D=256 B={B} S={S} d_model={dm}", flush=True)
    q, kh, v = G.qkv_project(dev_bf16(x), dev_bf16(w), Hq, Hkv, 1e6, 8.0, dev_f32(gk) if norm else None, W.EPS, pos0)
    torch.cuda.synchronize()
    wq, wk, wv = w[:Hq * Dh], w[Hq * Dh:(Hq + Hkv) * Dh], w[(Hq + Hkv) * Dh:]
    rq, rk, rv = A.qkv_project(x, wq, wk, wv, Hq, Hkv)
    assert_proj(host(q), rq, "q")
    assert_proj(host(v), rv, "v")
    ref = np.empty((B, Hkv, S, Dh))
    for b in range(B):
        pos = (0 if pos0 is None else pos0[b]) + np.arange(S)
        ref[b] = A.qknorm_rope(rk[b], gk, W.EPS, pos, 1e6, 8.0, norm).transpose(1, 0, 2)
    assert_proj(host(kh), ref, "khat")


def test_attention_block_d256_from_input():
    """A Gemma 3 1B-shaped sublayer (d_model 1152, 4 query heads and 1 kv
    head of 256) from its input, local layer, against the oracle's block."""
    B, S, dm, Hq, Hkv, Dh = 1, 700, 1152, 4, 1, 256
    x, w, gq, gk = _proj_inputs_d(30, B, S, dm, Hq, Hkv, Dh)
    wo = W.host_weight_bf16((dm, Hq * Dh), W.seed_of(30, 0, W.T_V))
    gi, gp = W.host_gamma(dm, W.seed_of(30, 0, W.T_CK)), W.host_gamma(dm, W.seed_of(30, 0, W.T_CV))
    window = 300
    xd = dev_bf16(x)
    h = G.rmsnorm(xd, dev_f32(gi), W.EPS)
    q, kh, v = G.qkv_project(h, dev_bf16(w), Hq, Hkv, W.ROPE_BASE_LOCAL, 1.0, dev_f32(gk), W.EPS)
    o = G.prefill_khat(q, kh, v, A.LOCAL, window, W.ROPE_BASE_LOCAL, 1.0, dev_f32(gq), W.EPS)
    out = G.rmsnorm(G.o_project(o, dev_bf16(wo)), dev_f32(gp), W.EPS, residual=xd)
    torch.cuda.synchronize()
    wq, wk, wv = w[:Hq * Dh], w[Hq * Dh:(Hq + Hkv) * Dh], w[(Hq + Hkv) * Dh:]
    ref = A.attention_block(x, wq, wk, wv, wo, Hq, Hkv, gi, gp, gq, gk, W.EPS, A.LOCAL, window, W.ROPE_BASE_LOCAL, 1.0)
    rq, rk, rv = A.qkv_project(A.residual_rms_norm(x, gi, W.EPS), wq, wk, wv, Hq, Hkv)
    assert_parity(host(o), A.prefill(rq, rk, rv, A.LOCAL, window, W.ROPE_BASE_LOCAL, 1.0, gq, gk, W.EPS),
                  "attention output", max_abs=MAX_ABS_SUBLAYER_O)
    assert_sublayer(host(out), ref, x)


# ---------------------------------------------------------------- input norm folded into the projection
# (x / rms(x) * gamma) W^T = (1 / rms(x)) * x (W diag(gamma))^T: the gamma goes
# into the weight once, the per-token 1 / rms(x) is applied to the fp32
# projections, and the normed copy of x is never written.
@pytest.mark.parametrize("T,width", [(300, 5376), (7, 1152), (5, 8), (64, 8192)])
def test_rms_scale_matches_definition(T, width):
    x = W.bf16_round(W.host_normal_bf16((T, width), W.seed_of(40, width, W.T_X)) * 2.5)
    s = G.rms_scale(dev_bf16(x), W.EPS)
    torch.cuda.synchronize()
    xr = x.astype(np.float64)
    ref = 1.0 / np.sqrt(np.mean(xr * xr, axis=-1) + W.EPS)
    # fp32 sum of squares and reciprocal square root: a few ulp of fp32
    np.testing.assert_allclose(host(s), ref, rtol=1e-5, atol=0)


@pytest.mark.parametrize("rows,width", [(384, 256), (3, 1152), (1, 8)])
def test_fold_norm_weight_is_one_rounding_of_the_product(rows, width):
    w = W.host_weight_bf16((rows, width), W.seed_of(41, width, W.T_W))
    g = W.host_gamma(width, W.seed_of(41, width, W.T_GK))
    out = G.fold_norm_weight(dev_bf16(w), dev_f32(g))
    torch.cuda.synchronize()
    ref = W.bf16_round(w.astype(np.float32) * g.astype(np.float32))
    assert np.array_equal(host(out), ref.astype(np.float64))
    wd = dev_bf16(w)
    G.fold_norm_weight(wd, dev_f32(g), out=wd)  # in place
    torch.cuda.synchronize()
    assert np.array_equal(host(wd), ref.astype(np.float64))


@pytest.mark.parametrize("Dh,B,S,dm,Hq,Hkv,pos0", [
    (128, 2, 300, 256, 4, 2, [0, 5000]),
    (128, 1, 640, 320, 3, 1, None),
    (256, 1, 513, 1152, 4, 1, [17]),
])
def test_qkv_project_with_x_scale_matches_oracle(Dh, B, S, dm, Hq, Hkv, pos0):
    """The folded projection computes x W'^T times the token's scale: against
    the oracle's projection of the exactly scaled x with the same folded
    weights (W' rounded to bf16 on the host), at the projection's own gate."""
    x = W.host_normal_bf16((B, S, dm), W.seed_of(42, Dh, W.T_X))
    w = W.host_weight_bf16(((Hq + 2 * Hkv) * Dh, dm), W.seed_of(42, Dh, W.T_W))
    gi = W.host_gamma(dm, W.seed_of(42, Dh, W.T_CK))
    gk = W.host_gamma(Dh, W.seed_of(42, Dh, W.T_GK))
    base, scale = 1e6, 8.0
    xd = dev_bf16(x)
    sc = G.rms_scale(xd, W.EPS)
    wf = G.fold_norm_weight(dev_bf16(w), dev_f32(gi))
    print(f"qkv_project x_scale D={Dh} B={B} S={S} d_model={dm}", flush=True)
    q, kh, v = G.qkv_project(xd, wf, Hq, Hkv, base, scale, dev_f32(gk), W.EPS, pos0, x_scale=sc)
    torch.cuda.synchronize()
    xr = x.astype(np.float64)
    xs = xr / np.sqrt(np.mean(xr * xr, axis=-1, keepdims=True) + W.EPS)
    wfold = W.bf16_round(w.astype(np.float32) * gi.astype(np.float32))
    wq, wk, wv = wfold[:Hq * Dh], wfold[Hq * Dh:(Hq + Hkv) * Dh], wfold[(Hq + Hkv) * Dh:]
    rq, rk, rv = A.qkv_project(xs, wq, wk, wv, Hq, Hkv)
    assert_proj(host(q), rq, "q")
    assert_proj(host(v), rv, "v")
    ref = np.empty((B, Hkv, S, Dh))
    for b in range(B):
        pos = (0 if pos0 is None else pos0[b]) + np.arange(S)
        ref[b] = A.qknorm_rope(rk[b], gk, W.EPS, pos, base, scale, True).transpose(1, 0, 2)
    assert_proj(host(kh), ref, "khat")


@pytest.mark.parametrize("Dh,kind", [(128, A.LOCAL), (128, A.GLOBAL), (256, A.LOCAL)])
def test_attention_block_folded_input_norm_end_to_end(Dh, kind):
    """The whole sublayer with the input RMSNorm folded into the projection
    (rms_scale + fold_norm_weight + qkv_project(x_scale)), against the
    oracle's block, at the same gates as the unfolded sublayer."""
    B, S, Hq, Hkv = (2, 500, 4, 2) if Dh == 128 else (1, 700, 4, 1)
    dm = 256 if Dh == 128 else 1152
    cfg = 43 + Dh
    x = W.host_normal_bf16((B, S, dm), W.seed_of(cfg, kind, W.T_X))
    w = W.host_weight_bf16(((Hq + 2 * Hkv) * Dh, dm), W.seed_of(cfg, kind, W.T_W))
    wo = W.host_weight_bf16((dm, Hq * Dh), W.seed_of(cfg, kind, W.T_V))
    gq, gk = W.host_gamma(Dh, W.seed_of(cfg, kind, W.T_GQ)), W.host_gamma(Dh, W.seed_of(cfg, kind, W.T_GK))
    gi, gp = W.host_gamma(dm, W.seed_of(cfg, kind, W.T_CK)), W.host_gamma(dm, W.seed_of(cfg, kind, W.T_CV))
    base, scale = (W.ROPE_BASE_LOCAL, 1.0) if kind == A.LOCAL else (W.ROPE_BASE_GLOBAL, 8.0)
    window = 200
    xd = dev_bf16(x)
    wf = G.fold_norm_weight(dev_bf16(w), dev_f32(gi))
    q, kh, v = G.qkv_project(xd, wf, Hq, Hkv, base, scale, dev_f32(gk), W.EPS, x_scale=G.rms_scale(xd, W.EPS))
    o = G.prefill_khat(q, kh, v, kind, window, base, scale, dev_f32(gq), W.EPS)
    out = G.rmsnorm(G.o_project(o, dev_bf16(wo)), dev_f32(gp), W.EPS, residual=xd)
    torch.cuda.synchronize()
    wq, wk, wv = w[:Hq * Dh], w[Hq * Dh:(Hq + Hkv) * Dh], w[(Hq + Hkv) * Dh:]
    ref = A.attention_block(x, wq, wk, wv, wo, Hq, Hkv, gi, gp, gq, gk, W.EPS, kind, window, base, scale)
    rq, rk, rv = A.qkv_project(A.residual_rms_norm(x, gi, W.EPS), wq, wk, wv, Hq, Hkv)
    assert_parity(host(o), A.prefill(rq, rk, rv, kind, window, base, scale, gq, gk, W.EPS), "attention output",
                  max_abs=MAX_ABS_SUBLAYER_O)
    assert_sublayer(host(out), ref, x)


def test_qkv_project_x_scale_27b_sampled_rows():
    """The folded input norm at the 27B layer shape (8192 tokens, d_model
    5376): raw x, the norm's gamma folded into W, the per-token scale from
    rms_scale; the oracle projects 40 sampled tokens of the exactly normed x
    with the host-folded weights."""
    B, S, dm, Hq, Hkv = 1, 8192, W.D_MODEL_27B, 32, 16
    x, w, _, gk = _proj_inputs(47, B, S, dm, Hq, Hkv)
    gi = W.host_gamma(dm, W.seed_of(47, 0, W.T_CK))
    base, scale = W.ROPE_BASE_LOCAL, 1.0
    print("qkv_project x_scale 27B 8192 x 5376", flush=True)
    xd = dev_bf16(x)
    q, kh, v = G.qkv_project(xd, G.fold_norm_weight(dev_bf16(w), dev_f32(gi)), Hq, Hkv, base, scale, dev_f32(gk),
                             W.EPS, x_scale=G.rms_scale(xd, W.EPS))
    torch.cuda.synchronize()
    toks = np.unique(np.concatenate([[0, 255, 256, 8191], np.random.default_rng(7).integers(0, S, 36)]))
    xr = x[:, toks].astype(np.float64)
    xs = xr / np.sqrt(np.mean(xr * xr, axis=-1, keepdims=True) + W.EPS)
    wf = W.bf16_round(w.astype(np.float32) * gi.astype(np.float32))
    rq, rk, rv = A.qkv_project(xs, *_split(wf, Hq, Hkv), Hq, Hkv)
    ti = torch.as_tensor(toks, device="cuda")
    assert_proj(host(q[:, ti]), rq, "q")
    assert_proj(host(v[:, ti]), rv, "v")
    ref = A.qknorm_rope(rk[0], gk, W.EPS, toks, base, scale, True).transpose(1, 0, 2)[None]
    assert_proj(host(kh[:, :, ti]), ref, "khat")
