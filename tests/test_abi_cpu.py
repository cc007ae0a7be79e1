"""The C-ABI library loads, exports every declared symbol, and rejects bad
arguments before any launch (no GPU needed: nothing here reaches a kernel)."""
import ctypes
import os
import re

import pytest

import global_gqa_amd as G

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "g3attn.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(g3attn_\w+)\s*\(", src)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(G.LIB_PATH):
        pytest.skip("libg3attn.so not built")
    return G.lib()


def test_exports_every_declared_symbol(L):
    names = _declared()
    assert {"g3attn_qknorm_rope", "g3attn_prefill", "g3attn_decode"} <= set(names)
    for n in names:
        assert hasattr(L, n), n
    assert L.g3attn_version() >= 101


def test_workspace_sizes(L):
    assert L.g3attn_prefill_workspace_size(1, 8192, 32, 16, 128) == 16 * 8192 * 128 * 2 + 16 * 32 * 8 * 4
    assert L.g3attn_prefill_workspace_size(0, 8192, 32, 16, 128) == 0
    ring = G.KVCacheC(0, 0, 1024, 1)
    lin = G.KVCacheC(0, 0, 40000, 0)
    # ring: one split (512 sequence x kv-head pairs); linear: positions 0..32768 in splits of 4096 -> 9
    assert L.g3attn_decode_workspace_size(32, 32, 16, 128, 32768, ctypes.byref(ring)) == 32 * 32 * 1 * 130 * 4
    # fewer pairs (32): the ring splits into 128-slot pieces (8 x 32 = 256 workgroups, one per CU)
    assert L.g3attn_decode_workspace_size(2, 32, 16, 128, 32768, ctypes.byref(ring)) == 2 * 32 * 8 * 130 * 4
    assert L.g3attn_decode_workspace_size(32, 32, 16, 128, 32768, ctypes.byref(lin)) == 32 * 32 * 9 * 130 * 4
    # head dim 256 (Gemma 3 1B: 4 query heads, 1 kv head): keys [1][1][4096][256] bf16, then 8 flags per
    # 256-position tile of G = 1 (8 waves x 32 rows; the most work items any group size gives)
    assert L.g3attn_prefill_workspace_size(1, 4096, 4, 1, 256) == 4096 * 256 * 2 + 16 * 8 * 4
    # 4 sequence x kv-head pairs over 128 units of 256 slots: one-unit splits give 512 workgroups, at least
    # one per CU, so the split stays at 256 slots -> 128 splits
    assert L.g3attn_decode_workspace_size(4, 4, 1, 256, 32767, ctypes.byref(G.KVCacheC(0, 0, 32768, 0))) == \
        4 * 4 * 128 * 258 * 4
    assert L.g3attn_decode_workspace_size(1, 4, 1, 64, 100, ctypes.byref(ring)) == 0


FAKE = 1 << 20  # a 16-byte aligned non-null address: validation fails before any use


def _prefill(L, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, B=1, S=64, Hq=4, Hkv=2, D=128, kind=G.LOCAL, window=1024,
             base=1e4, scale=1.0, gq=None, gk=None, eps=1e-6, sm=0.0, spans=None, n_spans=0, pos0=None, cache=None,
             ws=FAKE, ws_bytes=1 << 30, stream=None)
    a.update(kw)
    return L.g3attn_prefill(a["q"], a["k"], a["v"], a["o"], a["B"], a["S"], a["Hq"], a["Hkv"], a["D"], a["kind"],
                            a["window"], a["base"], a["scale"], a["gq"], a["gk"], a["eps"], a["sm"], a["spans"],
                            a["n_spans"], a["pos0"], a["cache"], a["ws"], a["ws_bytes"], a["stream"])


def _err(L):
    return L.g3attn_last_error().decode()


def test_prefill_validation_errors(L):
    assert _prefill(L, D=64) == G.G3_EUNSUPPORTED and "D=64" in _err(L)
    assert _prefill(L, Hq=6, Hkv=4) == G.G3_EINVAL and "multiple" in _err(L)
    assert _prefill(L, Hq=6, Hkv=2) == G.G3_EUNSUPPORTED
    assert _prefill(L, S=0) == G.G3_EINVAL
    assert _prefill(L, kind=7) == G.G3_EINVAL
    assert _prefill(L, window=0) == G.G3_EINVAL
    assert _prefill(L, base=0.5) == G.G3_EINVAL
    assert _prefill(L, scale=0.0) == G.G3_EINVAL
    assert _prefill(L, sm=-1.0) == G.G3_EINVAL
    assert _prefill(L, q=FAKE + 2) == G.G3_EINVAL and "aligned" in _err(L)
    assert _prefill(L, ws_bytes=10) == G.G3_EWORKSPACE
    assert _prefill(L, ws=FAKE + 16) == G.G3_EINVAL
    # per-sequence element offsets are 32-bit: S * Hkv * D must stay below 2^31
    assert _prefill(L, S=1 << 20, Hq=16, Hkv=16) == G.G3_EUNSUPPORTED and "32-bit" in _err(L)
    sp = (G.Span * 2)(G.Span(0, 10, 20), G.Span(0, 15, 30))
    assert _prefill(L, spans=sp, n_spans=2) == G.G3_EINVAL and "overlapping" in _err(L)
    sp = (G.Span * 1)(G.Span(0, 60, 70))
    assert _prefill(L, spans=sp, n_spans=1) == G.G3_EINVAL and "outside" in _err(L)
    sp = (G.Span * 1)(G.Span(1, 0, 8))
    assert _prefill(L, spans=sp, n_spans=1) == G.G3_EINVAL
    assert _prefill(L, n_spans=65, spans=sp) == G.G3_EINVAL
    ring = G.KVCacheC(FAKE, FAKE, 512, 1)
    assert _prefill(L, cache=ctypes.byref(ring)) == G.G3_EINVAL and "ring" in _err(L)
    ring = G.KVCacheC(FAKE, FAKE, 1024, 1)
    assert _prefill(L, cache=ctypes.byref(ring), kind=G.GLOBAL) == G.G3_EINVAL
    lin = G.KVCacheC(FAKE, FAKE, 100, 0)
    p0 = (ctypes.c_int32 * 1)(50)
    assert _prefill(L, cache=ctypes.byref(lin), pos0=p0) == G.G3_EINVAL and "capacity" in _err(L)
    p0 = (ctypes.c_int32 * 1)(-1)
    assert _prefill(L, pos0=p0) == G.G3_EINVAL


def test_decode_validation_errors(L):
    ring = G.KVCacheC(FAKE, FAKE, 1024, 1)
    lin = G.KVCacheC(FAKE, FAKE, 1000, 0)

    def dec(**kw):
        a = dict(B=2, Hq=4, Hkv=2, D=128, maxp=500, cache=ctypes.byref(ring), kind=G.LOCAL, window=1024,
                 ws_bytes=1 << 30, positions=FAKE)
        a.update(kw)
        return L.g3attn_decode(FAKE, FAKE, FAKE, FAKE, a["B"], a["Hq"], a["Hkv"], a["D"], a["positions"], a["maxp"],
                               a["cache"], a["kind"], a["window"], 1e4, 1.0, None, None, 1e-6, 0.0, FAKE,
                               a["ws_bytes"], None)
    assert dec(D=64) == G.G3_EUNSUPPORTED and "D=64" in _err(L)
    assert dec(B=0) == G.G3_EINVAL
    assert dec(cache=None) == G.G3_EINVAL
    assert dec(positions=None) == G.G3_EINVAL
    assert dec(window=2048) == G.G3_EINVAL
    assert dec(kind=G.GLOBAL) == G.G3_EINVAL
    assert dec(cache=ctypes.byref(lin), kind=G.GLOBAL, maxp=1000) == G.G3_EINVAL and "capacity" in _err(L)
    assert dec(ws_bytes=100) == G.G3_EWORKSPACE
    assert dec(maxp=-1) == G.G3_EINVAL


def test_qknorm_rope_validation_errors(L):
    def call(**kw):
        a = dict(q=FAKE, k=FAKE, qo=FAKE, ko=FAKE, T=4, Hq=4, Hkv=2, D=128, base=1e4, scale=1.0, pos=FAKE)
        a.update(kw)
        return L.g3attn_qknorm_rope(a["q"], a["k"], a["qo"], a["ko"], None, None, 1e-6, a["pos"], a["T"], a["Hq"],
                                    a["Hkv"], a["D"], a["base"], a["scale"], None)
    assert call(D=64) == G.G3_EUNSUPPORTED
    assert call(qo=None) == G.G3_EINVAL
    assert call(pos=None) == G.G3_EINVAL
    assert call(scale=-1.0) == G.G3_EINVAL
    assert call(T=-1) == G.G3_EINVAL
    assert call(T=0) == G.G3_OK  # nothing to do, nothing launched


def test_timing_events_hook_validation(L):
    assert L.g3attn_set_timing_events(FAKE, None) == G.G3_EINVAL
    assert L.g3attn_set_timing_events(None, None) == G.G3_OK


def test_layer_schedule_matches_oracle():
    import oracle

    assert [G.layer_kind(i) for i in range(62)] == [oracle.layer_kind(i) for i in range(62)]


def test_qkv_project_validation_errors(L):
    def call(**kw):
        a = dict(x=FAKE, w=FAKE, q=FAKE, kh=FAKE, v=FAKE, B=1, S=64, dm=256, Hq=4, Hkv=2, D=128, base=1e4,
                 scale=1.0, eps=1e-6, pos0=None)
        a.update(kw)
        return L.g3attn_qkv_project(a["x"], None, a["w"], a["q"], a["kh"], a["v"], a["B"], a["S"], a["dm"],
                                    a["Hq"], a["Hkv"], a["D"], a["base"], a["scale"], None, a["eps"], a["pos0"],
                                    None)
    assert call(D=64) == G.G3_EUNSUPPORTED and "128 or 256" in _err(L)
    assert call(dm=100) == G.G3_EUNSUPPORTED and "multiple of 64" in _err(L)
    assert call(dm=0) == G.G3_EUNSUPPORTED
    assert call(B=0) == G.G3_EINVAL
    assert call(S=-1) == G.G3_EINVAL
    assert call(Hkv=0) == G.G3_EINVAL
    assert call(base=1.0) == G.G3_EINVAL
    assert call(eps=-1.0) == G.G3_EINVAL
    assert call(w=None) == G.G3_EINVAL and "non-NULL" in _err(L)
    assert call(kh=FAKE + 8) == G.G3_EINVAL and "aligned" in _err(L)
    assert call(Hq=70000, Hkv=1) == G.G3_EINVAL and "heads" in _err(L)
    p0 = (ctypes.c_int32 * 1)(-3)
    assert call(pos0=p0) == G.G3_EINVAL and "pos0" in _err(L)


def test_rms_scale_and_fold_validation_errors(L):
    assert L.g3attn_rms_scale(FAKE, 1e-6, FAKE, 0, 64, None) == G.G3_EINVAL
    assert L.g3attn_rms_scale(FAKE, 1e-6, FAKE, 4, 12, None) == G.G3_EUNSUPPORTED and "multiple of 8" in _err(L)
    assert L.g3attn_rms_scale(FAKE, -1.0, FAKE, 4, 64, None) == G.G3_EINVAL and "eps" in _err(L)
    assert L.g3attn_rms_scale(FAKE, 1e-6, None, 4, 64, None) == G.G3_EINVAL and "non-NULL" in _err(L)
    assert L.g3attn_rms_scale(FAKE + 8, 1e-6, FAKE, 4, 64, None) == G.G3_EINVAL and "aligned" in _err(L)
    assert L.g3attn_fold_norm_weight(FAKE, FAKE, FAKE, 0, 64, None) == G.G3_EINVAL
    assert L.g3attn_fold_norm_weight(FAKE, FAKE, FAKE, 4, 60, None) == G.G3_EUNSUPPORTED
    assert L.g3attn_fold_norm_weight(FAKE, None, FAKE, 4, 64, None) == G.G3_EINVAL and "non-NULL" in _err(L)
    assert L.g3attn_fold_norm_weight(FAKE, FAKE, FAKE + 8, 4, 64, None) == G.G3_EINVAL and "aligned" in _err(L)


def test_prefill_khat_validation_errors(L):
    def call(**kw):
        a = dict(q=FAKE, kh=FAKE, v=FAKE, o=FAKE, B=1, S=64, Hq=4, Hkv=2, D=128, kind=G.LOCAL, window=1024,
                 ws_bytes=1 << 30, ws=FAKE)
        a.update(kw)
        return L.g3attn_prefill_khat(a["q"], a["kh"], a["v"], a["o"], a["B"], a["S"], a["Hq"], a["Hkv"], a["D"],
                                     a["kind"], a["window"], 1e4, 1.0, None, 1e-6, 0.0, None, 0, None, None, a["ws"],
                                     a["ws_bytes"], None)
    assert call(kh=None) == G.G3_EINVAL and "khat" in _err(L)
    assert call(D=64) == G.G3_EUNSUPPORTED
    assert call(kind=3) == G.G3_EINVAL
    assert call(ws_bytes=8) == G.G3_EWORKSPACE
    assert call(o=FAKE + 4) == G.G3_EINVAL and "aligned" in _err(L)


def test_o_project_and_rmsnorm_validation_errors(L):
    def oproj(**kw):
        a = dict(attn=FAKE, w=FAKE, y=FAKE, T=64, n_in=4096, n_out=5376)
        a.update(kw)
        return L.g3attn_o_project(a["attn"], a["w"], a["y"], a["T"], a["n_in"], a["n_out"], None)
    assert oproj(n_in=100) == G.G3_EUNSUPPORTED and "multiple of 64" in _err(L)
    assert oproj(n_out=200) == G.G3_EUNSUPPORTED and "multiple of 128" in _err(L)
    assert oproj(T=0) == G.G3_EINVAL
    assert oproj(w=None) == G.G3_EINVAL
    assert oproj(y=FAKE + 2) == G.G3_EINVAL and "aligned" in _err(L)

    def norm(**kw):
        a = dict(x=FAKE, res=None, out=FAKE, T=4, W=5376, eps=1e-6)
        a.update(kw)
        return L.g3attn_rmsnorm(a["x"], a["res"], None, a["eps"], a["out"], a["T"], a["W"], None)
    assert norm(W=5377) == G.G3_EUNSUPPORTED
    assert norm(W=16384) == G.G3_EUNSUPPORTED and "8192" in _err(L)
    assert norm(T=0) == G.G3_EINVAL
    assert norm(eps=-1.0) == G.G3_EINVAL
    assert norm(out=None) == G.G3_EINVAL
    assert norm(res=FAKE + 4) == G.G3_EINVAL and "aligned" in _err(L)


def test_decode_noalloc_rejects_partials_beyond_its_static_array(L):
    """g3attn_decode_noalloc refuses, before any launch, a call whose split-K
    partials exceed its static array (512 sequences x 32 heads x 9 splits of
    a 32K cache: 76.7 MB > 16 MiB); the limit is the header's."""
    src = open(os.path.join(ROOT, "include", "g3attn.h")).read()
    assert re.search(r"#define G3_DECODE_NOALLOC_MAX_BYTES \(\(size_t\)16 << 20\)", src)
    assert G.DECODE_NOALLOC_MAX_BYTES == 16 << 20
    lin = G.KVCacheC(FAKE, FAKE, 40000, 0)
    need = L.g3attn_decode_workspace_size(512, 32, 16, 128, 32768, ctypes.byref(lin))
    assert need == 512 * 32 * 9 * 130 * 4 > G.DECODE_NOALLOC_MAX_BYTES
    rc = L.g3attn_decode_noalloc(FAKE, FAKE, FAKE, FAKE, 512, 32, 16, 128, FAKE, 32768, ctypes.byref(lin), G.GLOBAL,
                                 1024, 1e6, 1.0, None, None, 1e-6, 0.0, None)
    assert rc == G.G3_EWORKSPACE
    assert b"static array" in L.g3attn_last_error()
    # argument errors are still reported as for g3attn_decode
    rc = L.g3attn_decode_noalloc(FAKE, FAKE, FAKE, FAKE, 1, 3, 2, 128, FAKE, 10, ctypes.byref(lin), G.GLOBAL, 1024,
                                 1e6, 1.0, None, None, 1e-6, 0.0, None)
    assert rc == G.G3_EINVAL


def test_probe_library_exports_and_rejects_bad_arguments():
    """The roofline probes' library loads and checks its arguments before any
    device work (no GPU needed for these calls)."""
    from global_gqa_amd import probes

    if not os.path.exists(probes.PROBE_LIB_PATH):
        pytest.skip("libg3probe.so not built")
    P = probes._probe_lib()
    d = ctypes.c_double()
    assert P.g3probe_mfma(0, 10, 1, ctypes.byref(d), ctypes.byref(d), ctypes.byref(d)) == -1
    assert P.g3probe_mfma(4, 10, 1, None, ctypes.byref(d), ctypes.byref(d)) == -1
    assert P.g3probe_stream(None, 1 << 20, 4, 1, 0, ctypes.byref(d), ctypes.byref(d)) == -1
    assert P.g3probe_stream(ctypes.c_void_p(16), 8, 4, 1, 0, ctypes.byref(d), ctypes.byref(d)) == -1
    assert P.g3probe_stream(ctypes.c_void_p(16), 48, 4, 1, 1, ctypes.byref(d), ctypes.byref(d)) == -1
