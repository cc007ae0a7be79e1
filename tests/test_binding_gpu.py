"""The binding launches on the stream a torch user expects: its raw handle of
the current stream is the one torch reports, on the default stream and inside
a ``torch.cuda.stream`` context, and a decode issued inside such a context
runs on that stream (its result is there once that stream is synchronised)."""
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import global_gqa_amd as G  # noqa: E402


def test_current_stream_handle_matches_torch():
    assert G._stream(None) == torch.cuda.current_stream().cuda_stream
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        assert G._stream(None) == side.cuda_stream == torch.cuda.current_stream().cuda_stream
    assert G._stream(side) == side.cuda_stream
    assert G._stream(None) == torch.cuda.current_stream().cuda_stream


def test_decode_on_a_side_stream_matches_the_default_stream():
    torch.manual_seed(3)
    B, Hq, Hkv, D, cap, p = 2, 4, 2, 128, 256, 200
    dev = "cuda"
    q = torch.randn(B, Hq, D, device=dev).to(torch.bfloat16)
    kn = torch.randn(B, Hkv, D, device=dev).to(torch.bfloat16)
    vn = torch.randn(B, Hkv, D, device=dev).to(torch.bfloat16)
    ck = torch.randn(B, Hkv, cap, D, device=dev).to(torch.bfloat16)
    cv = torch.randn(B, Hkv, cap, D, device=dev).to(torch.bfloat16)
    gq = torch.ones(D, device=dev)
    gk = torch.ones(D, device=dev)
    pos = torch.full((B,), p, dtype=torch.int32, device=dev)
    outs = []
    for use_side in (False, True):
        cache = G.KVCache(ck.clone(), cv.clone(), is_ring=False)
        torch.cuda.synchronize()
        if use_side:
            side = torch.cuda.Stream()
            with torch.cuda.stream(side):
                o = G.decode(q, kn, vn, pos, p, cache, G.GLOBAL, G.WINDOW, 1e6, 1.0, gq, gk, 1e-6)
            side.synchronize()
        else:
            o = G.decode(q, kn, vn, pos, p, cache, G.GLOBAL, G.WINDOW, 1e6, 1.0, gq, gk, 1e-6)
            torch.cuda.synchronize()
        outs.append(o.float().cpu())
    assert torch.equal(outs[0], outs[1])
