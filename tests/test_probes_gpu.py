"""The roofline probes (libg3probe.so) run on the GPU and report sane rates:
a short MFMA loop and a short streaming read.  The rates themselves are
measurements, not pinned values; this checks the plumbing and the units."""
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from global_gqa_amd import probes  # noqa: E402


def test_mfma_probe_reports_a_rate_and_a_clock():
    r = probes.mfma_ceiling(workgroups=256, iters=200, reps=2)
    # 256 x 4 waves x 6400 MFMAs of 32768 flop: well under a second at any plausible rate
    assert 50.0 < r["tflops"] < 2600.0, r
    assert 0.5 < r["clock_ghz"] < 3.0, r
    assert r["ms"] > 0.0


def test_stream_probe_reports_a_read_rate():
    r = probes.hbm_read_ceiling(nbytes=256 << 20, reps=2)
    assert 100.0 < r["gbps"] < 20000.0, r  # 256 MiB can be partly cache-resident: a loose upper bound
    assert {x["pattern"] for x in r["runs"]} == {"grid-stride", "per-workgroup blocks"}
