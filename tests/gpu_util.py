"""Helpers shared by the GPU parity tests (no attention arithmetic here)."""
import numpy as np

# Gate for unit-scale bf16 inputs with fp32 accumulation: max-abs and
# mean-abs error against the fp64 oracle, plus a relative-L2 gate because
# outputs shrink like 1/sqrt(visible keys) at long rows, where the absolute
# gates alone would accept an all-zero output.
MAX_ABS = 2e-2
MEAN_ABS = 2e-3
REL_L2 = 1e-2


def dev_bf16(x, device="cuda"):
    import torch

    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device=device, dtype=torch.bfloat16)


def dev_f32(x, device="cuda"):
    import torch

    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device)


def host(t):
    import torch

    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def errors(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    d = np.abs(got - ref)
    rel = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300)
    return dict(max_abs=float(d.max()), mean_abs=float(d.mean()), rel_l2=float(rel))


def assert_parity(got, ref, what="", max_abs=MAX_ABS):
    e = errors(got, ref)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    assert e["max_abs"] <= max_abs and e["mean_abs"] <= MEAN_ABS and e["rel_l2"] <= REL_L2, f"{what}: {e}"
    return e


def assert_rowwise_bf16(got, ref, what=""):
    """Per-element check of a bf16 vector output (norm/rotation results):
    |err| <= 2^-8 |ref| + 2^-8 * rms of the row (bf16 rounding of the output
    is at most 2^-9 relative)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = np.sqrt(np.mean(ref * ref, axis=-1, keepdims=True))
    tol = 2.0 ** -8 * np.abs(ref) + 2.0 ** -8 * rms * 0.05 + 1e-30
    bad = np.abs(got - ref) > tol
    assert not bad.any(), f"{what}: {bad.sum()} elements out of tolerance; worst {np.abs(got - ref)[bad].max()}"
