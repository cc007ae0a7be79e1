"""Plain fp64 CPU oracle for the Gemma 3 local/global GQA attention stack.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with
the HIP path (``global_gqa_amd``) and imports nothing from it.

Sources (the Gemma 3 Technical Report and pages that restate it):
  * Gemma 3 Technical Report, section 2 "Model Architecture": GQA, QK-norm in
    place of Gemma 2's logit soft-capping, 5:1 local/global interleave with a
    local first layer, RoPE base 10k (local) and 1M (global) with position
    interpolation on the global layers.
  * Gemma 3 Technical Report, section 1 "Introduction": local span of 1024
    tokens; only global layers see long context.
  * "Gemma explained: What's new in Gemma 3", section on vision encoding:
    bidirectional attention inside image-token spans; and the 27B module
    print: q/k/v/o projection widths (Hq=32, Hkv=16, head_dim=128) and
    ``q_norm``/``k_norm`` RMSNorm over (128,) with eps 1e-6.

Every parity pin of this package is a ``-m "not gpu"`` test under ``tests/``.
"""
from .attention import (  # noqa: F401
    LOCAL,
    GLOBAL,
    layer_kind,
    rms_norm,
    rope_inv_freq,
    rope,
    qknorm_rope,
    visibility,
    visible_interval,
    attend,
    prefill,
    prefill_chunk,
    decode,
    ring_slot,
)
