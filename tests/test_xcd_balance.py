"""The prefill kernels' item order (which query tile each workgroup runs,
and so which XCD it runs on) spreads the causal work of a global layer
evenly over the 8 XCDs, and is a bijection onto the work items.

The dispatcher sends hardware workgroup x to XCD x mod 8.  A global layer's
items are query tiles whose key-tile counts range from 1 to S/64; with fewer
than 8 (sequence, kv head) runs (the 1B model's one kv head, the 2K single
layer's two) whole runs cannot be spread over the XCDs and contiguous blocks
would load one XCD with the heaviest tiles.  Checked on the host with the
kernels' own (host-and-device) functions, built by hipcc."""
import os
import shutil
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EXE = os.path.join(ROOT, "_build", "xcd_balance_check")


@pytest.fixture(scope="module")
def exe():
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    os.makedirs(os.path.dirname(EXE), exist_ok=True)
    cmd = [hipcc, "-O1", "-std=c++17", "--offload-arch=gfx950", "-I", os.path.join(ROOT, "global_gqa_amd", "csrc"),
           os.path.join(ROOT, "tests", "xcd_balance_check.cpp"), "-o", EXE]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return EXE


def _items(exe, n_groups, nq, local):
    out = subprocess.run([exe, str(n_groups), str(nq), str(int(local))], capture_output=True, text=True, check=True)
    return np.array([[int(t) for t in line.split()] for line in out.stdout.split("\n") if line.strip()])


def _key_tiles(qt, rows, S, tile):
    """Key tiles of a causal global-layer item: rows [qt*rows, (qt+1)*rows) see keys 0..last row."""
    return -(-min((qt + 1) * rows, S) // tile)


# (runs = B * Hkv, positions per workgroup, S, key-tile size): the global layers of the bench blocks
SHAPES = {
    "27b-8k (D=128, G=2)": (16, 128, 8192, 64),
    "1b-32k (D=256, G=4)": (1, 64, 32768, 32),
    "single-layer-2k (D=128, G=2)": (2, 128, 2048, 64),
    "mixed-mask-4k (D=128, G=2)": (16, 128, 4096, 64),
    "two runs of 8K (D=256, G=4)": (2, 64, 8192, 32),
}


@pytest.mark.parametrize("name", list(SHAPES))
def test_global_layer_work_is_even_over_xcds(exe, name):
    n_groups, rows, S, tile = SHAPES[name]
    nq = -(-S // rows)
    it = _items(exe, n_groups, nq, False)
    n = n_groups * nq
    # a bijection onto the items
    assert sorted(it[:, 1].tolist()) == list(range(n))
    assert len({(b, q) for b, q in it[:, 2:4].tolist()}) == n
    load = np.zeros(8)
    for xcd, _, _, qt in it:
        load[xcd] += _key_tiles(qt, rows, S, tile)
    if n >= 8 * 8:  # at least 8 items per XCD: the shares must be even
        assert load.max() <= 1.05 * load.mean(), (name, load)
    # on every XCD the heaviest items go first (longest-processing-time order)
    for xcd in range(8):
        w = [_key_tiles(qt, rows, S, tile) for x, _, _, qt in it if x == xcd]
        if n_groups % 8 != 0:
            assert all(w[i] >= w[i + 1] for i in range(len(w) - 1)), (name, xcd)


def test_local_layers_keep_runs_together(exe):
    """Local layers keep a run's neighbouring query tiles on one XCD (their
    K/V windows overlap in that XCD's L2)."""
    it = _items(exe, 1, 512, True)
    for xcd in range(8):
        qts = sorted(qt for x, _, _, qt in it if x == xcd)
        assert qts == list(range(qts[0], qts[0] + 64)), xcd


@pytest.mark.parametrize("n_groups,nq,grid", [(16, 64, 256), (16, 32, 256), (2, 32, 32), (1, 512, 256)])
def test_local_spread_schedule(exe, n_groups, nq, grid):
    """Local layers with several items per workgroup: every item runs exactly
    once; every workgroup whose items include one of a run's short first
    query tiles (qt < 8: fewer keys than the window) runs it first, so those
    workgroups fall out of step with the rest; at every step an XCD's
    workgroups cover consecutive query tiles of at most a few runs (their K/V
    windows overlap in that XCD's L2)."""
    out = subprocess.run([exe, str(n_groups), str(nq), "1", str(grid)], capture_output=True, text=True, check=True)
    it = np.array([[int(t) for t in line.split()] for line in out.stdout.split("\n") if line.strip()])
    n, K = n_groups * nq, n_groups * nq // grid
    assert sorted(it[:, 2].tolist()) == list(range(n))
    per_wg = it.reshape(grid, K, 5)
    for w in per_wg:
        qts = w[:, 4].tolist()
        assert len(set(w[:, 3].tolist())) == 1  # one run per workgroup
        if min(qts) < 8:
            assert qts[0] == min(qts)
    for xcd in range(8):
        for kk in range(K):
            sel = it[(it[:, 0] == xcd) & (it[:, 1] == kk)]
            for bg in set(sel[:, 3].tolist()):
                q = sorted(sel[sel[:, 3] == bg][:, 4].tolist())
                assert q == list(range(q[0], q[0] + len(q))), (xcd, kk, bg, q)
