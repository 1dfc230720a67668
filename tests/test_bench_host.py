"""Host-side logic of bench.py, on the CPU: the entry count behind its
`value` (effective TFLOP/s = 4 * 64 * entries / time), the one-GPU guard,
and the check that ties the HBM traffic figure to the kernel sources it was
measured on."""
from __future__ import annotations

import os
import subprocess
import sys

import numpy as np
import pytest

import bench
from oracle import bsga_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _random_csr(heads, B, rng):
    row_ptr, cols = [0], []
    for _ in range(heads * B):
        keep = np.flatnonzero(rng.random(B) < rng.uniform(0.0, 1.0))
        cols.append(keep)
        row_ptr.append(row_ptr[-1] + keep.size)
    col = np.concatenate(cols) if cols else np.zeros(0, np.int64)
    return np.array(row_ptr, np.int32), col.astype(np.int32)


def _allowed_pairs(frames, ppf, spf, block, row_ptr, col_idx, heads):
    """Brute force over the token mask of the method: query q may attend to
    token t iff q or t is a special token or the block pair (blk(q), blk(t))
    is selected.  Returns (patch-patch pairs, pairs with a special token)."""
    spec, patch = O.token_roles(frames, ppf, spf)
    n = frames * (ppf + spf)
    B = O.num_blocks(patch.size, block)
    blk = np.full(n, B, dtype=np.int64)  # specials index a spare row/column
    for i in range(B):
        blk[patch[O.block_members(patch.size, block, i)]] = i
    is_spec = np.zeros(n, dtype=bool)
    is_spec[spec] = True
    pp = sp = 0
    for h in range(heads):
        sel = np.zeros((B + 1, B + 1), dtype=bool)
        for i in range(B):
            sel[i, col_idx[row_ptr[h * B + i]:row_ptr[h * B + i + 1]]] = True
        allowed = is_spec[:, None] | is_spec[None, :] | sel[blk[:, None], blk[None, :]]
        both_patch = ~is_spec[:, None] & ~is_spec[None, :]
        pp += int(np.count_nonzero(allowed & both_patch))
        sp += int(np.count_nonzero(allowed & ~both_patch))
    return pp, sp


@pytest.mark.parametrize("frames,ppf,spf,block,heads", [
    (3, 50, 5, 64, 2),     # 150 patches: blocks of 64, 64, 22
    (2, 150, 5, 128, 3),   # 300 patches: 128, 128, 44
    (4, 64, 0, 64, 1),     # no special tokens, full blocks
    (1, 7, 3, 128, 2),     # a single partial block
])
def test_computed_entries_match_token_mask(frames, ppf, spf, block, heads):
    rng = np.random.default_rng(frames * 1000 + ppf)
    B = O.num_blocks(frames * ppf, block)
    row_ptr, col_idx = _random_csr(heads, B, rng)
    got = bench.computed_entries(row_ptr, col_idx, frames * ppf, block, heads, frames * spf)
    assert got == _allowed_pairs(frames, ppf, spf, block, row_ptr, col_idx, heads)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stdout + r.stderr
    assert "{" not in r.stdout  # no JSON line for a configuration it did not measure


def test_traffic_figure_only_for_its_sources(tmp_path, monkeypatch):
    path = tmp_path / "traffic.txt"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(path))
    digest = bench.kernel_source_digest()
    w = "vggt-32f-518-h16-b128"
    path.write_text(f"# comment: ignored\nworkload: {w}\nkernel_source_sha256: {digest}\n"
                    "hbm_bytes_per_launch: 2156610572\n")
    assert bench.recorded_traffic(w) == 2156610572.0
    # measured on another workload: not this one's figure
    assert bench.recorded_traffic("vggt-8f-518-h16-b64") is None
    path.write_text(f"workload: {w}\nkernel_source_sha256: " + "0" * 64 +
                    "\nhbm_bytes_per_launch: 5\n")
    assert bench.recorded_traffic(w) is None
    path.write_text(f"workload: {w}\nkernel_source_sha256: {digest}\n")
    assert bench.recorded_traffic(w) is None
    path.write_text(f"kernel_source_sha256: {digest}\nhbm_bytes_per_launch: 5\n")
    assert bench.recorded_traffic(w) is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.txt"))
    assert bench.recorded_traffic(w) is None
    # the committed summary names the default workload
    monkeypatch.setattr(bench, "TRAFFIC_FILE", os.path.join(ROOT, "profiles",
                                                            "attn_patch_rows_32f_hbm_traffic.txt"))
    from block_sparse_global_bsga_amd import synth
    text = open(bench.TRAFFIC_FILE).read()
    assert f"workload: {synth.CONFIGS[3].name}" in text
