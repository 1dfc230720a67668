"""bsga_layer called from a plain C program (tests/c_layer.c: device memory
and workspace from the HIP runtime, the null stream, no Python or torch in
its process), built by build() into _build/c_layer.

Per case the C caller's outputs (probabilities, CSR, O, LSE) must equal,
byte for byte, those of the same call through the Python binding on the
same inputs, and meet the oracle bar of the other parity tests: the CSR
bit-exact against the oracle's selection of the GPU's own probabilities, and
on the checked heads every output row within 2e-2 rms(O_dense) once half an
ulp of each stored bf16 value is set aside, |dLSE| <= 2e-3.
"""
from __future__ import annotations

import os
import subprocess

import numpy as np
import pytest

from block_sparse_global_bsga_amd import synth
from oracle import bsga_oracle as O

pytestmark = pytest.mark.gpu

O_TOL = 2e-2
LSE_TOL = 2e-3

CASES = {
    "tiny-4f-b64": (lambda: synth.generate(synth.CONFIGS[1]), None),
    "ragged-b128-specials": (lambda: synth.random_layer(3, 10, 13, 2, 128, seed=11, kind="corr",
                                                        special_per_frame=5), None),
    "vggt-8f-b64-pairs": (lambda: synth.generate(synth.CONFIGS[2]), [0, 7]),
}


@pytest.fixture(scope="module")
def c_layer(tmp_path_factory):
    from block_sparse_global_bsga_amd import build
    if os.path.exists(build.C_CALLER):
        return build.C_CALLER
    return build.build_c_caller(str(tmp_path_factory.mktemp("c_caller") / "c_layer"))


@pytest.mark.parametrize("name", list(CASES))
def test_c_caller_layer(c_layer, tmp_path, name):
    import torch
    from block_sparse_global_bsga_amd import bsga
    from gpu_helpers import compare_rows, head_f64, layer_shape, say, to_dev
    make, heads = CASES[name]
    x = make()
    cfg = x.cfg
    H, N = cfg.heads, cfg.tokens
    shape = layer_shape(cfg)
    B = bsga.num_blocks(shape)
    say(f"[c caller] {name}: N={N} H={H} b={cfg.block} rho={cfg.rho} tau={cfg.tau}")
    src, dst = tmp_path / "qkv.bin", tmp_path / "out.bin"
    np.concatenate([x.q.ravel(), x.k.ravel(), x.v.ravel()]).astype(np.uint16).tofile(src)
    r = subprocess.run([c_layer, str(src), str(dst), str(cfg.frames), str(cfg.patches_per_frame),
                        str(cfg.special_per_frame), str(H), str(cfg.block), repr(cfg.rho),
                        repr(cfg.tau)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    raw = np.fromfile(dst, dtype=np.uint8)
    at = 0

    def take(dtype, count):
        nonlocal at
        a = raw[at:at + count * np.dtype(dtype).itemsize].view(dtype)
        at += count * np.dtype(dtype).itemsize
        return a

    probs = take(np.float32, H * B * B).reshape(H, B, B)
    rp = take(np.int32, H * B + 1)
    ci = take(np.int32, int(rp[-1]))
    o_bits = take(np.uint16, H * N * 64).reshape(H, N, 64)
    lse = take(np.float32, H * N).reshape(H, N)
    assert at == raw.size
    # the same call through the Python binding
    ref = bsga.layer(shape, to_dev(x.q), to_dev(x.k), to_dev(x.v), cfg.rho, cfg.tau)
    torch.cuda.synchronize()
    nnz = int(ref.row_ptr[-1])
    assert np.array_equal(probs, ref.probs.cpu().numpy())
    assert np.array_equal(rp, ref.row_ptr.cpu().numpy())
    assert np.array_equal(ci, ref.col_idx[:nnz].cpu().numpy())
    assert np.array_equal(o_bits, ref.o.view(torch.int16).cpu().numpy().view(np.uint16))
    assert np.array_equal(lse, ref.lse.cpu().numpy())
    # against the oracle
    ref_rp, ref_ci = O.select_blocks(probs, cfg.tau, cfg.rho)
    assert np.array_equal(rp, ref_rp) and np.array_equal(ci, ref_ci), "mask differs"
    o = synth.bf16_bits_to_f64(o_bits)
    rp64, ci64 = rp.astype(np.int64), ci.astype(np.int64)
    worst_o = worst_l = worst_raw = acc = cnt = 0.0
    for h in (range(H) if heads is None else heads):
        qh, kh, vh = head_f64(x, h)
        out = O.layer_head(qh, kh, vh, cfg.frames, cfg.patches_per_frame, cfg.special_per_frame,
                           cfg.block, O.kept_lists(rp64, ci64, h, B))
        for c0 in range(0, N, 2048):  # rms(O_dense) over the head's rows
            dense, _ = O.softmax_attention(qh[c0:c0 + 2048], kh, vh)
            acc += float(np.sum(dense ** 2))
            cnt += dense.size
        eo, el, _, _, rw = compare_rows(out, o[h], lse[h])
        worst_o, worst_l, worst_raw = max(worst_o, eo), max(worst_l, el), max(worst_raw, rw)
    rms = (acc / cnt) ** 0.5
    say(f"   C caller == Python binding byte for byte ({nnz} CSR entries); O err beyond bf16 "
        f"rounding {worst_o / rms:.2e} rms (plain {worst_raw / rms:.2e}), |dLSE| {worst_l:.1e}")
    assert worst_o <= O_TOL * rms and worst_l <= LSE_TOL
