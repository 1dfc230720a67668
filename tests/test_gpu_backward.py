"""Backward of the layer's attention (bsga_attn_backward) against the oracle's
gradients for the same mask.

The forward runs through bsga_layer (mask, O, LSE); dO is seeded N(0,1)
rounded to bf16; the oracle differentiates the plain masked softmax attention
in float64 on the same bf16 inputs.  Bar, per gradient tensor of a head:
max |g_gpu - g_oracle| <= 2e-2 * rms(g_oracle).  (With P and dS as single
bf16 operands and D from the stored bf16 O, dQ missed this by an order of
magnitude on the peaked synthetic heads, since a query's dS are small
differences that sum to zero; the kernels therefore use hi + lo operands and
recompute D from P and dP.)
"""
from __future__ import annotations

import numpy as np
import pytest

from block_sparse_global_bsga_amd import synth
from oracle import bsga_oracle as O

pytestmark = pytest.mark.gpu

G_TOL = 2e-2

CASES = {
    "tiny-4f": (lambda: synth.generate(synth.CONFIGS[1]), None),
    "ragged-b128": (lambda: synth.random_layer(3, 10, 13, 2, 128, seed=11, kind="corr"), None),
    "multi-frame-block-b64": (lambda: synth.random_layer(5, 5, 10, 3, 64, seed=12), None),
    "no-special-b64": (lambda: synth.random_layer(2, 16, 16, 2, 64, seed=13, special_per_frame=0,
                                                  kind="corr"), None),
    "single-block": (lambda: synth.random_layer(1, 8, 8, 1, 128, seed=15), None),
    "vggt-8f": (lambda: synth.generate(synth.CONFIGS[2]), [0, 7]),
    "vggt-32f": (lambda: synth.generate(synth.CONFIGS[3]), [5]),
}


@pytest.fixture(scope="module")
def lib():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from block_sparse_global_bsga_amd import bsga
    return bsga


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("tau", [None, 0.0])
def test_backward(lib, name, tau):
    import torch
    from gpu_helpers import head_f64, layer_shape, say, to_dev
    make, heads = CASES[name]
    x = make()
    cfg = x.cfg
    tau = cfg.tau if tau is None else tau
    shape = layer_shape(cfg)
    say(f"[backward] {name} N={cfg.tokens} H={cfg.heads} b={cfg.block} tau={tau}")
    q, k, v = to_dev(x.q), to_dev(x.k), to_dev(x.v)
    bufs = lib.layer(shape, q, k, v, cfg.rho, tau, x.rho_per_head)
    rng = np.random.default_rng(77)
    do_bits = synth.fp32_to_bf16_bits(
        rng.standard_normal((cfg.heads, cfg.tokens, 64), dtype=np.float32))
    d_o = to_dev(do_bits)
    dq, dk, dv = lib.attn_backward(shape, q, k, v, bufs.o, bufs.lse, d_o, bufs.row_ptr,
                                   bufs.col_idx)
    torch.cuda.synchronize()
    rp = bufs.row_ptr.cpu().numpy().astype(np.int64)
    ci = bufs.col_idx.cpu().numpy()[:rp[-1]]
    B = lib.num_blocks(shape)
    g_gpu = [t.cpu().numpy() for t in (dq, dk, dv)]
    worst = [0.0, 0.0, 0.0]
    for h in (range(cfg.heads) if heads is None else heads):
        qh, kh, vh = head_f64(x, h)
        doh = synth.bf16_bits_to_f64(do_bits[h])
        ref = O.attention_backward_head(qh, kh, vh, doh, cfg.frames, cfg.patches_per_frame,
                                        cfg.special_per_frame, cfg.block,
                                        O.kept_lists(rp, ci, h, B))
        for j in range(3):
            rms = float(np.sqrt(np.mean(ref[j] ** 2)))
            err = float(np.abs(g_gpu[j][h] - ref[j]).max())
            worst[j] = max(worst[j], err / rms)
    say(f"   max err / rms(grad): dQ {worst[0]:.2e}, dK {worst[1]:.2e}, dV {worst[2]:.2e}")
    assert max(worst) <= G_TOL


def test_backward_dense_mask_equals_dense(lib):
    """rho = 0, tau = 1 keeps every block: the gradients equal those of dense
    attention (oracle with no mask)."""
    import torch
    from gpu_helpers import head_f64, layer_shape, to_dev
    x = synth.random_layer(3, 10, 13, 2, 128, seed=21, kind="corr")
    cfg = x.cfg
    shape = layer_shape(cfg)
    q, k, v = to_dev(x.q), to_dev(x.k), to_dev(x.v)
    bufs = lib.layer(shape, q, k, v, 0.0, 1.0)
    d_o = to_dev(synth.fp32_to_bf16_bits(
        np.random.default_rng(3).standard_normal((cfg.heads, cfg.tokens, 64), dtype=np.float32)))
    grads = lib.attn_backward(shape, q, k, v, bufs.o, bufs.lse, d_o, bufs.row_ptr, bufs.col_idx)
    torch.cuda.synchronize()
    dob = synth.bf16_bits_to_f64(d_o.view(torch.int16).cpu().numpy().view(np.uint16))
    for h in range(cfg.heads):
        qh, kh, vh = head_f64(x, h)
        ref = O.attention_backward_head(qh, kh, vh, dob[h], cfg.frames, cfg.patches_per_frame,
                                        cfg.special_per_frame, cfg.block, None)
        for g, r in zip(grads, ref):
            assert np.abs(g[h].cpu().numpy() - r).max() <= G_TOL * np.sqrt(np.mean(r ** 2))
