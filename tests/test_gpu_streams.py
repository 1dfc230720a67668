"""Two layers in flight at once.  Every call only enqueues kernels on the
caller's stream and keeps no state between calls (bsga_select_static aside),
so work on two streams must not interfere: an 8-frame b = 64 layer with its
backward (bsga_layer, bsga_attn_backward) on one stream and a ragged
b = 128 layer in training mode with its backward (bsga_layer_train,
bsga_attn_backward_o32) on another, each three times without
synchronisation in between, must reproduce the sequential results byte for
byte (mask, O, LSE, float32 rows, every gradient; all kernels are
deterministic)."""
from __future__ import annotations

import numpy as np
import pytest

from block_sparse_global_bsga_amd import synth

pytestmark = pytest.mark.gpu


def test_two_streams_match_sequential():
    import torch
    from block_sparse_global_bsga_amd import bsga
    from gpu_helpers import layer_shape, say, to_dev
    x1 = synth.generate(synth.CONFIGS[2])
    x2 = synth.random_layer(6, 19, 23, 3, 128, seed=77, kind="corr", special_per_frame=5)
    say(f"[streams] {x1.cfg.name} (N={x1.cfg.tokens}) beside {x2.cfg.name} (N={x2.cfg.tokens})")
    sh1, sh2 = layer_shape(x1.cfg), layer_shape(x2.cfg)
    dev = torch.device("cuda:0")
    q1, k1, v1 = to_dev(x1.q), to_dev(x1.k), to_dev(x1.v)
    q2, k2, v2 = to_dev(x2.q), to_dev(x2.k), to_dev(x2.v)
    rng = np.random.default_rng(31)
    do1 = to_dev(synth.fp32_to_bf16_bits(rng.standard_normal(x1.q.shape, dtype=np.float32)))
    do2 = to_dev(synth.fp32_to_bf16_bits(rng.standard_normal(x2.q.shape, dtype=np.float32)))
    c1, c2 = x1.cfg, x2.cfg

    def work1(bufs, grads):
        bsga.layer(sh1, q1, k1, v1, c1.rho, c1.tau, bufs=bufs)
        bsga.attn_backward(sh1, q1, k1, v1, bufs.o, bufs.lse, do1, bufs.row_ptr, bufs.col_idx,
                           dq=grads[0], dk=grads[1], dv=grads[2])

    def work2(bufs, o32, grads):
        bsga.layer_train(sh2, q2, k2, v2, c2.rho, c2.tau, bufs=bufs, o32=o32)
        bsga.attn_backward(sh2, q2, k2, v2, o32, bufs.lse, do2, bufs.row_ptr, bufs.col_idx,
                           dq=grads[0], dk=grads[1], dv=grads[2])

    def new_grads(x):
        return [torch.empty(x.q.shape, dtype=torch.float32, device=dev) for _ in range(3)]

    def snapshot(bufs, grads, o32=None):
        nnz = int(bufs.row_ptr[-1])
        out = [bufs.probs, bufs.row_ptr, bufs.col_idx[:nnz], bufs.o.view(torch.int16), bufs.lse]
        out += grads + ([o32] if o32 is not None else [])
        return [t.clone() for t in out]

    # sequential reference
    r1b, r1g = bsga.LayerBuffers(sh1, dev), new_grads(x1)
    r2b, r2g = bsga.LayerBuffers(sh2, dev), new_grads(x2)
    r2o = torch.empty(x2.q.shape, dtype=torch.float32, device=dev)
    work1(r1b, r1g)
    torch.cuda.synchronize()
    work2(r2b, r2o, r2g)
    torch.cuda.synchronize()
    want1, want2 = snapshot(r1b, r1g), snapshot(r2b, r2g, r2o)
    # the same work on two streams at once (buffers allocated up front)
    b1, g1 = bsga.LayerBuffers(sh1, dev), new_grads(x1)
    b2, g2 = bsga.LayerBuffers(sh2, dev), new_grads(x2)
    o2 = torch.empty(x2.q.shape, dtype=torch.float32, device=dev)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    for _ in range(3):
        with torch.cuda.stream(s1):
            work1(b1, g1)
        with torch.cuda.stream(s2):
            work2(b2, o2, g2)
    torch.cuda.synchronize()
    names = ["probs", "row_ptr", "col_idx", "o", "lse", "dq", "dk", "dv", "o32"]
    for w, g, n in zip(want1, snapshot(b1, g1), names):
        assert torch.equal(w, g), ("stream 1", n)
    for w, g, n in zip(want2, snapshot(b2, g2, o2), names):
        assert torch.equal(w, g), ("stream 2", n)
    say("   both streams byte-equal to the sequential run (mask, O, LSE, o32, gradients)")
