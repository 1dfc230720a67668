"""bsga_layer captured into a HIP graph and replayed.  The library allocates
nothing, copies nothing to or from the host and never synchronises, and every
kernel runs on the caller's stream, so a serving loop can capture a layer
once (torch.cuda.CUDAGraph on torch's capture stream) and replay it.

For the 8-frame (b = 64, aligned pairs) and 32-frame (b = 128, ordered rows
with the split last round) layers, and the 200-frame head-wise budgets at a
small size: the graph is replayed three times, with eager layer calls on other
inputs and synchronisations between the replays, and every replay's mask
(probabilities and CSR), O and LSE must equal the eager call on the same
inputs byte for byte.  The replay time is printed beside the eager time.
A training step (bsga_layer_train, then bsga_attn_backward_o32) is captured
the same way, at b = 64 (aligned pairs) and b = 128.
"""
from __future__ import annotations

import numpy as np
import pytest

from block_sparse_global_bsga_amd import synth

pytestmark = pytest.mark.gpu


def _cases():
    return {
        "vggt-8f": (synth.CONFIGS[2], None),
        "vggt-32f": (synth.CONFIGS[3], None),
        "perhead-4f": (synth.LayerConfig(name="perhead-4f-518-h4-b128", frames=4, grid_h=37,
                                         grid_w=37, heads=4, block=128, rho=0.85, tau=0.9,
                                         per_head_rho_mean=0.85, seed=4700), True),
    }


@pytest.mark.parametrize("name", list(_cases()))
def test_layer_graph_replay(name):
    import torch
    from block_sparse_global_bsga_amd import bsga
    from gpu_helpers import layer_shape, say, to_dev
    cfg, _ = _cases()[name]
    x = synth.generate(cfg)
    rho_h = None if x.rho_per_head is None else [float(r) for r in x.rho_per_head]
    shape = layer_shape(cfg)
    q, k, v = to_dev(x.q), to_dev(x.k), to_dev(x.v)
    # other inputs for the eager work between replays
    q2 = to_dev(synth.fp32_to_bf16_bits(
        np.random.default_rng(cfg.seed + 1).standard_normal(x.q.shape, dtype=np.float32)))
    ref = bsga.layer(shape, q, k, v, cfg.rho, cfg.tau, rho_h)
    torch.cuda.synchronize()
    nnz = int(ref.row_ptr[-1])
    want = (ref.probs.clone(), ref.row_ptr.clone(), ref.col_idx[:nnz].clone(),
            ref.o.view(torch.int16).clone(), ref.lse.clone())
    bufs = bsga.LayerBuffers(shape, q.device)
    other = bsga.LayerBuffers(shape, q.device)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        bsga.layer(shape, q, k, v, cfg.rho, cfg.tau, rho_h, bufs=bufs)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        bsga.layer(shape, q, k, v, cfg.rho, cfg.tau, rho_h, bufs=bufs)
    torch.cuda.synchronize()
    for rep in range(3):
        # scribble over the outputs eagerly, so a replay that wrote nothing fails
        bufs.o.view(torch.int16).fill_(0x7fc0)
        bufs.lse.fill_(-1.0)
        bufs.probs.fill_(-1.0)
        bufs.col_idx.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = (bufs.probs, bufs.row_ptr, bufs.col_idx[:nnz], bufs.o.view(torch.int16), bufs.lse)
        for w, gt, what in zip(want, got, ("probs", "row_ptr", "col_idx", "o", "lse")):
            assert torch.equal(w, gt), (name, rep, what)
        bsga.layer(shape, q2, k, v, cfg.rho, cfg.tau, rho_h, bufs=other)
        torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    ev[0].record()
    for _ in range(10):
        g.replay()
    ev[1].record()
    for _ in range(10):
        bsga.layer(shape, q, k, v, cfg.rho, cfg.tau, rho_h, bufs=bufs)
    ev[2].record()
    torch.cuda.synchronize()
    say(f"[graph] {name}: 3 replays byte-equal to the eager layer; replay "
        f"{ev[0].elapsed_time(ev[1]) / 10:.4f} ms, eager {ev[1].elapsed_time(ev[2]) / 10:.4f} ms")


@pytest.mark.parametrize("name", ["vggt-8f", "ragged-b128"])
def test_training_step_graph_replay(name):
    """A training step, bsga_layer_train then bsga_attn_backward_o32 on the
    float32 rows, captured into one HIP graph with every buffer (outputs,
    gradients, workspaces) allocated beforehand: three replays, with eager
    steps on other inputs and synchronisations between them, must each
    reproduce the eager step byte for byte (mask, O, LSE, float32 rows, dQ,
    dK, dV)."""
    import torch
    from block_sparse_global_bsga_amd import bsga
    from gpu_helpers import layer_shape, say, to_dev
    if name == "vggt-8f":
        x = synth.generate(synth.CONFIGS[2])
    else:
        x = synth.random_layer(3, 10, 13, 2, 128, seed=11, kind="corr", special_per_frame=5)
    cfg = x.cfg
    shape = layer_shape(cfg)
    dev = torch.device("cuda:0")
    q, k, v = to_dev(x.q), to_dev(x.k), to_dev(x.v)
    rng = np.random.default_rng(cfg.seed + 7)
    d_o = to_dev(synth.fp32_to_bf16_bits(rng.standard_normal(x.q.shape, dtype=np.float32)))
    q2 = to_dev(synth.fp32_to_bf16_bits(rng.standard_normal(x.q.shape, dtype=np.float32)))

    def new_outputs():
        return (bsga.LayerBuffers(shape, dev), torch.empty(x.q.shape, dtype=torch.float32, device=dev),
                [torch.empty(x.q.shape, dtype=torch.float32, device=dev) for _ in range(3)],
                bsga.workspace(shape, bsga.OP_BACKWARD, dev))

    def step(qq, outs):
        bufs, o32, g, ws = outs
        bsga.layer_train(shape, qq, k, v, cfg.rho, cfg.tau, bufs=bufs, o32=o32)
        bsga.attn_backward(shape, qq, k, v, o32, bufs.lse, d_o, bufs.row_ptr, bufs.col_idx,
                           dq=g[0], dk=g[1], dv=g[2], ws=ws)

    def snap(outs):
        bufs, o32, g, _ = outs
        nnz = int(bufs.row_ptr[-1])
        return [t.clone() for t in (bufs.probs, bufs.row_ptr, bufs.col_idx[:nnz],
                                    bufs.o.view(torch.int16), bufs.lse, o32, *g)]

    ref = new_outputs()
    step(q, ref)
    torch.cuda.synchronize()
    want = snap(ref)
    outs, other = new_outputs(), new_outputs()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(q, outs)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(q, outs)
    torch.cuda.synchronize()
    names = ("probs", "row_ptr", "col_idx", "o", "lse", "o32", "dq", "dk", "dv")
    for rep in range(3):
        bufs, o32, g, _ = outs
        bufs.o.view(torch.int16).fill_(0x7fc0)
        bufs.lse.fill_(-1.0)
        o32.fill_(float("nan"))
        for t in g:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for w, got, n in zip(want, snap(outs), names):
            assert torch.equal(w, got), (name, rep, n)
        step(q2, other)
        torch.cuda.synchronize()
    say(f"[graph] training step {cfg.name}: 3 replays byte-equal to the eager step")
