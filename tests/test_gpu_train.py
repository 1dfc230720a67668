"""Training mode: bsga_layer_train (P as a float16 pair hi + lo in the P V
products, the final rows also written as float32) and bsga_attn_backward_o32
(D = dO . O from those float32 rows, so the dQ kernel skips its first sweep).

Per case, through the C ABI:
* the mask of bsga_layer_train equals bsga_layer's byte for byte (the mask
  prediction and selection are the same calls);
* o is bf16(o32), element for element (round to nearest even), so the bf16
  output is the float32 row rounded once;
* the float32 rows against the oracle's float64 rows (every row at the small
  shapes, sampled query blocks and special rows at 32 frames):
  max |o32 - O_oracle| <= 2e-3 rms(O_dense), a tenth of the output bar and
  with no rounding allowance (the measured error is printed beside it);
* the gradients of bsga_attn_backward_o32 against the oracle's float64
  gradients for the same mask, to the backward's bar (max error <= 2e-2 rms
  of the gradient), and their distance to bsga_attn_backward's (D from the
  dQ kernel's own sweep) is printed.
"""
from __future__ import annotations

import numpy as np
import pytest

from block_sparse_global_bsga_amd import synth
from oracle import bsga_oracle as O

pytestmark = pytest.mark.gpu

O32_TOL = 2e-3
G_TOL = 2e-2

CASES = {
    "tiny-4f": (lambda: synth.generate(synth.CONFIGS[1]), None),
    "ragged-b128": (lambda: synth.random_layer(3, 10, 13, 2, 128, seed=11, kind="corr"), None),
    "position-b128-tau0": (lambda: synth.random_layer(4, 7, 12, 3, 128, seed=55, kind="pos",
                                                      rho=0.73, tau=0.0), None),
    "multi-frame-block-b64": (lambda: synth.random_layer(5, 5, 10, 3, 64, seed=12), None),
    "vggt-8f": (lambda: synth.generate(synth.CONFIGS[2]), [0, 7]),
    "vggt-32f": (lambda: synth.generate(synth.CONFIGS[3]), [5]),
}


def _bf16_rne_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bits, round to nearest even (finite inputs)."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)


@pytest.mark.parametrize("name", list(CASES))
def test_layer_train_and_backward_o32(name):
    import torch
    from block_sparse_global_bsga_amd import bsga
    from gpu_helpers import head_f64, layer_shape, say, to_dev
    make, heads = CASES[name]
    x = make()
    cfg = x.cfg
    shape = layer_shape(cfg)
    B = bsga.num_blocks(shape)
    say(f"[train] {name} N={cfg.tokens} H={cfg.heads} b={cfg.block} tau={cfg.tau}")
    q, k, v = to_dev(x.q), to_dev(x.k), to_dev(x.v)
    ref = bsga.layer(shape, q, k, v, cfg.rho, cfg.tau, x.rho_per_head)
    bufs, o32 = bsga.layer_train(shape, q, k, v, cfg.rho, cfg.tau, x.rho_per_head)
    torch.cuda.synchronize()
    nnz = int(ref.row_ptr[-1])
    assert torch.equal(ref.probs, bufs.probs) and torch.equal(ref.row_ptr, bufs.row_ptr)
    assert torch.equal(ref.col_idx[:nnz], bufs.col_idx[:nnz])
    o32n = o32.cpu().numpy()
    o_bits = bufs.o.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(_bf16_rne_bits(o32n), o_bits), "o is not bf16(o32)"
    rp = bufs.row_ptr.cpu().numpy().astype(np.int64)
    ci = bufs.col_idx.cpu().numpy()[:rp[-1]].astype(np.int64)
    lse = bufs.lse.cpu().numpy()
    spec, _ = O.token_roles(cfg.frames, cfg.patches_per_frame, cfg.special_per_frame)
    rng = np.random.default_rng(91)
    acc = cnt = 0.0
    worst_o = worst_l = 0.0
    for h in (range(cfg.heads) if heads is None else heads):
        qh, kh, vh = head_f64(x, h)
        kept = O.kept_lists(rp, ci, h, B)
        if B > 48:
            blocks = sorted({0, B - 1} | set(rng.choice(B, size=4, replace=False).tolist()))
            out = O.layer_head(qh, kh, vh, cfg.frames, cfg.patches_per_frame,
                               cfg.special_per_frame, cfg.block, kept, query_blocks=blocks,
                               special_queries=False)
            if spec.size:
                sq = np.sort(rng.choice(spec, size=min(8, spec.size), replace=False))
                so, sl = O.softmax_attention(qh[sq], kh, vh)
                for r, t in enumerate(sq):
                    out[int(t)] = (so[r], sl[r])
        else:
            out = O.layer_head(qh, kh, vh, cfg.frames, cfg.patches_per_frame,
                               cfg.special_per_frame, cfg.block, kept)
        toks = np.fromiter(out.keys(), dtype=np.int64)
        dense, _ = O.softmax_attention(qh[toks], kh, vh)
        acc += float(np.sum(dense ** 2))
        cnt += dense.size
        ro = np.stack([out[int(t)][0] for t in toks])
        rl = np.array([out[int(t)][1] for t in toks])
        fin = np.isfinite(rl)
        worst_o = max(worst_o, float(np.abs(o32n[h][toks] - ro).max()))
        if fin.any():
            worst_l = max(worst_l, float(np.abs(lse[h][toks][fin] - rl[fin]).max()))
    rms = (acc / cnt) ** 0.5
    say(f"   o32: max err {worst_o / rms:.3e} rms(O_dense) (bar {O32_TOL}), max|dLSE| "
        f"{worst_l:.1e}; o == bf16(o32); mask equal to bsga_layer's")
    assert worst_o <= O32_TOL * rms
    assert worst_l <= 2e-3
    # backward from the float32 rows
    do_bits = synth.fp32_to_bf16_bits(
        np.random.default_rng(77).standard_normal((cfg.heads, cfg.tokens, 64), dtype=np.float32))
    d_o = to_dev(do_bits)
    g32 = bsga.attn_backward(shape, q, k, v, o32, bufs.lse, d_o, bufs.row_ptr, bufs.col_idx)
    g16 = bsga.attn_backward(shape, q, k, v, ref.o, ref.lse, d_o, ref.row_ptr, ref.col_idx)
    torch.cuda.synchronize()
    g_gpu = [t.cpu().numpy() for t in g32]
    g_sweep = [t.cpu().numpy() for t in g16]
    worst = [0.0, 0.0, 0.0]
    apart = [0.0, 0.0, 0.0]
    for h in (range(cfg.heads) if heads is None else heads):
        qh, kh, vh = head_f64(x, h)
        doh = synth.bf16_bits_to_f64(do_bits[h])
        refg = O.attention_backward_head(qh, kh, vh, doh, cfg.frames, cfg.patches_per_frame,
                                         cfg.special_per_frame, cfg.block,
                                         O.kept_lists(rp, ci, h, B))
        for j in range(3):
            r = float(np.sqrt(np.mean(refg[j] ** 2)))
            worst[j] = max(worst[j], float(np.abs(g_gpu[j][h] - refg[j]).max()) / r)
            apart[j] = max(apart[j], float(np.abs(g_gpu[j][h] - g_sweep[j][h]).max()) / r)
    say(f"   backward from o32: max err / rms(grad) dQ {worst[0]:.2e} dK {worst[1]:.2e} "
        f"dV {worst[2]:.2e}; from the sweep's D: {apart[0]:.1e} {apart[1]:.1e} {apart[2]:.1e} apart")
    assert max(worst) <= G_TOL
