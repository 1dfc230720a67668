"""The largest block count the selection accepts: B = 4096 key blocks per head
(BSGA_MAX_BLOCKS), at b = 128 (one frame of 512 x 1024 patches, 524,293
tokens) and at b = 64 (one frame of 512 x 512 patches, 262,149 tokens), one
head, five special tokens.  At this size the selection sorts every row with
its workgroup-per-row path (rows longer than 512 blocks), the probability
matrix is 64 MB, the patch-row call orders 4096 query blocks per head
(b = 128) or runs 2048 aligned pairs of 64-blocks (b = 64).

rho 0.99 and tau 0 keep k = floor(4096 * 0.01) = 40 blocks per row, so the
oracle can follow sampled query blocks over their kept keys in seconds.

Checks, through bsga_layer (the kernel sequence bench.py times):
* masks: all 4096 CSR rows bit-exact against the oracle's selection of the
  GPU's own float32 probabilities;
* outputs: the first, the last and one seeded query block against the
  oracle, to the bar of the other parity tests (2e-2 rms(O_dense) once half
  an ulp of each stored bf16 value is set aside; |dLSE| <= 2e-3), rms(O_dense)
  over the same rows from the dense softmax over all 524,293 (262,149) keys;
* training mode at the same size (bsga_layer_train): the mask equals
  bsga_layer's, o = bf16(o32) element for element, and the float32 rows of
  the same query blocks lie within 2e-3 rms(O_dense) of the oracle.
"""
from __future__ import annotations

import numpy as np
import pytest

from block_sparse_global_bsga_amd import synth
from oracle import bsga_oracle as O

pytestmark = pytest.mark.gpu

O_TOL = 2e-2
LSE_TOL = 2e-3
O32_TOL = 2e-3


def _bf16_rne_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bits, round to nearest even (finite inputs)."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)


@pytest.mark.parametrize("block, grid_w", [(128, 1024), (64, 512)])
def test_max_blocks(block, grid_w):
    import torch
    from block_sparse_global_bsga_amd import bsga
    from gpu_helpers import compare_rows, from_dev_bf16, head_f64, layer_shape, say, to_dev
    x = synth.random_layer(1, 512, grid_w, 1, block, seed=4500 + block, special_per_frame=5,
                           kind="diffuse", rho=0.99, tau=0.0)
    cfg = x.cfg
    shape = layer_shape(cfg)
    B = bsga.num_blocks(shape)
    assert B == 4096
    say(f"[max blocks] {cfg.name}: N={cfg.tokens} B={B} b={block}")
    q, k, v = to_dev(x.q), to_dev(x.k), to_dev(x.v)
    bufs = bsga.layer(shape, q, k, v, cfg.rho, cfg.tau)
    torch.cuda.synchronize()
    rp = bufs.row_ptr.cpu().numpy().astype(np.int64)
    ci = bufs.col_idx[:int(rp[-1])].cpu().numpy().astype(np.int64)
    probs = bufs.probs.cpu().numpy()
    kh = O.keep_count(B, cfg.rho)
    assert kh == 40
    for i in range(B):
        ref, _, _ = O.select_row(probs[0, i], kh, cfg.tau)
        assert np.array_equal(ci[rp[i]:rp[i + 1]], ref), i
    say(f"   masks: all {B} rows bit-exact, {kh} blocks per row")
    o, lse = from_dev_bf16(bufs.o[0]), bufs.lse[0].cpu().numpy()
    # training mode on the same inputs
    tb, o32 = bsga.layer_train(shape, q, k, v, cfg.rho, cfg.tau)
    torch.cuda.synchronize()
    assert torch.equal(tb.row_ptr, bufs.row_ptr)
    assert torch.equal(tb.col_idx[:int(rp[-1])], bufs.col_idx[:int(rp[-1])])
    o32n = o32[0].cpu().numpy()
    assert np.array_equal(_bf16_rne_bits(o32n),
                          tb.o[0].view(torch.int16).cpu().numpy().view(np.uint16)), "o != bf16(o32)"
    del bufs, tb, o32, q, k, v
    torch.cuda.empty_cache()
    blocks = sorted({0, B - 1, int(np.random.default_rng(4600 + block).integers(1, B - 1))})
    qh, kh_, vh = head_f64(x, 0)
    out = O.layer_head(qh, kh_, vh, cfg.frames, cfg.patches_per_frame, cfg.special_per_frame,
                       cfg.block, O.kept_lists(rp, ci, 0, B), query_blocks=blocks,
                       special_queries=False)
    toks = np.fromiter(out.keys(), dtype=np.int64)
    acc = 0.0
    for c0 in range(0, toks.size, 32):
        dense, _ = O.softmax_attention(qh[toks[c0:c0 + 32]], kh_, vh)
        acc += float(np.sum(dense ** 2))
    rms = (acc / (toks.size * 64)) ** 0.5
    eo, el, _, _, raw = compare_rows(out, o, lse)
    ro = np.stack([out[int(t)][0] for t in toks])
    e32 = float(np.abs(o32n[toks] - ro).max())
    say(f"   query blocks {blocks}: err beyond bf16 rounding {eo / rms:.3e} rms(O_dense) "
        f"(plain {raw / rms:.3e}), max|dLSE| = {el:.3e}; training mode: mask equal, "
        f"o = bf16(o32), o32 err {e32 / rms:.3e} rms(O_dense)")
    assert eo <= O_TOL * rms
    assert el <= LSE_TOL
    assert e32 <= O32_TOL * rms
