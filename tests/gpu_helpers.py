"""Shared plumbing of the GPU parity tests: upload seeded inputs, run the HIP
path through the C ABI, and evaluate the oracle on the same bits."""
from __future__ import annotations

import sys

import numpy as np
import torch

from block_sparse_global_bsga_amd import synth
from oracle import bsga_oracle as O

DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(bits.view(np.int16)).to(DEV).view(torch.bfloat16)


def from_dev_bf16(t: torch.Tensor) -> np.ndarray:
    return synth.bf16_bits_to_f64(t.view(torch.int16).cpu().numpy().view(np.uint16))


def layer_shape(cfg):
    from block_sparse_global_bsga_amd import bsga
    return bsga.LayerShape(cfg.frames, cfg.patches_per_frame, cfg.special_per_frame,
                           cfg.heads, cfg.block)


def head_f64(x: synth.LayerInputs, h: int):
    return (synth.bf16_bits_to_f64(x.q[h]), synth.bf16_bits_to_f64(x.k[h]),
            synth.bf16_bits_to_f64(x.v[h]))


def kept_from_csr(row_ptr: np.ndarray, col_idx: np.ndarray, h: int, B: int):
    return O.kept_lists(row_ptr, col_idx, h, B)


def oracle_rows(x: synth.LayerInputs, h: int, kept, query_blocks, *,
                include_special_keys=True, special_queries=True):
    c = x.cfg
    q, k, v = head_f64(x, h)
    return O.layer_head(q, k, v, c.frames, c.patches_per_frame, c.special_per_frame,
                        c.block, kept, query_blocks=query_blocks,
                        include_special_keys=include_special_keys,
                        special_queries=special_queries)


BF16_HALF_ULP = 2.0 ** -8  # relative rounding bound of one bf16 round-to-nearest


def compare_rows(out: dict, o_gpu: np.ndarray, lse_gpu: np.ndarray, roundings: int = 1):
    """Compare the oracle's rows with the GPU's.

    Returns (excess, lse_err, ms, n, raw): ``excess`` is max over elements of
    |O_gpu - O_oracle| minus the bf16 output format's own rounding allowance
    (``roundings`` half-ulps of |O_oracle|) -- the arithmetic error the
    tolerance applies to; ``raw`` is the plain max |O_gpu - O_oracle|; ``ms``
    is the oracle rows' mean square (for an rms estimate)."""
    toks = np.fromiter(out.keys(), dtype=np.int64)
    o_ref = np.stack([out[int(t)][0] for t in toks])
    l_ref = np.array([out[int(t)][1] for t in toks])
    diff = np.abs(o_gpu[toks] - o_ref)
    excess = diff - roundings * BF16_HALF_ULP * np.abs(o_ref)
    l_g = lse_gpu[toks].astype(np.float64)
    both_inf = np.isneginf(l_ref) & np.isneginf(l_g)
    l_err = np.zeros_like(l_ref)
    np.subtract(l_g, l_ref, out=l_err, where=~both_inf)
    l_err = np.abs(l_err)
    return (float(max(excess.max(), 0.0)), float(l_err.max()), float(np.mean(o_ref ** 2)),
            len(toks), float(diff.max()))
