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


def bf16_half_ulp(x: np.ndarray) -> np.ndarray:
    """Half a unit in the last place of each bf16 value in ``x`` (float64
    holding bf16 values exactly): 2^(floor(log2 |x|) - 8), the most that one
    round-to-nearest into bf16 can have moved a value that rounded to x
    (8 significant bits); 0 for x = 0."""
    ax = np.abs(np.asarray(x, dtype=np.float64))
    out = np.zeros_like(ax)
    nz = ax > 0
    out[nz] = np.ldexp(1.0, (np.floor(np.log2(ax[nz])) - 8).astype(np.int64))
    return out


def compare_rows(out: dict, o_gpu: np.ndarray, lse_gpu: np.ndarray,
                 o_intermediate: np.ndarray = None):
    """Compare the oracle's rows with the GPU's.

    The GPU output is bf16, so every element carries its own rounding: at
    most half an ulp of the stored value (one rounding), plus half an ulp of
    the intermediate bf16 row when the path stored one and merged it again
    (``o_intermediate``: the patch rows of bsga_sparse_attn before
    bsga_special_dense merges them in place).

    Returns (excess, lse_err, ms, n, raw): ``excess`` is the max over elements
    of |O_gpu - O_oracle| minus that elementwise rounding allowance (the
    arithmetic error the tolerance applies to, floored at 0); ``raw`` is the
    plain max |O_gpu - O_oracle|; ``ms`` is the oracle rows' mean square."""
    toks = np.fromiter(out.keys(), dtype=np.int64)
    o_ref = np.stack([out[int(t)][0] for t in toks])
    l_ref = np.array([out[int(t)][1] for t in toks])
    got = o_gpu[toks]
    diff = np.abs(got - o_ref)
    allow = bf16_half_ulp(got)
    if o_intermediate is not None:
        allow = allow + bf16_half_ulp(o_intermediate[toks])
    excess = diff - allow
    l_g = lse_gpu[toks].astype(np.float64)
    both_inf = np.isneginf(l_ref) & np.isneginf(l_g)
    l_err = np.zeros_like(l_ref)
    np.subtract(l_g, l_ref, out=l_err, where=~both_inf)
    l_err = np.abs(l_err)
    return (float(max(excess.max(), 0.0)), float(l_err.max()), float(np.mean(o_ref ** 2)),
            len(toks), float(diff.max()))


def score_prob_bounds(q_patch: np.ndarray, k_patch: np.ndarray, block: int):
    """Oracle pooled scores and probabilities of one head with the error
    bounds the GPU's arithmetic must meet.

    The GPU pools in float32 (each mean within (n + 1) 2^-24 mean|x| of the
    exact one, n rows), splits each float32 mean into three bf16 terms (exact
    to 2^-24 of it), accumulates the six exact cross products of 64 dims in
    float32 (at most 6 * 64 + 3 roundings, each 2^-24 of the running sum of
    magnitudes; the three dropped small products are below 2^-23 of |x||y|),
    and scales by 1/8 exactly.  So with eq, ek the mean bounds,
      |dS_ij| <= [ sum_d (eq |Kb| + |Qb| ek + eq ek)
                   + 387 2^-24 sum_d (|Qb| + eq)(|Kb| + ek) ] / 8.
    The float32 softmax of the GPU's S then moves P_j relative to the
    oracle's by at most exp(2 max_j |dS_j|) - 1 plus its own roundings
    (S_j - max, expf, the sum of B terms, the division):
      |dP_j| <= P_j (2.01 max|dS| + 2^-24 (|S_j - max S| + B + 6)) + 2^-149.
    Returns (S, P, S_bound, P_bound_fn) where P_bound_fn(max_ds_per_row)
    gives the P bound from the GPU's observed per-row max |dS|."""
    from oracle import bsga_oracle as O
    qb, kb, s, p = O.predict_head(q_patch, k_patch, block)
    n = q_patch.shape[0]
    B = qb.shape[0]
    cnt = np.array([O.block_members(n, block, i).shape[0] for i in range(B)], dtype=np.float64)
    eq = (cnt + 1)[:, None] * 2.0 ** -24 * O.block_means(np.abs(q_patch), block)
    ek = (cnt + 1)[:, None] * 2.0 ** -24 * O.block_means(np.abs(k_patch), block)
    aq, ak = np.abs(qb), np.abs(kb)
    e1 = eq @ ak.T + aq @ ek.T + eq @ ek.T
    e2 = (aq + eq) @ (ak + ek).T
    s_bound = (e1 + 387 * 2.0 ** -24 * e2) / 8.0

    def p_bound(max_ds_row: np.ndarray) -> np.ndarray:
        spread = np.abs(s - s.max(axis=1, keepdims=True))
        rel = 2.01 * max_ds_row[:, None] + 2.0 ** -24 * (spread + B + 6)
        return p * rel + 2.0 ** -149

    return s, p, s_bound, p_bound
