"""Plain, slow, fp64 CPU oracle for block-sparse global attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the tests, the smoke check of the build entry and
the CPU-baseline leg of the benchmark use it.  It shares no code with the HIP
library (no kernels, headers, helpers, tables or constants) and never imports
it.

Sources (cited by page title and section; no line numbers):

* [BSGA] "Block-Sparse Global Attention for Efficient Multi-View Geometry
  Transformers" (CVPR 2026 notes page): the overall-framework flowchart, key
  design 1 (block-mask prediction, equations "Attention" and "SparseAttn"),
  key design 2 (Top-K + CDF two-threshold block selection), key design 3
  (special tokens take a dense path).
* [HeSS] "HeSS: Head Sensitivity Score for Sparsity Redistribution in VGGT"
  (review page), "proposed method": head-wise masked block-sparse attention
  with a per-head budget.

Every step below is the plain definition, in the pages' order:

    split tokens -> pool Q,K per block of b patch tokens -> S = P_b(Q) P_b(K)^T
    / sqrt(d_h) -> row softmax over key blocks -> keep >= k top-ranked blocks
    and add blocks until the cumulative probability reaches tau -> masked
    softmax attention over the kept blocks; special tokens dense.

Readings taken where the pages are silent or ambiguous (all listed in the
design document):

* the 1/sqrt(d_h) scale is applied to the pooled scores as in the dense
  attention formula;
* masked entries of SparseAttn are excluded from the softmax (weight 0, i.e.
  logit -inf), not set to logit 0;
* B is the number of key blocks of one query-block row, B = ceil(N_p / b);
* both thresholds are prefixes of one ranking, so the kept set is the first
  max(k, n_tau) ranked blocks;
* ranking: probability descending, ties by lower block index;
* k = floor(B (1 - rho)) evaluated in exact decimal arithmetic with rho on a
  1e-6 grid;
* the cumulative probability is summed in float64 in rank order over the
  given float32 probabilities, n_tau = min{n : c_n >= tau}; tau <= 0 gives
  n_tau = 0; tau >= 1 (full coverage) gives n_tau = B; a row whose sum never
  reaches tau keeps all B blocks;
* the last patch block may be partial; its mean is over its valid tokens;
* special tokens: 5 per frame, first in each frame; special queries attend to
  every token; patch queries attend to every special token plus the patch
  tokens of their kept blocks, all in one softmax;
* head-wise budgets ([HeSS], iterative capping, no formula given): keep
  fractions 1 - rho_h proportional to positive per-head weights, clipped to
  [1 - rho_max, 1 - rho_min], with their mean fixed at 1 - mean_rho;
* query probe ([SAF3R] section 4): the probe is the mean query of all N tokens
  of the head; only patch keys are ranked (special keys stay dense); ties go to
  the lower patch index; the top-k keys are mapped to the patch blocks that
  hold them, and every query block of the head keeps those blocks.

[SAF3R] "SAF3R: Dynamic Sparse Attention for Feed-Forward 3D Reconstruction
Transformers" (news page), section 4 (query-probe Top-K kernel and its online
estimate through the mean query).
"""
from __future__ import annotations

import math
from typing import List, Optional, Sequence, Tuple

import numpy as np


# ----------------------------------------------------------------------------
# token split  ([BSGA] framework flowchart; key design 3)
# ----------------------------------------------------------------------------
def token_roles(frames: int, patches_per_frame: int,
                special_per_frame: int) -> Tuple[np.ndarray, np.ndarray]:
    """Token indices of the special tokens X_s and of the patch tokens X_p.

    Each frame contributes its special tokens (camera, then registers)
    followed by its patch tokens in raster order; tokens run frame-major.
    The patch list is in increasing token order, which defines patch order
    p = 0 .. N_p-1 used for blocking."""
    per = patches_per_frame + special_per_frame
    special, patch = [], []
    for f in range(frames):
        for j in range(per):
            (special if j < special_per_frame else patch).append(f * per + j)
    return np.array(special, dtype=np.int64), np.array(patch, dtype=np.int64)


# ----------------------------------------------------------------------------
# block-mask prediction  ([BSGA] key design 1)
# ----------------------------------------------------------------------------
def num_blocks(n_patch: int, block: int) -> int:
    """Number of patch blocks B = ceil(N_p / b)."""
    return -(-n_patch // block)


def block_members(n_patch: int, block: int, i: int) -> np.ndarray:
    """Patch positions of block i: b consecutive patches (last one partial)."""
    return np.arange(i * block, min((i + 1) * block, n_patch))


def block_means(x_patch: np.ndarray, block: int) -> np.ndarray:
    """Average pooling P_b(X): row i is the arithmetic mean of the patch rows
    of block i (valid rows only for a partial last block)."""
    n = x_patch.shape[0]
    B = num_blocks(n, block)
    out = np.empty((B, x_patch.shape[1]), dtype=np.float64)
    for i in range(B):
        rows = x_patch[block_members(n, block, i)].astype(np.float64)
        out[i] = rows.sum(axis=0) / rows.shape[0]
    return out


def pooled_scores(qbar: np.ndarray, kbar: np.ndarray) -> np.ndarray:
    """S = P_b(Q) P_b(K)^T / sqrt(d_h)."""
    d = qbar.shape[1]
    return (qbar @ kbar.T) / math.sqrt(d)


def row_softmax(s: np.ndarray) -> np.ndarray:
    """Softmax of every row over the key-block axis (max subtracted)."""
    m = s.max(axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / e.sum(axis=-1, keepdims=True)


def predict_head(q_patch: np.ndarray, k_patch: np.ndarray, block: int):
    """Block-importance distribution of one head: returns (Qbar, Kbar, S, P)."""
    qbar = block_means(q_patch, block)
    kbar = block_means(k_patch, block)
    s = pooled_scores(qbar, kbar)
    return qbar, kbar, s, row_softmax(s)


# ----------------------------------------------------------------------------
# two-threshold selection  ([BSGA] key design 2; [HeSS] per-head budget)
# ----------------------------------------------------------------------------
def keep_count(n_blocks: int, rho: float) -> int:
    """k = floor(B (1 - rho)), exact: rho is read as a decimal on a 1e-6 grid."""
    r = int(round(rho * 1_000_000))
    return (n_blocks * (1_000_000 - r)) // 1_000_000


def rank_order(p_row: np.ndarray) -> np.ndarray:
    """Block indices ranked by probability descending, lower index first on
    ties."""
    j = np.arange(p_row.shape[0])
    return np.lexsort((j, -p_row.astype(np.float64)))


def coverage_count(p_ranked: np.ndarray, tau: float) -> int:
    """n_tau: the smallest n whose cumulative probability c_n of the n
    top-ranked blocks reaches tau (float64, summed in rank order)."""
    B = p_ranked.shape[0]
    if tau <= 0.0:
        return 0
    if tau >= 1.0:
        return B
    c = np.cumsum(p_ranked.astype(np.float64))
    hit = np.nonzero(c >= tau)[0]
    return int(hit[0]) + 1 if hit.size else B


def select_row(p_row: np.ndarray, k: int, tau: float):
    """Kept key blocks of one query-block row, ascending; also returns the
    kept count and n_tau."""
    order = rank_order(p_row)
    n_tau = coverage_count(p_row[order], tau)
    count = min(p_row.shape[0], max(k, n_tau))
    return np.sort(order[:count]), count, n_tau


def select_blocks(probs: np.ndarray, tau: float, rho: float,
                  rho_per_head: Optional[Sequence[float]] = None):
    """Selection of every row of probs[H][B][B] -> CSR (row_ptr, col_idx),
    rows ordered head-major then query block."""
    H, B, _ = probs.shape
    row_ptr = np.zeros(H * B + 1, dtype=np.int64)
    cols = []
    for h in range(H):
        k = keep_count(B, rho if rho_per_head is None else rho_per_head[h])
        for i in range(B):
            sel, _, _ = select_row(probs[h, i], k, tau)
            cols.append(sel)
            row_ptr[h * B + i + 1] = row_ptr[h * B + i] + sel.shape[0]
    col_idx = np.concatenate(cols) if cols else np.zeros(0, np.int64)
    return row_ptr, col_idx


# ----------------------------------------------------------------------------
# attention  ([BSGA] equations Attention and SparseAttn; key design 3)
# ----------------------------------------------------------------------------
def softmax_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray):
    """softmax(q k^T / sqrt(d_h)) v over exactly the given keys.

    Returns (O, LSE) with LSE = log sum_t exp(l_t) (natural log).  With no
    keys, O = 0 and LSE = -inf."""
    nq, d = q.shape
    if k.shape[0] == 0:
        return np.zeros((nq, v.shape[1])), np.full(nq, -np.inf)
    logits = (q @ k.T) / math.sqrt(d)
    m = logits.max(axis=1, keepdims=True)
    e = np.exp(logits - m)
    z = e.sum(axis=1, keepdims=True)
    return (e @ v) / z, (m + np.log(z))[:, 0]


def patch_block_tokens(patch_tok: np.ndarray, block: int,
                       blocks: Sequence[int]) -> np.ndarray:
    n = patch_tok.shape[0]
    if len(blocks) == 0:
        return np.zeros(0, dtype=np.int64)
    return np.concatenate([patch_tok[block_members(n, block, j)] for j in blocks])


def layer_head(q: np.ndarray, k: np.ndarray, v: np.ndarray, frames: int,
               patches_per_frame: int, special_per_frame: int, block: int,
               kept: Optional[List[np.ndarray]],
               query_blocks: Optional[Sequence[int]] = None,
               include_special_keys: bool = True,
               special_queries: bool = True):
    """Output rows of one head of the layer.

    kept[i] lists the kept key blocks of query block i (None = dense: every
    token attends to every token).  Patch queries attend to the patch tokens
    of their kept blocks plus (if include_special_keys) every special token;
    special queries attend to every token.  Returns {token: (o_row, lse)} for
    the patch tokens of ``query_blocks`` (all blocks if None) and, if
    ``special_queries``, every special token."""
    spec, patch = token_roles(frames, patches_per_frame, special_per_frame)
    n = patch.shape[0]
    B = num_blocks(n, block)
    out = {}
    qb = range(B) if query_blocks is None else query_blocks
    all_tok = np.arange(q.shape[0])
    for i in qb:
        qt = patch[block_members(n, block, i)]
        if kept is None:
            keys = all_tok
        else:
            keys = patch_block_tokens(patch, block, kept[i])
            if include_special_keys:
                keys = np.concatenate([keys, spec])
        o, lse = softmax_attention(q[qt], k[keys], v[keys])
        for r, t in enumerate(qt):
            out[int(t)] = (o[r], lse[r])
    if special_queries and spec.shape[0]:
        o, lse = softmax_attention(q[spec], k, v)
        for r, t in enumerate(spec):
            out[int(t)] = (o[r], lse[r])
    return out


def kept_lists(row_ptr: np.ndarray, col_idx: np.ndarray, head: int,
               n_blocks: int) -> List[np.ndarray]:
    base = head * n_blocks
    return [np.asarray(col_idx[row_ptr[base + i]:row_ptr[base + i + 1]])
            for i in range(n_blocks)]


def computed_entries(frames: int, patches_per_frame: int,
                     special_per_frame: int, block: int,
                     row_ptr: np.ndarray, col_idx: np.ndarray,
                     heads: int) -> Tuple[int, int]:
    """(patch-patch entries computed, special entries computed) summed over
    heads: exact block sizes, the partial last block counted by its valid
    tokens; special entries = N_s*N + N_p*N_s per head."""
    n_p = frames * patches_per_frame
    n_s = frames * special_per_frame
    B = num_blocks(n_p, block)
    size = np.array([block_members(n_p, block, j).shape[0] for j in range(B)],
                    dtype=np.int64)
    pp = 0
    for h in range(heads):
        for i in range(B):
            cols = col_idx[row_ptr[h * B + i]:row_ptr[h * B + i + 1]]
            pp += int(size[i]) * int(size[np.asarray(cols, dtype=np.int64)].sum())
    ns = heads * (n_s * (n_p + n_s) + n_p * n_s)
    return pp, ns


# ----------------------------------------------------------------------------
# head-wise budget redistribution  ([HeSS] proposed method)
# ----------------------------------------------------------------------------
def redistribute_budget(weights: Sequence[float], mean_rho: float, rho_min: float,
                        rho_max: float) -> List[float]:
    """Per-head rho from per-head weights: keep fractions kappa_h = 1 - rho_h
    proportional to the weights, clipped to [1 - rho_max, 1 - rho_min], with
    mean kappa_h = 1 - mean_rho (the budget a clipped head cannot take goes to
    the others).

    Solved exactly in rational arithmetic: the clipped total
    f(lam) = sum_h clamp(lam w_h, lo, hi) is piecewise linear in lam with
    breakpoints lo / w_h and hi / w_h; the segment containing the target is
    found among the sorted breakpoints and solved linearly."""
    from fractions import Fraction
    w = [Fraction(float(x)) for x in weights]
    lo, hi = 1 - Fraction(float(rho_max)), 1 - Fraction(float(rho_min))
    target = len(w) * (1 - Fraction(float(mean_rho)))
    if hi == lo:
        return [float(mean_rho)] * len(w)

    def clipped_total(lam):
        return sum(min(max(lam * x, lo), hi) for x in w)

    points = sorted(set([lo / x for x in w] + [hi / x for x in w]))
    lam = points[-1]
    if target <= clipped_total(points[0]):
        lam = points[0]
    for a, b in zip(points, points[1:]):
        fa, fb = clipped_total(a), clipped_total(b)
        if fa <= target <= fb:
            lam = a if fb == fa else a + (target - fa) * (b - a) / (fb - fa)
            break
    return [float(1 - min(max(lam * x, lo), hi)) for x in w]


# ----------------------------------------------------------------------------
# query-probe Top-K selection  ([SAF3R] section 4: query-probe Top-K kernel)
# ----------------------------------------------------------------------------
def probe_scores(q: np.ndarray, k: np.ndarray, frames: int, patches_per_frame: int,
                 special_per_frame: int) -> np.ndarray:
    """Score of every patch key against the mean query of all N tokens,
    qbar . k_p / sqrt(d_h), in patch order."""
    _, patch = token_roles(frames, patches_per_frame, special_per_frame)
    qbar = q.mean(axis=0)
    return (k[patch] @ qbar) / math.sqrt(q.shape[1])


def probe_blocks(scores: np.ndarray, block: int, topk: int) -> np.ndarray:
    """Patch blocks (ascending) holding at least one of the topk best patch
    keys, keys ranked by score descending, then lower patch index."""
    n = scores.shape[0]
    kk = max(0, min(int(topk), n))
    if kk == 0:
        return np.zeros(0, dtype=np.int64)
    order = np.lexsort((np.arange(n), -scores))
    return np.unique(order[:kk] // block)


# ----------------------------------------------------------------------------
# output error  ([SAF3R] section 4, offline head profiling)
# ----------------------------------------------------------------------------
def nmse(o_full: np.ndarray, o_sparse: np.ndarray) -> float:
    """||O_full - O_sparse||^2 / ||O_full||^2 over all entries of one head."""
    num = float(np.sum((o_full - o_sparse) ** 2))
    den = float(np.sum(o_full ** 2))
    if den == 0.0:
        return 0.0 if num == 0.0 else math.inf
    return num / den


# ----------------------------------------------------------------------------
# backward of the layer's attention for a fixed mask  ([BSGA] outlook: sparse
# attention inside training; the block selection itself is not differentiated)
# ----------------------------------------------------------------------------
def attention_backward_head(q: np.ndarray, k: np.ndarray, v: np.ndarray, d_o: np.ndarray,
                            frames: int, patches_per_frame: int, special_per_frame: int,
                            block: int, kept: Optional[List[np.ndarray]],
                            query_blocks: Optional[Sequence[int]] = None,
                            special_queries=True):
    """Gradients (dQ, dK, dV) of L = sum(O * dO) for one head, where O is the
    layer's output (patch queries over their kept patch blocks and every
    special key, special queries over every key; kept = None: dense).

    Per query, with its allowed keys t, logits l_t = q . k_t / sqrt(d),
    P_t = softmax(l)_t and O = sum_t P_t v_t:
      dV_t += P_t dO,  dP_t = dO . v_t,  D = dO . O,  dS_t = P_t (dP_t - D),
      dQ = sum_t dS_t k_t / sqrt(d),  dK_t += dS_t q / sqrt(d).
    Computed one query block (and the special queries) at a time.

    query_blocks / special_queries restrict the loss to some queries: only
    the listed patch query blocks (all if None) and the special queries
    (all if True, none if False, else the listed special tokens) contribute.
    The dQ rows of those queries are then the full gradient; dK and dV hold
    only their contributions (the full dK, dV are the sums over a partition
    of the queries)."""
    spec, patch = token_roles(frames, patches_per_frame, special_per_frame)
    n = patch.shape[0]
    B = num_blocks(n, block)
    scale = 1.0 / math.sqrt(q.shape[1])
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    all_tok = np.arange(q.shape[0])
    groups = []
    for i in (range(B) if query_blocks is None else query_blocks):
        qt = patch[block_members(n, block, i)]
        if kept is None:
            keys = all_tok
        else:
            keys = np.concatenate([patch_block_tokens(patch, block, kept[i]), spec])
        groups.append((qt, keys))
    if special_queries is True:
        sq = spec
    elif special_queries is False:
        sq = spec[:0]
    else:
        sq = np.asarray(special_queries, dtype=np.int64)
        assert np.all(np.isin(sq, spec)), "special_queries must be special tokens"
    if sq.shape[0]:
        groups.append((sq, all_tok))
    for qt, keys in groups:
        if keys.shape[0] == 0:
            continue
        logits = (q[qt] @ k[keys].T) * scale
        m = logits.max(axis=1, keepdims=True)
        e = np.exp(logits - m)
        p = e / e.sum(axis=1, keepdims=True)
        o = p @ v[keys]
        dp = d_o[qt] @ v[keys].T
        dd = np.sum(d_o[qt] * o, axis=1, keepdims=True)
        ds = p * (dp - dd)
        dq[qt] += (ds @ k[keys]) * scale
        # the keys of one query group are distinct, so a plain indexed add is exact
        dk[keys] += (ds.T @ q[qt]) * scale
        dv[keys] += p.T @ d_o[qt]
    return dq, dk, dv
