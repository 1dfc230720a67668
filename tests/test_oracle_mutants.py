"""Each plausible mistake planted in a copy of the oracle (on the CPU) must
make at least one pin fail.  This shows the pins constrain every step."""
import importlib.util
import math
import os

import numpy as np
import pytest

import oracle_pins

ORACLE_PATH = os.path.join(os.path.dirname(os.path.dirname(__file__)),
                           "oracle", "bsga_oracle.py")


def fresh_oracle():
    spec = importlib.util.spec_from_file_location("oracle_mutant", ORACLE_PATH)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _no_scale(O):
    O.pooled_scores = lambda qb, kb: qb @ kb.T


def _transposed_scores(O):
    O.pooled_scores = lambda qb, kb: (kb @ qb.T) / math.sqrt(qb.shape[1])


def _softmax_wrong_axis(O):
    def f(s):
        e = np.exp(s - s.max(axis=0, keepdims=True))
        return e / e.sum(axis=0, keepdims=True)
    O.row_softmax = f


def _ascending_rank(O):
    O.rank_order = lambda p: np.lexsort((np.arange(p.shape[0]), p.astype(np.float64)))


def _tie_high_index(O):
    O.rank_order = lambda p: np.lexsort((-np.arange(p.shape[0]), -p.astype(np.float64)))


def _strict_coverage(O):
    orig = O.coverage_count

    def f(pr, tau):
        if tau <= 0 or tau >= 1:
            return orig(pr, tau)
        c = np.cumsum(pr.astype(np.float64))
        hit = np.nonzero(c > tau)[0]
        return int(hit[0]) + 1 if hit.size else pr.shape[0]
    O.coverage_count = f


def _coverage_off_by_one(O):
    orig = O.coverage_count
    O.coverage_count = lambda pr, tau: max(0, orig(pr, tau) - 1)


def _min_not_max(O):
    def f(p_row, k, tau):
        order = O.rank_order(p_row)
        n_tau = O.coverage_count(p_row[order], tau)
        count = min(k, n_tau)
        return np.sort(order[:count]), count, n_tau
    O.select_row = f


def _ceil_keep(O):
    O.keep_count = lambda B, rho: int(math.ceil(B * (1 - rho)))


def _binary_float_keep(O):
    O.keep_count = lambda B, rho: int(math.floor(B * (1 - rho)))


def _pool_divides_by_b(O):
    def f(x, block):
        n = x.shape[0]
        B = O.num_blocks(n, block)
        out = np.zeros((B, x.shape[1]))
        for i in range(B):
            out[i] = x[O.block_members(n, block, i)].sum(axis=0) / block
        return out
    O.block_means = f


def _specials_last(O):
    def f(frames, P, S):
        per = P + S
        sp = [f_ * per + P + j for f_ in range(frames) for j in range(S)]
        pa = [f_ * per + j for f_ in range(frames) for j in range(P)]
        return np.array(sp, dtype=np.int64), np.array(pa, dtype=np.int64)
    O.token_roles = f


def _attn_no_scale(O):
    def f(q, k, v):
        if k.shape[0] == 0:
            return np.zeros((q.shape[0], v.shape[1])), np.full(q.shape[0], -np.inf)
        lg = q @ k.T
        m = lg.max(axis=1, keepdims=True)
        e = np.exp(lg - m)
        z = e.sum(axis=1, keepdims=True)
        return (e @ v) / z, (m + np.log(z))[:, 0]
    O.softmax_attention = f


def _lse_no_max(O):
    orig = O.softmax_attention

    def f(q, k, v):
        o, l = orig(q, k, v)
        if k.shape[0] == 0:
            return o, l
        lg = (q @ k.T) / math.sqrt(q.shape[1])
        return o, l - lg.max(axis=1)
    O.softmax_attention = f


def _masked_as_zero_logit(O):
    """Literal (QK^T * M) / sqrt(d): masked entries become logit 0."""
    orig_layer = O.layer_head

    def f(q, k, v, frames, P, S, block, kept, query_blocks=None,
          include_special_keys=True, special_queries=True):
        out = orig_layer(q, k, v, frames, P, S, block, kept, query_blocks,
                         include_special_keys, special_queries)
        if kept is None:
            return out
        spec, patch = O.token_roles(frames, P, S)
        n = patch.shape[0]
        B = O.num_blocks(n, block)
        for i in (range(B) if query_blocks is None else query_blocks):
            qt = patch[O.block_members(n, block, i)]
            keys = set(O.patch_block_tokens(patch, block, kept[i]).tolist()) | set(spec.tolist())
            dropped = np.array(sorted(set(range(q.shape[0])) - keys), dtype=np.int64)
            for t in qt:
                lg = np.concatenate([(q[t] @ k[sorted(keys)].T) / math.sqrt(q.shape[1]),
                                     np.zeros(dropped.shape[0])])
                vv = np.concatenate([v[sorted(keys)], v[dropped]])
                w = np.exp(lg - lg.max())
                out[int(t)] = (w @ vv / w.sum(), lg.max() + math.log(w.sum()))
        return out
    O.layer_head = f


def _no_special_keys(O):
    orig = O.layer_head

    def f(q, k, v, frames, P, S, block, kept, query_blocks=None,
          include_special_keys=True, special_queries=True):
        return orig(q, k, v, frames, P, S, block, kept, query_blocks, False,
                    special_queries)
    O.layer_head = f


def _special_queries_sparse(O):
    """Special queries restricted to special keys instead of every token."""
    orig = O.layer_head

    def f(q, k, v, frames, P, S, block, kept, query_blocks=None,
          include_special_keys=True, special_queries=True):
        out = orig(q, k, v, frames, P, S, block, kept, query_blocks,
                   include_special_keys, special_queries)
        if kept is not None and special_queries:
            spec, _ = O.token_roles(frames, P, S)
            o, l = O.softmax_attention(q[spec], k[spec], v[spec])
            for r, t in enumerate(spec):
                out[int(t)] = (o[r], l[r])
        return out
    O.layer_head = f


def _entries_ignore_partial(O):
    def f(frames, P, S, block, row_ptr, col_idx, heads):
        n_p, n_s = frames * P, frames * S
        pp = int(row_ptr[-1]) * block * block
        return pp, heads * (n_s * (n_p + n_s) + n_p * n_s)
    O.computed_entries = f


def _budget_one_sided(O):
    # a single pass of upper capping, then a clip at the lower bound without
    # re-solving (the budget no longer adds up, or a head stays capped wrongly)
    def f(weights, mean_rho, rho_min, rho_max):
        w = np.asarray(weights, dtype=np.float64)
        lo, hi, tot = 1 - rho_max, 1 - rho_min, len(w) * (1 - mean_rho)
        kappa = np.full(len(w), np.nan)
        free = np.ones(len(w), dtype=bool)
        while True:
            lam = (tot - np.nansum(np.where(free, 0, kappa))) / w[free].sum()
            over = free & (lam * w > hi)
            if not over.any():
                break
            kappa[over] = hi
            free &= ~over
        kappa[free] = np.maximum(lam * w[free], lo)
        return list(1 - kappa)
    O.redistribute_budget = f


def _budget_unclipped(O):
    def f(weights, mean_rho, rho_min, rho_max):
        w = np.asarray(weights, dtype=np.float64)
        return list(1 - len(w) * (1 - mean_rho) * w / w.sum())
    O.redistribute_budget = f


def _budget_inverse(O):
    # denser attention for the less sensitive heads
    real = O.redistribute_budget
    O.redistribute_budget = lambda w, *a: real([1.0 / x for x in w], *a)


def _probe_patch_queries_only(O):
    def f(q, k, frames, P, S):
        _, patch = O.token_roles(frames, P, S)
        return (k[patch] @ q[patch].mean(axis=0)) / math.sqrt(q.shape[1])
    O.probe_scores = f


def _probe_ascending(O):
    real = O.probe_blocks
    O.probe_blocks = lambda scores, block, topk: real(-scores, block, topk)


def _probe_tie_high_index(O):
    def f(scores, block, topk):
        n = scores.shape[0]
        kk = max(0, min(int(topk), n))
        order = np.lexsort((-np.arange(n), -scores))
        return np.unique(order[:kk] // block) if kk else np.zeros(0, dtype=np.int64)
    O.probe_blocks = f


def _nmse_normalised_by_sparse(O):
    O.nmse = lambda a, b: float(np.sum((a - b) ** 2) / max(np.sum(b ** 2), 1e-300))


def _nmse_no_square(O):
    O.nmse = lambda a, b: float(np.sum(np.abs(a - b)) / max(np.sum(np.abs(a)), 1e-300))


def _backward_without_d(O):
    # treats dS as P * dP, dropping the D = dO . O term of the softmax Jacobian
    def f(q, k, v, d_o, frames, P, S, block, kept):
        spec, patch = O.token_roles(frames, P, S)
        n = patch.shape[0]
        scale = 1.0 / math.sqrt(q.shape[1])
        dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
        groups = []
        for i in range(O.num_blocks(n, block)):
            qt = patch[O.block_members(n, block, i)]
            keys = (np.arange(q.shape[0]) if kept is None else
                    np.concatenate([O.patch_block_tokens(patch, block, kept[i]), spec]))
            groups.append((qt, keys))
        if spec.shape[0]:
            groups.append((spec, np.arange(q.shape[0])))
        for qt, keys in groups:
            logits = (q[qt] @ k[keys].T) * scale
            p = np.exp(logits - logits.max(axis=1, keepdims=True))
            p /= p.sum(axis=1, keepdims=True)
            ds = p * (d_o[qt] @ v[keys].T)
            dq[qt] += (ds @ k[keys]) * scale
            np.add.at(dk, keys, (ds.T @ q[qt]) * scale)
            np.add.at(dv, keys, p.T @ d_o[qt])
        return dq, dk, dv
    O.attention_backward_head = f


def _backward_dense_mask(O):
    real = O.attention_backward_head
    O.attention_backward_head = lambda q, k, v, d_o, F, P, S, b, kept: real(q, k, v, d_o, F, P, S,
                                                                             b, None)


def _backward_unscaled_dk(O):
    real = O.attention_backward_head

    def f(*a):
        dq, dk, dv = real(*a)
        return dq, dk * math.sqrt(a[0].shape[1]), dv
    O.attention_backward_head = f


MUTANTS = [_no_scale, _transposed_scores, _softmax_wrong_axis, _ascending_rank,
           _tie_high_index, _strict_coverage, _coverage_off_by_one,
           _min_not_max, _ceil_keep, _binary_float_keep, _pool_divides_by_b,
           _specials_last, _attn_no_scale, _lse_no_max, _masked_as_zero_logit,
           _no_special_keys, _special_queries_sparse, _entries_ignore_partial,
           _budget_one_sided, _budget_unclipped, _budget_inverse,
           _probe_patch_queries_only, _probe_ascending, _probe_tie_high_index,
           _nmse_normalised_by_sparse, _nmse_no_square,
           _backward_without_d, _backward_dense_mask, _backward_unscaled_dk]


@pytest.mark.parametrize("mutate", MUTANTS, ids=lambda f: f.__name__.strip("_"))
def test_mutant_is_caught(mutate):
    O = fresh_oracle()
    mutate(O)
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(O)
        except Exception:  # an assertion, or a crash on a wrong shape
            failed.append(pin.__name__)
    assert failed, f"no pin catches mutant {mutate.__name__}"
