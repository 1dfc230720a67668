"""Pins that tie the CPU oracle to facts fixed by the pages and by mathematics,
not to the oracle itself: hand-worked examples (tests/golden), closed forms,
invariants, exact rational arithmetic and a library routine for the one case
that reduces to one (dense attention == torch's scaled_dot_product_attention).

Each pin takes the oracle module as its argument so that the mutation test
can run the same pins against copies of the oracle with a planted mistake.

Page shorthand: [BSGA] = "Block-Sparse Global Attention for Efficient
Multi-View Geometry Transformers"; [HeSS] = "HeSS: Head Sensitivity Score for
Sparsity Redistribution in VGGT".
"""
from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- token split
def pin_token_split_golden(O):
    """[BSGA] key design 3: per frame one camera + four register tokens next to
    the patch tokens; the reading puts them first in each frame."""
    g = _golden("token_split.json")
    for case in g["cases"]:
        s, p = O.token_roles(case["frames"], case["patches_per_frame"],
                             case["special_per_frame"])
        assert s.tolist() == case["special"], case
        assert p.tolist() == case["patch"], case


# -------------------------------------------------------------- block counts
def pin_keep_counts_golden(O):
    """[BSGA] key design 2: k = floor(B (1 - rho)); B and k of the five layer
    shapes worked by hand."""
    g = _golden("keep_counts.json")
    for case in g["cases"]:
        B = O.num_blocks(case["n_patch"], case["block"])
        assert B == case["B"], case
        for rho, k in zip(case["rho"], case["k"]):
            assert O.keep_count(B, rho) == k, (case, rho)


def pin_keep_count_exact_decimal(O):
    """k against exact rational arithmetic on decimals (brute force)."""
    rng = np.random.default_rng(7)
    for _ in range(3000):
        B = int(rng.integers(1, 20000))
        r = int(rng.integers(0, 1_000_001))
        rho = r / 1_000_000
        want = math.floor(B * (1 - Fraction(r, 1_000_000)))
        assert O.keep_count(B, rho) == want, (B, rho)
    # values whose binary float product would land just below an integer
    assert O.keep_count(2140, 0.9) == 214
    assert O.keep_count(10, 0.7) == 3
    assert O.keep_count(100, 0.29) == 71


# ------------------------------------------------------------------- pooling
def pin_pool_golden(O):
    """[BSGA] key design 1: average pooling per block of b patch tokens; the
    last block is partial (mean over its valid rows)."""
    g = _golden("pool_scores.json")["pool"]
    x = np.array(g["x"], dtype=np.float64)
    got = O.block_means(x, g["block"])
    assert np.array_equal(got, np.array(g["means"])), got


def pin_pool_closed_forms(O):
    rng = np.random.default_rng(1)
    d = 64
    # identical rows pool to that row
    row = rng.standard_normal(d)
    x = np.tile(row, (128 * 3, 1))
    assert np.allclose(O.block_means(x, 128), np.tile(row, (3, 1)), atol=1e-14)
    # an arithmetic progression pools to its midpoint, also for a partial block
    n, b = 300, 64
    a, c = rng.standard_normal(d), rng.standard_normal(d)
    x = a + np.arange(n)[:, None] * c
    m = O.block_means(x, b)
    for i in range(m.shape[0]):
        lo, hi = i * b, min((i + 1) * b, n) - 1
        assert np.allclose(m[i], a + (lo + hi) / 2 * c, rtol=1e-12, atol=1e-10)
    assert m.shape[0] == 5


# -------------------------------------------------------------------- scores
def pin_scores_golden(O):
    """S = P_b(Q) P_b(K)^T / sqrt(d_h) on a hand-worked d_h = 4 example."""
    g = _golden("pool_scores.json")["scores"]
    s = O.pooled_scores(np.array(g["qbar"], float), np.array(g["kbar"], float))
    assert s.shape == tuple(g["shape"])
    assert np.allclose(s, np.array(g["S"]), rtol=0, atol=1e-15)


def pin_softmax_closed_forms(O):
    p = O.row_softmax(np.array([[0.0, math.log(3.0)],
                                [math.log(1), math.log(2)],
                                [5.0, 5.0]]))
    assert np.allclose(p, [[0.25, 0.75], [1 / 3, 2 / 3], [0.5, 0.5]], atol=1e-15)
    p = O.row_softmax(np.array([[math.log(1), math.log(2), math.log(5)]]) + 700.0)
    assert np.allclose(p, [[1 / 8, 2 / 8, 5 / 8]], atol=1e-14)
    rng = np.random.default_rng(2)
    s = rng.standard_normal((7, 33)) * 10
    p = O.row_softmax(s)
    assert np.allclose(p.sum(axis=1), 1.0, atol=1e-13)
    # rank-preserving along a row, and order of rows kept
    assert np.array_equal(np.argsort(p, axis=1, kind="stable"),
                          np.argsort(s, axis=1, kind="stable"))


# ----------------------------------------------------------------- selection
def pin_select_golden(O):
    """Hand-worked two-threshold selections on dyadic rows ([BSGA] key
    design 2): ranking, ties by index, inclusive coverage, union = max."""
    g = _golden("select_worked.json")
    for row in g["rows"]:
        p = np.array([Fraction(x).numerator / Fraction(x).denominator
                      for x in row["p"]], dtype=np.float32)
        B = p.shape[0]
        for case in row["cases"]:
            k = O.keep_count(B, case["rho"])
            sel, count, n_tau = O.select_row(p, k, case["tau"])
            assert sel.tolist() == case["kept"], (row["p"], case, sel)
            assert count == len(case["kept"])


def _exact_n_tau(p32, tau):
    """min n with the exact rational sum of the n top-ranked values >= tau."""
    B = len(p32)
    order = sorted(range(B), key=lambda j: (-Fraction(float(p32[j])), j))
    if tau <= 0:
        return order, 0
    if tau >= 1:
        return order, B
    t = Fraction(tau)
    c = Fraction(0)
    for n, j in enumerate(order, start=1):
        c += Fraction(float(p32[j]))
        if c >= t:
            return order, n
    return order, B


def pin_select_exact_rational(O):
    """The oracle's rank order and n_tau equal an exact-rational brute force
    on random float32 rows: flat, peaked, with exact ties and tiny values."""
    rng = np.random.default_rng(3)
    for it in range(600):
        B = int(rng.integers(1, 70))
        kind = it % 4
        if kind == 0:
            s = rng.standard_normal(B) * 0.05
        elif kind == 1:
            s = rng.standard_normal(B) * 8
        elif kind == 2:
            s = rng.integers(0, 3, B).astype(np.float64)  # exact ties
        else:
            s = rng.standard_normal(B) * 30  # many values far below 2^-29
        e = np.exp(s - s.max())
        p = (e / e.sum()).astype(np.float32)
        tau = float(rng.choice([0.0, 0.5, 0.9, 0.95, 0.999, 1.0, rng.random()]))
        rho = float(rng.choice([0.0, 0.5, 0.75, 0.9, 1.0]))
        order, n_tau = _exact_n_tau(p, tau)
        assert O.rank_order(p).tolist() == order
        k = O.keep_count(B, rho)
        sel, count, got_ntau = O.select_row(p, k, tau)
        assert got_ntau == n_tau, (B, kind, tau)
        assert count == min(B, max(k, n_tau))
        assert sel.tolist() == sorted(order[:count])


def pin_select_invariants(O):
    """count >= k; kept mass >= tau unless everything is kept; minimal; a
    prefix of the ranking; ascending output."""
    rng = np.random.default_rng(4)
    for _ in range(300):
        B = int(rng.integers(2, 200))
        s = rng.standard_normal(B) * rng.choice([0.1, 1, 5])
        e = np.exp(s - s.max())
        p = (e / e.sum()).astype(np.float32)
        rho, tau = float(rng.random()), float(rng.random())
        k = O.keep_count(B, rho)
        sel, count, n_tau = O.select_row(p, k, tau)
        assert count >= k and len(sel) == count
        assert np.all(np.diff(sel) > 0)
        mass = float(np.sum(p[sel].astype(np.float64)))
        if count < B:
            assert mass >= tau - 1e-12
        # minimal: one block fewer breaks a threshold
        if count > k:
            ranked = p[np.lexsort((np.arange(B), -p.astype(np.float64)))]
            assert float(np.sum(ranked[:count - 1].astype(np.float64))) < tau
        # prefix of the ranking: every kept block outranks every dropped one
        dropped = np.setdiff1d(np.arange(B), sel)
        if dropped.size and sel.size:
            worst_kept = min(sel, key=lambda j: (p[j], -j))
            best_drop = max(dropped, key=lambda j: (p[j], -j))
            assert (p[worst_kept], -worst_kept) > (p[best_drop], -best_drop)


def pin_select_special_cases(O):
    """tau = 0 keeps exactly k; rho = 0 with tau = 1 keeps all; equal
    probabilities keep the lowest indices; k = 0 and tau = 0 keeps none."""
    rng = np.random.default_rng(5)
    for B in (1, 7, 64, 343):
        e = np.exp(rng.standard_normal(B))
        p = (e / e.sum()).astype(np.float32)
        for rho in (0.0, 0.25, 0.75):
            k = O.keep_count(B, rho)
            assert O.select_row(p, k, 0.0)[1] == k
        assert O.select_row(p, O.keep_count(B, 0.0), 1.0)[0].tolist() == list(range(B))
        assert O.select_row(p, O.keep_count(B, 1.0), 0.0)[0].tolist() == []
        flat = np.full(B, np.float32(1.0 / B))
        sel, count, n_tau = O.select_row(flat, O.keep_count(B, 0.5), 0.6)
        assert sel.tolist() == list(range(count))
        # n_tau: first n with n * fp32(1/B) >= 0.6 (exact products of a dyadic)
        want = next(n for n in range(1, B + 1)
                    if Fraction(float(flat[0])) * n >= Fraction(0.6))
        assert n_tau == want
    # a row whose sum stays below tau keeps everything
    p = np.array([0.5, 0.25, 0.2], dtype=np.float32)
    assert O.select_row(p, 0, 0.99)[0].tolist() == [0, 1, 2]


def pin_select_csr(O):
    """CSR of a [H][B][B] probability tensor with per-head budgets ([HeSS]
    head-wise budgets): rows head-major, columns ascending, per-head k."""
    rng = np.random.default_rng(6)
    H, B = 3, 9
    s = rng.standard_normal((H, B, B))
    e = np.exp(s - s.max(axis=2, keepdims=True))
    p = (e / e.sum(axis=2, keepdims=True)).astype(np.float32)
    rho_h = [0.0, 0.5, 1.0]
    rp, ci = O.select_blocks(p, 0.0, 0.3, rho_h)
    assert rp.tolist() == [0] + list(np.cumsum([9] * 9 + [4] * 9 + [0] * 9))
    assert ci[:9].tolist() == list(range(9))
    rp2, _ = O.select_blocks(p, 0.0, 0.5)
    assert np.all(np.diff(rp2) == 4)


# ----------------------------------------------------------------- attention
def pin_attention_closed_forms(O):
    """Single key, two keys with weights 1:3, constant V, linearity in V."""
    d = 4
    q = np.array([[2.0, 0, 0, 0]])
    k = np.array([[0.0, 0, 0, 0], [math.log(3.0), 0, 0, 0]])
    v = np.array([[4.0, 0, 0, 0], [0, 4.0, 0, 0]])
    o, lse = O.softmax_attention(q, k, v)
    assert np.allclose(o, [[1.0, 3.0, 0, 0]], atol=1e-14)
    assert abs(lse[0] - math.log(4.0)) < 1e-14
    o, lse = O.softmax_attention(q, k[1:], v[1:])
    assert np.allclose(o, v[1:]) and abs(lse[0] - math.log(3.0)) < 1e-14
    rng = np.random.default_rng(8)
    q, k = rng.standard_normal((5, 64)), rng.standard_normal((40, 64))
    v = np.tile(rng.standard_normal(64), (40, 1))
    o, _ = O.softmax_attention(q, k, v)
    assert np.allclose(o, v[:5], atol=1e-13)
    v = rng.standard_normal((40, 64))
    o1, l1 = O.softmax_attention(q, k, v)
    o2, l2 = O.softmax_attention(q, k, -2.5 * v)
    assert np.allclose(o2, -2.5 * o1, atol=1e-13) and np.allclose(l1, l2)
    # equal logits: LSE = logit + log(n)
    o, lse = O.softmax_attention(np.zeros((1, 64)), k, v)
    assert abs(lse[0] - math.log(40)) < 1e-13
    assert np.allclose(o[0], v.mean(axis=0), atol=1e-13)


def pin_attention_brute_force(O):
    """softmax_attention against a per-query, per-key Python loop with
    math.exp (no vectorisation, no max subtraction: small logits)."""
    rng = np.random.default_rng(9)
    d = 8
    q, k, v = (rng.standard_normal((n, d)) for n in (3, 11, 11))
    o, lse = O.softmax_attention(q, k, v)
    for a in range(3):
        w = [math.exp(sum(q[a, i] * k[t, i] for i in range(d)) / math.sqrt(d))
             for t in range(11)]
        z = sum(w)
        for i in range(d):
            assert abs(o[a, i] - sum(w[t] * v[t, i] for t in range(11)) / z) < 1e-12
        assert abs(lse[a] - math.log(z)) < 1e-12


def pin_dense_equals_library(O):
    """Dense attention is torch.nn.functional.scaled_dot_product_attention
    ([BSGA] equation Attention) — a library routine, float64 on the CPU."""
    import torch
    rng = np.random.default_rng(10)
    q, k, v = (rng.standard_normal((96, 64)) * 2 for _ in range(3))
    o, _ = O.softmax_attention(q, k, v)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(k)[None],
        torch.from_numpy(v)[None]).numpy()[0]
    assert np.allclose(o, ref, rtol=0, atol=1e-12)


def pin_lse_merge_identity(O):
    """Attention over a key set equals the LSE merge of attention over any
    split of it (so the LSE the oracle reports is the true log-partition)."""
    rng = np.random.default_rng(11)
    q, k, v = (rng.standard_normal((6, 64)) * 1.5 for _ in range(3))
    k, v = rng.standard_normal((50, 64)) * 1.5, rng.standard_normal((50, 64))
    o, l = O.softmax_attention(q, k, v)
    cut = rng.permutation(50)
    a, b = cut[:17], cut[17:]
    oa, la = O.softmax_attention(q, k[a], v[a])
    ob, lb = O.softmax_attention(q, k[b], v[b])
    m = np.maximum(la, lb)
    wa, wb = np.exp(la - m), np.exp(lb - m)
    merged = (wa[:, None] * oa + wb[:, None] * ob) / (wa + wb)[:, None]
    assert np.allclose(o, merged, atol=1e-13)
    assert np.allclose(l, m + np.log(wa + wb), atol=1e-13)


def _layer_dense_full(O, x, F, P, S, b, kept):
    out = O.layer_head(x[0], x[1], x[2], F, P, S, b, kept)
    return np.array([out[t][0] for t in range(x[0].shape[0])]), \
        np.array([out[t][1] for t in range(x[0].shape[0])])


def pin_full_mask_is_dense(O):
    """rho = 0 with tau = 1 keeps every block, and the layer then equals dense
    softmax attention over all tokens; special rows equal the dense rows for
    any mask ([BSGA] key design 3)."""
    rng = np.random.default_rng(12)
    F, P, S, b, d = 3, 20, 2, 16, 64
    N = F * (P + S)
    x = [rng.standard_normal((N, d)) * 1.3 for _ in range(3)]
    spec, patch = O.token_roles(F, P, S)
    _, _, _, p = O.predict_head(x[0][patch], x[1][patch], b)
    p32 = p.astype(np.float32)
    B = p.shape[0]
    kept = [O.select_row(p32[i], O.keep_count(B, 0.0), 1.0)[0] for i in range(B)]
    assert all(len(c) == B for c in kept)
    o_s, l_s = _layer_dense_full(O, x, F, P, S, b, kept)
    o_d, l_d = O.softmax_attention(x[0], x[1], x[2])
    assert np.allclose(o_s, o_d, atol=1e-13) and np.allclose(l_s, l_d, atol=1e-13)
    kept = [np.array([i]) for i in range(B)]  # a sparse mask
    o_x, l_x = _layer_dense_full(O, x, F, P, S, b, kept)
    assert np.allclose(o_x[spec], o_d[spec], atol=1e-13)
    assert not np.allclose(o_x[patch], o_d[patch], atol=1e-3)


def pin_first_shape_fp32_originals(O):
    """The tiny four-frame shape is stated in float32; the GPU path takes its
    bf16-rounded copy, and the invariants of the method must hold on the
    float32 originals themselves ([BSGA] key design 2: count >= k, kept mass
    >= tau unless every block is kept, a minimal prefix of the ranking;
    rho = 0 with tau = 1 keeps every block and the layer then equals dense
    softmax attention; [BSGA] key design 3: special rows are dense rows)."""
    from block_sparse_global_bsga_amd import synth
    cfg = synth.CONFIGS[1]
    x = synth.generate(cfg, keep_fp32=True)
    spec, patch = O.token_roles(cfg.frames, cfg.patches_per_frame, cfg.special_per_frame)
    for h in range(cfg.heads):
        q, k, v = (t[h].astype(np.float64) for t in (x.q32, x.k32, x.v32))
        _, _, _, p = O.predict_head(q[patch], k[patch], cfg.block)
        p32 = p.astype(np.float32)
        B = p.shape[0]
        kk = O.keep_count(B, cfg.rho)
        kept = []
        for i in range(B):
            sel, count, _ = O.select_row(p32[i], kk, cfg.tau)
            assert count >= kk and len(sel) == count
            ranked = np.sort(p32[i].astype(np.float64))[::-1]
            if count < B:
                assert float(np.sum(p32[i][sel].astype(np.float64))) >= cfg.tau
            if count > kk:
                assert float(np.sum(ranked[:count - 1])) < cfg.tau
            kept.append(sel)
        # the configured mask: special rows equal the dense rows
        out = O.layer_head(q, k, v, cfg.frames, cfg.patches_per_frame, cfg.special_per_frame,
                           cfg.block, kept)
        o_d, l_d = O.softmax_attention(q, k, v)
        for t in spec:
            assert np.allclose(out[int(t)][0], o_d[t], atol=1e-13)
            assert abs(out[int(t)][1] - l_d[t]) < 1e-12
        # the full mask is dense attention
        full = [O.select_row(p32[i], O.keep_count(B, 0.0), 1.0)[0] for i in range(B)]
        assert all(len(c) == B for c in full)
        out = O.layer_head(q, k, v, cfg.frames, cfg.patches_per_frame, cfg.special_per_frame,
                           cfg.block, full)
        o_f = np.array([out[t][0] for t in range(q.shape[0])])
        assert np.allclose(o_f, o_d, atol=1e-13)


def pin_layer_worked_example(O):
    """End-to-end hand-worked layer (d_h = 4): pooling, scores, softmax,
    selection and attention with special keys, values in closed form."""
    g = _golden("layer_worked.json")
    F, P, S, b = g["frames"], g["patches_per_frame"], g["special_per_frame"], g["block"]
    L3 = math.log(3.0)
    named = {"L7": math.log(7.0), "L3+1": L3 + 1.0, "L3-1": L3 - 1.0}
    sub = lambda a: [[named[e] if isinstance(e, str) else float(e) for e in r]  # noqa: E731
                     for r in a]
    q, k, v = (np.array(sub(g[n]), dtype=np.float64) for n in ("q", "k", "v"))
    spec, patch = O.token_roles(F, P, S)
    _, _, s, p = O.predict_head(q[patch], k[patch], b)
    assert np.allclose(s, [[0.0, L3], [math.log(7.0), 0.0]], atol=1e-14)
    assert np.allclose(p, [[0.25, 0.75], [7 / 8, 1 / 8]], atol=1e-14)
    B = p.shape[0]
    kept = [O.select_row(p[i].astype(np.float32), O.keep_count(B, g["rho"]),
                         g["tau"])[0] for i in range(B)]
    assert [c.tolist() for c in kept] == g["kept"]
    out = O.layer_head(q, k, v, F, P, S, b, kept)
    e = math.e
    z0 = 3 * e + 3 / e + 1
    want = {1: ([3 * e / z0, 3 / e / z0, 1 / z0, 0.0], math.log(z0)),
            3: ([0.0, 0.0, 1 / 15, 14 / 15], math.log(15.0)),
            0: (list(v.mean(axis=0)), math.log(5.0))}
    for t, (o_w, l_w) in want.items():
        assert np.allclose(out[t][0], o_w, atol=1e-14), (t, out[t][0], o_w)
        assert abs(out[t][1] - l_w) < 1e-14, t


def pin_computed_entries(O):
    """Entry count of a full mask is N^2 per head (exact block sizes)."""
    F, P, S, b, H = 3, 50, 5, 64, 2
    n_p = F * P
    B = O.num_blocks(n_p, b)
    rp = np.arange(0, H * B * B + 1, B)
    ci = np.tile(np.arange(B), H * B)
    pp, ns = O.computed_entries(F, P, S, b, rp, ci, H)
    N = F * (P + S)
    assert pp + ns == H * N * N and pp == H * n_p * n_p


def pin_budget_golden(O):
    """[HeSS] proposed method: hand-worked redistributions (one head capped
    high, one clipped low, both bounds active, equal weights)."""
    from fractions import Fraction
    g = _golden("budget_worked.json")
    for c in g["cases"]:
        got = O.redistribute_budget(c["weights"], c["mean_rho"], c["rho_min"], c["rho_max"])
        want = [float(Fraction(x)) for x in c["rho"]]
        assert np.allclose(got, want, rtol=0, atol=1e-15), (c["note"], got, want)


def pin_budget_invariants(O):
    """Mean preserved, bounds respected, heavier heads never sparser, scale
    invariance in the weights, no clipping -> exactly proportional; checked
    against a float64 bisection of the defining equation on random cases."""
    rng = np.random.default_rng(17)
    for trial in range(150):
        H = int(rng.integers(1, 24))
        w = np.exp(rng.normal(0.0, 1.5, size=H))
        lo_r, hi_r = sorted(rng.uniform(0.0, 1.0, size=2))
        mean = float(rng.uniform(lo_r, hi_r))
        rho = np.array(O.redistribute_budget(w, mean, lo_r, hi_r))
        assert abs(rho.mean() - mean) < 1e-12, trial
        assert np.all(rho >= lo_r - 1e-15) and np.all(rho <= hi_r + 1e-15)
        order = np.argsort(w)
        assert np.all(np.diff(rho[order]) <= 1e-15)
        rho2 = np.array(O.redistribute_budget(w * 7.25, mean, lo_r, hi_r))
        assert np.allclose(rho, rho2, atol=1e-15)
        # independent solve: bisection on lambda of sum clamp(lam w) = H (1 - mean)
        lo, hi, tot = 1 - hi_r, 1 - lo_r, H * (1 - mean)
        a, b = lo / w.max(), hi / w.min()
        for _ in range(200):
            m = 0.5 * (a + b)
            if np.clip(m * w, lo, hi).sum() < tot:
                a = m
            else:
                b = m
        ref = 1 - np.clip(0.5 * (a + b) * w, lo, hi)
        assert np.allclose(rho, ref, atol=1e-9), trial
    # wide bounds: plain proportional split
    w = np.array([1.0, 2.0, 3.0, 4.0])
    rho = O.redistribute_budget(w, 0.75, 0.0, 1.0)
    assert np.allclose(1 - np.array(rho), 4 * 0.25 * w / w.sum(), atol=1e-15)


def pin_probe_golden(O):
    """[SAF3R] section 4: hand-worked ranking, tie and block mapping, and a
    hand-worked probe (mean query over all tokens, specials included)."""
    g = _golden("probe_worked.json")
    sc = np.array(g["scores"], dtype=np.float64)
    for c in g["cases"]:
        got = O.probe_blocks(sc, g["block"], c["topk"]).tolist()
        assert got == c["blocks"], (c, got)
    pr = g["probe"]
    r = O.probe_scores(np.array(pr["q"], dtype=np.float64), np.array(pr["k"], dtype=np.float64),
                       pr["frames"], pr["patches_per_frame"], pr["special_per_frame"])
    assert np.allclose(r, pr["scores"], atol=1e-15), r


def pin_probe_identity(O):
    """The probe score of a key equals the mean over all queries of the full
    score matrix column (the page's linearity argument, computed the long way
    round), and a planted key aligned with the mean query ranks first."""
    rng = np.random.default_rng(23)
    F, P, S, D = 3, 20, 5, 16
    N = F * (P + S)
    q = rng.standard_normal((N, D)) + 0.7
    k = rng.standard_normal((N, D))
    _, patch = O.token_roles(F, P, S)
    full = (q @ k.T) / math.sqrt(D)
    r = O.probe_scores(q, k, F, P, S)
    assert np.allclose(r, full.mean(axis=0)[patch], atol=1e-12)
    k[patch[37]] = 5.0 * q.mean(axis=0)
    r = O.probe_scores(q, k, F, P, S)
    assert O.probe_blocks(r, 8, 1).tolist() == [37 // 8]


def pin_nmse_closed_forms(O):
    """||A - B||^2 / ||A||^2: zero for equal outputs, one against zero,
    (1 - c)^2 for B = c A, and a hand-worked pair."""
    rng = np.random.default_rng(5)
    a = rng.standard_normal((7, 4))
    assert O.nmse(a, a) == 0.0
    assert abs(O.nmse(a, np.zeros_like(a)) - 1.0) < 1e-15
    assert abs(O.nmse(a, 0.25 * a) - 0.5625) < 1e-14
    x = np.array([[3.0, 4.0]])
    assert abs(O.nmse(x, np.array([[3.0, 2.0]])) - 4.0 / 25.0) < 1e-15
    assert O.nmse(np.zeros((2, 2)), np.zeros((2, 2))) == 0.0


def _tiny_backward_case(seed=0):
    rng = np.random.default_rng(seed)
    F, P, S, b, D = 2, 6, 1, 2, 4
    N = F * (P + S)
    q, k, v, do = (rng.standard_normal((N, D)) for _ in range(4))
    B = (F * P + b - 1) // b
    kept = [np.array(sorted(rng.choice(B, size=2, replace=False))) for _ in range(B)]
    return (F, P, S, b), q, k, v, do, kept


def pin_backward_finite_differences(O):
    """Gradients of L = sum(O * dO) against central differences of the
    oracle's own forward (layer_head), on a tiny masked layer."""
    (F, P, S, b), q, k, v, do, kept = _tiny_backward_case()
    dq, dk, dv = O.attention_backward_head(q, k, v, do, F, P, S, b, kept)

    def loss(q_, k_, v_):
        out = O.layer_head(q_, k_, v_, F, P, S, b, kept)
        return sum(float(np.dot(out[t][0], do[t])) for t in out)
    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for idx in list(np.ndindex(x.shape))[::3]:
            args = {"q_": q, "k_": k, "v_": v}
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args[name + "_"] = xp
            lp = loss(**args)
            args[name + "_"] = xm
            lm = loss(**args)
            assert abs((lp - lm) / (2 * h) - g[idx]) < 1e-7, (name, idx)


def pin_backward_autograd(O):
    """The same gradients from torch autograd of a plain masked softmax
    attention in float64 (mask written out token by token)."""
    import torch
    (F, P, S, b), q, k, v, do, kept = _tiny_backward_case(1)
    spec, patch = O.token_roles(F, P, S)
    N = q.shape[0]
    allowed = np.zeros((N, N), dtype=bool)
    allowed[spec, :] = True
    allowed[:, spec] = True
    for pi, qt in enumerate(patch):
        for pj, kt in enumerate(patch):
            if (pj // b) in set(kept[pi // b].tolist()):
                allowed[qt, kt] = True
    tq, tk, tv = (torch.tensor(a, requires_grad=True) for a in (q, k, v))
    logits = (tq @ tk.T) / math.sqrt(q.shape[1])
    logits = logits.masked_fill(~torch.tensor(allowed), float("-inf"))
    out = torch.softmax(logits, dim=1) @ tv
    (out * torch.tensor(do)).sum().backward()
    dq, dk, dv = O.attention_backward_head(q, k, v, do, F, P, S, b, kept)
    for g, t in ((dq, tq), (dk, tk), (dv, tv)):
        assert np.allclose(g, t.grad.numpy(), atol=1e-12)


def pin_backward_closed_forms(O):
    """A query with a single allowed key has zero logit gradients (dQ = dK =
    0) and passes dO straight to that key's dV; dense gradients of dV sum to
    the column sums of dO (softmax rows sum to 1)."""
    rng = np.random.default_rng(4)
    q, k, v, do = (rng.standard_normal((3, 4)) for _ in range(4))
    # one frame, no specials, blocks of 1 token, each query keeps only its own block
    dq, dk, dv = O.attention_backward_head(q, k, v, do, 1, 3, 0, 1,
                                           [np.array([0]), np.array([1]), np.array([2])])
    assert np.allclose(dq, 0.0, atol=1e-15) and np.allclose(dk, 0.0, atol=1e-15)
    assert np.allclose(dv, do, atol=1e-15)
    dq, dk, dv = O.attention_backward_head(q, k, v, do, 1, 3, 0, 1, None)
    assert np.allclose(dv.sum(axis=0), do.sum(axis=0), atol=1e-12)


def pin_backward_query_subsets(O):
    """Restricted to some queries, the gradients are those of the loss over
    those output rows only (central differences of the oracle's forward), and
    the restricted calls over a partition of the queries add up to the full
    gradients."""
    (F, P, S, b), q, k, v, do, kept = _tiny_backward_case(2)
    spec, _ = O.token_roles(F, P, S)
    B = (F * P + b - 1) // b
    part = O.attention_backward_head(q, k, v, do, F, P, S, b, kept, query_blocks=[1],
                                     special_queries=[int(spec[-1])])
    rows = set(O.layer_head(q, k, v, F, P, S, b, kept, query_blocks=[1],
                            special_queries=False)) | {int(spec[-1])}

    def loss(q_, k_, v_):
        out = O.layer_head(q_, k_, v_, F, P, S, b, kept)
        return sum(float(np.dot(out[t][0], do[t])) for t in out if t in rows)
    h = 1e-6
    for name, x, g in (("q", q, part[0]), ("k", k, part[1]), ("v", v, part[2])):
        for idx in list(np.ndindex(x.shape))[::2]:
            args = {"q_": q, "k_": k, "v_": v}
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args[name + "_"] = xp
            lp = loss(**args)
            args[name + "_"] = xm
            lm = loss(**args)
            assert abs((lp - lm) / (2 * h) - g[idx]) < 1e-7, (name, idx)
    full = O.attention_backward_head(q, k, v, do, F, P, S, b, kept)
    acc = [np.zeros_like(q) for _ in range(3)]
    for i in range(B):
        for a, g in zip(acc, O.attention_backward_head(q, k, v, do, F, P, S, b, kept,
                                                       query_blocks=[i], special_queries=False)):
            a += g
    for a, g in zip(acc, O.attention_backward_head(q, k, v, do, F, P, S, b, kept,
                                                   query_blocks=[], special_queries=True)):
        a += g
    for a, g in zip(acc, full):
        assert np.allclose(a, g, atol=1e-13, rtol=0)


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
