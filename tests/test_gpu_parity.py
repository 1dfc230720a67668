"""HIP path vs the CPU oracle, element by element, through the C ABI.

Bars (see the tolerance notes next to each check):
* block masks (row_ptr, col_idx): bit-exact when both sides select from the
  same float32 probabilities (the GPU's);
* attention outputs: max |O_gpu - O_oracle| <= 2e-2 * rms(O_dense) for bf16
  inputs, the oracle run on the GPU's mask.  The outputs are bf16, so each
  element also carries the format's own rounding: half an ulp of the stored
  bf16 value, 2^(floor(log2|O_gpu|) - 8), is set aside elementwise (plus half
  an ulp of the intermediate bf16 patch row for rows that bsga_special_dense
  merges in place); the plain max error is printed next to the asserted one;
* LSE: |err| <= 2e-3 (float32 sums of exp of exactly-computed bf16 dot
  products; the slack covers the approximate exp2 and float32 accumulation);
* pooled means: within the float32 summation bound;
* pooled scores S (the optional output of bsga_predict_mask): within the
  float32 error bound of the GPU's arithmetic (float32 means, three-way bf16
  split, float32 accumulation of 6 x 64 exact products);
* probabilities: |P_gpu - P_oracle| <= P_oracle * (2 max|dS| + (B + 4) 2^-24),
  the relative bound that error in S and the float32 softmax allow.
"""
from __future__ import annotations

import numpy as np
import pytest

from block_sparse_global_bsga_amd import synth
from oracle import bsga_oracle as O

pytestmark = pytest.mark.gpu

O_TOL = 2e-2
LSE_TOL = 2e-3


def _cases():
    c = synth.CONFIGS
    return {
        "tiny-4f": (lambda: synth.generate(c[1]), None),
        "vggt-8f": (lambda: synth.generate(c[2]), 16),
        "vggt-32f": (lambda: synth.generate(c[3]), 4),
        "ragged-b128": (lambda: synth.random_layer(3, 10, 13, 2, 128, seed=11, kind="corr"), None),
        "multi-frame-block-b64": (lambda: synth.random_layer(5, 5, 10, 3, 64, seed=12), None),
        "no-special-b64": (lambda: synth.random_layer(2, 16, 16, 2, 64, seed=13, special_per_frame=0,
                                                      kind="corr"), None),
        "position-b128": (lambda: synth.random_layer(4, 12, 12, 2, 128, seed=14, kind="pos"), None),
        "single-block": (lambda: synth.random_layer(1, 8, 8, 1, 128, seed=15), None),
        # 400 query blocks: 50 per XCD left for a last round of 96 slots
        "over-half-b128": (lambda: synth.random_layer(1, 40, 80, 16, 128, seed=21), None),
        # one head, 64 + 1 key tiles: the special rows split into 65 key
        # ranges, more than one 64-lane pass of the split-K reduce
        "special-65-splits": (lambda: synth.random_layer(8, 32, 32, 1, 128, seed=22), None),
    }


CASES = _cases()
_cache = {}


def inputs(name):
    if name not in _cache:
        _cache.clear()
        _cache[name] = CASES[name][0]()
    return _cache[name]


def sample_blocks(name, B, h):
    per = CASES[name][1]
    if per is None or per >= B:
        return list(range(B))
    rng = np.random.default_rng(100 + h)
    pick = set(rng.choice(B, size=per, replace=False).tolist())
    pick.update({0, B - 1})  # always the first and the (partial) last block
    return sorted(pick)


@pytest.fixture(scope="module")
def lib():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from block_sparse_global_bsga_amd import bsga
    return bsga


def _upload(x):
    from gpu_helpers import to_dev
    return to_dev(x.q), to_dev(x.k), to_dev(x.v)


@pytest.mark.parametrize("name", list(CASES))
def test_predict_mask(lib, name):
    from gpu_helpers import layer_shape, say, score_prob_bounds
    x = inputs(name)
    cfg = x.cfg
    say(f"[predict_mask] {name} {cfg.frames}f P={cfg.patches_per_frame} b={cfg.block}")
    shape = layer_shape(cfg)
    q, k, _ = _upload(x)
    probs, scores, qbar, kbar = lib.predict_mask(shape, q, k, want_means=True, want_scores=True)
    probs2 = lib.predict_mask(shape, q, k)
    probs, scores, qbar, kbar, probs2 = (t.cpu().numpy() for t in (probs, scores, qbar, kbar, probs2))
    # the optional outputs change nothing else
    assert np.array_equal(probs, probs2)
    _, patch = O.token_roles(cfg.frames, cfg.patches_per_frame, cfg.special_per_frame)
    worst_s = worst_p = worst_s_abs = worst_p_rel = 0.0
    for h in range(cfg.heads):
        qp = synth.bf16_bits_to_f64(x.q[h][patch])
        kp = synth.bf16_bits_to_f64(x.k[h][patch])
        qb, kb, _, _ = O.predict_head(qp, kp, cfg.block)
        for mine, ref, rows in ((qbar[h], qb, qp), (kbar[h], kb, kp)):
            # float32 summation bound: (n+1) u sum|x| / n per element
            absmean = O.block_means(np.abs(rows), cfg.block)
            n = np.array([O.block_members(rows.shape[0], cfg.block, i).shape[0]
                          for i in range(ref.shape[0])])[:, None]
            bound = (n + 1) * 2.0 ** -24 * absmean + 1e-30
            assert np.all(np.abs(mine - ref) <= bound), (name, h)
        s_ref, p_ref, s_bound, p_bound = score_prob_bounds(qp, kp, cfg.block)
        ds = np.abs(scores[h] - s_ref)
        worst_s = max(worst_s, float((ds / s_bound).max()))
        worst_s_abs = max(worst_s_abs, float(ds.max()))
        dp = np.abs(probs[h] - p_ref)
        worst_p = max(worst_p, float((dp / p_bound(ds.max(axis=1))).max()))
        worst_p_rel = max(worst_p_rel, float((dp / np.maximum(p_ref, 1e-300)).max()))
    say(f"   S: max |dS| {worst_s_abs:.2e}, {worst_s:.3f} of its bound; P: max rel err "
        f"{worst_p_rel:.2e}, {worst_p:.3f} of its bound")
    assert worst_s <= 1.0
    assert worst_p <= 1.0


SELECT_PARAMS = [("config", None), ("full", (0.0, 1.0)), ("empty", (1.0, 0.0)),
                 ("topk-only", (0.75, 0.0)), ("cdf-only", (0.0, 0.5)),
                 ("per-head", "per-head")]


@pytest.mark.parametrize("name", ["tiny-4f", "vggt-8f", "vggt-32f", "ragged-b128",
                                  "multi-frame-block-b64", "single-block"])
@pytest.mark.parametrize("param", [p[0] for p in SELECT_PARAMS])
def test_select_bitexact(lib, name, param):
    import torch
    from gpu_helpers import layer_shape, say
    x = inputs(name)
    cfg = x.cfg
    shape = layer_shape(cfg)
    q, k, _ = _upload(x)
    probs = lib.predict_mask(shape, q, k)
    rho, tau, rho_h = cfg.rho, cfg.tau, None
    spec = dict(SELECT_PARAMS)[param]
    if spec == "per-head":
        rng = np.random.default_rng(5)
        rho_h = rng.choice([0.0, 0.5, 0.75, 0.9, 0.95, 1.0], size=cfg.heads).tolist()
    elif spec is not None:
        rho, tau = spec
    say(f"[select] {name} {param} rho={rho} tau={tau} rho_h={rho_h}")
    row_ptr, col_idx = lib.select(shape, probs, rho, tau, rho_h)
    torch.cuda.synchronize()
    rp = row_ptr.cpu().numpy().astype(np.int64)
    ci = col_idx.cpu().numpy()[:rp[-1]]
    p32 = probs.cpu().numpy()
    ref_rp, ref_ci = O.select_blocks(p32, tau, rho, rho_h)
    assert np.array_equal(rp, ref_rp), (name, param)
    assert np.array_equal(ci, ref_ci), (name, param)


@pytest.mark.parametrize("tau", [0.0, 0.9])
def test_select_with_redistributed_budgets(lib, tau):
    """Per-head rho from bsga_redistribute (weights spread over 1..13, mean
    0.8, rho in [0.5, 0.95]) through bsga_select; the reference selects with
    the oracle's own redistribution of the same weights."""
    import torch
    from gpu_helpers import layer_shape, say
    x = inputs("vggt-32f")
    cfg = x.cfg
    shape = layer_shape(cfg)
    weights = [1.0 + (h * 7919) % 13 for h in range(cfg.heads)]
    rho_h = lib.redistribute(weights, 0.8, 0.5, 0.95)
    rho_ref = O.redistribute_budget(weights, 0.8, 0.5, 0.95)
    say(f"[select-redistributed] tau={tau} rho_h={[round(r, 4) for r in rho_h]}")
    q, k, _ = _upload(x)
    probs = lib.predict_mask(shape, q, k)
    row_ptr, col_idx = lib.select(shape, probs, cfg.rho, tau, rho_h)
    torch.cuda.synchronize()
    rp = row_ptr.cpu().numpy().astype(np.int64)
    ci = col_idx.cpu().numpy()[:rp[-1]]
    ref_rp, ref_ci = O.select_blocks(probs.cpu().numpy(), tau, cfg.rho, rho_ref)
    assert np.array_equal(rp, ref_rp) and np.array_equal(ci, ref_ci)


def test_select_ties_and_flat_rows(lib):
    """Uniform rows and rows with many exact ties, uploaded directly."""
    import torch
    from gpu_helpers import DEV, say
    shape = lib.LayerShape(frames=1, patches_per_frame=64 * 300 - 17, special_per_frame=5,
                           heads=3, block=64)
    B = lib.num_blocks(shape)
    rng = np.random.default_rng(21)
    p = np.empty((3, B, B), dtype=np.float32)
    p[0] = np.float32(1.0 / B)
    lv = rng.integers(0, 4, size=(B, B)).astype(np.float64)
    p[1] = (np.exp(lv) / np.exp(lv).sum(axis=1, keepdims=True)).astype(np.float32)
    s = rng.standard_normal((B, B)) * 20
    e = np.exp(s - s.max(axis=1, keepdims=True))
    p[2] = (e / e.sum(axis=1, keepdims=True)).astype(np.float32)
    probs = torch.from_numpy(p).to(DEV)
    for rho, tau in ((0.5, 0.6), (0.9, 0.99), (0.0, 0.999999), (0.97, 0.3)):
        say(f"[select ties] rho={rho} tau={tau}")
        row_ptr, col_idx = lib.select(shape, probs, rho, tau)
        rp = row_ptr.cpu().numpy().astype(np.int64)
        ref_rp, ref_ci = O.select_blocks(p, tau, rho)
        assert np.array_equal(rp, ref_rp)
        assert np.array_equal(col_idx.cpu().numpy()[:rp[-1]], ref_ci)


def _rms_dense(x, blocks_per_head):
    """rms of the oracle's dense output over the sampled rows."""
    from gpu_helpers import oracle_rows
    acc, cnt = 0.0, 0
    for h, blocks in blocks_per_head.items():
        out = oracle_rows(x, h, None, blocks)
        o = np.stack([r[0] for r in out.values()])
        acc += float(np.sum(o ** 2))
        cnt += o.size
    return (acc / cnt) ** 0.5


@pytest.mark.parametrize("name", list(CASES))
def test_layer_parity(lib, name):
    """bsga_layer end to end; the oracle runs on the GPU's mask."""
    import torch
    from gpu_helpers import compare_rows, from_dev_bf16, oracle_rows, layer_shape, say
    x = inputs(name)
    cfg = x.cfg
    shape = layer_shape(cfg)
    say(f"[layer] {name} N={cfg.tokens} H={cfg.heads} b={cfg.block} rho={cfg.rho} tau={cfg.tau}")
    q, k, v = _upload(x)
    bufs = lib.layer(shape, q, k, v, cfg.rho, cfg.tau, x.rho_per_head)
    torch.cuda.synchronize()
    rp = bufs.row_ptr.cpu().numpy().astype(np.int64)
    ci = bufs.col_idx.cpu().numpy()[:rp[-1]]
    o = from_dev_bf16(bufs.o)
    lse = bufs.lse.cpu().numpy()
    B = lib.num_blocks(shape)
    sampled = {h: sample_blocks(name, B, h) for h in range(cfg.heads)}
    rms = _rms_dense(x, sampled)
    worst_o = worst_l = worst_raw = 0.0
    for h in range(cfg.heads):
        kept = O.kept_lists(rp, ci, h, B)
        out = oracle_rows(x, h, kept, sampled[h])
        eo, el, _, _, raw = compare_rows(out, o[h], lse[h])
        worst_o, worst_l, worst_raw = max(worst_o, eo), max(worst_l, el), max(worst_raw, raw)
    say(f"   err beyond bf16 rounding {worst_o / rms:.3e} rms(O_dense) (plain max|dO| "
        f"{worst_raw / rms:.3e} rms, rms = {rms:.4f}); max|dLSE| = {worst_l:.3e}")
    assert worst_o <= O_TOL * rms
    assert worst_l <= LSE_TOL


@pytest.mark.parametrize("name", ["tiny-4f", "vggt-8f", "ragged-b128", "multi-frame-block-b64",
                                  "no-special-b64", "single-block"])
def test_separate_calls(lib, name):
    """predict -> select -> sparse_attn -> special_dense as separate calls:
    sparse_attn alone matches the oracle's patch-only attention, the merged
    result matches the oracle layer (two bf16 roundings on patch rows), and
    the packed variants give the same bytes as the self-packing calls."""
    import torch
    from gpu_helpers import compare_rows, from_dev_bf16, oracle_rows, layer_shape, say
    x = inputs(name)
    cfg = x.cfg
    shape = layer_shape(cfg)
    say(f"[calls] {name}")
    q, k, v = _upload(x)
    bufs = lib.layer(shape, q, k, v, cfg.rho, cfg.tau, x.rho_per_head)
    probs = lib.predict_mask(shape, q, k)
    row_ptr, col_idx = lib.select(shape, probs, cfg.rho, cfg.tau, x.rho_per_head)
    o, lse = lib.sparse_attn(shape, q, k, v, row_ptr, col_idx)
    kv = lib.pack_kv(shape, k, v)
    o2, lse2 = torch.zeros_like(o), torch.zeros_like(lse)
    lib.sparse_attn_packed(shape, q, kv, row_ptr, col_idx, o2, lse2)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o2.view(torch.int16)) and torch.equal(lse, lse2)
    rp = row_ptr.cpu().numpy().astype(np.int64)
    ci = col_idx.cpu().numpy()[:rp[-1]]
    o_np, lse_np = from_dev_bf16(o), lse.cpu().numpy()
    o_first = o_np.copy()  # the patch rows before the in-place merge
    B = lib.num_blocks(shape)
    sampled = {h: sample_blocks(name, B, h) for h in range(cfg.heads)}
    rms = _rms_dense(x, sampled)
    worst = worst_raw = 0.0
    for h in range(cfg.heads):
        out = oracle_rows(x, h, O.kept_lists(rp, ci, h, B), sampled[h],
                          include_special_keys=False, special_queries=False)
        eo, el, _, _, raw = compare_rows(out, o_np[h], lse_np[h])
        worst, worst_raw = max(worst, eo), max(worst_raw, raw)
        assert el <= LSE_TOL
    say(f"   sparse-only err beyond bf16 rounding {worst / rms:.3e} rms (plain {worst_raw / rms:.3e})")
    assert worst <= O_TOL * rms
    lib.special_dense(shape, q, k, v, o, lse)
    lib.special_dense_packed(shape, q, kv, o2, lse2)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o2.view(torch.int16)) and torch.equal(lse, lse2)
    assert torch.equal(bufs.probs, probs)
    assert torch.equal(bufs.row_ptr, row_ptr)
    n = int(rp[-1])
    assert torch.equal(bufs.col_idx[:n], col_idx[:n])
    o_np, lse_np = from_dev_bf16(o), lse.cpu().numpy()
    worst = worst_raw = 0.0
    for h in range(cfg.heads):
        out = oracle_rows(x, h, O.kept_lists(rp, ci, h, B), sampled[h])
        eo, el, _, _, raw = compare_rows(out, o_np[h], lse_np[h], o_intermediate=o_first[h])
        worst, worst_raw = max(worst, eo), max(worst_raw, raw)
        assert el <= LSE_TOL
    say(f"   merged err beyond two bf16 roundings {worst / rms:.3e} rms (plain {worst_raw / rms:.3e})")
    assert worst <= O_TOL * rms
    # the layer's two row calls on the same packed K/V give the layer's bytes
    o3, lse3 = torch.zeros_like(o), torch.zeros_like(lse)
    lib.patch_rows_packed(shape, q, kv, row_ptr, col_idx, o3, lse3)
    lib.special_rows_packed(shape, q, kv, o3, lse3)
    torch.cuda.synchronize()
    assert torch.equal(bufs.o.view(torch.int16), o3.view(torch.int16))
    assert torch.equal(bufs.lse, lse3)


@pytest.mark.parametrize("name", ["tiny-4f", "vggt-8f", "vggt-32f", "ragged-b128",
                                  "multi-frame-block-b64", "no-special-b64"])
def test_dense_parity(lib, name):
    import torch
    from gpu_helpers import compare_rows, from_dev_bf16, oracle_rows, layer_shape, say
    x = inputs(name)
    cfg = x.cfg
    shape = layer_shape(cfg)
    say(f"[dense] {name}")
    q, k, v = _upload(x)
    o, lse = lib.dense_attn(shape, q, k, v)
    torch.cuda.synchronize()
    o_np, lse_np = from_dev_bf16(o), lse.cpu().numpy()
    B = lib.num_blocks(shape)
    sampled = {h: sample_blocks(name, B, h) for h in range(cfg.heads)}
    worst_o = worst_l = worst_raw = 0.0
    acc = cnt = 0.0
    for h in range(cfg.heads):
        out = oracle_rows(x, h, None, sampled[h])
        eo, el, ms, n, raw = compare_rows(out, o_np[h], lse_np[h])
        worst_o, worst_l, worst_raw = max(worst_o, eo), max(worst_l, el), max(worst_raw, raw)
        acc, cnt = acc + ms * n, cnt + n
    rms = (acc / cnt) ** 0.5
    say(f"   err beyond bf16 rounding {worst_o / rms:.3e} rms (plain {worst_raw / rms:.3e}); "
        f"max|dLSE| = {worst_l:.3e}")
    assert worst_o <= O_TOL * rms and worst_l <= LSE_TOL
    kv = lib.pack_kv(shape, k, v)
    o2, lse2 = torch.zeros_like(o), torch.zeros_like(lse)
    lib.dense_attn_packed(shape, q, kv, o2, lse2)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o2.view(torch.int16)) and torch.equal(lse, lse2)


@pytest.mark.parametrize("name", ["tiny-4f", "ragged-b128", "multi-frame-block-b64"])
def test_full_mask_is_dense(lib, name):
    """rho = 0, tau = 1 keeps every block; the layer then equals dense
    attention (both against the oracle's dense rows, and bit-for-bit equal
    masks: every row lists all B blocks)."""
    import torch
    from gpu_helpers import compare_rows, from_dev_bf16, oracle_rows, layer_shape, say
    x = inputs(name)
    cfg = x.cfg
    shape = layer_shape(cfg)
    say(f"[full mask] {name}")
    q, k, v = _upload(x)
    bufs = lib.layer(shape, q, k, v, 0.0, 1.0)
    torch.cuda.synchronize()
    B = lib.num_blocks(shape)
    rp = bufs.row_ptr.cpu().numpy()
    assert np.all(np.diff(rp) == B)
    ci = bufs.col_idx.cpu().numpy()[:rp[-1]]
    assert np.array_equal(ci, np.tile(np.arange(B), cfg.heads * B))
    o, lse = from_dev_bf16(bufs.o), bufs.lse.cpu().numpy()
    acc = cnt = worst = worst_raw = 0.0
    for h in range(cfg.heads):
        out = oracle_rows(x, h, None, list(range(B)))
        eo, el, ms, n, raw = compare_rows(out, o[h], lse[h])
        worst, worst_raw = max(worst, eo), max(worst_raw, raw)
        acc, cnt = acc + ms * n, cnt + n
        assert el <= LSE_TOL
    rms = (acc / cnt) ** 0.5
    say(f"   err beyond bf16 rounding {worst / rms:.3e} rms (plain {worst_raw / rms:.3e})")
    assert worst <= O_TOL * rms


def test_empty_rows_use_special_keys_only(lib):
    """rho = 1, tau = 0 keeps no patch block: patch queries see only the
    special tokens (a valid corner of the two thresholds)."""
    import torch
    from gpu_helpers import compare_rows, from_dev_bf16, oracle_rows, layer_shape, say
    x = inputs("ragged-b128")
    cfg = x.cfg
    shape = layer_shape(cfg)
    say("[empty rows] ragged-b128")
    q, k, v = _upload(x)
    bufs = lib.layer(shape, q, k, v, 1.0, 0.0)
    torch.cuda.synchronize()
    assert int(bufs.row_ptr[-1].item()) == 0
    B = lib.num_blocks(shape)
    o, lse = from_dev_bf16(bufs.o), bufs.lse.cpu().numpy()
    for h in range(cfg.heads):
        out = oracle_rows(x, h, [np.zeros(0, np.int64)] * B, list(range(B)))
        eo, el, ms, _, raw = compare_rows(out, o[h], lse[h])
        say(f"   head {h}: err beyond bf16 rounding {eo / ms ** 0.5:.3e} rms "
            f"(plain {raw / ms ** 0.5:.3e})")
        assert eo <= O_TOL * ms ** 0.5 and el <= LSE_TOL


def test_layer_is_deterministic(lib):
    import torch
    from gpu_helpers import layer_shape, say
    x = inputs("vggt-8f")
    shape = layer_shape(x.cfg)
    say("[determinism] vggt-8f")
    q, k, v = _upload(x)
    a = lib.layer(shape, q, k, v, x.cfg.rho, x.cfg.tau)
    o1, l1, p1 = a.o.clone(), a.lse.clone(), a.probs.clone()
    lib.layer(shape, q, k, v, x.cfg.rho, x.cfg.tau, bufs=a)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), a.o.view(torch.int16))
    assert torch.equal(l1, a.lse) and torch.equal(p1, a.probs)


def test_end_to_end_mask_vs_oracle_pipeline(lib):
    """Reported, not gated: masks from the GPU's probabilities vs masks from
    the oracle's own float64 probabilities; differences can only come from
    near-ties in the ranking or the coverage threshold."""
    import torch
    from gpu_helpers import layer_shape, say
    for name in ("tiny-4f", "vggt-8f", "vggt-32f"):
        x = inputs(name)
        cfg = x.cfg
        shape = layer_shape(cfg)
        q, k, _ = _upload(x)
        probs = lib.predict_mask(shape, q, k)
        rp, ci = lib.select(shape, probs, cfg.rho, cfg.tau)
        torch.cuda.synchronize()
        rp = rp.cpu().numpy().astype(np.int64)
        ci = ci.cpu().numpy()[:rp[-1]]
        _, patch = O.token_roles(cfg.frames, cfg.patches_per_frame, cfg.special_per_frame)
        p64 = np.stack([O.predict_head(synth.bf16_bits_to_f64(x.q[h][patch]),
                                       synth.bf16_bits_to_f64(x.k[h][patch]), cfg.block)[3]
                        for h in range(cfg.heads)])
        orp, oci = O.select_blocks(p64.astype(np.float32), cfg.tau, cfg.rho)
        B = lib.num_blocks(shape)
        rows = cfg.heads * B
        diff = sum(1 for r in range(rows)
                   if not np.array_equal(ci[rp[r]:rp[r + 1]], oci[orp[r]:orp[r + 1]]))
        say(f"[e2e mask] {name}: {diff} of {rows} rows differ from the float64 pipeline "
            f"(nnz gpu {rp[-1]}, oracle {orp[-1]})")


def _row_order(row_ptr, heads, blocks):
    """The order the patch-row call (with a workspace, B <= 4096) works each
    head's query blocks in: longest kept list first, ties by block index.
    Returns, per head-major position, the head-major row."""
    lens = np.diff(np.asarray(row_ptr, dtype=np.int64)).clip(0, blocks).reshape(heads, blocks)
    out = []
    for h in range(heads):
        order = sorted(range(blocks), key=lambda i: (-int(lens[h, i]), i))
        out += [h * blocks + i for i in order]
    return out


def _split_rows(rows, blocks, m, xcds=8, order=None):
    """Rows (head-major query blocks) that the patch-row call at b = 128 runs
    as key-range pieces: those at the positions of each XCD's last, partial
    round of m workgroup slots (positions are dealt to XCDs in equal
    contiguous ranges; ``order`` maps a position to its row), unless no piece
    count shortens that round."""
    from test_abi_host import tail_pieces
    per = -(-rows // xcds)
    rems = [(min(rows, (x + 1) * per) - x * per) % m for x in range(xcds)
            if min(rows, (x + 1) * per) > x * per]
    if tail_pieces(max(rems), blocks, m) == 0:
        return []
    out = []
    for x in range(xcds):
        r0 = x * per
        n_x = min(rows, r0 + per) - r0
        if n_x <= 0:
            break
        full = n_x // m * m
        out += list(range(r0 + full, r0 + n_x))
    return [order[p] for p in out] if order is not None else out


@pytest.mark.parametrize("name", ["vggt-32f", "ragged-b128", "over-half-b128"])
def test_patch_rows_tail_pieces(lib, name):
    """bsga_patch_rows_packed with its workspace works each head's query
    blocks longest kept list first and splits the rows of the last, partial
    round (the shortest) into key-range pieces, merged afterwards: those rows
    (every query) match the oracle within the usual bars, and every other row
    is byte-identical to the call without workspace (one workgroup per row,
    natural order)."""
    import torch
    from gpu_helpers import compare_rows, from_dev_bf16, layer_shape, oracle_rows, say
    x = inputs(name)
    cfg = x.cfg
    shape = layer_shape(cfg)
    q, k, v = _upload(x)
    probs = lib.predict_mask(shape, q, k)
    row_ptr, col_idx = lib.select(shape, probs, cfg.rho, cfg.tau, x.rho_per_head)
    kv = lib.pack_kv(shape, k, v)
    o1, l1 = torch.zeros_like(q), torch.zeros((cfg.heads, cfg.tokens), dtype=torch.float32,
                                              device=q.device)
    o2, l2 = torch.zeros_like(o1), torch.zeros_like(l1)
    lib.patch_rows_packed(shape, q, kv, row_ptr, col_idx, o1, l1, ws=None)
    lib.patch_rows_packed(shape, q, kv, row_ptr, col_idx, o2, l2)
    torch.cuda.synchronize()
    B = lib.num_blocks(shape)
    m = 3 * torch.cuda.get_device_properties(0).multi_processor_count // 8
    split = _split_rows(cfg.heads * B, B, m,
                        order=_row_order(row_ptr.cpu().numpy(), cfg.heads, B))
    say(f"[tail pieces] {name}: {len(split)} of {cfg.heads * B} query blocks split, {m} slots/XCD")
    assert split, "the shape should leave a partial last round"
    rp = row_ptr.cpu().numpy().astype(np.int64)
    ci = col_idx.cpu().numpy()[:rp[-1]]
    _, patch = O.token_roles(cfg.frames, cfg.patches_per_frame, cfg.special_per_frame)
    tok_of_block = [patch[O.block_members(cfg.n_patch, cfg.block, i)] for i in range(B)]
    same = torch.ones((cfg.heads, cfg.tokens), dtype=torch.bool, device=q.device)
    by_head = {}
    for r in split:
        h, i = divmod(r, B)
        by_head.setdefault(h, []).append(i)
        same[h, torch.from_numpy(tok_of_block[i]).to(q.device)] = False
    eq = (o1.view(torch.int16) == o2.view(torch.int16)).all(dim=2) & (l1 == l2)
    assert bool(eq[same].all()), "unsplit rows differ"
    o2n, l2n = from_dev_bf16(o2), l2.cpu().numpy()
    worst = worst_l = worst_raw = 0.0
    acc = cnt = 0.0
    for h, blocks in sorted(by_head.items()):
        blocks = blocks[:6]
        out = oracle_rows(x, h, O.kept_lists(rp, ci, h, B), blocks, special_queries=False)
        dense = oracle_rows(x, h, None, blocks, special_queries=False)
        d = np.stack([r[0] for r in dense.values()])
        acc += float(np.sum(d ** 2))
        cnt += d.size
        eo, el, _, _, raw = compare_rows(out, o2n[h], l2n[h])
        worst, worst_l, worst_raw = max(worst, eo), max(worst_l, el), max(worst_raw, raw)
    rms = (acc / cnt) ** 0.5
    say(f"   split rows: err beyond bf16 rounding {worst / rms:.3e} rms(O_dense) (plain "
        f"{worst_raw / rms:.3e}), |dLSE| {worst_l:.1e}")
    assert worst <= O_TOL * rms and worst_l <= LSE_TOL


def test_patch_rows_unsplit_when_last_round_large(lib):
    """720 query blocks (16 heads x 45) leave 90 per XCD for the last round of
    96 slots: no piece count shortens it, so the plan splits nothing, the
    workspace holds only the order of the query blocks (one int32 per row),
    and the call with a workspace (longest rows first) is byte-identical to
    the one without (natural order)."""
    import torch
    from gpu_helpers import layer_shape, say
    x = synth.random_layer(1, 72, 80, 16, 128, seed=21)
    cfg = x.cfg
    shape = layer_shape(cfg)
    B = lib.num_blocks(shape)
    m = 3 * torch.cuda.get_device_properties(0).multi_processor_count // 8
    if _split_rows(cfg.heads * B, B, m):
        pytest.skip(f"{m} slots per XCD split this shape")
    assert lib.workspace_bytes(shape, lib.OP_PATCH_ROWS_PACKED) == -(-cfg.heads * B * 4 // 256) * 256
    q, k, v = _upload(x)
    probs = lib.predict_mask(shape, q, k)
    row_ptr, col_idx = lib.select(shape, probs, cfg.rho, cfg.tau)
    kv = lib.pack_kv(shape, k, v)
    o1, l1 = torch.zeros_like(q), torch.zeros((cfg.heads, cfg.tokens), dtype=torch.float32,
                                              device=q.device)
    o2, l2 = torch.zeros_like(o1), torch.zeros_like(l1)
    lib.patch_rows_packed(shape, q, kv, row_ptr, col_idx, o1, l1, ws=None)
    lib.patch_rows_packed(shape, q, kv, row_ptr, col_idx, o2, l2)
    torch.cuda.synchronize()
    say(f"[unsplit last round] {cfg.heads * B} query blocks, {m} slots/XCD")
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)
