"""Query-probe Top-K selection (bsga_probe_select) against the oracle.

* probe scores: within twice the float32 rounding bound of the computation
  (a mean accumulated through 8 + 32 + ceil(N / 256) sequential additions per
  dimension, then a 64-term dot product): per key
  u (n_add sum_j |k_j| mean_i |q_ij| + 64 sum_j |k_j qbar_j|) / 8, u = 2^-24;
* block lists: bit-exact against the oracle's ranking of the GPU's own float32
  scores (the ranking is an integer decision, taken in the same precision);
* attention with the probe's lists through bsga_patch_rows_packed: the same
  output bars as the two-threshold path.
"""
from __future__ import annotations

import numpy as np
import pytest

from block_sparse_global_bsga_amd import synth
from oracle import bsga_oracle as O

pytestmark = pytest.mark.gpu

CASES = {
    "tiny-4f": lambda: synth.generate(synth.CONFIGS[1]),
    "vggt-8f": lambda: synth.generate(synth.CONFIGS[2]),
    "vggt-32f": lambda: synth.generate(synth.CONFIGS[3]),
    "ragged-b128": lambda: synth.random_layer(3, 10, 13, 2, 128, seed=11, kind="corr"),
    "no-special-b64": lambda: synth.random_layer(2, 16, 16, 2, 64, seed=13, special_per_frame=0,
                                                 kind="corr"),
}
_cache = {}


def inputs(name):
    if name not in _cache:
        _cache.clear()
        _cache[name] = CASES[name]()
    return _cache[name]


@pytest.fixture(scope="module")
def lib():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from block_sparse_global_bsga_amd import bsga
    return bsga


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("frac", [0.0, 1e-4, 0.02, 0.3, 1.0, 2.0])
def test_probe_select(lib, name, frac):
    import torch
    from gpu_helpers import head_f64, layer_shape, say, to_dev
    x = inputs(name)
    cfg = x.cfg
    shape = layer_shape(cfg)
    n_p = cfg.n_patch
    topk = {0.0: 0, 1e-4: 1}.get(frac, int(frac * n_p))
    say(f"[probe] {name} topk={topk} of {n_p}")
    q, k = to_dev(x.q), to_dev(x.k)
    rp, ci, sc = lib.probe_select(shape, q, k, topk, want_scores=True)
    torch.cuda.synchronize()
    rp = rp.cpu().numpy().astype(np.int64)
    ci = ci.cpu().numpy()[:rp[-1]].astype(np.int64)
    sc = sc.cpu().numpy()
    B = lib.num_blocks(shape)
    _, patch = O.token_roles(cfg.frames, cfg.patches_per_frame, cfg.special_per_frame)
    worst = 0.0
    for h in range(cfg.heads):
        qh, kh, _ = head_f64(x, h)
        ref = O.probe_scores(qh, kh, cfg.frames, cfg.patches_per_frame, cfg.special_per_frame)
        u = 2.0 ** -24
        n_add = 8 + 32 + -(-cfg.tokens // 256)
        ka = np.abs(kh[patch])
        bound = 2 * u * (n_add * ka @ np.abs(qh).mean(axis=0)
                         + 64 * ka @ np.abs(qh.mean(axis=0))) / 8.0 + 1e-30
        err = np.abs(sc[h].astype(np.float64) - ref)
        assert np.all(err <= bound), (h, float((err / bound).max()))
        worst = max(worst, float((err / bound).max()))
        want = O.probe_blocks(sc[h].astype(np.float64), cfg.block, topk)
        for i in range(B):
            r = h * B + i
            assert np.array_equal(ci[rp[r]:rp[r + 1]], want), (h, i)
    say(f"   max score error {worst:.2f} of the bound; kept blocks per head "
        f"{[int(rp[h * B + 1] - rp[h * B]) for h in range(cfg.heads)]}")


@pytest.mark.parametrize("name", ["tiny-4f", "vggt-32f", "ragged-b128"])
def test_probe_attention(lib, name):
    """bsga_patch_rows_packed over the probe's block lists equals the oracle's
    masked softmax over the same kept blocks plus every special key."""
    import torch
    from gpu_helpers import compare_rows, from_dev_bf16, layer_shape, oracle_rows, say, to_dev
    x = inputs(name)
    cfg = x.cfg
    shape = layer_shape(cfg)
    topk = max(1, cfg.n_patch // 50)
    q, k, v = to_dev(x.q), to_dev(x.k), to_dev(x.v)
    rp, ci = lib.probe_select(shape, q, k, topk)
    kv = lib.pack_kv(shape, k, v)
    o = torch.zeros_like(q)
    lse = torch.zeros((cfg.heads, cfg.tokens), dtype=torch.float32, device=q.device)
    lib.patch_rows_packed(shape, q, kv, rp, ci, o, lse)
    torch.cuda.synchronize()
    rph = rp.cpu().numpy().astype(np.int64)
    cih = ci.cpu().numpy()[:rph[-1]]
    o_h, lse_h = from_dev_bf16(o), lse.cpu().numpy()
    B = lib.num_blocks(shape)
    rng = np.random.default_rng(31)
    worst_o = worst_l = worst_raw = 0.0
    acc = cnt = 0.0
    for h in range(cfg.heads):
        blocks = sorted({0, B - 1} | set(rng.choice(B, size=min(B, 3), replace=False).tolist()))
        kept = O.kept_lists(rph, cih, h, B)
        out = oracle_rows(x, h, kept, blocks, special_queries=False)
        dense = oracle_rows(x, h, None, blocks, special_queries=False)
        d = np.stack([r[0] for r in dense.values()])
        acc += float(np.sum(d ** 2))
        cnt += d.size
        eo, el, _, _, raw = compare_rows(out, o_h[h], lse_h[h])
        worst_o, worst_l, worst_raw = max(worst_o, eo), max(worst_l, el), max(worst_raw, raw)
    rms = (acc / cnt) ** 0.5
    say(f"[probe-attn] {name} topk={topk}: err beyond bf16 rounding {worst_o / rms:.3e} "
        f"rms(O_dense) (plain {worst_raw / rms:.3e}), dLSE {worst_l:.2e}")
    assert worst_o <= 2e-2 * rms and worst_l <= 2e-3
