"""Backward of the layer's attention (bsga_attn_backward) against the oracle's
gradients for the same mask.

The forward runs through bsga_layer (mask, O, LSE); dO is seeded N(0,1)
rounded to bf16; the oracle differentiates the plain masked softmax attention
in float64 on the same bf16 inputs.  Bar, per gradient tensor of a head:
max |g_gpu - g_oracle| <= 2e-2 * rms(g_oracle).  (With P and dS as single
bf16 operands and D from the stored bf16 O, dQ missed this by an order of
magnitude on the peaked synthetic heads, since a query's dS are small
differences that sum to zero; the kernels therefore feed dS to the dQ and dK
products as a bf16 pair hi + lo, P to the dV product once as float16 (11
significant bits), and recompute D from P and dP.)
"""
from __future__ import annotations

import numpy as np
import pytest

from block_sparse_global_bsga_amd import synth
from oracle import bsga_oracle as O

pytestmark = pytest.mark.gpu

G_TOL = 2e-2

CASES = {
    "tiny-4f": (lambda: synth.generate(synth.CONFIGS[1]), None),
    "ragged-b128": (lambda: synth.random_layer(3, 10, 13, 2, 128, seed=11, kind="corr"), None),
    "multi-frame-block-b64": (lambda: synth.random_layer(5, 5, 10, 3, 64, seed=12), None),
    "no-special-b64": (lambda: synth.random_layer(2, 16, 16, 2, 64, seed=13, special_per_frame=0,
                                                  kind="corr"), None),
    "single-block": (lambda: synth.random_layer(1, 8, 8, 1, 128, seed=15), None),
    "vggt-8f": (lambda: synth.generate(synth.CONFIGS[2]), [0, 7]),
    "vggt-32f": (lambda: synth.generate(synth.CONFIGS[3]), [5]),
}


@pytest.fixture(scope="module")
def lib():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from block_sparse_global_bsga_amd import bsga
    return bsga


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("tau", [None, 0.0])
def test_backward(lib, name, tau):
    import torch
    from gpu_helpers import head_f64, layer_shape, say, to_dev
    make, heads = CASES[name]
    x = make()
    cfg = x.cfg
    tau = cfg.tau if tau is None else tau
    shape = layer_shape(cfg)
    say(f"[backward] {name} N={cfg.tokens} H={cfg.heads} b={cfg.block} tau={tau}")
    q, k, v = to_dev(x.q), to_dev(x.k), to_dev(x.v)
    bufs = lib.layer(shape, q, k, v, cfg.rho, tau, x.rho_per_head)
    rng = np.random.default_rng(77)
    do_bits = synth.fp32_to_bf16_bits(
        rng.standard_normal((cfg.heads, cfg.tokens, 64), dtype=np.float32))
    d_o = to_dev(do_bits)
    dq, dk, dv = lib.attn_backward(shape, q, k, v, bufs.o, bufs.lse, d_o, bufs.row_ptr,
                                   bufs.col_idx)
    torch.cuda.synchronize()
    rp = bufs.row_ptr.cpu().numpy().astype(np.int64)
    ci = bufs.col_idx.cpu().numpy()[:rp[-1]]
    B = lib.num_blocks(shape)
    g_gpu = [t.cpu().numpy() for t in (dq, dk, dv)]
    worst = [0.0, 0.0, 0.0]
    for h in (range(cfg.heads) if heads is None else heads):
        qh, kh, vh = head_f64(x, h)
        doh = synth.bf16_bits_to_f64(do_bits[h])
        ref = O.attention_backward_head(qh, kh, vh, doh, cfg.frames, cfg.patches_per_frame,
                                        cfg.special_per_frame, cfg.block,
                                        O.kept_lists(rp, ci, h, B))
        for j in range(3):
            rms = float(np.sqrt(np.mean(ref[j] ** 2)))
            err = float(np.abs(g_gpu[j][h] - ref[j]).max())
            worst[j] = max(worst[j], err / rms)
    say(f"   max err / rms(grad): dQ {worst[0]:.2e}, dK {worst[1]:.2e}, dV {worst[2]:.2e}")
    assert max(worst) <= G_TOL


def test_backward_dense_mask_equals_dense(lib):
    """rho = 0, tau = 1 keeps every block: the gradients equal those of dense
    attention (oracle with no mask)."""
    import torch
    from gpu_helpers import head_f64, layer_shape, to_dev
    x = synth.random_layer(3, 10, 13, 2, 128, seed=21, kind="corr")
    cfg = x.cfg
    shape = layer_shape(cfg)
    q, k, v = to_dev(x.q), to_dev(x.k), to_dev(x.v)
    bufs = lib.layer(shape, q, k, v, 0.0, 1.0)
    d_o = to_dev(synth.fp32_to_bf16_bits(
        np.random.default_rng(3).standard_normal((cfg.heads, cfg.tokens, 64), dtype=np.float32)))
    grads = lib.attn_backward(shape, q, k, v, bufs.o, bufs.lse, d_o, bufs.row_ptr, bufs.col_idx)
    torch.cuda.synchronize()
    dob = synth.bf16_bits_to_f64(d_o.view(torch.int16).cpu().numpy().view(np.uint16))
    for h in range(cfg.heads):
        qh, kh, vh = head_f64(x, h)
        ref = O.attention_backward_head(qh, kh, vh, dob[h], cfg.frames, cfg.patches_per_frame,
                                        cfg.special_per_frame, cfg.block, None)
        for g, r in zip(grads, ref):
            assert np.abs(g[h].cpu().numpy() - r).max() <= G_TOL * np.sqrt(np.mean(r ** 2))


@pytest.mark.parametrize("via", ["sweep", "o32"])
@pytest.mark.parametrize("index", [4, 5])
def test_backward_full_size(lib, index, via):
    """Full-size layers (100 frames, 78,200 tokens; 200 frames, 274,800
    tokens, per-head rho).  The oracle cannot afford every query row there,
    so:

    * dQ of sampled query rows (a patch query block per checked head, the
      partial last block for the first, and 8 special queries) is exact
      oracle parity: max |dQ_gpu - dQ_oracle| <= 2e-2 rms(dQ_oracle rows);
    * dV and dK of sampled keys (patch keys of two key blocks and 4 special
      keys per checked head) must satisfy the gradient formulas with the
      forward's own outputs: P_qk = exp(q.k/8 - LSE_q) over every query q
      that sees key k, dV_k = sum_q P_qk dO_q, dK_k = sum_q P_qk (dO_q.v_k -
      D_q) q_q / 8 with D_q = dO_q . O_q.  Bounds: 1e-4 of the matching sum
      of magnitudes, plus for dK the effect of O's bf16 rounding on D_q
      (|dD_q| <= 2^-8 |dO_q| |O_q|), and for dV the float16 rounding of each
      weight P_qk (relative at most 2^-11, dO exact in float16), i.e.
      (2^-11 + 1e-4) sum_q P_qk |dO_q|.  With via = "o32" the forward is
      bsga_layer_train and the backward bsga_attn_backward_o32: D_q = dO_q .
      O_q from the float32 rows on both sides (the GPU sums its 64 products in
      float32: |dD_q| <= 2^-16 |dO_q| |O_q| set aside instead of 2^-8);
    * over all keys of each head: sum_k dV_k = sum_q dO_q (softmax rows sum
      to one) within (2^-11 + 1e-5) sum_q |dO_q| (the float16 weights of a
      row sum to one within 2^-11 of their sum), and sum_k dK_k = 0 (a
      query's dS sum to zero) within 1e-5 of sum_q |q_q| |dO_q| max_k |v_k| /
      8: a row's float32 weights sum to one within about 1e-6, and D is
      formed from the same weights as dS."""
    _full_size_backward(lib, synth.generate(synth.CONFIGS[index]), via, 8000 + index)


@pytest.mark.parametrize("via", ["sweep", "o32"])
@pytest.mark.parametrize("block, grid_w", [(128, 1024), (64, 512)])
def test_backward_max_blocks(lib, block, grid_w, via):
    """The largest block count the selection takes, B = 4096 (the layers of
    test_gpu_max_sizes: one frame of 512 x 1024 patches at b = 128, 512 x 512
    at b = 64, five special tokens, rho 0.99, tau 0, 40 kept blocks per row):
    the transposed mask at its largest, through both backward calls, to the
    checks of test_backward_full_size (dQ rows of sampled query blocks exact
    against the oracle, dV and dK of sampled keys against the gradient
    formulas, the column sums over every key)."""
    x = synth.random_layer(1, 512, grid_w, 1, block, seed=4500 + block, special_per_frame=5,
                           kind="diffuse", rho=0.99, tau=0.0)
    _full_size_backward(lib, x, via, 8100 + block)


def _full_size_backward(lib, x, via, seed):
    import torch
    from gpu_helpers import from_dev_bf16, head_f64, layer_shape, say, to_dev
    cfg = x.cfg
    H, N = cfg.heads, cfg.tokens
    say(f"[backward-full-size] {cfg.name}: N={N} H={H} b={cfg.block} ({via})")
    shape = layer_shape(cfg)
    q, k, v = to_dev(x.q), to_dev(x.k), to_dev(x.v)
    if via == "o32":
        bufs, o_fwd = lib.layer_train(shape, q, k, v, cfg.rho, cfg.tau, x.rho_per_head)
    else:
        bufs = lib.layer(shape, q, k, v, cfg.rho, cfg.tau, x.rho_per_head)
        o_fwd = bufs.o
    rng = np.random.default_rng(seed)
    do_bits = synth.fp32_to_bf16_bits(rng.standard_normal((H, N, 64), dtype=np.float32))
    d_o = to_dev(do_bits)
    dq, dk, dv = lib.attn_backward(shape, q, k, v, o_fwd, bufs.lse, d_o, bufs.row_ptr,
                                   bufs.col_idx)
    torch.cuda.synchronize()
    say(f"   layer and backward done ({via})")
    B = lib.num_blocks(shape)
    rp = bufs.row_ptr.cpu().numpy().astype(np.int64)
    ci = bufs.col_idx.cpu().numpy()[:rp[-1]].astype(np.int64)
    lse_all = bufs.lse.cpu().numpy().astype(np.float64)
    o_all = o_fwd
    d_round = 2.0 ** -16 if via == "o32" else 2.0 ** -8  # the forward rows' rounding
    del q, k, v
    spec, patch = O.token_roles(cfg.frames, cfg.patches_per_frame, cfg.special_per_frame)
    n_p = patch.shape[0]
    rho_h = list(x.rho_per_head) if x.rho_per_head is not None else [cfg.rho] * H
    heads = sorted({0, H - 1} | {int(np.argmin(rho_h)), int(np.argmax(rho_h))})
    worst = {"dq": 0.0, "dv": 0.0, "dk": 0.0, "sum_dv": 0.0, "sum_dk": 0.0}
    for h in range(H):
        # column-sum identities over all keys of the head
        dvh = dv[h].double().cpu().numpy()
        dkh = dk[h].double().cpu().numpy()
        doh = synth.bf16_bits_to_f64(do_bits[h])
        qh = synth.bf16_bits_to_f64(x.q[h])
        vmax = float(np.sqrt((synth.bf16_bits_to_f64(x.v[h]) ** 2).sum(axis=1)).max())
        r_dv = np.abs(dvh.sum(axis=0) - doh.sum(axis=0)) / np.abs(doh).sum(axis=0)
        mag = float(np.sum(np.linalg.norm(qh, axis=1) * np.linalg.norm(doh, axis=1))) * vmax / 8
        r_dk = np.abs(dkh.sum(axis=0)) / mag
        worst["sum_dv"] = max(worst["sum_dv"], float(r_dv.max()))
        worst["sum_dk"] = max(worst["sum_dk"], float(r_dk.max()))
        assert r_dv.max() <= 2.0 ** -11 + 1e-5 and r_dk.max() <= 1e-5, (h, r_dv.max(), r_dk.max())
        if h not in heads:
            continue
        qh, kh, vh = head_f64(x, h)
        kept = O.kept_lists(rp, ci, h, B)
        # --- dQ rows: exact oracle parity
        blk = B - 1 if h == heads[0] else int(rng.integers(0, B))
        sq = np.sort(rng.choice(spec, size=min(8, spec.shape[0]), replace=False))
        ref = O.attention_backward_head(qh, kh, vh, doh, cfg.frames, cfg.patches_per_frame,
                                        cfg.special_per_frame, cfg.block, kept,
                                        query_blocks=[blk], special_queries=sq)[0]
        rows = np.concatenate([patch[O.block_members(n_p, cfg.block, blk)], sq])
        got = dq[h][torch.from_numpy(rows).to(dq.device)].double().cpu().numpy()
        rms = float(np.sqrt(np.mean(ref[rows] ** 2)))
        worst["dq"] = max(worst["dq"], float(np.abs(got - ref[rows]).max()) / rms)
        # --- dV, dK of sampled keys against the forward's LSE and O
        oh = o_all[h].double().cpu().numpy() if via == "o32" else from_dev_bf16(o_all[h])
        lse = lse_all[h]
        dd = np.sum(doh * oh, axis=1)
        seen_by = [[] for _ in range(B)]  # query blocks keeping each key block
        for i, cols in enumerate(kept):
            for j in cols:
                seen_by[int(j)].append(i)
        kblocks = rng.choice(B, size=2, replace=False)
        keys = [int(t) for j in kblocks
                for t in rng.choice(patch[O.block_members(n_p, cfg.block, int(j))], size=4,
                                    replace=False)]
        keys += [int(t) for t in rng.choice(spec, size=min(4, spec.shape[0]), replace=False)]
        dvg = dv[h][torch.tensor(keys, device=dv.device)].double().cpu().numpy()
        dkg = dk[h][torch.tensor(keys, device=dk.device)].double().cpu().numpy()
        pos = {int(t): i for i, t in enumerate(patch)}
        for r, t in enumerate(keys):
            if t in pos:
                qs = np.concatenate([patch[O.block_members(n_p, cfg.block, i)]
                                     for i in seen_by[pos[t] // cfg.block]] + [spec])
            else:
                qs = np.arange(N)
            p = np.exp(qh[qs] @ kh[t] / 8.0 - lse[qs])
            dp = doh[qs] @ vh[t]
            dv_ref = p @ doh[qs]
            dk_ref = (p * (dp - dd[qs])) @ qh[qs] / 8.0
            b_dv = (2.0 ** -11 + 1e-4) * (p @ np.abs(doh[qs])) + 1e-30
            b_dk = (1e-4 * ((p * (np.abs(dp) + np.abs(dd[qs]))) @ np.abs(qh[qs]))
                    + d_round * (p * np.linalg.norm(doh[qs], axis=1)
                                   * np.linalg.norm(oh[qs], axis=1)) @ np.abs(qh[qs])) / 8.0
            worst["dv"] = max(worst["dv"], float((np.abs(dvg[r] - dv_ref) / b_dv).max()))
            worst["dk"] = max(worst["dk"], float((np.abs(dkg[r] - dk_ref) / b_dk).max()))
    say(f"   dQ rows err {worst['dq']:.2e} rms; sampled keys: dV {worst['dv']:.2f}, "
        f"dK {worst['dk']:.2f} of their bounds; column sums: dV {worst['sum_dv']:.2e}, "
        f"dK {worst['sum_dk']:.2e}")
    assert worst["dq"] <= G_TOL
    assert worst["dv"] <= 1.0 and worst["dk"] <= 1.0
