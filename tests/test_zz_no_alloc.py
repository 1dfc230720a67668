"""bsga_select_static (the selection without a workspace, for callers that
cannot allocate) against bsga_select through the C ABI: bit-identical CSR on
two calls in a row, the second on a smaller input, then at the row limit
(65,536 rows), then a small input again.  The array the static call uses
keeps the previous call's contents, which must never leak into a result."""
from __future__ import annotations

import numpy as np
import pytest

pytestmark = pytest.mark.gpu


def _probs(rng, H, B, spread):
    s = rng.standard_normal((H, B, B)) * spread
    e = np.exp(s - s.max(axis=2, keepdims=True))
    return (e / e.sum(axis=2, keepdims=True)).astype(np.float32)


def _check(lib, shape, p_np, rho, tau, rho_h=None):
    import torch
    from gpu_helpers import DEV, say
    probs = torch.from_numpy(p_np).to(DEV)
    rp_a, ci_a = lib.select(shape, probs, rho, tau, rho_h)
    rp_b = torch.full_like(rp_a, -7)
    ci_b = torch.full_like(ci_a, -7)
    lib.select_static(shape, probs, rho, tau, rho_h, row_ptr=rp_b, col_idx=ci_b)
    torch.cuda.synchronize()
    n = int(rp_a[-1].item())
    say(f"[no-alloc select] H={shape.heads} B={lib.num_blocks(shape)} rows="
        f"{shape.heads * lib.num_blocks(shape)} nnz={n} rho={rho} tau={tau}")
    assert torch.equal(rp_a, rp_b)
    assert torch.equal(ci_a[:n], ci_b[:n])


def test_select_static_matches_select():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from block_sparse_global_bsga_amd import bsga as lib
    rng = np.random.default_rng(77)
    # 16 heads x 343 blocks (the 32-frame shape), then a smaller 8-head,
    # 172-block input with per-head budgets
    big = lib.LayerShape(32, 1369, 5, 16, 128)
    _check(lib, big, _probs(rng, 16, lib.num_blocks(big), 0.3), 0.75, 0.9)
    small = lib.LayerShape(8, 1369, 5, 8, 64)
    rho_h = [0.5, 0.75, 0.9, 0.95, 0.0, 1.0, 0.3, 0.6]
    _check(lib, small, _probs(rng, 8, lib.num_blocks(small), 2.0), 0.75, 0.5, rho_h)
    # the row limit: 64 heads x 1024 blocks = 65,536 rows (sorted by the LDS
    # kernel, B > 512), then a tiny input again
    limit = lib.LayerShape(1, 128 * 1024, 0, 64, 128)
    assert 64 * lib.num_blocks(limit) == lib.SELECT_STATIC_MAX_ROWS
    _check(lib, limit, _probs(rng, 64, 1024, 0.05), 0.9, 0.8)
    tiny = lib.LayerShape(1, 100, 2, 2, 64)
    _check(lib, tiny, _probs(rng, 2, lib.num_blocks(tiny), 1.0), 0.5, 0.9)
