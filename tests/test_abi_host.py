"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every symbol include/bsga.h declares, host-only calls return the right
values, and invalid arguments are rejected before anything is launched."""
import ctypes
import json
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bsga.h")

bsga = pytest.importorskip("block_sparse_global_bsga_amd.bsga",
                           reason="libbsga.so not built")
lib = bsga._lib
S = bsga.LayerShape


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\w[\w\s\*]*?\b(bsga_\w+)\(", text, flags=re.M)))


def test_exports_every_declared_symbol():
    names = declared_symbols()
    assert len(names) >= 12
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(bsga.EXPORTS) == names


def test_version_and_status_strings():
    assert bsga.version() == 3
    for s in range(6):
        assert bsga.status_string(s)
    assert bsga.status_string(99) == "unknown status"


def test_block_and_keep_counts_match_golden():
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "keep_counts.json")))
    for case in g["cases"]:
        # n_patch = frames * P with one frame holding all patches
        shape = S(frames=1, patches_per_frame=case["n_patch"], special_per_frame=5, heads=2,
                  block=case["block"])
        assert bsga.num_blocks(shape) == case["B"]
        for rho, k in zip(case["rho"], case["k"]):
            assert bsga.keep_count(case["B"], rho) == k


def test_keep_count_matches_oracle_definition():
    from oracle import bsga_oracle as O
    import numpy as np
    rng = np.random.default_rng(0)
    for _ in range(2000):
        B = int(rng.integers(0, 9000))
        rho = float(rng.integers(0, 1_000_001)) / 1e6
        assert bsga.keep_count(B, rho) == O.keep_count(B, rho)


def tail_pieces(max_rem, blocks, m=96, max_pieces=16):
    """Pieces per leftover row, as the plan defines them: for a largest
    leftover of at most half a round, as many as fit one round (at most
    max_pieces); for a fuller round the count whose ceil(max_rem p / m)
    rounds of 1/p of a row, plus 1 / (blocks + 1) of a row per piece, finish
    first, if under 0.8 of a row; else none."""
    if max_rem == 0:
        return 0
    if m // max_rem >= 2:
        return min(max_pieces, m // max_rem)
    best, pieces = 0.8, 0
    for p in range(2, max_pieces + 1):
        cost = (-(-max_rem * p // m)) / p + p / (blocks + 1)
        if cost < best:
            best, pieces = cost, p
    return pieces


def tail_bytes(rows, blocks, m=96, xcds=8, max_pieces=16):
    """Workspace of the split last round: rows dealt to XCDs in equal
    contiguous ranges, m slots per XCD, tail_pieces pieces per leftover row."""
    per = -(-rows // xcds)
    rems = [(min(rows, (x + 1) * per) - x * per) % m for x in range(xcds)
            if min(rows, (x + 1) * per) > x * per]
    return sum(rems) * tail_pieces(max(rems), blocks, m, max_pieces) * 128 * 66 * 4


def test_capacity_and_workspace_sizes():
    shape = S(32, 1369, 5, 16, 128)
    assert bsga.csr_capacity(shape) == 16 * 343 * 343
    sizes = {op: bsga.workspace_bytes(shape, op) for op in range(6)}
    assert sizes[bsga.OP_LAYER] >= max(sizes.values()) - 1
    assert sizes[bsga.OP_SPARSE_ATTN] >= 2 * 16 * (43904 + 256) * 64 * 2
    # probe selection: partial sums, mean query, scores, block lists, counts
    assert bsga.workspace_bytes(shape, bsga.OP_PROBE_SELECT) >= 16 * 43808 * 4
    # per-head NMSE: one float64 pair per head and chunk of 1024 rows
    assert bsga.workspace_bytes(shape, bsga.OP_NMSE) >= 16 * 43 * 16
    out = ctypes.c_size_t()
    assert bsga.workspace_bytes(shape, bsga.OP_BACKWARD) >= 7 * 16 * 44032 * 128
    # patch rows at b = 128: float32 partials (64 values, max and sum per
    # query) of the last round's split rows, then the order of the query
    # blocks (one int32 per row, for B <= 4096).  Without a device the plan
    # assumes 96 workgroup slots per XCD: 5488 rows are 686 per XCD, 14 of
    # them in the last round, split into 96 // 14 = 6 pieces each
    up = lambda x: -(-x // 256) * 256  # noqa: E731
    tail = bsga.workspace_bytes(shape, bsga.OP_PATCH_ROWS_PACKED)
    assert tail_bytes(5488, 343) == 8 * 14 * 6 * 128 * 66 * 4
    assert tail_bytes(5488, 343) + up(5488 * 4) <= tail <= tail_bytes(5488, 343) + up(5488 * 4) + 512
    assert bsga.workspace_bytes(shape, bsga.OP_LAYER) >= tail
    # patch rows at b = 64: the aligned-pair lists (a key-tile list of up to
    # ceil(B / 2) entries and its length per pair of query blocks), then the
    # split last round of the pair rows.  The 8-frame layer: B = 172, 86 pair
    # rows per head, 1376 rows, 172 per XCD, 76 in the last round of 96
    # slots: no piece count shortens it
    pairs = up(16 * 86 * 86 * 4) + up(16 * 86 * 4)
    assert tail_bytes(1376, 86) == 0
    assert bsga.workspace_bytes(S(8, 1369, 5, 16, 64), bsga.OP_PATCH_ROWS_PACKED) == pairs
    # past 4096 pair rows (B > 8192) the pair lists' LDS would not fit: the
    # call keeps the unpaired 64-row kernel, which needs no workspace
    assert bsga.workspace_bytes(S(400, 1369, 5, 2, 64), bsga.OP_PATCH_ROWS_PACKED) == 0
    assert bsga.workspace_bytes(S(382, 1369, 5, 2, 64), bsga.OP_PATCH_ROWS_PACKED) > 0
    # the four-frame layer: B = 16, 8 pair rows per head, 32 rows (4 heads),
    # 4 per XCD, split into 96 // 4 = 24 -> 16 pieces each
    pairs = up(4 * 8 * 8 * 4) + up(4 * 8 * 4)
    assert tail_bytes(32, 8) == 8 * 4 * 16 * 128 * 66 * 4
    assert pairs + tail_bytes(32, 8) <= bsga.workspace_bytes(S(4, 256, 5, 4, 64),
                                                          bsga.OP_PATCH_ROWS_PACKED) \
        <= pairs + tail_bytes(32, 8) + 512
    # 400 rows (16 heads x 25 blocks): 50 per XCD, more than half a round: 3
    # pieces each, in two rounds of a third of a row
    assert tail_pieces(50, 25) == 3 and tail_bytes(400, 25) == 8 * 50 * 3 * 128 * 66 * 4
    assert tail_bytes(400, 25) + up(400 * 4) <= bsga.workspace_bytes(
        S(1, 3200, 5, 16, 128), bsga.OP_PATCH_ROWS_PACKED) <= tail_bytes(400, 25) + up(400 * 4) + 512
    # the 100- and 200-frame layers: 64 and 56 of 96 slots in the last round
    assert tail_pieces(64, 608) == 3 and tail_pieces(56, 2140) == 12
    # 720 rows (16 x 45): 90 per XCD, no piece count shortens the round
    assert tail_pieces(90, 45) == 0
    assert bsga.workspace_bytes(S(1, 5760, 5, 16, 128), bsga.OP_PATCH_ROWS_PACKED) == up(720 * 4)
    # past B = 4096 the rows keep their natural order: no order array
    assert tail_bytes(4097, 4097) <= bsga.workspace_bytes(
        S(1, 4097 * 128, 0, 1, 128), bsga.OP_PATCH_ROWS_PACKED) <= tail_bytes(4097, 4097) + 512
    # 8 rows: one per XCD, split into the most pieces (16)
    assert tail_bytes(8, 8) == 8 * 1 * 16 * 128 * 66 * 4
    assert tail_bytes(8, 8) + up(8 * 4) <= bsga.workspace_bytes(
        S(1, 1024, 5, 1, 128), bsga.OP_PATCH_ROWS_PACKED) <= tail_bytes(8, 8) + up(8 * 4) + 512
    # 64 rows: 8 per XCD, 96 // 8 = 12 pieces
    assert tail_bytes(64, 8) == 8 * 8 * 12 * 128 * 66 * 4
    assert tail_bytes(64, 8) + up(64 * 4) <= bsga.workspace_bytes(
        S(1, 1024, 5, 8, 128), bsga.OP_PATCH_ROWS_PACKED) <= tail_bytes(64, 8) + up(64 * 4) + 512
    assert lib.bsga_workspace_bytes(ctypes.byref(shape.c()), bsga.OP_PATCH_ROWS_PACKED + 1,
                                    ctypes.byref(out)) == bsga.ERR_INVALID_ARG


def special_splits(heads, special_tiles, key_tiles, slots=768):
    """Key ranges of the special rows, as the plan defines them: the count
    minimising rounds of workgroups (heads x special query tiles x ranges
    over `slots`) times (tiles per range + 1), fewest ranges on ties."""
    best = None
    for want in range(1, min(key_tiles, 1024) + 1):
        tps = -(-key_tiles // want)
        ns = -(-key_tiles // tps)
        cost = -(-heads * special_tiles * ns // slots) * (tps + 1)
        if best is None or cost < best[0]:
            best = (cost, ns)
    return best[1]


def test_special_rows_workspace():
    """The special rows' split-K workspace holds float32 partial rows (64
    values, max and sum) for every (head, padded special row, key range)."""
    def expect(shape, ns):
        slots = shape.heads * (-(-shape.frames * shape.special_per_frame // 128) * 128) * ns
        return ((slots * 64 * 4 + 255) & ~255) + slots * 2 * 4
    # 32 frames: 16 heads x 2 special query tiles; 343 + 2 key tiles split
    # into 23 ranges of 15 (736 workgroups, one round of 768 slots)
    c3 = S(32, 1369, 5, 16, 128)
    assert special_splits(16, 2, 345) == 23
    assert bsga.workspace_bytes(c3, bsga.OP_SPECIAL_DENSE_PACKED) == expect(c3, 23)
    # one head, 8 frames of 32 x 32 patches: 64 + 1 key tiles, one range each
    one = S(8, 1024, 5, 1, 128)
    assert special_splits(1, 1, 65) == 65
    assert bsga.workspace_bytes(one, bsga.OP_SPECIAL_DENSE_PACKED) == expect(one, 65)
    assert bsga.workspace_bytes(S(4, 256, 0, 2, 64), bsga.OP_SPECIAL_DENSE_PACKED) == 0


def test_probe_select_validation():
    """Argument checks of bsga_probe_select run before any launch (no GPU)."""
    shape = S(2, 16, 5, 2, 64)
    c = shape.c()
    buf = (ctypes.c_uint8 * 4096)()
    p16 = ctypes.addressof(buf) + (-ctypes.addressof(buf)) % 256
    cap = bsga.csr_capacity(shape)
    ok_args = [ctypes.byref(c), p16, p16, 3, None, p16, p16, cap, p16, 1 << 40, None]
    for i, bad in [(1, None), (2, p16 + 2), (3, -1), (4, p16 + 2), (5, None), (7, cap - 1),
                   (8, None)]:
        args = list(ok_args)
        args[i] = bad
        assert lib.bsga_probe_select(*args) != bsga.OK, i


def _status(fn, *args):
    return fn(*args)


def test_invalid_shapes_rejected():
    out = ctypes.c_int32()
    bad = [S(0, 10, 5, 1, 64), S(1, 0, 5, 1, 64), S(1, 10, -1, 1, 64), S(1, 10, 5, 0, 64)]
    for s in bad:
        assert lib.bsga_num_blocks(ctypes.byref(s.c()), ctypes.byref(out)) == bsga.ERR_INVALID_ARG
    for s in [S(1, 10, 5, 1, 32), S(1, 10, 5, 1, 256)]:
        assert lib.bsga_num_blocks(ctypes.byref(s.c()), ctypes.byref(out)) == bsga.ERR_UNSUPPORTED
    s = S(1, 10, 5, 1, 64, head_dim=128)
    assert lib.bsga_num_blocks(ctypes.byref(s.c()), ctypes.byref(out)) == bsga.ERR_UNSUPPORTED
    assert lib.bsga_num_blocks(None, ctypes.byref(out)) == bsga.ERR_INVALID_ARG
    # too many tokens for 32-bit byte offsets within a head (N + 256 >= 2^24)
    s = S(40000, 1369, 5, 1, 128)
    assert lib.bsga_num_blocks(ctypes.byref(s.c()), ctypes.byref(out)) == bsga.ERR_UNSUPPORTED
    s = S(12211, 1369, 5, 1, 128)    # 16,777,914 tokens
    assert lib.bsga_num_blocks(ctypes.byref(s.c()), ctypes.byref(out)) == bsga.ERR_UNSUPPORTED
    s = S(12210, 1369, 5, 1, 128)    # 16,776,540 tokens: largest accepted frame count here
    assert lib.bsga_num_blocks(ctypes.byref(s.c()), ctypes.byref(out)) == bsga.OK


def test_keep_count_rejects_bad_rho():
    out = ctypes.c_int32()
    for rho in (-0.1, 1.5, float("nan")):
        assert lib.bsga_keep_count(10, rho, ctypes.byref(out)) == bsga.ERR_INVALID_ARG


FAKE = 0x10000  # never dereferenced: validation fails before any launch


def test_validation_before_launch():
    shape = S(4, 256, 5, 4, 64)
    sh = ctypes.byref(shape.c())
    ws = bsga.workspace_bytes(shape, bsga.OP_LAYER)
    cap = bsga.csr_capacity(shape)
    # null and misaligned tensors
    assert lib.bsga_predict_mask(sh, None, FAKE, FAKE, None, None, None, FAKE, ws, None) == bsga.ERR_INVALID_ARG
    assert lib.bsga_predict_mask(sh, FAKE + 2, FAKE, FAKE, None, None, None, FAKE, ws, None) == bsga.ERR_MISALIGNED
    assert lib.bsga_predict_mask(sh, FAKE, FAKE, FAKE + 1, None, None, None, FAKE, ws, None) == bsga.ERR_MISALIGNED
    # the optional score output: aligned, and not the probabilities' own buffer
    assert lib.bsga_predict_mask(sh, FAKE, FAKE, FAKE, FAKE + 2, None, None, FAKE, ws, None) == bsga.ERR_MISALIGNED
    assert lib.bsga_predict_mask(sh, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, ws, None) == bsga.ERR_INVALID_ARG
    # workspace: missing, short, misaligned
    assert lib.bsga_predict_mask(sh, FAKE, FAKE, FAKE, None, None, None, None, ws, None) == bsga.ERR_WORKSPACE
    assert lib.bsga_predict_mask(sh, FAKE, FAKE, FAKE, None, None, None, FAKE, 16, None) == bsga.ERR_WORKSPACE
    assert lib.bsga_predict_mask(sh, FAKE, FAKE, FAKE, None, None, None, FAKE + 16, ws, None) == bsga.ERR_WORKSPACE
    # select: rho / tau / capacity
    for rho, tau in ((-0.5, 0.9), (1.01, 0.9), (float("nan"), 0.9), (0.5, float("nan"))):
        assert lib.bsga_select(sh, FAKE, None, rho, tau, FAKE, FAKE, cap, FAKE, ws, None) \
            == bsga.ERR_INVALID_ARG
    assert lib.bsga_select(sh, FAKE, None, 0.5, 0.9, FAKE, FAKE, cap - 1, FAKE, ws, None) \
        == bsga.ERR_INVALID_ARG
    rh = (ctypes.c_double * 4)(0.5, 0.5, 2.0, 0.5)
    assert lib.bsga_select(sh, FAKE, ctypes.cast(rh, ctypes.c_void_p), 0.5, 0.9, FAKE, FAKE, cap,
                           FAKE, ws, None) == bsga.ERR_INVALID_ARG
    # attention calls
    assert lib.bsga_sparse_attn(sh, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE + 8, FAKE, FAKE, ws, None) \
        == bsga.ERR_MISALIGNED
    assert lib.bsga_dense_attn(sh, FAKE, FAKE, None, FAKE, FAKE, FAKE, ws, None) == bsga.ERR_INVALID_ARG
    assert lib.bsga_special_dense(sh, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, None) == bsga.ERR_WORKSPACE
    assert lib.bsga_layer(sh, FAKE, FAKE, FAKE, None, 0.5, 0.9, FAKE, FAKE, FAKE, cap, FAKE, FAKE,
                          FAKE, ws - 1, None) == bsga.ERR_WORKSPACE
    # training mode: the float32 rows are required and 16-byte aligned
    assert lib.bsga_layer_train(sh, FAKE, FAKE, FAKE, None, 0.5, 0.9, FAKE, FAKE, FAKE, cap, FAKE,
                                FAKE, None, FAKE, ws, None) == bsga.ERR_INVALID_ARG
    assert lib.bsga_layer_train(sh, FAKE, FAKE, FAKE, None, 0.5, 0.9, FAKE, FAKE, FAKE, cap, FAKE,
                                FAKE, FAKE + 4, FAKE, ws, None) == bsga.ERR_MISALIGNED
    assert lib.bsga_layer_train(sh, FAKE, FAKE, FAKE, None, 0.5, 0.9, FAKE, FAKE, FAKE, cap, FAKE,
                                FAKE, FAKE, FAKE, ws - 1, None) == bsga.ERR_WORKSPACE
    wsb = bsga.workspace_bytes(shape, bsga.OP_BACKWARD)
    assert lib.bsga_attn_backward_o32(sh, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE,
                                      FAKE, FAKE, FAKE, wsb, None) == bsga.ERR_INVALID_ARG
    assert lib.bsga_attn_backward_o32(sh, FAKE, FAKE, FAKE, FAKE + 8, FAKE, FAKE, FAKE, FAKE, FAKE,
                                      FAKE, FAKE, FAKE, wsb, None) == bsga.ERR_MISALIGNED
    assert lib.bsga_attn_backward_o32(sh, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                      FAKE, FAKE, FAKE, wsb - 1, None) == bsga.ERR_WORKSPACE
    # the selection without a workspace: its row limit, then the usual checks
    # (all before any HIP call)
    over = S(1, 128 * 1025, 0, 64, 128)  # 64 heads x 1025 blocks > 65,536 rows
    assert bsga.num_blocks(over) * 64 > bsga.SELECT_STATIC_MAX_ROWS
    assert lib.bsga_select_static(ctypes.byref(over.c()), FAKE, None, 0.5, 0.9, FAKE, FAKE,
                                  1 << 40, None) == bsga.ERR_UNSUPPORTED
    assert lib.bsga_select_static(sh, FAKE, None, 1.5, 0.9, FAKE, FAKE, cap, None) \
        == bsga.ERR_INVALID_ARG
    assert lib.bsga_select_static(sh, FAKE + 2, None, 0.5, 0.9, FAKE, FAKE, cap, None) \
        == bsga.ERR_MISALIGNED
    assert lib.bsga_select_static(sh, FAKE, None, 0.5, 0.9, FAKE, FAKE, cap - 1, None) \
        == bsga.ERR_INVALID_ARG
    # selection beyond the sort's capacity
    big = S(1, 64 * 5000, 0, 1, 64)
    assert lib.bsga_select(ctypes.byref(big.c()), FAKE, None, 0.5, 0.9, FAKE, FAKE, 1 << 40, FAKE,
                           1 << 40, None) == bsga.ERR_UNSUPPORTED
