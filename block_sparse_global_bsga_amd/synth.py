"""Seeded synthetic inputs shaped like one global-attention layer of a
VGGT-style multi-view transformer.

This module only *draws inputs*.  It holds none of the attention method's
arithmetic (no pooling, scores, softmax, selection or attention), so that both
the HIP path and the CPU oracle can consume the same bits without sharing any
computation.

Token layout (one batch, heads outermost): ``X[h][t][d]`` with ``t`` running
frame-major; every frame is ``special_per_frame`` special tokens (one camera
token followed by register tokens) and then its patch tokens in raster order.
The pages ("Block-Sparse Global Attention for Efficient Multi-View Geometry
Transformers", design point 3) say only that each frame gets one camera and
four register tokens; putting them first in the frame is the reading taken.

Workloads (the pages measure on public datasets with trained weights, neither
of which is available; these seeded generators stand in for them):

* correspondence heads: 256 scene points with latents ``z ~ N(0, I_64)`` (drawn
  per head); each frame's patches carry the labels ``p mod 256`` in a seeded
  per-frame order; patch ``Q = 3 z + N(0,1)`` and ``K = 3 z + N(0,1)``
  (independent noise) — this plants sparse cross-frame correspondences;
* position heads: ``Q, K = code(y, x) + N(0,1)`` with a 2-D sin/cos code
  (frequencies ``10000^(-i/16)``, i < 16; groups sin(y w), cos(y w),
  sin(x w), cos(x w));
* diffuse heads: ``Q, K ~ N(0,1)``;
* special-token Q, K and every V row: ``N(0,1)``;
* optional "sink" keys: a seeded 10 % of patch positions (shared by all heads)
  whose K rows are multiplied by 4.

Random streams: numpy PCG64 seeded with ``1000 + config index`` and drawn in a
fixed order, so every run and both sides see identical inputs.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional

import numpy as np

HEAD_DIM = 64
N_LATENT = 256
SPECIAL_PER_FRAME = 5
RHO_CHOICES = (0.5, 0.75, 0.9, 0.95)


@dataclasses.dataclass
class LayerConfig:
    name: str
    frames: int
    grid_h: int
    grid_w: int
    heads: int
    block: int
    rho: float
    tau: float
    special_per_frame: int = SPECIAL_PER_FRAME
    head_dim: int = HEAD_DIM
    position_head_frac: float = 0.0
    diffuse_head_frac: float = 0.0
    sink_frac: float = 0.0
    per_head_rho_mean: Optional[float] = None
    input_dtype: str = "bf16"
    seed: int = 1000

    @property
    def patches_per_frame(self) -> int:
        return self.grid_h * self.grid_w

    @property
    def tokens(self) -> int:
        return self.frames * (self.patches_per_frame + self.special_per_frame)

    @property
    def n_patch(self) -> int:
        return self.frames * self.patches_per_frame

    @property
    def n_special(self) -> int:
        return self.frames * self.special_per_frame


def _cfg(i: int, **kw) -> LayerConfig:
    return LayerConfig(seed=1000 + i, **kw)


# The five layer shapes: tiny instance, then VGGT-shaped global layers at
# 518x518 (37x37 patches of 14 px) or 294x518 (21x37 patches).
CONFIGS = {
    1: _cfg(1, name="tiny-4f-16x16-h4-b64", frames=4, grid_h=16, grid_w=16,
            heads=4, block=64, rho=0.5, tau=0.9, input_dtype="fp32"),
    2: _cfg(2, name="vggt-8f-518-h16-b64", frames=8, grid_h=37, grid_w=37,
            heads=16, block=64, rho=0.75, tau=0.9, position_head_frac=0.2),
    3: _cfg(3, name="vggt-32f-518-h16-b128", frames=32, grid_h=37, grid_w=37,
            heads=16, block=128, rho=0.75, tau=0.9, sink_frac=0.1),
    4: _cfg(4, name="vggt-100f-294x518-h16-b128", frames=100, grid_h=21,
            grid_w=37, heads=16, block=128, rho=0.85, tau=0.95),
    5: _cfg(5, name="vggt-200f-518-h16-b128-perhead", frames=200, grid_h=37,
            grid_w=37, heads=16, block=128, rho=0.85, tau=0.9,
            position_head_frac=0.25, diffuse_head_frac=0.5,
            per_head_rho_mean=0.85),
}


def fp32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest even); raw uint16."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + bias) >> 16).astype(np.uint16)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    """Exact widening of raw bfloat16 bits to float64."""
    u = b.astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    u = b.astype(np.uint32) << 16
    return u.view(np.float32)


def position_code(grid_h: int, grid_w: int, dim: int = HEAD_DIM) -> np.ndarray:
    """2-D sin/cos code of every (y, x) in raster order, shape [gh*gw, dim]."""
    nf = dim // 4
    w = 10000.0 ** (-np.arange(nf, dtype=np.float64) / nf)
    y, x = np.meshgrid(np.arange(grid_h), np.arange(grid_w), indexing="ij")
    y = y.reshape(-1, 1).astype(np.float64)
    x = x.reshape(-1, 1).astype(np.float64)
    code = np.concatenate([np.sin(y * w), np.cos(y * w), np.sin(x * w),
                           np.cos(x * w)], axis=1)
    return code.astype(np.float32)


def draw_per_head_rho(rng: np.random.Generator, heads: int, mean: float,
                      choices=RHO_CHOICES) -> np.ndarray:
    """i.i.d. draws from ``choices`` (in exact hundredths), redrawn until the
    heads' mean equals ``mean`` exactly."""
    hund = np.array([round(c * 100) for c in choices], dtype=np.int64)
    target = round(mean * 100) * heads
    for _ in range(1_000_000):
        pick = rng.integers(0, len(hund), size=heads)
        if int(hund[pick].sum()) == target:
            return hund[pick].astype(np.float64) / 100.0
    raise RuntimeError("per-head budget draw did not converge")


@dataclasses.dataclass
class LayerInputs:
    cfg: LayerConfig
    q: np.ndarray  # uint16 bf16 bits [H][N][64]
    k: np.ndarray
    v: np.ndarray
    head_types: List[str]
    rho_per_head: Optional[np.ndarray]
    labels: np.ndarray  # [F][P] scene-point label of each patch
    sinks: Optional[np.ndarray]  # patch indices whose K rows were scaled

    @property
    def shape(self):
        c = self.cfg
        return dict(frames=c.frames, patches_per_frame=c.patches_per_frame,
                    special_per_frame=c.special_per_frame, heads=c.heads,
                    head_dim=c.head_dim, block=c.block)


def _head_types(rng: np.random.Generator, cfg: LayerConfig) -> List[str]:
    H = cfg.heads
    n_pos = int(round(cfg.position_head_frac * H))
    n_dif = int(round(cfg.diffuse_head_frac * H))
    types = ["corr"] * H
    if n_pos or n_dif:
        order = rng.permutation(H)
        for h in order[:n_pos]:
            types[h] = "pos"
        for h in order[n_pos:n_pos + n_dif]:
            types[h] = "diffuse"
    return types


def generate(cfg: LayerConfig, seed: Optional[int] = None,
             keep_fp32: bool = False) -> LayerInputs:
    """Draw Q, K, V for one layer.  Memory is bounded by one head at a time in
    float32.  The result holds bf16 bits; with ``keep_fp32`` the float32
    originals (before rounding) are attached as ``q32``/``k32``/``v32``."""
    rng = np.random.Generator(np.random.PCG64(cfg.seed if seed is None else seed))
    F, P, S, H, D = (cfg.frames, cfg.patches_per_frame, cfg.special_per_frame,
                     cfg.heads, cfg.head_dim)
    N = cfg.tokens
    # 1. label of every patch: p mod 256 in a seeded per-frame order
    base = np.arange(P) % N_LATENT
    labels = np.stack([base[rng.permutation(P)] for _ in range(F)])
    # 2. head types, per-head budgets, sinks
    types = _head_types(rng, cfg)
    rho_h = None
    if cfg.per_head_rho_mean is not None:
        rho_h = draw_per_head_rho(rng, H, cfg.per_head_rho_mean)
    sinks = None
    if cfg.sink_frac > 0:
        n_sink = int(round(cfg.sink_frac * F * P))
        sinks = np.sort(rng.choice(F * P, size=n_sink, replace=False))
    code = position_code(cfg.grid_h, cfg.grid_w, D)
    # token index of every patch and special row
    tok = np.arange(N).reshape(F, P + S)
    spec_tok = tok[:, :S].reshape(-1)
    patch_tok = tok[:, S:].reshape(-1)
    q = np.empty((H, N, D), dtype=np.uint16)
    k = np.empty((H, N, D), dtype=np.uint16)
    v = np.empty((H, N, D), dtype=np.uint16)
    f32 = [np.empty((H, N, D), dtype=np.float32) for _ in range(3)] if keep_fp32 else None
    lab = labels.reshape(-1)
    for h in range(H):
        qh = np.empty((N, D), dtype=np.float32)
        kh = np.empty((N, D), dtype=np.float32)
        if types[h] == "corr":
            z = rng.standard_normal((N_LATENT, D), dtype=np.float32)
            qh[patch_tok] = 3.0 * z[lab] + rng.standard_normal((F * P, D), dtype=np.float32)
            kh[patch_tok] = 3.0 * z[lab] + rng.standard_normal((F * P, D), dtype=np.float32)
        elif types[h] == "pos":
            c = np.tile(code, (F, 1))
            qh[patch_tok] = c + rng.standard_normal((F * P, D), dtype=np.float32)
            kh[patch_tok] = c + rng.standard_normal((F * P, D), dtype=np.float32)
        else:
            qh[patch_tok] = rng.standard_normal((F * P, D), dtype=np.float32)
            kh[patch_tok] = rng.standard_normal((F * P, D), dtype=np.float32)
        qh[spec_tok] = rng.standard_normal((F * S, D), dtype=np.float32)
        kh[spec_tok] = rng.standard_normal((F * S, D), dtype=np.float32)
        if sinks is not None:
            kh[patch_tok[sinks]] *= 4.0
        vh = rng.standard_normal((N, D), dtype=np.float32)
        q[h] = fp32_to_bf16_bits(qh)
        k[h] = fp32_to_bf16_bits(kh)
        v[h] = fp32_to_bf16_bits(vh)
        if f32 is not None:
            f32[0][h], f32[1][h], f32[2][h] = qh, kh, vh
    out = LayerInputs(cfg=cfg, q=q, k=k, v=v, head_types=types,
                      rho_per_head=rho_h, labels=labels, sinks=sinks)
    if f32 is not None:
        out.q32, out.k32, out.v32 = f32
    return out


def random_layer(frames: int, grid_h: int, grid_w: int, heads: int, block: int,
                 seed: int, special_per_frame: int = SPECIAL_PER_FRAME,
                 kind: str = "diffuse", rho: float = 0.5,
                 tau: float = 0.9) -> LayerInputs:
    """Small generic instance for edge cases; ``kind`` is ``diffuse`` (all
    N(0,1)), ``corr`` (planted correspondences) or ``pos`` (position code)."""
    frac = dict(diffuse=(0.0, 1.0), corr=(0.0, 0.0), pos=(1.0, 0.0))[kind]
    cfg = LayerConfig(name=f"rand-{kind}-{frames}f-{grid_h}x{grid_w}-h{heads}-b{block}",
                      frames=frames, grid_h=grid_h, grid_w=grid_w, heads=heads,
                      block=block, rho=rho, tau=tau,
                      special_per_frame=special_per_frame, seed=seed,
                      position_head_frac=frac[0], diffuse_head_frac=frac[1])
    return generate(cfg)
