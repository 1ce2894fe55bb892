"""Seeded synthetic video-token inputs (Q, K, V in bf16) for VC-Attention.

This module only draws inputs; it holds none of the method's arithmetic and
is the one piece shared by the GPU path's callers and the oracle's tests.

The real workloads of the pages (Wan2.2, MiniMax-H3 activations, the 100
Wan2.2 heads) are not available, so seeded tensors of the same shapes and of
the structure the pages describe stand in for them:

* tokens are a flattened (t, h, w) latent grid, index j = (t*Hg + h)*W + w;
* Q ~ N(0, 1); K = N(0, 1) + a per-(head, channel) offset ~ N(0, 0.5^2);
* V is a smooth spatio-temporal field (a sum of 8 random low-frequency
  sinusoids over (t/T, h/Hg, w/W), amplitudes ~ N(0, 1/8)) plus
  0.3 * N(0, 1) noise, with a few outlier tokens scaled up in a few
  channels that change from head to head, the outlier structure the
  MarkTechPost abstract on VC-Attention describes (a handful of tokens,
  with no channel pattern that holds across heads);
* the classifier-free-guidance pair (B = 2) shares the V field, noise and
  outliers, plus an independent N(0, 0.1^2) perturbation per batch entry;
* everything is rounded to bf16 (round to nearest even) last.
"""
from __future__ import annotations

import dataclasses
import math
from concurrent.futures import ThreadPoolExecutor

import numpy as np


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    B: int
    H: int
    d: int
    grid: tuple  # (T, Hg, W)
    outlier_frac: float
    outlier_factor: float
    outlier_ch: int
    cfg_pair: bool = False

    @property
    def L(self) -> int:
        return self.grid[0] * self.grid[1] * self.grid[2]

    @property
    def attn_flop(self) -> float:
        return 4.0 * self.B * self.H * float(self.L) ** 2 * self.d


# The five workloads: a tiny parity case, a mid-size case, the Wan2.2 720p
# shape (81 frames at 1280x720 -> 21x45x80 latent tokens), a long stress case
# (243 frames at 1344x768 under 4x temporal / 16x spatial compression, an
# assumed grid) and a CFG pair with small heads and heavier outliers.
CONFIGS = [
    Config("tiny", 1, 2, 64, (4, 16, 16), 0.01, 20.0, 4),
    Config("mid", 1, 40, 128, (21, 30, 52), 0.005, 30.0, 4),
    Config("wan720p", 1, 40, 128, (21, 45, 80), 0.005, 30.0, 4),
    Config("long", 1, 24, 128, (61, 48, 84), 0.005, 30.0, 4),
    Config("cfg", 2, 24, 64, (13, 30, 45), 0.02, 50.0, 8, cfg_pair=True),
]


def custom(B, H, L, d, grid=None, outlier_frac=0.01, outlier_factor=20.0, outlier_ch=4,
           cfg_pair=False, name="custom") -> Config:
    """An ad-hoc shape (e.g. a ragged L for edge cases); grid defaults to a
    one-row (1, 1, L) layout."""
    if grid is None:
        grid = (1, 1, L)
    assert grid[0] * grid[1] * grid[2] == L
    return Config(name, B, H, d, tuple(grid), outlier_frac, outlier_factor,
                  min(outlier_ch, d), cfg_pair)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest even."""
    u = np.ascontiguousarray(x, np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def _rng(seed, *key):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), *key])))


def _value_base(cfg: Config, seed: int, h: int) -> np.ndarray:
    """Shared part of V for head h (field + noise + outliers), float32 [L, d]."""
    T, Hg, W = cfg.grid
    L, d = cfg.L, cfg.d
    r = _rng(seed, 7, h)
    freq = r.uniform(0.0, 2.0, size=(8, 3))
    phase = r.uniform(0.0, 2.0 * math.pi, size=(8, d))
    amp = r.normal(0.0, math.sqrt(1.0 / 8.0), size=(8, d))
    t = np.arange(T, dtype=np.float64)[:, None, None] / T
    hh = np.arange(Hg, dtype=np.float64)[None, :, None] / Hg
    w = np.arange(W, dtype=np.float64)[None, None, :] / W
    theta = np.empty((8, L), np.float64)
    for s in range(8):
        theta[s] = (2.0 * math.pi * (freq[s, 0] * t + freq[s, 1] * hh + freq[s, 2] * w)).reshape(L)
    # sum_s a sin(theta + phi) = [sin theta, cos theta] @ [a cos phi; a sin phi]
    basis = np.concatenate([np.sin(theta), np.cos(theta)], axis=0).T  # [L, 16]
    coef = np.concatenate([amp * np.cos(phase), amp * np.sin(phase)], axis=0)  # [16, d]
    v = (basis @ coef).astype(np.float32)
    v += np.float32(0.3) * r.standard_normal((L, d), dtype=np.float32)
    n_tok = int(round(cfg.outlier_frac * L))
    if n_tok > 0:
        toks = r.choice(L, size=n_tok, replace=False)
        chans = r.choice(d, size=cfg.outlier_ch, replace=False)
        v[np.ix_(toks, chans)] *= np.float32(cfg.outlier_factor)
    return v


def _head(cfg: Config, seed: int, b: int, h: int, vbase):
    L, d = cfg.L, cfg.d
    r = _rng(seed, 1, b, h)
    q = r.standard_normal((L, d), dtype=np.float32)
    koff = r.normal(0.0, 0.5, size=(1, d)).astype(np.float32)
    k = r.standard_normal((L, d), dtype=np.float32) + koff
    v = vbase
    if cfg.cfg_pair:
        v = vbase + np.float32(0.1) * r.standard_normal((L, d), dtype=np.float32)
    return f32_to_bf16_bits(q), f32_to_bf16_bits(k), f32_to_bf16_bits(v)


def make_inputs(cfg: Config, seed: int, threads: int = 8):
    """Returns (q, k, v) as bf16 bit patterns, numpy uint16 [B, H, L, d]."""
    B, H, L, d = cfg.B, cfg.H, cfg.L, cfg.d
    q = np.empty((B, H, L, d), np.uint16)
    k = np.empty_like(q)
    v = np.empty_like(q)

    def work(h):
        vb = _value_base(cfg, seed, h)
        for b in range(B):
            q[b, h], k[b, h], v[b, h] = _head(cfg, seed, b, h, vb)

    with ThreadPoolExecutor(max(1, threads)) as ex:
        list(ex.map(work, range(H)))
    return q, k, v


def random_perms(B: int, H: int, L: int, seed: int) -> np.ndarray:
    """Seeded uniformly random token permutations, int32 [B, H, L]; a stress
    input for the joint K/V permutation (every block mixes unrelated tokens)."""
    out = np.empty((B, H, L), np.int32)
    for b in range(B):
        for h in range(H):
            out[b, h] = _rng(seed, 3, b, h).permutation(L).astype(np.int32)
    return out


def identity_perms(B: int, H: int, L: int) -> np.ndarray:
    return np.broadcast_to(np.arange(L, dtype=np.int32), (B, H, L)).copy()
