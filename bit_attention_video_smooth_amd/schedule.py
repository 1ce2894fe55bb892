"""Grouping schedule over the denoising steps, and a per-layer session that
reuses the permutation between groupings.

The MarkTechPost abstract (quoted in the yifor post on VC-Attention) and its
Chinese summary state the amortisation: grouping (the k-means that fixes the
token permutation) runs only during the first quarter of the denoising
steps, and a permutation is reused across 4 adjacent steps; the block means,
scales and codes are recomputed every step from that step's Q, K, V.

Reading taken here: with N steps, grouping runs at step s when
s < ceil(group_frac * N) and s is a multiple of `reuse`; every other step
takes the permutation of the latest grouping (so after the first quarter the
permutation is frozen).  Each attention layer keeps its own permutation.

Optionally (warm_start=True) each grouping after the first starts k-means
from the centroids the previous grouping ended with, instead of the seeded
init: the clusters of adjacent denoising steps are close, so the Lloyd
rounds start near their fixed point.

Host logic only: every step still runs the library's prepare (with or
without k-means) and attention kernels.
"""
from __future__ import annotations

import dataclasses
import math

import torch

from . import api


@dataclasses.dataclass(frozen=True)
class GroupingSchedule:
    num_steps: int
    group_frac: float = 0.25
    reuse: int = 4

    def __post_init__(self):
        if self.num_steps < 1 or self.reuse < 1 or not (0.0 <= self.group_frac <= 1.0):
            raise ValueError("num_steps >= 1, reuse >= 1 and group_frac in [0, 1] required")

    @property
    def grouping_window(self) -> int:
        """Steps [0, window) may regroup; at least step 0 always groups."""
        return max(1, math.ceil(self.group_frac * self.num_steps))

    def regroup(self, step: int) -> bool:
        if not (0 <= step < self.num_steps):
            raise ValueError("step %d outside [0, %d)" % (step, self.num_steps))
        return step < self.grouping_window and step % self.reuse == 0

    def grouping_steps(self) -> list[int]:
        return [s for s in range(self.num_steps) if self.regroup(s)]

    def amortised(self, ms_grouping_prepare: float, ms_reuse_prepare: float) -> float:
        """Mean prepare time per step given the two measured prepare costs."""
        n = len(self.grouping_steps())
        return (n * ms_grouping_prepare + (self.num_steps - n) * ms_reuse_prepare) / self.num_steps


class VCAttentionLayer:
    """One attention layer's state across the denoising steps: the prepared
    buffers, the prepare workspace and the current permutation (in
    `prepared.perm`).  `forward` runs one step: prepare (with k-means on a
    grouping step, else with the layer's permutation) and attention.  With
    warm_start the layer also keeps the k-means centroids of its latest
    grouping and starts the next grouping from them."""

    def __init__(self, B, H, L, d, schedule: GroupingSchedule, *, seed=0, kmeans_iters=8, v_scale_mode=0,
                 z_off=8, skip_lambda=0.0, warm_start=False, device="cuda"):
        self.shape = (B, H, L, d)
        self.schedule = schedule
        self.seed, self.kmeans_iters, self.v_scale_mode = seed, kmeans_iters, v_scale_mode
        self.z_off, self.skip_lambda = z_off, skip_lambda
        self.prepared = api.alloc_prepared(B, H, L, d, device)
        self.ws = api.workspace(B, H, L, d, kmeans_iters=kmeans_iters, device=device)
        self.out = torch.empty((B, H, L, d), dtype=torch.float32, device=device)
        self.grouped_at = None  # step of the latest grouping
        self.warm_start = warm_start
        self.centroids = (torch.empty((B, H, api.nblocks(L), d), dtype=torch.float32, device=device)
                          if warm_start else None)

    def forward(self, q, k, v, step: int, stream=None) -> torch.Tensor:
        if tuple(q.shape) != self.shape:
            raise ValueError("shape %s, layer built for %s" % (tuple(q.shape), self.shape))
        regroup = self.schedule.regroup(step) or self.grouped_at is None
        common = dict(kmeans_iters=self.kmeans_iters, seed=self.seed, v_scale_mode=self.v_scale_mode,
                      out=self.prepared, ws=self.ws, stream=stream)
        if regroup and self.warm_start:
            api.prepare(q, k, v, centroids_in=None if self.grouped_at is None else self.centroids,
                        centroids_out=self.centroids, **common)
        else:
            api.prepare(q, k, v, perm_in=None if regroup else self.prepared.perm, **common)
        if regroup:
            self.grouped_at = step
        return api.attention(self.prepared, z_off=self.z_off, out=self.out, skip_lambda=self.skip_lambda,
                             stream=stream)
