"""Token-ordering ablation of V-Smooth (measurement, not the attention path).

The MarkTechPost abstract (yifor post on VC-Attention) compares three ways of
cutting the value tokens into blocks by the share of block energy the block
mean removes: sequence order (8% over 100 Wan2.2 heads), DeltaQuant's static
cube (12%) and k-means sorted (36%).  This module builds the static-cube
permutation from the latent grid and measures, on the library's own prepare
outputs, the block energy the means remove and the relative error of the
reconstructed values mean + scale * E4M3(code).  The statistics are plain
reductions over device tensors; every code, scale and mean comes from the
library's kernels.
"""
from __future__ import annotations

import numpy as np
import torch

from . import api


def cube_permutation(grid, cube=(2, 8, 8)) -> np.ndarray:
    """Static-cube order of a (T, Hg, W) latent grid flattened as
    j = (t*Hg + h)*W + w: tokens sorted by cube (t//ct, h//ch, w//cw), in
    sequence order inside a cube.  Returns int32 [T*Hg*W]."""
    T, Hg, W = grid
    ct, ch, cw = cube
    t, h, w = np.meshgrid(np.arange(T), np.arange(Hg), np.arange(W), indexing="ij")
    order = np.lexsort(((w // cw).ravel(), (h // ch).ravel(), (t // ct).ravel()))  # stable
    return order.astype(np.int32)


@torch.no_grad()
def value_stats(P: api.Prepared, v: torch.Tensor) -> dict:
    """Per (batch, head): `energy_removed` = 1 - sum |v - mean_block|^2 /
    sum |v|^2 over the permuted blocks, and `v_rel_err` = |v_hat - v| / |v|
    with v_hat = mean + scale * decode(code), both from P.  v: bf16
    [B,H,L,d] device tensor.  Returns numpy float64 arrays [B,H]."""
    B, H, L, d = P.shape
    nb = api.nblocks(L)
    energy = np.empty((B, H))
    err = np.empty((B, H))
    codes = api.v_codes_natural(P.v8)  # [B,H,nb,d,128], natural key order within a block
    for b in range(B):
        for h in range(H):
            x = v[b, h].float()[P.perm[b, h].long()].double()               # [L,d], permuted
            xp = torch.zeros((nb * api.BLK, d), dtype=torch.float64, device=x.device)
            xp[:L] = x
            xb = xp.view(nb, api.BLK, d)
            n = torch.full((nb, 1, 1), float(api.BLK), dtype=torch.float64, device=x.device)
            n[-1] = L - (nb - 1) * api.BLK
            valid = (torch.arange(api.BLK, device=x.device)[None, :, None] < n).double()
            mu = P.v_mean[b, h].double()[:, None, :]                           # [nb,1,d]
            tot = (x * x).sum()
            resid = (((xb - mu) * valid) ** 2).sum()
            dec = codes[b, h].view(torch.float8_e4m3fn).float().double().transpose(1, 2)  # [nb,128,d]
            xhat = mu + P.v_scale[b, h].double()[:, None, :] * dec
            e = (((xhat - xb) * valid) ** 2).sum()
            energy[b, h] = float(1.0 - resid / tot)
            err[b, h] = float(torch.sqrt(e / tot))
    return {"energy_removed": energy, "v_rel_err": err}


@torch.no_grad()
def sage_value_stats(P: api.SagePrepared, v: torch.Tensor) -> dict:
    """Relative error |v_hat - v| / |v| per (batch, head) of the SAGE-style V
    codes, v_hat = s_c * decode(code) with one scale per channel and no
    block mean (TensorRT-LLM blog, "Quantized Attention", v block size 1).
    Returns numpy float64 [B,H]."""
    B, H, L, d = P.shape
    codes = api.v_codes_natural(P.v8)  # [B,H,nb,d,128]
    err = np.empty((B, H))
    for b in range(B):
        for h in range(H):
            x = v[b, h].double()                                              # [L,d]
            dec = codes[b, h].view(torch.float8_e4m3fn).float().double()      # [nb,d,128]
            dec = dec.transpose(1, 2).reshape(-1, d)[:L]                       # [L,d]
            xhat = P.v_scale[b, h].double()[None, :] * dec
            err[b, h] = float(torch.sqrt(((xhat - x) ** 2).sum() / (x * x).sum()))
    return {"v_rel_err": err}


@torch.no_grad()
def fp4_value_stats(P: api.Prepared, v: torch.Tensor) -> dict:
    """Relative error |v_hat - v| / |v| per (batch, head) of a 4-bit prepare:
    v_hat = mean_b + 2^e * E2M1(code), one power-of-two scale per (block,
    channel, key group).  Returns numpy float64 [B,H]."""
    B, H, L, d = P.shape
    nb = api.nblocks(L)
    codes, exps = api.v4_codes_natural(P)                   # [B,H,nb,d,128], [B,H,nb,d,4]
    table = torch.tensor([0, 0.5, 1, 1.5, 2, 3, 4, 6, -0.0, -0.5, -1, -1.5, -2, -3, -4, -6],
                         dtype=torch.float64, device=v.device)
    group = torch.arange(api.BLK, device=v.device) // 32      # key group of each in-block key
    err = np.empty((B, H))
    for b in range(B):
        for h in range(H):
            x = v[b, h].float()[P.perm[b, h].long()].double()                  # permuted rows [L,d]
            sc = torch.ldexp(torch.ones((), dtype=torch.float64, device=v.device),
                             exps[b, h].long()[..., group] - 127)               # [nb,d,128]
            xhat = P.v_mean[b, h].double()[:, :, None] + table[codes[b, h].long()] * sc
            xhat = xhat.transpose(1, 2).reshape(-1, d)[:L]
            err[b, h] = float(torch.sqrt(((xhat - x) ** 2).sum() / (x * x).sum()))
    return {"v_rel_err": err}
