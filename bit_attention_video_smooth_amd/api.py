"""Torch-tensor conveniences over the C ABI: allocate outputs, call the
library, return tensors.  No arithmetic of the method happens here."""
from __future__ import annotations

import dataclasses

import torch

from . import _lib

BLK = 128


def nblocks(L: int) -> int:
    return (L + BLK - 1) // BLK


def _require(cond, msg):
    """Argument check that survives python -O (the C ABI cannot see tensor
    sizes, so a mis-sized buffer must be caught here)."""
    if not cond:
        raise ValueError(msg)


def _check_bf16_inputs(q, k, v):
    for name, t in (("q", q), ("k", k), ("v", v)):
        _require(t.dtype == torch.bfloat16, "%s must be bfloat16, got %s" % (name, t.dtype))
        _require(t.is_contiguous(), "%s must be contiguous" % name)
        _require(t.dim() == 4 and t.shape == q.shape,
                 "%s must be [B,H,L,d]%s, got %s" % (name, "" if name == "q" else " like q", tuple(t.shape)))
        _require(t.device == q.device, "%s is on %s, q on %s" % (name, t.device, q.device))


def _check_out(out, shape, device):
    _require(out.dtype in (torch.float32, torch.bfloat16), "out must be float32 or bfloat16, got %s" % out.dtype)
    _require(out.is_contiguous(), "out must be contiguous")
    _require(tuple(out.shape) == tuple(shape), "out must be %s, got %s" % (tuple(shape), tuple(out.shape)))
    _require(out.device == device, "out is on %s, the inputs on %s" % (out.device, device))


@dataclasses.dataclass
class Prepared:
    shape: tuple
    q8: torch.Tensor
    k8: torch.Tensor
    v8: torch.Tensor
    q_scale: torch.Tensor
    k_scale: torch.Tensor
    v_scale: torch.Tensor
    v_mean: torch.Tensor
    perm: torch.Tensor
    kmeans_obj: torch.Tensor
    v_format: int = 0  # 0: E4M3 residual; 1: E2M1 residual (v8 / v_scale hold packed codes / E8M0 bytes)

    def c(self) -> _lib.vc_prepared:
        return _lib.vc_prepared(*(t.data_ptr() for t in (
            self.q8, self.k8, self.v8, self.q_scale, self.k_scale, self.v_scale, self.v_mean,
            self.perm, self.kmeans_obj)))


def alloc_prepared(B, H, L, d, device="cuda") -> Prepared:
    nb = nblocks(L)
    Lp = nb * BLK
    u8 = dict(dtype=torch.uint8, device=device)
    f32 = dict(dtype=torch.float32, device=device)
    return Prepared((B, H, L, d),
                    torch.empty((B, H, Lp, d), **u8), torch.empty((B, H, Lp, d), **u8),
                    torch.empty((B, H, nb, d, BLK), **u8),
                    torch.empty((B, H, nb), **f32), torch.empty((B, H, nb), **f32),
                    torch.empty((B, H, nb, d), **f32), torch.empty((B, H, nb, d), **f32),
                    torch.empty((B, H, L), dtype=torch.int32, device=device),
                    torch.empty((B, H), dtype=torch.float64, device=device))


def workspace(B, H, L, d, *, kmeans_k=0, kmeans_iters=8, device="cuda") -> torch.Tensor:
    n = _lib.vsmooth_workspace_bytes(_lib.shape_of(B, H, L, d),
                                     _lib.make_params(kmeans_k, kmeans_iters))
    return torch.empty(max(n, 16), dtype=torch.uint8, device=device)


def prepare(q, k, v, *, perm_in=None, kmeans_k=0, kmeans_iters=8, seed=0, smooth_k=1,
            v_scale_mode=0, out: Prepared | None = None, ws: torch.Tensor | None = None,
            centroids_in: torch.Tensor | None = None, centroids_out: torch.Tensor | None = None,
            v_format=0, stream=None) -> Prepared:
    """vsmooth_prepare on bf16 [B,H,L,d] device tensors; with centroids_in
    and/or centroids_out (fp32 [B,H,k,d]) vsmooth_prepare_warm, whose k-means
    starts from centroids_in (None: the seeded init) and leaves its final
    centroids in centroids_out (may be the same tensor)."""
    _check_bf16_inputs(q, k, v)
    B, H, L, d = q.shape
    if perm_in is not None:
        _require(perm_in.dtype == torch.int32 and perm_in.is_contiguous() and tuple(perm_in.shape) == (B, H, L)
                 and perm_in.device == q.device, "perm_in must be contiguous int32 [B,H,L] on the inputs' device")
    warm = centroids_in is not None or centroids_out is not None
    if warm:
        if perm_in is not None:
            raise ValueError("centroids and perm_in exclude each other (a warm start runs k-means)")
        kk = kmeans_k if kmeans_k > 0 else nblocks(L)
        for t in (centroids_in, centroids_out):
            if t is not None:
                _require(t.dtype == torch.float32 and t.is_contiguous() and tuple(t.shape) == (B, H, kk, d)
                         and t.device == q.device, "centroids must be contiguous float32 [B,H,%d,%d]" % (kk, d))
    shape = _lib.shape_of(B, H, L, d)
    params = _lib.make_params(kmeans_k, kmeans_iters, seed, smooth_k, v_scale_mode, v_format)
    out = out if out is not None else alloc_prepared(B, H, L, d, q.device)
    out.v_format = v_format
    if ws is None:
        ws = workspace(B, H, L, d, kmeans_k=kmeans_k, kmeans_iters=kmeans_iters, device=q.device)
    if warm:
        _lib.vsmooth_prepare_warm(shape, params, q, k, v, centroids_in, centroids_out, out.c(), ws, ws.numel(),
                                  stream)
    else:
        _lib.vsmooth_prepare(shape, params, q, k, v, perm_in, out.c(), ws, ws.numel(), stream)
    return out


def _prob_cast(prep: Prepared, prob_cast):
    return (1 if prep.v_format == 1 else 0) if prob_cast is None else prob_cast


def attention(prep: Prepared, *, z_off=8, out_dtype=torch.float32, out=None, skip_lambda=0.0, prob_cast=None,
              stream=None):
    """vc_attention_fwd: O [B,H,L,d] in fp32 or bf16 (skip_lambda: the Skip
    Softmax threshold, 0 = off; prob_cast: 0 ExpCast-FP8, 1 exp-then-cast,
    default 0, or 1 for a 4-bit prepare, which needs it)."""
    B, H, L, d = prep.shape
    if out is None:
        out = torch.empty((B, H, L, d), dtype=out_dtype, device=prep.q8.device)
    _check_out(out, (B, H, L, d), prep.q8.device)
    od = 1 if out.dtype == torch.bfloat16 else 0
    params = _lib.vc_attn_params(z_off, od, skip_lambda, _prob_cast(prep, prob_cast), prep.v_format)
    _lib.vc_attention_fwd(_lib.shape_of(B, H, L, d), params, prep.c(), out, stream)
    return out


def attention_dump(prep: Prepared, bh: int, q_tile: int, *, z_off=8, skip_lambda=0.0, prob_cast=None,
                   stream=None):
    """vc_attention_fwd_dump: returns (O fp32, S [256, Lp] fp32, P [256, Lp] u8)."""
    B, H, L, d = prep.shape
    Lp = nblocks(L) * BLK
    dev = prep.q8.device
    out = torch.empty((B, H, L, d), dtype=torch.float32, device=dev)
    s = torch.zeros((256, Lp), dtype=torch.float32, device=dev)
    p = torch.zeros((256, Lp), dtype=torch.uint8, device=dev)
    params = _lib.vc_attn_params(z_off, 0, skip_lambda, _prob_cast(prep, prob_cast), prep.v_format)
    _lib.vc_attention_fwd_dump(_lib.shape_of(B, H, L, d), params, prep.c(), out, bh, q_tile, s, p, stream)
    return out, s, p


# ----------------------------------------------- SAGE-style baseline --

SAGE_QK = {"int8": _lib.VC_SAGE_QK_INT8, "fp8": _lib.VC_SAGE_QK_FP8}


@dataclasses.dataclass
class SagePrepared:
    shape: tuple
    qk_dtype: str
    smooth_k: int
    q8: torch.Tensor
    k8: torch.Tensor
    v8: torch.Tensor
    q_scale: torch.Tensor
    k_scale: torch.Tensor
    v_scale: torch.Tensor

    def c(self) -> _lib.vc_sage_prepared:
        return _lib.vc_sage_prepared(*(t.data_ptr() for t in (
            self.q8, self.k8, self.v8, self.q_scale, self.k_scale, self.v_scale)))

    def params(self) -> _lib.vc_sage_params:
        return _lib.make_sage_params(SAGE_QK[self.qk_dtype], self.smooth_k)


def sage_prepare(q, k, v, *, qk_dtype="int8", smooth_k=1, out: SagePrepared | None = None,
                 ws: torch.Tensor | None = None, stream=None) -> SagePrepared:
    """vc_sage_prepare on bf16 [B,H,L,d] device tensors (qk_dtype "int8" or
    "fp8"; q/k/v block sizes 1/16/1, V in FP8 E4M3)."""
    _check_bf16_inputs(q, k, v)
    B, H, L, d = q.shape
    if qk_dtype not in SAGE_QK:
        raise ValueError("qk_dtype must be 'int8' or 'fp8'")
    shape = _lib.shape_of(B, H, L, d)
    if out is None:
        nb = nblocks(L)
        Lp = nb * BLK
        u8 = dict(dtype=torch.uint8, device=q.device)
        f32 = dict(dtype=torch.float32, device=q.device)
        out = SagePrepared((B, H, L, d), qk_dtype, smooth_k,
                           torch.empty((B, H, Lp, d), **u8), torch.empty((B, H, Lp, d), **u8),
                           torch.empty((B, H, nb, d, BLK), **u8), torch.empty((B, H, Lp), **f32),
                           torch.empty((B, H, Lp // 16), **f32), torch.empty((B, H, d), **f32))
    else:
        out.qk_dtype, out.smooth_k = qk_dtype, smooth_k
    if ws is None:
        ws = torch.empty(max(_lib.vc_sage_workspace_bytes(shape), 16), dtype=torch.uint8, device=q.device)
    _lib.vc_sage_prepare(shape, out.params(), q, k, v, out.c(), ws, ws.numel(), stream)
    return out


def sage_attention(prep: SagePrepared, *, z_off=8, prob_cast=1, out_dtype=torch.float32, out=None, stream=None):
    """vc_sage_attention_fwd: O [B,H,L,d] (prob_cast 1: exp-then-cast bytes,
    the SageAttention line's FP8 P; 0: ExpCast)."""
    B, H, L, d = prep.shape
    if out is None:
        out = torch.empty((B, H, L, d), dtype=out_dtype, device=prep.q8.device)
    _check_out(out, (B, H, L, d), prep.q8.device)
    od = 1 if out.dtype == torch.bfloat16 else 0
    params = _lib.vc_attn_params(z_off, od, 0.0, prob_cast)
    _lib.vc_sage_attention_fwd(_lib.shape_of(B, H, L, d), prep.params(), params, prep.c(), out, stream)
    return out


def sage_attention_dump(prep: SagePrepared, bh: int, q_tile: int, *, z_off=8, prob_cast=1, stream=None):
    """vc_sage_attention_fwd_dump: (O fp32, S [256, Lp] fp32, P [256, Lp] u8)."""
    B, H, L, d = prep.shape
    Lp = nblocks(L) * BLK
    dev = prep.q8.device
    out = torch.empty((B, H, L, d), dtype=torch.float32, device=dev)
    s = torch.zeros((256, Lp), dtype=torch.float32, device=dev)
    p = torch.zeros((256, Lp), dtype=torch.uint8, device=dev)
    params = _lib.vc_attn_params(z_off, 0, 0.0, prob_cast)
    _lib.vc_sage_attention_fwd_dump(_lib.shape_of(B, H, L, d), prep.params(), params, prep.c(), out, bh, q_tile,
                                    s, p, stream)
    return out, s, p


def attention_bf16(q, k, v, *, out_dtype=torch.float32, out=None, stream=None):
    """vc_attention_fwd_bf16 on bf16 [B,H,L,d] device tensors."""
    _check_bf16_inputs(q, k, v)
    B, H, L, d = q.shape
    if out is None:
        out = torch.empty((B, H, L, d), dtype=out_dtype, device=q.device)
    _check_out(out, (B, H, L, d), q.device)
    od = 1 if out.dtype == torch.bfloat16 else 0
    _lib.vc_attention_fwd_bf16(_lib.shape_of(B, H, L, d), q, k, v, out, od, stream)
    return out


def expcast(S, c8, krow, stream=None):
    n = S.numel()
    out = torch.empty(S.shape, dtype=torch.uint8, device=S.device)
    _lib.vc_debug_expcast(S, c8, krow, n, out, stream)
    return out


def e4m3_encode(x, stream=None):
    out = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    _lib.vc_debug_e4m3_encode(x, x.numel(), out, stream)
    return out


def mfma_fp8(a, b, stream=None):
    n = a.shape[0]
    c = torch.empty((n, 16, 16), dtype=torch.float32, device=a.device)
    _lib.vc_debug_mfma_fp8(a, b, c, n, stream)
    return c


# Slot order of a 128-key block in the V residual layout (vc_attention.h):
# slot pos holds key kk with pos = 32*((kk%16)//4) + 4*(kk//16) + (kk%4).
def key_of_slot():
    import numpy as np
    pos = np.arange(BLK)
    return 16 * ((pos % 32) // 4) + 4 * (pos // 32) + (pos % 4)


def v4_codes_natural(prep: Prepared):
    """The E2M1 residual of a 4-bit prepare: (codes [B,H,nb,d,128] one code
    per byte in natural key order, E8M0 bytes [B,H,nb,d,4]).  The 4-bit
    layout keeps keys in slot order already (slot 2t in the low nibble of
    byte t), so this only unpacks the nibbles."""
    B, H, L, d = prep.shape
    nb = nblocks(L)
    packed = prep.v8.reshape(-1)[:B * H * nb * d * BLK // 2].view(B, H, nb, d, BLK // 2)
    codes = torch.stack([packed & 0xF, packed >> 4], dim=-1).reshape(B, H, nb, d, BLK)
    exps = prep.v_scale.view(torch.uint8).view(B, H, nb, d, 4)
    return codes, exps


def v_codes_natural(v8):
    """Reorder the V residual codes [..., 128 slots] into natural key order."""
    import numpy as np
    kos = key_of_slot()
    inv = np.empty(BLK, np.int64)
    inv[kos] = np.arange(BLK)
    if isinstance(v8, torch.Tensor):
        return v8[..., torch.as_tensor(inv, device=v8.device)]
    return v8[..., inv]
