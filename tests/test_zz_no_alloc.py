"""vsmooth_prepare_noalloc, the prepare entry point for callers that cannot
allocate device memory, against vsmooth_prepare with a caller workspace:
two calls in a row through the C ABI, the second on a smaller problem (so
the fixed scratch holds the first call's leftovers), every output bit for
bit equal.  k-means runs in both calls, so the scratch carries centroids,
assignments and sort counts; a third call with a supplied permutation uses
only the K-mean part of it."""
import numpy as np
import pytest
import torch

from bit_attention_video_smooth_amd import _lib, api, synth

pytestmark = pytest.mark.gpu


FIELDS = ("q8", "k8", "v8", "q_scale", "k_scale", "v_scale", "v_mean", "perm", "kmeans_obj")


def _tensors(P):
    return [getattr(P, f) for f in FIELDS]


def dev_bf16(u16):
    return torch.from_numpy(np.ascontiguousarray(u16)).view(torch.bfloat16).cuda()


def _prep_pair(cfg, seed, perm_in=None, kmeans_iters=8):
    q, k, v = (dev_bf16(a) for a in synth.make_inputs(cfg, seed))
    B, H, L, d = q.shape
    shape = _lib.shape_of(B, H, L, d)
    params = _lib.make_params(kmeans_iters=kmeans_iters, seed=seed)
    ref = api.alloc_prepared(B, H, L, d)
    got = api.alloc_prepared(B, H, L, d)
    # the outputs start with different garbage so that an unwritten byte shows
    for t in _tensors(got):
        t.fill_(0x5A if t.dtype == torch.uint8 else 7)
    ws = torch.empty(max(_lib.vsmooth_workspace_bytes(shape, params), 16), dtype=torch.uint8, device="cuda")
    _lib.vsmooth_prepare(shape, params, q, k, v, perm_in, ref.c(), ws, ws.numel())
    _lib.vsmooth_prepare_noalloc(shape, params, q, k, v, perm_in, got.c())
    torch.cuda.synchronize()
    return ref, got


def _same(ref, got):
    for f, a, b in zip(FIELDS, _tensors(ref), _tensors(got)):
        if a.dtype == torch.float64:
            assert torch.equal(a.isnan(), b.isnan()), f
            assert torch.equal(torch.nan_to_num(a), torch.nan_to_num(b))
        else:
            assert torch.equal(a, b), f


def test_noalloc_prepare_equals_workspace_prepare():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    big = synth.custom(1, 4, 5000, 128)
    small = synth.custom(1, 2, 1024, 64, grid=(4, 16, 16))
    print("noalloc: B=1 H=4 L=5000 d=128, k-means", flush=True)
    ref, got = _prep_pair(big, 11)
    _same(ref, got)
    print("noalloc: B=1 H=2 L=1024 d=64, k-means (second, smaller call)", flush=True)
    ref2, got2 = _prep_pair(small, 12)
    _same(ref2, got2)
    print("noalloc: B=1 H=2 L=1024 d=64, permutation supplied", flush=True)
    ref3, got3 = _prep_pair(small, 13, perm_in=ref2.perm)
    _same(ref3, got3)
    # the attention over the no-alloc prepare equals the one over the other
    o_ref = api.attention(ref2)
    o_got = api.attention(got2)
    torch.cuda.synchronize()
    assert torch.equal(o_ref, o_got)
