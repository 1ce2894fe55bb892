"""Element offsets beyond 2^31: B*H*L*d = 72 * 262,067 * 128 = 2.4e9 elements
(the ABI accepts up to 2^40), so every index into Q, K, V, the codes and the
output of the last heads needs 64-bit arithmetic.  Inputs are made on the
GPU (seeded), the permutations are random, and the last head and a middle
head are checked against the oracle: Q/K/V codes, scales and means
bit-exact; the first and the ragged last query tile of the last head: bytes
bit-exact given the kernel's scores, the given-S bar (rel-L2 1e-4), and end
to end the output bar or its excess accounted for by one-code byte flips of
the matrix core's inexact score sums (parity_util).  About 40 GB of device
memory."""
import os
import sys

import numpy as np
import pytest
import torch

import oracle

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
from parity_util import check_explained, explain_vsmooth_rows  # noqa: E402

pytestmark = pytest.mark.gpu

B, H, L, D = 1, 72, 262067, 128


@pytest.fixture(scope="module")
def api():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    from bit_attention_video_smooth_amd import api as a
    a._lib.load()
    return a


def _bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def test_offsets_beyond_2_31_elements(api):
    assert B * H * L * D > 2 ** 31
    g = torch.Generator(device="cuda").manual_seed(11)
    qkv = []
    for _ in range(3):
        t = torch.empty((B, H, L, D), dtype=torch.bfloat16, device="cuda")
        for h in range(H):  # one head at a time keeps the fp32 temporaries small
            t[0, h] = torch.randn((L, D), generator=g, device="cuda").to(torch.bfloat16)
        qkv.append(t)
    q, k, v = qkv
    k[0] += 0.5  # a K channel offset, so that K smoothing does something
    perm = torch.stack([torch.randperm(L, generator=g, device="cuda") for _ in range(H)])[None].to(torch.int32)
    P = api.prepare(q, k, v, perm_in=perm.contiguous())
    out = api.attention(P)
    torch.cuda.synchronize()
    for h in (H // 2, H - 1):
        qh, kh, vh = _bits(q[0, h]), _bits(k[0, h]), _bits(v[0, h])
        ph = perm[0, h].cpu().numpy()
        o = oracle.prepare_head(qh, kh, vh, ph)
        got = {"q8": P.q8[0, h], "k8": P.k8[0, h], "v8": api.v_codes_natural(P.v8[0, h]), "q_scale": P.q_scale[0, h],
               "k_scale": P.k_scale[0, h], "v_scale": P.v_scale[0, h], "v_mean": P.v_mean[0, h]}
        for n, t in got.items():
            assert np.array_equal(t.cpu().numpy().view(np.uint8), o[n].view(np.uint8)), (h, n)
        if h != H - 1:
            continue
        nqt = (L + 255) // 256
        for qt in (0, nqt - 1):
            r0, r1 = 256 * qt, min(L, 256 * qt + 256)
            _, S, Pb = api.attention_dump(P, h, qt)
            S, Pb = S.cpu().numpy()[:r1 - r0], Pb.cpu().numpy()[:r1 - r0]
            got_rows = out[0, h, r0:r1].cpu().numpy()
            ref, refS, delta, flips = explain_vsmooth_rows(o, L, (r0, r1), S, Pb)
            check_explained("2.4e9 elements, head %d tile %d" % (h, qt), got_rows, ref, refS, delta, flips)
