"""GPU parity over seeded random shapes (B, H, L, d and the permutation all
drawn; L includes values next to block boundaries), through the C ABI.
Per case: Q/K/V codes, scales and means bit-exact against the oracle, and,
given the kernel's own scores, the output within the given-S bar (rel-L2
1e-4, max-abs 1e-3 of max).  End to end, against the oracle's exactly
rounded scores, every case as in test_gpu_parity (the output bar, or the
excess over it accounted for by one-code byte flips of the matrix core's
inexact score sums), and the median over the cases within the output bar."""
import os
import sys

import numpy as np
import pytest
import torch

import oracle
from bit_attention_video_smooth_amd import synth

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
from parity_util import GIVEN_S_MAXABS, GIVEN_S_REL, REL_L2, rel_l2  # noqa: E402
from test_gpu_parity import _explain, _kernel_scores, _oracle_out, dev_bf16  # noqa: E402

pytestmark = pytest.mark.gpu


def _shapes(n=10, seed=2026):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        d = int(rng.choice([64, 128]))
        B, H = int(rng.integers(1, 3)), int(rng.integers(1, 4))
        if i % 3 == 0:
            L = int(128 * rng.integers(1, 20) + rng.choice([-1, 0, 1]))  # next to a block boundary
        else:
            L = int(rng.integers(1, 3000))
        L = max(L, 1)
        out.append((B, H, L, d, int(rng.integers(1 << 30))))
    out.append((1, 1, 5000, 128, 7))
    return out


SHAPES = _shapes()


@pytest.fixture(scope="module")
def api():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    from bit_attention_video_smooth_amd import api as a
    a._lib.load()
    return a


def test_random_shapes_match_oracle(api):
    ends = []
    for B, H, L, d, seed in SHAPES:
        q, k, v = synth.make_inputs(synth.custom(B, H, L, d), seed % 100000)
        perm = synth.random_perms(B, H, L, seed % 1000)
        P = api.prepare(dev_bf16(q), dev_bf16(k), dev_bf16(v), perm_in=torch.from_numpy(perm).cuda())
        g = {n: getattr(P, n).cpu().numpy() for n in ("q8", "k8", "q_scale", "k_scale", "v_scale", "v_mean")}
        g["v8"] = api.v_codes_natural(P.v8).cpu().numpy()
        for b in range(B):
            for h in range(H):
                o = oracle.prepare_head(q[b, h], k[b, h], v[b, h], perm[b, h])
                for n in ("q8", "k8", "v8", "q_scale", "k_scale", "v_scale", "v_mean"):
                    assert np.array_equal(g[n][b, h].view(np.uint8), o[n].view(np.uint8)), ((B, H, L, d), n)
        out = api.attention(P).cpu().numpy()
        r, _, _ = _explain("random shape", api, P, q, k, v, perm, out)
        ends.append(r)
    ends = np.array(ends)
    print("end-to-end rel-L2 over %d shapes: median %.3g max %.3g" % (len(ends), np.median(ends), ends.max()))
    assert np.median(ends) <= REL_L2


@pytest.mark.parametrize("qk", ["int8", "fp8"])
def test_random_shapes_sage_match_oracle(api, qk):
    """The SAGE-style baseline over the same shapes: codes and scales
    bit-exact; per case the given-S bar and the end-to-end check of
    test_gpu_sage (INT8: the output bar itself); the median within the
    output bar."""
    import test_gpu_sage as ts
    ends = []
    for B, H, L, d, seed in SHAPES[:6]:
        q, k, v = synth.make_inputs(synth.custom(B, H, L, d), seed % 100000)
        P = api.sage_prepare(dev_bf16(q), dev_bf16(k), dev_bf16(v), qk_dtype=qk)
        g = {n: getattr(P, n).cpu().numpy() for n in ("q8", "k8", "q_scale", "k_scale", "v_scale")}
        g["v8"] = api.v_codes_natural(P.v8).cpu().numpy()
        for b in range(B):
            for h in range(H):
                o = oracle.sage_prepare_head(q[b, h], k[b, h], v[b, h], qk, 1)
                for n in ("q8", "k8", "v8", "q_scale", "k_scale", "v_scale"):
                    assert np.array_equal(g[n][b, h].view(np.uint8), o[n].view(np.uint8)), ((B, H, L, d), qk, n)
        out = api.sage_attention(P).cpu().numpy()
        r, _, within = ts._explain("random shape sage %s" % qk, api, P, q, k, v, qk, out, 1)
        if qk == "int8":
            assert within
        ends.append(r)
    ends = np.array(ends)
    assert np.median(ends) <= REL_L2


def test_random_shapes_fp4_match_oracle(api):
    """4-bit V-Smooth over the same shapes: codes, means and E8M0 scales
    bit-exact; per case the given-S bar and the end-to-end accounting of
    test_gpu_fp4v."""
    import test_gpu_fp4v as tf
    for B, H, L, d, seed in SHAPES[:6]:
        q, k, v = synth.make_inputs(synth.custom(B, H, L, d), seed % 100000)
        perm = synth.random_perms(B, H, L, seed % 1000)
        P = api.prepare(dev_bf16(q), dev_bf16(k), dev_bf16(v), perm_in=torch.from_numpy(perm).cuda(), v_format=1)
        codes, exps = (t.cpu().numpy() for t in api.v4_codes_natural(P))
        for b in range(B):
            for h in range(H):
                o = oracle.prepare_head_fp4v(q[b, h], k[b, h], v[b, h], perm[b, h])
                assert np.array_equal(codes[b, h], o["v4"]) and np.array_equal(exps[b, h], o["v_exp"]), (B, H, L, d)
        out = api.attention(P).cpu().numpy()
        tf._explain_fp4("random shape fp4", api, P, q, k, v, perm, out)
