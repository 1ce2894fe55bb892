"""GPU parity of 4-bit V-Smooth (E2M1 V residual and probabilities with
power-of-two scales per 32-key group, on the scaled FP4 matrix cores; FP8
per-block Q/K, exact block means) against the oracle, through the C ABI.

Bars: Q/K codes, means, E2M1 residual codes and E8M0 scales bit-exact; given
the kernel's own scores, the dumped E2M1 probability codes equal the
oracle's (one-code differences allowed at a rate below 1e-4, where
v_exp_f32's last-bit error could straddle a rounding midpoint) and the output
is within rel-L2 1e-4, max-abs 1e-3 of max; end to end, against the oracle's
exactly rounded scores, the deviation beyond that accounted for by the
probability values the matrix core's inexact score sums change (codes one
step apart, or a group's power-of-two scale moved when its largest
probability crosses a power of two; parity_util.explain_fp4_rows).  The key
group of in-block key kk is kk div 32."""
import os
import sys

import numpy as np
import pytest
import torch

import oracle
from bit_attention_video_smooth_amd import synth

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
from parity_util import check_explained, explain_fp4_rows  # noqa: E402

pytestmark = pytest.mark.gpu

SHAPES = [(1, 2, 1024, 64, (4, 16, 16)), (1, 3, 300, 128, None), (2, 2, 129, 64, None),
          (1, 1, 1, 128, None), (1, 2, 4000, 128, None), (1, 1, 520, 64, None),
          (1, 1, 500, 128, None)]


@pytest.fixture(scope="module")
def api():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    from bit_attention_video_smooth_amd import api as a
    a._lib.load()
    return a


def dev_bf16(u16):
    return torch.from_numpy(np.ascontiguousarray(u16)).view(torch.bfloat16).cuda()


def rel_l2(a, b):
    return float(np.linalg.norm((a - b).ravel()) / np.linalg.norm(b.ravel()))


def _inputs(B, H, L, d, seed, grid=None):
    return synth.make_inputs(synth.custom(B, H, L, d, grid=grid), seed)


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("smooth_k", [1, 0])
def test_fp4v_prepare_bit_exact(api, shape, smooth_k):
    B, H, L, d, grid = shape
    q, k, v = _inputs(B, H, L, d, 600 + L, grid)
    perm = synth.random_perms(B, H, L, 17)
    P = api.prepare(dev_bf16(q), dev_bf16(k), dev_bf16(v), perm_in=torch.from_numpy(perm).cuda(),
                    smooth_k=smooth_k, v_format=1)
    codes, exps = (t.cpu().numpy() for t in api.v4_codes_natural(P))
    g = {n: getattr(P, n).cpu().numpy() for n in ("q8", "k8", "q_scale", "k_scale", "v_mean")}
    for b in range(B):
        for h in range(H):
            o = oracle.prepare_head_fp4v(q[b, h], k[b, h], v[b, h], perm[b, h], smooth_k)
            for n in ("q8", "k8", "q_scale", "k_scale", "v_mean"):
                assert np.array_equal(g[n][b, h].view(np.uint8), o[n].view(np.uint8)), n
            for n, x, y in (("v4", codes[b, h], o["v4"]), ("v_exp", exps[b, h], o["v_exp"])):
                if not np.array_equal(x, y):
                    idx = np.argwhere(x != y)[:5]
                    pytest.fail("%s mismatch at %s: gpu %s oracle %s" % (n, idx.tolist(), x[tuple(idx.T)],
                                                                          y[tuple(idx.T)]))


def _oracle_out(q, k, v, perm, scores=None):
    B, H, L, d = q.shape
    out = np.empty((B, H, L, d), np.float32)
    for b in range(B):
        for h in range(H):
            o = oracle.prepare_head_fp4v(q[b, h], k[b, h], v[b, h], perm[b, h])
            sc = None if scores is None else np.ascontiguousarray(scores[b, h])
            out[b, h] = oracle.attention_head_fp4v(o, L, scores=sc)
    return out


@pytest.mark.parametrize("shape", SHAPES)
def test_fp4v_attention_matches_oracle(api, shape):
    B, H, L, d, grid = shape
    q, k, v = _inputs(B, H, L, d, 700 + L, grid)
    perm = synth.random_perms(B, H, L, 19)
    P = api.prepare(dev_bf16(q), dev_bf16(k), dev_bf16(v), perm_in=torch.from_numpy(perm).cuda(), v_format=1)
    out = api.attention(P).cpu().numpy()
    _explain_fp4("fp4 P V", api, P, q, k, v, perm, out)


def _explain_fp4(tag, api, P, q, k, v, perm, out):
    """Whole-output end-to-end check of the 4-bit path, every query tile."""
    B, H, L, d = q.shape
    nqt = (L + 255) // 256
    refs, refSs, deltas, flips = [], [], [], []
    for bh in range(B * H):
        b, h = divmod(bh, H)
        o = oracle.prepare_head_fp4v(q[b, h], k[b, h], v[b, h], perm[b, h])
        for qt in range(nqt):
            od, s, pb = api.attention_dump(P, bh, qt)
            if qt == 0 and bh == 0:  # the dumping instance computes what the plain one does
                assert torch.equal(od, api.attention(P))
            r0, r1 = qt * 256, min(L, qt * 256 + 256)
            ref, refS, delta, fl = explain_fp4_rows(o, L, (r0, r1), s.cpu().numpy()[:r1 - r0],
                                                    pb.cpu().numpy()[:r1 - r0])
            refs.append(ref)
            refSs.append(refS)
            deltas.append(delta)
            flips.append(fl)
    got = out.reshape(B * H, L, d)
    return check_explained("%s %s" % (tag, (B, H, L, d)), got.reshape(-1, d), np.concatenate(refs),
                           np.concatenate(refSs), np.concatenate(deltas), np.concatenate(flips))


def test_fp4v_bf16_output(api):
    B, H, L, d, grid = SHAPES[0]
    q, k, v = _inputs(B, H, L, d, 11, grid)
    P = api.prepare(dev_bf16(q), dev_bf16(k), dev_bf16(v), v_format=1)
    o32 = api.attention(P).cpu().numpy()
    o16 = api.attention(P, out_dtype=torch.bfloat16).float().cpu().numpy()
    assert np.array_equal(o16, torch.from_numpy(o32).to(torch.bfloat16).float().numpy())


def test_fp4v_uniform_attention_exact(api):
    """The oracle's closed-form case on the GPU: identical Q rows and K rows,
    V = block constant plus an exactly representable E2M1 residual; the
    output is the plain mean of V (to fp32 accumulation)."""
    import os
    import sys
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    import test_oracle_fp4_pins as pins
    L, d = 288, 64
    q, k, v, vf = pins._uniform_inputs(L, d, 4)
    P = api.prepare(dev_bf16(q[None, None]), dev_bf16(k[None, None]), dev_bf16(v[None, None]),
                    perm_in=torch.arange(L, dtype=torch.int32, device="cuda")[None, None].contiguous(), v_format=1)
    out = api.attention(P).cpu().numpy()[0, 0]
    np.testing.assert_allclose(out, np.tile(vf.mean(axis=0), (L, 1)), rtol=1e-5, atol=1e-5)


def test_fp4_value_stats_match_oracle(api):
    """The ablation's 4-bit V error (mean + 2^e E2M1(code) against v) from the
    library's codes equals the same statistic of the oracle's codes."""
    from bit_attention_video_smooth_amd.ablation import fp4_value_stats
    B, H, L, d, grid = SHAPES[1]
    q, k, v = _inputs(B, H, L, d, 13, grid)
    perm = synth.random_perms(B, H, L, 23)
    vd = dev_bf16(v)
    P = api.prepare(dev_bf16(q), dev_bf16(k), vd, perm_in=torch.from_numpy(perm).cuda(), v_format=1)
    st = fp4_value_stats(P, vd)["v_rel_err"]
    j = np.arange(128)
    for b in range(B):
        for h in range(H):
            o = oracle.prepare_head_fp4v(q[b, h], k[b, h], v[b, h], perm[b, h])
            x = oracle.bf16_to_f32(v[b, h]).astype(np.float64)[perm[b, h]]
            sc = 2.0 ** (o["v_exp"].astype(np.int64)[..., j // 32] - 127)                # [nb,d,128]
            xh = o["v_mean"].astype(np.float64)[:, :, None] + oracle.e2m1_decode(o["v4"]) * sc
            xh = xh.transpose(0, 2, 1).reshape(-1, d)[:L]
            ref = np.sqrt(((xh - x) ** 2).sum() / (x * x).sum())
            assert abs(st[b, h] - ref) <= 1e-9 * ref, (st[b, h], ref)
