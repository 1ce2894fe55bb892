"""The per-layer session over denoising steps on the GPU: grouping steps
run k-means on that step's V, the other steps reuse the latest permutation
(passed back into the library as perm_in = the layer's own perm buffer),
and every step's output equals a direct prepare + attention with that
permutation; one reuse step is checked against the oracle (bytes given the
kernel's scores, given-S bar, end to end as in test_gpu_parity)."""
import os
import sys

import numpy as np
import pytest
import torch

import oracle
from bit_attention_video_smooth_amd import synth

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
from parity_util import check_explained, explain_vsmooth_rows  # noqa: E402
from bit_attention_video_smooth_amd.schedule import GroupingSchedule, VCAttentionLayer

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def api():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    from bit_attention_video_smooth_amd import api as a
    a._lib.load()
    return a


def dev_bf16(u16):
    return torch.from_numpy(np.ascontiguousarray(u16)).view(torch.bfloat16).cuda()


def test_session_regroups_on_schedule_and_reuses_permutation(api):
    cfg = synth.CONFIGS[0]
    B, H, L, d = cfg.B, cfg.H, cfg.L, cfg.d
    q, k, v = synth.make_inputs(cfg, 0)
    sched = GroupingSchedule(8, group_frac=0.5, reuse=2)    # groups at steps 0 and 2
    assert sched.grouping_steps() == [0, 2]
    layer = VCAttentionLayer(B, H, L, d, sched, seed=5)
    rng = np.random.default_rng(1)
    vf = oracle.bf16_to_f32(v)
    perms = {}
    for step in range(8):
        # V drifts from step to step, as activations do over denoising
        vs = synth.f32_to_bf16_bits((vf + 0.05 * step * rng.normal(size=vf.shape)).astype(np.float32))
        out = layer.forward(dev_bf16(q), dev_bf16(k), dev_bf16(vs), step).clone()
        perm = layer.prepared.perm.clone()
        if sched.regroup(step):
            ref_P = api.prepare(dev_bf16(q), dev_bf16(k), dev_bf16(vs), seed=5)
            assert torch.equal(perm, ref_P.perm)
            perms[step] = perm
        else:
            g = max(s for s in perms if s <= step)
            assert torch.equal(perm, perms[g])
            ref_P = api.prepare(dev_bf16(q), dev_bf16(k), dev_bf16(vs), perm_in=perms[g])
        ref = api.attention(ref_P)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), step
        if step == 5:  # a reuse step against the oracle, every query tile
            pn = perm.cpu().numpy()
            for h in range(H):
                o = oracle.prepare_head(q[0, h], k[0, h], vs[0, h], pn[0, h])
                for qt in range((L + 255) // 256):
                    r0, r1 = 256 * qt, min(L, 256 * qt + 256)
                    _, S, Pb = api.attention_dump(layer.prepared, h, qt)
                    ref, refS, delta, flips = explain_vsmooth_rows(o, L, (r0, r1), S.cpu().numpy()[:r1 - r0],
                                                                   Pb.cpu().numpy()[:r1 - r0])
                    check_explained("schedule step 5 head %d tile %d" % (h, qt), out[0, h, r0:r1].cpu().numpy(),
                                    ref, refS, delta, flips)
    assert layer.grouped_at == 2


# -------------------------------------------------- warm-started k-means --

def test_warm_start_composes(api):
    """8 Lloyd rounds from the seeded init equal 4 rounds, then 4 more
    warm-started from the centroids those left (vsmooth_prepare_warm with
    centroids_out aliasing centroids_in): same permutation, codes, objective
    and centroids, bit for bit."""
    cfg = synth.CONFIGS[0]
    B, H, L, d = cfg.B, cfg.H, cfg.L, cfg.d
    q, k, v = (dev_bf16(a) for a in synth.make_inputs(cfg, 3))
    nb = (L + 127) // 128
    C8 = torch.empty((B, H, nb, d), dtype=torch.float32, device="cuda")
    P8 = api.prepare(q, k, v, seed=4, kmeans_iters=8, centroids_out=C8)
    C = torch.empty_like(C8)
    api.prepare(q, k, v, seed=4, kmeans_iters=4, centroids_out=C)
    Pw = api.prepare(q, k, v, seed=4, kmeans_iters=4, centroids_in=C, centroids_out=C)
    torch.cuda.synchronize()
    assert torch.equal(Pw.perm, P8.perm)
    assert torch.equal(Pw.kmeans_obj, P8.kmeans_obj)
    assert torch.equal(Pw.v8, P8.v8) and torch.equal(Pw.v_mean, P8.v_mean)
    assert torch.equal(C, C8)
    # the plain entry point and the warm one with no centroids agree
    P0 = api.prepare(q, k, v, seed=4, kmeans_iters=8)
    torch.cuda.synchronize()
    assert torch.equal(P0.perm, P8.perm)


def test_warm_start_matches_oracle(api):
    """Warm start from centroids the oracle computed: the GPU objective is
    within 1% of the oracle's warm-started objective, and its final
    centroids are close to the oracle's."""
    cfg = synth.CONFIGS[0]
    B, H, L, d = cfg.B, cfg.H, cfg.L, cfg.d
    q, k, v = synth.make_inputs(cfg, 6)
    nb = (L + 127) // 128
    init = np.stack([oracle.kmeans(v[0, h], nb, 2, 77 + h)[1] for h in range(H)])[None]  # [1,H,k,d]
    Cg = torch.empty((B, H, nb, d), dtype=torch.float32, device="cuda")
    P = api.prepare(dev_bf16(q), dev_bf16(k), dev_bf16(v), kmeans_iters=4,
                    centroids_in=torch.from_numpy(init).cuda(), centroids_out=Cg)
    obj = P.kmeans_obj.cpu().numpy()
    Cg = Cg.cpu().numpy()
    for h in range(H):
        a, C, J = oracle.kmeans_warm(v[0, h], init[0, h], 4)
        rel = float(np.linalg.norm(Cg[0, h] - C) / np.linalg.norm(C))
        print("warm start head %d: gpu J %.7g oracle J %.7g, centroid rel diff %.2e" % (h, obj[0, h], J, rel))
        assert abs(obj[0, h] / J - 1) <= 0.01
        assert rel <= 1e-2


def test_session_warm_start(api):
    """A session with warm_start: the first grouping is seeded, later ones
    start from the previous grouping's centroids; every step equals the
    direct calls it stands for."""
    cfg = synth.CONFIGS[0]
    B, H, L, d = cfg.B, cfg.H, cfg.L, cfg.d
    q, k, v = synth.make_inputs(cfg, 0)
    sched = GroupingSchedule(8, group_frac=0.5, reuse=2)    # groups at steps 0 and 2
    layer = VCAttentionLayer(B, H, L, d, sched, seed=5, warm_start=True)
    nb = (L + 127) // 128
    C = torch.empty((B, H, nb, d), dtype=torch.float32, device="cuda")
    rng = np.random.default_rng(2)
    vf = oracle.bf16_to_f32(v)
    cold = {}
    for step in range(4):
        vs = synth.f32_to_bf16_bits((vf + 0.05 * step * rng.normal(size=vf.shape)).astype(np.float32))
        out = layer.forward(dev_bf16(q), dev_bf16(k), dev_bf16(vs), step).clone()
        if step == 0:
            ref_P = api.prepare(dev_bf16(q), dev_bf16(k), dev_bf16(vs), seed=5, centroids_out=C)
        elif step == 2:
            ref_P = api.prepare(dev_bf16(q), dev_bf16(k), dev_bf16(vs), seed=5, centroids_in=C, centroids_out=C)
            cold_P = api.prepare(dev_bf16(q), dev_bf16(k), dev_bf16(vs), seed=5)
            cold = (cold_P.kmeans_obj.cpu().numpy(), ref_P.kmeans_obj.cpu().numpy())
        else:
            ref_P = api.prepare(dev_bf16(q), dev_bf16(k), dev_bf16(vs), perm_in=layer.prepared.perm.clone())
        ref = api.attention(ref_P)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), step
        assert torch.equal(layer.prepared.perm, ref_P.perm), step
    assert torch.equal(layer.centroids, C)
    print("step 2 k-means objective per head: seeded %s, warm-started %s" % (cold[0], cold[1]))
