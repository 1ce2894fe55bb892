"""The per-layer session over denoising steps on the GPU: grouping steps
run k-means on that step's V, the other steps reuse the latest permutation
(passed back into the library as perm_in = the layer's own perm buffer),
and every step's output equals a direct prepare + attention with that
permutation; one reuse step is checked against the oracle."""
import numpy as np
import pytest
import torch

import oracle
from bit_attention_video_smooth_amd import synth
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
        if step == 5:  # a reuse step against the oracle
            pn = perm.cpu().numpy()
            for h in range(H):
                o = oracle.prepare_head(q[0, h], k[0, h], vs[0, h], pn[0, h])
                r = oracle.attention_head(o, L)
                got = out[0, h].cpu().numpy()
                rel = float(np.linalg.norm(got - r) / np.linalg.norm(r))
                print("schedule step 5 head %d: rel-L2 %.3g" % (h, rel))
                assert rel <= 2e-3
    assert layer.grouped_at == 2
