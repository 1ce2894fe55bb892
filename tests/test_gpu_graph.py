"""A whole step (prepare with k-means, then attention) captured into one HIP
graph through torch.cuda.CUDAGraph and replayed: the library records only
kernel launches (no memset or copy nodes), so every replay must reproduce the
eager result bit for bit.  Replays alternate with eager work on other
inputs and synchronisations, as a serving loop would."""
import numpy as np
import pytest
import torch

from bit_attention_video_smooth_amd import synth

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


@pytest.mark.parametrize("skip_lambda", [0.0, 0.3])
def test_step_graph_replays_match_eager(api, skip_lambda):
    cfg = synth.custom(1, 2, 1500, 128, grid=(3, 20, 25))
    B, H, L, d = cfg.B, cfg.H, cfg.L, cfg.d
    q, k, v = (dev_bf16(a) for a in synth.make_inputs(cfg, 4))
    P = api.alloc_prepared(B, H, L, d)
    ws = api.workspace(B, H, L, d)
    out = torch.empty((B, H, L, d), dtype=torch.float32, device="cuda")
    s = torch.cuda.Stream()

    def step():
        api.prepare(q, k, v, seed=7, out=P, ws=ws, stream=torch.cuda.current_stream())
        api.attention(P, out=out, skip_lambda=skip_lambda, stream=torch.cuda.current_stream())

    # eager reference, on the side stream that will also capture
    with torch.cuda.stream(s):
        step()
    s.synchronize()
    ref, ref_perm = out.clone(), P.perm.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step()
    other = [dev_bf16(a) for a in synth.make_inputs(cfg, 5)]
    for rep in range(3):
        out.zero_()
        P.perm.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), rep
        assert torch.equal(P.perm, ref_perm), rep
        # eager work in between, on other inputs
        Po = api.prepare(*other, seed=1)
        api.attention(Po)
        torch.cuda.synchronize()
