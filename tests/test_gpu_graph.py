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


@pytest.mark.parametrize("recipe", ["sage_int8", "sage_fp8", "fp4", "warm"])
def test_other_paths_graph_replays_match_eager(api, recipe):
    """The SAGE baseline, 4-bit V-Smooth and the warm-started k-means step
    captured the same way.  The warm step carries its centroids from one
    replay to the next (centroids_out aliases centroids_in), so every replay
    is checked against the eager chain of the same length."""
    cfg = synth.custom(1, 2, 1300, 64, grid=(2, 25, 26))
    B, H, L, d = cfg.B, cfg.H, cfg.L, cfg.d
    q, k, v = (dev_bf16(a) for a in synth.make_inputs(cfg, 6))
    out = torch.empty((B, H, L, d), dtype=torch.float32, device="cuda")
    s = torch.cuda.Stream()
    if recipe.startswith("sage"):
        qk = recipe[5:]
        SP = api.sage_prepare(q, k, v, qk_dtype=qk)
        sws = torch.empty(max(16, api._lib.vc_sage_workspace_bytes(api._lib.shape_of(B, H, L, d))),
                          dtype=torch.uint8, device="cuda")

        def step():
            api.sage_prepare(q, k, v, qk_dtype=qk, out=SP, ws=sws, stream=torch.cuda.current_stream())
            api.sage_attention(SP, out=out, stream=torch.cuda.current_stream())
    else:
        P = api.alloc_prepared(B, H, L, d)
        ws = api.workspace(B, H, L, d)
        nb = api.nblocks(L)
        C = torch.zeros((B, H, nb, d), dtype=torch.float32, device="cuda")
        C0 = None
        if recipe == "warm":
            C0 = torch.empty_like(C)
            api.prepare(q, k, v, seed=2, kmeans_iters=2, centroids_out=C0)
            C.copy_(C0)

        def step():
            st = torch.cuda.current_stream()
            if recipe == "fp4":
                api.prepare(q, k, v, seed=7, out=P, ws=ws, v_format=1, stream=st)
            else:
                api.prepare(q, k, v, kmeans_iters=2, out=P, ws=ws, centroids_in=C, centroids_out=C, stream=st)
            api.attention(P, out=out, stream=st)
    # eager chain of three steps, recording each output
    refs = []
    with torch.cuda.stream(s):
        for _ in range(3):
            step()
            s.synchronize()
            refs.append(out.clone())
    if recipe == "warm":
        C.copy_(C0)  # restart the chain for the replays
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step()
    if recipe == "warm":
        C.copy_(C0)  # capture does not run the kernels, but start from a known state anyway
    torch.cuda.synchronize()
    for rep in range(3):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        ref = refs[rep] if recipe == "warm" else refs[0]
        assert torch.equal(out, ref), (recipe, rep)
        Po = api.prepare(*(dev_bf16(a) for a in synth.make_inputs(cfg, 8)), seed=1)
        api.attention(Po)
        torch.cuda.synchronize()
