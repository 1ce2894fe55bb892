"""Calls on different streams are independent (the C ABI's contract): two
problems prepared and attended at the same time from two host threads, each
on its own stream with its own buffers, give bit for bit what they give
when run alone."""
import threading

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


def test_concurrent_streams_match_sequential(api):
    cfgs = [synth.custom(1, 2, 3000, 128), synth.custom(1, 3, 2000, 64, grid=(2, 25, 40))]
    data = [[dev_bf16(a) for a in synth.make_inputs(c, 30 + i)] for i, c in enumerate(cfgs)]
    refs = []
    for q, k, v in data:
        P = api.prepare(q, k, v, seed=3)
        refs.append((api.attention(P).clone(), P.perm.clone(), P.v8.clone()))
    torch.cuda.synchronize()
    got = [None, None]
    errors = []

    def work(i):
        try:
            q, k, v = data[i]
            B, H, L, d = q.shape
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                P = api.alloc_prepared(B, H, L, d)
                ws = api.workspace(B, H, L, d)
                out = torch.empty((B, H, L, d), dtype=torch.float32, device="cuda")
                for _ in range(4):
                    api.prepare(q, k, v, seed=3, out=P, ws=ws, stream=s)
                    api.attention(P, out=out, stream=s)
            s.synchronize()
            got[i] = (out, P.perm, P.v8)
        except Exception as e:  # reported on the main thread
            errors.append(repr(e))

    ts = [threading.Thread(target=work, args=(i,)) for i in range(2)]
    for t in ts:
        t.start()
    for t in ts:
        t.join(timeout=120)
    assert not errors, errors
    for i in range(2):
        for a, b in zip(got[i], refs[i]):
            assert torch.equal(a, b), i
