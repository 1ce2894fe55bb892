"""The Python binding checks what the C ABI cannot see (tensor dtypes,
shapes, contiguity, devices, and the size of a caller's output tensor)
before it calls the library, with ValueError rather than assert, so the
checks also hold under python -O.  Host-only: every case is rejected before
any GPU work."""
import pytest
import torch

from bit_attention_video_smooth_amd import api

Q = torch.zeros(1, 2, 64, 64, dtype=torch.bfloat16)


@pytest.mark.parametrize("args", [
    (Q.float(), Q, Q),              # wrong dtype
    (Q, Q[:, :1], Q),               # k shape differs
    (Q[0], Q[0], Q[0]),             # not 4-D
    (Q, Q.transpose(2, 3), Q),      # not contiguous
])
def test_inputs_rejected(args):
    for fn in (api.attention_bf16, api.prepare, api.sage_prepare):
        with pytest.raises(ValueError):
            fn(*args)


def test_out_tensor_checked():
    with pytest.raises(ValueError, match="out must be"):
        api.attention_bf16(Q, Q, Q, out=torch.empty(1, 2, 64, 32))
    with pytest.raises(ValueError, match="out must be"):
        api.attention_bf16(Q, Q, Q, out=torch.empty(1, 2, 64, 64, dtype=torch.float16))
    with pytest.raises(ValueError, match="contiguous"):
        api.attention_bf16(Q, Q, Q, out=torch.empty(1, 2, 64, 64).transpose(2, 3))


def test_perm_and_centroids_checked():
    with pytest.raises(ValueError, match="perm_in"):
        api.prepare(Q, Q, Q, perm_in=torch.zeros(1, 2, 64, dtype=torch.int64))
    with pytest.raises(ValueError, match="centroids"):
        api.prepare(Q, Q, Q, centroids_in=torch.zeros(1, 2, 3, 64))
