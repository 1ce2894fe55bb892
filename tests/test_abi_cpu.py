"""Host-only checks of the C ABI: the library loads, exports every symbol the
header declares, and rejects bad arguments before launching anything (no
GPU is touched by these calls)."""
import ctypes
import os
import re

import pytest

from bit_attention_video_smooth_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "vc_attention.h")


def _declared():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?(?:int|char\s*\*|const char\s*\*)\s*\*?\s*(\w+)\s*\(", txt, re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libvcattn.so is not built; run __graft_entry__.build()")
    return _lib.load()


def test_exports_every_declared_symbol(lib):
    names = _declared()
    assert set(names) == set(_lib.EXPORTS), names
    for n in names:
        assert hasattr(lib, n)


def test_version(lib):
    assert _lib.vc_version() == 2


def test_prepared_sizes(lib):
    s = _lib.shape_of(2, 3, 300, 64)
    b = _lib.vc_prepared_sizes(s)
    nb, Lp = 3, 384
    assert b == [6 * Lp * 64, 6 * Lp * 64, 6 * nb * 64 * 128, 6 * nb * 4, 6 * nb * 4,
                 6 * nb * 64 * 4, 6 * nb * 64 * 4, 6 * 300 * 4, 6 * 8]


def test_workspace_bytes_positive(lib):
    n = _lib.vsmooth_workspace_bytes(_lib.shape_of(1, 40, 75600, 128), _lib.make_params())
    assert n > 40 * 75600 * 4  # at least the assignment array


@pytest.mark.parametrize("B,H,L,d,code", [(1, 1, 100, 96, _lib.VC_ERR_UNSUPPORTED),
                                          (0, 1, 100, 64, _lib.VC_ERR_INVALID),
                                          (1, 1, 0, 64, _lib.VC_ERR_INVALID),
                                          (1, -2, 10, 128, _lib.VC_ERR_INVALID)])
def test_bad_shape_rejected(lib, B, H, L, d, code):
    with pytest.raises(_lib.VCError) as e:
        _lib.vc_prepared_sizes(_lib.shape_of(B, H, L, d))
    assert e.value.code == code
    assert _lib.vc_last_error() != ""


def test_bad_params_rejected(lib):
    s = _lib.shape_of(1, 1, 256, 64)
    p = _lib.make_params()
    p.block = 64
    with pytest.raises(_lib.VCError) as e:
        _lib.vsmooth_workspace_bytes(s, p)
    assert e.value.code == _lib.VC_ERR_UNSUPPORTED
    for field, val in [("kmeans_iters", -1), ("v_scale_mode", 2), ("smooth_k", 3), ("kmeans_k", 257),
                       ("v_format", 2)]:
        p = _lib.make_params()
        setattr(p, field, val)
        with pytest.raises(_lib.VCError) as e:
            _lib.vsmooth_workspace_bytes(s, p)
        assert e.value.code == _lib.VC_ERR_INVALID, field


FAKE = 0x10000  # aligned, never dereferenced: validation fails first


def _prep(**over):
    f = dict(q8=FAKE, k8=FAKE, v8=FAKE, q_scale=FAKE, k_scale=FAKE, v_scale=FAKE, v_mean=FAKE,
             perm=FAKE, kmeans_obj=None)
    f.update(over)
    return _lib.vc_prepared(*[f[n] for n, _ in _lib.vc_prepared._fields_])


def test_prepare_rejects_null_and_misaligned(lib):
    s = _lib.shape_of(1, 1, 256, 64)
    p = _lib.make_params()
    with pytest.raises(_lib.VCError) as e:
        _lib.vsmooth_prepare(s, p, 0, FAKE, FAKE, None, _prep(), FAKE, 1 << 30, 0)
    assert e.value.code == _lib.VC_ERR_INVALID and "q" in str(e.value)
    with pytest.raises(_lib.VCError) as e:
        _lib.vsmooth_prepare(s, p, FAKE + 4, FAKE, FAKE, None, _prep(), FAKE, 1 << 30, 0)
    assert e.value.code == _lib.VC_ERR_INVALID and "aligned" in str(e.value)
    with pytest.raises(_lib.VCError) as e:
        _lib.vsmooth_prepare(s, p, FAKE, FAKE, FAKE, None, _prep(v8=0), FAKE, 1 << 30, 0)
    assert e.value.code == _lib.VC_ERR_INVALID


def test_prepare_rejects_small_workspace(lib):
    s = _lib.shape_of(1, 2, 1000, 128)
    p = _lib.make_params()
    need = _lib.vsmooth_workspace_bytes(s, p)
    with pytest.raises(_lib.VCError) as e:
        _lib.vsmooth_prepare(s, p, FAKE, FAKE, FAKE, None, _prep(), FAKE, need - 1, 0)
    assert e.value.code == _lib.VC_ERR_WORKSPACE


def test_attention_rejects_bad_params(lib):
    s = _lib.shape_of(1, 1, 256, 64)
    for z, od in [(9, 0), (-1, 0), (8, 2)]:
        with pytest.raises(_lib.VCError) as e:
            _lib.vc_attention_fwd(s, _lib.vc_attn_params(z, od), _prep(), FAKE, 0)
        assert e.value.code == _lib.VC_ERR_INVALID
    for pc in (-1, 2):
        with pytest.raises(_lib.VCError) as e:
            _lib.vc_attention_fwd(s, _lib.vc_attn_params(8, 0, 0.0, pc), _prep(), FAKE, 0)
        assert e.value.code == _lib.VC_ERR_INVALID
    for lam in (-0.1, 1.5, float("nan")):
        with pytest.raises(_lib.VCError) as e:
            _lib.vc_attention_fwd(s, _lib.vc_attn_params(8, 0, lam), _prep(), FAKE, 0)
        assert e.value.code == _lib.VC_ERR_INVALID
    with pytest.raises(_lib.VCError):
        _lib.vc_attention_fwd(s, _lib.vc_attn_params(8, 0), _prep(q_scale=0), FAKE, 0)
    with pytest.raises(_lib.VCError) as e:
        _lib.vc_attention_fwd_dump(s, _lib.vc_attn_params(8, 0), _prep(), FAKE, 5, 0, FAKE, FAKE, 0)
    assert e.value.code == _lib.VC_ERR_INVALID


def test_bf16_rejects(lib):
    with pytest.raises(_lib.VCError) as e:
        _lib.vc_attention_fwd_bf16(_lib.shape_of(1, 1, 64, 80), FAKE, FAKE, FAKE, FAKE, 0, 0)
    assert e.value.code == _lib.VC_ERR_UNSUPPORTED
    with pytest.raises(_lib.VCError):
        _lib.vc_attention_fwd_bf16(_lib.shape_of(1, 1, 64, 64), FAKE, FAKE, FAKE, FAKE, 3, 0)


def test_debug_entry_points_validate(lib):
    with pytest.raises(_lib.VCError):
        _lib.vc_debug_expcast(FAKE, FAKE, 0, 10, FAKE, 0)
    with pytest.raises(_lib.VCError):
        _lib.vc_debug_e4m3_encode(FAKE, -1, FAKE, 0)
    _lib.vc_debug_e4m3_encode(FAKE, 0, FAKE, 0)  # n == 0 is a no-op
    with pytest.raises(_lib.VCError):
        _lib.vc_debug_mfma_fp8(FAKE, 0, FAKE, 1, 0)
    for blocks, iters, out in [(0, 10, FAKE), (1 << 21, 10, FAKE), (256, 0, FAKE), (256, 1 << 25, FAKE),
                               (256, 10, 0)]:
        with pytest.raises(_lib.VCError) as e:
            _lib.vc_debug_mfma_rate(blocks, iters, out, 0)
        assert e.value.code == _lib.VC_ERR_INVALID


def _sprep(**over):
    f = dict(q8=FAKE, k8=FAKE, v8=FAKE, q_scale=FAKE, k_scale=FAKE, v_scale=FAKE)
    f.update(over)
    return _lib.vc_sage_prepared(*[f[n] for n, _ in _lib.vc_sage_prepared._fields_])


def test_sage_sizes_and_workspace(lib):
    s = _lib.shape_of(2, 3, 300, 64)
    nb, Lp = 3, 384
    assert _lib.vc_sage_prepared_sizes(s) == [6 * Lp * 64, 6 * Lp * 64, 6 * nb * 64 * 128, 6 * Lp * 4,
                                              6 * (Lp // 16) * 4, 6 * 64 * 4]
    assert _lib.vc_sage_workspace_bytes(s) >= 6 * 64 * (8 + 4 + 4 + 4)


def test_sage_rejects_bad_recipe(lib):
    s = _lib.shape_of(1, 1, 256, 64)
    ap = _lib.vc_attn_params(8, 0, 0.0, 1)
    for field, val in [("qk_dtype", 2), ("v_dtype", 1), ("q_block_size", 2), ("k_block_size", 128),
                       ("v_block_size", 16)]:
        p = _lib.make_sage_params()
        setattr(p, field, val)
        with pytest.raises(_lib.VCError) as e:
            _lib.vc_sage_attention_fwd(s, p, ap, _sprep(), FAKE, 0)
        assert e.value.code == _lib.VC_ERR_UNSUPPORTED, field
        with pytest.raises(_lib.VCError) as e:
            _lib.vc_sage_prepare(s, p, FAKE, FAKE, FAKE, _sprep(), FAKE, 1 << 30, 0)
        assert e.value.code == _lib.VC_ERR_UNSUPPORTED, field
    p = _lib.make_sage_params(smooth_k=2)
    with pytest.raises(_lib.VCError) as e:
        _lib.vc_sage_prepare(s, p, FAKE, FAKE, FAKE, _sprep(), FAKE, 1 << 30, 0)
    assert e.value.code == _lib.VC_ERR_INVALID


def test_sage_rejects_bad_arguments(lib):
    s = _lib.shape_of(1, 2, 1000, 128)
    p = _lib.make_sage_params()
    need = _lib.vc_sage_workspace_bytes(s)
    with pytest.raises(_lib.VCError) as e:
        _lib.vc_sage_prepare(s, p, FAKE, FAKE, FAKE, _sprep(), FAKE, need - 1, 0)
    assert e.value.code == _lib.VC_ERR_WORKSPACE
    with pytest.raises(_lib.VCError) as e:
        _lib.vc_sage_prepare(s, p, FAKE, FAKE + 8, FAKE, _sprep(), FAKE, need, 0)
    assert e.value.code == _lib.VC_ERR_INVALID
    with pytest.raises(_lib.VCError) as e:
        _lib.vc_sage_attention_fwd(s, p, _lib.vc_attn_params(8, 0, 0.5, 1), _sprep(), FAKE, 0)
    assert e.value.code == _lib.VC_ERR_UNSUPPORTED  # the baseline runs dense
    for pc in (-1, 2):
        with pytest.raises(_lib.VCError) as e:
            _lib.vc_sage_attention_fwd(s, p, _lib.vc_attn_params(8, 0, 0.0, pc), _sprep(), FAKE, 0)
        assert e.value.code == _lib.VC_ERR_INVALID
    with pytest.raises(_lib.VCError) as e:
        _lib.vc_sage_attention_fwd(s, p, _lib.vc_attn_params(8, 0, 0.0, 1), _sprep(v_scale=0), FAKE, 0)
    assert e.value.code == _lib.VC_ERR_INVALID
    with pytest.raises(_lib.VCError) as e:
        _lib.vc_sage_attention_fwd_dump(s, p, _lib.vc_attn_params(8, 0, 0.0, 1), _sprep(), FAKE, 2, 0, FAKE,
                                        FAKE, 0)
    assert e.value.code == _lib.VC_ERR_INVALID


def test_fp4_v_format_rules(lib):
    s = _lib.shape_of(1, 1, 256, 64)
    p = _lib.make_params(v_scale_mode=1, v_format=1)   # FP4 scales are powers of two already
    with pytest.raises(_lib.VCError) as e:
        _lib.vsmooth_workspace_bytes(s, p)
    assert e.value.code == _lib.VC_ERR_INVALID
    assert _lib.vsmooth_workspace_bytes(s, _lib.make_params(v_format=1)) > 0
    for pc, lam, code in [(0, 0.0, _lib.VC_ERR_UNSUPPORTED), (1, 0.5, _lib.VC_ERR_UNSUPPORTED)]:
        with pytest.raises(_lib.VCError) as e:
            _lib.vc_attention_fwd(s, _lib.vc_attn_params(8, 0, lam, pc, 1), _prep(), FAKE, 0)
        assert e.value.code == code
    with pytest.raises(_lib.VCError) as e:
        _lib.vc_attention_fwd(s, _lib.vc_attn_params(8, 0, 0.0, 1, 2), _prep(), FAKE, 0)
    assert e.value.code == _lib.VC_ERR_INVALID
    with pytest.raises(_lib.VCError) as e:
        _lib.vc_sage_attention_fwd(s, _lib.make_sage_params(), _lib.vc_attn_params(8, 0, 0.0, 1, 1), _sprep(),
                                   FAKE, 0)
    assert e.value.code == _lib.VC_ERR_UNSUPPORTED


def test_error_text_is_per_thread(lib):
    """vc_last_error() is thread-local: an error raised on one thread is not
    seen by another, and a fresh thread starts with an empty text."""
    import threading
    s = _lib.shape_of(1, 1, 256, 64)
    seen = {}

    def failing():
        with pytest.raises(_lib.VCError):
            _lib.vc_attention_fwd(s, _lib.vc_attn_params(9, 0), _prep(), FAKE, 0)
        seen["failing"] = _lib.vc_last_error()
        barrier.wait()  # stay alive while the other thread looks
        barrier.wait()

    def clean():
        barrier.wait()
        seen["clean"] = _lib.vc_last_error()
        barrier.wait()

    barrier = threading.Barrier(2, timeout=30)
    ts = [threading.Thread(target=failing, daemon=True), threading.Thread(target=clean, daemon=True)]
    for t in ts:
        t.start()
    for t in ts:
        t.join(timeout=60)
    assert seen["failing"] != ""
    assert seen["clean"] == ""


@pytest.mark.parametrize("L,d", [(8388480 + 1, 128), (16777088 + 1, 64), (2 ** 31 - 1, 128)])
def test_head_beyond_32bit_offsets_rejected(lib, L, d):
    # one head's padded K/V in bf16 (2 Lp d bytes) must stay below 2^31
    with pytest.raises(_lib.VCError) as e:
        _lib.vc_prepared_sizes(_lib.shape_of(1, 1, L, d))
    assert e.value.code == _lib.VC_ERR_INVALID
    assert "2^31" in str(e.value) or "too large" in str(e.value)


@pytest.mark.parametrize("L,d", [(8388480, 128), (16777088, 64)])
def test_longest_head_accepted(lib, L, d):
    b = _lib.vc_prepared_sizes(_lib.shape_of(1, 1, L, d))
    assert b[0] == ((L + 127) // 128) * 128 * d


def test_noalloc_rejects_shape_beyond_scratch(lib):
    # the long workload (24 heads of L = 245,952) needs ~114 MiB of workspace
    # with k-means, more than the fixed 64 MiB scratch; the check comes before
    # any pointer is looked at or any device call is made
    s = _lib.shape_of(1, 24, 245952, 128)
    p = _lib.make_params()
    need = _lib.vsmooth_workspace_bytes(s, p)
    assert need > 64 << 20
    with pytest.raises(_lib.VCError) as e:
        _lib.vsmooth_prepare_noalloc(s, p, None, None, None, None, _lib.vc_prepared(), stream=0)
    assert e.value.code == _lib.VC_ERR_WORKSPACE
    assert "scratch" in str(e.value)


def test_noalloc_fits_the_benchmark_workload(lib):
    s = _lib.shape_of(1, 40, 75600, 128)
    assert _lib.vsmooth_workspace_bytes(s, _lib.make_params()) <= 64 << 20
