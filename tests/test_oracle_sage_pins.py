"""Pins of the oracle's SAGE-style baseline against facts outside the oracle.

The baseline follows the TensorRT-LLM blog, "Quantized Attention": QK^T in
INT8 or FP8, PV in FP8 E4M3, one Q scale per query token, one K scale per 16
consecutive keys, one V scale per channel taken over all tokens of a head.
Each test below would fail for a plausible slip in the oracle:
  * the INT8 codec: round-to-nearest-even on exact ties, and the bound
    |x - s*code| <= s/2 (a floor, a wrong qmax or an off-by-one clamp fails);
  * granularity: every query row, every 16-key group and every channel
    reaches the top code (a per-block scale would not), while single K rows
    and single V blocks do not;
  * the score coefficients: the oracle's P bytes against the dequantised
    scores computed in float64 by NumPy with a running maximum (a wrong
    scale index or a missing C0 moves them far outside one E4M3 step);
  * group structure: exchanging two keys inside a 16-key group leaves the
    output bit-identical, across groups it does not;
  * a special case where SAGE and V-Smooth coincide (power-of-two scales,
    zero block means, every row/group/block reaching the same amax): both
    oracles give the same bytes and the same output;
  * fp64 brute-force softmax attention within the quantisation band.
"""
import numpy as np
import pytest

from bit_attention_video_smooth_amd import synth


def _bf16(x):
    return synth.f32_to_bf16_bits(np.asarray(x, np.float32))


def _f32(u16):
    import oracle
    return oracle.bf16_to_f32(u16)


def _rand_head(L, d, seed, koff=0.5):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((L, d))
    k = rng.standard_normal((L, d)) + koff * rng.standard_normal(d)
    v = rng.standard_normal((L, d))
    return _bf16(q), _bf16(k), _bf16(v)


def _i8(codes):
    return codes.view(np.int8).astype(np.int64)


# ------------------------------------------------------------ INT8 codec --

def test_int8_ties_to_even_and_bound(oracle_mod):
    d = 64
    # row amax 127 gives scale 1 exactly: every code is the rounded value
    row = np.zeros(d, np.float32)
    row[0] = 127.0
    ties = np.array([0.5, 1.5, 2.5, 3.5, -0.5, -1.5, -2.5, 10.5, 11.5, -126.5], np.float32)
    row[1:1 + len(ties)] = ties
    near = np.array([2.25, 2.75, -2.75, 126.75], np.float32)
    row[20:20 + len(near)] = near
    q = np.tile(row, (3, 1))
    k = _bf16(np.ones((3, d)))
    P = oracle_mod.sage_prepare_head(_bf16(q), k, k, "int8", smooth_k=0)
    assert P["q_scale"][0] == np.float32(1.0)
    c = _i8(P["q8"][0])
    assert c[0] == 127
    assert c[1:1 + len(ties)].tolist() == [0, 2, 2, 4, 0, -2, -2, 10, 12, -126]
    assert c[20:20 + len(near)].tolist() == [2, 3, -3, 127]

    # random rows: |x - s code| <= s/2, plus the fp32 rounding of x * inv
    # (127 * 2^-24 in code units) and of s * inv against 1 (2^-23 |x|)
    q, k, v = _rand_head(300, 64, 1)
    P = oracle_mod.sage_prepare_head(q, k, v, "int8", smooth_k=0)
    x = _f32(q).astype(np.float64)
    s = P["q_scale"][:300].astype(np.float64)[:, None]
    err = np.abs(x - s * _i8(P["q8"][:300]))
    assert np.all(err <= s * (0.5 + 2.5e-5))
    assert err.max() > 0.49 * s.min()  # the bound is nearly reached: codes are rounded, not truncated


# ------------------------------------------------------------ granularity --

@pytest.mark.parametrize("qk", ["int8", "fp8"])
def test_scale_granularity(oracle_mod, qk):
    L, d = 300, 64
    q, k, v = _rand_head(L, d, 2)
    P = oracle_mod.sage_prepare_head(q, k, v, qk, smooth_k=1)
    top = 127 if qk == "int8" else 448.0
    mag = (lambda c: np.abs(_i8(c))) if qk == "int8" else (lambda c: np.abs(oracle_mod.e4m3_decode(c)))
    qm = mag(P["q8"][:L]).max(axis=1)
    assert np.all(qm == top)                              # one scale per query token
    km = mag(P["k8"][:L])
    gm = [km[g:g + 16].max() for g in range(0, L, 16)]
    assert np.all(np.asarray(gm) == top)                   # one scale per 16 keys ...
    assert np.mean(km.max(axis=1) == top) < 0.5            # ... not one per key
    assert np.all(P["q_scale"][L:] == 0) and np.all(P["q8"][L:] == 0)
    assert P["k_scale"].shape == ((P["k8"].shape[0]) // 16,)
    vm = np.abs(oracle_mod.e4m3_decode(P["v8"]))           # [nb, d, 128]
    assert np.all(vm.max(axis=(0, 2)) == 448.0)           # one scale per channel ...
    assert np.any(vm.max(axis=2) < 448.0)                  # ... not one per block
    assert np.all(P["v8"][-1, :, L - 2 * 128:] == 0)       # padded slots


# ---------------------------------------------------- score coefficients --

@pytest.mark.parametrize("qk", ["int8", "fp8"])
def test_bytes_follow_dequantised_scores(oracle_mod, qk):
    """exp-then-cast bytes against p = 2^(z - m_b + z_off), z the dequantised
    score in log2 units and m_b the running block maximum, all in float64."""
    L, d, z_off = 300, 64, 8
    q, k, v = _rand_head(L, d, 3)
    P = oracle_mod.sage_prepare_head(q, k, v, qk, smooth_k=1)
    O, by, S = oracle_mod.sage_attention_head(P, L, qk, z_off=z_off, prob_cast=1, want_bytes=True)
    dec = (lambda c: _i8(c).astype(np.float64)) if qk == "int8" else oracle_mod.e4m3_decode
    qd = dec(P["q8"][:L]) * P["q_scale"][:L, None].astype(np.float64)
    Lp = P["k8"].shape[0]
    ks = np.repeat(P["k_scale"].astype(np.float64), 16)[:, None]
    kd = dec(P["k8"]) * ks
    z = (qd @ kd.T) * (np.log2(np.e) / np.sqrt(d))       # [L, Lp]
    z[:, L:] = -np.inf
    nb = Lp // 128
    bmax = z.reshape(L, nb, 128).max(axis=2)
    run = np.maximum.accumulate(bmax, axis=1)              # running max after block b
    ref = np.exp2(z - np.repeat(run, 128, axis=1) + z_off)[:, :L]
    got = oracle_mod.e4m3_decode(by[:, :L])
    # one E4M3 step (relative 2^-4 for normals, 2^-9 absolute for subnormals)
    assert np.all(np.abs(got - ref) <= np.maximum(ref * 2.0 ** -4, 2.0 ** -9) * 1.01)


# ------------------------------------------------------- group structure --

def test_swap_inside_group_is_exact(oracle_mod):
    L, d = 300, 64
    q, k, v = _rand_head(L, d, 4)

    def run(perm):
        P = oracle_mod.sage_prepare_head(q, k[perm], v[perm], "int8", smooth_k=1)
        return oracle_mod.sage_attention_head(P, L, "int8", prob_cast=0)

    ident = np.arange(L)
    base = run(ident)
    same = ident.copy()
    same[[3, 12]] = same[[12, 3]]          # keys 3 and 12: both in group 0
    np.testing.assert_array_equal(run(same), base)
    across = ident.copy()
    across[[3, 20]] = across[[20, 3]]      # group 0 <-> group 1, same 128-key block
    assert not np.array_equal(run(across), base)


# ------------------------------------------- a case where SAGE = V-Smooth --

def _coincident_inputs(L, d, seed):
    """Q and K rows each hold +-7 (scale 7/448 = 2^-6 for every token, 16-key
    group and 128-token block); V blocks are made of (x, -x) token pairs, so
    each block mean is exactly 0, and every block of every channel holds
    +-3.5 (scale 3.5/448 = 2^-7 per channel and per block)."""
    rng = np.random.default_rng(seed)
    q = np.clip(rng.standard_normal((L, d)), -6.5, 6.5)
    k = np.clip(rng.standard_normal((L, d)), -6.5, 6.5)
    q[:, 0] = 7.0 * np.where(rng.random(L) < 0.5, -1.0, 1.0)
    k[:, 1] = 7.0 * np.where(rng.random(L) < 0.5, -1.0, 1.0)
    v = np.empty((L, d))
    for b0 in range(0, L, 128):
        n = min(128, L - b0)
        assert n % 2 == 0
        x = np.clip(rng.standard_normal((n // 2, d)), -3.0, 3.0)
        x[0] = 3.5
        v[b0:b0 + n:2] = x
        v[b0 + 1:b0 + n:2] = -x
    return _bf16(q), _bf16(k), _bf16(v)


@pytest.mark.parametrize("prob_cast", [0, 1])
def test_sage_equals_vsmooth_where_they_coincide(oracle_mod, prob_cast):
    L, d = 300, 64
    q, k, v = _coincident_inputs(L, d, 5)
    S_ = oracle_mod.sage_prepare_head(q, k, v, "fp8", smooth_k=0)
    V_ = oracle_mod.prepare_head(q, k, v, np.arange(L, dtype=np.int32), smooth_k=0)
    # the two prepares produce the same codes and scales here
    np.testing.assert_array_equal(S_["q8"], V_["q8"])
    np.testing.assert_array_equal(S_["k8"], V_["k8"])
    np.testing.assert_array_equal(S_["v8"], V_["v8"])
    assert np.all(V_["v_mean"] == 0) and np.all(V_["v_scale"] == S_["v_scale"][None, :])
    Os, bs, _ = oracle_mod.sage_attention_head(S_, L, "fp8", prob_cast=prob_cast, want_bytes=True)
    Ov, bv, _, _ = oracle_mod.attention_head(V_, L, prob_cast=prob_cast, want_bytes=True)
    np.testing.assert_array_equal(bs, bv)
    np.testing.assert_allclose(Os, Ov, rtol=2.5e-7, atol=1e-30)


# ------------------------------------------------------------ vs fp64 --

@pytest.mark.parametrize("qk", ["int8", "fp8"])
@pytest.mark.parametrize("prob_cast", [0, 1])
def test_sage_within_band_of_exact_attention(oracle_mod, qk, prob_cast):
    cfg = synth.CONFIGS[0]
    q, k, v = synth.make_inputs(cfg, 0)
    L = cfg.L
    qh, kh, vh = q[0, 1], k[0, 1], v[0, 1]
    P = oracle_mod.sage_prepare_head(qh, kh, vh, qk, smooth_k=1)
    rows = (0, 256)
    O = oracle_mod.sage_attention_head(P, L, qk, prob_cast=prob_cast, rows=rows)
    ref = oracle_mod.attention_f64(_f32(qh), _f32(kh), _f32(vh), rows=rows)
    rel = np.linalg.norm(O - ref) / np.linalg.norm(ref)
    assert rel < 6e-2, rel
