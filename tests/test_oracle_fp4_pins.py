"""Pins of the oracle's 4-bit V-Smooth path (E2M1 residual and
probabilities with power-of-two scales per 32-key group; MarkTechPost
abstract: 4-bit V-Smooth, ExpCast for the 8-bit kernel only) against facts
outside the oracle:
  * E2M1 values from the format (OCP MX: 1 mantissa bit, exponent bias 1,
    largest 6, smallest subnormal 0.5);
  * the encoder against NumPy's round-half-even at one mantissa bit (a
    different algorithm from the oracle's nearest-code search);
  * the E8M0 rule by its defining inequality;
  * the residual codes within half a step, every key group (32 consecutive
    slots of the permuted block) reaching the top codes;
  * a block whose first 32 slots are large and the rest small keeps the
    small values at their own fine scale (an interleaved grouping, which
    mixes slots of every quarter into each group, would zero them);
  * P codes against dequantised float64 scores with a running maximum;
  * a closed form: uniform attention on inputs built so that every
    quantisation is exact gives the plain mean of V, and the 8-bit
    exp-then-cast oracle gives the same.
"""
import numpy as np
import pytest

from bit_attention_video_smooth_amd import synth

MAGS = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float64)


def _bf16(x):
    return synth.f32_to_bf16_bits(np.asarray(x, np.float32))


def _rne_e2m1(x):
    """Round-half-even of |x| at one mantissa bit (spacing 0.5 below 2, 1 in
    [2, 4), 2 in [4, 6]), saturating at 6; the sign kept."""
    a = np.abs(x)
    q = np.where(a < 2, 0.5, np.where(a < 4, 1.0, 2.0))
    v = np.minimum(np.round(a / q) * q, 6.0)
    return np.copysign(v, x)


def test_e2m1_values(oracle_mod):
    dec = oracle_mod.e2m1_decode(np.arange(16))
    assert np.array_equal(dec[:8], MAGS)
    assert np.array_equal(dec[8:], -MAGS)
    assert np.signbit(dec[8])                          # code 8 is -0
    assert dec[7] == 6.0 and dec[2] == 1.0 and dec[1] == 0.5
    assert np.array_equal(oracle_mod.e2m1_encode(dec), np.arange(16))  # round trip


def test_e2m1_encoder_rounds_half_even(oracle_mod):
    x = np.concatenate([np.linspace(-7.5, 7.5, 30001),
                        (MAGS[1:] + MAGS[:-1]) / 2, -(MAGS[1:] + MAGS[:-1]) / 2])
    got = oracle_mod.e2m1_decode(oracle_mod.e2m1_encode(x))
    assert np.array_equal(np.abs(got), np.abs(_rne_e2m1(x)))
    # the midpoints themselves: 0.25 -> 0, 0.75 -> 1, 1.25 -> 1, 1.75 -> 2, 2.5 -> 2, 3.5 -> 4, 5 -> 4
    mids = (MAGS[1:] + MAGS[:-1]) / 2
    assert oracle_mod.e2m1_decode(oracle_mod.e2m1_encode(mids)).tolist() == [0, 1, 1, 2, 2, 4, 4]


def test_e8m0_rule(oracle_mod):
    rng = np.random.default_rng(0)
    for A in np.exp(rng.uniform(-60, 60, 500)):
        e = oracle_mod.e8m0_exp(A)
        assert 6.0 * 2.0 ** (e - 1) < A <= 6.0 * 2.0 ** e
    for k in (-5, 0, 3):
        assert oracle_mod.e8m0_exp(6.0 * 2.0 ** k) == k
    assert oracle_mod.e8m0_exp(0.0) == -127 and oracle_mod.e8m0_exp(1e-31) == -127


def _group(j):
    """Key group of in-block slot j: 32 consecutive slots (the plain reading;
    the pages name 4-bit V-Smooth but not its groups)."""
    return j // 32


def test_fp4v_groups_are_contiguous_slots(oracle_mod):
    """Residual values 4 in every channel of slots 0..31 of the block and
    values in [0.1, 0.4] in slots 32..127: with groups of 32 consecutive
    slots, groups 1..3 take the scale 2^-4 and keep every small value within
    half an E2M1 step of it (the E8M0 rule puts 0.4 <= 6 * 2^-4); a grouping
    that puts any of slots 0..31 into those groups gives them scale 2^0, at
    which values below 0.25 encode to 0."""
    L, d = 128, 64
    rng = np.random.default_rng(7)
    x = rng.uniform(0.1, 0.4, (48, d)) * rng.choice([-1.0, 1.0], (48, d))
    small = np.concatenate([x, -x])                  # (x, -x) pairs: mean exactly 0
    big = 4.0 * np.concatenate([np.ones((16, d)), -np.ones((16, d))])
    res = np.concatenate([big, small])
    v = _bf16(res)                                   # bf16 keeps the pairs exact negatives
    q = _bf16(rng.standard_normal((L, d)))
    k = _bf16(rng.standard_normal((L, d)))
    perm = np.arange(L, dtype=np.int32)
    P4 = oracle_mod.prepare_head_fp4v(q, k, v, perm)
    e = P4["v_exp"][0].astype(int) - 127             # [d, 4]
    assert np.all(e[:, 0] >= 0) and np.all(e[:, 1:] <= -3)
    r = (oracle_mod.bf16_to_f32(v).astype(np.float32) - P4["v_mean"][0][None, :]).astype(np.float64)
    yh = oracle_mod.e2m1_decode(P4["v4"][0]).T * (2.0 ** e[:, np.arange(128) // 32]).T  # [128, d]
    tail = r[32:]
    assert np.all(np.abs(yh[32:] - tail) <= 2.0 ** e[:, 1:].max() * 0.5 + 1e-12)
    assert np.count_nonzero(yh[32:]) >= 0.95 * tail.size


def test_fp4v_prepare(oracle_mod):
    cfg = synth.CONFIGS[0]
    q, k, v = synth.make_inputs(cfg, 1)
    L, d = cfg.L - 100, cfg.d                                   # a ragged last block
    q, k, v = q[0, 0, :L], k[0, 0, :L], v[0, 0, :L]
    perm = synth.random_perms(1, 1, L, 3)[0, 0]
    P4 = oracle_mod.prepare_head_fp4v(q, k, v, perm)
    P8 = oracle_mod.prepare_head(q, k, v, perm)
    for n in ("q8", "k8", "q_scale", "k_scale", "v_mean"):
        assert np.array_equal(P4[n], P8[n]), n
    x = oracle_mod.bf16_to_f32(v).astype(np.float64)[perm]      # permuted rows
    nb = P4["v4"].shape[0]
    j = np.arange(128)
    tops = []
    for b in range(nb):
        n = min(128, L - 128 * b)
        r = (x[128 * b:128 * b + n].astype(np.float32) - P4["v_mean"][b][None, :]).astype(np.float64)  # [n, d]
        for c in range(d):
            e = P4["v_exp"][b, c].astype(int) - 127                  # [4]
            sc = 2.0 ** e[_group(j[:n])]
            y = r[:, c] / sc
            yh = oracle_mod.e2m1_decode(P4["v4"][b, c, :n])
            half = np.where(np.abs(y) < 2, 0.25, np.where(np.abs(y) < 4, 0.5, 1.0))
            assert np.all(np.abs(y - yh) <= half)
            assert np.all(P4["v4"][b, c, n:] == 0)
            for g in range(4):
                sel = _group(j[:n]) == g
                if np.any(r[sel, c] != 0):
                    tops.append(np.abs(yh[sel]).max())
    assert min(tops) >= 3.0                                       # each group's top lands on 3, 4 or 6


def test_fp4v_bytes_follow_dequantised_scores(oracle_mod):
    cfg = synth.CONFIGS[0]
    q, k, v = synth.make_inputs(cfg, 2)
    L, d, z_off = 300, cfg.d, 8
    q, k, v = q[0, 1, :L], k[0, 1, :L], v[0, 1, :L]
    perm = np.arange(L, dtype=np.int32)
    P4 = oracle_mod.prepare_head_fp4v(q, k, v, perm)
    _, codes, S, ph = oracle_mod.attention_head_fp4v(P4, L, z_off, want_bytes=True)
    qd = oracle_mod.e4m3_decode(P4["q8"][:L]) * np.repeat(P4["q_scale"], 128)[:L, None]
    kd = oracle_mod.e4m3_decode(P4["k8"]) * np.repeat(P4["k_scale"], 128)[:, None]
    z = (qd @ kd.T) * (np.log2(np.e) / np.sqrt(d))
    Lp = z.shape[1]
    z[:, L:] = -np.inf
    nb = Lp // 128
    run = np.maximum.accumulate(z.reshape(L, nb, 128).max(axis=2), axis=1)
    p = np.exp2(z - np.repeat(run, 128, axis=1) + z_off)
    ref = np.zeros_like(p)
    g = _group(np.arange(Lp) % 128)
    for b in range(nb):
        for gg in range(4):
            cols = np.nonzero((np.arange(Lp) // 128 == b) & (g == gg))[0]
            A = p[:, cols].max(axis=1)
            e = np.array([oracle_mod.e8m0_exp(a) for a in A])
            sc = 2.0 ** e[:, None]
            ref[:, cols] = np.where(e[:, None] > -127, _rne_e2m1(p[:, cols] / sc) * sc, 0.0)
    ph = ph.astype(np.float64)[:, :L]
    ref = ref[:, :L]
    same = ph == ref
    print("fp4 P: %.5f of the codes equal the float64 reference" % same.mean())
    assert same.mean() > 0.995
    # elsewhere one step apart (the reference sits at a rounding midpoint to
    # within the fp32 rounding of the score)
    step = np.maximum(np.abs(ref), np.abs(ph)) / 2
    assert np.all(np.abs(ph - ref)[~same] <= step[~same] * 1.001 + 1e-30)


def _uniform_inputs(L, d, seed):
    """Identical Q rows and identical K rows (every score equal, so P is
    exact: 2^z_off at every key), and V = block constant mu_b plus a residual
    whose values are E2M1 values times 2^-4, in (x, -x) pairs inside each key
    group of 32 consecutive slots (block means exactly mu_b) with every group
    reaching 6 * 2^-4."""
    rng = np.random.default_rng(seed)
    q = np.tile(rng.standard_normal(d), (L, 1))
    k = np.tile(rng.standard_normal(d), (L, 1))
    v = np.empty((L, d))
    for b0 in range(0, L, 128):
        n = min(128, L - b0)
        assert n % 32 == 0
        mu = rng.integers(-3, 4, size=d).astype(np.float64)
        res = np.zeros((n, d))
        for a in range(0, n, 32):                 # keys a .. a+31: two 16-key rows
            vals = rng.choice(MAGS, size=(16, d)) * rng.choice([-1.0, 1.0], size=(16, d))
            vals[0] = 6.0
            res[a:a + 16] = vals                  # keys a + t and a + 16 + t share the group a // 32
            res[a + 16:a + 32] = -vals
        v[b0:b0 + n] = mu[None, :] + res * 2.0 ** -4
    return _bf16(q), _bf16(k), _bf16(v), v


def test_fp4v_uniform_attention_is_exact(oracle_mod):
    L, d = 288, 64                                 # blocks of 128, 128 and 32 keys
    q, k, v, vf = _uniform_inputs(L, d, 4)
    assert np.array_equal(oracle_mod.bf16_to_f32(v).astype(np.float64), vf)
    perm = np.arange(L, dtype=np.int32)
    P4 = oracle_mod.prepare_head_fp4v(q, k, v, perm)
    O4 = oracle_mod.attention_head_fp4v(P4, L)
    exact = vf.mean(axis=0)
    np.testing.assert_allclose(O4, np.tile(exact, (L, 1)), rtol=1e-6, atol=1e-6)
    P8 = oracle_mod.prepare_head(q, k, v, perm)
    O8 = oracle_mod.attention_head(P8, L, prob_cast=1)
    np.testing.assert_allclose(O4, O8, rtol=1e-6, atol=1e-6)


@pytest.mark.parametrize("h", [0, 1])
def test_fp4v_band_of_exact_attention(oracle_mod, h):
    """Regression guard only (parity unpinned against fp64: the pages print
    no error for the 4-bit path)."""
    cfg = synth.CONFIGS[0]
    q, k, v = synth.make_inputs(cfg, 0)
    L = cfg.L
    perm = np.arange(L, dtype=np.int32)
    P4 = oracle_mod.prepare_head_fp4v(q[0, h], k[0, h], v[0, h], perm)
    O = oracle_mod.attention_head_fp4v(P4, L, rows=(0, 256))
    ref = oracle_mod.attention_f64(oracle_mod.bf16_to_f32(q[0, h]), oracle_mod.bf16_to_f32(k[0, h]),
                                   oracle_mod.bf16_to_f32(v[0, h]), rows=(0, 256))
    rel = np.linalg.norm(O - ref) / np.linalg.norm(ref)
    print("fp4 P V head %d: rel-L2 %.4f against fp64" % (h, rel))
    assert rel < 0.3
