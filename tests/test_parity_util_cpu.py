"""The byte-flip accounting used by the GPU parity tests (parity_util),
checked on the CPU against the oracle itself: perturb the oracle's exactly
rounded scores by a relative amount like the FP8 matrix core's rounding,
let the oracle attend with the perturbed scores, and the flip term computed
in float64 from the two byte sets must equal the oracle's own change of
output (the oracle sums in another order and rounds to fp32, so to ~1e-6
relative).  With equal scores it must vanish."""
import os
import sys

import numpy as np
import pytest

import oracle
from bit_attention_video_smooth_amd import synth

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
from parity_util import _block_running_max, flip_attribution, vsmooth_coef, vsmooth_vhat  # noqa: E402


def _head(L, d, seed):
    cfg = synth.custom(1, 1, L, d)
    q, k, v = synth.make_inputs(cfg, seed)
    perm = synth.random_perms(1, 1, L, seed)
    return oracle.prepare_head(q[0, 0], k[0, 0], v[0, 0], perm[0, 0])


@pytest.mark.parametrize("L,d,seed,prob_cast", [(700, 64, 1, 0), (1000, 128, 2, 0), (300, 64, 3, 1)])
def test_flip_term_equals_oracle_change(oracle_mod, L, d, seed, prob_cast):
    o = _head(L, d, seed)
    ref, by_E, S_E, _ = oracle.attention_head(o, L, want_bytes=True, prob_cast=prob_cast)
    rng = np.random.default_rng(seed)
    S_K = (S_E.astype(np.float64) * (1 + 2.0 ** -11 * rng.standard_normal(S_E.shape))).astype(np.float32)
    refK, by_K, _, _ = oracle.attention_head(o, L, want_bytes=True, scores=S_K, prob_cast=prob_cast)
    flips = by_K.astype(int) - by_E.astype(int)
    assert (flips != 0).sum() > 20  # the perturbation does flip bytes
    assert np.abs(flips).max() <= 1
    delta, fl = flip_attribution(S_K, by_K, S_E, by_E, vsmooth_coef(o, (0, L), d), vsmooth_vhat(o), L)
    assert np.array_equal(fl, flips)
    change = refK.astype(np.float64) - ref.astype(np.float64)
    err = np.linalg.norm(change - delta) / np.linalg.norm(ref)
    rel_change = np.linalg.norm(change) / np.linalg.norm(ref)
    print("L=%d d=%d: %d flips, oracle change %.3g, unexplained %.3g" % (L, d, (flips != 0).sum(), rel_change, err))
    assert err <= 2e-6 and err <= 0.01 * rel_change


def test_flip_term_vanishes_without_flips(oracle_mod):
    L, d = 500, 128
    o = _head(L, d, 4)
    _, by, S, _ = oracle.attention_head(o, L, want_bytes=True)
    delta, fl = flip_attribution(S, by, S, by, vsmooth_coef(o, (0, L), d), vsmooth_vhat(o), L)
    assert not fl.any() and np.abs(delta).max() == 0.0


def test_running_max_matches_a_plain_loop(oracle_mod):
    L, d = 300, 64
    o = _head(L, d, 5)
    _, _, S, _ = oracle.attention_head(o, L, want_bytes=True)
    coef = vsmooth_coef(o, (0, L), d)
    m = _block_running_max(S, coef, L)
    n, Lp = S.shape
    for i in (0, 17, n - 1):
        run = -np.inf
        for b in range(Lp // 128):
            t = -np.inf
            for j in range(b * 128, min(L, b * 128 + 128)):
                t = max(t, np.float32(S[i, j]) * np.float32(coef[i, j]))
            run = max(run, t)
            assert m[i, b] == np.float32(run)


def test_skip_softmax_decision_flips_accounted(oracle_mod):
    """With Skip Softmax, perturbed scores also move rejection decisions that
    sit at the threshold; explain_vsmooth_rows exempts exactly those
    (row, block) pairs from the one-code rule, and the flip term still
    equals the oracle's change of output."""
    from parity_util import explain_vsmooth_rows
    L, d, lam = 1500, 64, 0.3
    o = _head(L, d, 6)
    S_E = oracle.attention_head(o, L, want_bytes=True, skip_lambda=lam)[2]
    rng = np.random.default_rng(6)
    S_K = (S_E.astype(np.float64) * (1 + 2.0 ** -9 * rng.standard_normal(S_E.shape))).astype(np.float32)
    outK, by_K, _, _ = oracle.attention_head(o, L, want_bytes=True, scores=S_K, skip_lambda=lam)
    ref, refS, delta, flips = explain_vsmooth_rows(o, L, (0, L), S_K, by_K, skip_lambda=lam)
    by_E = oracle.attention_head(o, L, want_bytes=True, skip_lambda=lam)[1]
    raw = by_K.astype(int) - by_E.astype(int)
    assert np.abs(raw).max() > 1           # some decision did flip
    assert np.abs(flips).max() <= 1        # and only those were exempted
    change = outK.astype(np.float64) - ref.astype(np.float64)
    assert np.linalg.norm(change - delta) / np.linalg.norm(ref) <= 2e-6


@pytest.mark.parametrize("L,d,seed", [(700, 64, 8), (1000, 128, 9)])
def test_fp4_flip_term_equals_oracle_change(oracle_mod, L, d, seed):
    """The 4-bit form (probability values with their group scales): perturbed
    scores change codes and some group scales; the flip term still equals
    the oracle's own change of output."""
    from parity_util import explain_fp4_rows
    cfg = synth.custom(1, 1, L, d)
    q, k, v = synth.make_inputs(cfg, seed)
    perm = synth.random_perms(1, 1, L, seed)
    o = oracle.prepare_head_fp4v(q[0, 0], k[0, 0], v[0, 0], perm[0, 0])
    S_E = oracle.attention_head_fp4v(o, L, want_bytes=True)[2]
    rng = np.random.default_rng(seed)
    S_K = (S_E.astype(np.float64) * (1 + 2.0 ** -11 * rng.standard_normal(S_E.shape))).astype(np.float32)
    outK, c_K, _, _ = oracle.attention_head_fp4v(o, L, want_bytes=True, scores=S_K)
    ref, refS, delta, _ = explain_fp4_rows(o, L, (0, L), S_K, c_K)
    change = outK.astype(np.float64) - ref.astype(np.float64)
    assert np.linalg.norm(change) / np.linalg.norm(ref) > 1e-4
    assert np.linalg.norm(change - delta) / np.linalg.norm(ref) <= 2e-6
