"""Shared parity bars and the byte-flip accounting of the end-to-end error
(test helper module; not collected by pytest).

Bars.  Given the kernel's own fp32 scores S (dumped), every later step is
unique: the oracle must then reproduce the kernel's probability bytes bit
for bit and its output within rel-L2 1e-4 and max-abs 1e-3 * max|O|.  End to
end, against the oracle's exactly rounded scores, the stated output bar is
rel-L2 <= 1e-3 and max-abs <= 1e-2 * max|O_ref|.

Why the end-to-end comparison needs an accounting.  The FP8 matrix core does
not round its 128-term score sums exactly (its error is bounded in
test_fp8_matrix_core_sum_error_bound), so a probability byte whose
pre-rounding value lies next to a rounding midpoint can come out one code
apart.  That is a property of the scores, not of the softmax or P V
arithmetic.  The output is a weighted mean, O = sum_j w_j v_j / sum_j w_j,
with w_j = decode(byte_j) * 2^(m_b(j) - m_final) (the byte is relative to
the running maximum m_b of its block), so for two byte sets K (kernel) and E
(exact scores) the identity

    O_K - O_E = sum_j (w_K,j - w_E,j) (v_j - O_E) / sum_j w_K,j

holds exactly.  `flip_attribution` evaluates its right-hand side in float64
from the two byte sets and the dequantised values; the end-to-end check then
requires that (a) every byte difference is one code and (b) what remains of
the kernel's end-to-end deviation after subtracting the flip term is within
the given-S bar.  A case whose plain end-to-end error exceeds the output bar
is thereby shown to be entirely the one-code flips of the matrix core's
inexact sums, with the rest of the kernel's arithmetic held to the given-S
bar.  The plain output bar itself is asserted on the benchmark workloads'
full-size sampled rows (test_gpu_fullsize.py).
"""
import numpy as np

import oracle

REL_L2 = 1e-3
MAXABS = 1e-2
GIVEN_S_REL, GIVEN_S_MAXABS = 1e-4, 1e-3
# kernel byte mismatches (one code each) per dumped tile, against the
# oracle's exactly rounded scores
BYTE_MISMATCH_CAP = 5e-4


def rel_l2(a, b):
    return float(np.linalg.norm((a - b).ravel()) / np.linalg.norm(b.ravel()))


def max_rel(a, b):
    return float(np.abs(a - b).max() / np.abs(b).max())


def _block_running_max(S, coef, L):
    """Running maximum m_b of fp32(S * coef) over the valid keys of blocks
    0..b, per row (float32, as the oracle and the kernel take it)."""
    n, Lp = S.shape
    nb = Lp // 128
    valid = (np.arange(Lp) < L)[None, :]
    t = np.where(valid, (S.astype(np.float32) * coef.astype(np.float32)).astype(np.float32), -np.inf)
    return np.maximum.accumulate(t.reshape(n, nb, 128).max(axis=2), axis=1)


def _weights(S, p, coef, L):
    """w_j = p_j 2^(m_b(j) - m_final): p the decoded probability values
    (relative to the running maximum of their block) [n, Lp]."""
    m = _block_running_max(S, coef, L).astype(np.float64)
    scale = np.exp2(m - m[:, -1:])                        # [n, nb]
    return p.astype(np.float64) * np.repeat(scale, 128, axis=1)


def flip_attribution(S_K, by_K, S_E, by_E, coef, vhat, L, p_K=None, p_E=None):
    """Flip term of the end-to-end deviation for rows with kernel scores/bytes
    (S_K, by_K) and exact-score oracle scores/bytes (S_E, by_E), each
    [n, Lp]; coef [n, Lp] the fp32 score coefficient of every (row, key);
    vhat [Lp, d] the dequantised values in key order (float64).  The
    probability values are the E4M3 decodes of the bytes unless given
    (p_K, p_E: 4-bit values with their group scales).  Returns (delta [n, d],
    flips [n, Lp] int code differences)."""
    flips = by_K.astype(np.int32) - by_E.astype(np.int32)
    if p_K is None:
        p_K, p_E = oracle.e4m3_decode(by_K), oracle.e4m3_decode(by_E)
    wK, wE = _weights(S_K, p_K, coef, L), _weights(S_E, p_E, coef, L)
    lE, lK = wE.sum(axis=1), wK.sum(axis=1)
    OE = (wE @ vhat) / lE[:, None]
    dw = wK - wE
    delta = (dw @ vhat - dw.sum(axis=1)[:, None] * OE) / lK[:, None]
    return delta, flips


def vsmooth_coef(o, rows, d):
    """c_b = fp32(fp32(s_q s_k,b) C0) for every (row, key) of V-Smooth."""
    r0, r1 = rows
    nb = o["k_scale"].shape[0]
    qb = np.minimum(np.arange(r0, r1) // 128, nb - 1)
    cb = (o["q_scale"][qb][:, None].astype(np.float32) * o["k_scale"][None, :].astype(np.float32)).astype(np.float32)
    cb = (cb * np.float32(oracle.C0(d))).astype(np.float32)
    return np.repeat(cb, 128, axis=1)


def vsmooth_vhat(o):
    """Dequantised values mean + s_v * E4M3(code) [Lp, d] in key (slot) order."""
    nb, d, _ = o["v8"].shape
    r = oracle.e4m3_decode(o["v8"]).astype(np.float64)               # [nb, d, 128]
    vh = o["v_mean"][:, :, None].astype(np.float64) + o["v_scale"][:, :, None].astype(np.float64) * r
    return vh.transpose(0, 2, 1).reshape(nb * 128, d)


def sage_coef(o, rows, d):
    """c_ij = fp32(fp32(s_q,i C0) s_k,j/16) for every (row, key) of SAGE."""
    r0, r1 = rows
    sq = (o["q_scale"][r0:r1].astype(np.float32) * np.float32(oracle.C0(d))).astype(np.float32)
    ks = np.repeat(o["k_scale"].astype(np.float32), 16)
    return (sq[:, None] * ks[None, :]).astype(np.float32)


def sage_vhat(o):
    nb, d, _ = o["v8"].shape
    r = oracle.e4m3_decode(o["v8"]).astype(np.float64).transpose(0, 2, 1).reshape(nb * 128, d)
    return r * o["v_scale"][None, :].astype(np.float64)


def fp4_vhat(o):
    """Dequantised 4-bit values mean + 2^e E2M1(code) [Lp, d] in key order
    (group of in-block key kk: kk div 32)."""
    nb, d, _ = o["v4"].shape
    e = o["v_exp"].astype(np.int64)[..., np.arange(128) // 32] - 127          # [nb, d, 128]
    vh = o["v_mean"][:, :, None].astype(np.float64) + oracle.e2m1_decode(o["v4"]) * np.exp2(e)
    return vh.transpose(0, 2, 1).reshape(nb * 128, d)


def explain_fp4_rows(o, L, rows, S_K, codes_K):
    """Oracle side of the end-to-end check for 4-bit V-Smooth rows of one head
    (oracle.prepare_head_fp4v output `o`), given the kernel's dumped scores
    and E2M1 probability codes [n, Lp]: the kernel's codes equal the
    oracle's given the kernel's scores (one-code differences where
    v_exp_f32's last bit straddles a rounding midpoint, rate below 1e-4).
    The flip term uses the probability values with their group scales: a
    score error can move a group's largest probability across a power of
    two and so change the group's scale and all its codes at once, which
    the values account for.  Returns (ref, refS, delta, flips); the flips
    are left at zero (no one-code rule for 4-bit groups)."""
    d = o["q8"].shape[1]
    S_K = np.ascontiguousarray(S_K)
    ref, c_E, S_E, p_E = oracle.attention_head_fp4v(o, L, rows=rows, want_bytes=True)
    refS, c_S, _, p_S = oracle.attention_head_fp4v(o, L, rows=rows, want_bytes=True, scores=S_K)
    dd = c_S.astype(np.int32) - codes_K.astype(np.int32)
    assert (dd != 0).mean() <= 1e-4, "codes given the kernel's scores"
    n_changed = int((c_S != c_E).sum())
    delta, _ = flip_attribution(S_K, c_S, S_E, c_E, vsmooth_coef(o, rows, d), fp4_vhat(o), L, p_K=p_S, p_E=p_E)
    print("   4-bit: %d probability codes differ from the exact-score ones" % n_changed)
    return ref, refS, delta, np.zeros(c_S.shape, np.int32)


def check_explained(tag, got, ref, refS, delta, flips):
    """The end-to-end check on one set of rows (arrays [n, d] or stacked):
    given-S bar; every byte difference one code; the deviation left after
    subtracting the flip term within the given-S bar.  Returns (end-to-end
    rel-L2, max-abs/max, whether the plain output bar holds)."""
    rs, mas = rel_l2(got, refS), max_rel(got, refS)
    r, ma = rel_l2(got, ref), max_rel(got, ref)
    resid = got.astype(np.float64) - ref.astype(np.float64) - delta
    rr = float(np.linalg.norm(resid.ravel()) / np.linalg.norm(ref.ravel()))
    rm = float(np.abs(resid).max() / np.abs(ref).max())
    nflip = int((flips != 0).sum())
    within = r <= REL_L2 and ma <= MAXABS
    print("%s: end-to-end rel-L2 %.3g max-abs/max %.3g (%s the output bar) | given kernel S %.3g / %.3g | "
          "%d one-code flips; after the flip term %.3g / %.3g"
          % (tag, r, ma, "within" if within else "OUTSIDE", rs, mas, nflip, rr, rm))
    assert rs <= GIVEN_S_REL and mas <= GIVEN_S_MAXABS, (tag, rs, mas)
    assert np.abs(flips).max(initial=0) <= 1, tag
    assert rr <= GIVEN_S_REL and rm <= GIVEN_S_MAXABS, (tag, rr, rm)
    return r, ma, within


def explain_vsmooth_rows(o, L, rows, S_K, by_K, z_off=8, skip_lambda=0.0, prob_cast=0):
    """Oracle side of the end-to-end check for V-Smooth rows `rows` of one
    head (oracle.prepare_head output `o`), given the kernel's dumped scores
    and bytes [n, Lp] of those rows: the kernel's bytes must equal the
    oracle's given the kernel's scores.  Returns (ref, refS, delta, flips)."""
    d = o["q8"].shape[1]
    S_K = np.ascontiguousarray(S_K)
    ref, by_E, S_E, _ = oracle.attention_head(o, L, z_off, rows=rows, want_bytes=True, skip_lambda=skip_lambda,
                                              prob_cast=prob_cast)
    refS, by_S, _, _ = oracle.attention_head(o, L, z_off, rows=rows, want_bytes=True, scores=S_K,
                                             skip_lambda=skip_lambda, prob_cast=prob_cast)
    dd = by_S.astype(np.int32) - by_K.astype(np.int32)
    if prob_cast == 0:
        assert not dd.any(), "bytes given the kernel's scores"
    else:  # v_exp_f32's last bit may straddle an E4M3 midpoint: one code, rarely
        assert np.abs(dd).max() <= 1 and (dd != 0).mean() <= 1e-4
    coef = vsmooth_coef(o, rows, d)
    delta, flips = flip_attribution(S_K, by_K, S_E, by_E, coef, vsmooth_vhat(o), L)
    if skip_lambda > 0:
        flips = _rejection_flips(S_E, S_K, by_K, by_E, coef, L, skip_lambda, flips)
    return ref, refS, delta, flips


def _rejection_flips(S_E, S_K, by_K, by_E, coef, L, skip_lambda, flips):
    """Skip Softmax: a (row, block) whose rejection test fp32(t - m) <
    log2(lambda) is decided differently on the two sides changes all its
    bytes at once.  That is allowed only where the two sides' scores put the
    test on opposite sides of the threshold (the decision follows the
    scores); those entries are then left out of the one-code rule (the flip
    term still accounts for them)."""
    n, Lp = S_E.shape
    nb = Lp // 128
    zK = ~by_K.reshape(n, nb, 128).any(axis=2)
    zE = ~by_E.reshape(n, nb, 128).any(axis=2)
    differ = zK != zE
    if not differ.any():
        return flips
    thr = np.float32(oracle.skip_threshold(skip_lambda))

    def gaps(S):
        m = _block_running_max(S, coef, L)
        valid = (np.arange(Lp) < L)[None, :]
        t = np.where(valid, (S * coef).astype(np.float32), -np.inf).reshape(n, nb, 128).max(axis=2)
        mprev = np.concatenate([np.full((n, 1), -np.inf, np.float32), m[:, :-1]], axis=1)
        return (t - mprev).astype(np.float32)   # +inf on block 0: never rejected

    gE, gK = gaps(S_E), gaps(S_K)
    # the side whose bytes are all zero rejected the block; the other kept it
    assert np.all((gK[differ] < thr) == zK[differ]) and np.all((gE[differ] < thr) == zE[differ])
    out = flips.copy()
    out.reshape(n, nb, 128)[differ] = 0
    print("   %d (row, block) rejection decisions differ (threshold %.4g; gaps on the two sides within %.3g)"
          % (int(differ.sum()), float(thr), float(np.abs(gE[differ] - gK[differ]).max())))
    return out
