"""Pins of the CPU oracle against what the VC-Attention pages and mathematics
fix.  None of these compares the oracle with itself: each check uses a
closed form, a library routine, a printed number (tests/golden), brute
force on tiny inputs, or an invariant of the method."""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

from bit_attention_video_smooth_amd import synth

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_constants.json")))


def _positive_code_values():
    """The 126 positive finite E4M3FN values listed from the format: 7
    subnormals k*2^-9 and 15 binades of 8 mantissa steps, capped at 448."""
    vals = [k * 2.0 ** -9 for k in range(1, 8)]
    for e in range(-6, 9):
        for m in range(8):
            v = (1 + m / 8) * 2.0 ** e
            if v <= 448:
                vals.append(v)
    return np.array(vals)


# ---------------------------------------------------------------- codec ----

def test_e4m3_decode_matches_library_and_format(oracle_mod):
    codes = np.arange(256, dtype=np.uint8)
    dec = oracle_mod.e4m3_decode(codes)
    lib = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    nan = np.isnan(lib)
    assert list(np.nonzero(nan)[0]) == [0x7F, 0xFF]
    assert np.isnan(dec[nan]).all()
    assert np.array_equal(dec[~nan], lib[~nan])
    pos = _positive_code_values()
    assert np.array_equal(dec[1:0x7F], pos)
    assert dec[0x7E] == 448.0 and dec[0x08] == 2.0 ** -6 and dec[0x01] == 2.0 ** -9


def _nearest_code(x):
    """Independent encoder: nearest value in the sorted code table, ties to
    the even code, saturating at 448."""
    table = np.concatenate([[0.0], _positive_code_values()])  # index == code
    a = np.minimum(np.abs(x.astype(np.float64)), 448.0)
    hi = np.clip(np.searchsorted(table, a, side="left"), 1, len(table) - 1)
    lo = hi - 1
    dlo = a - table[lo]
    dhi = table[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    code = np.where(a == table[hi], hi, code).astype(np.uint8)
    sign = (np.signbit(x)).astype(np.uint8) << 7
    return code | sign


def test_e4m3_encode_dense_ties_and_library(oracle_mod):
    # every (sign, exponent, top 7 mantissa bits) with |x| <= 448, crossed with
    # low-16-bit patterns that make exact ties and near-ties at every guard bit
    hi16 = np.arange(0, 0x43E0 + 1, dtype=np.uint32)
    lows = np.array([0, 1, 0x7FFF, 0x8000, 0x8001, 0xFFFF, 0x4000, 0xC000], np.uint32)
    u = (hi16[:, None] << 16 | lows[None, :]).ravel()
    u = np.concatenate([u, u | np.uint32(0x80000000)])
    x = u.view(np.float32)
    x = x[np.abs(x) <= 448.0]
    rnd = np.random.default_rng(0).uniform(-448, 448, 2_000_000).astype(np.float32)
    x = np.concatenate([x, rnd, np.float32([448.0, -448.0, 2.0 ** -10, 3 * 2.0 ** -10, 0.0])])
    got = oracle_mod.e4m3_encode(x)
    assert np.array_equal(got, _nearest_code(x))
    lib = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, lib)


def test_e4m3_saturates(oracle_mod):
    x = np.float32([449.0, 464.0, 1e6, -1e30, 3.0e38])
    assert list(oracle_mod.e4m3_encode(x)) == [0x7E, 0x7E, 0x7E, 0xFE, 0x7E]


def test_powers_of_two_map_to_8k_plus_56(oracle_mod):
    g = GOLD["e4m3_log_map"]
    for kk in range(-6, 9):
        assert oracle_mod.e4m3_encode(np.float32(2.0 ** kk)).item() == g["slope"] * kk + g["offset"]


# ------------------------------------------------------------- ExpCast ----

def test_expcast_integer_scores(oracle_mod):
    # p = 2^z with integer z: the byte is exactly 8(z + z_off) + 56 (beta rounds away)
    for z_off in (0, 8):
        z = np.arange(-6 - z_off, 1, dtype=np.float32)
        got = oracle_mod.expcast_z(z, z_off)
        assert np.array_equal(got, (8 * (z + z_off) + 56).astype(np.uint8))


def test_expcast_constants(oracle_mod):
    assert oracle_mod.KB(8) == np.float32(56 + GOLD["expcast_beta"]["value"] + 64)
    assert np.float32(oracle_mod.KB(8)).view(np.uint32) == 0x42EF4CCD
    assert oracle_mod.C0(128) == np.float32(math.log2(math.e) / math.sqrt(128))


def _exp_then_cast(z, z_off):
    p = np.exp2(z.astype(np.float64) + z_off).astype(np.float32)
    return torch.from_numpy(p).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


@pytest.mark.parametrize("octave", [1, 2, 3, 5, 9])
def test_expcast_agreement_per_doubling(oracle_mod, octave):
    g = GOLD["expcast_agreement_per_doubling"]
    z = np.linspace(-octave, -octave + 1, 400_001, endpoint=False).astype(np.float32)
    a = oracle_mod.expcast_z(z, 8).astype(int)
    b = _exp_then_cast(z, 8).astype(int)
    agree = np.mean(a == b)
    assert abs(agree - g["value"]) < 0.0015, agree
    assert np.abs(a - b).max() <= g["rest_within_codes"]


def _log2_error(oracle_mod, z, z_off=8):
    by = oracle_mod.expcast_z(z, z_off)
    return np.log2(oracle_mod.e4m3_decode(by)) - (z.astype(np.float64) + z_off)


def test_expcast_error_range_and_centering(oracle_mod):
    # normal range of the P code (p >= 2^-6 after the z_off shift)
    z = np.linspace(-14, 0, 2_000_001).astype(np.float32)
    err = _log2_error(oracle_mod, z)
    lo, hi = err.min(), err.max()
    assert -0.1070 < lo < -0.1055 and 0.1030 < hi < 0.1045, (lo, hi)
    assert abs((lo + hi) / 2) < 0.0025  # beta centres the error
    delta = hi - lo
    worst_tv = math.tanh(delta * math.log(2) / 4)
    assert worst_tv <= GOLD["expcast_tv_bound"]["value"]
    assert worst_tv > 0.0360  # the bound is tight: the pages' 3.64%


def _tv(p, q):
    return 0.5 * np.abs(p / p.sum() - q / q.sum()).sum()


def test_expcast_two_level_row_reaches_bound(oracle_mod):
    z = np.linspace(-6, 0, 600_001).astype(np.float32)
    err = _log2_error(oracle_mod, z)
    za, zb = z[np.argmax(err)], z[np.argmin(err)]
    R = 2.0 ** (err.max() - err.min())
    w = 1 / (1 + math.sqrt(R))  # mass fraction on the over-estimated level
    # build a row: n_a copies of za, n_b of zb with exact masses in ratio w:(1-w)
    pa, pb = 2.0 ** float(za), 2.0 ** float(zb)
    n_a = 1000
    n_b = int(round(n_a * pa * (1 - w) / (w * pb)))
    row = np.concatenate([np.full(n_a, za), np.full(n_b, zb)]).astype(np.float32)
    exact = np.exp2(row.astype(np.float64))
    approx = oracle_mod.e4m3_decode(oracle_mod.expcast_z(row, 8))
    tv = _tv(exact, approx)
    assert abs(tv - math.tanh((err.max() - err.min()) * math.log(2) / 4)) < 2e-4
    assert tv <= GOLD["expcast_tv_bound"]["value"] + 2e-4


@pytest.mark.parametrize("z_off,sigma", [(8, 0.5), (8, 2.0), (8, 3.0), (0, 2.0), (0, 3.0)])
def test_expcast_random_rows_tv_bound(oracle_mod, z_off, sigma):
    rng = np.random.default_rng(int(sigma * 10) + z_off)
    for _ in range(20):
        s = rng.normal(0, sigma, 4096)
        z = (s - s.max()).astype(np.float32)
        exact = np.exp2(z.astype(np.float64))
        approx = oracle_mod.e4m3_decode(oracle_mod.expcast_z(z, z_off))
        under = exact * 2.0 ** z_off < 2.0 ** -6
        U = exact[under].sum() / exact.sum()
        assert _tv(exact, approx) <= GOLD["expcast_tv_bound"]["value"] + U + 1e-12


def test_expcast_clamps_at_zero(oracle_mod):
    z = np.float32([-20, -100, -1e6])
    assert list(oracle_mod.expcast_z(z, 8)) == [0, 0, 0]


# ------------------------------------------------------------ SplitMix64 --

def test_splitmix64_vectors(oracle_mod):
    v = GOLD["splitmix64_vectors"]
    assert [oracle_mod.splitmix64(0, i) for i in range(4)] == [int(x, 16) for x in v["seed0"]]
    assert [oracle_mod.splitmix64(1234567, i) for i in range(3)] == [int(x) for x in v["seed1234567"]]


def test_kmeans_init_indices_distinct_in_strata(oracle_mod):
    for L, k in [(1024, 8), (1000, 7), (130, 2), (5, 5), (75600, 591)]:
        idx = oracle_mod.kmeans_init_indices(L, k, 12345)
        assert len(set(idx.tolist())) == k
        for c, j in enumerate(idx):
            assert c * L // k <= j < (c + 1) * L // k


# ---------------------------------------------------------------- k-means --

def _bf16(x):
    return synth.f32_to_bf16_bits(np.asarray(x, np.float32))


def test_kmeans_objective_monotone_and_means(oracle_mod):
    cfg = synth.CONFIGS[0]
    q, k, v = synth.make_inputs(cfg, 0)
    vh = v[0, 1]
    a, C, hist = oracle_mod.kmeans(vh, 8, 8, 7, history=True)
    assert np.all(np.diff(hist) <= 1e-9 * hist[0])
    x = oracle_mod.bf16_to_f32(vh).astype(np.float64)
    for c in range(8):
        mem = x[a == c]
        if len(mem):
            assert np.array_equal(C[c], mem.mean(axis=0).astype(np.float32))
    # the assignment is a nearest-centroid assignment of the previous centroids,
    # so J after the update cannot exceed what brute force says for this a
    J = ((x - C[a].astype(np.float64)) ** 2).sum()
    assert abs(J - hist[-1]) <= 1e-9 * J


def test_kmeans_brute_force_optimum_tiny(oracle_mod):
    rng = np.random.default_rng(3)
    for trial in range(6):
        L, d, k = 9, 2, 3
        centers = rng.normal(0, 5, (k, d))
        pts = centers[rng.integers(0, k, L)] + rng.normal(0, 0.3, (L, d))
        xb = _bf16(pts)
        x = oracle_mod.bf16_to_f32(xb).astype(np.float64)
        best = math.inf
        for lab in itertools.product(range(k), repeat=L):
            lab = np.array(lab)
            J = sum(((x[lab == c] - x[lab == c].mean(0)) ** 2).sum() for c in range(k) if (lab == c).any())
            best = min(best, J)
        a, C, J = oracle_mod.kmeans(xb, k, 10, 100 + trial)
        assert J >= best - 1e-9
        # well separated clusters: Lloyd from stratified seeds reaches the optimum
        # whenever every initial centroid lands in a different true cluster
        init = oracle_mod.kmeans_init_indices(L, k, 100 + trial)
        true_lab = np.argmin(((x[:, None, :] - centers[None]) ** 2).sum(-1), axis=1)
        if len(set(true_lab[init].tolist())) == k:
            assert abs(J - best) <= 1e-9 * max(best, 1)


def test_kmeans_recovers_separated_clusters(oracle_mod):
    rng = np.random.default_rng(5)
    k, d, per = 6, 16, 50
    centers = rng.normal(0, 20, (k, d))
    lab = np.repeat(np.arange(k), per)
    pts = centers[lab] + rng.normal(0, 0.1, (k * per, d))
    # strata of the init are contiguous index ranges, one per true cluster
    a, C, J = oracle_mod.kmeans(_bf16(pts), k, 5, 1)
    # same partition up to relabelling
    pairs = set(zip(a.tolist(), lab.tolist()))
    assert len(pairs) == k


def test_stable_perm_matches_library_sort(oracle_mod):
    rng = np.random.default_rng(0)
    a = rng.integers(0, 37, 5000).astype(np.int32)
    p = oracle_mod.stable_perm(a, 37)
    assert np.array_equal(p, np.argsort(a, kind="stable"))


# ---------------------------------------------------------- quantisation --

def _head(cfg_idx=0, h=0, seed=0):
    cfg = synth.CONFIGS[cfg_idx]
    q, k, v = synth.make_inputs(cfg, seed)
    return q[0, h], k[0, h], v[0, h]


@pytest.mark.parametrize("v_mode", [0, 1])
def test_prepare_invariants(oracle_mod, v_mode):
    cfg = synth.custom(1, 1, 300, 64)
    q, k, v = (a[0, 0] for a in synth.make_inputs(cfg, 11))
    L, d = q.shape
    perm = synth.random_perms(1, 1, L, 4)[0, 0]
    P = oracle_mod.prepare_head(q, k, v, perm, smooth_k=1, v_mode=v_mode)
    f = oracle_mod.bf16_to_f32
    kb = f(k).astype(np.float64).mean(0).astype(np.float32)
    assert np.array_equal(P["kbar"], kb)
    nb = 3
    for b in range(nb):
        n = min(128, L - 128 * b)
        sl = slice(128 * b, 128 * b + n)
        # Q: original order, scalar scale, max element at the top code
        qb = f(q[sl])
        A = np.abs(qb).max()
        assert P["q_scale"][b] == np.float32(A / np.float32(448))
        codes = P["q8"][sl]
        assert (codes & 0x7F).max() == 0x7E
        deq = oracle_mod.e4m3_decode(codes) * np.float64(P["q_scale"][b])
        assert np.all(np.abs(deq - qb) <= np.abs(qb) * 2 ** -4 + 2 ** -9 * P["q_scale"][b] + 1e-30)
        assert not P["q8"][128 * b + n:128 * (b + 1)].any()
        # V: exact mean of the permuted block, residual codes
        vb = f(v[perm[sl]]).astype(np.float64)
        mu = vb.mean(0).astype(np.float32)
        assert np.array_equal(P["v_mean"][b], mu)
        r = (vb.astype(np.float32) - mu).astype(np.float64)
        Ac = np.abs(r).max(0)
        s = P["v_scale"][b]
        if v_mode == 0:
            assert np.array_equal(s, (Ac.astype(np.float32) / np.float32(448)).astype(np.float32))
        else:
            e = np.log2(s.astype(np.float64))
            assert np.array_equal(e, np.round(e))
            assert np.all(Ac <= 448 * s) and np.all(448 * s < 2 * Ac)
        deq = oracle_mod.e4m3_decode(P["v8"][b][:, :n]).T * s.astype(np.float64)
        assert np.all(np.abs(deq - r) <= np.abs(r) * 2 ** -4 + 2 ** -9 * s + 1e-30)
        assert not P["v8"][b][:, n:].any()
    # bits per element of the stored mean: 32 bits / 128 tokens
    assert P["v_mean"].dtype.itemsize * 8 / 128 == 0.25


def test_zero_block_quantises_to_zero(oracle_mod):
    L, d = 256, 64
    z = np.zeros((L, d), np.uint16)
    rnd = _bf16(np.random.default_rng(0).normal(size=(L, d)))
    perm = np.arange(L, dtype=np.int32)
    P = oracle_mod.prepare_head(z, z, z, perm)
    assert not P["q8"].any() and not P["k8"].any() and not P["v8"].any()
    assert not P["q_scale"].any() and not P["v_scale"].any()
    out = oracle_mod.attention_head(P, L)
    assert np.all(out == 0)
    P = oracle_mod.prepare_head(rnd, rnd, z, perm)
    assert np.all(oracle_mod.attention_head(P, L) == 0)


# ------------------------------------------------------------ attention --

@pytest.mark.parametrize("L,d", [(1024, 64), (300, 64), (200, 128), (129, 32)])
def test_mean_restore_algebra_is_exact(oracle_mod, L, d):
    """Quantisation off, exact exp2: the blockwise loop with mean restore from
    the per-block row sums equals softmax attention, for any block means."""
    rng = np.random.default_rng(L + d)
    qf = rng.normal(size=(L, d))
    kf = rng.normal(size=(L, d)) + rng.normal(0, 0.5, d)
    vf = rng.normal(size=(L, d)) * 2
    perm = rng.permutation(L)
    nb = (L + 127) // 128
    for means in (np.zeros((nb, d), np.float32), rng.normal(0, 3, (nb, d)).astype(np.float32)):
        ex = oracle_mod.attention_exact_blockwise(qf, kf[perm], vf[perm], means)
        ref = oracle_mod.attention_f64(qf, kf, vf)
        assert np.abs(ex - ref).max() <= 4e-7 * np.abs(ref).max()


def test_joint_permutation_invariance(oracle_mod):
    rng = np.random.default_rng(1)
    L, d = 500, 64
    q, k, v = rng.normal(size=(3, L, d))
    p = rng.permutation(L)
    a = oracle_mod.attention_f64(q, k, v)
    b = oracle_mod.attention_f64(q, k[p], v[p])
    assert np.abs(a - b).max() < 1e-13


def _rel(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def test_quantised_oracle_error_band_tiny(oracle_mod):
    """Quantised vs fp64: the pages print no bound for the output error
    (parity unpinned); this is a regression guard.  Both the identity and the
    k-means permutation must land in the same band."""
    cfg = synth.CONFIGS[0]
    q, k, v = synth.make_inputs(cfg, 0)
    f = oracle_mod.bf16_to_f32
    for h in range(cfg.H):
        L = cfg.L
        ref = oracle_mod.attention_f64(f(q[0, h]), f(k[0, h]), f(v[0, h]))
        a, C, J = oracle_mod.kmeans(v[0, h], 8, 8, oracle_mod.head_seed(0, 0, h, cfg.H))
        for perm in (oracle_mod.stable_perm(a, 8), np.arange(L, dtype=np.int32)):
            P = oracle_mod.prepare_head(q[0, h], k[0, h], v[0, h], perm)
            e8 = _rel(oracle_mod.attention_head(P, L, 8), ref)
            e0 = _rel(oracle_mod.attention_head(P, L, 0), ref)
            assert e8 < 6e-2
            assert e8 < e0  # z_off = 8 keeps the tail the literal offset underflows


def test_quantised_matches_exact_when_values_exact(oracle_mod):
    """Powers-of-two inputs that E4M3 holds exactly and constant V blocks:
    then V-Smooth's residual is 0 and the output is the row-sum-weighted mean,
    i.e. the block mean exactly."""
    L, d = 256, 64
    rng = np.random.default_rng(2)
    q = _bf16(2.0 ** rng.integers(-3, 2, (L, d)) * rng.choice([-1, 1], (L, d)))
    k = _bf16(2.0 ** rng.integers(-3, 2, (L, d)) * rng.choice([-1, 1], (L, d)))
    val = rng.normal(size=d).astype(np.float32)
    v = _bf16(np.broadcast_to(val, (L, d)))
    P = oracle_mod.prepare_head(q, k, v, np.arange(L, dtype=np.int32))
    assert not P["v8"].any()
    out = oracle_mod.attention_head(P, L)
    assert np.allclose(out, oracle_mod.bf16_to_f32(v)[0], rtol=1e-6, atol=0)


def _block_energy_removed(x, order, blk=128):
    xs = x[order]
    L = len(xs)
    res = 0.0
    for s in range(0, L, blk):
        blkv = xs[s:s + blk]
        res += ((blkv - blkv.mean(0)) ** 2).sum()
    return 1 - res / (xs ** 2).sum()


def test_block_energy_ordering_direction(oracle_mod):
    """The pages: sequence order < static cube < sorted (8% / 12% / 36%).
    Synthetic data: check the direction."""
    g = GOLD["block_energy_removed"]
    assert g["sequence_order"] < g["static_cube"] < g["after_sorting"]
    cfg = synth.CONFIGS[0]
    _, _, v = synth.make_inputs(cfg, 0)
    T, Hg, W = cfg.grid
    t, h, w = np.meshgrid(np.arange(T), np.arange(Hg), np.arange(W), indexing="ij")
    j = ((t * Hg + h) * W + w).ravel()
    cube = np.lexsort(((w // 8).ravel(), (h // 8).ravel(), (t // 2).ravel()))
    cube_order = j[cube]
    for hh in range(cfg.H):
        x = oracle_mod.bf16_to_f32(v[0, hh]).astype(np.float64)
        a, C, J = oracle_mod.kmeans(v[0, hh], 8, 8, oracle_mod.head_seed(0, 0, hh, cfg.H))
        e_seq = _block_energy_removed(x, np.arange(cfg.L))
        e_cube = _block_energy_removed(x, cube_order)
        e_km = _block_energy_removed(x, oracle_mod.stable_perm(a, 8))
        assert e_seq < e_cube < e_km, (e_seq, e_cube, e_km)


def test_oracle_bytes_are_expcast_of_scores(oracle_mod):
    """The bytes the attention loop uses are ExpCast of its own S with the
    per-block running max: check the first block of every row directly."""
    cfg = synth.custom(1, 1, 256, 64)
    q, k, v = (a[0, 0] for a in synth.make_inputs(cfg, 5))
    P = oracle_mod.prepare_head(q, k, v, np.arange(256, dtype=np.int32))
    out, by, S, y = oracle_mod.attention_head(P, 256, rows=(0, 16), want_bytes=True)
    qd = oracle_mod.e4m3_decode(P["q8"][:16])
    kd = oracle_mod.e4m3_decode(P["k8"][:128])
    S0 = (qd @ kd.T).astype(np.float32)
    assert np.array_equal(S0, S[:, :128])
    cb = np.float32(np.float32(P["q_scale"][0] * P["k_scale"][0]) * oracle_mod.C0(64))
    t = (S0.max(1) * cb).astype(np.float32)
    krow = (oracle_mod.KB(8) - np.float32(8) * t).astype(np.float32)
    ref = oracle_mod.expcast(S0, np.float32(8) * cb, krow[:, None])
    assert np.array_equal(ref, by[:, :128])
    assert (by[:, :128].max(1) == 120).all()  # the row max lands on 2^8
    assert np.array_equal(np.clip(np.rint(y[:, :128].astype(np.float64)), 0, 126).astype(np.uint8), by[:, :128])


def test_synth_bf16_rounding_matches_library():
    x = np.random.default_rng(0).normal(0, 30, 1_000_000).astype(np.float32)
    x[:4] = [0.0, -0.0, 1.00390625, 1.01171875]  # exact bf16 ties
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(synth.f32_to_bf16_bits(x), ref)


def test_given_scores_path_reproduces_exact_path(oracle_mod):
    """Feeding the oracle its own exactly rounded scores through the `scores`
    input reproduces its output and bytes bit for bit (the input only replaces
    the dot product; every later step is shared)."""
    cfg = synth.custom(1, 1, 700, 64)
    q, k, v = synth.make_inputs(cfg, 3)
    perm = synth.random_perms(1, 1, 700, 3)[0, 0]
    o = oracle_mod.prepare_head(q[0, 0], k[0, 0], v[0, 0], perm)
    out, by, S, _ = oracle_mod.attention_head(o, 700, 8, want_bytes=True)
    out2, by2, S2, _ = oracle_mod.attention_head(o, 700, 8, want_bytes=True, scores=S[:700].copy())
    assert np.array_equal(out, out2) and np.array_equal(by, by2) and np.array_equal(S, S2)
    # and a perturbed score (made the row's new maximum) changes only its row
    S3 = S.copy()
    S3[5, 10] = 4.0 * np.abs(S[5]).max() + 1.0
    _, by3, _, _ = oracle_mod.attention_head(o, 700, 8, want_bytes=True, scores=S3)
    assert not np.array_equal(by3[5], by[5]) and np.array_equal(by3[6:], by[6:])


# ---------------------------------------------------- Skip Softmax (BLASST) --
# [TRT] "Sparse Attention with Skip Softmax": query row i drops KV block j
# when exp(m~ - m) falls below the threshold lambda, with m~ the largest score
# of the block and m the running maximum; a dropped block contributes no
# exponentials and no PV product.

def _skip_brute(qf, kf_perm, v_perm, lam):
    """fp64 softmax attention over the kept blocks only, with the rejection
    rule evaluated as printed, in natural-log units, blocks in ascending
    order.  Returns (O, kept [L, nb])."""
    L, d = qf.shape
    nb = (L + 127) // 128
    s = qf @ kf_perm.T / math.sqrt(d)
    kept = np.zeros((L, nb), bool)
    out = np.empty((L, d))
    for i in range(L):
        m = -np.inf
        for b in range(nb):
            mt = s[i, 128 * b:128 * b + 128].max()
            if m > -np.inf and math.exp(mt - m) < lam:
                continue
            kept[i, b] = True
            m = max(m, mt)
        cols = np.concatenate([np.arange(128 * b, min(L, 128 * b + 128)) for b in np.nonzero(kept[i])[0]])
        w = np.exp(s[i, cols] - s[i, cols].max())
        out[i] = w @ v_perm[cols] / w.sum()
    return out, kept


@pytest.mark.parametrize("lam", [0.05, 0.3])
def test_skip_softmax_exact_blockwise_matches_brute_force(oracle_mod, lam):
    """Quantisation off: the blockwise loop with Skip Softmax equals softmax
    attention restricted to the blocks the printed rule keeps."""
    rng = np.random.default_rng(17)
    L, d = 900, 64
    qf = rng.normal(size=(L, d))
    # keys whose blocks differ in score scale, so that some are rejected
    kf = rng.normal(size=(L, d)) * np.repeat(rng.uniform(0.2, 1.6, (L + 127) // 128), 128)[:L, None]
    vf = rng.normal(size=(L, d)) * 2
    nb = (L + 127) // 128
    means = rng.normal(0, 1, (nb, d)).astype(np.float32)
    lam_eff = 2.0 ** float(oracle_mod.skip_threshold(lam))  # the fp32 threshold the loop uses
    ref, kept = _skip_brute(qf, kf, vf, lam_eff)
    frac = 1 - kept.mean()
    assert 0.05 < frac < 0.95, frac
    got = oracle_mod.attention_exact_blockwise(qf, kf, vf, means, skip_lambda=lam)
    assert np.abs(got - ref).max() <= 4e-7 * np.abs(ref).max()
    # and lambda = 0 keeps every block
    full = oracle_mod.attention_exact_blockwise(qf, kf, vf, means)
    assert np.abs(full - oracle_mod.attention_f64(qf, kf, vf)).max() <= 4e-7 * np.abs(full).max()


def test_skip_softmax_quantised_rejects_by_the_printed_rule(oracle_mod):
    """Quantised path: the rejected (row, block) pairs are those where
    exp(m~ - m) < lambda with m~ and m from the same scores in natural-log
    units; a rejected block gets bytes 0, and every kept block keeps exactly
    the bytes of the run without rejection (a rejected block never moves the
    running maximum).  lambda = 0 changes nothing."""
    cfg = synth.custom(1, 1, 1000, 64)
    q, k, v = synth.make_inputs(cfg, 21)
    q, k, v = q[0, 0], k[0, 0], v[0, 0]
    # stretch the keys of some blocks so that their scores fall behind
    kf = oracle_mod.bf16_to_f32(k) * np.repeat(np.random.default_rng(2).uniform(0.2, 1.5, 8), 128)[:1000, None]
    k = synth.f32_to_bf16_bits(kf.astype(np.float32))
    perm = np.arange(1000, dtype=np.int32)
    o = oracle_mod.prepare_head(q, k, v, perm)
    L, lam = 1000, 0.3
    out0, by0, S0, _ = oracle_mod.attention_head(o, L, want_bytes=True)
    outz, byz, _, _ = oracle_mod.attention_head(o, L, want_bytes=True, skip_lambda=0.0)
    assert np.array_equal(out0, outz) and np.array_equal(by0, byz)
    out1, by1, S1, _ = oracle_mod.attention_head(o, L, want_bytes=True, skip_lambda=lam)
    assert np.array_equal(S0, S1)
    nb = 8
    cb = (np.float32(o["q_scale"][np.arange(L) // 128][:, None] * o["k_scale"][None, :])
          * oracle_mod.C0(64)).astype(np.float32)                          # [L, nb]
    Sv = S0[:, :L].astype(np.float64)
    bmax = np.stack([Sv[:, 128 * b:min(L, 128 * b + 128)].max(1) for b in range(nb)], 1)
    t = (bmax * cb).astype(np.float32).astype(np.float64)                 # log2 units
    m_before = np.concatenate([np.full((L, 1), -np.inf), np.maximum.accumulate(t, 1)[:, :-1]], 1)
    with np.errstate(invalid="ignore"):
        rule = np.exp((t - m_before) * math.log(2.0)) < lam               # natural-log units
    near = np.abs((t - m_before) - math.log2(lam)) < 1e-5
    live = by0.reshape(L, nb, 128).any(2)          # blocks with a nonzero byte when nothing is rejected
    rej = ~by1.reshape(L, nb, 128).any(2) & live
    assert np.all((rej == rule) | near | ~live)
    assert 0.02 < rule.mean() < 0.9, rule.mean()
    kept = np.repeat(~rule, 128, axis=1)
    assert np.array_equal(by1[kept], by0[kept])
    assert not by1[~kept].any()


# ------------------------------------------------- exp-then-cast (the baseline) --

def test_exp_then_cast_bytes_are_library_cast_of_exp2(oracle_mod):
    """prob_cast=1: every byte is the library's E4M3 cast of 2^z, z = S c_b -
    m' + z_off (computed here in fp64 from the oracle's own S and scales); the
    row max lands on 2^8; and against ExpCast the bytes agree in the
    proportion the pages give per doubling (79.6%), differing by one code
    otherwise (on bytes above the subnormal range)."""
    cfg = synth.custom(1, 1, 256, 64)
    q, k, v = (a[0, 0] for a in synth.make_inputs(cfg, 9))
    P = oracle_mod.prepare_head(q, k, v, np.arange(256, dtype=np.int32))
    out, by, S, z = oracle_mod.attention_head(P, 256, rows=(0, 64), want_bytes=True, prob_cast=1)
    cb = np.float32(np.float32(P["q_scale"][0] * P["k_scale"][0]) * oracle_mod.C0(64))
    S0 = S[:, :128].astype(np.float64)
    t = (S[:, :128].max(1) * cb).astype(np.float32).astype(np.float64)
    zz = S0 * np.float64(cb) - t[:, None] + 8.0
    assert np.allclose(z[:, :128], zz, rtol=0, atol=1e-5)
    ref = torch.from_numpy(np.exp2(z[:, :128].astype(np.float64)).astype(np.float32)).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ref, by[:, :128])
    assert (by[:, :128].max(1) == 120).all()
    _, bye, _, _ = oracle_mod.attention_head(P, 256, rows=(0, 64), want_bytes=True)
    big = by[:, :128] >= 16
    agree = float((bye[:, :128][big] == by[:, :128][big]).mean())
    assert np.abs(bye[:, :128][big].astype(int) - by[:, :128][big].astype(int)).max() <= 1
    assert abs(agree - GOLD["expcast_agreement_per_doubling"]["value"]) < 0.05, agree


def test_kmeans_warm_start_composes(oracle_mod):
    """Lloyd rounds compose: 8 rounds from the seeded init equal 4 rounds
    followed by 4 more warm-started from the centroids those left (same
    assignment, centroids and objective); a warm start with 0 rounds is the
    nearest-centroid assignment of the given centroids."""
    cfg = synth.CONFIGS[0]
    q, k, v = synth.make_inputs(cfg, 0)
    vh = v[0, 0]
    a8, C8, J8 = oracle_mod.kmeans(vh, 8, 8, 99)
    a4, C4, J4 = oracle_mod.kmeans(vh, 8, 4, 99)
    aw, Cw, Jw = oracle_mod.kmeans_warm(vh, C4, 4)
    assert np.array_equal(aw, a8) and np.array_equal(Cw, C8) and Jw == J8
    a0, C0_, J0 = oracle_mod.kmeans_warm(vh, C8, 0)
    x = oracle_mod.bf16_to_f32(vh).astype(np.float64)
    d2 = ((x[:, None, :] - C8.astype(np.float64)[None]) ** 2).sum(-1)
    assert np.array_equal(a0, d2.argmin(1)) and np.array_equal(C0_, C8)
    # warm-starting from converged centroids does not raise the objective
    _, _, hist = oracle_mod.kmeans_warm(vh, C8, 4, history=True)
    assert np.all(np.diff(hist) <= 1e-9 * hist[0]) and hist[-1] <= J8 * (1 + 1e-12)


def test_v_smooth_beats_plain_quantisation(oracle_mod):
    """Direction check on the value term (agihunt V-Smooth bullet: only the
    residual after the block mean is quantised): with the same permutation
    and the same per-(block, channel) amax/448 scale rule, mean + E4M3
    residual reconstructs V better than E4M3 of V itself, on every head of
    the tiny workload, in k-means and in sequence order."""
    cfg = synth.CONFIGS[0]
    _, _, v = synth.make_inputs(cfg, 0)
    q = k = v  # Q and K do not enter the value reconstruction
    L, d = cfg.L, cfg.d
    for h in range(cfg.H):
        x = oracle_mod.bf16_to_f32(v[0, h]).astype(np.float64)
        a, _, _ = oracle_mod.kmeans(v[0, h], 8, 8, oracle_mod.head_seed(0, 0, h, cfg.H))
        for perm in (oracle_mod.stable_perm(a, 8), np.arange(L, dtype=np.int32)):
            P = oracle_mod.prepare_head(q[0, h], k[0, h], v[0, h], perm)
            xp = x[perm].reshape(L // 128, 128, d)                          # permuted blocks
            dec = oracle_mod.e4m3_decode(P["v8"]).transpose(0, 2, 1)           # [nb,128,d]
            smooth = P["v_mean"][:, None, :] + P["v_scale"][:, None, :].astype(np.float64) * dec
            amax = np.abs(xp.astype(np.float32)).max(axis=1)                   # [nb,d]
            s = (amax / np.float32(448)).astype(np.float32)
            inv = (np.float32(448) / amax).astype(np.float32)
            plain = s[:, None, :].astype(np.float64) * oracle_mod.e4m3_decode(
                oracle_mod.e4m3_encode((xp.astype(np.float32) * inv[:, None, :]).astype(np.float32)))
            e_s = np.linalg.norm(smooth - xp) / np.linalg.norm(xp)
            e_p = np.linalg.norm(plain - xp) / np.linalg.norm(xp)
            assert e_s < e_p, (h, e_s, e_p)
