"""The error decomposition of the oracle (oracle.attention_parts: the method
with only QK, only P or only V quantised; MarkTechPost abstract: after QK
smoothing the value term carries most of the output error), each part
pinned to something outside the oracle's blockwise loop:
  * exact: fp64 brute-force softmax attention (oracle.brute);
  * QK only: brute force on the dequantised per-block FP8 Q and K codes
    (K after its mean; softmax is unchanged by it) with exact V;
  * V only: brute force with exact Q, K and the V-Smooth reconstruction
    mean + s_v E4M3(code) of V, in the permuted order;
  * P only: within the pages' ExpCast bound, per row and channel
    |O_P - O| <= 2 (0.0364 + U) max_j |v_j - O|, 0.0364 the worst-case
    total variation of ExpCast probabilities (PAPER: MarkTechPost abstract,
    ExpCast-FP8 paragraph) and U the exact mass of the row below the
    underflow tail, 2^-14 of its maximum;
and the orderings' value errors against each other."""
import numpy as np
import pytest

import oracle
from bit_attention_video_smooth_amd import synth
from bit_attention_video_smooth_amd.ablation import cube_permutation


def _head(cfg_idx=0, h=0, seed=0):
    cfg = synth.CONFIGS[cfg_idx]
    q, k, v = synth.make_inputs(cfg, seed)
    return cfg, q[0, h], k[0, h], v[0, h]


def _rel(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


@pytest.mark.parametrize("perm_kind", ["identity", "random"])
def test_parts_against_brute_force(oracle_mod, perm_kind):
    cfg, q, k, v = _head(0, 1, 3)
    L, d = cfg.L, cfg.d
    perm = np.arange(L, dtype=np.int32) if perm_kind == "identity" else synth.random_perms(1, 1, L, 5)[0, 0]
    P = oracle.attention_parts(q, k, v, perm)
    f = oracle.bf16_to_f32
    qf, kf, vf = (f(a).astype(np.float64) for a in (q, k, v))
    exact = oracle.attention_f64(qf, kf, vf)
    assert _rel(P["exact"], exact) <= 1e-6
    o = oracle.prepare_head(q, k, v, perm)
    nb = oracle.nblocks(L)
    qb = np.minimum(np.arange(L) // 128, nb - 1)
    qd = oracle.e4m3_decode(o["q8"][:L]) * o["q_scale"][qb][:, None]
    kd = oracle.e4m3_decode(o["k8"][:L]) * o["k_scale"][qb][:, None]      # permuted order
    assert _rel(P["qk"], oracle.attention_f64(qd, kd, vf[perm])) <= 1e-6
    r = oracle.e4m3_decode(o["v8"]) * o["v_scale"][:, :, None]
    vd = (o["v_mean"][:, :, None] + r).transpose(0, 2, 1).reshape(-1, d)[:L]
    assert _rel(P["v"], oracle.attention_f64(qf[:, :], kf[perm], vd)) <= 1e-6


def test_p_only_within_expcast_bound(oracle_mod):
    cfg, q, k, v = _head(0, 0, 4)
    L, d = cfg.L, cfg.d
    perm = np.arange(L, dtype=np.int32)
    P = oracle.attention_parts(q, k, v, perm)
    f = oracle.bf16_to_f32
    qf, kf, vf = (f(a).astype(np.float64) for a in (q, k, v))
    z = (qf @ kf.T) * (np.log2(np.e) / np.sqrt(d))
    z -= z.max(axis=1, keepdims=True)
    p = np.exp2(z)
    p /= p.sum(axis=1, keepdims=True)
    U = np.where(z < -14, p, 0.0).sum(axis=1)                             # underflow-tail mass
    O = P["exact"].astype(np.float64)
    spread = np.abs(vf[None, :, :] - O[:, None, :]).max(axis=1)           # max_j |v_j - O|, [L, d]
    bound = 2 * (0.0364 + U)[:, None] * spread + 1e-6
    err = np.abs(P["p"] - O)
    print("P only: worst error / bound %.3f" % float((err / bound).max()))
    assert np.all(err <= bound)


def test_decomposition_is_consistent(oracle_mod):
    """Each part positive and below the whole; the whole roughly the
    quadrature sum of the parts (the three errors are nearly independent)."""
    cfg, q, k, v = _head(0, 0, 0)
    P = oracle.attention_parts(q, k, v, np.arange(cfg.L, dtype=np.int32))
    e = {n: _rel(P[n], P["exact"]) for n in ("qk", "p", "v", "all")}
    print(e)
    for n in ("qk", "p", "v"):
        assert 0 < e[n] < e["all"]
    quad = np.sqrt(e["qk"] ** 2 + e["p"] ** 2 + e["v"] ** 2)
    assert 0.7 * quad <= e["all"] <= 1.3 * quad


def test_value_term_follows_ordering(oracle_mod):
    """On the tiny workload (smooth value field over a 4x16x16 grid) the
    V-only error falls from sequence order to the static 2x8x8 cube to the
    k-means order, as the block energy the pages report for the three
    orderings does, while QK-only and P-only errors stay put (the joint K/V
    permutation changes only the per-block K scales)."""
    cfg, q, k, v = _head(0, 0, 0)
    L = cfg.L
    seq = np.arange(L, dtype=np.int32)
    cube = cube_permutation(cfg.grid)
    a, _, _ = oracle.kmeans(v, oracle.nblocks(L), 8, oracle.head_seed(0, 0, 0, cfg.H))
    km = oracle.stable_perm(a, oracle.nblocks(L))
    ev = {}
    for name, perm in (("sequence", seq), ("cube", cube), ("kmeans", km)):
        P = oracle.attention_parts(q, k, v, perm)
        ev[name] = {n: _rel(P[n], P["exact"]) for n in ("qk", "p", "v")}
    print(ev)
    assert ev["kmeans"]["v"] < ev["cube"]["v"] < ev["sequence"]["v"]
    for n in ("qk", "p"):
        vals = [ev[o][n] for o in ev]
        assert max(vals) <= 1.5 * min(vals)
