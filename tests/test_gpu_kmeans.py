"""GPU parity of the k-means steps themselves, index by index (aikraft.ru
"Reshenie": lightweight k-means groups similar tokens; MarkTechPost abstract:
blocks of 128 after sorting), through the C ABI.

A warm start with 0 rounds is one nearest-centroid assignment of the given
centroids followed by the stable sort by cluster; with 1 round the members
of each cluster are then averaged. The library returns the permutation, and
since that is a stable sort by cluster, the library's assignment can be read
back from it once the candidates of each token are known:

  * assignment: every token whose two best exact scores x.c - |c|^2/2 (fp64)
    are further apart than the library's error bound gets exactly the
    oracle's centroid; a token inside the bound may get any centroid within
    it. The bound: the centroid enters as a bf16 high part plus a bf16 low
    part, which leaves at most 2^-16 |c_i| per element, and the products add
    up in fp32 over d terms with |c|^2 in fp32; 2^-14 (sum |x_i||c_i| +
    |c|^2 / 2) covers both several times over.
  * update: every cluster whose members agree with the oracle's has a
    bit-identical centroid (both sides sum bf16 values in fp64, which is
    exact here whatever the order, divide once and round to fp32); empty
    clusters keep the given centroid.
"""
import numpy as np
import pytest
import torch

import oracle
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


def _candidates(v_head, C, chunk=2048):
    """Exact scores and, per token, the centroids within the error bound of
    the best one (a dict token -> sorted candidates, only where there are
    several) and the best centroid (lowest index among exact ties); tokens
    in chunks so that large k stays within host memory."""
    x_all = oracle.bf16_to_f32(v_head).astype(np.float64)
    C = C.astype(np.float64)
    half = 0.5 * (C * C).sum(axis=1)
    aC = np.abs(C).T
    best = np.empty(x_all.shape[0], np.int64)
    ties = {}
    for t0 in range(0, x_all.shape[0], chunk):
        x = x_all[t0:t0 + chunk]
        S = x @ C.T - half[None, :]
        E = 2.0 ** -14 * (np.abs(x) @ aC + half[None, :])
        b = np.argmax(S, axis=1)
        rows = np.arange(x.shape[0])
        near = (S[rows, b][:, None] - S) <= (E[rows, b][:, None] + E)
        best[t0:t0 + x.shape[0]] = b
        for t in np.nonzero(near.sum(axis=1) > 1)[0]:
            ties[int(t0 + t)] = tuple(np.nonzero(near[t])[0].tolist())
    return best, ties


def _labels_from_perm(perm, a_ref, ties):
    """The assignment whose stable sort is perm, taking every token's label
    from its candidates (the oracle's label where it has no others); None if
    no such assignment exists. Scanning perm in order, the smallest feasible
    label is always the safe choice: labels must not decrease along perm,
    and tokens sharing a label must appear in increasing index order."""
    lab = np.empty(perm.size, np.int64)
    cur, last = -1, -1
    for t in perm.tolist():
        for c in ties.get(t, (int(a_ref[t]),)):
            if c > cur or (c == cur and t > last):
                break
        else:
            return None
        cur, last = c, t
        lab[t] = c
    return lab


def _check_head(api, v_head, C, P_perm, Cout=None, label=""):
    a_ref, _, _ = oracle.kmeans_warm(v_head, C, 0)
    best, ties = _candidates(v_head, C)
    clear = np.ones(a_ref.size, bool)
    clear[list(ties)] = False
    assert np.array_equal(a_ref[clear], best[clear]), "oracle and fp64 scores disagree away from ties"
    lab = _labels_from_perm(P_perm, a_ref, ties)
    assert lab is not None, "%s: the permutation is no stable sort of any admissible assignment" % label
    assert np.array_equal(np.argsort(lab, kind="stable"), P_perm)
    flips = int((lab != a_ref).sum())
    print("k-means assign %s: %d tokens, %d within the bound of a second centroid, %d assigned differently"
          % (label, a_ref.size, len(ties), flips))
    assert np.array_equal(lab[clear], a_ref[clear])
    if Cout is None:
        return
    _, C1, _ = oracle.kmeans_warm(v_head, C, 1)
    k = C.shape[0]
    same = 0
    for c in range(k):
        mg, mo = lab == c, a_ref == c
        if not np.array_equal(mg, mo):
            continue
        same += 1
        if not mo.any():
            assert np.array_equal(Cout[c].view(np.uint32), C[c].view(np.uint32)), "empty cluster %d moved" % c
        else:
            assert np.array_equal(Cout[c].view(np.uint32), C1[c].view(np.uint32)), \
                "%s cluster %d: centroid differs (max |d| %.3g)" % (label, c, np.abs(Cout[c] - C1[c]).max())
    print("k-means update %s: %d of %d centroids compared bit-exact" % (label, same, k))
    assert same >= k - 2 * flips


CASES = [  # B, H, L, d, k, grid, outlier settings
    (1, 2, 1024, 64, 8, (4, 16, 16), {}),
    (1, 2, 4096, 128, 32, (4, 32, 32), {}),
    (2, 1, 3000, 64, 24, None, {}),
    (1, 2, 9000, 128, 71, (9, 25, 40), {"outlier_frac": 0.005, "outlier_factor": 30.0}),  # a 7-centroid last tile
    (1, 1, 700, 128, 6, None, {}),
    (1, 1, 500, 128, 1, None, {}),           # one cluster: the identity permutation
    (1, 1, 300, 64, 300, None, {}),          # k = L, the largest k a shape allows
]

# k in the thousands and the library's largest k (16384); centroids are
# tokens with a small seeded jitter (a k-means round on the CPU would
# dominate the test's time)
LARGE_K = [(1, 1, 5000, 64, 4096), (1, 1, 16500, 64, 16384), (1, 1, 3000, 128, 1500)]


@pytest.mark.parametrize("case", CASES)
@pytest.mark.parametrize("rounds", [0, 1])
def test_kmeans_steps_match_oracle(api, case, rounds):
    B, H, L, d, k, grid, extra = case
    q, kk, v = synth.make_inputs(synth.custom(B, H, L, d, grid=grid, **extra), 60 + L)
    # realistic centroids: the oracle's own k-means after one round
    C = np.stack([np.stack([oracle.kmeans(v[b, h], k, 1, 1000 + 7 * b + h)[1] for h in range(H)])
                  for b in range(B)])
    Cout = torch.empty((B, H, k, d), dtype=torch.float32, device="cuda")
    P = api.prepare(dev_bf16(q), dev_bf16(kk), dev_bf16(v), kmeans_k=k, kmeans_iters=rounds,
                    centroids_in=torch.from_numpy(C).cuda(), centroids_out=Cout)
    perm = P.perm.cpu().numpy()
    Cout = Cout.cpu().numpy()
    for b in range(B):
        for h in range(H):
            _check_head(api, v[b, h], C[b, h], perm[b, h], Cout[b, h] if rounds == 1 else None,
                        "%s rounds=%d b=%d h=%d" % ((B, H, L, d, k), rounds, b, h))


@pytest.mark.parametrize("case", LARGE_K)
def test_kmeans_steps_large_k(api, case):
    """One round: the permutation checks the assignment, the centroids the
    update."""
    rounds = 1
    B, H, L, d, k = case
    q, kk, v = synth.make_inputs(synth.custom(B, H, L, d), 70 + k)
    rng = np.random.default_rng(k)
    pick = np.sort(rng.choice(L, size=k, replace=False))
    x = oracle.bf16_to_f32(v[0, 0])
    C = (x[pick] + 0.05 * rng.standard_normal((k, d))).astype(np.float32)[None, None]
    Cout = torch.empty((B, H, k, d), dtype=torch.float32, device="cuda")
    P = api.prepare(dev_bf16(q), dev_bf16(kk), dev_bf16(v), kmeans_k=k, kmeans_iters=rounds,
                    centroids_in=torch.from_numpy(C).cuda(), centroids_out=Cout)
    _check_head(api, v[0, 0], C[0, 0], P.perm.cpu().numpy()[0, 0], Cout.cpu().numpy()[0, 0] if rounds == 1 else None,
                "%s rounds=%d" % ((B, H, L, d, k), rounds))


def test_kmeans_steps_full_size(api):
    """The Wan 720p head shape (L = 75,600, d = 128, k = 591 centroids),
    heads 0 and 1 of that workload's recipe, in one launch."""
    cfg = synth.CONFIGS[2]
    L, d = cfg.L, cfg.d
    k = (L + 127) // 128
    q, kk, v = synth.make_inputs(synth.custom(1, 2, L, d, grid=cfg.grid, outlier_frac=cfg.outlier_frac,
                                              outlier_factor=cfg.outlier_factor), 5)
    C = np.stack([oracle.kmeans(v[0, h], k, 1, 77 + h)[1] for h in range(2)])[None]
    Cout = torch.empty((1, 2, k, d), dtype=torch.float32, device="cuda")
    P = api.prepare(dev_bf16(q), dev_bf16(kk), dev_bf16(v), kmeans_iters=1,
                    centroids_in=torch.from_numpy(C).cuda(), centroids_out=Cout)
    perm = P.perm.cpu().numpy()
    Cout = Cout.cpu().numpy()
    for h in range(2):
        _check_head(api, v[0, h], C[0, h], perm[0, h], Cout[0, h], "wan720p head %d" % h)
