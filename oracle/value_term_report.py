"""Error decomposition of the quantised attention by token ordering: a
measurement made with the oracle (test infrastructure, CPU only).

For sampled heads and query rows of a synthetic workload and for three
orderings of the value tokens -- sequence order, the static 2x8x8 cube of
the latent grid, and the k-means order (seeded Lloyd, k = number of blocks,
8 rounds, stable sort by cluster) -- it reports the output error against
exact softmax attention with only Q/K, only P or only V quantised, and with
all three (oracle.attention_parts), the value term's share of the squared
error e_V^2 / (e_QK^2 + e_P^2 + e_V^2) (the MarkTechPost abstract reports
the value term's share of the output error on Wan2.2 after QK smoothing),
the block energy the block mean removes and the value reconstruction error
(the abstract's block-energy comparison of the three orderings), and, for
the k-means order, how many clusters each 128-slot block holds and the
objective after every Lloyd round.

Usage: python -m oracle.value_term_report [--config 2] [--heads 0,39]
       [--tiles 0,147]   (prints one JSON object)
"""
from __future__ import annotations

import argparse
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from bit_attention_video_smooth_amd import synth  # noqa: E402
from bit_attention_video_smooth_amd.ablation import cube_permutation  # noqa: E402


def _rel(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def value_block_stats(v, perm, o):
    """Block energy removed by the means, 1 - sum|v - mu_b|^2 / sum|v|^2, and
    |v_hat - v| / |v| with v_hat = mu_b + s_v E4M3(code), over one head."""
    L, d = v.shape
    nb = oracle.nblocks(L)
    x = oracle.bf16_to_f32(v).astype(np.float64)[perm]
    xp = np.zeros((nb * 128, d))
    xp[:L] = x
    mu = np.repeat(o["v_mean"].astype(np.float64), 128, axis=0)
    r = oracle.e4m3_decode(o["v8"]) * o["v_scale"][:, :, None]
    xh = mu + r.transpose(0, 2, 1).reshape(nb * 128, d)
    tot = float((x * x).sum())
    return (1.0 - float(((xp - mu)[:L] ** 2).sum()) / tot,
            float(np.sqrt(((xh - xp)[:L] ** 2).sum() / tot)))


def report(cfg_idx=2, heads=(0, 39), tiles=(0, 147)):
    cfg = synth.CONFIGS[cfg_idx]
    q, k, v = synth.make_inputs(cfg, cfg_idx)
    L, nb = cfg.L, oracle.nblocks(cfg.L)
    out = {"workload": cfg.name, "heads": list(heads), "query_tiles": list(tiles), "orderings": {}}
    for h in heads:
        b, hh = divmod(h, cfg.H)
        a, _, hist = oracle.kmeans(v[b, hh], nb, 8, oracle.head_seed(cfg_idx, b, hh, cfg.H), history=True)
        km = oracle.stable_perm(a, nb)
        per_block = np.array([len(np.unique(a[km[i * 128:(i + 1) * 128]])) for i in range(nb)])
        sizes = np.bincount(a, minlength=nb)
        out.setdefault("kmeans", {})[str(h)] = {
            "objective_per_round": [float(x) for x in hist],
            "clusters_per_block": {"mean": float(per_block.mean()), "max": int(per_block.max()),
                                   "one_cluster_blocks": float((per_block == 1).mean())},
            "cluster_size": {"min": int(sizes.min()), "median": float(np.median(sizes)),
                             "max": int(sizes.max()), "empty": int((sizes == 0).sum())}}
        for name, perm in (("sequence", np.arange(L, dtype=np.int32)), ("cube", cube_permutation(cfg.grid)),
                           ("kmeans", km)):
            o = oracle.prepare_head(q[b, hh], k[b, hh], v[b, hh], perm)
            energy, verr = value_block_stats(v[b, hh], perm, o)
            parts = {n: [] for n in ("exact", "qk", "p", "v", "all")}
            for t in tiles:
                rows = (256 * t, min(L, 256 * t + 256))
                P = oracle.attention_parts(q[b, hh], k[b, hh], v[b, hh], perm, rows=rows)
                for n in parts:
                    parts[n].append(P[n])
            P = {n: np.concatenate(x) for n, x in parts.items()}
            e = {n: _rel(P[n], P["exact"]) for n in ("qk", "p", "v", "all")}
            share = e["v"] ** 2 / (e["qk"] ** 2 + e["p"] ** 2 + e["v"] ** 2)
            out["orderings"].setdefault(name, {})[str(h)] = {
                "output_rel_err": e, "value_term_share": share, "energy_removed": energy, "v_rel_err": verr}
            print("%s head %d %s: %s share %.3f energy %.3f v_err %.4f" % (cfg.name, h, name, e, share, energy, verr),
                  file=sys.stderr, flush=True)
    for name, per_head in out["orderings"].items():
        hs = list(per_head.values())
        per_head["mean"] = {"value_term_share": float(np.mean([x["value_term_share"] for x in hs])),
                            "output_rel_err": {n: float(np.mean([x["output_rel_err"][n] for x in hs]))
                                               for n in ("qk", "p", "v", "all")},
                            "energy_removed": float(np.mean([x["energy_removed"] for x in hs])),
                            "v_rel_err": float(np.mean([x["v_rel_err"] for x in hs]))}
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--config", type=int, default=2)
    ap.add_argument("--heads", default="0,39")
    ap.add_argument("--tiles", default="0,147")
    a = ap.parse_args()
    print(json.dumps(report(a.config, tuple(int(x) for x in a.heads.split(",")),
                            tuple(int(x) for x in a.tiles.split(",")))))


if __name__ == "__main__":
    main()
