"""Benchmark of the VC-Attention hot path on one MI355X.

A step is one pass of the whole path over one batch of synthetic input: the
V-Smooth prepare (seeded k-means, 8 Lloyd rounds, K smoothing, permutation,
Q/K/V-residual FP8 quantisation) followed by the fused FP8 attention kernel.
The default workload is the Wan2.2-shaped 720p case (B=1, H=40, L=75,600,
d=128).  Inputs are resident in HBM before timing starts.

Prints one JSON line.  `value` is attention FLOP (4 B H L^2 d) per step
divided by the step time; the attention kernel alone, the BF16 kernel on the
same inputs and the prepare stage are reported beside it, with the dominant
kernel's roofline and the CPU oracle timed on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

FP8_PEAK_TFLOPS = 5000.0   # MI355X dense FP8 matrix peak
BF16_PEAK_TFLOPS = 2500.0  # MI355X dense BF16 matrix peak
FP4_PEAK_TFLOPS = 10100.0  # MI355X dense FP4 matrix peak
HBM_PEAK_GBS = 8000.0


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--config", type=int, default=2, help="workload index (0 tiny .. 4 cfg)")
    p.add_argument("--cpu-rows", type=int, default=-1, help="query rows of the CPU oracle sample (-1: auto)")
    p.add_argument("--no-cpu", action="store_true")
    p.add_argument("--no-bf16", action="store_true")
    p.add_argument("--no-sage", action="store_true", help="skip the SAGE-style baseline leg")
    p.add_argument("--no-warm", action="store_true", help="skip the k-means warm-start leg")
    p.add_argument("--no-fp4", action="store_true", help="skip the 4-bit V-Smooth leg")
    p.add_argument("--no-configs", action="store_true", help="skip timing the other workloads")
    p.add_argument("--v-scale-mode", type=int, default=0)
    p.add_argument("--skip-lambda", type=float, default=0.5,
                   help="Skip Softmax threshold of the extra, reported (not timed-step) attention run; 0: none")
    p.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                   help="only run a plain device copy of MIB MiB (negation, fp32) three times: the "
                        "reference kernel of known size that calibrates the HBM byte counters")
    return p.parse_args()


# Sources the attention kernel is built from; the committed HBM-traffic
# summary records their hash and is ignored once any of them changes.
KERNEL_SOURCES = ["bit_attention_video_smooth_amd/csrc/vc_attn_fp8.hip",
                  "bit_attention_video_smooth_amd/csrc/vc_attn_fp8w_kernel.hpp",
                  "bit_attention_video_smooth_amd/csrc/vc_attn_fp8_kernel.hpp",
                  "bit_attention_video_smooth_amd/csrc/vc_device.hpp",
                  "bit_attention_video_smooth_amd/csrc/vc_lds.hpp",
                  "bit_attention_video_smooth_amd/csrc/vc_internal.hpp",
                  "bit_attention_video_smooth_amd/build.py"]
TRAFFIC_SUMMARY = "profiles/attn_fp8_wan720p_hbm_traffic.txt"


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload):
    """HBM bytes per launch of the attention kernel from the committed
    FETCH_SIZE / WRITE_SIZE summary (already scaled by the copy-kernel
    factors), or None if the summary is absent, is for another workload, or
    was taken on different kernel sources."""
    path = os.path.join(ROOT, TRAFFIC_SUMMARY)
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if "=" in line and not line.lstrip().startswith("#"):
                key, val = line.split("=", 1)
                kv[key.strip()] = val.strip()
    if kv.get("workload") != workload or kv.get("source_sha256") != kernel_source_hash():
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def skip_fractions(p_full, p_skip, nb):
    """From the ExpCast bytes of one 256-query tile without and with Skip
    Softmax ([256, nb*128] uint8): the fraction of (row, block) pairs that
    have a nonzero byte without rejection and none with it, and the
    fraction of (wave, block) pairs -- 32 rows, one matrix-core tile -- whose
    rows all reject (the kernel skips bytes and P V only then)."""
    # compare first: any() of a uint8 tensor is uint8, on which ~ is a bitwise not
    live = (p_full.view(256, nb, 128) != 0).any(2)
    rej = ~(p_skip.view(256, nb, 128) != 0).any(2) & live
    wlive = live.view(8, 32, nb).any(1)
    wrej = (rej | ~live).view(8, 32, nb).all(1) & wlive
    return (float(rej.float().sum() / live.float().sum()), float(wrej.float().sum() / wlive.float().sum()))


def copy_probe(mib):
    import torch
    n = (mib << 20) // 4
    x = torch.ones(n, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    for _ in range(3):
        torch.neg(x, out=y)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_read": n * 4, "copy_probe_bytes_written": n * 4, "launches": 3}))


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: this library has no multi-GPU path "
              "(the workload shards by (batch, head) with no exchange between GPUs)", file=sys.stderr)
        sys.exit(2)
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return
    import numpy as np
    import torch

    from bit_attention_video_smooth_amd import api, synth

    torch.cuda.set_device(0)
    cfg = synth.CONFIGS[args.config]
    B, H, L, d = cfg.B, cfg.H, cfg.L, cfg.d
    flop = cfg.attn_flop
    t0 = time.time()
    qn, kn, vn = synth.make_inputs(cfg, args.config, threads=16)
    print("inputs generated in %.1fs" % (time.time() - t0), file=sys.stderr, flush=True)
    dev = lambda a: torch.from_numpy(a).view(torch.bfloat16).cuda()
    q, k, v = dev(qn), dev(kn), dev(vn)
    P = api.alloc_prepared(B, H, L, d)
    ws = api.workspace(B, H, L, d)
    out = torch.empty((B, H, L, d), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        api.prepare(q, k, v, seed=args.config, v_scale_mode=args.v_scale_mode, out=P, ws=ws)
        if ev is not None:
            ev[1].record(stream)
        api.attention(P, out=out)
        if ev is not None:
            ev[2].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(args.steps):
        step(evs[i])
    stop.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    ms_step = total_ms / args.steps
    prep_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    attn_each = [e[1].elapsed_time(e[2]) for e in evs]
    attn_ms = float(np.mean(attn_each))
    print("step %.3f ms (prepare %.3f, attention %.3f)" % (ms_step, prep_ms, attn_ms), file=sys.stderr, flush=True)
    h00 = (qn[0, 0].copy(), kn[0, 0].copy(), vn[0, 0].copy())
    # head (0, 0) of the timed step's output and permutation, for the parity sample
    out00 = out[0, 0].cpu().numpy()
    perm00 = P.perm[0, 0].cpu().numpy()
    codes00 = {n: getattr(P, n)[0, 0].cpu().numpy() for n in ("q8", "k8", "q_scale", "k_scale", "v_scale", "v_mean")}
    codes00["v8"] = api.v_codes_natural(P.v8[0:1, 0:1]).cpu().numpy()[0, 0]
    obj00 = float(P.kmeans_obj[0, 0].cpu())
    dump00 = api.attention_dump(P, 0, 0)
    if args.v_scale_mode not in (0, 1):
        sys.exit("--v-scale-mode must be 0 or 1")

    # prepare without k-means (permutation reused, as across adjacent steps),
    # each repetition after a 512 MiB write that flushes the last-level cache
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    qev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for i in range(args.steps):
        flush.fill_(i & 0xFF)
        qev[i][0].record(stream)
        api.prepare(q, k, v, perm_in=P.perm, out=P, ws=ws, v_scale_mode=args.v_scale_mode)
        qev[i][1].record(stream)
    torch.cuda.synchronize()
    quant_each = [e[0].elapsed_time(e[1]) for e in qev]
    quant_ms = float(np.mean(quant_each))
    del flush
    E = B * H * L * d
    nb = api.nblocks(L)
    quant_bytes = 3 * E * 2 + 3 * E * 1 + B * H * nb * d * 8 + B * H * L * 4
    # the same step's attention on V prepared with the other V-scale mode
    P1 = api.alloc_prepared(B, H, L, d)
    api.prepare(q, k, v, perm_in=P.perm, out=P1, ws=ws, v_scale_mode=1 - args.v_scale_mode)
    api.attention(P1, out=out)
    torch.cuda.synchronize()
    ev[0].record(stream)
    for _ in range(args.steps):
        api.attention(P1, out=out)
    ev[1].record(stream)
    torch.cuda.synchronize()
    other_ms = ev[0].elapsed_time(ev[1]) / args.steps
    del P1
    # Skip Softmax on the same prepared inputs: time, and the fraction of
    # (row, block) pairs rejected in one sampled query tile (blocks whose
    # bytes are all zero with rejection but not without)
    skip = None
    if args.skip_lambda > 0:
        bh, qt = (B * H) // 2, api.nblocks(L) // 4
        _, _, pf = api.attention_dump(P, bh, qt)

        def skip_run(lam, n):
            api.attention(P, out=out, skip_lambda=lam)
            torch.cuda.synchronize()
            ev[0].record(stream)
            for _ in range(n):
                api.attention(P, out=out, skip_lambda=lam)
            ev[1].record(stream)
            torch.cuda.synchronize()
            ms = ev[0].elapsed_time(ev[1]) / n
            _, _, pb = api.attention_dump(P, bh, qt, skip_lambda=lam)
            row_frac, wave_frac = skip_fractions(pf, pb, nb)
            return {"lambda": lam, "ms": ms, "speedup_vs_no_rejection": attn_ms / ms,
                    "rejected_fraction_sample": row_frac, "wave_rejected_fraction_sample": wave_frac}

        skip = skip_run(args.skip_lambda, args.steps)
        skip.update({"dense_equivalent_tflops": flop / skip["ms"] / 1e9,
                     "sample": "query tile %d of head %d (256 rows x %d blocks)" % (qt, bh, nb),
                     # the threshold's range: a few launches each
                     "sweep": [skip_run(lam, max(2, args.steps // 4)) for lam in (0.05, 0.3, 0.9)]})
        print("skip softmax lambda %g: %.3f ms" % (args.skip_lambda, skip["ms"]), file=sys.stderr, flush=True)
    bf16 = None
    if not args.no_bf16:
        ob = torch.empty((B, H, L, d), dtype=torch.float32, device="cuda")
        api.attention_bf16(q, k, v, out=ob)
        torch.cuda.synchronize()
        ev[0].record(stream)
        n16 = max(1, args.steps // 2)
        for _ in range(n16):
            api.attention_bf16(q, k, v, out=ob)
        ev[1].record(stream)
        torch.cuda.synchronize()
        bf16_ms = ev[0].elapsed_time(ev[1]) / n16
        bclock = clock_under_load(lambda: api.attention_bf16(q, k, v, out=ob), stream, n=48)
        bf16 = {"ms": bf16_ms, "tflops": flop / bf16_ms / 1e9,
                "frac_bf16_peak": flop / bf16_ms / 1e9 / BF16_PEAK_TFLOPS,
                "fp8_speedup_over_bf16": bf16_ms / attn_ms,
                "sclk_mhz": bclock["sclk_mhz"], "socket_power_w": bclock["socket_power_w"]}
        print("bf16 attention %.3f ms" % bf16_ms, file=sys.stderr, flush=True)

    # the FP8 path ExpCast replaces (fp32 exp2, then the E4M3 conversion), on
    # the same prepared inputs
    api.attention(P, out=out, prob_cast=1)
    torch.cuda.synchronize()
    ev[0].record(stream)
    for _ in range(args.steps):
        api.attention(P, out=out, prob_cast=1)
    ev[1].record(stream)
    torch.cuda.synchronize()
    naive_ms = ev[0].elapsed_time(ev[1]) / args.steps
    exp_then_cast = {"ms": naive_ms, "tflops": flop / naive_ms / 1e9, "expcast_speedup": naive_ms / attn_ms}
    print("exp-then-cast attention %.3f ms" % naive_ms, file=sys.stderr, flush=True)

    # k-means warm start across steps: V drifts a little (next denoising
    # step); 8 seeded Lloyd rounds against 4 rounds started from the previous
    # step's final centroids
    warm = None
    if not args.no_warm:
        nbk = api.nblocks(L)
        C = torch.empty((B, H, nbk, d), dtype=torch.float32, device="cuda")
        api.prepare(q, k, v, seed=args.config, out=P, ws=ws, centroids_out=C)
        g = torch.Generator(device="cuda").manual_seed(1234)
        v2 = (v.float() + 0.05 * torch.randn(v.shape, generator=g, device="cuda")).to(torch.bfloat16)
        api.prepare(q, k, v2, seed=args.config, out=P, ws=ws)
        j_cold = P.kmeans_obj.clone()
        C2 = torch.empty_like(C)
        ev[0].record(stream)
        for _ in range(args.steps):
            api.prepare(q, k, v2, kmeans_iters=4, out=P, ws=ws, centroids_in=C, centroids_out=C2)
        ev[1].record(stream)
        torch.cuda.synchronize()
        warm_ms = ev[0].elapsed_time(ev[1]) / args.steps
        ratio = (P.kmeans_obj / j_cold).cpu().numpy()
        warm = {"kmeans_iters": 4, "prepare_ms": warm_ms, "seeded_8_rounds_prepare_ms": prep_ms,
                "objective_ratio_vs_seeded_8": {"mean": float(ratio.mean()), "max": float(ratio.max())},
                "drift": "v + 0.05 N(0,1) between the two steps"}
        del v2
        api.prepare(q, k, v, seed=args.config, v_scale_mode=args.v_scale_mode, out=P, ws=ws)  # restore P
        print("warm start: prepare %.3f ms, objective ratio %.4f" % (warm_ms, float(ratio.mean())),
              file=sys.stderr, flush=True)

    # 4-bit V-Smooth (E2M1 residual and probabilities, power-of-two scales per
    # 32-key group, scaled FP4 matrix cores) on the same inputs and permutation
    fp4 = None
    P4 = None
    if not args.no_fp4:
        P4 = api.alloc_prepared(B, H, L, d)
        api.prepare(q, k, v, perm_in=P.perm, out=P4, ws=ws, v_format=1)
        api.attention(P4, out=out)
        torch.cuda.synchronize()
        ev[0].record(stream)
        for _ in range(args.steps):
            api.prepare(q, k, v, perm_in=P.perm, out=P4, ws=ws, v_format=1)
        ev[1].record(stream)
        torch.cuda.synchronize()
        p4_ms = ev[0].elapsed_time(ev[1]) / args.steps
        ev[0].record(stream)
        for _ in range(args.steps):
            api.attention(P4, out=out)
        ev[1].record(stream)
        torch.cuda.synchronize()
        a4_ms = ev[0].elapsed_time(ev[1]) / args.steps
        fp4 = {"prepare_ms_without_kmeans": p4_ms, "attention_ms": a4_ms, "tflops": flop / a4_ms / 1e9,
               "frac_fp4_peak": flop / a4_ms / 1e9 / FP4_PEAK_TFLOPS,
               "vs_fp8_expcast": attn_ms / a4_ms, "vs_fp8_exp_then_cast": naive_ms / a4_ms}
        print("fp4 V-Smooth: prepare %.3f ms, attention %.3f ms" % (p4_ms, a4_ms), file=sys.stderr, flush=True)

    # SAGE-style baseline (TensorRT-LLM blog, "Quantized Attention": one Q
    # scale per token, one K scale per 16 keys, INT8 or FP8 QK^T, FP8 PV with
    # one V scale per channel, exp-then-cast P) on the same inputs
    sage = None
    SP = None
    if not args.no_sage:
        sage = {}
        sws = torch.empty(max(16, api._lib.vc_sage_workspace_bytes(api._lib.shape_of(B, H, L, d))),
                          dtype=torch.uint8, device="cuda")
        for qk in ("int8", "fp8"):
            SP = api.sage_prepare(q, k, v, qk_dtype=qk, out=SP, ws=sws)
            api.sage_attention(SP, out=out)
            torch.cuda.synchronize()
            ev[0].record(stream)
            for _ in range(args.steps):
                api.sage_prepare(q, k, v, qk_dtype=qk, out=SP, ws=sws)
            ev[1].record(stream)
            torch.cuda.synchronize()
            sp_ms = ev[0].elapsed_time(ev[1]) / args.steps
            ev[0].record(stream)
            for _ in range(args.steps):
                api.sage_attention(SP, out=out)
            ev[1].record(stream)
            torch.cuda.synchronize()
            sa_ms = ev[0].elapsed_time(ev[1]) / args.steps
            sage["qk_" + qk] = {"prepare_ms": sp_ms, "attention_ms": sa_ms, "tflops": flop / sa_ms / 1e9,
                                "vc_attention_speedup": sa_ms / attn_ms,
                                "vc_speedup_with_prepare": (sp_ms + sa_ms) / (quant_ms + attn_ms)}
            print("sage %s: prepare %.3f ms, attention %.3f ms" % (qk, sp_ms, sa_ms), file=sys.stderr, flush=True)
        sage["note"] = ("P bytes by exp-then-cast; vc_speedup_with_prepare compares against the V-Smooth "
                        "prepare without k-means (permutation reused)")

    # V-Smooth token-ordering ablation on this workload (prepare outputs of
    # the library; statistics averaged over heads)
    from bit_attention_video_smooth_amd.ablation import (cube_permutation, fp4_value_stats, sage_value_stats,
                                                         value_stats)
    ablation = {}
    orders = {"sequence": torch.arange(L, dtype=torch.int32, device="cuda").expand(B, H, L).contiguous(),
              "static_cube_2x8x8": torch.from_numpy(cube_permutation(cfg.grid)).cuda().expand(B, H, L).contiguous(),
              "kmeans": P.perm.clone()}
    Pa = api.alloc_prepared(B, H, L, d)
    for name, perm in orders.items():
        api.prepare(q, k, v, perm_in=perm, out=Pa, ws=ws, v_scale_mode=args.v_scale_mode)
        st = value_stats(Pa, v)
        ablation[name] = {"energy_removed": float(st["energy_removed"].mean()),
                          "v_rel_err": float(st["v_rel_err"].mean())}
    del Pa
    if P4 is not None:  # the 4-bit residual in k-means order
        ablation["kmeans_fp4_residual"] = {"v_rel_err": float(fp4_value_stats(P4, v)["v_rel_err"].mean())}
        del P4
    if SP is not None:  # the SAGE recipe's V codes: one scale per channel, no block mean
        ablation["sage_per_channel"] = {"v_rel_err": float(sage_value_stats(SP, v)["v_rel_err"].mean())}
        del SP

    clock = clock_under_load(lambda: api.attention(P, out=out), stream, n=80)
    ceiling = matrix_core_ceiling(stream)
    print("matrix-core ceiling: %.0f TFLOP/s at %s MHz, %s W; attention at %s MHz, %s W"
          % (ceiling["tflops"], ceiling["sclk_mhz"], ceiling["socket_power_w"], clock["sclk_mhz"],
             clock["socket_power_w"]), file=sys.stderr, flush=True)

    # the other workloads: prepare (with and without k-means) and attention
    configs = None
    if not args.no_configs:
        del P, ws, out, q, k, v, qn, kn, vn
        torch.cuda.empty_cache()
        configs = {cfg.name: {"attention_ms": attn_ms, "tflops": attn_tflops_of(flop, attn_ms),
                              "frac_fp8_peak": attn_tflops_of(flop, attn_ms) / FP8_PEAK_TFLOPS,
                              "prepare_ms_with_kmeans": prep_ms, "prepare_ms_without_kmeans": quant_ms,
                              "prepare_gbs_without_kmeans": quant_bytes / quant_ms / 1e6, "measured": "timed step"}}
        for ci, c in enumerate(synth.CONFIGS):
            if ci != args.config:
                configs[c.name] = time_config(c, ci, stream)
                print("config %s: %s" % (c.name, configs[c.name]), file=sys.stderr, flush=True)

    attn_tflops = flop / attn_ms / 1e9
    res = {
        "metric": "FP8 attention TFLOP/s (4*B*H*L^2*d) & % FP8 MFMA peak, Wan2.2-shaped L=75,600",
        "value": flop / ms_step / 1e9,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3",
        "data": "synthetic (seeded video-token tensors, bf16)",
        "config": {"workload": "%s: B=%d H=%d L=%d d=%d, V-Smooth k-means (k=%d, 8 rounds) + FP8 ExpCast attention"
                               % (cfg.name, B, H, L, d, nb, ), "B": B, "H": H, "L": L, "d": d,
                   "v_scale_mode": args.v_scale_mode},
        "frac_fp8_peak_step": flop / ms_step / 1e9 / FP8_PEAK_TFLOPS,
        "attention": {"ms": attn_ms, "tflops": attn_tflops, "frac_fp8_peak": attn_tflops / FP8_PEAK_TFLOPS,
                      "ms_median": float(np.median(attn_each)), "ms_min": float(np.min(attn_each))},
        "device": {"name": torch.cuda.get_device_name(0),
                   "compute_units": torch.cuda.get_device_properties(0).multi_processor_count, **clock},
        "frac_fp8_peak_at_measured_clock": (attn_tflops / (FP8_PEAK_TFLOPS * clock["sclk_mhz"] / 2400.0)
                                            if clock.get("sclk_mhz") else None),
        # the FP8 products alone (no memory traffic): what the matrix cores
        # sustain on this machine, and the attention kernel's share of it
        "matrix_core_ceiling": {**ceiling, "attention_frac_of_ceiling": attn_tflops / ceiling["tflops"]},
        "attention_other_v_scale_mode": {"v_scale_mode": 1 - args.v_scale_mode, "ms": other_ms,
                                         "tflops": flop / other_ms / 1e9,
                                         "frac_fp8_peak": flop / other_ms / 1e9 / FP8_PEAK_TFLOPS},
        "prepare": {"ms_with_kmeans": prep_ms, "ms_without_kmeans": quant_ms,
                    "ms_without_kmeans_median": float(np.median(quant_each)),
                    "ms_without_kmeans_min": float(np.min(quant_each)),
                    "quant_algorithmic_bytes": quant_bytes,
                    "quant_gbs": quant_bytes / quant_ms / 1e6,
                    "gbs_with_kmeans": quant_bytes / prep_ms / 1e6,
                    # k-means = prepare with minus without; its assign steps
                    # do 2*B*H*L*k*d FLOP per round (k = nb centroids)
                    "kmeans": {"ms": prep_ms - quant_ms, "rounds": 8, "k": nb,
                               "assign_tflop": 2.0 * B * H * L * nb * d * 8 / 1e12,
                               "assign_tflops_over_kmeans_time": 2.0 * B * H * L * nb * d * 8 / (prep_ms - quant_ms) / 1e9,
                               "frac_bf16_peak": 2.0 * B * H * L * nb * d * 8 / (prep_ms - quant_ms) / 1e9
                               / BF16_PEAK_TFLOPS}},
        "bf16_attention": bf16,
        "exp_then_cast_attention": exp_then_cast,
        "sage_baseline": sage,
        "fp4_v_smooth": fp4,
        "skip_softmax": skip,
        "configs": configs,
        "grouping_schedule": grouping_schedule(prep_ms, quant_ms, attn_ms),
        "kmeans_warm_start": warm,
        "v_smooth_ablation": ablation,
        "roofline": {"bound": "mfma", "achieved": attn_tflops, "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": attn_tflops / FP8_PEAK_TFLOPS, "traffic": measured_traffic(cfg.name)},
        "cpu_baseline": None,
    }
    if not args.no_cpu:
        res["cpu_baseline"] = cpu_baseline(cfg, h00, args.cpu_rows, perm00, codes00, out00, obj00, dump00, args.config)
    print(json.dumps(res))


def attn_tflops_of(flop, ms):
    return flop / ms / 1e9


def time_config(c, ci, stream, reps=None):
    """Prepare (seeded k-means, 8 rounds; and with the permutation passed
    back in) and FP8 attention times of one more workload, on its own
    seeded synthetic inputs; all buffers freed afterwards."""
    import numpy as np
    import torch

    from bit_attention_video_smooth_amd import api, synth
    B, H, L, d = c.B, c.H, c.L, c.d
    qn, kn, vn = synth.make_inputs(c, ci, threads=16)
    dev = lambda a: torch.from_numpy(a).view(torch.bfloat16).cuda()
    q, k, v = dev(qn), dev(kn), dev(vn)
    del qn, kn, vn
    P = api.alloc_prepared(B, H, L, d)
    ws = api.workspace(B, H, L, d)
    out = torch.empty((B, H, L, d), dtype=torch.float32, device="cuda")
    flop = c.attn_flop
    n = reps or (3 if flop > 2e14 else 10)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]

    def timed(fn, k):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(k):
            ev[0].record(stream)
            fn()
            ev[1].record(stream)
            torch.cuda.synchronize()
            ts.append(ev[0].elapsed_time(ev[1]))
        return float(np.median(ts))

    p_km = timed(lambda: api.prepare(q, k, v, seed=ci, out=P, ws=ws), 3)
    p_q = timed(lambda: api.prepare(q, k, v, perm_in=P.perm, out=P, ws=ws), 3)
    a_ms = timed(lambda: api.attention(P, out=out), n)
    nb = api.nblocks(L)
    E = B * H * L * d
    qbytes = 3 * E * 2 + 3 * E * 1 + B * H * nb * d * 8 + B * H * L * 4
    r = {"B": B, "H": H, "L": L, "d": d, "attention_ms": a_ms, "tflops": attn_tflops_of(flop, a_ms),
         "frac_fp8_peak": attn_tflops_of(flop, a_ms) / FP8_PEAK_TFLOPS, "prepare_ms_with_kmeans": p_km,
         "prepare_ms_without_kmeans": p_q, "prepare_gbs_without_kmeans": qbytes / p_q / 1e6,
         "measured": "median of %d attention launches, 3 prepares each" % n}
    del P, ws, out, q, k, v
    torch.cuda.empty_cache()
    return r


def clock_under_load(launch, stream, n=20):
    """Shader clock and power cap (rocm-smi) and socket power (amd-smi) read
    while n launches keep the GPU busy (queued first, so the readings fall
    inside them); fields that could not be read are None."""
    import re
    import subprocess

    import torch
    for _ in range(n):
        launch()
    info = {"sclk_mhz": None, "power_cap_w": None, "socket_power_w": None,
            "clock_source": "rocm-smi (clock, cap) and amd-smi (socket power) during %d launches" % n}
    try:
        # rocm-smi is a Python script: run it with this interpreter, not
        # through its "env python3" line, so no process in between replaces
        # itself (under a profiler that preloads into every process, such an
        # exec would come after that process had opened the GPU)
        import shutil
        import sys
        # socket power first: amd-smi reports a short running average, so it is
        # read while the queued launches are certainly still running
        amd = shutil.which("amd-smi") or "/opt/rocm/bin/amd-smi"
        r = subprocess.run([sys.executable, amd, "metric", "--power"], capture_output=True, text=True, timeout=60)
        m = re.search(r"SOCKET_POWER:\s*([\d.]+)", r.stdout)
        if m:
            info["socket_power_w"] = float(m.group(1))
        smi = shutil.which("rocm-smi") or "/opt/rocm/bin/rocm-smi"
        r = subprocess.run([sys.executable, smi, "--showclocks", "--showmaxpower"], capture_output=True, text=True,
                           timeout=30)
        txt = r.stdout
        m = re.search(r"sclk clock level:\s*\w+:\s*\((\d+)\s*Mhz\)", txt, re.I)
        if m:
            info["sclk_mhz"] = float(m.group(1))
        m = re.search(r"Max Graphics Package Power \(W\):\s*([\d.]+)", txt, re.I)
        if m:
            info["power_cap_w"] = float(m.group(1))
    except (OSError, subprocess.SubprocessError):
        pass
    torch.cuda.synchronize()
    return info


def matrix_core_ceiling(stream, blocks=1024, iters=5000, reps=40):
    """FP8 rate, clock and socket power of the matrix cores alone: the
    library's stream of independent 32x32x64 FP8 products from registers
    (vc_debug_mfma_rate, no memory traffic), timed with HIP events on the
    stream it runs on, then sampled like the attention kernel."""
    import torch
    from bit_attention_video_smooth_amd import _lib
    out = torch.empty(blocks * 512, dtype=torch.float32, device="cuda")
    launch = lambda: _lib.vc_debug_mfma_rate(blocks, iters, out, stream)
    for _ in range(3):
        launch()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        launch()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    flop = blocks * 8 * 4 * iters * 2 * 32 * 32 * 64
    clock = clock_under_load(launch, stream, n=1200)
    return {"tflops": flop / ms / 1e9, "frac_fp8_peak": flop / ms / 1e9 / FP8_PEAK_TFLOPS,
            "ms_per_launch": ms, "sclk_mhz": clock["sclk_mhz"], "socket_power_w": clock["socket_power_w"],
            "kernel": "vc_debug_mfma_rate: %d workgroups x 8 waves x %d x 4 independent 32x32x64 FP8 products"
                      % (blocks, iters)}


def grouping_schedule(prep_ms, quant_ms, attn_ms, num_steps=40):
    """Amortised prepare cost over a denoising schedule where grouping
    (k-means) runs only in the first 25% of the steps and a permutation is
    reused across 4 adjacent steps, from the two prepare times measured
    above (with k-means, and with the permutation passed back in)."""
    from bit_attention_video_smooth_amd.schedule import GroupingSchedule
    s = GroupingSchedule(num_steps)
    n = len(s.grouping_steps())
    amort = s.amortised(prep_ms, quant_ms)
    return {"num_steps": num_steps, "group_frac": s.group_frac, "reuse": s.reuse, "grouping_steps": n,
            "prepare_ms_amortised": amort, "step_ms_amortised": amort + attn_ms,
            "grouping_share_of_attention": n * (prep_ms - quant_ms) / (num_steps * attn_ms)}


def cpu_baseline(cfg, h00, rows, perm00, codes00, out00, obj00, dump00, seed):
    """The CPU oracle, as it stands, on a bounded sample of the same workload
    -- head (0, 0), prepared with the permutation the GPU's k-means chose,
    then blockwise attention for `rows` query rows against all L keys;
    throughput is that sample's attention FLOP over the oracle's attention
    time -- and the parity of the timed step on that sample: prepare codes
    and scales, output rows against the oracle (end to end), ExpCast bytes
    of query tile 0 given the kernel's own scores, and the k-means
    objective against the oracle's k-means from the same seed."""
    import numpy as np

    import oracle
    L, d = cfg.L, cfg.d
    qh, kh, vh = h00
    t0 = time.time()
    P = oracle.prepare_head(qh, kh, vh, perm00)
    t_prep = time.time() - t0
    if rows <= 0:  # size the sample to about 12 s of oracle time
        probe = min(L, 4 * oracle.num_threads())
        t0 = time.time()
        oracle.attention_head(P, L, 8, rows=(0, probe))
        per_row = (time.time() - t0) / probe
        rows = int(max(probe, min(L, 12.0 / max(per_row, 1e-9))))
    rows = min(rows, L)
    t0 = time.time()
    ref = oracle.attention_head(P, L, 8, rows=(0, rows))
    t_attn = time.time() - t0
    fl = 4.0 * rows * L * d
    cpu = None
    try:
        with open("/proc/cpuinfo") as f:
            cpu = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), None)
    except OSError:
        pass
    # parity of the timed step on head (0, 0)
    codes = {n: bool(np.array_equal(np.asarray(codes00[n]).view(np.uint8), np.asarray(P[n]).view(np.uint8)))
             for n in ("q8", "k8", "v8", "q_scale", "k_scale", "v_scale", "v_mean")}
    got = out00[:rows].astype(np.float64)
    refd = ref.astype(np.float64)
    rel = float(np.linalg.norm(got - refd) / np.linalg.norm(refd))
    mab = float(np.abs(got - refd).max() / np.abs(refd).max())
    _, s_k, b_k = dump00
    nr = min(256, L)
    S = s_k.cpu().numpy()[:nr]
    _, by_o, _, _ = oracle.attention_head(P, L, 8, rows=(0, nr), want_bytes=True, scores=S)
    by_k = b_k.cpu().numpy()[:nr, :L]
    mism = float(np.mean(by_k != by_o[:, :L]))
    t0 = time.time()
    nb = oracle.nblocks(L)
    _, _, obj_o = oracle.kmeans(vh, nb, 8, oracle.head_seed(seed, 0, 0, cfg.H))
    t_km = time.time() - t0
    parity = {"sample": "head (0,0)", "codes_and_scales_bit_exact": codes,
              "output_rel_l2": rel, "output_max_abs_over_max": mab, "output_rows": rows,
              "bar": "rel-L2 <= 1e-3, max-abs <= 1e-2 max|O| (end to end, oracle with exactly rounded scores)",
              "byte_mismatch_given_kernel_scores": mism, "byte_sample": "query tile 0 (%d rows x %d keys)" % (nr, L),
              "kmeans_objective_ratio": obj00 / float(obj_o), "kmeans_oracle_s": t_km}
    return {"value": fl / t_attn / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(), "cpu_model": cpu,
            "kind": "oracle",
            "sample": "head (0,0) of %s: oracle prepare (the GPU's k-means permutation, %.2fs) then blockwise "
                      "ExpCast attention for %d query rows x %d keys (%.2fs); k-means not included"
                      % (cfg.name, t_prep, rows, L, t_attn),
            "parity": parity}


if __name__ == "__main__":
    main()
