"""CPU oracle for VC-Attention (V-Smooth + ExpCast-FP8).

TEST INFRASTRUCTURE ONLY.  This package is the plain, slow reference that
the GPU library is checked against.  Only the test suite, the smoke check
and the CPU-baseline leg of the benchmark may import it; the product path
never does.  It shares no code with the HIP library: the arithmetic lives in
``vc_oracle.c`` (plain C, compiled with gcc) and ``brute.py`` (NumPy fp64),
and this module only marshals NumPy arrays into it.

Every function states the passage of the VC-Attention pages it follows; the
C source carries the step-by-step definitions.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "vc_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

BLK = 128

CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-fno-fast-math",
          "-ffp-contract=off", "-Wall", "-Wno-unused-function"]


def build(force: bool = False) -> str:
    """Compile vc_oracle.c into liboracle.so with gcc (no GPU involved)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    with _lock:
        if _lib is None:
            build()
            L = ctypes.CDLL(_LIB)
            P = ctypes.c_void_p
            i32, i64, u64, f32 = ctypes.c_int, ctypes.c_int64, ctypes.c_uint64, ctypes.c_float
            L.vco_e4m3_decode.restype = ctypes.c_double
            L.vco_e4m3_decode.argtypes = [ctypes.c_uint8]
            L.vco_e4m3_encode.restype = ctypes.c_uint8
            L.vco_e4m3_encode.argtypes = [f32]
            L.vco_e4m3_encode_array.argtypes = [P, P, i64]
            L.vco_e4m3_decode_array.argtypes = [P, P, i64]
            L.vco_splitmix64.restype = u64
            L.vco_splitmix64.argtypes = [u64, u64]
            L.vco_head_seed.restype = u64
            L.vco_head_seed.argtypes = [u64, i32, i32, i32]
            L.vco_kmeans_init_indices.argtypes = [i32, i32, u64, P]
            L.vco_k_mean.argtypes = [P, i32, i32, P]
            L.vco_kmeans.restype = ctypes.c_double
            L.vco_kmeans.argtypes = [P, i32, i32, i32, i32, u64, P, P, P]
            L.vco_kmeans_warm.restype = ctypes.c_double
            L.vco_kmeans_warm.argtypes = [P, i32, i32, i32, i32, P, P, P, P]
            L.vco_stable_perm.argtypes = [P, i32, i32, P]
            L.vco_prepare_head.argtypes = [P, P, P, i32, i32, i32, i32, P, P, P, P, P, P, P, P, P]
            L.vco_expcast.argtypes = [P, i64, f32, f32, P]
            L.vco_expcast_rows.argtypes = [P, P, P, i64, P]
            L.vco_kb.restype = f32
            L.vco_kb.argtypes = [i32]
            L.vco_c0.restype = f32
            L.vco_c0.argtypes = [i32]
            L.vco_attention_rows.argtypes = [i32, i32, i32, i32, P, P, P, P, P, P, P, P, P, P,
                                             i32, i32, P, P, P, P, P, f32, P]
            L.vco_e2m1_decode.restype = ctypes.c_double
            L.vco_e2m1_decode.argtypes = [ctypes.c_uint8]
            L.vco_e2m1_encode_array.argtypes = [P, P, i64]
            L.vco_e8m0_exp.restype = i32
            L.vco_e8m0_exp.argtypes = [ctypes.c_double]
            L.vco_prepare_head_fp4v.argtypes = [P, P, P, i32, i32, i32, P, P, P, P, P, P, P, P]
            L.vco_sage_prepare_head.argtypes = [P, P, P, i32, i32, i32, i32, P, P, P, P, P, P]
            L.vco_sage_rows.argtypes = [i32, i32, i32, i32, i32, P, P, P, P, P, P, i32, i32, P, P, P, P]
            L.vco_num_threads.restype = i32
            L.vco_prepare.argtypes = [i32, i32, i32, i32, i32, i32, u64, i32, i32, P, P, P, P,
                                      P, P, P, P, P, P, P, P, P]
            _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# --------------------------------------------------------------------------
# E4M3FN codec (format definition; the "8 log2 v + 56" reading of the
# MarkTechPost abstract fixes exponent bias 7).
# --------------------------------------------------------------------------

def e4m3_encode(x) -> np.ndarray:
    """Saturating round-to-nearest-even fp32 -> E4M3FN byte."""
    x = _c(x, np.float32)
    out = np.empty(x.shape, np.uint8)
    lib().vco_e4m3_encode_array(_p(x), _p(out), x.size)
    return out


def e4m3_decode(b) -> np.ndarray:
    """E4M3FN byte -> exact value (float64)."""
    b = _c(b, np.uint8)
    out = np.empty(b.shape, np.float64)
    lib().vco_e4m3_decode_array(_p(b), _p(out), b.size)
    return out


# --------------------------------------------------------------------------
# Seeded draws (SplitMix64, counter-based).
# --------------------------------------------------------------------------

def splitmix64(seed: int, i: int) -> int:
    return int(lib().vco_splitmix64(seed & (2**64 - 1), i))


def head_seed(seed: int, b: int, h: int, H: int) -> int:
    return int(lib().vco_head_seed(seed & (2**64 - 1), b, h, H))


def kmeans_init_indices(L: int, k: int, seed_bh: int) -> np.ndarray:
    out = np.empty(k, np.int32)
    lib().vco_kmeans_init_indices(L, k, seed_bh, _p(out))
    return out


# --------------------------------------------------------------------------
# V-Smooth preprocessing (agihunt summary, V-Smooth bullet; MarkTechPost
# abstract; aikraft.ru "Reshenie").
# --------------------------------------------------------------------------

def k_mean(k_bf16_head: np.ndarray) -> np.ndarray:
    k = _c(k_bf16_head, np.uint16)
    L, d = k.shape
    out = np.empty(d, np.float32)
    lib().vco_k_mean(_p(k), L, d, _p(out))
    return out


def kmeans(v_bf16_head: np.ndarray, k: int, iters: int, seed_bh: int, history: bool = False):
    """Lloyd k-means on one head's value rows.  Returns (assign, centroids, J)
    or, with history=True, (assign, centroids, J_hist[iters+1])."""
    v = _c(v_bf16_head, np.uint16)
    L, d = v.shape
    a = np.empty(L, np.int32)
    C = np.empty((k, d), np.float32)
    hist = np.empty(iters + 1, np.float64) if history else None
    J = lib().vco_kmeans(_p(v), L, d, k, iters, seed_bh, _p(a), _p(C), _p(hist))
    return (a, C, hist) if history else (a, C, J)


def kmeans_warm(v_bf16_head: np.ndarray, init: np.ndarray, iters: int, history: bool = False):
    """Lloyd k-means on one head's value rows started from the given
    centroids init [k, d] (the previous grouping's centroids, carried across
    denoising steps).  Returns (assign, centroids, J) or, with history=True,
    (assign, centroids, J_hist[iters+1])."""
    v = _c(v_bf16_head, np.uint16)
    C0_ = _c(init, np.float32)
    L, d = v.shape
    k = C0_.shape[0]
    a = np.empty(L, np.int32)
    C = np.empty((k, d), np.float32)
    hist = np.empty(iters + 1, np.float64) if history else None
    J = lib().vco_kmeans_warm(_p(v), L, d, k, iters, _p(C0_), _p(a), _p(C), _p(hist))
    return (a, C, hist) if history else (a, C, J)


def stable_perm(assign: np.ndarray, k: int) -> np.ndarray:
    a = _c(assign, np.int32)
    out = np.empty(a.size, np.int32)
    lib().vco_stable_perm(_p(a), a.size, k, _p(out))
    return out


def nblocks(L: int) -> int:
    return (L + BLK - 1) // BLK


def prepare_head(q, k, v, perm, smooth_k: int = 1, v_mode: int = 0):
    """Steps a1, a6-a8 for one head given the permutation.  q, k, v: bf16 bits
    [L, d].  Returns a dict of q8 [Lp,d], k8 [Lp,d], v8 [nb,d,128] (natural
    slot order), q_scale [nb], k_scale [nb], v_scale [nb,d], v_mean [nb,d],
    kbar [d]."""
    q, k, v = (_c(a, np.uint16) for a in (q, k, v))
    perm = _c(perm, np.int32)
    L, d = q.shape
    nb = nblocks(L)
    Lp = nb * BLK
    o = dict(q8=np.empty((Lp, d), np.uint8), k8=np.empty((Lp, d), np.uint8),
             v8=np.empty((nb, d, BLK), np.uint8), q_scale=np.empty(nb, np.float32),
             k_scale=np.empty(nb, np.float32), v_scale=np.empty((nb, d), np.float32),
             v_mean=np.empty((nb, d), np.float32), kbar=np.empty(d, np.float32))
    lib().vco_prepare_head(_p(q), _p(k), _p(v), L, d, smooth_k, v_mode, _p(perm),
                           _p(o["q8"]), _p(o["k8"]), _p(o["v8"]), _p(o["q_scale"]),
                           _p(o["k_scale"]), _p(o["v_scale"]), _p(o["v_mean"]), _p(o["kbar"]))
    return o


def prepare(q, k, v, *, kmeans_k=0, kmeans_iters=8, seed=0, smooth_k=1, v_mode=0, perm_in=None):
    """Whole-tensor prepare over [B,H,L,d] bf16 bits (OpenMP over heads)."""
    q, k, v = (_c(a, np.uint16) for a in (q, k, v))
    B, H, L, d = q.shape
    nb = nblocks(L)
    Lp = nb * BLK
    o = dict(q8=np.empty((B, H, Lp, d), np.uint8), k8=np.empty((B, H, Lp, d), np.uint8),
             v8=np.empty((B, H, nb, d, BLK), np.uint8), q_scale=np.empty((B, H, nb), np.float32),
             k_scale=np.empty((B, H, nb), np.float32), v_scale=np.empty((B, H, nb, d), np.float32),
             v_mean=np.empty((B, H, nb, d), np.float32), perm=np.empty((B, H, L), np.int32),
             kmeans_obj=np.empty((B, H), np.float64))
    pin = None if perm_in is None else _c(perm_in, np.int32)
    lib().vco_prepare(B, H, L, d, kmeans_k, kmeans_iters, seed & (2**64 - 1), smooth_k, v_mode,
                      _p(q), _p(k), _p(v), _p(pin), _p(o["q8"]), _p(o["k8"]), _p(o["v8"]),
                      _p(o["q_scale"]), _p(o["k_scale"]), _p(o["v_scale"]), _p(o["v_mean"]),
                      _p(o["perm"]), _p(o["kmeans_obj"]))
    return o


# --------------------------------------------------------------------------
# ExpCast-FP8 (MarkTechPost abstract: one fused multiply-add from the
# log2-domain score, beta = -0.35; aikraft.ru: p = 2^z written as E4M3).
# --------------------------------------------------------------------------

def KB(z_off: int = 8) -> np.float32:
    return np.float32(lib().vco_kb(z_off))


def C0(d: int) -> np.float32:
    return np.float32(lib().vco_c0(d))


def expcast(S, c8, krow) -> np.ndarray:
    """byte = min(max(rne(fma(S, c8, krow)), 0), 126); c8, krow scalars or
    arrays broadcastable to S."""
    S = _c(S, np.float32)
    if np.ndim(c8) == 0 and np.ndim(krow) == 0:
        out = np.empty(S.shape, np.uint8)
        lib().vco_expcast(_p(S), S.size, float(np.float32(c8)), float(np.float32(krow)), _p(out))
        return out
    c8a = _c(np.broadcast_to(np.float32(c8) if np.ndim(c8) == 0 else c8, S.shape), np.float32)
    kra = _c(np.broadcast_to(np.float32(krow) if np.ndim(krow) == 0 else krow, S.shape), np.float32)
    out = np.empty(S.shape, np.uint8)
    lib().vco_expcast_rows(_p(S), _p(c8a), _p(kra), S.size, _p(out))
    return out


def expcast_z(z, z_off: int = 8) -> np.ndarray:
    """ExpCast byte of p = 2^(z + z_off) for a log2-domain score z <= 0
    (running max already subtracted): fma(z, 8, KB)."""
    return expcast(z, np.float32(8.0), KB(z_off))


# --------------------------------------------------------------------------
# Blockwise attention.
# --------------------------------------------------------------------------

def skip_threshold(skip_lambda: float) -> np.float32:
    """fp32(log2(lambda)) in double rounded once; -inf (reject nothing) for
    lambda = 0.  The pages' rule exp(m~ - m) < lambda ([TRT] "Sparse
    Attention with Skip Softmax") is then fp32(t - m) < this, in log2 units."""
    lam = float(skip_lambda)
    if not (0.0 <= lam <= 1.0):
        raise ValueError("skip_lambda must lie in [0, 1]")
    return np.float32(-np.inf) if lam == 0.0 else np.float32(np.log2(np.float64(lam)))


def attention_head(prep: dict, L: int, z_off: int = 8, rows=None, want_bytes=False, scores=None,
                   skip_lambda: float = 0.0, prob_cast: int = 0):
    """Quantised VC-Attention for one head from prepare_head() output.
    rows: (r0, r1) or None for all.  Returns O [r1-r0, d] fp32 (and, with
    want_bytes, the ExpCast bytes, S values and pre-rounding y values
    [r1-r0, Lp] of every block).  scores: optional fp32 [r1-r0, Lp] used in
    place of the exactly rounded Q8 K8^T sums (every later step is unique
    given the scores).  skip_lambda: the Skip Softmax threshold (0: off).
    prob_cast: 0 ExpCast-FP8 bytes (the method), 1 exp-then-cast (the fp32
    exponential 2^z, correctly rounded, cast to E4M3; y then holds z)."""
    if prob_cast not in (0, 1):
        raise ValueError("prob_cast must be 0 or 1")
    q8 = _c(prep["q8"], np.uint8)
    k8 = _c(prep["k8"], np.uint8)
    v8 = _c(prep["v8"], np.uint8)
    qs, ks = _c(prep["q_scale"], np.float32), _c(prep["k_scale"], np.float32)
    vs, vm = _c(prep["v_scale"], np.float32), _c(prep["v_mean"], np.float32)
    d = q8.shape[1]
    Lp = k8.shape[0]
    r0, r1 = (0, L) if rows is None else rows
    out = np.empty((r1 - r0, d), np.float32)
    by = np.empty((r1 - r0, Lp), np.uint8) if want_bytes else None
    S = np.empty((r1 - r0, Lp), np.float32) if want_bytes else None
    y = np.empty((r1 - r0, Lp), np.float32) if want_bytes else None
    sin = None
    if scores is not None:
        sin = _c(scores, np.float32)
        assert sin.shape == (r1 - r0, Lp)
    lib().vco_attention_rows(2 if prob_cast else 0, L, d, z_off, _p(q8), _p(k8), _p(v8), _p(qs), _p(ks), _p(vs),
                             _p(vm), None, None, None, r0, r1, _p(out), _p(by), _p(S), _p(y), _p(sin),
                             skip_threshold(skip_lambda), None)
    return (out, by, S, y) if want_bytes else out


def attention_exact_blockwise(qf, kf_perm, v_perm, v_mean, skip_lambda: float = 0.0, rows=None):
    """Mode 1 of the blockwise loop: no quantisation, exact exp2, in double.
    qf [L,d], kf_perm [L,d] keys in permuted order, v_perm [L,d] values in
    permuted order, v_mean [nb,d] any per-block vector (the algebra must hold
    for any mean).  skip_lambda as in attention_head.  rows: (r0, r1) or None
    for all.  Returns O [r1-r0,d] (fp32)."""
    qf = _c(qf, np.float64)
    L, d = qf.shape
    nb = nblocks(L)
    Lp = nb * BLK
    kf = np.zeros((Lp, d), np.float64)
    kf[:L] = kf_perm
    vp = np.zeros((Lp, d), np.float64)
    vp[:L] = v_perm
    vm = _c(v_mean, np.float32)
    rf = np.zeros((nb, d, BLK), np.float64)
    for b in range(nb):
        n = min(BLK, L - b * BLK)
        rf[b, :, :n] = (vp[b * BLK:b * BLK + n] - vm[b].astype(np.float64)).T
    r0, r1 = (0, L) if rows is None else rows
    out = np.empty((r1 - r0, d), np.float32)
    lib().vco_attention_rows(1, L, d, 8, None, None, None, None, None, None, _p(vm),
                             _p(qf), _p(kf), _p(rf), r0, r1, _p(out), None, None, None, None,
                             skip_threshold(skip_lambda), None)
    return out


# --------------------------------------------------------------------------
# SAGE-style baseline (TensorRT-LLM blog, "Quantized Attention": QK^T in
# INT8 or FP8, PV in FP8, q/k/v block sizes 1/16/1 with the V scale per
# channel).  The readings where the blog is silent are listed in vc_oracle.c.
# --------------------------------------------------------------------------

SAGE_QK = {"int8": 1, "fp8": 0}


def attention_p_only(qf, kf_perm, v_perm, v_mean, z_off: int = 8, rows=None):
    """Mode 4 of the blockwise loop: real-valued scores (double sums rounded
    once to fp32, scale 1) and values, with only the probabilities
    quantised, by ExpCast-FP8 against the running maximum as in the method.
    Arguments as attention_exact_blockwise.  Returns O [L,d] (fp32)."""
    qf = _c(qf, np.float64)
    L, d = qf.shape
    nb = nblocks(L)
    Lp = nb * BLK
    kf = np.zeros((Lp, d), np.float64)
    kf[:L] = kf_perm
    vp = np.zeros((Lp, d), np.float64)
    vp[:L] = v_perm
    vm = _c(v_mean, np.float32)
    rf = np.zeros((nb, d, BLK), np.float64)
    for b in range(nb):
        n = min(BLK, L - b * BLK)
        rf[b, :, :n] = (vp[b * BLK:b * BLK + n] - vm[b].astype(np.float64)).T
    r0, r1 = (0, L) if rows is None else rows
    out = np.empty((r1 - r0, d), np.float32)
    lib().vco_attention_rows(4, L, d, z_off, None, None, None, None, None, None, _p(vm),
                             _p(qf), _p(kf), _p(rf), r0, r1, _p(out), None, None, None, None,
                             np.float32(-np.inf), None)
    return out


def attention_parts(q, k, v, perm, z_off: int = 8, smooth_k: int = 1, rows=None):
    """The method's output for one head with each quantised quantity switched
    on alone, for the error decomposition of the value term ([MTP] abstract:
    after QK smoothing, the value term carries most of the output error).
    q, k, v: bf16 bits [L,d]; perm [L]; rows (r0, r1) or None for all.
    Returns a dict of O [r1-r0,d] fp32:
      exact -- no quantisation (softmax(Q K^T / sqrt(d)) V, blockwise in
               double, mode 1);
      qk    -- Q and K replaced by their dequantised per-block FP8 codes
               (K after its mean is subtracted), probabilities and values
               exact;
      p     -- scores and values exact, probabilities ExpCast-FP8 (mode 4);
      v     -- scores and probabilities exact, V replaced by its V-Smooth
               reconstruction mean + s_v E4M3(code) in the permuted order;
      all   -- the method (mode 0)."""
    o = prepare_head(q, k, v, perm, smooth_k)
    perm = _c(perm, np.int64)
    L, d = _c(q, np.uint16).shape
    nb = nblocks(L)
    qf = bf16_to_f32(q).astype(np.float64)
    kp = bf16_to_f32(k).astype(np.float64)[perm]
    vp = bf16_to_f32(v).astype(np.float64)[perm]
    qb = np.minimum(np.arange(L) // BLK, nb - 1)
    qd = e4m3_decode(o["q8"][:L]) * o["q_scale"][qb][:, None].astype(np.float64)
    kd = e4m3_decode(o["k8"][:L]) * o["k_scale"][qb][:, None].astype(np.float64)
    r = e4m3_decode(o["v8"]) * o["v_scale"][:, :, None].astype(np.float64)          # [nb, d, 128]
    vd = (o["v_mean"][:, :, None].astype(np.float64) + r).transpose(0, 2, 1).reshape(nb * BLK, d)[:L]
    mu = o["v_mean"]
    return {"exact": attention_exact_blockwise(qf, kp, vp, mu, rows=rows),
            "qk": attention_exact_blockwise(qd, kd, vp, mu, rows=rows),
            "p": attention_p_only(qf, kp, vp, mu, z_off, rows=rows),
            "v": attention_exact_blockwise(qf, kp, vd, mu, rows=rows),
            "all": attention_head(o, L, z_off, rows=rows)}


def sage_prepare_head(q, k, v, qk_dtype: str = "int8", smooth_k: int = 1):
    """One head, sequence order.  q, k, v: bf16 bits [L, d].  Returns q8, k8
    [Lp, d] (INT8 two's complement or E4M3 bytes), v8 [nb, d, 128] E4M3
    (natural slot order), q_scale [Lp], k_scale [Lp/16], v_scale [d]."""
    q, k, v = (_c(a, np.uint16) for a in (q, k, v))
    L, d = q.shape
    nb = nblocks(L)
    Lp = nb * BLK
    o = dict(q8=np.empty((Lp, d), np.uint8), k8=np.empty((Lp, d), np.uint8),
             v8=np.empty((nb, d, BLK), np.uint8), q_scale=np.empty(Lp, np.float32),
             k_scale=np.empty(Lp // 16, np.float32), v_scale=np.empty(d, np.float32))
    lib().vco_sage_prepare_head(_p(q), _p(k), _p(v), L, d, SAGE_QK[qk_dtype], smooth_k,
                                _p(o["q8"]), _p(o["k8"]), _p(o["v8"]), _p(o["q_scale"]),
                                _p(o["k_scale"]), _p(o["v_scale"]))
    return o


def sage_attention_head(prep: dict, L: int, qk_dtype: str = "int8", z_off: int = 8, prob_cast: int = 1,
                        rows=None, want_bytes=False, scores=None):
    """SAGE-style attention for one head from sage_prepare_head() output.
    Returns O [r1-r0, d] fp32 (with want_bytes also the P bytes and scores
    [r1-r0, Lp]).  scores: optional fp32 [r1-r0, Lp] in place of the exact
    Q8 K8^T sums.  prob_cast 1: exp-then-cast P bytes; 0: ExpCast."""
    if prob_cast not in (0, 1):
        raise ValueError("prob_cast must be 0 or 1")
    q8, k8, v8 = (_c(prep[n], np.uint8) for n in ("q8", "k8", "v8"))
    qs, ks, vs = (_c(prep[n], np.float32) for n in ("q_scale", "k_scale", "v_scale"))
    d = q8.shape[1]
    Lp = k8.shape[0]
    r0, r1 = (0, L) if rows is None else rows
    out = np.empty((r1 - r0, d), np.float32)
    by = np.empty((r1 - r0, Lp), np.uint8) if want_bytes else None
    S = np.empty((r1 - r0, Lp), np.float32) if want_bytes else None
    sin = None
    if scores is not None:
        sin = _c(scores, np.float32)
        assert sin.shape == (r1 - r0, Lp)
    lib().vco_sage_rows(prob_cast, SAGE_QK[qk_dtype], L, d, z_off, _p(q8), _p(k8), _p(v8), _p(qs), _p(ks),
                        _p(vs), r0, r1, _p(out), _p(by), _p(S), _p(sin))
    return (out, by, S) if want_bytes else out


# --------------------------------------------------------------------------
# 4-bit V-Smooth (MarkTechPost abstract: 4-bit V-Smooth; ExpCast applies to
# the 8-bit kernel only): E2M1 residual and probabilities with power-of-two
# (E8M0) scales per 32-key group.  Readings in vc_oracle.c.
# --------------------------------------------------------------------------

def e2m1_decode(c) -> np.ndarray:
    c = np.asarray(c, np.uint8)
    table = np.array([lib().vco_e2m1_decode(t) for t in range(16)], np.float64)
    return table[c & 15]


def e2m1_encode(x) -> np.ndarray:
    x = _c(x, np.float64)
    out = np.empty(x.shape, np.uint8)
    lib().vco_e2m1_encode_array(_p(x), _p(out), x.size)
    return out


def e8m0_exp(A: float) -> int:
    return int(lib().vco_e8m0_exp(float(A)))


def prepare_head_fp4v(q, k, v, perm, smooth_k: int = 1):
    """As prepare_head, with the V residual in E2M1: v4 [nb, d, 128] codes
    (natural key order) and v_exp [nb, d, 4] (e + 127 per key group) in
    place of v8 and v_scale."""
    q, k, v = (_c(a, np.uint16) for a in (q, k, v))
    perm = _c(perm, np.int32)
    L, d = q.shape
    nb = nblocks(L)
    Lp = nb * BLK
    o = dict(q8=np.empty((Lp, d), np.uint8), k8=np.empty((Lp, d), np.uint8),
             v4=np.empty((nb, d, BLK), np.uint8), v_exp=np.empty((nb, d, 4), np.uint8),
             q_scale=np.empty(nb, np.float32), k_scale=np.empty(nb, np.float32),
             v_mean=np.empty((nb, d), np.float32))
    lib().vco_prepare_head_fp4v(_p(q), _p(k), _p(v), L, d, smooth_k, _p(perm), _p(o["q8"]), _p(o["k8"]),
                                _p(o["v4"]), _p(o["v_exp"]), _p(o["q_scale"]), _p(o["k_scale"]),
                                _p(o["v_mean"]))
    return o


def attention_head_fp4v(prep: dict, L: int, z_off: int = 8, rows=None, want_bytes=False, scores=None):
    """4-bit P V (mode 3) for one head from prepare_head_fp4v() output.
    Returns O [r1-r0, d] fp32 (with want_bytes also the E2M1 codes of P, the
    scores and the values phat, each [r1-r0, Lp])."""
    q8, k8, v4, ve = (_c(prep[n], np.uint8) for n in ("q8", "k8", "v4", "v_exp"))
    qs, ks, vm = (_c(prep[n], np.float32) for n in ("q_scale", "k_scale", "v_mean"))
    d = q8.shape[1]
    Lp = k8.shape[0]
    r0, r1 = (0, L) if rows is None else rows
    out = np.empty((r1 - r0, d), np.float32)
    by = np.empty((r1 - r0, Lp), np.uint8) if want_bytes else None
    S = np.empty((r1 - r0, Lp), np.float32) if want_bytes else None
    y = np.empty((r1 - r0, Lp), np.float32) if want_bytes else None
    sin = None
    if scores is not None:
        sin = _c(scores, np.float32)
        assert sin.shape == (r1 - r0, Lp)
    lib().vco_attention_rows(3, L, d, z_off, _p(q8), _p(k8), _p(v4), _p(qs), _p(ks), None, _p(vm),
                             None, None, None, r0, r1, _p(out), _p(by), _p(S), _p(y), _p(sin),
                             np.float32(-np.inf), _p(ve))
    return (out, by, S, y) if want_bytes else out


def num_threads() -> int:
    return int(lib().vco_num_threads())


from .brute import attention_f64, bf16_to_f32  # noqa: E402,F401
