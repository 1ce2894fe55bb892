"""Exact (fp64) non-causal softmax attention, the textbook definition.

TEST INFRASTRUCTURE ONLY (part of the oracle).  softmax(Q K^T / sqrt(d)) V
computed in float64 with NumPy's matmul and exp as library steps; no
blocking, no online softmax.  This is what every quantised result is an
approximation of (TensorRT-LLM blog, "Quantized Attention": an attention op
is QK^T, softmax, then PV).
"""
from __future__ import annotations

import numpy as np


def bf16_to_f32(u16: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32 values (exact widening)."""
    u = np.ascontiguousarray(u16, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32)


def attention_f64(q, k, v, rows=None):
    """q, k, v: [L, d] float arrays (any float dtype; promoted to float64).
    rows: optional (r0, r1) slice of query rows.  Returns [rows, d] float64."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    if rows is not None:
        q = q[rows[0]:rows[1]]
    d = q.shape[1]
    s = (q @ k.T) / np.sqrt(d)
    s -= s.max(axis=1, keepdims=True)
    p = np.exp(s)
    return (p @ v) / p.sum(axis=1, keepdims=True)
