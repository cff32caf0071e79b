"""Independent reference attentions used to pin the oracle (test infrastructure only).

Written without the block-selection machinery and without importing
``oracle.infv2_ref``:

  * ``causal_attention``: textbook causal softmax attention with GQA head
    sharing, the result InfLLM v2 must reduce to when every block is selected
    (MiniCPM4 summary page, "InfLLM v2" section, paragraph "Initial and local
    tokens always selected": shorter than k*m tokens degenerates exactly to
    dense attention; "Design principles summary": no overhead for short inputs);
  * ``sink_window_attention``: attention restricted to the first ``init``
    blocks and the ``local`` most recent blocks, the result when top-k only
    holds the forced blocks (same paragraph: initial blocks get infinite
    relevance, the local window is always kept).
"""
from __future__ import annotations

import math

import numpy as np


def _softmax_attend(q: np.ndarray, keys: np.ndarray, vals: np.ndarray, scale: float) -> np.ndarray:
    logits = np.array([scale * float(np.dot(q, k)) for k in keys])
    top = logits.max()
    w = np.exp(logits - top)
    w = w / w.sum()
    return w @ vals


def causal_attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, positions, scale: float) -> np.ndarray:
    """q: [R][Hq][d] (row r at positions[r]); K, V: [Hkv][n][d].  Returns [R][Hq][d]."""
    hq, hkv = q.shape[1], K.shape[0]
    g = hq // hkv
    out = np.zeros(q.shape, dtype=np.float64)
    for r, i in enumerate(positions):
        for h in range(hq):
            kv = h // g
            out[r, h] = _softmax_attend(q[r, h], K[kv, :i + 1], V[kv, :i + 1], scale)
    return out


def sink_window_attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, positions, scale: float,
                          block: int, init: int, local: int) -> np.ndarray:
    """Attention over blocks {0..init-1} and the last ``local`` blocks up to position i."""
    hq, hkv = q.shape[1], K.shape[0]
    g = hq // hkv
    out = np.zeros(q.shape, dtype=np.float64)
    for r, i in enumerate(positions):
        cur = i // block
        keep = [t for t in range(i + 1)
                if (t // block) < init or (t // block) > cur - local]
        for h in range(hq):
            kv = h // g
            out[r, h] = _softmax_attend(q[r, h], K[kv, keep], V[kv, keep], scale)
    return out


def logsumexp_closed_form_geometric(a: float, b: float, count: int) -> float:
    """log sum_{j<count} exp(a*j + b), summed as a geometric series."""
    if count <= 0:
        return -math.inf
    if a == 0.0:
        return b + math.log(count)
    # sum = e^b (e^{a count} - 1) / (e^a - 1); written stably for a > 0
    if a > 0:
        return b + a * (count - 1) + math.log(-math.expm1(-a * count)) - math.log(-math.expm1(-a))
    return b + math.log(math.expm1(a * count) / math.expm1(a))
