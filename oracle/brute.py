"""Brute-force re-derivation of InfLLM v2 selection and attention on tiny inputs.

Test infrastructure only.  Every definition of the MiniCPM4 summary page
("InfLLM v2" section: paragraphs "Semantic kernels for block relevance
scoring" with eqs. S, r_kernel and r_block, "Query group sharing" with eq.
r_group, "Top-K implementation", "Initial and local tokens always selected")
is evaluated here with pure-Python loops and exact summation (math.fsum),
and the top-k is found by enumerating every subset: the chosen set must
maximise the exact (rational) total score, and among maximisers the one with
the smallest block indices wins.  Does not import ``oracle.infv2_ref``.
"""
from __future__ import annotations

import itertools
import math
import struct
from fractions import Fraction
from typing import List, Sequence


def to_fp32(x: float) -> float:
    """Nearest float32 (the C conversion rounds to nearest, ties to even)."""
    return struct.unpack("f", struct.pack("f", x))[0]


def brute_compress(K: Sequence[Sequence[float]], upto: int, p: int, s: int) -> List[List[float]]:
    """Mean of every kernel lying wholly in tokens [0, upto)."""
    d = len(K[0])
    out = []
    j = 0
    while j * s + p <= upto:
        out.append([math.fsum(K[t][e] for t in range(j * s, j * s + p)) / p for e in range(d)])
        j += 1
    return out


def brute_coarse_lse(qg, K, i: int, coarse: int, score_scale: float = 1.0):
    """Per-head LogSumExp over the coarse kernels (spans of ``coarse`` tokens at
    stride ``coarse``) lying wholly in [0, i]; None if there is none."""
    kb = brute_compress(K, i + 1, coarse, coarse)
    if not kb:
        return None
    out = []
    for h in range(len(qg)):
        z = [score_scale * math.fsum(qg[h][e] * row[e] for e in range(len(row))) for row in kb]
        top = max(z)
        out.append(top + math.log(math.fsum(math.exp(v - top) for v in z)))
    return out


def brute_block_scores(qg, K, i: int, m: int, p: int, s: int, score_scale: float = 1.0,
                       round_ck=None, lse_override=None):
    """Block scores S_j (j = 0..floor(i/m)) for query heads ``qg`` at position i
    (with ``lse_override`` as the per-head normaliser when given)."""
    G = len(qg)
    kb = brute_compress(K, i + 1, p, s)
    if round_ck is not None:
        kb = [[round_ck(x) for x in row] for row in kb]
    z = [[score_scale * math.fsum(qg[h][e] * kb[j][e] for e in range(len(kb[j])))
          for j in range(len(kb))] for h in range(G)]
    lse = []
    for h in range(G):
        if not z[h]:
            lse.append(-math.inf)
            continue
        top = max(z[h])
        lse.append(top + math.log(math.fsum(math.exp(v - top) for v in z[h])))
    if lse_override is not None and kb:
        lse = list(lse_override)
    R = [math.fsum(math.exp(z[h][j] - lse[h]) for h in range(G)) / G for j in range(len(kb))]
    c = i // m
    S = []
    for blk in range(c + 1):
        vals = [R[j] for j in range(len(kb)) if j * s < (blk + 1) * m and j * s + p > blk * m]
        S.append(max(vals) if vals else -math.inf)
    return S, R, lse


def brute_select(S: Sequence[float], c: int, k: int, init: int, local: int) -> List[int]:
    """Top-k with forced blocks by exhaustive search over candidate subsets."""
    forced = sorted({b for b in range(c + 1) if b < init or b > c - local})
    if c + 1 <= k:
        return list(range(c + 1))
    cand = [b for b in range(c + 1) if b not in forced]
    kp = k - len(forced)
    def exact(v):
        return Fraction(-1) if v == -math.inf else Fraction(v)
    best_sum, best = None, None
    for sub in itertools.combinations(cand, kp):     # combinations come in lexicographic order
        tot = sum((exact(S[b]) for b in sub), Fraction(0))
        if best_sum is None or tot > best_sum:
            best_sum, best = tot, sub
    return sorted(forced + list(best))


def brute_attend(qh, K, V, i: int, sel: Sequence[int], m: int, scale: float) -> List[float]:
    """One head's softmax attention at position i over the selected blocks."""
    n = len(K)
    toks = sorted({t for b in sel if b >= 0 for t in range(b * m, min((b + 1) * m, n)) if t <= i})
    a = [scale * math.fsum(qh[e] * K[t][e] for e in range(len(qh))) for t in toks]
    top = max(a)
    w = [math.exp(x - top) for x in a]
    tot = math.fsum(w)
    d = len(V[0])
    return [math.fsum(w[r] * V[t][e] for r, t in enumerate(toks)) / tot for e in range(d)]
