"""Plain float64 CPU oracle for the InfLLM v2 sparse-attention hot path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only the test-suite, the smoke check and the bench's
CPU-baseline leg use it.  It shares no code with the HIP library.

Source of every step: the MiniCPM4 technical-report summary page
("MiniCPM4: Ultra-Efficient LLMs on End Devices", paper-graph-ui), section
"InfLLM v2: Trainable Sparse Attention for Both Prefilling and Decoding",
cited below as [IV2 <paragraph>]; the block-score formula is also restated
cleanly in the Korean review page (dimensionstp), section "3-2. Module
breakdown, 1) InfLLM v2", cited as [Review 3-2].

Readings taken where the pages are silent or garbled:
  * only complete kernels exist: n_c(n) = floor((n - p)/s) + 1 for n >= p;
  * row i (absolute position) sees kernel j^ only if it lies wholly in
    [0, i]: j^*s + p <= i + 1 (causality of the pooled keys);
  * selection logits are score_scale * (q . kbar) with score_scale = 1 as
    printed (the ABI keeps it a parameter); attention uses attn_scale,
    default 1/sqrt(d) (standard scaled dot-product attention);
  * the LogSumExp is taken per query head; the group score is the mean of the
    per-head softmax values per kernel; the block score is then the max over
    the visible kernels overlapping the block;
  * blocks are 0 .. ceil(n/m) - 1, the last one possibly partial;
  * forced set F = {0 .. init-1} U {c-local+1 .. c} with c = floor(i/m);
    top-k counts the forced blocks; if c + 1 <= k every block is taken
    (exact dense degeneration); ties in the score go to the lower block;
  * compressed keys are the exact mean rounded once to their storage type
    (fp32 by default, or bf16).

Every function here is pinned by tests/test_oracle_pins.py against closed
forms, invariants, a brute-force loop implementation (oracle/brute.py) and an
independent dense attention (oracle/dense_ref.py); the backward functions are
pinned by central differences of the forward, by autograd of dense causal
attention when every block is selected, and by the softmax invariants.
"""
from __future__ import annotations

from dataclasses import dataclass
from functools import lru_cache
from typing import Iterable, List, Optional, Sequence

import numpy as np

NEG_INF = -np.inf


# ---------------------------------------------------------------------------
# parameters
# ---------------------------------------------------------------------------
@dataclass(frozen=True)
class Params:
    """Hyper-parameters of the method (names follow the pages' notation)."""
    head_dim: int          # d
    num_q_heads: int       # Hq
    num_kv_heads: int      # Hkv; |group| = Hq / Hkv
    block_size: int        # m   [IV2 Block-level key-value partitioning]
    kernel_size: int       # p   [IV2 Semantic kernels]
    kernel_stride: int     # s   [IV2 Semantic kernels]
    topk: int              # k, counts the forced blocks
    init_blocks: int = 1   # [IV2 Initial and local tokens always selected]
    local_blocks: int = 1
    score_scale: float = 1.0
    attn_scale: Optional[float] = None   # None -> 1/sqrt(d)
    ck_dtype: str = "fp32"               # storage of the compressed keys

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def scale(self) -> float:
        return 1.0 / np.sqrt(self.head_dim) if self.attn_scale is None else float(self.attn_scale)


# ---------------------------------------------------------------------------
# storage rounding (round to nearest, ties to even) of exact float64 values
# ---------------------------------------------------------------------------
def round_to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64 values once to the fp32 or bf16 grid, ties to even.

    fp32 and bf16 share the exponent range (normal binades from 2^-126); fp32
    keeps 23 fraction bits, bf16 keeps 7.  Values are returned as float64.
    """
    x = np.asarray(x, dtype=np.float64)
    if dtype == "fp64":
        return x.copy()
    frac_bits = {"fp32": 23, "bf16": 7}[dtype]
    _, e = np.frexp(x)                       # x = f * 2^e with 0.5 <= |f| < 1
    binade = np.maximum(e - 1, -126)         # floor(log2|x|), clamped to the subnormal range
    q = binade - frac_bits                   # exponent of one unit in the last place
    y = np.ldexp(np.rint(np.ldexp(x, -q)), q)
    y = np.where(x == 0.0, x, y)
    big = np.abs(y) >= 2.0 ** 128
    return np.where(big, np.copysign(np.inf, x), y)


# ---------------------------------------------------------------------------
# step 1: semantic kernels and compressed keys
# ---------------------------------------------------------------------------
def num_kernels(n: int, p: int, s: int) -> int:
    """Number of complete kernels S_j^ = K[j^ s : j^ s + p] over n keys.

    [IV2 Semantic kernels, eq. S]: kernels start every s tokens and span p
    tokens; only kernels whose p keys all exist are formed.
    """
    if n < p:
        return 0
    return (n - p) // s + 1


def compress_keys(K: np.ndarray, p: int, s: int, ck_dtype: str = "fp32") -> np.ndarray:
    """Compressed keys kbar_j^ = Mean(K[j^ s : j^ s + p]) per KV head.

    [IV2 Semantic kernels, "What this computes"; "Why mean pooling"].
    K: [Hkv][n][d] float64.  Returns [Hkv][n_c][d] float64 holding the mean
    rounded once to ``ck_dtype``.
    """
    hkv, n, d = K.shape
    nc = num_kernels(n, p, s)
    ck = np.empty((hkv, nc, d), dtype=np.float64)
    for jh in range(nc):
        ck[:, jh, :] = K[:, jh * s: jh * s + p, :].sum(axis=1) / p
    return round_to_storage(ck, ck_dtype)


def append_token(K: np.ndarray, V: np.ndarray, n: int, k_new: np.ndarray, v_new: np.ndarray,
                 ck: np.ndarray, p: int, s: int, ck_dtype: str = "fp32") -> int:
    """One decode step's cache update, in place: the new token's key and value
    go to position n, and the kernel the token completes (if any) gets its
    compressed key.  Returns the new length n + 1.

    [IV2 Semantic kernels] with the complete-kernel reading: kernel j^ covers
    [j^ s, j^ s + p), so the token at position n completes kernel
    (n + 1 - p) / s exactly when n + 1 >= p and s divides n + 1 - p.
    K, V: [Hkv][cap][d]; k_new, v_new: [Hkv][d]; ck: [Hkv][ccap][d].
    """
    K[:, n, :] = k_new
    V[:, n, :] = v_new
    if n + 1 >= p and (n + 1 - p) % s == 0:
        jh = (n + 1 - p) // s
        ck[:, jh, :] = round_to_storage(K[:, jh * s: jh * s + p, :].sum(axis=1) / p, ck_dtype)
    return n + 1


# ---------------------------------------------------------------------------
# step 2: which kernels touch which block
# ---------------------------------------------------------------------------
@lru_cache(maxsize=64)
def _overlap_table(nblocks: int, nkernels: int, m: int, p: int, s: int) -> np.ndarray:
    """Padded table [nblocks][w] of kernel ids whose span meets block j, -1 padded.

    [IV2 Semantic kernels, eq. r_block; Review 3-2]: a kernel counts for block
    B_j when S_j^ and B_j share a token, i.e. [j^ s, j^ s + p) meets
    [j m, (j+1) m).  Evaluated literally for every (block, kernel) pair.
    """
    starts = np.arange(nkernels, dtype=np.int64) * s
    rows: List[np.ndarray] = []
    for j in range(nblocks):
        meets = (starts < (j + 1) * m) & (starts + p > j * m)
        rows.append(np.nonzero(meets)[0])
    width = max([r.shape[0] for r in rows] + [1])
    tab = np.full((nblocks, width), -1, dtype=np.int64)
    for j, r in enumerate(rows):
        tab[j, :r.shape[0]] = r
    tab.setflags(write=False)
    return tab


def _pow2(x: int) -> int:
    return 1 << max(0, int(x) - 1).bit_length()


def block_overlaps(nblocks: int, nkernels: int, m: int, p: int, s: int) -> np.ndarray:
    """Rows 0..nblocks-1 of the overlap table, counting kernels 0..nkernels-1 only.

    The table is evaluated once for power-of-two sizes and sliced; kernel ids at
    or beyond ``nkernels`` are replaced by -1.
    """
    tab = _overlap_table(_pow2(nblocks), _pow2(nkernels), int(m), int(p), int(s))[:nblocks]
    return np.where(tab < nkernels, tab, -1)


# ---------------------------------------------------------------------------
# steps 3-6: scores and selection for one query position and one group
# ---------------------------------------------------------------------------
@dataclass
class RowSelection:
    sel: np.ndarray        # int64 [k], ascending, -1 padded
    S: np.ndarray          # float64 [c+1] block scores (-inf: no visible kernel)
    forced: np.ndarray     # bool [c+1]
    R: np.ndarray          # float64 [n_vis] group score per visible kernel
    lse: np.ndarray        # float64 [G] per-head LogSumExp
    z: np.ndarray          # float64 [G][n_vis] logits
    dense: bool            # c + 1 <= k: every block taken
    kprime: int            # number of scored picks, k - |F| (0 when dense)


def forced_blocks(c: int, init: int, local: int) -> np.ndarray:
    """F = initial blocks U local window, inside [0, c].

    [IV2 Initial and local tokens always selected]: B_0 gets infinite score;
    the blocks of a local window ending at the query's own block are always kept.
    """
    f = np.zeros(c + 1, dtype=bool)
    f[:max(0, min(init, c + 1))] = True
    f[max(0, c - local + 1):c + 1] = True
    return f


def select_row(qg: np.ndarray, ckg: np.ndarray, i: int, prm: Params,
               lse: Optional[np.ndarray] = None) -> RowSelection:
    """Block scores and top-k selection for query position i of one group.

    qg: [G][d] the group's query heads (float64); ckg: [n_c][d] compressed keys
    of the group's KV head (at least the kernels visible to row i).  lse: a
    per-head normaliser to use in place of the exact LogSumExp of pass 1 (the
    coarse approximation, select_row_coarse); None takes the exact one.
    """
    lse_in = lse
    m, p, s = prm.block_size, prm.kernel_size, prm.kernel_stride
    G = qg.shape[0]
    vis = num_kernels(i + 1, p, s)               # kernels lying wholly in [0, i]
    c = i // m                                   # the query's own block

    # [IV2 Semantic kernels, eq. r_kernel]: logits and a softmax over kernels,
    # per head; [IV2 Top-K implementation]: pass 1 LogSumExp, pass 2 normalise.
    z = prm.score_scale * (qg @ ckg[:vis].T)     # [G][vis]
    if vis > 0:
        zmax = z.max(axis=1)
        lse = zmax + np.log(np.exp(z - zmax[:, None]).sum(axis=1))
        if lse_in is not None:
            lse = np.asarray(lse_in, dtype=np.float64)
        prob = np.exp(z - lse[:, None])          # r_kernel per head
        # [IV2 Query group sharing, eq. r_group]: mean over the group's heads
        R = prob.sum(axis=0) / G
    else:
        lse = np.full(G, NEG_INF)
        R = np.zeros(0)

    # [IV2 eq. r_block; Review 3-2]: max over the kernels meeting the block
    tab = block_overlaps(c + 1, vis, m, p, s)
    r_ext = np.concatenate([R, [NEG_INF]])
    S = r_ext[np.where(tab >= 0, tab, vis)].max(axis=1)

    forced = forced_blocks(c, prm.init_blocks, prm.local_blocks)
    k = prm.topk
    if c + 1 <= k:
        # [IV2 Initial and local tokens ...]: shorter than k*m -> dense
        chosen = np.arange(c + 1, dtype=np.int64)
        dense, kprime = True, 0
    else:
        kprime = k - int(forced.sum())
        cand = np.nonzero(~forced)[0]
        order = np.lexsort((cand, -S[cand]))     # score descending, then lower block first
        top = cand[order[:kprime]]
        chosen = np.sort(np.concatenate([np.nonzero(forced)[0], top]))
        dense = False
    sel = np.full(k, -1, dtype=np.int64)
    sel[:chosen.shape[0]] = chosen
    return RowSelection(sel=sel, S=S, forced=forced, R=R, lse=lse, z=z, dense=dense,
                        kprime=kprime)


def coarse_lse(qg: np.ndarray, ckcg: np.ndarray, i: int, prm: Params, coarse: int):
    """[IV2 Efficient LSE approximation]: the per-head LogSumExp of pass 1 taken
    over coarse kernels instead of the fine ones.  Reading: a coarse kernel is a
    span of `coarse` tokens at stride `coarse` (complete ones only, as for the
    fine kernels), its key the mean of those keys (compress_keys(K, coarse,
    coarse)), and row i sees it when it lies wholly in [0, i].  Its logits use
    the same score_scale.  Returns None when row i sees no coarse kernel.
    """
    vis = num_kernels(i + 1, coarse, coarse)
    if vis == 0:
        return None
    z = prm.score_scale * (qg @ ckcg[:vis].T)
    zmax = z.max(axis=1)
    return zmax + np.log(np.exp(z - zmax[:, None]).sum(axis=1))


def select_row_coarse(qg: np.ndarray, ckg: np.ndarray, ckcg: np.ndarray, i: int, prm: Params,
                      coarse: int) -> RowSelection:
    """Selection with the coarse-kernel LogSumExp in pass 1 and the fine kernels
    in pass 2 ([IV2 Efficient LSE approximation; Complexity analysis, Stage 1]).
    A row that sees no coarse kernel keeps the exact normaliser."""
    return select_row(qg, ckg, i, prm, lse=coarse_lse(qg, ckcg, i, prm, coarse))


# ---------------------------------------------------------------------------
# step 7: exact softmax attention over the selected blocks
# ---------------------------------------------------------------------------
def selected_tokens(sel: np.ndarray, i: int, n: int, m: int) -> np.ndarray:
    """T_i = union of the selected blocks' tokens, limited to t < n and t <= i."""
    toks = [np.arange(j * m, min((j + 1) * m, n, i + 1), dtype=np.int64)
            for j in sel.tolist() if j >= 0]
    if not toks:
        return np.zeros(0, dtype=np.int64)
    return np.unique(np.concatenate(toks))


def attend_row(qg: np.ndarray, Kg: np.ndarray, Vg: np.ndarray, i: int, sel: np.ndarray,
               prm: Params):
    """Softmax attention of the group's heads at position i over the selected blocks.

    [IV2 Complexity analysis, Stage 2]: each query token attends the k*m tokens
    of its selected blocks; [IV2 opening]: standard weighted sum of values.
    Returns (o [G][d], lse [G], prob_row_sum [G]).
    """
    n = Kg.shape[0]
    T = selected_tokens(sel, i, n, prm.block_size)
    a = prm.scale * (qg @ Kg[T].T)               # [G][|T|]
    amax = a.max(axis=1)
    lse = amax + np.log(np.exp(a - amax[:, None]).sum(axis=1))
    prob = np.exp(a - lse[:, None])
    return prob @ Vg[T], lse, prob.sum(axis=1)


# ---------------------------------------------------------------------------
# drivers: decode (one row per sequence) and prefill (rows of one sequence)
# ---------------------------------------------------------------------------
def decode(q: np.ndarray, Ks: Sequence[np.ndarray], Vs: Sequence[np.ndarray], prm: Params,
           cks: Optional[Sequence[np.ndarray]] = None, with_rows: bool = False):
    """Decode step: sequence b's query q[b] sits at position n_b - 1.

    q: [B][Hq][d]; Ks/Vs: per sequence [Hkv][n_b][d].  Returns block_idx
    [B][Hkv][k] and out [B][Hq][d] (and the RowSelection objects if asked).
    """
    B = q.shape[0]
    G, hkv = prm.group, prm.num_kv_heads
    idx = np.full((B, hkv, prm.topk), -1, dtype=np.int64)
    out = np.zeros((B, prm.num_q_heads, prm.head_dim))
    rows = []
    for b in range(B):
        K, V = Ks[b], Vs[b]
        n = K.shape[1]
        ck = compress_keys(K, prm.kernel_size, prm.kernel_stride, prm.ck_dtype) \
            if cks is None else cks[b]
        rb = []
        for g in range(hkv):
            qg = q[b, g * G:(g + 1) * G]
            rs = select_row(qg, ck[g], n - 1, prm)
            idx[b, g] = rs.sel
            out[b, g * G:(g + 1) * G] = attend_row(qg, K[g], V[g], n - 1, rs.sel, prm)[0]
            rb.append(rs)
        rows.append(rb)
    return (idx, out, rows) if with_rows else (idx, out)


def prefill(q: np.ndarray, K: np.ndarray, V: np.ndarray, prm: Params,
            positions: Optional[Iterable[int]] = None, ck: Optional[np.ndarray] = None,
            with_rows: bool = False):
    """Prefill of one sequence: query row r sits at position r.

    q: [L][Hq][d] (all rows of the sequence); K, V: [Hkv][n][d] with n >= L.
    ``positions`` picks the rows to evaluate (default: all).  Returns
    block_idx [R][Hkv][k] and out [R][Hq][d] for the chosen rows.
    """
    G, hkv = prm.group, prm.num_kv_heads
    pos = list(range(q.shape[0])) if positions is None else [int(x) for x in positions]
    if ck is None:
        ck = compress_keys(K, prm.kernel_size, prm.kernel_stride, prm.ck_dtype)
    idx = np.full((len(pos), hkv, prm.topk), -1, dtype=np.int64)
    out = np.zeros((len(pos), prm.num_q_heads, prm.head_dim))
    rows = []
    for r, i in enumerate(pos):
        rr = []
        for g in range(hkv):
            qg = q[i, g * G:(g + 1) * G]
            rs = select_row(qg, ck[g], i, prm)
            idx[r, g] = rs.sel
            out[r, g * G:(g + 1) * G] = attend_row(qg, K[g], V[g], i, rs.sel, prm)[0]
            rr.append(rs)
        rows.append(rr)
    return (idx, out, rows) if with_rows else (idx, out)


def attend_with_selection(q_rows: np.ndarray, K: np.ndarray, V: np.ndarray,
                          positions: Sequence[int], sel: np.ndarray, prm: Params) -> np.ndarray:
    """Attention only (step 7) for given rows and a given selection [R][Hkv][k]."""
    G, hkv = prm.group, prm.num_kv_heads
    out = np.zeros((len(positions), prm.num_q_heads, prm.head_dim))
    for r, i in enumerate(positions):
        for g in range(hkv):
            qg = q_rows[r, g * G:(g + 1) * G]
            out[r, g * G:(g + 1) * G] = attend_row(qg, K[g], V[g], int(i), np.asarray(sel[r, g]), prm)[0]
    return out


# ---------------------------------------------------------------------------
# backward of step 7: training through the sparse attention
# ---------------------------------------------------------------------------
def attend_row_grad(qg: np.ndarray, Kg: np.ndarray, Vg: np.ndarray, i: int, sel: np.ndarray,
                    prm: Params, dog: np.ndarray):
    """Gradients of one row's attention (the group's heads) for an upstream gradient dog [G][d].

    [IV2 Training-time considerations] and [IV2 Why mean pooling]: top-k is not
    differentiable and no gradient passes through the selection, so the selected
    set is a constant here and the compressed keys, which only feed the
    selection, receive none; K and V receive gradient only through the
    attention of stage 2.  With a = scale * q K_T^T, P = softmax(a) per head and
    o = P V_T, the chain rule gives
        dV_T = P^T dO,   dP = dO V_T^T,   dA = P * (dP - rowsum(P * dP)),
        dq = scale * dA K_T,   dK_T = scale * dA^T q.
    Returns (dq [G][d], T, dK_T [|T|][d], dV_T [|T|][d], lse [G]); a row with no
    visible selected token has output 0 and every gradient 0.
    """
    n = Kg.shape[0]
    T = selected_tokens(sel, i, n, prm.block_size)
    G, d = qg.shape
    if T.size == 0:
        return (np.zeros((G, d)), T, np.zeros((0, d)), np.zeros((0, d)),
                np.full(G, NEG_INF))
    kt, vt = Kg[T], Vg[T]
    a = prm.scale * (qg @ kt.T)                  # [G][|T|]
    amax = a.max(axis=1)
    lse = amax + np.log(np.exp(a - amax[:, None]).sum(axis=1))
    prob = np.exp(a - lse[:, None])
    dv_t = prob.T @ dog                          # [|T|][d]
    dprob = dog @ vt.T                           # [G][|T|]
    da = prob * (dprob - (prob * dprob).sum(axis=1, keepdims=True))
    dq = prm.scale * (da @ kt)
    dk_t = prm.scale * (da.T @ qg)
    return dq, T, dk_t, dv_t, lse


def attention_backward(q_rows: np.ndarray, K: np.ndarray, V: np.ndarray, positions: Sequence[int],
                       sel: np.ndarray, prm: Params, dout: np.ndarray):
    """Gradients of sum(dout * attend_with_selection(q_rows, K, V, positions, sel)).

    q_rows, dout [R][Hq][d]; K, V [Hkv][n][d]; sel [R][Hkv][k].  Contributions
    of every row to a token's dK / dV are summed.  Returns (dQ [R][Hq][d],
    dK [Hkv][n][d], dV [Hkv][n][d], lse [R][Hq]).
    """
    G, hkv = prm.group, prm.num_kv_heads
    dQ = np.zeros(q_rows.shape)
    dK = np.zeros(K.shape)
    dV = np.zeros(V.shape)
    lse = np.zeros(q_rows.shape[:2])
    for r, i in enumerate(positions):
        for g in range(hkv):
            hs = slice(g * G, (g + 1) * G)
            dq, T, dk_t, dv_t, l = attend_row_grad(q_rows[r, hs], K[g], V[g], int(i),
                                                   np.asarray(sel[r, g]), prm, dout[r, hs])
            dQ[r, hs] = dq
            dK[g, T] += dk_t
            dV[g, T] += dv_t
            lse[r, hs] = l
    return dQ, dK, dV, lse


def block_grad(q_rows: np.ndarray, K: np.ndarray, V: np.ndarray, positions: Sequence[int],
               sel: np.ndarray, prm: Params, dout: np.ndarray, g: int, j: int):
    """dK and dV of the tokens of block j of KV head g only, summed over the rows
    that selected it (the same chain rule as attend_row_grad).  Cheaper than
    attention_backward when a few blocks of a long sequence are checked.
    Returns (dK [m'][d], dV [m'][d]) for tokens j*m .. min((j+1)*m, n) - 1."""
    G, m = prm.group, prm.block_size
    n = K.shape[1]
    t0, t1 = j * m, min((j + 1) * m, n)
    dk = np.zeros((t1 - t0, K.shape[2]))
    dv = np.zeros((t1 - t0, V.shape[2]))
    hs = slice(g * G, (g + 1) * G)
    for r, i in enumerate(positions):
        if j not in set(np.asarray(sel[r, g]).tolist()) or t0 > i:
            continue
        dq, T, dk_t, dv_t, _ = attend_row_grad(q_rows[r, hs], K[g], V[g], int(i),
                                               np.asarray(sel[r, g]), prm, dout[r, hs])
        mask = (T >= t0) & (T < t1)
        dk[T[mask] - t0] += dk_t[mask]
        dv[T[mask] - t0] += dv_t[mask]
    return dk, dv
