"""Pins of the float64 oracle against things other than itself.

Each test names the property of the pages (MiniCPM4 summary page, section
"InfLLM v2") or of mathematics that it checks: closed forms, a hand-worked
example (tests/golden/hand_example.json), brute-force loops with exhaustive
top-k search (oracle/brute.py), an independent dense / sink+window attention
(oracle/dense_ref.py), invariances and structural counts.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

from oracle import brute, dense_ref
from oracle import infv2_ref as ref
from synth import bf16_bits_to_f32, f32_to_bf16_bits, make_workload

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _params(**kw):
    base = dict(head_dim=16, num_q_heads=4, num_kv_heads=2, block_size=16, kernel_size=8,
                kernel_stride=4, topk=5, init_blocks=1, local_blocks=2, ck_dtype="fp64")
    base.update(kw)
    return ref.Params(**base)


def _bf16_values(rng, shape, scale=1.0):
    """Random values exactly representable in bf16 (so every sum of a few is exact in fp64)."""
    x = (rng.standard_normal(shape) * scale).astype(np.float32)
    return bf16_bits_to_f32(f32_to_bf16_bits(x)).astype(np.float64)


# ---------------------------------------------------------------------------
# storage rounding
# ---------------------------------------------------------------------------
def test_round_fp32_matches_ieee_cast():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-40, 38, 20000),
                        [0.0, -0.0, 1.0, 2.0 ** -149, 2.0 ** -126 * 1.5, 3.4e38]])
    # exact ties: midpoints between adjacent float32 values
    f = rng.standard_normal(2000).astype(np.float32)
    nxt = np.nextafter(f, np.float32(np.inf))
    mids = (f.astype(np.float64) + nxt.astype(np.float64)) / 2
    x = np.concatenate([x, mids])
    got = ref.round_to_storage(x, "fp32")
    want = x.astype(np.float32).astype(np.float64)
    assert np.array_equal(got, want)


def test_round_bf16_matches_exhaustive_nearest_even():
    allbits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    with np.errstate(invalid="ignore"):
        vals = bf16_bits_to_f32(allbits).astype(np.float64)
    ok = np.isfinite(vals)
    vals, bits = vals[ok], allbits[ok]
    order = np.argsort(vals, kind="stable")
    vals, bits = vals[order], bits[order]
    keep = np.concatenate([[True], np.diff(vals) > 0])     # drop -0 duplicate
    vals, bits = vals[keep], bits[keep]
    rng = np.random.default_rng(2)
    x = rng.standard_normal(5000) * 10.0 ** rng.integers(-30, 30, 5000)
    mids = (vals[:-1] + vals[1:]) / 2
    x = np.concatenate([x, mids[rng.integers(0, mids.shape[0], 3000)]])
    x = x[np.abs(x) < vals[-1]]
    pos = np.searchsorted(vals, x)
    lo, hi = vals[np.maximum(pos - 1, 0)], vals[np.minimum(pos, vals.shape[0] - 1)]
    lob, hib = bits[np.maximum(pos - 1, 0)], bits[np.minimum(pos, vals.shape[0] - 1)]
    dlo, dhi = x - lo, hi - x
    even_lo = (lob & 1) == 0
    want = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, np.where(even_lo, lo, hi)))
    want = np.where(x == hi, hi, want)
    got = ref.round_to_storage(x, "bf16")
    assert np.array_equal(got, want)
    # the input encoder rounds float32 the same way
    f = rng.standard_normal(5000).astype(np.float32)
    assert np.array_equal(bf16_bits_to_f32(f32_to_bf16_bits(f)).astype(np.float64),
                          ref.round_to_storage(f.astype(np.float64), "bf16"))


# ---------------------------------------------------------------------------
# step 1: kernels and mean pooling  [IV2 Semantic kernels]
# ---------------------------------------------------------------------------
def test_num_kernels_counts_complete_spans():
    for p, s in [(32, 16), (8, 4), (5, 3), (4, 4), (7, 1)]:
        for n in range(0, 200):
            want = sum(1 for j in range(n + 1) if j * s + p <= n)
            assert ref.num_kernels(n, p, s) == want


def test_kernel_count_ratio_and_token_multiplicity():
    # [IV2 Complexity analysis]: kernels ~ l/s; [IV2 Hyperparameter configuration]:
    # with p=32, s=16 each token lies in two kernels.
    n, p, s = 131072, 32, 16
    nc = ref.num_kernels(n, p, s)
    assert nc == 8191 and abs(nc / n - 1 / s) < 1e-3
    cover = np.zeros(n, dtype=np.int64)
    for j in range(nc):
        cover[j * s:j * s + p] += 1
    assert np.all(cover[p - s:nc * s] == p // s)


def test_overlap_table_five_kernels_per_interior_block():
    tab = ref.block_overlaps(2048, 8191, 64, 32, 16)
    for j in [1, 2, 100, 2046]:
        assert tab[j][tab[j] >= 0].tolist() == list(range(4 * j - 1, 4 * j + 4))
    assert tab[0][tab[0] >= 0].tolist() == [0, 1, 2, 3]
    assert tab[2047][tab[2047] >= 0].tolist() == [8187, 8188, 8189, 8190]


def test_compress_constant_linear_and_brute():
    rng = np.random.default_rng(3)
    p, s = 8, 4
    c = _bf16_values(rng, (1, 1, 16))
    K = np.repeat(c, 50, axis=1)
    ck = ref.compress_keys(K, p, s, "fp32")
    assert np.array_equal(ck, np.repeat(c, ref.num_kernels(50, p, s), axis=1))
    A, B = _bf16_values(rng, (2, 50, 16)), _bf16_values(rng, (2, 50, 16))
    lin = ref.compress_keys(2.0 * A - B, p, s, "fp64")
    assert np.allclose(lin, 2.0 * ref.compress_keys(A, p, s, "fp64")
                       - ref.compress_keys(B, p, s, "fp64"), atol=1e-13)
    # literal loops with exact summation, then the same single rounding
    want = brute.brute_compress(A[0].tolist(), 50, p, s)
    got = ref.compress_keys(A, p, s, "fp32")[0]
    assert np.array_equal(got, np.array([[brute.to_fp32(v) for v in row] for row in want]))


# ---------------------------------------------------------------------------
# hand-worked example
# ---------------------------------------------------------------------------
def _eval_expr(e):
    return float(eval(e, {"__builtins__": {}}, {"exp": math.exp, "sqrt": math.sqrt}))


@pytest.mark.parametrize("case", ["plain", "straddle"])
def test_hand_worked_example(case):
    fx = json.load(open(os.path.join(GOLDEN, "hand_example.json")))
    pr = dict(fx["params"])
    scale = _eval_expr(pr.pop("attn_scale_expr"))
    prm = ref.Params(attn_scale=scale, ck_dtype="fp64", **pr)
    cs = fx["cases"][case]
    n, i = fx["n"], fx["position"]
    K = np.zeros((1, n, 2))
    K[0, cs["x_hot"], 0] = 8.0
    V = np.stack([np.arange(n, dtype=np.float64), np.ones(n)], axis=1)[None]
    q = np.array(fx["queries"])
    ck = ref.compress_keys(K, prm.kernel_size, prm.kernel_stride, "fp64")
    assert ck[0, :, 0].tolist() == cs["ck_first_coord"] and np.all(ck[0, :, 1] == 0)
    rs = ref.select_row(q, ck[0], i, prm)
    # kernel scores ordered as derived
    groups = cs["score_order_desc_kernels"]
    for a, b in zip(groups, groups[1:]):
        assert min(rs.R[a]) > max(rs.R[b])
    for grp in groups:
        assert np.ptp(rs.R[grp]) < 1e-15
    for blk, kern in cs["block_scores_equal_kernel"].items():
        assert rs.S[int(blk)] == rs.R[kern]
    assert rs.sel[rs.sel >= 0].tolist() == cs["selection"]
    o, _, _ = ref.attend_row(q, K[0], V[0], i, rs.sel, prm)
    want = np.array([[_eval_expr(e) for e in cs["out_head0_expr"]],
                     [_eval_expr(e) for e in cs["out_head1_expr"]]])
    assert np.allclose(o, want, rtol=1e-13, atol=1e-13)


# ---------------------------------------------------------------------------
# closed form: a ramp of keys gives geometric logits
# ---------------------------------------------------------------------------
def test_ramp_closed_form_lse_scores_and_selection():
    # K_t = (t / n) e0 so kbar_j^ = ((j^ s + (p-1)/2) / n) e0 and the logits of a
    # head with q = a e0 are an arithmetic sequence; LSE is a geometric sum.
    m, p, s, d, n = 16, 8, 4, 8, 400
    prm = _params(head_dim=d, num_q_heads=2, num_kv_heads=1, block_size=m, kernel_size=p,
                  kernel_stride=s, topk=6, init_blocks=1, local_blocks=2, ck_dtype="fp64")
    K = np.zeros((1, n, d))
    K[0, :, 0] = np.arange(n) / n
    q = np.zeros((2, d))
    q[0, 0], q[1, 0] = 30.0, 10.0
    ck = ref.compress_keys(K, p, s, "fp64")
    for i in [130, 211, 399]:
        rs = ref.select_row(q, ck[0], i, prm)
        vis = ref.num_kernels(i + 1, p, s)
        for h, a in enumerate([30.0, 10.0]):
            slope, icpt = a * s / n, a * (p - 1) / 2 / n
            assert abs(rs.lse[h] - dense_ref.logsumexp_closed_form_geometric(slope, icpt, vis)) < 1e-12
        # increasing logits: each block's score is its last visible kernel's; the
        # selection is F plus the k' blocks just below the local window
        c = i // m
        kp = prm.topk - 3
        want = sorted({0, c - 1, c} | set(range(c - 1 - kp, c - 1)))
        assert rs.sel.tolist() == want
        assert np.all(np.diff(rs.S[1:c]) > 0)


# ---------------------------------------------------------------------------
# brute force on tiny inputs  [all definitions + exhaustive top-k]
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("G,seed", [(1, 10), (2, 11), (16, 12), (2, 13)])
def test_selection_matches_brute_force(G, seed):
    rng = np.random.default_rng(seed)
    m, p, s, d, n = 16, 8, 4, 8, 200
    prm = _params(head_dim=d, num_q_heads=G, num_kv_heads=1, block_size=m, kernel_size=p,
                  kernel_stride=s, topk=7, init_blocks=1, local_blocks=2, ck_dtype="fp64",
                  score_scale=0.7)
    K = _bf16_values(rng, (1, n, d))
    K[0, 48:64] += 2.0            # a planted block
    q = _bf16_values(rng, (G, d))
    ck = ref.compress_keys(K, p, s, "fp64")
    checked = 0
    for i in range(0, n, 7):
        rs = ref.select_row(q, ck[0], i, prm)
        S, R, lse = brute.brute_block_scores(q.tolist(), K[0].tolist(), i, m, p, s, 0.7)
        assert np.allclose(rs.S, S, rtol=1e-12, atol=0)
        assert np.allclose(rs.R, R, rtol=1e-12, atol=1e-300)
        c = i // m
        want = brute.brute_select(S, c, prm.topk, 1, 2)
        assert rs.sel[rs.sel >= 0].tolist() == want
        checked += 1
    assert checked > 20


def test_brute_force_on_exact_structural_ties():
    # duplicated key windows give equal block scores; exhaustive search and the
    # oracle must both keep the lower block  [tie rule reading]
    rng = np.random.default_rng(5)
    m, p, s, d, n = 16, 8, 4, 8, 256
    prm = _params(head_dim=d, num_q_heads=2, num_kv_heads=1, block_size=m, kernel_size=p,
                  kernel_stride=s, topk=4, init_blocks=1, local_blocks=2, ck_dtype="fp64")
    K = _bf16_values(rng, (1, n, d), 0.2)
    hot = np.zeros(d)
    hot[0] = 4.0
    # block 5 (tokens 80-95) is hot; the kernels meeting it span tokens 76-99, and
    # block 10 (tokens 160-175) gets an identical copy of that whole neighbourhood
    K[0, 80:96] += hot
    K[0, 156:180] = K[0, 76:100]
    q = np.zeros((2, d))
    q[:, 0] = 3.0
    ck = ref.compress_keys(K, p, s, "fp64")
    i = 250
    rs = ref.select_row(q, ck[0], i, prm)
    assert rs.S[5] == rs.S[10]
    S, _, _ = brute.brute_block_scores(q.tolist(), K[0].tolist(), i, m, p, s)
    assert brute.brute_select(S, i // m, 4, 1, 2) == rs.sel.tolist()
    assert 5 in rs.sel and 10 not in rs.sel


# ---------------------------------------------------------------------------
# attention: dense reduction, sink+window, row sums, brute attention
# ---------------------------------------------------------------------------
def test_dense_reduction_when_topk_covers_everything():
    rng = np.random.default_rng(6)
    n, d = 130, 16
    prm = _params(head_dim=d, num_q_heads=4, num_kv_heads=2, topk=9, ck_dtype="fp64")
    q, K, V = rng.standard_normal((n, 4, d)), rng.standard_normal((2, n, d)), rng.standard_normal((2, n, d))
    pos = list(range(0, n, 3))
    _, out = ref.prefill(q, K, V, prm, positions=pos)
    want = dense_ref.causal_attention(q[pos], K, V, pos, prm.scale)
    assert np.max(np.abs(out - want)) < 1e-12


def test_dense_below_k_times_m_and_sparse_above():
    rng = np.random.default_rng(7)
    m, k = 16, 4
    n, d = 200, 8
    prm = _params(head_dim=d, num_q_heads=2, num_kv_heads=1, topk=k, local_blocks=1)
    q, K, V = rng.standard_normal((n, 2, d)), rng.standard_normal((1, n, d)), rng.standard_normal((1, n, d))
    pos = [0, 17, k * m - 1, k * m, 150]
    idx, out = ref.prefill(q, K, V, prm, positions=pos)
    want = dense_ref.causal_attention(q[pos], K, V, pos, prm.scale)
    for r, i in enumerate(pos):
        if i < k * m:
            assert np.max(np.abs(out[r] - want[r])) < 1e-12
            assert idx[r, 0].tolist()[: i // m + 1] == list(range(i // m + 1))
        else:
            assert (idx[r, 0] >= 0).sum() == k and np.max(np.abs(out[r] - want[r])) > 1e-6


def test_forced_only_equals_sink_window_attention():
    rng = np.random.default_rng(8)
    n, d = 300, 8
    prm = _params(head_dim=d, num_q_heads=4, num_kv_heads=1, topk=3, init_blocks=1, local_blocks=2)
    q, K, V = rng.standard_normal((n, 4, d)), rng.standard_normal((1, n, d)), rng.standard_normal((1, n, d))
    pos = [64, 99, 180, 299]
    idx, out = ref.prefill(q, K, V, prm, positions=pos)
    for r, i in enumerate(pos):
        c = i // 16
        assert idx[r, 0].tolist() == sorted({0, c - 1, c})
    want = dense_ref.sink_window_attention(q[pos], K, V, pos, prm.scale, 16, 1, 2)
    assert np.max(np.abs(out - want)) < 1e-12


def test_attention_matches_brute_loops_and_sums_to_one():
    rng = np.random.default_rng(9)
    n, d = 120, 8
    prm = _params(head_dim=d, num_q_heads=2, num_kv_heads=1, topk=4)
    q, K, V = rng.standard_normal((n, 2, d)), rng.standard_normal((1, n, d)), rng.standard_normal((1, n, d))
    for i in [70, 100, 119]:
        ck = ref.compress_keys(K, 8, 4, "fp64")
        rs = ref.select_row(q[i], ck[0], i, prm)
        o, lse, psum = ref.attend_row(q[i], K[0], V[0], i, rs.sel, prm)
        assert np.allclose(psum, 1.0, atol=1e-14)
        for h in range(2):
            want = brute.brute_attend(q[i, h].tolist(), K[0].tolist(), V[0].tolist(), i,
                                      rs.sel.tolist(), 16, prm.scale)
            assert np.allclose(o[h], want, atol=1e-13)


def test_kernel_softmax_and_group_scores_sum_to_one():
    rng = np.random.default_rng(10)
    n, d = 500, 16
    prm = _params(head_dim=d, num_q_heads=16, num_kv_heads=1)
    q, K = rng.standard_normal((16, d)) * 2, rng.standard_normal((1, n, d))
    ck = ref.compress_keys(K, 8, 4, "fp64")
    rs = ref.select_row(q, ck[0], 480, prm)
    assert np.allclose(np.exp(rs.z - rs.lse[:, None]).sum(axis=1), 1.0, atol=1e-13)
    assert abs(rs.R.sum() - 1.0) < 1e-13


# ---------------------------------------------------------------------------
# causality, invariances, consistency, needle, varlen
# ---------------------------------------------------------------------------
def test_future_keys_do_not_change_a_row():
    rng = np.random.default_rng(11)
    n, d = 260, 8
    prm = _params(head_dim=d, num_q_heads=4, num_kv_heads=2, topk=4)
    q, K, V = rng.standard_normal((n, 4, d)), rng.standard_normal((2, n, d)), rng.standard_normal((2, n, d))
    i = 170
    idx1, out1 = ref.prefill(q, K, V, prm, positions=[i])
    K2, V2 = K.copy(), V.copy()
    K2[:, i + 1:] = rng.standard_normal(K2[:, i + 1:].shape) * 5
    V2[:, i + 1:] = rng.standard_normal(V2[:, i + 1:].shape) * 5
    idx2, out2 = ref.prefill(q, K2, V2, prm, positions=[i])
    assert np.array_equal(idx1, idx2) and np.array_equal(out1, out2)
    assert idx1.max() <= i // 16


def test_invariances_key_shift_head_permutation_value_scale():
    rng = np.random.default_rng(12)
    n, d = 400, 16
    prm = _params(head_dim=d, num_q_heads=8, num_kv_heads=2, topk=6)
    q, K, V = rng.standard_normal((n, 8, d)), rng.standard_normal((2, n, d)), rng.standard_normal((2, n, d))
    pos = [200, 333, 399]
    idx, out = ref.prefill(q, K, V, prm, positions=pos)
    # a common offset on every key shifts each head's logits by a constant:
    # the kernel softmax, the selection and the attention are unchanged
    shift = rng.standard_normal(d)
    idx2, out2 = ref.prefill(q, K + shift, V, prm, positions=pos)
    assert np.array_equal(idx, idx2) and np.allclose(out, out2, atol=1e-10)
    # permuting heads inside a group permutes outputs, selection unchanged
    perm = np.array([2, 0, 3, 1, 5, 7, 4, 6])
    idx3, out3 = ref.prefill(q[:, perm], K, V, prm, positions=pos)
    assert np.array_equal(idx, idx3) and np.allclose(out3, out[:, perm], atol=1e-13)
    # scaling values scales outputs
    _, out4 = ref.prefill(q, K, 3.0 * V, prm, positions=pos)
    assert np.allclose(out4, 3.0 * out, atol=1e-12)


def test_decode_equals_last_prefill_row_and_row_subsets():
    # [IV2 Design principles summary]: token-level queries, so decoding at
    # length n is the prefill row n-1
    rng = np.random.default_rng(13)
    n, d = 333, 16
    prm = _params(head_dim=d, num_q_heads=4, num_kv_heads=2, topk=5)
    q, K, V = rng.standard_normal((n, 4, d)), rng.standard_normal((2, n, d)), rng.standard_normal((2, n, d))
    idx_p, out_p = ref.prefill(q, K, V, prm)
    idx_d, out_d = ref.decode(q[n - 1:n], [K], [V], prm)
    assert np.array_equal(idx_d[0], idx_p[n - 1]) and np.max(np.abs(out_d[0] - out_p[n - 1])) < 1e-12
    # evaluating a subset of rows gives the same rows (chunking does not matter)
    sub = list(range(100, 180))
    idx_s, out_s = ref.prefill(q, K, V, prm, positions=sub)
    assert np.array_equal(idx_s, idx_p[sub]) and np.array_equal(out_s, out_p[sub])


def test_planted_needle_blocks_are_selected():
    rng = np.random.default_rng(14)
    n, d, m = 2048, 32, 64
    prm = ref.Params(head_dim=d, num_q_heads=4, num_kv_heads=1, block_size=m, kernel_size=32,
                     kernel_stride=16, topk=12, init_blocks=1, local_blocks=2, ck_dtype="fp32")
    K = rng.standard_normal((1, n, d))
    u = rng.standard_normal(d)
    u /= np.linalg.norm(u)
    planted = [3, 9, 17, 22, 28]
    for j in planted:
        K[0, j * m:(j + 1) * m] += 3 * u
    q = rng.standard_normal((4, d)) + 8.0 * u
    ck = ref.compress_keys(K, 32, 16, "fp32")
    rs = ref.select_row(q, ck[0], n - 1, prm)
    assert set(planted) <= set(rs.sel.tolist())


def test_varlen_batch_equals_separate_sequences():
    wl = make_workload(mode="decode", io_dtype="bf16", lens=[300, 517, 129], num_q_heads=4,
                       num_kv_heads=2, head_dim=16, block_size=16, kernel_size=8, kernel_stride=4,
                       topk=5, init_blocks=1, local_blocks=2, n_planted=2, seed=15)
    prm = ref.Params(head_dim=16, num_q_heads=4, num_kv_heads=2, block_size=16, kernel_size=8,
                     kernel_stride=4, topk=5, init_blocks=1, local_blocks=2)
    q = wl.q_f64()
    Ks = [wl.k_f64(b) for b in range(3)]
    Vs = [wl.v_f64(b) for b in range(3)]
    idx, out = ref.decode(q, Ks, Vs, prm)
    for b in range(3):
        i1, o1 = ref.decode(q[b:b + 1], [Ks[b]], [Vs[b]], prm)
        assert np.array_equal(i1[0], idx[b]) and np.array_equal(o1[0], out[b])


def test_bf16_compressed_keys_round_the_exact_mean_once():
    rng = np.random.default_rng(16)
    K = _bf16_values(rng, (2, 100, 16))
    exact = ref.compress_keys(K, 8, 4, "fp64")
    ck = ref.compress_keys(K, 8, 4, "bf16")
    assert np.array_equal(ck, ref.round_to_storage(exact, "bf16"))
    assert np.max(np.abs(ck - exact) / np.maximum(np.abs(exact), 1e-30)) <= 2.0 ** -8


def test_append_token_by_token_equals_compressing_the_whole_cache():
    # the cache after n appends equals the cache holding the n tokens, and its
    # compressed keys equal a fresh compression of those tokens (bit for bit)
    rng = np.random.default_rng(17)
    hkv, n, d, p, s = 2, 150, 8, 8, 4
    Kfull = rng.standard_normal((hkv, n, d))
    Vfull = rng.standard_normal((hkv, n, d))
    for ck_dtype in ["fp32", "bf16"]:
        K = np.zeros((hkv, n + 5, d))
        V = np.zeros_like(K)
        ck = np.full((hkv, ref.num_kernels(n, p, s) + 3, d), np.nan)
        ln = 0
        completed = []
        for t in range(n):
            before = np.isnan(ck[:, :, 0]).sum()
            ln = ref.append_token(K, V, ln, Kfull[:, t], Vfull[:, t], ck, p, s, ck_dtype)
            if np.isnan(ck[:, :, 0]).sum() < before:
                completed.append(t)
        assert ln == n
        assert np.array_equal(K[:, :n], Kfull) and np.array_equal(V[:, :n], Vfull)
        nc = ref.num_kernels(n, p, s)
        assert np.array_equal(ck[:, :nc], ref.compress_keys(Kfull, p, s, ck_dtype))
        assert np.isnan(ck[:, nc:]).all()
        # kernel j completes at token j s + p - 1
        assert completed == [j * s + p - 1 for j in range(nc)]


# ---------------------------------------------------------------------------
# backward of the sparse attention (training through stage 2)
# ---------------------------------------------------------------------------
def _bwd_case(seed, n=14, positions=(3, 7, 9, 13), sel_rows=None):
    """Tiny case: d=4, Hq=4, Hkv=2, m=4; random valid selections (ascending, -1 padded)."""
    prm = _params(head_dim=4, num_q_heads=4, num_kv_heads=2, block_size=4, kernel_size=2,
                  kernel_stride=2, topk=3, local_blocks=1)
    rng = np.random.default_rng(seed)
    R = len(positions)
    q = rng.standard_normal((R, 4, 4))
    K = rng.standard_normal((2, n, 4))
    V = rng.standard_normal((2, n, 4))
    dout = rng.standard_normal((R, 4, 4))
    sel = np.full((R, 2, prm.topk), -1, dtype=np.int64)
    for r, i in enumerate(positions):
        c = i // prm.block_size
        for g in range(2):
            # own block always, plus a random subset of the earlier ones
            others = rng.permutation(c)[:rng.integers(0, prm.topk)].tolist()
            blocks = sorted(set(others[:prm.topk - 1] + [c]))
            sel[r, g, :len(blocks)] = blocks
    if sel_rows is not None:
        sel = sel_rows(sel)
    return prm, q, K, V, dout, sel, list(positions)


def test_backward_matches_central_differences_of_the_forward():
    """[IV2 Training-time considerations]: gradients flow to q, K, V through the
    attention over a fixed selection.  The analytic oracle gradient must equal
    the numerical derivative of the (separately pinned) forward oracle."""
    prm, q, K, V, dout, sel, pos = _bwd_case(5)

    def loss(q_, K_, V_):
        return float((dout * ref.attend_with_selection(q_, K_, V_, pos, sel, prm)).sum())

    dQ, dK, dV, _ = ref.attention_backward(q, K, V, pos, sel, prm, dout)
    h = 1e-5
    for arr, grad, which in ((q, dQ, 0), (K, dK, 1), (V, dV, 2)):
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            args = [q.copy(), K.copy(), V.copy()]
            args[which][idx] += h
            fp = loss(*args)
            args[which][idx] -= 2 * h
            fm = loss(*args)
            num[idx] = (fp - fm) / (2 * h)
        assert np.max(np.abs(num - grad)) < 1e-8 * max(1.0, np.max(np.abs(grad))), which
    # at least some tokens get no gradient (not attended by any row) and some do
    assert np.any(np.all(dK == 0, axis=-1)) and np.any(np.any(dK != 0, axis=-1))


def test_backward_dense_case_equals_autograd_of_causal_attention():
    """[IV2 Initial and local tokens always selected]: with every block selected the
    method is dense causal attention, whose gradient torch's autograd gives."""
    import torch
    n = 14
    pos = list(range(n))
    prm, q, K, V, dout, sel, _ = _bwd_case(6, n=n, positions=pos)
    nb = -(-n // prm.block_size)
    sel = np.full((n, 2, nb), -1, dtype=np.int64)
    for r, i in enumerate(pos):
        sel[r, :, :i // prm.block_size + 1] = np.arange(i // prm.block_size + 1)
    prm = ref.Params(**{**prm.__dict__, "topk": nb})
    dQ, dK, dV, _ = ref.attention_backward(q, K, V, pos, sel, prm, dout)

    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, K, V))
    kx = tk.repeat_interleave(2, dim=0)          # head h uses KV head h // G
    vx = tv.repeat_interleave(2, dim=0)
    logits = torch.einsum("rhd,htd->hrt", tq, kx) * prm.scale
    mask = torch.tensor(np.arange(n)[None, :] <= np.array(pos)[:, None])
    logits = logits.masked_fill(~mask[None], float("-inf"))
    out = torch.einsum("hrt,htd->rhd", torch.softmax(logits, dim=-1), vx)
    (out * torch.tensor(dout)).sum().backward()
    assert np.allclose(dQ, tq.grad.numpy(), rtol=0, atol=1e-12)
    assert np.allclose(dK, tk.grad.numpy(), rtol=0, atol=1e-12)
    assert np.allclose(dV, tv.grad.numpy(), rtol=0, atol=1e-12)


def test_backward_invariants_and_block_slices():
    """Softmax structure: each row's probabilities sum to one, so per row and head
    sum_t dA_t = 0 (the keys' gradients sum to zero over the sequence) and
    sum_t dV_t = dO; tokens no row attends get no gradient; block_grad is the
    per-block slice of the full backward."""
    prm, q, K, V, dout, sel, pos = _bwd_case(7, n=22, positions=(0, 5, 8, 12, 17, 21))
    dQ, dK, dV, lse = ref.attention_backward(q, K, V, pos, sel, prm, dout)
    G = prm.group
    for g in range(2):
        assert np.allclose(dK[g].sum(axis=0), 0.0, atol=1e-12)
        assert np.allclose(dV[g].sum(axis=0), dout[:, g * G:(g + 1) * G].sum(axis=(0, 1)), atol=1e-12)
        seen = np.zeros(K.shape[1], dtype=bool)
        for r, i in enumerate(pos):
            seen[ref.selected_tokens(sel[r, g], i, K.shape[1], prm.block_size)] = True
        assert np.all(dK[g][~seen] == 0) and np.all(dV[g][~seen] == 0)
        for j in range(-(-K.shape[1] // prm.block_size)):
            bk, bv = ref.block_grad(q, K, V, pos, sel, prm, dout, g, j)
            t0 = j * prm.block_size
            assert np.allclose(bk, dK[g, t0:t0 + len(bk)], atol=1e-13)
            assert np.allclose(bv, dV[g, t0:t0 + len(bv)], atol=1e-13)
    # lse is the forward's LogSumExp
    for r, i in enumerate(pos):
        for g in range(2):
            _, l, _ = ref.attend_row(q[r, g * G:(g + 1) * G], K[g], V[g], i, sel[r, g], prm)
            assert np.allclose(lse[r, g * G:(g + 1) * G], l, atol=1e-13)


def test_backward_row_without_visible_tokens_is_zero():
    """A row whose selection holds no token at or before it (all -1 padding) has
    output 0 (the kernels' convention) and contributes no gradient."""
    prm, q, K, V, dout, sel, pos = _bwd_case(8, sel_rows=lambda s: np.where(
        np.arange(s.shape[0])[:, None, None] == 1, -1, s))
    dQ, dK, dV, _ = ref.attention_backward(q, K, V, pos, sel, prm, dout)
    assert np.all(dQ[1] == 0)
    dQ2, dK2, dV2, _ = ref.attention_backward(np.delete(q, 1, 0), K, V, [p for r, p in enumerate(pos) if r != 1],
                                              np.delete(sel, 1, 0), prm, np.delete(dout, 1, 0))
    assert np.allclose(dK, dK2, atol=1e-14) and np.allclose(dV, dV2, atol=1e-14)


# ---------------------------------------------------------------------------
# coarse-kernel LogSumExp (the pages' approximate pass 1)
# ---------------------------------------------------------------------------
def test_coarse_lse_equals_exact_when_coarse_kernels_are_the_fine_ones():
    """[IV2 Efficient LSE approximation]: with non-overlapping fine kernels
    (p = s) and coarse size s, the coarse kernels are the fine kernels, so the
    approximation is exact: same normaliser, scores and selection."""
    prm = _params(kernel_size=4, kernel_stride=4, topk=4, local_blocks=1)
    rng = np.random.default_rng(60)
    n = 140
    K = rng.standard_normal((2, n, 16))
    q = rng.standard_normal((n, 4, 16))
    ck = ref.compress_keys(K, 4, 4, "fp64")
    for i in (15, 64, 99, 139):
        for g in range(2):
            qg = q[i, 2 * g:2 * g + 2]
            a = ref.select_row(qg, ck[g], i, prm)
            b = ref.select_row_coarse(qg, ck[g], ck[g], i, prm, 4)
            assert np.array_equal(a.sel, b.sel)
            assert np.allclose(a.S, b.S, rtol=1e-14, atol=0) and np.allclose(a.lse, b.lse, rtol=1e-14)


def test_coarse_lse_closed_form_for_constant_keys():
    """Every key equal to u: every fine and coarse logit is z = q.u, so the exact
    normaliser is z + log(n_fine) and the coarse one z + log(n_coarse); each
    kernel's per-head score becomes 1 / n_coarse instead of 1 / n_fine."""
    prm = _params(kernel_size=8, kernel_stride=4, topk=5)
    rng = np.random.default_rng(61)
    n, d, coarse = 200, 16, 32
    u = rng.standard_normal(d)
    K = np.broadcast_to(u, (2, n, d)).copy()
    q = rng.standard_normal((4, d))
    ck = ref.compress_keys(K, 8, 4, "fp64")
    ckc = ref.compress_keys(K, coarse, coarse, "fp64")
    for i in (63, 150, 199):
        nf, nc = ref.num_kernels(i + 1, 8, 4), ref.num_kernels(i + 1, coarse, coarse)
        rs = ref.select_row_coarse(q[:2], ck[0], ckc[0], i, prm, coarse)
        z = q[:2] @ u
        assert np.allclose(rs.lse, z + np.log(nc), rtol=1e-13)
        assert np.allclose(rs.R, 1.0 / nc, rtol=1e-12)
        assert np.allclose(ref.select_row(q[:2], ck[0], i, prm).R, 1.0 / nf, rtol=1e-12)


@pytest.mark.parametrize("seed", [62, 63])
def test_coarse_lse_matches_brute_force(seed):
    """The coarse normaliser, scores and selection against the pure-Python loops
    (brute_coarse_lse, brute_block_scores with that normaliser, exhaustive top-k)."""
    prm = _params(block_size=8, kernel_size=4, kernel_stride=2, topk=4, local_blocks=1)
    rng = np.random.default_rng(seed)
    n, d, G, coarse = 72, 3, 2, 16
    K = _bf16_values(rng, (1, n, d))
    q = _bf16_values(rng, (G, d))
    ck = ref.compress_keys(K, 4, 2, "fp64")
    ckc = ref.compress_keys(K, coarse, coarse, "fp64")
    for i in (7, 15, 40, 71):
        rs = ref.select_row_coarse(q, ck[0], ckc[0], i, prm, coarse)
        lb = brute.brute_coarse_lse(q.tolist(), K[0].tolist(), i, coarse)
        if lb is None:
            assert i + 1 < coarse
            lb = brute.brute_block_scores(q.tolist(), K[0].tolist(), i, 8, 4, 2)[2]
        assert np.allclose(rs.lse, lb, rtol=1e-13)
        S, _, _ = brute.brute_block_scores(q.tolist(), K[0].tolist(), i, 8, 4, 2, lse_override=lb)
        assert np.allclose(rs.S, S, rtol=1e-12)
        want = brute.brute_select(S, i // 8, prm.topk, prm.init_blocks, prm.local_blocks)
        assert rs.sel[rs.sel >= 0].tolist() == want
