"""GPU parity: the HIP path (through the C ABI) against the float64 oracle.

Selections must match bit-exactly except across near-ties inside the relative
1e-4 band (tests/parity.py); outputs must be allclose with (2e-2, 1e-2) for
bf16 inputs and (1e-5, 1e-5) for fp32 inputs, the oracle evaluated on the
GPU's selection.  Compressed keys must match bit-exactly (both sides round the
exact mean once).  Every test prints what it runs before touching the GPU.
"""
import math

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import infv2_ref as ref  # noqa: E402
from synth import make_config, make_workload  # noqa: E402
from tests.parity import accept_selection, assert_close  # noqa: E402

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[gpu-test] {msg}", flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import trainable_block_sparse_amd as tbs
    tbs.load_library()
    yield


def _harness():
    from tests import gpu_harness
    return gpu_harness


def params_of(wl, ck_dtype="fp32", **over):
    kw = dict(head_dim=wl.head_dim, num_q_heads=wl.num_q_heads, num_kv_heads=wl.num_kv_heads,
              block_size=wl.block_size, kernel_size=wl.kernel_size, kernel_stride=wl.kernel_stride,
              topk=wl.topk, init_blocks=wl.init_blocks, local_blocks=wl.local_blocks,
              score_scale=wl.score_scale, attn_scale=wl.attn_scale, ck_dtype=ck_dtype)
    kw.update(over)
    return ref.Params(**kw)


def _check_rows(gpu_idx, gpu_score, rowsels, label):
    """Selection acceptance over rows; returns (#exact, #band)."""
    exact = band = 0
    worst_rel = 0.0
    for r, rs in enumerate(rowsels):
        verdict = accept_selection(gpu_idx[r], rs)
        assert not verdict.startswith("fail"), f"{label} row {r}: {verdict}"
        exact += verdict == "exact"
        band += verdict == "band"
        sel = gpu_idx[r][gpu_idx[r] >= 0]
        want = rs.S[sel]
        got = gpu_score[r][:sel.shape[0]]
        fin = np.isfinite(want)
        assert np.array_equal(np.isfinite(got), fin), f"{label} row {r}: -inf pattern"
        if fin.any():
            rel = np.max(np.abs(got[fin] - want[fin]) / np.maximum(np.abs(want[fin]), 1e-30))
            worst_rel = max(worst_rel, float(rel))
    assert worst_rel < 1e-4, f"{label}: block-score relative error {worst_rel:.2e}"
    _say(f"{label}: {exact} exact, {band} within the near-tie band, score rel err {worst_rel:.1e}")
    return exact, band


# ---------------------------------------------------------------------------- decode
def _run_decode(wl, ck_dtype="fp32", label="decode"):
    h = _harness()
    _say(f"{label}: lens={wl.lens.tolist()[:4]}{'...' if wl.batch > 4 else ''} B={wl.batch} "
         f"io={wl.io_dtype} ck={ck_dtype} k={wl.topk} local={wl.local_blocks}")
    dev = h.DeviceWorkload(wl, ck_dtype)
    dev.compress()
    idx_t, score_t = dev.select_decode()
    out_t = dev.attn_decode(idx_t)
    torch.cuda.synchronize()
    idx = idx_t.cpu().numpy().astype(np.int64)
    score = score_t.cpu().numpy().astype(np.float64)
    out = h.from_device(out_t, wl.io_dtype)
    prm = params_of(wl, ck_dtype)
    # compressed keys bit-exact
    cks = dev.ck_host()
    q = wl.q_f64()
    for b in range(wl.batch):
        K = wl.k_f64(b)
        want_ck = ref.compress_keys(K, wl.kernel_size, wl.kernel_stride, ck_dtype)
        assert np.array_equal(cks[b], want_ck), f"{label}: compressed keys differ (seq {b})"
    rows, idx_rows, score_rows = [], [], []
    for b in range(wl.batch):
        K = wl.k_f64(b)
        n = K.shape[1]
        G = prm.group
        for g in range(wl.num_kv_heads):
            rs = ref.select_row(q[b, g * G:(g + 1) * G], cks[b][g], n - 1, prm)
            rows.append(rs)
            idx_rows.append(idx[b, g])
            score_rows.append(score[b, g])
    _check_rows(np.array(idx_rows), np.array(score_rows), rows, label)
    want = np.zeros_like(out)
    for b in range(wl.batch):
        n = int(wl.lens[b])
        want[b] = ref.attend_with_selection(q[b:b + 1], wl.k_f64(b), wl.v_f64(b), [n - 1],
                                            idx[b:b + 1], prm)[0]
    err = assert_close(out, want, wl.io_dtype, label)
    _say(f"{label}: output max abs err {err:.2e}, {dev.check_canaries()} guarded buffers untouched")
    return dev, idx, out


def _small(mode="decode", lens=(300,), io="bf16", hkv=2, topk=8, local=2, init=1, seed=0, **kw):
    return make_workload(mode=mode, io_dtype=io, lens=list(lens), num_q_heads=16 * hkv,
                         num_kv_heads=hkv, topk=topk, init_blocks=init, local_blocks=local,
                         n_planted=kw.pop("n_planted", 3), seed=seed, **kw)


def test_decode_ragged_small_batch():
    wl = _small(lens=[1, 31, 32, 33, 63, 64, 65, 100, 513, 1000, 4097], topk=8, local=2, seed=21)
    _run_decode(wl, label="decode ragged bf16")


@pytest.mark.parametrize("io,nseq,lo,hi", [("bf16", 96, 1, 3000), ("fp32", 4, 10000, 30000)])
def test_decode_many_sequences_and_long_fp32(io, nseq, lo, hi):
    """A batch of 96 ragged bf16 sequences (grid depth in the batch, short caches
    next to empty-ish ones) and fp32 inputs at 10K-30K tokens (the vector-ALU
    scoring pass over thousands of kernels)."""
    lens = np.random.default_rng(151 + nseq).integers(lo, hi, size=nseq, endpoint=True).tolist()
    wl = _small(lens=lens, io=io, topk=16, local=2, seed=151 + nseq, n_planted=4)
    _run_decode(wl, label=f"decode {io} {nseq} sequences of {lo}-{hi}")


def test_decode_fp32_ragged_and_bf16_ck():
    wl = _small(lens=[700, 1024, 2049], io="fp32", topk=6, local=1, seed=22)
    _run_decode(wl, label="decode fp32")
    wl2 = _small(lens=[700, 1024, 2049], io="bf16", topk=6, local=1, seed=23)
    _run_decode(wl2, ck_dtype="bf16", label="decode bf16 ck-bf16")


def test_decode_scaled_logits_and_no_init():
    wl = _small(lens=[3000, 5000], topk=10, local=3, init=0, seed=24, score_scale=1 / math.sqrt(128))
    _run_decode(wl, label="decode score_scale=1/sqrt(d) init=0")


def test_decode_forced_only_and_dense():
    wl = _small(lens=[2000, 130], topk=3, local=2, init=1, seed=25)    # k == |F|
    _run_decode(wl, label="decode forced-only")
    wl = _small(lens=[500, 511, 512], topk=8, local=2, seed=26)        # c + 1 <= k: dense
    _run_decode(wl, label="decode dense")


@pytest.mark.parametrize("ck_dtype", ["fp32", "bf16"])
def test_compress_incremental_token_by_token(ck_dtype):
    """Decode-style cache growth: the compressed keys of a prefix, then one call
    per appended token for the kernel it completes (few-kernel path), equal the
    oracle's compressed keys of the whole sequence bit for bit."""
    h = _harness()
    wl = _small(lens=[3001, 700, 4500], topk=8, local=2, seed=29)
    _say(f"incremental compress ck={ck_dtype}")
    dev = h.DeviceWorkload(wl, ck_dtype)
    p, s = wl.kernel_size, wl.kernel_stride
    lens = wl.lens.astype(np.int64)
    start = lens - 60
    dev.compress(kv_lens=torch.tensor(start, device="cuda"))
    for step in range(1, 61):
        cur = start + step
        begin = np.array([max(0, h.num_kernels(int(n) - 1, p, s)) for n in cur], dtype=np.int64)
        new = max(h.num_kernels(int(n), p, s) - int(b0) for n, b0 in zip(cur, begin))
        dev.compress(kv_lens=torch.tensor(cur, device="cuda"),
                     ck_begin=torch.tensor(begin, device="cuda"), max_new=max(new, 1))
    torch.cuda.synchronize()
    cks = dev.ck_host()
    for b in range(wl.batch):
        want = ref.compress_keys(wl.k_f64(b), p, s, ck_dtype)
        assert np.array_equal(cks[b], want), f"sequence {b}"


@pytest.mark.parametrize("io,ck_dtype", [("bf16", "fp32"), ("bf16", "bf16"), ("fp32", "fp32")])
def test_append_kv_token_by_token(io, ck_dtype):
    """Decode-loop cache growth through infv2_append_kv: caches that start with a
    prefix, then one appended token per call, end up equal to the full K/V bit
    for bit, with compressed keys equal to the oracle's and lengths advanced; a
    full cache is left unchanged."""
    import trainable_block_sparse_amd as tbs
    h = _harness()
    wl = _small(lens=[400, 97, 1000], io=io, topk=8, local=2, seed=91)
    _say(f"append_kv io={io} ck={ck_dtype}")
    dev = h.DeviceWorkload(wl, ck_dtype)
    final = wl.lens.astype(np.int64)
    start = np.array([300, 10, 937], dtype=np.int64)
    offs = wl.kv_offsets
    hkv, d = wl.num_kv_heads, wl.head_dim
    # caches hold only the prefix; compressed keys of the prefix
    k_full, v_full = dev.k.clone(), dev.v.clone()
    for b in range(wl.batch):
        base, cap = int(offs[b]) * hkv * d, int(final[b])
        kb = dev.k[base: base + hkv * cap * d].view(hkv, cap, d)
        vb = dev.v[base: base + hkv * cap * d].view(hkv, cap, d)
        kb[:, int(start[b]):].zero_()
        vb[:, int(start[b]):].zero_()
    lens = torch.tensor(start, dtype=torch.int64, device="cuda")
    dev.compress(kv_lens=lens)
    steps = int((final - start).max()) + 2            # two extra calls hit full caches
    for step in range(steps):
        pos = np.minimum(start + step, final - 1)     # rows fed when a cache is already full are ignored
        kn = torch.stack([k_full[int(offs[b]) * hkv * d:].view(-1)[: hkv * int(final[b]) * d]
                          .view(hkv, int(final[b]), d)[:, int(pos[b])] for b in range(wl.batch)])
        vn = torch.stack([v_full[int(offs[b]) * hkv * d:].view(-1)[: hkv * int(final[b]) * d]
                          .view(hkv, int(final[b]), d)[:, int(pos[b])] for b in range(wl.batch)])
        tbs.infv2_append_kv(dev.cfg, kn.contiguous(), vn.contiguous(), dev.k, dev.v, dev.kv_offsets,
                            lens, dev.ck_offsets, dev.ck, wl.batch)
    torch.cuda.synchronize()
    assert lens.cpu().numpy().tolist() == final.tolist()
    assert torch.equal(dev.k, k_full) and torch.equal(dev.v, v_full)
    cks = dev.ck_host()
    for b in range(wl.batch):
        assert np.array_equal(cks[b], ref.compress_keys(wl.k_f64(b), wl.kernel_size,
                                                        wl.kernel_stride, ck_dtype)), f"seq {b}"


def test_dense_rows_without_scores():
    """Rows shorter than k*m with no block scores requested: the ids-only path
    gives the dense selection and the attention equals the oracle's."""
    import trainable_block_sparse_amd as tbs
    h = _harness()
    wl = _small(lens=[500, 1, 512, 64], topk=8, local=2, seed=92)
    _say("dense decode rows without scores")
    dev = h.DeviceWorkload(wl)
    dev.compress()
    B = wl.batch
    idx = torch.full((B, 2, 8), 7, dtype=torch.int32, device="cuda")
    tbs.infv2_select_blocks(dev.cfg, tbs.INFV2_MODE_DECODE, dev.q, B, 0, dev.ck, dev.ck_offsets,
                            dev.kv_offsets, dev.kv_lens, B, dev.max_len, idx, None,
                            dev.ws(tbs.OP_SELECT_DECODE, B, B, dev.max_len))
    out = h.from_device(dev.attn_decode(idx), "bf16")
    got = idx.cpu().numpy()
    prm = params_of(wl)
    q = wl.q_f64()
    for b in range(B):
        n = int(wl.lens[b])
        c = (n - 1) // 64
        want = np.array([r if r <= c else -1 for r in range(8)])
        assert (got[b] == want).all(), (b, got[b])
        ref_out = ref.attend_with_selection(q[b:b + 1], wl.k_f64(b), wl.v_f64(b), [n - 1],
                                            got[b:b + 1].astype(np.int64), prm)[0]
        assert_close(out[b], ref_out, "bf16", f"dense seq {b}")
    _say("dense prefill rows without scores")
    wp = _small(mode="prefill", lens=[700], topk=12, local=2, seed=93)
    devp = h.DeviceWorkload(wp)
    devp.compress()
    idxp = torch.full((700, 2, 12), 7, dtype=torch.int32, device="cuda")
    tbs.infv2_select_blocks(devp.cfg, tbs.INFV2_MODE_PREFILL, devp.q, 700, 0, devp.ck,
                            devp.ck_offsets, devp.kv_offsets, None, 1, 700, idxp, None,
                            devp.ws(tbs.OP_SELECT_PREFILL, 700, 1, 700))
    gp = idxp.cpu().numpy()
    for i in [0, 63, 64, 400, 699]:
        c = i // 64
        assert (gp[i] == np.array([r if r <= c else -1 for r in range(12)])).all(), i


def test_decode_first_token_attends_itself():
    h = _harness()
    wl = _small(lens=[1], topk=4, local=1, seed=27)
    _say("decode n=1")
    dev = h.DeviceWorkload(wl)
    dev.compress()
    idx, _ = dev.select_decode()
    out = h.from_device(dev.attn_decode(idx), "bf16")
    assert idx.cpu().numpy()[0, 0].tolist() == [0, -1, -1, -1]
    v0 = wl.v_f64(0)[:, 0, :]                                   # [Hkv][d]
    want = np.repeat(v0, 16, axis=0)
    assert np.array_equal(out[0], want)


@pytest.mark.parametrize("m", [32, 128])
def test_other_block_sizes(m):
    """Block sizes other than 64: decode (matrix cores, partial 64-key tiles) and
    prefill (vector-ALU attention)."""
    wl = _small(lens=[900, 2600], topk=6, local=2, seed=71 + m, block_size=m)
    _run_decode(wl, label=f"decode block {m}")
    wl = _small(mode="prefill", lens=[1300], topk=6, local=2, seed=72 + m, block_size=m)
    _run_prefill(wl, 500, label=f"prefill block {m}")


def test_large_topk():
    """Top-k at the supported maximum in decode (1024 blocks: 256 attention
    splits, a wide top-k window) and a bf16 prefill with top-k 160 (above what
    the matrix-core prefill attention takes, so the vector-ALU path serves it)."""
    wl = _small(lens=[1024 * 64 + 77, 1500 * 64], hkv=1, topk=1024, local=4, seed=81, n_planted=6)
    _run_decode(wl, label="decode top-k 1024")
    wl = _small(mode="prefill", lens=[12000], topk=160, local=4, seed=82, n_planted=6)
    rng = np.random.default_rng(82)
    pos = sorted(set(rng.integers(0, 12000, 40).tolist()) | {0, 10239, 10240, 11999})
    _run_prefill(wl, 4000, positions=pos, label="prefill top-k 160")


def test_prefill_topk128_union_at_capacity():
    """Top-k 128 in bf16 prefill: 16 rows x 128 selections, the most the
    matrix-core kernel's row-group union takes (2048 entries)."""
    wl = _small(mode="prefill", lens=[12000], topk=128, local=4, seed=83, n_planted=6)
    rng = np.random.default_rng(83)
    pos = sorted(set(rng.integers(8192, 12000, 40).tolist()) | set(range(12000 - 32, 12000)))
    _run_prefill(wl, 4000, positions=pos, label="prefill top-k 128")


def test_decode_batch_with_an_empty_sequence():
    """An empty cache (length 0) in a packed batch: no blocks (all ids -1), a zero
    output row, and the other sequences unaffected."""
    h = _harness()
    wl = _small(lens=[700, 0, 1, 3000], topk=8, local=2, seed=61)
    _say("decode batch with an empty sequence: lens [700, 0, 1, 3000]")
    dev = h.DeviceWorkload(wl)
    dev.compress()
    idx_t, _ = dev.select_decode()
    out = h.from_device(dev.attn_decode(idx_t), "bf16")
    idx = idx_t.cpu().numpy().astype(np.int64)
    assert (idx[1] == -1).all()
    assert not out[1].any()
    prm = params_of(wl)
    q = wl.q_f64()
    cks = dev.ck_host()
    for b in [0, 2, 3]:
        K = wl.k_f64(b)
        n = K.shape[1]
        for g in range(wl.num_kv_heads):
            rs = ref.select_row(q[b, 16 * g:16 * g + 16], cks[b][g], n - 1, prm)
            assert not accept_selection(idx[b, g], rs).startswith("fail")
        want = ref.attend_with_selection(q[b:b + 1], K, wl.v_f64(b), [n - 1], idx[b:b + 1], prm)
        assert_close(out[b], want[0], "bf16", f"seq {b}")


@pytest.mark.parametrize("cfg", [0, 1, 2, 4])
def test_decode_configs(cfg):
    wl = make_config(cfg)
    if cfg == 0:
        # the decode row of the tiny config: query row 1023 at position 1023
        wl = make_workload(mode="decode", io_dtype="fp32", lens=[1024], num_q_heads=16,
                           num_kv_heads=1, topk=8, init_blocks=1, local_blocks=2, n_planted=4, seed=0)
    _run_decode(wl, label=f"config {cfg} decode")


@pytest.mark.parametrize("topk,n", [(256, 20000), (1024, 70000)])
def test_decode_split_limits(topk, n):
    # one selected block per split at k = 256 (256 splits, small batch) and four
    # per split at the largest k (again 256 splits): the merge's limit both ways
    wl = _small(lens=[n], hkv=1, topk=topk, local=4, seed=29, n_planted=8)
    _run_decode(wl, label=f"decode k={topk}")


def test_decode_max_blocks_per_sequence():
    wl = _small(lens=[16384 * 64], hkv=1, topk=64, local=4, seed=28, n_planted=8)
    _run_decode(wl, label="decode 16384 blocks")


# ---------------------------------------------------------------------------- prefill
def _run_prefill(wl, chunk, ck_dtype="fp32", positions=None, label="prefill"):
    h = _harness()
    L = int(wl.lens[0])
    _say(f"{label}: L={L} chunk={chunk} io={wl.io_dtype} ck={ck_dtype} k={wl.topk}")
    dev = h.DeviceWorkload(wl, ck_dtype)
    idx_t, score_t, out_t = dev.prefill(chunk)
    torch.cuda.synchronize()
    idx = idx_t.cpu().numpy().astype(np.int64)
    score = score_t.cpu().numpy().astype(np.float64)
    out = h.from_device(out_t, wl.io_dtype)
    prm = params_of(wl, ck_dtype)
    K, V = wl.k_f64(0), wl.v_f64(0)
    ck = dev.ck_host()[0]
    assert np.array_equal(ck, ref.compress_keys(K, wl.kernel_size, wl.kernel_stride, ck_dtype)), \
        f"{label}: compressed keys differ"
    pos = list(range(L)) if positions is None else list(positions)
    q = wl.q_f64()
    G = prm.group
    rows, idx_rows, score_rows = [], [], []
    for i in pos:
        for g in range(wl.num_kv_heads):
            rows.append(ref.select_row(q[i, g * G:(g + 1) * G], ck[g], i, prm))
            idx_rows.append(idx[i, g])
            score_rows.append(score[i, g])
    _check_rows(np.array(idx_rows), np.array(score_rows), rows, label)
    want = ref.attend_with_selection(q[pos], K, V, pos, idx[pos], prm)
    err = assert_close(out[pos], want, wl.io_dtype, label)
    _say(f"{label}: output max abs err {err:.2e} over {len(pos)} rows, "
         f"{dev.check_canaries()} guarded buffers untouched")
    return dev, idx, out


def test_prefill_config0_all_rows_and_chunking():
    wl = make_config(0)
    _, idx_a, out_a = _run_prefill(wl, 1024, label="config 0 prefill")
    h = _harness()
    _say("config 0 prefill, 4 chunks of 256 vs one chunk")
    dev = h.DeviceWorkload(wl)
    idx_t, _, out_t = dev.prefill(256)
    assert np.array_equal(idx_t.cpu().numpy(), idx_a)
    assert np.array_equal(h.from_device(out_t, "fp32"), out_a)


def test_prefill_small_bf16_ragged_chunks():
    wl = _small(mode="prefill", lens=[1000], topk=6, local=1, init=1, seed=31,
                score_scale=1 / math.sqrt(128))
    _run_prefill(wl, 300, label="prefill bf16 ragged chunks")


def test_prefill_bf16_ck_and_forced_only():
    wl = _small(mode="prefill", lens=[777], topk=8, local=2, seed=32)
    _run_prefill(wl, 777, ck_dtype="bf16", label="prefill ck-bf16")
    wl = _small(mode="prefill", lens=[600], topk=3, local=2, seed=33)
    _run_prefill(wl, 250, label="prefill forced-only")


def test_prefill_config3_last_chunk_all_rows():
    """Config 3 (32K, chunks of 4096): every row of the last chunk (all 256
    16-row groups of the attention kernel), plus sampled rows of the others."""
    wl = make_config(3)
    rng = np.random.default_rng(303)
    L = int(wl.lens[0])
    pos = sorted(set(rng.integers(0, L - wl.chunk, 48).tolist()) | set(range(L - wl.chunk, L))
                 | {0, 63, 64, 4095, 4096, 4097, 8191})
    _run_prefill(wl, wl.chunk, positions=pos, label="config 3 prefill")


def _boundary_ties(rows):
    """Selections whose k'-th and (k'+1)-th candidate scores are exactly equal."""
    n = 0
    for rs in rows:
        cand = np.nonzero(~rs.forced)[0]
        sc = np.sort(rs.S[cand])[::-1]
        if rs.kprime > 0 and sc.shape[0] > rs.kprime and sc[rs.kprime - 1] == sc[rs.kprime]:
            n += 1
    return n


@pytest.mark.parametrize("cfg", [1, 2])
def test_decode_configs_many_queries(cfg):
    """Configs 1 and 2 at full size over 32 decode queries each: selections,
    block scores and outputs against the oracle, in guarded buffers; reports how
    many selections had an exact tie at the k-boundary."""
    from synth import extra_decode_queries
    h = _harness()
    wl = make_config(cfg)
    nq = 32
    _say(f"config {cfg} decode, {nq} queries")
    dev = h.DeviceWorkload(wl)
    dev.compress()
    qbits = extra_decode_queries(wl, nq)                       # [nq][1][Hq][d]
    prm = params_of(wl)
    K, V = wl.k_f64(0), wl.v_f64(0)
    n = K.shape[1]
    ck = dev.ck_host()[0]
    assert np.array_equal(ck, ref.compress_keys(K, wl.kernel_size, wl.kernel_stride, "fp32"))
    from synth import bf16_bits_to_f32
    rows, idx_rows, score_rows, outs, wants = [], [], [], [], []
    for r in range(nq):
        q_t = h.to_device(qbits[r])
        idx_t, score_t = dev.select_decode(q_t)
        out = h.from_device(dev.attn_decode(idx_t, q_t), "bf16")
        q = bf16_bits_to_f32(qbits[r]).astype(np.float64)
        gi = idx_t.cpu().numpy().astype(np.int64)
        gs = score_t.cpu().numpy().astype(np.float64)
        for g in range(wl.num_kv_heads):
            rows.append(ref.select_row(q[0, 16 * g:16 * g + 16], ck[g], n - 1, prm))
            idx_rows.append(gi[0, g])
            score_rows.append(gs[0, g])
        want = ref.attend_with_selection(q, K, V, [n - 1], gi, prm)
        assert_close(out, want, "bf16", f"config {cfg} query {r}")
    exact, band = _check_rows(np.array(idx_rows), np.array(score_rows), rows, f"config {cfg} decode x{nq}")
    _say(f"config {cfg}: {_boundary_ties(rows)} of {len(rows)} selections have an exact tie at the "
         f"k-boundary; {dev.check_canaries()} guarded buffers untouched")


@pytest.mark.parametrize("m,p,s,topk,L", [(16, 256, 256, 24, 20000), (128, 64, 32, 12, 6000)])
def test_prefill_other_kernel_geometries(m, p, s, topk, L):
    """bf16 prefill with kernel sizes and strides other than 32 / 16: a 64-kernel
    tile of stride 256 spans more than 512 blocks of 16 (the selection's
    multi-range path), and kernels of 64 at stride 32 over blocks of 128."""
    wl = _small(mode="prefill", lens=[L], topk=topk, local=2, seed=140 + m, block_size=m,
                kernel_size=p, kernel_stride=s)
    rng = np.random.default_rng(140 + m)
    pos = sorted(set(rng.integers(0, L, 96).tolist()) | set(range(L - 64, L)) | {p - 1, p, L // 2})
    _run_prefill(wl, 4096, positions=pos, label=f"prefill m={m} p={p} s={s}")


def test_default_scales_equal_explicit_ones():
    """attn_scale = 0 and score_scale = 0 in the C struct select 1/sqrt(d) and 1:
    the same bits as passing those values."""
    import dataclasses
    import math as _m
    import trainable_block_sparse_amd as tbs
    h = _harness()
    wl = _small(lens=[5000, 900], topk=8, local=2, seed=151)
    _say("default scales vs explicit")
    dev = h.DeviceWorkload(wl)
    dev.compress()
    idx0, _ = dev.select_decode()
    out0 = dev.attn_decode(idx0)
    dev.cfg = dataclasses.replace(dev.cfg, attn_scale=float(np.float32(1.0 / _m.sqrt(128))),
                                  score_scale=1.0)
    idx1, _ = dev.select_decode()
    out1 = dev.attn_decode(idx1)
    dev.cfg = dataclasses.replace(dev.cfg, attn_scale=0.0, score_scale=0.0)
    idx2, _ = dev.select_decode()
    out2 = dev.attn_decode(idx2)
    torch.cuda.synchronize()
    assert torch.equal(idx0, idx1) and torch.equal(out0, out1)
    assert torch.equal(idx0, idx2) and torch.equal(out0, out2)
    assert tbs.Config().to_c().attn_scale == 0.0


def _with_keys(wl, keys_of_seq):
    """Replace the keys of every sequence of a workload by keys_of_seq(b, [Hkv][n][d])."""
    from synth import f32_to_bf16_bits
    parts = []
    for b in range(wl.batch):
        n = int(wl.lens[b])
        kf = np.asarray(keys_of_seq(b, (wl.num_kv_heads, n, wl.head_dim)), dtype=np.float32)
        parts.append((f32_to_bf16_bits(kf) if wl.io_dtype == "bf16" else kf).reshape(-1))
    wl.k = np.concatenate(parts)
    return wl


def _levels(n_levels, seed):
    """Keys constant inside each 64-token block, one of n_levels multiples of a
    direction: many exactly equal block scores, so the top-k boundary falls
    inside a run of ties."""
    rng = np.random.default_rng(seed)

    def keys(b, shape):
        hkv, n, d = shape
        u = rng.standard_normal(d)
        u /= np.linalg.norm(u)
        lvl = rng.integers(0, n_levels, size=(hkv, -(-n // 64)))
        return np.repeat(lvl, 64, axis=1)[:, :n, None] * 0.5 * u[None, None, :]
    return keys


def test_selection_with_massive_ties():
    """All scores equal (the lowest blocks win) and a few distinct score levels
    (the boundary falls inside long runs of equal scores)."""
    zero = lambda b, shape: np.zeros(shape)
    wl = _with_keys(_small(lens=[7000, 20000], topk=16, local=2, seed=51), zero)
    _run_decode(wl, label="decode all-equal scores")
    wl = _with_keys(_small(lens=[9000, 33000], topk=24, local=3, seed=52), _levels(3, 52))
    _run_decode(wl, label="decode 3 score levels")
    wl = _with_keys(_small(lens=[5000], topk=20, local=2, seed=53), _levels(6, 53))
    _run_decode(wl, label="decode 6 score levels")
    wl = _with_keys(_small(mode="prefill", lens=[2000], topk=8, local=2, seed=54), _levels(2, 54))
    _run_prefill(wl, 700, label="prefill 2 score levels")
    wl = _with_keys(_small(mode="prefill", lens=[1500], topk=6, local=1, seed=55), zero)
    _run_prefill(wl, 1500, label="prefill all-equal scores")


def _isolated_high(n_high, seed):
    """Keys constant inside each 64-token block: one level of a direction for
    every block but n_high isolated ones per KV head at twice that level.  The
    blocks whose overlapping kernels see only the common level all score exactly
    alike (hundreds of them); the high blocks and their neighbours differ."""
    rng = np.random.default_rng(seed)

    def keys(b, shape):
        hkv, n, d = shape
        u = rng.standard_normal(d)
        u /= np.linalg.norm(u)
        nb = -(-n // 64)
        lvl = np.ones((hkv, nb))
        for g in range(hkv):
            lvl[g, rng.choice(np.arange(8, nb - 16, 4), size=n_high, replace=False)] = 2.0
        return np.repeat(lvl, 64, axis=1)[:, :n, None] * 0.5 * u[None, None, :]
    return keys


def _ties_with_keys_above(wl, ck, rows):
    """The oracle's view: at each (row, KV head) more than 256 candidates share
    the score of the k'-th largest, and some score above it."""
    prm = params_of(wl)
    q = wl.q_f64()
    for i in rows:
        for g in range(wl.num_kv_heads):
            qi = q[0 if wl.mode == "decode" else i, 16 * g:16 * g + 16]
            rs = ref.select_row(qi, ck[g], i, prm)
            sc = rs.S[~rs.forced]
            thr = np.sort(sc)[::-1][rs.kprime - 1]
            assert (sc == thr).sum() > 256 and (sc > thr).sum() > 0, (i, g)


def _fused_step_equals(dev, wl, idx, out):
    """infv2_decode_step on the cache of a _run_decode (compressed keys complete:
    the step rebuilds the newest kernel's key with the same bits) gives the same
    selection and output as the separate calls."""
    import trainable_block_sparse_amd as tbs
    h = _harness()
    B = wl.batch
    ws = torch.zeros(tbs.infv2_workspace_bytes(dev.cfg, tbs.OP_DECODE_STEP, B, B, dev.max_len),
                     dtype=torch.uint8, device="cuda")
    idx_s = dev.guarded((B, wl.num_kv_heads, wl.topk), torch.int32)
    out_s = dev.guarded(tuple(dev.q.shape), dev.q.dtype)
    lens = torch.tensor(wl.lens.astype(np.int64), device="cuda")
    tbs.infv2_decode_step(dev.cfg, dev.q, dev.k, dev.v, dev.kv_offsets, lens, dev.ck_offsets, dev.ck,
                          B, dev.max_len, idx_s, out_s, ws)
    torch.cuda.synchronize()
    assert np.array_equal(idx_s.cpu().numpy().astype(np.int64), idx), "decode step: selection"
    assert np.array_equal(h.from_device(out_s, wl.io_dtype), out), "decode step: output"
    _say(f"decode step equal; {dev.check_canaries()} guarded buffers untouched")


def test_decode_beyond_2048_blocks():
    """A 200K-token cache (3125 blocks: 13 block keys per top-k thread, the
    16-key register instantiation and two bitmap words per lane in the fused
    step) at k = 64, against the oracle, and the fused step against the
    separate calls."""
    wl = _small(lens=[200000], topk=64, local=4, seed=63, n_planted=6)
    dev, idx, out = _run_decode(wl, label="decode 200K")
    _fused_step_equals(dev, wl, idx, out)


def test_selection_ties_at_threshold_with_keys_above():
    """More than 256 candidates share the score at the top-k threshold (more
    than the rank step takes, so the narrowing ends on a single key value) and
    a few candidates score above it: the selection keeps those and the lowest
    blocks of the tied run, in the decode selection, the fused decode step (its
    own top-k) and the prefill selection."""
    wl = _with_keys(_small(lens=[40000], topk=40, local=2, seed=61), _isolated_high(6, 61))
    K = wl.k_f64(0)
    _ties_with_keys_above(wl, ref.compress_keys(K, wl.kernel_size, wl.kernel_stride, "fp32"),
                          [K.shape[1] - 1])
    dev, idx, out = _run_decode(wl, label="decode: ties at the threshold, keys above")
    _fused_step_equals(dev, wl, idx, out)
    wp = _with_keys(_small(mode="prefill", lens=[24000], topk=40, local=2, seed=62), _isolated_high(6, 62))
    Kp = wp.k_f64(0)
    _ties_with_keys_above(wp, ref.compress_keys(Kp, wp.kernel_size, wp.kernel_stride, "fp32"),
                          [23999, 20000])
    _run_prefill(wp, 4000, positions=[0, 4095, 20000, 23000, 23999],
                 label="prefill: ties at the threshold, keys above")


def test_prefill_chunks_on_two_streams():
    """Concurrent calls on two streams with their own workspaces, as the header
    allows: each chunk's attention on a second stream while the next chunk's
    compression and selection run on the first.  Same compressed keys,
    selections and outputs, bit for bit, as the calls made one after another."""
    import trainable_block_sparse_amd as tbs
    h = _harness()
    wl = _small(mode="prefill", lens=[12000], topk=16, local=2, seed=91)
    L, C = 12000, 2000
    _say("prefill chunks on two streams")
    a = h.DeviceWorkload(wl)
    idx_a, _, out_a = a.prefill(C)
    b = h.DeviceWorkload(wl)
    p, s = wl.kernel_size, wl.kernel_stride
    idx_b = b.guarded((L, wl.num_kv_heads, b.cfg.topk), torch.int32)
    out_b = b.guarded(tuple(b.q.shape), b.q.dtype)
    ws = b.ws(tbs.OP_SELECT_PREFILL, C, 1, L)
    wsa = b.ws(tbs.OP_ATTN_PREFILL, C, 1, L)
    starts = list(range(0, L, C))
    lens = [torch.tensor([min(L, q0 + C)], dtype=torch.int64, device="cuda") for q0 in starts]
    begins = [torch.tensor([h.num_kernels(q0, p, s)], dtype=torch.int64, device="cuda") for q0 in starts]
    torch.cuda.synchronize()
    main, side = torch.cuda.current_stream(), torch.cuda.Stream()
    side.wait_stream(main)
    for c, q0 in enumerate(starts):
        q1 = min(L, q0 + C)
        tbs.infv2_compress_keys(b.cfg, b.k, b.kv_offsets, lens[c], b.ck_offsets, begins[c], 1, q1,
                                h.num_kernels(q1, p, s) - h.num_kernels(q0, p, s), b.ck)
        tbs.infv2_select_blocks(b.cfg, tbs.INFV2_MODE_PREFILL, b.q[q0:q1], q1 - q0, q0, b.ck,
                                b.ck_offsets, b.kv_offsets, None, 1, q1, idx_b[q0:q1], None, ws)
        side.wait_stream(main)
        with torch.cuda.stream(side):
            tbs.infv2_sparse_attn_prefill(b.cfg, b.q[q0:q1], q1 - q0, q0, b.k, b.v, b.kv_offsets,
                                          idx_b[q0:q1], out_b[q0:q1], wsa)
    main.wait_stream(side)
    torch.cuda.synchronize()
    assert torch.equal(a.ck, b.ck), "compressed keys"
    assert torch.equal(idx_a, idx_b), "selection"
    assert torch.equal(out_a, out_b), "output"
    _say(f"two streams equal; {b.check_canaries()} guarded buffers untouched")


def test_varlen_prefill_equals_per_sequence_calls():
    """Serving-style prefill: three sequences, each with a chunk of rows starting
    mid-sequence, in one varlen call.  Selections and outputs equal the
    single-sequence calls bit for bit and the oracle on sampled rows; the
    selection run as one launch (workspace for all rows) equals the one run
    sequence after sequence."""
    import trainable_block_sparse_amd as tbs
    from synth import f32_to_bf16_bits
    h = _harness()
    wl = _small(lens=[5000, 1200, 9000], topk=16, local=4, seed=101)
    _say("varlen prefill: 3 sequences, chunks (2000@3000, 700@500, 3000@6000)")
    dev = h.DeviceWorkload(wl)
    dev.compress()
    starts = np.array([3000, 500, 6000], dtype=np.int64)
    rows = np.array([2000, 700, 3000], dtype=np.int32)
    rng = np.random.default_rng(101)
    qf = rng.standard_normal((int(rows.sum()), wl.num_q_heads, wl.head_dim), dtype=np.float32)
    qbits = f32_to_bf16_bits(qf)
    q = h.to_device(qbits)
    cfg, hkv, k = dev.cfg, wl.num_kv_heads, 16
    T = int(rows.sum())
    idx_v = torch.empty((T, hkv, k), dtype=torch.int32, device="cuda")
    out_v = torch.empty_like(q)
    max_len = int((starts + rows).max())
    ws_s = dev.ws(tbs.OP_SELECT_PREFILL, int(rows.max()), 1, max_len)
    ws_a = torch.zeros(max(256, tbs.infv2_workspace_bytes(cfg, tbs.OP_ATTN_PREFILL, int(rows.max()), 1,
                                                         max_len)), dtype=torch.uint8, device="cuda")
    tbs.infv2_select_blocks_varlen(cfg, q, rows, starts, dev.ck, dev.ck_offsets, dev.kv_offsets,
                                   idx_v, None, ws_s)
    tbs.infv2_sparse_attn_prefill_varlen(cfg, q, rows, starts, dev.k, dev.v, dev.kv_offsets, idx_v,
                                         out_v, ws_a)
    # a workspace for all rows of the call: the selection runs as one launch per
    # kernel for the three sequences (above: sequence after sequence)
    ws_all = dev.ws(tbs.OP_SELECT_PREFILL, T, 3, max_len)
    idx_1 = torch.empty_like(idx_v)
    score_1 = torch.empty((T, hkv, k), dtype=torch.float32, device="cuda")
    score_v = torch.empty_like(score_1)
    tbs.infv2_select_blocks_varlen(cfg, q, rows, starts, dev.ck, dev.ck_offsets, dev.kv_offsets,
                                   idx_1, score_1, ws_all)
    tbs.infv2_select_blocks_varlen(cfg, q, rows, starts, dev.ck, dev.ck_offsets, dev.kv_offsets,
                                   idx_v, score_v, ws_s)
    torch.cuda.synchronize()
    assert torch.equal(idx_1, idx_v), "one-launch selection differs from sequence after sequence"
    # bit patterns: padding slots hold NaN
    assert torch.equal(score_1.view(torch.int32), score_v.view(torch.int32)), "one-launch block scores differ"
    r0 = 0
    prm = params_of(wl)
    for b in range(3):
        r1 = r0 + int(rows[b])
        idx_s = torch.empty((int(rows[b]), hkv, k), dtype=torch.int32, device="cuda")
        out_s = torch.empty((int(rows[b]), wl.num_q_heads, wl.head_dim), dtype=q.dtype, device="cuda")
        nb = int(starts[b]) + int(rows[b])
        tbs.infv2_select_blocks(cfg, tbs.INFV2_MODE_PREFILL, q[r0:r1], int(rows[b]), int(starts[b]),
                                dev.ck, dev.ck_offsets[b:], dev.kv_offsets[b:], None, 1, nb, idx_s,
                                None, ws_s)
        tbs.infv2_sparse_attn_prefill(cfg, q[r0:r1], int(rows[b]), int(starts[b]), dev.k, dev.v,
                                      dev.kv_offsets[b:], idx_s, out_s, ws_a)
        torch.cuda.synchronize()
        assert torch.equal(idx_v[r0:r1], idx_s), f"seq {b}: selection"
        assert torch.equal(out_v[r0:r1], out_s), f"seq {b}: output"
        # oracle on a few rows of the chunk
        K = wl.k_f64(b)
        ck = dev.ck_host()[b]
        qrows = h.from_device(q[r0:r1], "bf16")
        picks = [0, int(rows[b]) // 2, int(rows[b]) - 1]
        gi = idx_v[r0:r1].cpu().numpy().astype(np.int64)
        for loc in picks:
            i = int(starts[b]) + loc
            for g in range(hkv):
                rs = ref.select_row(qrows[loc, 16 * g:16 * g + 16], ck[g], i, prm)
                assert not accept_selection(gi[loc, g], rs).startswith("fail"), (b, loc, g)
        want = ref.attend_with_selection(qrows[picks], K, wl.v_f64(b), [int(starts[b]) + x for x in picks],
                                         gi[picks], prm)
        assert_close(h.from_device(out_v[r0:r1], "bf16")[picks], want, "bf16", f"varlen seq {b}")
        r0 = r1


def test_varlen_prefill_more_sequences_than_one_launch_takes():
    """70 short sequences in one varlen call: more than one launch holds (64
    sequences per launch), so both the selection (workspace for all rows) and
    the attention run in two launches.  Selections and outputs equal the
    single-sequence calls bit for bit, and the oracle on sampled rows."""
    import trainable_block_sparse_amd as tbs
    from synth import f32_to_bf16_bits
    h = _harness()
    rng = np.random.default_rng(131)
    nseq = 70
    lens = rng.integers(40, 400, size=nseq, endpoint=True)
    wl = _small(lens=lens.tolist(), topk=4, local=1, seed=131, n_planted=1)
    _say(f"varlen prefill: {nseq} sequences of 40-400 tokens, the last rows of each")
    dev = h.DeviceWorkload(wl)
    dev.compress()
    rows = np.array([int(rng.integers(1, n, endpoint=True)) for n in lens], dtype=np.int32)
    starts = (lens - rows).astype(np.int64)
    T = int(rows.sum())
    qf = rng.standard_normal((T, wl.num_q_heads, wl.head_dim), dtype=np.float32)
    q = h.to_device(f32_to_bf16_bits(qf))
    cfg, hkv, k = dev.cfg, wl.num_kv_heads, wl.topk
    max_len = int(lens.max())
    ws_all = dev.ws(tbs.OP_SELECT_PREFILL, T, nseq, max_len)
    ws_a = torch.zeros(max(256, tbs.infv2_workspace_bytes(cfg, tbs.OP_ATTN_PREFILL, int(rows.max()), 1,
                                                         max_len)), dtype=torch.uint8, device="cuda")
    idx_v = torch.empty((T, hkv, k), dtype=torch.int32, device="cuda")
    out_v = torch.empty_like(q)
    tbs.infv2_select_blocks_varlen(cfg, q, rows, starts, dev.ck, dev.ck_offsets, dev.kv_offsets,
                                   idx_v, None, ws_all)
    tbs.infv2_sparse_attn_prefill_varlen(cfg, q, rows, starts, dev.k, dev.v, dev.kv_offsets, idx_v,
                                         out_v, ws_a)
    torch.cuda.synchronize()
    ws_s = dev.ws(tbs.OP_SELECT_PREFILL, int(rows.max()), 1, max_len)
    prm = params_of(wl)
    qrows_all = h.from_device(q, "bf16")
    r0 = 0
    checked = 0
    for b in range(nseq):
        r1 = r0 + int(rows[b])
        idx_s = torch.empty((int(rows[b]), hkv, k), dtype=torch.int32, device="cuda")
        out_s = torch.empty((int(rows[b]), wl.num_q_heads, wl.head_dim), dtype=q.dtype, device="cuda")
        nb = int(starts[b]) + int(rows[b])
        tbs.infv2_select_blocks(cfg, tbs.INFV2_MODE_PREFILL, q[r0:r1], int(rows[b]), int(starts[b]),
                                dev.ck, dev.ck_offsets[b:], dev.kv_offsets[b:], None, 1, nb, idx_s,
                                None, ws_s)
        tbs.infv2_sparse_attn_prefill(cfg, q[r0:r1], int(rows[b]), int(starts[b]), dev.k, dev.v,
                                      dev.kv_offsets[b:], idx_s, out_s, ws_a)
        torch.cuda.synchronize()
        assert torch.equal(idx_v[r0:r1], idx_s), f"seq {b}: selection"
        assert torch.equal(out_v[r0:r1], out_s), f"seq {b}: output"
        if b % 9 == 0 or b >= 63:           # the oracle on the last row of some sequences
            K = wl.k_f64(b)
            ck = dev.ck_host()[b]
            loc = int(rows[b]) - 1
            i = int(starts[b]) + loc
            gi = idx_v[r0:r1].cpu().numpy().astype(np.int64)
            for g in range(hkv):
                rs = ref.select_row(qrows_all[r0 + loc, 16 * g:16 * g + 16], ck[g], i, prm)
                assert not accept_selection(gi[loc, g], rs).startswith("fail"), (b, loc, g)
            want = ref.attend_with_selection(qrows_all[r0 + loc:r0 + loc + 1], K, wl.v_f64(b), [i],
                                             gi[loc:loc + 1], prm)
            assert_close(h.from_device(out_v[r0 + loc:r0 + loc + 1], "bf16"), want, "bf16", f"varlen seq {b}")
            checked += 1
        r0 = r1
    assert checked >= 10


@pytest.mark.parametrize("io,ck_dtype,keys", [("bf16", "fp32", "random"), ("bf16", "bf16", "random"),
                                              ("fp32", "fp32", "random"), ("bf16", "fp32", "levels"),
                                              ("bf16", "fp32", "equal"), ("bf16", "fp32", "batch16"),
                                              ("bf16", "bf16", "batch16")])
def test_decode_step_equals_separate_calls(io, ck_dtype, keys):
    """infv2_decode_step (compressed key of the kernel the newest token completes,
    selection, attention in one call; with bf16 the compression runs inside the
    selection's first kernel, and at small batches the top-k inside the
    attention) equals infv2_compress_keys + infv2_select_blocks +
    infv2_sparse_attn_decode bit for bit, over 40 steps of growing caches that
    complete a kernel every 16 tokens; the compressed keys end equal to the
    oracle's.  keys: random, three score levels (top-k boundary inside runs of
    equal scores), all equal (the lowest blocks win), or batch16: 16 sequences
    of 20K-40K tokens at k = 64, a grid where the logits pass takes plain loads
    and the attention's waves run two tiles each."""
    import trainable_block_sparse_amd as tbs
    from synth import extra_decode_queries
    h = _harness()
    if keys == "batch16":
        lens = np.random.default_rng(173).integers(20000, 40000, size=16, endpoint=True).tolist()
        wl = _small(lens=lens, io=io, topk=64, local=4, seed=173)
    else:
        wl = _small(lens=[3001, 700, 4500, 33], io=io, topk=8, local=2, seed=171)
    if keys == "levels":
        wl = _with_keys(wl, _levels(3, 172))
    elif keys == "equal":
        wl = _with_keys(wl, lambda b, shape: np.zeros(shape))
    _say(f"decode step vs separate calls io={io} ck={ck_dtype} keys={keys}")
    a = h.DeviceWorkload(wl, ck_dtype)
    b = h.DeviceWorkload(wl, ck_dtype)
    p, s = wl.kernel_size, wl.kernel_stride
    final = wl.lens.astype(np.int64)
    start = np.maximum(final - 40, 1)
    for dev in (a, b):
        dev.compress(kv_lens=torch.tensor(start - 1, device="cuda"))
    qs = h.to_device(extra_decode_queries(wl, 41))
    B, hkv, k = wl.batch, wl.num_kv_heads, wl.topk
    ws_step = torch.zeros(tbs.infv2_workspace_bytes(a.cfg, tbs.OP_DECODE_STEP, B, B, a.max_len),
                          dtype=torch.uint8, device="cuda")
    ws_s = b.ws(tbs.OP_SELECT_DECODE, B, B, b.max_len)
    ws_a = b.ws(tbs.OP_ATTN_DECODE, B, B, b.max_len)
    for step in range(41):
        cur = np.minimum(start + step, final)
        lens = torch.tensor(cur, dtype=torch.int64, device="cuda")
        idx_a = a.guarded((B, hkv, k), torch.int32)
        out_a = a.guarded(tuple(qs[step].shape), qs[step].dtype)
        tbs.infv2_decode_step(a.cfg, qs[step], a.k, a.v, a.kv_offsets, lens, a.ck_offsets, a.ck, B,
                              a.max_len, idx_a, out_a, ws_step)
        # separate calls: the newest token's kernel (or, when it completes none, the
        # last complete one again: the same value), then selection and attention
        begin = torch.tensor([max(0, h.num_kernels(int(n), p, s) - 1) for n in cur], device="cuda")
        b.compress(kv_lens=lens, ck_begin=begin, max_new=1)
        idx_b = torch.empty((B, hkv, k), dtype=torch.int32, device="cuda")
        tbs.infv2_select_blocks(b.cfg, tbs.INFV2_MODE_DECODE, qs[step], B, 0, b.ck, b.ck_offsets,
                                b.kv_offsets, lens, B, b.max_len, idx_b, None, ws_s)
        out_b = torch.empty_like(qs[step])
        tbs.infv2_sparse_attn_decode(b.cfg, qs[step], b.k, b.v, b.kv_offsets, lens, B, b.max_len,
                                     idx_b, out_b, ws_a)
        torch.cuda.synchronize()
        assert torch.equal(idx_a, idx_b), f"step {step}: selection differs"
        assert torch.equal(out_a, out_b), f"step {step}: output differs"
    assert torch.equal(a.ck, b.ck)
    cks = a.ck_host()
    for sq in range(B):
        assert np.array_equal(cks[sq], ref.compress_keys(wl.k_f64(sq), p, s, ck_dtype)), f"seq {sq}"
    _say(f"decode step: 41 steps equal, {a.check_canaries()} guarded buffers untouched")


@pytest.mark.parametrize("io,ck_dtype,keys", [("bf16", "fp32", "random"), ("bf16", "bf16", "random"),
                                              ("bf16", "fp32", "batch16"), ("fp32", "fp32", "random")])
def test_decode_step_append_equals_append_then_step(io, ck_dtype, keys):
    """infv2_decode_step_append (the new token's K/V written into the caches by
    the step's first kernel, the lengths advanced by its last) equals
    infv2_append_kv followed by infv2_decode_step bit for bit, over 41 steps
    that complete a kernel every 16 tokens: selections and outputs every step;
    caches, compressed keys and lengths at the end.  The cache rows past the
    start are cleared first, so a row the step fails to write shows; the
    shortest sequences reach their capacity and take no-op appends.  fp32
    inputs take the two-call path."""
    import trainable_block_sparse_amd as tbs
    from synth import extra_decode_queries
    h = _harness()
    if keys == "batch16":
        lens = np.random.default_rng(183).integers(20000, 40000, size=16, endpoint=True).tolist()
        wl = _small(lens=lens, io=io, topk=64, local=4, seed=183)
    else:
        wl = _small(lens=[3001, 700, 4500, 33], io=io, topk=8, local=2, seed=181)
    _say(f"decode step with append vs append + step io={io} ck={ck_dtype} keys={keys}")
    a = h.DeviceWorkload(wl, ck_dtype)
    b = h.DeviceWorkload(wl, ck_dtype)
    B, hkv, d, k = wl.batch, wl.num_kv_heads, wl.head_dim, wl.topk
    cap = wl.lens.astype(np.int64)
    off = np.concatenate([[0], np.cumsum(cap)])
    start = np.maximum(cap - 40, 1)
    k_full = a.k.clone().reshape(-1, d)
    v_full = a.v.clone().reshape(-1, d)

    def rows_of(bi, g, lo, hi):
        base = int(off[bi]) * hkv + g * int(cap[bi])
        return slice(base + lo, base + hi)
    for dev in (a, b):
        kk, vv = dev.k.view(-1, d), dev.v.view(-1, d)
        for bi in range(B):
            for g in range(hkv):
                kk[rows_of(bi, g, int(start[bi]), int(cap[bi]))] = 0
                vv[rows_of(bi, g, int(start[bi]), int(cap[bi]))] = 0
        dev.kv_lens.copy_(torch.tensor(start, device="cuda"))
        dev.compress(kv_lens=dev.kv_lens)
    qs = h.to_device(extra_decode_queries(wl, 41))
    ws_a = torch.zeros(tbs.infv2_workspace_bytes(a.cfg, tbs.OP_DECODE_STEP, B, B, a.max_len),
                       dtype=torch.uint8, device="cuda")
    ws_b = torch.zeros_like(ws_a)
    for step in range(41):
        pos = np.minimum(start + step, cap - 1)          # the row appended (ignored when full)
        idx_rows = [rows_of(bi, g, int(pos[bi]), int(pos[bi]) + 1) for bi in range(B) for g in range(hkv)]
        k_new = torch.cat([k_full[r] for r in idx_rows]).reshape(B, hkv, d).contiguous()
        v_new = torch.cat([v_full[r] for r in idx_rows]).reshape(B, hkv, d).contiguous()
        idx_a = a.guarded((B, hkv, k), torch.int32)
        out_a = a.guarded(tuple(qs[step].shape), qs[step].dtype)
        tbs.infv2_decode_step_append(a.cfg, qs[step], k_new, v_new, a.k, a.v, a.kv_offsets, a.kv_lens,
                                     a.ck_offsets, a.ck, B, a.max_len, idx_a, out_a, ws_a)
        tbs.infv2_append_kv(b.cfg, k_new, v_new, b.k, b.v, b.kv_offsets, b.kv_lens, b.ck_offsets, b.ck, B)
        idx_b = torch.empty((B, hkv, k), dtype=torch.int32, device="cuda")
        out_b = torch.empty_like(qs[step])
        tbs.infv2_decode_step(b.cfg, qs[step], b.k, b.v, b.kv_offsets, b.kv_lens, b.ck_offsets, b.ck, B,
                              b.max_len, idx_b, out_b, ws_b)
        torch.cuda.synchronize()
        assert torch.equal(idx_a, idx_b), f"step {step}: selection differs"
        assert torch.equal(out_a, out_b), f"step {step}: output differs"
    assert torch.equal(a.kv_lens, b.kv_lens), "lengths"
    assert torch.equal(a.kv_lens.cpu(), torch.tensor(np.minimum(start + 41, cap))), "lengths advanced"
    assert torch.equal(a.k, b.k) and torch.equal(a.v, b.v), "caches"
    assert torch.equal(a.k.reshape(-1, d), k_full) and torch.equal(a.v.reshape(-1, d), v_full), \
        "caches refilled with the appended rows"
    assert torch.equal(a.ck, b.ck), "compressed keys"
    cks = a.ck_host()
    for sq in range(B):
        assert np.array_equal(cks[sq], ref.compress_keys(wl.k_f64(sq), wl.kernel_size, wl.kernel_stride,
                                                         ck_dtype)), f"seq {sq}"
    _say(f"decode step with append: 41 steps equal, {a.check_canaries()} guarded buffers untouched")


def test_decode_step_append_graph_replays():
    """A captured graph of three appending decode steps, replayed three times
    with eager work and synchronisations in between (lengths, caches and
    compressed keys advance on every replay), equals nine eager steps on a twin
    cache: each replay's last selection and output, and the final state."""
    import trainable_block_sparse_amd as tbs
    from synth import extra_decode_queries
    h = _harness()
    wl = _small(lens=[9000, 20000], topk=16, local=4, seed=187)
    _say("graph replays of the appending decode step")
    a = h.DeviceWorkload(wl)
    b = h.DeviceWorkload(wl)
    B, hkv, d, k = wl.batch, wl.num_kv_heads, wl.head_dim, wl.topk
    start = wl.lens.astype(np.int64) - 20                 # room for nine appends
    for dev in (a, b):
        dev.kv_lens.copy_(torch.tensor(start, device="cuda"))
        dev.compress(kv_lens=dev.kv_lens)
    qs = h.to_device(extra_decode_queries(wl, 3))
    rng = np.random.default_rng(187)
    kv_new = [torch.tensor(rng.standard_normal((B, hkv, d)), dtype=torch.float32, device="cuda").to(torch.bfloat16)
              for _ in range(6)]
    ws_a = torch.zeros(tbs.infv2_workspace_bytes(a.cfg, tbs.OP_DECODE_STEP, B, B, a.max_len),
                       dtype=torch.uint8, device="cuda")
    ws_b = torch.zeros_like(ws_a)
    idx_a = torch.empty((B, hkv, k), dtype=torch.int32, device="cuda")
    out_a = torch.empty_like(qs[0])

    def step(dev, i, ws, idx, out):
        tbs.infv2_decode_step_append(dev.cfg, qs[i], kv_new[2 * i], kv_new[2 * i + 1], dev.k, dev.v,
                                     dev.kv_offsets, dev.kv_lens, dev.ck_offsets, dev.ck, B, dev.max_len,
                                     idx, out, ws)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            for i in range(3):
                step(a, i, ws_a, idx_a, out_a)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    assert torch.equal(a.kv_lens.cpu(), torch.tensor(start)), "capture ran the steps"
    for rep in range(3):
        g.replay()
        torch.cuda.synchronize()
        _ = (a.q.float() * 2).sum().item()             # eager work between replays
        for i in range(3):
            idx_b = torch.empty((B, hkv, k), dtype=torch.int32, device="cuda")
            out_b = torch.empty_like(qs[0])
            step(b, i, ws_b, idx_b, out_b)
        torch.cuda.synchronize()
        assert torch.equal(idx_a, idx_b), f"replay {rep}: selection"
        assert torch.equal(out_a, out_b), f"replay {rep}: output"
        assert torch.equal(a.kv_lens, b.kv_lens), f"replay {rep}: lengths"
    assert torch.equal(a.kv_lens.cpu(), torch.tensor(start + 9))
    assert torch.equal(a.k, b.k) and torch.equal(a.v, b.v) and torch.equal(a.ck, b.ck)


def test_decode_equals_last_prefill_row():
    h = _harness()
    wl = _small(mode="prefill", lens=[1500], topk=8, local=2, seed=34)
    _say("decode vs prefill last row")
    dev = h.DeviceWorkload(wl)
    idx_p, _, out_p = dev.prefill(512)
    wd = _small(mode="decode", lens=[1500], topk=8, local=2, seed=34)
    # same K/V; query of the decode row = last prefill row
    wd.k, wd.v = wl.k, wl.v
    wd.q = wl.q[-1:].copy()
    devd = h.DeviceWorkload(wd)
    devd.compress()
    idx_d, _ = devd.select_decode()
    out_d = devd.attn_decode(idx_d)
    assert np.array_equal(idx_d.cpu().numpy()[0], idx_p.cpu().numpy()[-1])
    assert_close(h.from_device(out_d, "bf16")[0], h.from_device(out_p, "bf16")[-1], "bf16",
                 "decode vs prefill")


def test_decode_step_graph_replays_match_eager():
    """A captured decode step (compress + select + attend) replayed several times,
    with eager work and synchronisations in between, equals the eager result."""
    h = _harness()
    from synth import extra_decode_queries
    import trainable_block_sparse_amd as tbs
    wl = _small(lens=[9000, 20000], topk=16, local=4, seed=41)
    _say("graph replay of a decode step")
    dev = h.DeviceWorkload(wl)
    dev.compress()
    qs = h.to_device(extra_decode_queries(wl, 3))
    B = wl.batch
    idx = torch.empty((B, 2, 16), dtype=torch.int32, device="cuda")
    out = torch.empty_like(dev.q)
    ws_s = dev.ws(tbs.OP_SELECT_DECODE, B, B, dev.max_len)
    ws_a = dev.ws(tbs.OP_ATTN_DECODE, B, B, dev.max_len)
    qbuf = qs[0].clone()

    def step():
        dev.compress()
        tbs.infv2_select_blocks(dev.cfg, tbs.INFV2_MODE_DECODE, qbuf, B, 0, dev.ck, dev.ck_offsets,
                                dev.kv_offsets, dev.kv_lens, B, dev.max_len, idx, None, ws_s)
        tbs.infv2_sparse_attn_decode(dev.cfg, qbuf, dev.k, dev.v, dev.kv_offsets, dev.kv_lens, B,
                                     dev.max_len, idx, out, ws_a)

    eager = []
    for r in range(3):
        qbuf.copy_(qs[r])
        step()
        torch.cuda.synchronize()
        eager.append((idx.clone(), out.clone()))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            step()
    torch.cuda.current_stream().wait_stream(side)
    for rep in range(6):
        r = rep % 3
        qbuf.copy_(qs[r])
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(idx, eager[r][0]), f"replay {rep}: selection differs"
        assert torch.equal(out, eager[r][1]), f"replay {rep}: output differs"
        step()                     # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(out, eager[r][1])
