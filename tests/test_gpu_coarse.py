"""GPU parity of the coarse-kernel LogSumExp selection (the pages' approximate
first pass) against the oracle's select_row_coarse, with the same acceptance
rule as the exact selection (bit-exact ids except across near-ties inside the
relative 1e-4 band; block scores within a relative 1e-4).  The coarse
compressed keys must equal the oracle's bit for bit.  Each test also prints how
often the approximate selection equals the exact one (the approximation's
agreement), which is reported, not asserted.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import infv2_ref as ref  # noqa: E402
from synth import make_config, make_workload  # noqa: E402
from tests.parity import accept_selection  # noqa: E402

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


def _h():
    from tests import gpu_harness
    return gpu_harness


def _params(wl, ck_dtype="fp32"):
    return ref.Params(head_dim=wl.head_dim, num_q_heads=wl.num_q_heads, num_kv_heads=wl.num_kv_heads,
                      block_size=wl.block_size, kernel_size=wl.kernel_size,
                      kernel_stride=wl.kernel_stride, topk=wl.topk, init_blocks=wl.init_blocks,
                      local_blocks=wl.local_blocks, score_scale=wl.score_scale,
                      attn_scale=wl.attn_scale, ck_dtype=ck_dtype)


def agreement(pairs):
    """(fraction of identical selections, fraction of the exact selection's
    blocks that the approximate one also holds) over (approx ids, exact ids) pairs."""
    if not pairs:
        return 1.0, 1.0
    same = np.mean([np.array_equal(a, e) for a, e in pairs])
    shared = sum(len(set(a[a >= 0].tolist()) & set(e[e >= 0].tolist())) for a, e in pairs)
    total = sum(int((e >= 0).sum()) for _, e in pairs)
    return float(same), shared / max(1, total)


def _check(rows, idx, score, label):
    """rows: [(RowSelection, gpu ids, gpu scores)]; returns (#exact, #band)."""
    exact = band = 0
    worst = 0.0
    for r, (rs, gi, gs) in enumerate(rows):
        v = accept_selection(gi, rs)
        assert not v.startswith("fail"), f"{label} row {r}: {v}"
        exact += v == "exact"
        band += v == "band"
        sel = gi[gi >= 0]
        want, got = rs.S[sel], gs[:sel.shape[0]]
        fin = np.isfinite(want)
        assert np.array_equal(np.isfinite(got), fin), f"{label} row {r}: -inf pattern"
        if fin.any():
            worst = max(worst, float(np.max(np.abs(got[fin] - want[fin]) / np.maximum(np.abs(want[fin]), 1e-30))))
    assert worst < 1e-4, f"{label}: block-score relative error {worst:.2e}"
    return exact, band


def _run_decode(wl, coarse, ck_dtype="fp32", label="coarse decode"):
    h = _h()
    import trainable_block_sparse_amd as tbs
    _say(f"{label}: lens={wl.lens.tolist()[:4]} B={wl.batch} io={wl.io_dtype} ck={ck_dtype} coarse={coarse}")
    dev = h.DeviceWorkload(wl, ck_dtype)
    dev.compress()
    ckc, ckc_off, ncs = h.coarse_ck(dev, coarse)
    idx_t, score_t = h.select_coarse(dev, coarse, tbs.INFV2_MODE_DECODE, dev.q, wl.batch, 0, ckc,
                                     ckc_off, dev.max_len)
    idx_e, _ = dev.select_decode()
    torch.cuda.synchronize()
    idx, score = idx_t.cpu().numpy().astype(np.int64), score_t.cpu().numpy().astype(np.float64)
    idx_e = idx_e.cpu().numpy().astype(np.int64)
    prm = _params(wl, ck_dtype)
    q = wl.q_f64()
    G = prm.group
    raw = ckc.cpu().numpy()
    vals = h.bf16_bits_to_f32(raw.view(np.uint16)).astype(np.float64) if ck_dtype == "bf16" else raw.astype(np.float64)
    rows, base = [], 0
    for b in range(wl.batch):
        K = wl.k_f64(b)
        n = K.shape[1]
        ck = ref.compress_keys(K, wl.kernel_size, wl.kernel_stride, ck_dtype)
        ckc_o = ref.compress_keys(K, coarse, coarse, ck_dtype)
        got = vals[base:base + ncs[b] * wl.num_kv_heads * wl.head_dim].reshape(wl.num_kv_heads, ncs[b], wl.head_dim)
        base += ncs[b] * wl.num_kv_heads * wl.head_dim
        assert np.array_equal(got, ckc_o), f"{label}: coarse compressed keys of sequence {b}"
        for g in range(wl.num_kv_heads):
            rs = ref.select_row_coarse(q[b, g * G:(g + 1) * G], ck[g], ckc_o[g], n - 1, prm, coarse)
            rows.append((rs, idx[b, g], score[b, g]))
    ex, bd = _check(rows, idx, score, label)
    pairs = [(idx[b, g], idx_e[b, g]) for b in range(wl.batch) for g in range(wl.num_kv_heads)]
    agree, overlap = agreement(pairs)
    _say(f"{label}: {ex} exact, {bd} in the near-tie band; same selection as the exact pass 1 "
         f"in {agree:.0%} of (sequence, KV head), {overlap:.1%} of the selected blocks shared")


def test_coarse_decode_small_ragged():
    wl = make_workload(mode="decode", io_dtype="bf16", lens=[3000, 700, 150, 4100], num_q_heads=32,
                       num_kv_heads=2, topk=8, local_blocks=2, n_planted=3, seed=70)
    _run_decode(wl, 64, label="coarse decode 64")
    _run_decode(wl, 128, ck_dtype="bf16", label="coarse decode 128 ck-bf16")


def test_coarse_decode_fp32():
    wl = make_workload(mode="decode", io_dtype="fp32", lens=[2100, 999], num_q_heads=16,
                       num_kv_heads=1, topk=6, local_blocks=2, n_planted=2, seed=71)
    _run_decode(wl, 96, label="coarse decode fp32 96")


@pytest.mark.parametrize("cfg,coarse", [(1, 128), (2, 128), (2, 256), (4, 128)])
def test_coarse_decode_configs(cfg, coarse):
    _run_decode(make_config(cfg), coarse, label=f"config {cfg} coarse {coarse}")


def _run_prefill(wl, coarse, chunk, positions=None, label="coarse prefill", ck_dtype="fp32"):
    h = _h()
    import trainable_block_sparse_amd as tbs
    L = int(wl.lens[0])
    _say(f"{label}: L={L} chunk={chunk} coarse={coarse} io={wl.io_dtype} ck={ck_dtype}")
    dev = h.DeviceWorkload(wl, ck_dtype)
    idx_e, _, _ = dev.prefill(chunk)                 # exact (also writes the fine compressed keys)
    ckc, ckc_off, _ = h.coarse_ck(dev, coarse)
    idxs, scores = [], []
    for q0 in range(0, L, chunk):
        q1 = min(L, q0 + chunk)
        i_t, s_t = h.select_coarse(dev, coarse, tbs.INFV2_MODE_PREFILL, dev.q[q0:q1], q1 - q0, q0,
                                   ckc, ckc_off, q1)
        idxs.append(i_t)
        scores.append(s_t)
    torch.cuda.synchronize()
    idx = torch.cat(idxs).cpu().numpy().astype(np.int64)
    score = torch.cat(scores).cpu().numpy().astype(np.float64)
    idx_e = idx_e.cpu().numpy().astype(np.int64)
    prm = _params(wl, ck_dtype)
    K = wl.k_f64(0)
    ck = ref.compress_keys(K, wl.kernel_size, wl.kernel_stride, ck_dtype)
    ckc_o = ref.compress_keys(K, coarse, coarse, ck_dtype)
    q = wl.q_f64()
    G = prm.group
    pos = list(range(L)) if positions is None else list(positions)
    rows = []
    for i in pos:
        for g in range(wl.num_kv_heads):
            rs = ref.select_row_coarse(q[i, g * G:(g + 1) * G], ck[g], ckc_o[g], i, prm, coarse)
            rows.append((rs, idx[i, g], score[i, g]))
    ex, bd = _check(rows, idx, score, label)
    scored = [i for i in pos if i // wl.block_size + 1 > wl.topk]
    agree, overlap = agreement([(idx[i, g], idx_e[i, g]) for i in scored
                                for g in range(wl.num_kv_heads)])
    _say(f"{label}: {ex} exact, {bd} in the near-tie band over {len(pos)} rows; same selection as "
         f"the exact pass 1 in {agree:.0%} of the scored (row, KV head), {overlap:.1%} of the "
         f"selected blocks shared")


def test_coarse_prefill_small_chunks():
    wl = make_workload(mode="prefill", io_dtype="bf16", lens=[1000], num_q_heads=32, num_kv_heads=2,
                       topk=6, local_blocks=1, n_planted=3, seed=72)
    _run_prefill(wl, 64, 300, label="coarse prefill 64")
    _run_prefill(wl, 256, 1000, label="coarse prefill 256")
    # bf16 compressed keys: both passes read the key rows as stored
    _run_prefill(wl, 128, 400, label="coarse prefill 128 ck-bf16", ck_dtype="bf16")


def test_coarse_prefill_fp32():
    wl = make_workload(mode="prefill", io_dtype="fp32", lens=[700], num_q_heads=16, num_kv_heads=1,
                       topk=5, local_blocks=2, n_planted=2, seed=73)
    _run_prefill(wl, 128, 700, label="coarse prefill fp32")


def test_coarse_prefill_config3_sampled_rows():
    wl = make_config(3)
    L = int(wl.lens[0])
    rng = np.random.default_rng(74)
    pos = sorted(set(rng.integers(0, L, 40).tolist()) | {0, 62, 63, 64, 4095, 4096, L - 1})
    _run_prefill(wl, 128, wl.chunk, positions=pos, label="config 3 coarse 128")
