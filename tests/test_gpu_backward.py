"""GPU parity of the attention backward (training through the sparse attention).

The HIP backward (through the C ABI) against the float64 oracle's
attention_backward / attend_row_grad / block_grad, on the GPU's own selection
and with the GPU forward's output as the saved activation.  Gradients are
compared with the same allclose rule as the forward outputs: (2e-2, 1e-2) for
bf16 inputs and (1e-5, 1e-5) for fp32 inputs, after scaling by the gradient's
largest magnitude when that exceeds 1 (a gradient summed over many rows grows
with their number; the fp32 accumulation error grows with it, the bound stays
relative).  Tokens past the call's last row must be left untouched (NaN canaries).
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import infv2_ref as ref  # noqa: E402
from synth import make_config, make_workload, upstream_grad  # noqa: E402
from tests.parity import TOL  # noqa: E402

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


def _params(wl):
    return ref.Params(head_dim=wl.head_dim, num_q_heads=wl.num_q_heads, num_kv_heads=wl.num_kv_heads,
                      block_size=wl.block_size, kernel_size=wl.kernel_size,
                      kernel_stride=wl.kernel_stride, topk=wl.topk, init_blocks=wl.init_blocks,
                      local_blocks=wl.local_blocks, score_scale=wl.score_scale,
                      attn_scale=wl.attn_scale)


def grad_close(gpu, want, dtype, what):
    """allclose(atol, rtol) on values scaled by max(1, max|want|); returns the scaled max error."""
    atol, rtol = TOL[dtype]
    gpu = np.asarray(gpu, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert gpu.shape == want.shape, (gpu.shape, want.shape)
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite values"
    s = max(1.0, float(np.max(np.abs(want)))) if want.size else 1.0
    err = np.abs(gpu - want) / s - (atol + rtol * np.abs(want) / s)
    worst = float(np.max(err)) if err.size else -1.0
    assert worst <= 0.0, (f"{what}: allclose violated by {worst:.3e} (max abs err "
                          f"{np.max(np.abs(gpu - want)):.3e}, scale {s:.3g})")
    return float(np.max(np.abs(gpu - want)) / s) if gpu.size else 0.0


def _small(io="bf16", L=700, topk=6, local=2, init=1, m=64, seed=0, hkv=2, **kw):
    return make_workload(mode="prefill", io_dtype=io, lens=[L], num_q_heads=16 * hkv,
                         num_kv_heads=hkv, block_size=m, topk=topk, init_blocks=init,
                         local_blocks=local, n_planted=3, seed=seed, **kw)


def _forward_and_backward(wl, chunks, label):
    """GPU forward over the whole sequence (chunked), then one backward call per
    chunk in `chunks` ([(q0, q1)]).  Returns what the checks need."""
    h = _h()
    L = int(wl.lens[0])
    dev = h.DeviceWorkload(wl)
    idx_t, _, out_t = dev.prefill(max(q1 - q0 for q0, q1 in chunks))
    dout_t = h.to_device(upstream_grad(wl))
    res = []
    for q0, q1 in chunks:
        _say(f"{label}: backward rows [{q0}, {q1}) of L={L} io={wl.io_dtype} m={wl.block_size} "
             f"k={wl.topk}")
        dq, dk, dv = dev.attn_prefill_bwd(q0, q1, idx_t[q0:q1].contiguous(), out_t[q0:q1].contiguous(),
                                          dout_t[q0:q1].contiguous())
        torch.cuda.synchronize()
        res.append((q0, q1, h.from_device(dq, wl.io_dtype), h.from_device(dk, wl.io_dtype),
                    h.from_device(dv, wl.io_dtype)))
    idx = idx_t.cpu().numpy().astype(np.int64)
    dout = wl.decoded(upstream_grad(wl))
    return dev, idx, dout, res


def _check_full(wl, chunks, label):
    dev, idx, dout, res = _forward_and_backward(wl, chunks, label)
    prm = _params(wl)
    K, V, q = wl.k_f64(0), wl.v_f64(0), wl.q_f64()
    hkv, d = wl.num_kv_heads, wl.head_dim
    L = int(wl.lens[0])
    for q0, q1, dq, dk, dv in res:
        pos = list(range(q0, q1))
        wq, wk, wv, _ = ref.attention_backward(q[q0:q1], K, V, pos, idx[q0:q1], prm, dout[q0:q1])
        dk = dk.reshape(hkv, L, d)
        dv = dv.reshape(hkv, L, d)
        assert np.all(np.isnan(dk[:, q1:])) and np.all(np.isnan(dv[:, q1:])), \
            f"{label}: tokens past the last row were written"
        e1 = grad_close(dq, wq, wl.io_dtype, f"{label} dq")
        e2 = grad_close(dk[:, :q1], wk[:, :q1], wl.io_dtype, f"{label} dk")
        e3 = grad_close(dv[:, :q1], wv[:, :q1], wl.io_dtype, f"{label} dv")
        _say(f"{label} [{q0},{q1}): scaled max err dq {e1:.1e} dk {e2:.1e} dv {e3:.1e}")
    return dev, idx


def test_backward_fp32_small_all_rows():
    wl = _small(io="fp32", L=333, topk=5, seed=41)
    _check_full(wl, [(0, 333)], "bwd fp32 small")


def test_backward_bf16_two_chunks_ragged():
    wl = _small(io="bf16", L=1000, topk=6, seed=42)
    _check_full(wl, [(0, 600), (600, 1000)], "bwd bf16 chunks")


def test_backward_config0_fp32():
    wl = make_config(0)
    _check_full(wl, [(0, int(wl.lens[0]))], "bwd config 0")


@pytest.mark.parametrize("m", [32, 128])
def test_backward_other_block_sizes(m):
    wl = _small(io="bf16", L=555, topk=5, m=m, seed=43 + m)
    _check_full(wl, [(0, 555)], f"bwd bf16 m={m}")


def test_backward_dense_rows_and_large_topk():
    # every row dense (L <= k*m) and top-k far above the block count
    wl = _small(io="bf16", L=900, topk=40, local=3, seed=44)
    _check_full(wl, [(0, 900)], "bwd bf16 dense")


def test_backward_topk128_union_at_capacity():
    # 16 rows x 128 selections: the most the row pass's row-group union takes
    wl = _small(io="bf16", L=9000, topk=128, local=4, seed=45)
    _check_full(wl, [(8832, 8992)], "bwd bf16 top-k 128")


def test_backward_rows_without_visible_tokens():
    """Rows whose selection is all padding have zero dq and add nothing to dk / dv."""
    h = _h()
    wl = _small(io="bf16", L=300, topk=4, seed=45)
    L = 300
    dev = h.DeviceWorkload(wl)
    idx_t, _, out_t = dev.prefill(L)
    blank = [0, 5, 170, 299]
    idx_t[blank] = -1
    out_t[blank] = 0
    dout_t = h.to_device(upstream_grad(wl))
    _say("bwd rows with an empty selection")
    dq, dk, dv = dev.attn_prefill_bwd(0, L, idx_t, out_t, dout_t)
    torch.cuda.synchronize()
    dq = h.from_device(dq, "bf16")
    assert np.all(dq[blank] == 0)
    prm = _params(wl)
    idx = idx_t.cpu().numpy().astype(np.int64)
    wq, wk, wv, _ = ref.attention_backward(wl.q_f64(), wl.k_f64(0), wl.v_f64(0), list(range(L)), idx,
                                           prm, wl.decoded(upstream_grad(wl)))
    grad_close(dq, wq, "bf16", "dq")
    grad_close(h.from_device(dk, "bf16").reshape(wk.shape), wk, "bf16", "dk")
    grad_close(h.from_device(dv, "bf16").reshape(wv.shape), wv, "bf16", "dv")


def test_backward_is_deterministic():
    h = _h()
    wl = _small(io="bf16", L=800, topk=6, seed=46)
    dev, idx, dout, res = _forward_and_backward(wl, [(0, 800), (0, 800)], "bwd repeat")
    for a, b in zip(res[0][2:], res[1][2:]):
        assert np.array_equal(a, b)


def test_backward_config3_full_size_sampled():
    """The 32K training-size backward in one call: dq at sampled rows, dk / dv at
    sampled blocks against the oracle, and the softmax invariants over every token."""
    wl = make_config(3)
    L = int(wl.lens[0])
    dev, idx, dout, res = _forward_and_backward(wl, [(0, L)], "bwd config 3")
    _, _, dq, dk, dv = res[0]
    prm = _params(wl)
    hkv, d, G, m = wl.num_kv_heads, wl.head_dim, prm.group, wl.block_size
    K, V, q = wl.k_f64(0), wl.v_f64(0), wl.q_f64()
    dk = dk.reshape(hkv, L, d)
    dv = dv.reshape(hkv, L, d)
    rng = np.random.default_rng(77)
    rows = sorted(set(rng.integers(0, L, 12).tolist()) | {0, 63, 64, 4095, L - 1})
    for i in rows:
        for g in range(hkv):
            hs = slice(g * G, (g + 1) * G)
            wq = ref.attend_row_grad(q[i, hs], K[g], V[g], i, idx[i, g], prm, dout[i, hs])[0]
            grad_close(dq[i, hs], wq, "bf16", f"dq row {i} head {g}")
    nblk = L // m
    for g in range(hkv):
        users = np.array([(idx[:, g] == j).any(axis=1).sum() for j in range(nblk)])
        mid = [j for j in range(nblk // 4, nblk - 8) if 64 <= users[j] <= 400][:2]
        for j in [nblk - 1, nblk - 3] + mid:
            _say(f"bwd config 3: block {j} head {g} ({users[j]} rows)")
            wk, wv = ref.block_grad(q, K, V, range(L), idx, prm, dout, g, j)
            grad_close(dk[g, j * m:(j + 1) * m], wk, "bf16", f"dk block {j}")
            grad_close(dv[g, j * m:(j + 1) * m], wv, "bf16", f"dv block {j}")
        # sum_t dV_t = sum of dO over the group's heads; sum_t dK_t = 0 (bf16-rounded sums)
        sv = dv[g].sum(axis=0)
        want = dout[:, g * G:(g + 1) * G].sum(axis=(0, 1))
        scale = np.abs(dv[g]).sum(axis=0)
        assert np.all(np.abs(sv - want) <= 1e-2 * scale + 1e-2), "sum of dv"
        assert np.all(np.abs(dk[g].sum(axis=0)) <= 1e-2 * np.abs(dk[g]).sum(axis=0) + 1e-2), "sum of dk"
