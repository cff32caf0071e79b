"""GPU: the decode attention entry point that allocates nothing
(infv2_sparse_attn_decode_noalloc, static device scratch) gives the same
outputs as infv2_sparse_attn_decode with a caller workspace, bit for bit, on
two calls in a row (the second one smaller), and both agree with the float64
oracle on the GPU's selection.  Sizes beyond the static scratch are refused
before anything is launched."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import infv2_ref as ref  # noqa: E402
from synth import make_workload  # noqa: E402
from tests.parity import assert_close  # noqa: E402

pytestmark = pytest.mark.gpu


def _case(lens, seed):
    return make_workload(mode="decode", io_dtype="bf16", lens=list(lens), num_q_heads=32,
                         num_kv_heads=2, topk=16, init_blocks=1, local_blocks=4, n_planted=3,
                         seed=seed)


def _run(wl):
    import trainable_block_sparse_amd as tbs
    from tests import gpu_harness as h
    dev = h.DeviceWorkload(wl)
    dev.compress()
    idx, _ = dev.select_decode()
    want = dev.attn_decode(idx)
    got = torch.full_like(want, 0x7FC0)            # NaN bits: every element must be written
    tbs.infv2_sparse_attn_decode_noalloc(dev.cfg, dev.q, dev.k, dev.v, dev.kv_offsets, dev.kv_lens,
                                         wl.batch, dev.max_len, idx, got)
    torch.cuda.synchronize()
    assert torch.equal(got, want), "no-allocation decode differs from the workspace entry point"
    # and both meet the oracle on the GPU's selection
    out = h.from_device(got, "bf16")
    gi = idx.cpu().numpy().astype(np.int64)
    prm = ref.Params(head_dim=128, num_q_heads=32, num_kv_heads=2, block_size=64, kernel_size=32,
                     kernel_stride=16, topk=16, init_blocks=1, local_blocks=4)
    q = wl.q_f64()
    for b in range(wl.batch):
        n = int(wl.lens[b])
        w = ref.attend_with_selection(q[b:b + 1], wl.k_f64(b), wl.v_f64(b), [n - 1], gi[b:b + 1], prm)
        assert_close(out[b], w[0], "bf16", f"no-alloc decode seq {b}")


def test_noalloc_decode_matches_workspace_path_twice():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import trainable_block_sparse_amd as tbs
    tbs.load_library()
    print("[gpu-test] no-alloc decode: lens [9000, 20000, 700], then [3000]", flush=True)
    _run(_case([9000, 20000, 700], 301))
    _run(_case([3000], 302))                       # second call, smaller input


def test_noalloc_decode_rejects_sizes_beyond_the_scratch():
    import trainable_block_sparse_amd as tbs
    tbs.load_library()
    cfg = tbs.Config()
    need = tbs.infv2_workspace_bytes(cfg, tbs.OP_ATTN_DECODE, 512, 512, 131072)
    assert need > tbs.NOALLOC_SCRATCH_BYTES
    lib = tbs.load_library()
    import ctypes
    fake = 0x10000                                  # never dereferenced: refused on the host
    st = lib.infv2_sparse_attn_decode_noalloc(ctypes.byref(cfg.to_c()), fake, fake, fake, fake, None,
                                              512, 131072, fake, fake, None)
    assert st == 6, tbs.infv2_status_str(st)
