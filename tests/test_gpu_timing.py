"""GPU: the kernel-timing sessions bracket exactly the launches of one family,
on the stream they run on, and leave the results unchanged."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from synth import make_workload  # noqa: E402

pytestmark = pytest.mark.gpu


def test_timing_session_brackets_one_family():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import trainable_block_sparse_amd as tbs
    from tests import gpu_harness as h
    tbs.load_library()
    print("[gpu-test] timing session: decode B=2, lens 5000/9000", flush=True)
    wl = make_workload(mode="decode", io_dtype="bf16", lens=[5000, 9000], num_q_heads=32,
                       num_kv_heads=2, topk=16, init_blocks=1, local_blocks=4, n_planted=4, seed=31)
    dev = h.DeviceWorkload(wl)
    dev.compress()
    idx0, _ = dev.select_decode()
    out0 = dev.attn_decode(idx0)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        for fam, per_step in [("select_logits", 1), ("select_scores", 1), ("select_topk", 1), ("attn_decode", 1),
                              ("attn_merge", 1), ("attn_prefill", 0)]:
            tbs.infv2_timing_start(fam)
            for _ in range(3):
                idx, _ = dev.select_decode()
                out = dev.attn_decode(idx)
            ms, n = tbs.infv2_timing_stop()
            assert n == 3 * per_step, (fam, n)
            assert (ms > 0) == (per_step > 0), (fam, ms)
    side.synchronize()
    assert torch.equal(idx, idx0)
    assert np.array_equal(h.from_device(out, "bf16"), h.from_device(out0, "bf16"))
