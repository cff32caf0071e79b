"""Host-only checks of the C ABI (no GPU needed).

The library must load, export every function include/infv2.h declares, and
reject invalid arguments with the documented status before any HIP call (so
these calls are safe without a device: nothing is ever launched).
"""
import ctypes
import os
import re

import pytest

import trainable_block_sparse_amd as tbs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "infv2.h")
OK, ENULL, ESHAPE, EUNSUP, EWS = 0, 1, 2, 3, 4
FAKE = 0x10000          # a non-NULL pointer that is never dereferenced on these paths


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(tbs.LIB_PATH):
        from trainable_block_sparse_amd.build import build
        build()
    return tbs.load_library()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(infv2_\w+)\s*\(", text, re.M)))


def test_header_declares_the_four_entry_points():
    names = declared_functions()
    for n in ["infv2_compress_keys", "infv2_select_blocks", "infv2_sparse_attn_prefill",
              "infv2_sparse_attn_decode"]:
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 8
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(tbs.EXPORTED)


def test_abi_version_and_status_strings(lib):
    ver = int(re.search(r"#define INFV2_ABI_VERSION (\d+)", open(HEADER).read()).group(1))
    assert tbs.infv2_abi_version() == ver
    for st in range(7):
        assert tbs.infv2_status_str(st).startswith("INFV2_")


def test_num_kernels_formula(lib):
    cfg = tbs.Config()
    for n in [0, 1, 31, 32, 33, 47, 48, 131072]:
        want = 0 if n < 32 else (n - 32) // 16 + 1
        assert tbs.infv2_num_kernels(cfg, n) == want


def test_workspace_sizes_grow_with_the_problem(lib):
    cfg = tbs.Config()
    a = tbs.infv2_workspace_bytes(cfg, tbs.OP_SELECT_DECODE, 1, 1, 32768)
    b = tbs.infv2_workspace_bytes(cfg, tbs.OP_SELECT_DECODE, 1, 1, 131072)
    c = tbs.infv2_workspace_bytes(cfg, tbs.OP_SELECT_DECODE, 16, 16, 131072)
    assert 0 < a < b < c
    assert tbs.infv2_workspace_bytes(cfg, tbs.OP_ATTN_DECODE, 16, 16, 131072) > 0
    assert tbs.infv2_workspace_bytes(cfg, tbs.OP_SELECT_PREFILL, 4096, 1, 32768) >= 4096 * 2 * 512 * 4


@pytest.mark.parametrize("topk,hkv", [(64, 2), (8, 1), (256, 1), (1024, 4)])
def test_decode_attention_workspace_never_shrinks_with_the_batch(lib, topk, hkv):
    # the split of the selected blocks (one or four per thread block) depends on
    # the batch; a workspace sized for a batch must still serve every smaller one
    cfg = tbs.Config(num_q_heads=16 * hkv, num_kv_heads=hkv, topk=topk, local_blocks=2)
    sizes = [tbs.infv2_workspace_bytes(cfg, tbs.OP_ATTN_DECODE, b, b, 131072) for b in range(1, 65)]
    assert all(x <= y for x, y in zip(sizes, sizes[1:])), sizes
    # room for one partial (16 heads x d fp32 + the (max, sum) pairs) per split
    per_split = 16 * 128 * 4
    assert sizes[0] >= hkv * min(topk, 256 if topk <= 256 else (topk + 3) // 4) * per_split


def _c(cfg):
    return ctypes.byref(cfg.to_c())


def _compress(lib, cfg, k=FAKE, off=FAKE, ckoff=FAKE, ck=FAKE, batch=1, max_len=100):
    return lib.infv2_compress_keys(_c(cfg) if cfg is not None else None, k, off, None, ckoff, None,
                                   batch, max_len, -1, ck, None)


@pytest.mark.parametrize("cfg,want", [
    (tbs.Config(num_q_heads=30, num_kv_heads=4), ESHAPE),          # Hq % Hkv
    (tbs.Config(topk=4, init_blocks=1, local_blocks=4), ESHAPE),   # k < |F|
    (tbs.Config(kernel_size=8, kernel_stride=16), ESHAPE),         # p < s
    (tbs.Config(block_size=0), ESHAPE),
    (tbs.Config(head_dim=64), EUNSUP),
    (tbs.Config(num_q_heads=16, num_kv_heads=2), EUNSUP),          # group of 8
    (tbs.Config(block_size=48 + 1), EUNSUP),
    (tbs.Config(topk=2048), EUNSUP),
    (tbs.Config(kernel_size=512, kernel_stride=16), EUNSUP),
    (tbs.Config(attn_scale=-0.5), ESHAPE),                         # negative scales
    (tbs.Config(score_scale=-1.0), ESHAPE),
    (tbs.Config(attn_scale=float("inf")), ESHAPE),
    (tbs.Config(score_scale=float("nan")), ESHAPE),
])
def test_invalid_configs_rejected(lib, cfg, want):
    assert _compress(lib, cfg) == want


def test_zero_scales_select_the_defaults(lib):
    # 0 in the C struct means the default (score 1.0, attention 1/sqrt(d)); the
    # binding passes 0 when no attention scale is given and computes none itself
    assert tbs.Config().to_c().attn_scale == 0.0
    assert tbs.Config(attn_scale=0.25).to_c().attn_scale == 0.25
    # accepted by the validation (a workspace query launches nothing)
    for cfg in (tbs.Config(), tbs.Config(score_scale=0.0), tbs.Config(attn_scale=0.0, score_scale=0.0)):
        assert tbs.infv2_workspace_bytes(cfg, tbs.OP_SELECT_DECODE, 1, 1, 1000) > 0
    with pytest.raises(tbs.Infv2Error):
        tbs.infv2_workspace_bytes(tbs.Config(attn_scale=-1.0), tbs.OP_SELECT_DECODE, 1, 1, 1000)


def test_null_pointers_and_sizes_rejected(lib):
    cfg = tbs.Config()
    assert _compress(lib, None) == ENULL
    assert _compress(lib, cfg, k=None) == ENULL
    assert _compress(lib, cfg, ck=None) == ENULL
    assert _compress(lib, cfg, batch=0) == ESHAPE
    assert _compress(lib, cfg, max_len=-1) == ESHAPE
    assert _compress(lib, cfg, max_len=16385 * 64) == EUNSUP      # more than 16384 blocks


def test_select_and_attention_validation(lib):
    cfg = tbs.Config()
    c = _c(cfg)
    ws_need = tbs.infv2_workspace_bytes(cfg, tbs.OP_SELECT_DECODE, 2, 2, 5000)
    # decode: rows must equal batch; workspace must be large enough
    assert lib.infv2_select_blocks(c, 0, FAKE, 3, 0, FAKE, FAKE, FAKE, None, 2, 5000, FAKE, None,
                                   FAKE, ws_need, None) == ESHAPE
    assert lib.infv2_select_blocks(c, 0, FAKE, 2, 0, FAKE, FAKE, FAKE, None, 2, 5000, FAKE, None,
                                   FAKE, ws_need - 1, None) == EWS
    assert lib.infv2_select_blocks(c, 0, FAKE, 2, 0, FAKE, FAKE, FAKE, None, 2, 5000, FAKE, None,
                                   None, ws_need, None) == EWS
    assert lib.infv2_select_blocks(c, 0, FAKE, 2, 0, FAKE, FAKE, None, None, 2, 5000, FAKE, None,
                                   FAKE, ws_need, None) == ENULL
    # prefill: one sequence, rows inside max_len, known mode
    assert lib.infv2_select_blocks(c, 1, FAKE, 10, 0, FAKE, FAKE, FAKE, None, 2, 5000, FAKE, None,
                                   FAKE, 1 << 30, None) == ESHAPE
    assert lib.infv2_select_blocks(c, 1, FAKE, 10, 4995, FAKE, FAKE, FAKE, None, 1, 5000, FAKE,
                                   None, FAKE, 1 << 30, None) == ESHAPE
    assert lib.infv2_select_blocks(c, 7, FAKE, 10, 0, FAKE, FAKE, FAKE, None, 1, 5000, FAKE, None,
                                   FAKE, 1 << 30, None) == ESHAPE
    assert lib.infv2_select_blocks(c, 1, FAKE, 0, 0, FAKE, FAKE, FAKE, None, 1, 5000, FAKE, None,
                                   FAKE, 1 << 30, None) == OK       # empty chunk: nothing to do
    need_a = tbs.infv2_workspace_bytes(cfg, tbs.OP_ATTN_DECODE, 2, 2, 5000)
    assert lib.infv2_sparse_attn_decode(c, FAKE, FAKE, FAKE, FAKE, None, 2, 5000, FAKE, FAKE, FAKE,
                                        need_a - 1, None) == EWS
    assert lib.infv2_sparse_attn_decode(c, FAKE, None, FAKE, FAKE, None, 2, 5000, FAKE, FAKE, FAKE,
                                        need_a, None) == ENULL
    assert lib.infv2_sparse_attn_prefill(c, FAKE, -1, 0, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0,
                                         None) == ESHAPE
    assert lib.infv2_sparse_attn_prefill(c, FAKE, 0, 0, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0,
                                         None) == OK


def test_timing_session_state_machine(lib):
    # no GPU work: only the session bookkeeping, which never touches a device
    with pytest.raises(tbs.Infv2Error):
        tbs.infv2_timing_stop()                        # nothing open
    with pytest.raises(tbs.Infv2Error):
        tbs.infv2_timing_start(len(tbs.KERNELS))       # unknown family
    tbs.infv2_timing_start("attn_decode")
    with pytest.raises(tbs.Infv2Error):
        tbs.infv2_timing_start("compress")             # one session at a time
    assert tbs.infv2_timing_stop() == (0.0, 0)
    hdr = open(HEADER).read()
    assert int(re.search(r"INFV2_KERNEL_COUNT = (\d+)", hdr).group(1)) == len(tbs.KERNELS)


def test_varlen_prefill_and_append_validation(lib):
    import numpy as np
    cfg = tbs.Config()
    c = _c(cfg)
    rows = np.array([100, 0, 300], dtype=np.int32)
    starts = np.array([0, 50, 1000], dtype=np.int64)
    R, S = rows.ctypes.data, starts.ctypes.data
    need = max(tbs.infv2_workspace_bytes(cfg, tbs.OP_SELECT_PREFILL, int(r), 1, int(s + r))
               for r, s in zip(rows, starts) if r > 0)
    sel = lib.infv2_select_blocks_varlen
    assert sel(c, FAKE, 3, None, S, FAKE, FAKE, FAKE, FAKE, None, FAKE, need, None) == ENULL
    assert sel(c, FAKE, 0, R, S, FAKE, FAKE, FAKE, FAKE, None, FAKE, need, None) == ESHAPE
    assert sel(c, FAKE, 3, R, S, FAKE, FAKE, FAKE, FAKE, None, FAKE, need - 1, None) == EWS
    bad = np.array([100, -1, 300], dtype=np.int32)
    assert sel(c, FAKE, 3, bad.ctypes.data, S, FAKE, FAKE, FAKE, FAKE, None, FAKE, need, None) == ESHAPE
    far = np.array([0, 0, 16385 * 64], dtype=np.int64)
    assert sel(c, FAKE, 3, R, far.ctypes.data, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 40,
               None) == EUNSUP
    zero = np.zeros(3, dtype=np.int32)
    assert sel(c, FAKE, 3, zero.ctypes.data, S, FAKE, FAKE, FAKE, FAKE, None, None, 0, None) == OK
    att = lib.infv2_sparse_attn_prefill_varlen
    need_a = max(tbs.infv2_workspace_bytes(cfg, tbs.OP_ATTN_PREFILL, int(r), 1, int(s + r))
                 for r, s in zip(rows, starts) if r > 0)
    assert need_a == 0                  # the prefill attention needs no workspace
    assert att(c, FAKE, 3, R, S, None, FAKE, FAKE, FAKE, FAKE, FAKE, need_a, None) == ENULL
    app = lib.infv2_append_kv
    assert app(c, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, 2, None) == ENULL
    assert app(c, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, None) == ESHAPE


def test_backward_validation(lib):
    cfg = tbs.Config()
    c = _c(cfg)
    bwd = lib.infv2_sparse_attn_prefill_bwd
    rows, q0 = 1000, 3000
    need = tbs.infv2_workspace_bytes(cfg, tbs.OP_ATTN_PREFILL_BWD, rows, 1, q0 + rows)
    assert need > 0
    # grows with the rows and with the prefix (more blocks per KV head)
    assert tbs.infv2_workspace_bytes(cfg, tbs.OP_ATTN_PREFILL_BWD, 2 * rows, 1, q0 + 2 * rows) > need
    ptrs = [FAKE] * 10          # q k v kv_offsets block_idx out dout dq dk dv
    def call(p=ptrs, r=rows, s=q0, ws=FAKE, nb=need):
        qq, k, v, off, idx, out, dout, dq, dk, dv = p
        return bwd(c, qq, r, s, k, v, off, idx, out, dout, dq, dk, dv, ws, nb, None)
    for x in range(10):
        p = list(ptrs)
        p[x] = None
        assert call(p) == ENULL, x
    assert call(r=-1) == ESHAPE
    assert call(s=-5) == ESHAPE
    assert call(nb=need - 1) == EWS
    assert call(ws=None) == EWS
    assert call(r=0, ws=None, nb=0) == OK          # nothing to do, nothing launched
    assert call(r=1 << 21, s=0) == EUNSUP          # rows * topk above 2^30
    assert call(s=16384 * 64) == EUNSUP            # more blocks than supported


def test_coarse_selection_validation(lib):
    cfg = tbs.Config()            # p = 32, k = 64, m = 64
    c = _c(cfg)
    sel = lib.infv2_select_blocks_coarse
    need = tbs.infv2_workspace_bytes(cfg, tbs.OP_SELECT_COARSE_DECODE, 1, 1, 131072)
    assert need >= tbs.infv2_workspace_bytes(cfg, tbs.OP_SELECT_DECODE, 1, 1, 131072)
    def call(coarse=128, ckc=FAKE, ws=FAKE, nb=need, mode=0):
        return sel(c, coarse, mode, FAKE, 1, 0, FAKE, FAKE, ckc, FAKE, FAKE, None, 1, 131072,
                   FAKE, None, ws, nb, None)
    assert call(ckc=None) == ENULL
    assert call(coarse=16) == ESHAPE              # finer than the kernels
    assert call(coarse=257) == ESHAPE             # beyond the largest compressed kernel
    small = tbs.Config(topk=3, local_blocks=2)    # k * m = 192
    assert sel(_c(small), 193, 0, FAKE, 1, 0, FAKE, FAKE, FAKE, FAKE, FAKE, None, 1, 4096, FAKE,
               None, FAKE, 1 << 30, None) == ESHAPE  # a scored row might see no coarse kernel
    assert call(nb=need - 1) == EWS
    assert call(mode=7) == ESHAPE
