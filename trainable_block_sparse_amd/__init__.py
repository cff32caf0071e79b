"""Python binding of libinfv2, the InfLLM v2 sparse-attention hot path for MI355X.

The functions below carry the names of the C entry points declared in
include/infv2.h and only marshal arguments: torch tensors become device
pointers, the current torch stream becomes the hipStream_t.  Every step of the
computation runs in the library's HIP kernels; there is no Python or CPU
fallback.  If the library is missing or cannot be loaded, importing works but
every call raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libinfv2.so")

INFV2_FP32, INFV2_BF16 = 0, 1
INFV2_MODE_DECODE, INFV2_MODE_PREFILL = 0, 1
(OP_COMPRESS, OP_SELECT_DECODE, OP_SELECT_PREFILL, OP_ATTN_DECODE, OP_ATTN_PREFILL,
 OP_ATTN_PREFILL_BWD, OP_SELECT_COARSE_DECODE, OP_SELECT_COARSE_PREFILL, OP_DECODE_STEP) = range(9)
# kernel families for infv2_timing_start (infv2_kernel in infv2.h)
KERNELS = ("compress", "select_logits", "select_scores", "select_prefill", "select_topk",
           "attn_decode", "attn_merge", "attn_prefill", "vt_build", "append", "bwd_row",
           "bwd_index", "bwd_col")
KERNEL_ID = {name: i for i, name in enumerate(KERNELS)}
STATUS = {0: "INFV2_OK", 1: "INFV2_ERR_NULL", 2: "INFV2_ERR_SHAPE", 3: "INFV2_ERR_UNSUPPORTED",
          4: "INFV2_ERR_WORKSPACE", 5: "INFV2_ERR_DEVICE", 6: "INFV2_ERR_SCRATCH"}
NOALLOC_SCRATCH_BYTES = 32 << 20      # INFV2_NOALLOC_SCRATCH_BYTES


class Infv2Error(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)}")


class _CConfig(ctypes.Structure):
    _fields_ = [("head_dim", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("kernel_size", ctypes.c_int32), ("kernel_stride", ctypes.c_int32),
                ("topk", ctypes.c_int32), ("init_blocks", ctypes.c_int32),
                ("local_blocks", ctypes.c_int32), ("io_dtype", ctypes.c_int32),
                ("ck_dtype", ctypes.c_int32), ("score_scale", ctypes.c_float),
                ("attn_scale", ctypes.c_float)]


@dataclass(frozen=True)
class Config:
    """Method hyper-parameters; mirrors ``infv2_config``."""
    head_dim: int = 128
    num_q_heads: int = 32
    num_kv_heads: int = 2
    block_size: int = 64
    kernel_size: int = 32
    kernel_stride: int = 16
    topk: int = 64
    init_blocks: int = 1
    local_blocks: int = 4
    io_dtype: str = "bf16"
    ck_dtype: str = "fp32"
    score_scale: float = 1.0
    attn_scale: Optional[float] = None     # None: the library's default (0 in the C struct)

    def to_c(self) -> _CConfig:
        dt = {"fp32": INFV2_FP32, "bf16": INFV2_BF16}
        scale = 0.0 if self.attn_scale is None else self.attn_scale
        return _CConfig(self.head_dim, self.num_q_heads, self.num_kv_heads, self.block_size,
                        self.kernel_size, self.kernel_stride, self.topk, self.init_blocks,
                        self.local_blocks, dt[self.io_dtype], dt[self.ck_dtype],
                        float(self.score_scale), float(scale))


_lib = None
_load_error: Optional[str] = None


def load_library(path: str = LIB_PATH):
    """Load libinfv2.so (built by trainable_block_sparse_amd.build); raises if absent."""
    global _lib, _load_error
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        _load_error = f"{path} not found: build it with `python -m trainable_block_sparse_amd.build`"
        raise RuntimeError(_load_error)
    lib = ctypes.CDLL(path)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    cfgp = ctypes.POINTER(_CConfig)
    sig = {
        "infv2_compress_keys": (i32, [cfgp, vp, vp, vp, vp, vp, i32, i64, i64, vp, vp]),
        "infv2_append_kv": (i32, [cfgp, vp, vp, vp, vp, vp, vp, vp, vp, i32, vp]),
        "infv2_select_blocks_varlen": (i32, [cfgp, vp, i32, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
        "infv2_sparse_attn_prefill_varlen": (i32, [cfgp, vp, i32, vp, vp, vp, vp, vp, vp, vp, vp, sz,
                                                   vp]),
        "infv2_select_blocks": (i32, [cfgp, i32, vp, i32, i64, vp, vp, vp, vp, i32, i64, vp, vp,
                                      vp, sz, vp]),
        "infv2_select_blocks_coarse": (i32, [cfgp, i32, i32, vp, i32, i64, vp, vp, vp, vp, vp, vp,
                                             i32, i64, vp, vp, vp, sz, vp]),
        "infv2_sparse_attn_decode": (i32, [cfgp, vp, vp, vp, vp, vp, i32, i64, vp, vp, vp, sz, vp]),
        "infv2_sparse_attn_decode_noalloc": (i32, [cfgp, vp, vp, vp, vp, vp, i32, i64, vp, vp, vp]),
        "infv2_decode_step": (i32, [cfgp, vp, vp, vp, vp, vp, vp, vp, i32, i64, vp, vp, vp, sz, vp]),
        "infv2_decode_step_append": (i32, [cfgp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i64, vp, vp,
                                           vp, sz, vp]),
        "infv2_sparse_attn_prefill": (i32, [cfgp, vp, i32, i64, vp, vp, vp, vp, vp, vp, sz, vp]),
        "infv2_sparse_attn_prefill_bwd": (i32, [cfgp, vp, i32, i64, vp, vp, vp, vp, vp, vp, vp, vp,
                                                vp, vp, sz, vp]),
        "infv2_workspace_bytes": (i32, [cfgp, i32, i32, i32, i64, ctypes.POINTER(sz)]),
        "infv2_num_kernels": (i64, [cfgp, i64]),
        "infv2_status_str": (ctypes.c_char_p, [i32]),
        "infv2_abi_version": (i32, []),
        "infv2_timing_start": (i32, [i32]),
        "infv2_timing_stop": (i32, [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(i32)]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype, fn.argtypes = res, args
    _lib = lib
    return lib


EXPORTED = ("infv2_compress_keys", "infv2_append_kv", "infv2_select_blocks",
            "infv2_select_blocks_coarse", "infv2_sparse_attn_decode", "infv2_sparse_attn_decode_noalloc", "infv2_decode_step",
            "infv2_decode_step_append", "infv2_sparse_attn_prefill", "infv2_select_blocks_varlen",
            "infv2_sparse_attn_prefill_varlen", "infv2_sparse_attn_prefill_bwd", "infv2_workspace_bytes", "infv2_num_kernels",
            "infv2_status_str", "infv2_abi_version", "infv2_timing_start", "infv2_timing_stop")


# ---------------------------------------------------------------- marshalling helpers
def _ptr(t) -> Optional[int]:
    """Device pointer of a contiguous CUDA tensor (None passes NULL; ints pass through)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("tensor arguments must live in GPU memory")
    if not t.is_contiguous():
        raise ValueError("tensor arguments must be contiguous")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _nbytes(t) -> int:
    return 0 if t is None else t.numel() * t.element_size()


def _check(st: int, where: str) -> None:
    if st != 0:
        raise Infv2Error(st, where)


# ---------------------------------------------------------------- entry points
def infv2_abi_version() -> int:
    return load_library().infv2_abi_version()


def infv2_status_str(status: int) -> str:
    return load_library().infv2_status_str(status).decode()


def infv2_timing_start(kernel) -> None:
    """Open a timing session for one kernel family (name from KERNELS or its id)."""
    kid = KERNEL_ID[kernel] if isinstance(kernel, str) else int(kernel)
    _check(load_library().infv2_timing_start(kid), "infv2_timing_start")


def infv2_timing_stop():
    """Close the session: (summed milliseconds, number of bracketed launches)."""
    ms, n = ctypes.c_double(0.0), ctypes.c_int32(0)
    _check(load_library().infv2_timing_stop(ctypes.byref(ms), ctypes.byref(n)), "infv2_timing_stop")
    return ms.value, n.value


def infv2_num_kernels(cfg: Config, n: int) -> int:
    c = cfg.to_c()
    return load_library().infv2_num_kernels(ctypes.byref(c), n)


def infv2_workspace_bytes(cfg: Config, op: int, rows: int, batch: int, max_len: int) -> int:
    c = cfg.to_c()
    out = ctypes.c_size_t(0)
    _check(load_library().infv2_workspace_bytes(ctypes.byref(c), op, rows, batch, max_len,
                                                ctypes.byref(out)), "infv2_workspace_bytes")
    return out.value


def infv2_compress_keys(cfg: Config, k, kv_offsets, kv_lens, ck_offsets, ck_begin, batch: int,
                        max_len: int, max_new: int, ck, stream=None) -> None:
    c = cfg.to_c()
    _check(load_library().infv2_compress_keys(
        ctypes.byref(c), _ptr(k), _ptr(kv_offsets), _ptr(kv_lens), _ptr(ck_offsets),
        _ptr(ck_begin), batch, max_len, max_new, _ptr(ck), _stream(stream)), "infv2_compress_keys")


def _host_arrays(rows_per_seq, q_start_per_seq):
    """Host int32 / int64 arrays (kept alive by the caller's frame)."""
    import numpy as np
    r = np.ascontiguousarray(rows_per_seq, dtype=np.int32)
    s = np.ascontiguousarray(q_start_per_seq, dtype=np.int64)
    if r.shape != s.shape or r.ndim != 1:
        raise ValueError("rows_per_seq and q_start_per_seq must be 1-D of the same length")
    return r, s


def infv2_select_blocks_varlen(cfg: Config, q, rows_per_seq, q_start_per_seq, ck, ck_offsets,
                               kv_offsets, block_idx, block_score, ws, stream=None) -> None:
    c = cfg.to_c()
    r, s = _host_arrays(rows_per_seq, q_start_per_seq)
    _check(load_library().infv2_select_blocks_varlen(
        ctypes.byref(c), _ptr(q), int(r.shape[0]), r.ctypes.data, s.ctypes.data, _ptr(ck),
        _ptr(ck_offsets), _ptr(kv_offsets), _ptr(block_idx), _ptr(block_score), _ptr(ws),
        _nbytes(ws), _stream(stream)), "infv2_select_blocks_varlen")


def infv2_sparse_attn_prefill_varlen(cfg: Config, q, rows_per_seq, q_start_per_seq, k, v,
                                     kv_offsets, block_idx, out, ws, stream=None) -> None:
    c = cfg.to_c()
    r, s = _host_arrays(rows_per_seq, q_start_per_seq)
    _check(load_library().infv2_sparse_attn_prefill_varlen(
        ctypes.byref(c), _ptr(q), int(r.shape[0]), r.ctypes.data, s.ctypes.data, _ptr(k), _ptr(v),
        _ptr(kv_offsets), _ptr(block_idx), _ptr(out), _ptr(ws), _nbytes(ws), _stream(stream)),
        "infv2_sparse_attn_prefill_varlen")


def infv2_append_kv(cfg: Config, k_new, v_new, k, v, kv_offsets, kv_lens, ck_offsets, ck,
                    batch: int, stream=None) -> None:
    c = cfg.to_c()
    _check(load_library().infv2_append_kv(ctypes.byref(c), _ptr(k_new), _ptr(v_new), _ptr(k), _ptr(v),
                                          _ptr(kv_offsets), _ptr(kv_lens), _ptr(ck_offsets), _ptr(ck),
                                          batch, _stream(stream)), "infv2_append_kv")


def infv2_select_blocks(cfg: Config, mode: int, q, rows: int, q_start: int, ck, ck_offsets,
                        kv_offsets, kv_lens, batch: int, max_len: int, block_idx, block_score,
                        ws, stream=None) -> None:
    c = cfg.to_c()
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(load_library().infv2_select_blocks(
        ctypes.byref(c), mode, _ptr(q), rows, q_start, _ptr(ck), _ptr(ck_offsets),
        _ptr(kv_offsets), _ptr(kv_lens), batch, max_len, _ptr(block_idx), _ptr(block_score),
        _ptr(ws), nbytes, _stream(stream)), "infv2_select_blocks")


def infv2_select_blocks_coarse(cfg: Config, coarse: int, mode: int, q, rows: int, q_start: int, ck,
                               ck_offsets, ck_coarse, ckc_offsets, kv_offsets, kv_lens, batch: int,
                               max_len: int, block_idx, block_score, ws, stream=None) -> None:
    c = cfg.to_c()
    _check(load_library().infv2_select_blocks_coarse(
        ctypes.byref(c), coarse, mode, _ptr(q), rows, q_start, _ptr(ck), _ptr(ck_offsets),
        _ptr(ck_coarse), _ptr(ckc_offsets), _ptr(kv_offsets), _ptr(kv_lens), batch, max_len,
        _ptr(block_idx), _ptr(block_score), _ptr(ws), _nbytes(ws), _stream(stream)),
        "infv2_select_blocks_coarse")


def infv2_sparse_attn_decode(cfg: Config, q, k, v, kv_offsets, kv_lens, batch: int, max_len: int,
                             block_idx, out, ws, stream=None) -> None:
    c = cfg.to_c()
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(load_library().infv2_sparse_attn_decode(
        ctypes.byref(c), _ptr(q), _ptr(k), _ptr(v), _ptr(kv_offsets), _ptr(kv_lens), batch,
        max_len, _ptr(block_idx), _ptr(out), _ptr(ws), nbytes, _stream(stream)),
        "infv2_sparse_attn_decode")


def infv2_decode_step(cfg: Config, q, k, v, kv_offsets, kv_lens, ck_offsets, ck, batch: int,
                      max_len: int, block_idx, out, ws, stream=None) -> None:
    c = cfg.to_c()
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(load_library().infv2_decode_step(
        ctypes.byref(c), _ptr(q), _ptr(k), _ptr(v), _ptr(kv_offsets), _ptr(kv_lens), _ptr(ck_offsets),
        _ptr(ck), batch, max_len, _ptr(block_idx), _ptr(out), _ptr(ws), nbytes, _stream(stream)),
        "infv2_decode_step")


def infv2_decode_step_append(cfg: Config, q, k_new, v_new, k, v, kv_offsets, kv_lens, ck_offsets, ck,
                             batch: int, max_len: int, block_idx, out, ws, stream=None) -> None:
    c = cfg.to_c()
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(load_library().infv2_decode_step_append(
        ctypes.byref(c), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k), _ptr(v), _ptr(kv_offsets),
        _ptr(kv_lens), _ptr(ck_offsets), _ptr(ck), batch, max_len, _ptr(block_idx), _ptr(out), _ptr(ws),
        nbytes, _stream(stream)), "infv2_decode_step_append")


def infv2_sparse_attn_decode_noalloc(cfg: Config, q, k, v, kv_offsets, kv_lens, batch: int,
                                     max_len: int, block_idx, out, stream=None) -> None:
    c = cfg.to_c()
    _check(load_library().infv2_sparse_attn_decode_noalloc(
        ctypes.byref(c), _ptr(q), _ptr(k), _ptr(v), _ptr(kv_offsets), _ptr(kv_lens), batch,
        max_len, _ptr(block_idx), _ptr(out), _stream(stream)), "infv2_sparse_attn_decode_noalloc")


def infv2_sparse_attn_prefill(cfg: Config, q, rows: int, q_start: int, k, v, kv_offsets,
                              block_idx, out, ws=None, stream=None) -> None:
    c = cfg.to_c()
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(load_library().infv2_sparse_attn_prefill(
        ctypes.byref(c), _ptr(q), rows, q_start, _ptr(k), _ptr(v), _ptr(kv_offsets),
        _ptr(block_idx), _ptr(out), _ptr(ws), nbytes, _stream(stream)), "infv2_sparse_attn_prefill")


def infv2_sparse_attn_prefill_bwd(cfg: Config, q, rows: int, q_start: int, k, v, kv_offsets,
                                  block_idx, out, dout, dq, dk, dv, ws, stream=None) -> None:
    c = cfg.to_c()
    _check(load_library().infv2_sparse_attn_prefill_bwd(
        ctypes.byref(c), _ptr(q), rows, q_start, _ptr(k), _ptr(v), _ptr(kv_offsets),
        _ptr(block_idx), _ptr(out), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(ws),
        _nbytes(ws), _stream(stream)), "infv2_sparse_attn_prefill_bwd")


def workspace(cfg: Config, op: int, rows: int, batch: int, max_len: int, device="cuda"):
    """A zero-filled workspace tensor of the size the library asks for (at least 256 B)."""
    import torch
    n = max(256, infv2_workspace_bytes(cfg, op, rows, batch, max_len))
    return torch.zeros(n, dtype=torch.uint8, device=device)
