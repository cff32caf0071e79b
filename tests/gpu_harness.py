"""Device-side plumbing for the GPU parity tests and the bench.

Uploads a synthetic workload with torch (memory only) and drives the HIP path
through the Python binding of the C ABI.  bf16 tensors travel as their 16-bit
patterns (torch.int16), so no torch bf16 arithmetic is involved anywhere.
"""
from __future__ import annotations

from typing import List, Optional, Sequence

import numpy as np
import torch

import trainable_block_sparse_amd as tbs
from synth import Workload, bf16_bits_to_f32


def cfg_of(wl: Workload, ck_dtype: str = "fp32", **over) -> tbs.Config:
    kw = dict(head_dim=wl.head_dim, num_q_heads=wl.num_q_heads, num_kv_heads=wl.num_kv_heads,
              block_size=wl.block_size, kernel_size=wl.kernel_size,
              kernel_stride=wl.kernel_stride, topk=wl.topk, init_blocks=wl.init_blocks,
              local_blocks=wl.local_blocks, io_dtype=wl.io_dtype, ck_dtype=ck_dtype,
              score_scale=wl.score_scale, attn_scale=wl.attn_scale)
    kw.update(over)
    return tbs.Config(**kw)


def num_kernels(n: int, p: int, s: int) -> int:
    return 0 if n < p else (n - p) // s + 1


def to_device(arr: np.ndarray, device="cuda") -> torch.Tensor:
    if arr.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).to(device)
    return torch.from_numpy(np.ascontiguousarray(arr)).to(device)


def from_device(t: torch.Tensor, io_dtype: str) -> np.ndarray:
    a = t.detach().cpu().numpy()
    if io_dtype == "bf16":
        return bf16_bits_to_f32(a.view(np.uint16)).astype(np.float64)
    return a.astype(np.float64)


CANARY_PAD = 4096                   # elements guarded before and after each output buffer
_CANARY = {torch.int32: 0x5A5A5A5A, torch.float32: 0x7FA5A5A5, torch.int16: 0x7FA5}


def _canary_fill(t: torch.Tensor) -> None:
    if t.dtype == torch.float32:
        t.view(torch.int32).fill_(_CANARY[torch.float32])
    else:
        t.fill_(_CANARY[t.dtype])


def _canary_ok(t: torch.Tensor) -> bool:
    if t.dtype == torch.float32:
        t = t.view(torch.int32)
        return bool((t == _CANARY[torch.float32]).all())
    return bool((t == _CANARY[t.dtype]).all())


class DeviceWorkload:
    """A workload resident in GPU memory plus the calls of the hot path.  Every
    output buffer the calls write (compressed keys, block ids and scores,
    attention outputs) sits between two guard regions of CANARY_PAD elements
    holding a fixed pattern; check_canaries() asserts that no call wrote there."""

    def __init__(self, wl: Workload, ck_dtype: str = "fp32", device: str = "cuda", **cfg_over):
        self.wl = wl
        self.device = device
        self.cfg = cfg_of(wl, ck_dtype, **cfg_over)
        self.ck_dtype = ck_dtype
        self.k = to_device(wl.k, device)
        self.v = to_device(wl.v, device)
        self.q = to_device(wl.q, device)
        self.kv_offsets = torch.tensor(wl.kv_offsets, dtype=torch.int64, device=device)
        self.kv_lens = torch.tensor(wl.lens, dtype=torch.int64, device=device)
        self.max_len = int(wl.lens.max())
        ncs = [num_kernels(int(n), wl.kernel_size, wl.kernel_stride) for n in wl.lens]
        self.nc = ncs
        off = np.zeros(len(ncs) + 1, dtype=np.int64)
        off[1:] = np.cumsum(ncs)
        self.ck_offsets = torch.tensor(off, dtype=torch.int64, device=device)
        total = int(off[-1]) * wl.num_kv_heads * wl.head_dim
        tdt = torch.int16 if ck_dtype == "bf16" else torch.float32
        self._canaries = []
        self.ck = self.guarded((max(total, 1),), tdt)
        self.ck.zero_()
        self._ws = {}

    # ---------------------------------------------------------------- guarded outputs
    def guarded(self, shape, dtype) -> torch.Tensor:
        """An output tensor of `shape` inside a canary-filled buffer."""
        n = int(np.prod(shape))
        full = torch.empty(n + 2 * CANARY_PAD, dtype=dtype, device=self.device)
        _canary_fill(full)
        self._canaries.append((full, n))
        return full[CANARY_PAD:CANARY_PAD + n].view(tuple(shape))

    def check_canaries(self) -> int:
        """Assert every guard region is untouched; returns how many were checked."""
        torch.cuda.synchronize()
        for full, n in self._canaries:
            assert _canary_ok(full[:CANARY_PAD]), "a call wrote before its output buffer"
            assert _canary_ok(full[CANARY_PAD + n:]), "a call wrote past its output buffer"
        return len(self._canaries)

    # ---------------------------------------------------------------- workspaces
    def ws(self, op: int, rows: int, batch: int, max_len: int) -> torch.Tensor:
        need = max(256, tbs.infv2_workspace_bytes(self.cfg, op, rows, batch, max_len))
        key = op
        t = self._ws.get(key)
        if t is None or t.numel() < need:
            t = torch.zeros(need, dtype=torch.uint8, device=self.device)
            self._ws[key] = t
        return t

    # ---------------------------------------------------------------- step 1a
    def compress(self, kv_lens: Optional[torch.Tensor] = None, ck_begin: Optional[torch.Tensor] = None,
                 max_len: Optional[int] = None, max_new: int = -1) -> None:
        tbs.infv2_compress_keys(self.cfg, self.k, self.kv_offsets,
                                self.kv_lens if kv_lens is None else kv_lens, self.ck_offsets,
                                ck_begin, self.wl.batch, self.max_len if max_len is None else max_len,
                                max_new, self.ck)

    def ck_host(self) -> List[np.ndarray]:
        """Compressed keys per sequence as float64 [Hkv][n_c][d]."""
        raw = self.ck.detach().cpu().numpy()
        if self.ck_dtype == "bf16":
            vals = bf16_bits_to_f32(raw.view(np.uint16)).astype(np.float64)
        else:
            vals = raw.astype(np.float64)
        out, base = [], 0
        hkv, d = self.wl.num_kv_heads, self.wl.head_dim
        for nc in self.nc:
            out.append(vals[base:base + nc * hkv * d].reshape(hkv, nc, d))
            base += nc * hkv * d
        return out

    # ---------------------------------------------------------------- decode
    def select_decode(self, q: Optional[torch.Tensor] = None):
        B, hkv, k = self.wl.batch, self.wl.num_kv_heads, self.cfg.topk
        idx = self.guarded((B, hkv, k), torch.int32)
        score = self.guarded((B, hkv, k), torch.float32)
        ws = self.ws(tbs.OP_SELECT_DECODE, B, B, self.max_len)
        tbs.infv2_select_blocks(self.cfg, tbs.INFV2_MODE_DECODE, self.q if q is None else q, B, 0,
                                self.ck, self.ck_offsets, self.kv_offsets, self.kv_lens, B,
                                self.max_len, idx, score, ws)
        return idx, score

    def attn_decode(self, idx: torch.Tensor, q: Optional[torch.Tensor] = None) -> torch.Tensor:
        B = self.wl.batch
        qq = self.q if q is None else q
        out = self.guarded(tuple(qq.shape), qq.dtype)
        ws = self.ws(tbs.OP_ATTN_DECODE, B, B, self.max_len)
        tbs.infv2_sparse_attn_decode(self.cfg, self.q if q is None else q, self.k, self.v,
                                     self.kv_offsets, self.kv_lens, B, self.max_len, idx, out, ws)
        return out

    # ---------------------------------------------------------------- prefill
    def prefill_chunk(self, q0: int, q1: int):
        """Compress the kernels completed by rows [q0, q1), then select and attend them."""
        wl = self.wl
        p, s = wl.kernel_size, wl.kernel_stride
        lens = torch.tensor([q1], dtype=torch.int64, device=self.device)
        begin = torch.tensor([num_kernels(q0, p, s)], dtype=torch.int64, device=self.device)
        new = num_kernels(q1, p, s) - num_kernels(q0, p, s)
        self.compress(kv_lens=lens, ck_begin=begin, max_len=q1, max_new=new)
        rows = q1 - q0
        hkv, k = wl.num_kv_heads, self.cfg.topk
        q = self.q[q0:q1]
        idx = self.guarded((rows, hkv, k), torch.int32)
        score = self.guarded((rows, hkv, k), torch.float32)
        ws = self.ws(tbs.OP_SELECT_PREFILL, rows, 1, q1)
        tbs.infv2_select_blocks(self.cfg, tbs.INFV2_MODE_PREFILL, q, rows, q0, self.ck,
                                self.ck_offsets, self.kv_offsets, None, 1, q1, idx, score, ws)
        out = self.guarded(tuple(q.shape), q.dtype)
        wsa = self.ws(tbs.OP_ATTN_PREFILL, rows, 1, q1)
        tbs.infv2_sparse_attn_prefill(self.cfg, q, rows, q0, self.k, self.v, self.kv_offsets, idx,
                                      out, wsa)
        return idx, score, out

    def prefill(self, chunk: int):
        L = int(self.wl.lens[0])
        idxs, scores, outs = [], [], []
        for q0 in range(0, L, chunk):
            i, s, o = self.prefill_chunk(q0, min(L, q0 + chunk))
            idxs.append(i)
            scores.append(s)
            outs.append(o)
        return torch.cat(idxs), torch.cat(scores), torch.cat(outs)

    # ---------------------------------------------------------------- backward
    def attn_prefill_bwd(self, q0: int, q1: int, idx: torch.Tensor, out: torch.Tensor,
                         dout: torch.Tensor, dk: Optional[torch.Tensor] = None,
                         dv: Optional[torch.Tensor] = None):
        """Gradients of rows [q0, q1) (idx, out, dout hold those rows only).  dk / dv
        default to fresh buffers filled with NaN so untouched tokens stay visible."""
        rows = q1 - q0
        q = self.q[q0:q1]
        dq = torch.empty_like(q)
        if dk is None:
            dk = nan_like(self.k)
        if dv is None:
            dv = nan_like(self.v)
        ws = self.ws(tbs.OP_ATTN_PREFILL_BWD, rows, 1, q1)
        tbs.infv2_sparse_attn_prefill_bwd(self.cfg, q, rows, q0, self.k, self.v, self.kv_offsets,
                                          idx, out, dout, dq, dk, dv, ws)
        return dq, dk, dv


def nan_like(t: torch.Tensor) -> torch.Tensor:
    """Same shape and storage type, every element a quiet NaN (fp32 or bf16 bits)."""
    if t.dtype == torch.int16:
        return torch.full_like(t, 0x7FC0)
    return torch.full_like(t, float("nan"))


# ---------------------------------------------------------------- coarse-kernel LogSumExp
def coarse_ck(dev: DeviceWorkload, coarse: int, upto=None):
    """Coarse compressed keys (spans of `coarse` tokens at stride `coarse`) of every
    sequence, written by infv2_compress_keys with that kernel size and stride.
    Returns (ck tensor, offsets tensor, per-sequence counts)."""
    import dataclasses
    wl = dev.wl
    cfg_c = dataclasses.replace(dev.cfg, kernel_size=coarse, kernel_stride=coarse)
    lens = wl.lens if upto is None else np.asarray(upto)
    ncs = [num_kernels(int(n), coarse, coarse) for n in lens]
    off = np.zeros(len(ncs) + 1, dtype=np.int64)
    off[1:] = np.cumsum(ncs)
    tdt = torch.int16 if dev.ck_dtype == "bf16" else torch.float32
    ck = torch.zeros(max(1, int(off[-1]) * wl.num_kv_heads * wl.head_dim), dtype=tdt, device=dev.device)
    offs = torch.tensor(off, dtype=torch.int64, device=dev.device)
    kv_lens = torch.tensor(lens, dtype=torch.int64, device=dev.device)
    tbs.infv2_compress_keys(cfg_c, dev.k, dev.kv_offsets, kv_lens, offs, None, wl.batch,
                            int(np.max(lens)), -1, ck)
    return ck, offs, ncs


def select_coarse(dev: DeviceWorkload, coarse: int, mode: int, q, rows: int, q_start: int,
                  ckc, ckc_offsets, max_len: int, kv_lens=None):
    hkv, k = dev.wl.num_kv_heads, dev.cfg.topk
    idx = torch.empty((rows, hkv, k), dtype=torch.int32, device=dev.device)
    score = torch.empty((rows, hkv, k), dtype=torch.float32, device=dev.device)
    op = tbs.OP_SELECT_COARSE_DECODE if mode == tbs.INFV2_MODE_DECODE else tbs.OP_SELECT_COARSE_PREFILL
    batch = rows if mode == tbs.INFV2_MODE_DECODE else 1
    ws = dev.ws(op, rows, batch, max_len)
    tbs.infv2_select_blocks_coarse(dev.cfg, coarse, mode, q, rows, q_start, dev.ck, dev.ck_offsets,
                                   ckc, ckc_offsets, dev.kv_offsets,
                                   dev.kv_lens if kv_lens is None else kv_lens, batch, max_len,
                                   idx, score, ws)
    return idx, score
