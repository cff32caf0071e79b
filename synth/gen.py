"""Seeded synthetic workloads shaped like the long-context runs the MiniCPM4
pages measure (32K-128K tokens, 32 query heads over 2 KV heads, head size 128).

The pages measure on documents with trained weights; neither is available, so
these draws stand in for them: i.i.d. standard-normal Q/K/V with a few
"relevant" KV blocks planted along one random unit direction per KV head, so
that block selection has structure to find.

Memory layout produced here (and consumed by both the HIP path and the oracle):
  * K and V of sequence b occupy tokens [kv_offsets[b], kv_offsets[b+1]) of a
    packed buffer; inside that range the layout is [Hkv][n_b][d], i.e. each KV
    head's keys are contiguous ("KV cache contiguous per head").
  * decode queries: q[b][Hq][d], one row per sequence at position n_b - 1.
  * prefill queries: q[L][Hq][d], row r at position r.
bf16 tensors are carried as uint16 bit patterns (round-to-nearest-even from the
float32 draw); fp32 tensors as float32.

Draw order (fixed, numpy PCG64 ``default_rng(seed)``): sequence lengths (only
when drawn), then per sequence K, V, then per KV head the unit direction u and
the planted block ids, then all queries.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np


# --------------------------------------------------------------------------
# bf16 encoding (input encoding only; not part of the attention method)
# --------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); return uint16 bits."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((b >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((b + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact decode of bf16 bit patterns to float32."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32)
            << np.uint32(16)).view(np.float32)


# --------------------------------------------------------------------------
# workload container
# --------------------------------------------------------------------------
@dataclass
class Workload:
    name: str
    mode: str                 # "decode" or "prefill"
    io_dtype: str             # "fp32" or "bf16"
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int           # m
    kernel_size: int          # p
    kernel_stride: int        # s
    topk: int                 # k, counting the forced blocks
    init_blocks: int
    local_blocks: int
    lens: np.ndarray          # int64 [B]
    kv_offsets: np.ndarray    # int64 [B+1], token offsets of each sequence
    k: np.ndarray             # packed, float32 or uint16 bits
    v: np.ndarray
    q: np.ndarray             # decode [B][Hq][d]; prefill [L][Hq][d]
    planted: List[np.ndarray] = field(default_factory=list)  # per seq [Hkv][n_planted]
    chunk: int = 0            # prefill query-chunk rows (0: one chunk)
    seed: int = 0
    score_scale: float = 1.0
    attn_scale: Optional[float] = None   # None: 1/sqrt(head_dim)

    @property
    def batch(self) -> int:
        return int(self.lens.shape[0])

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    def _seq(self, arr: np.ndarray, b: int) -> np.ndarray:
        o0, o1 = int(self.kv_offsets[b]), int(self.kv_offsets[b + 1])
        n = o1 - o0
        step = self.num_kv_heads * self.head_dim
        return arr[o0 * step:o1 * step].reshape(self.num_kv_heads, n, self.head_dim)

    def k_seq(self, b: int) -> np.ndarray:
        return self._seq(self.k, b)

    def v_seq(self, b: int) -> np.ndarray:
        return self._seq(self.v, b)

    def decoded(self, arr: np.ndarray) -> np.ndarray:
        """Exact float64 values of a stored tensor (bf16 bits or float32)."""
        if self.io_dtype == "bf16":
            return bf16_bits_to_f32(arr).astype(np.float64)
        return np.asarray(arr, dtype=np.float32).astype(np.float64)

    def k_f64(self, b: int) -> np.ndarray:
        return self.decoded(self.k_seq(b))

    def v_f64(self, b: int) -> np.ndarray:
        return self.decoded(self.v_seq(b))

    def q_f64(self) -> np.ndarray:
        return self.decoded(self.q)

    def resolved_attn_scale(self) -> float:
        return (1.0 / np.sqrt(self.head_dim)) if self.attn_scale is None else float(self.attn_scale)


# --------------------------------------------------------------------------
# generator
# --------------------------------------------------------------------------
def _encode(x: np.ndarray, io_dtype: str) -> np.ndarray:
    if io_dtype == "bf16":
        return f32_to_bf16_bits(x)
    return np.ascontiguousarray(x, dtype=np.float32)


def make_workload(*, name: str = "custom", mode: str, io_dtype: str, lens, num_q_heads: int,
                  num_kv_heads: int, head_dim: int = 128, block_size: int = 64,
                  kernel_size: int = 32, kernel_stride: int = 16, topk: int = 64,
                  init_blocks: int = 1, local_blocks: int = 4, n_planted: int = 0,
                  plant_scale: float = 3.0, chunk: int = 0, seed: int = 0,
                  score_scale: float = 1.0, attn_scale: Optional[float] = None,
                  rng: Optional[np.random.Generator] = None) -> Workload:
    """Draw one workload.  ``lens`` is a list of sequence lengths (prefill: one)."""
    if rng is None:
        rng = np.random.default_rng(seed)
    lens = np.asarray(lens, dtype=np.int64).reshape(-1)
    if mode == "prefill" and lens.shape[0] != 1:
        raise ValueError("prefill workloads hold one sequence")
    hkv, d, m = num_kv_heads, head_dim, block_size
    offsets = np.zeros(lens.shape[0] + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(lens)
    k_parts, v_parts, planted = [], [], []
    for n in lens.tolist():
        kf = rng.standard_normal((hkv, n, d), dtype=np.float32)
        vf = rng.standard_normal((hkv, n, d), dtype=np.float32)
        nblk = -(-n // m)
        if mode == "decode":
            c_last = (n - 1) // m
            cand = np.arange(1, max(1, c_last - local_blocks + 1), dtype=np.int64)
        else:
            cand = np.arange(1, nblk, dtype=np.int64)
        seq_planted = np.zeros((hkv, 0), dtype=np.int64)
        rows = []
        for h in range(hkv):
            u = rng.standard_normal(d).astype(np.float64)
            u = (u / np.linalg.norm(u)).astype(np.float32)
            cnt = min(n_planted, cand.shape[0])
            ids = np.sort(rng.choice(cand, size=cnt, replace=False)) if cnt else np.zeros(0, np.int64)
            for j in ids.tolist():
                kf[h, j * m:min((j + 1) * m, n), :] += np.float32(plant_scale) * u
            rows.append(ids)
        if rows:
            seq_planted = np.stack(rows)
        planted.append(seq_planted)
        k_parts.append(_encode(kf, io_dtype).reshape(-1))
        v_parts.append(_encode(vf, io_dtype).reshape(-1))
        del kf, vf
    if mode == "decode":
        qf = rng.standard_normal((lens.shape[0], num_q_heads, d), dtype=np.float32)
    else:
        qf = rng.standard_normal((int(lens[0]), num_q_heads, d), dtype=np.float32)
    return Workload(name=name, mode=mode, io_dtype=io_dtype, num_q_heads=num_q_heads,
                    num_kv_heads=hkv, head_dim=d, block_size=m, kernel_size=kernel_size,
                    kernel_stride=kernel_stride, topk=topk, init_blocks=init_blocks,
                    local_blocks=local_blocks, lens=lens, kv_offsets=offsets,
                    k=np.concatenate(k_parts) if k_parts else np.zeros(0, np.uint16),
                    v=np.concatenate(v_parts) if v_parts else np.zeros(0, np.uint16),
                    q=_encode(qf, io_dtype), planted=planted, chunk=chunk, seed=seed,
                    score_scale=score_scale, attn_scale=attn_scale)


# The five workloads the measurements are quoted on.  Index = default seed.
CONFIGS = {
    0: dict(name="tiny_prefill_decode_fp32_L1024", mode="prefill", io_dtype="fp32", lens=[1024],
            num_q_heads=16, num_kv_heads=1, topk=8, init_blocks=1, local_blocks=2, n_planted=4),
    1: dict(name="decode_bf16_32k", mode="decode", io_dtype="bf16", lens=[32768],
            num_q_heads=32, num_kv_heads=2, topk=64, init_blocks=1, local_blocks=4, n_planted=16),
    2: dict(name="decode_bf16_128k", mode="decode", io_dtype="bf16", lens=[131072],
            num_q_heads=32, num_kv_heads=2, topk=64, init_blocks=1, local_blocks=4, n_planted=64),
    3: dict(name="chunked_prefill_bf16_32k", mode="prefill", io_dtype="bf16", lens=[32768],
            num_q_heads=32, num_kv_heads=2, topk=64, init_blocks=1, local_blocks=4, n_planted=32,
            chunk=4096),
    4: dict(name="batched_decode_bf16_16x64k-128k", mode="decode", io_dtype="bf16", lens=None,
            num_q_heads=32, num_kv_heads=2, topk=64, init_blocks=1, local_blocks=4, n_planted=64),
}


def make_config(index: int, seed: Optional[int] = None) -> Workload:
    """The workload of measurement config ``index`` (seed defaults to the index)."""
    params = dict(CONFIGS[index])
    seed = index if seed is None else seed
    rng = np.random.default_rng(seed)
    if params["lens"] is None:          # 16 sequences, lengths uniform on [65536, 131072]
        params["lens"] = rng.integers(65536, 131072, size=16, endpoint=True).tolist()
    return make_workload(seed=seed, rng=rng, **params)


def extra_decode_queries(wl: Workload, count: int, seed: int = 1_000_003) -> np.ndarray:
    """Further decode queries [count][B][Hq][d] (own stream, does not disturb ``wl``)."""
    rng = np.random.default_rng(seed + wl.seed)
    qf = rng.standard_normal((count, wl.batch, wl.num_q_heads, wl.head_dim), dtype=np.float32)
    return _encode(qf, wl.io_dtype)


def upstream_grad(wl: Workload, seed: int = 2_000_003) -> np.ndarray:
    """A gradient of the loss w.r.t. the attention output, shaped like ``wl.q``:
    i.i.d. N(0, 1), encoded in the workload's io dtype (own stream)."""
    rng = np.random.default_rng(seed + wl.seed)
    g = rng.standard_normal(wl.q.shape, dtype=np.float32)
    return _encode(g, wl.io_dtype)
