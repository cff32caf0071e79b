#!/usr/bin/env python3
"""Throughput of the InfLLM v2 hot path on one MI355X.

Main line: single-step decode at 128K context (batch 1, 32 query heads over 2
KV heads, head size 128, KV block 64, semantic kernels 32/16, top-k 64 with the
initial block and 4 local blocks forced).  One step = the whole path for one new
token: compressed key of the kernel the token completes, block selection
(logits, LogSumExp, group score, block max, top-k) and sparse attention.  The
step rotates through independent cache replicas ("layers") so that every step
reads its compressed keys and selected K/V from HBM rather than from the 256 MiB
Infinity Cache.  Inputs are resident in HBM before timing starts.

Also reported on the same line: 32K chunked prefill (TFLOPS of useful
selected-block attention FLOPs), the 32K training backward (gradients of q, K
and V through the sparse attention), batched decode of 16 sequences of 64K-128K,
the roofline fraction of the dominant kernel, and the float64 CPU oracle timed
on this host on a bounded sample.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "128K sparse-attn decode tok/s + HBM GB/s; 32K prefill TFLOPS; % of roofline"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ----------------------------------------------------------------------------- helpers
def num_kernels(n: int, p: int, s: int) -> int:
    return 0 if n < p else (n - p) // s + 1


def attended_tokens(idx: np.ndarray, positions: np.ndarray, n: np.ndarray, m: int) -> np.ndarray:
    """|T_i| per (row, KV head): tokens t <= i, t < n of the selected blocks."""
    blk = idx.astype(np.int64)
    start = blk * m
    end = np.minimum(np.minimum(start + m, (positions + 1)[:, None, None]), n[:, None, None])
    cnt = np.where(blk >= 0, np.maximum(end - start, 0), 0)
    return cnt.sum(axis=2)


class Timer:
    """Elapsed GPU time between events recorded on the current (library) stream."""

    def __init__(self, torch):
        self.torch = torch

    def event(self):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record()
        return e


_SLEEP_CYCLES_PER_MS = None


def queue_ahead(torch, ms: float) -> None:
    """Occupy the stream for about `ms` with a spin kernel, so that the launches
    queued behind it while it spins run back to back, as in a graph replay,
    instead of each starting on an idle GPU after the host's launch latency."""
    global _SLEEP_CYCLES_PER_MS
    if _SLEEP_CYCLES_PER_MS is None:
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        torch.cuda._sleep(1_000_000)
        b.record()
        torch.cuda.synchronize()
        _SLEEP_CYCLES_PER_MS = 1_000_000 / max(a.elapsed_time(b), 1e-3)
    torch.cuda._sleep(int(_SLEEP_CYCLES_PER_MS * ms))


MALL_BYTES = 256 << 20          # Infinity Cache of the MI355X
COLD_PASS_BYTES = 2 * MALL_BYTES  # bytes a timed pass must touch between two uses of a replica
_FLUSH = None


def flush_mall(torch) -> None:
    """Evict the Infinity Cache (and L2): read and write 1 GiB of scratch, four
    times the cache, so that the next steps find their inputs only in HBM."""
    global _FLUSH
    if _FLUSH is None:
        _FLUSH = torch.empty(2 * (128 << 20), dtype=torch.int32, device="cuda")   # 2 x 512 MiB
    a, b = _FLUSH[: 128 << 20], _FLUSH[128 << 20:]
    b.copy_(a)
    a.copy_(b)


def cold_replicas(step_bytes: int, floor: int = 8) -> int:
    """Replicas rotated per step so that a replica is used again only after at
    least COLD_PASS_BYTES of other steps' data."""
    return max(floor, -(-COLD_PASS_BYTES // max(1, step_bytes)))


def kernel_times(tbs, torch, run, steps: int, families, ahead_ms: float = 50.0,
                 passes: int = 2) -> dict:
    """Live per-kernel times: the library stamps every launch of one kernel
    family with a pair of HIP events while a session is open; eager passes of
    `steps` steps per family, each after an Infinity-Cache flush and queued
    behind a spin kernel of `ahead_ms` so the GPU runs the pass back to back.
    Of `passes` such passes the one with the lower mean is kept (timing noise
    only adds time; both passes start from a flushed cache)."""
    out = {}
    for fam in families:
        best = None
        for _ in range(passes):
            torch.cuda.synchronize()
            flush_mall(torch)
            queue_ahead(torch, ahead_ms)
            tbs.infv2_timing_start(fam)
            try:
                for t in range(steps):
                    run(t)
            finally:
                ms, n = tbs.infv2_timing_stop()
            if best is None or (n and best[1] and ms / n < best[0] / best[1]):
                best = (ms, n)
        ms, n = best
        out[fam] = {"launches_per_step": n / steps,
                    "us_per_launch": ms * 1e3 / n if n else None,
                    "us_per_step": ms * 1e3 / steps,
                    "passes": passes}
    return out


def roofline_of(times: dict, work: dict, bound: str, peak: float, unit: str, scale: float,
                workload: str) -> dict:
    """Roofline line of the dominant kernel: the largest time per step among the
    kernels that carry the step's algorithmic traffic or FLOPs (the others only
    pass intermediates between kernels and are reported in "kernels").  Beside
    the live time it carries the committed rocprofv3 average of the same kernel
    on the same workload, and the HBM traffic from the committed counter runs,
    each only while the kernel's sources are unchanged since they were taken."""
    cand = [f for f in work if times.get(f, {}).get("us_per_launch")]
    dom = max(cand, key=lambda f: times[f]["us_per_step"])
    us = times[dom]["us_per_launch"]
    achieved = work[dom] / (us * 1e-6) / scale
    prof = profiled(DURATION_FILE, workload, dom)
    rp = None
    if prof:
        a2 = work[dom] / (prof["avg_us"] * 1e-6) / scale
        rp = {"us_per_launch": prof["avg_us"], "achieved": a2, "frac": a2 / peak,
              "calls": prof["calls"], "kernel": prof["kernel"],
              "live_over_rocprof": us / prof["avg_us"], "source": "profiles/kernel_durations.json"}
    tr = profiled(TRAFFIC_FILE, workload, dom)
    traffic = None
    if tr:
        traffic = 1024.0 * (tr["fetch_kib_per_launch"] / tr["fetch_scale"]
                            + tr["write_kib_per_launch"] / tr["write_scale"])
    return {"bound": bound, "kernel": dom, "achieved": achieved, "peak": peak, "unit": unit,
            "frac": achieved / peak, "traffic": traffic, "us_per_launch": us,
            "work_per_launch": work[dom], "rocprof": rp, "workload": workload}


DURATION_FILE = os.path.join(ROOT, "profiles", "kernel_durations.json")
CALIBRATION_MIB = 256          # size of the copies that --copy-calibration runs for the counter passes
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
# kernel family -> (source file, rocprofv3 kernel-name prefixes)
KERNEL_SOURCE = {"attn_decode": ("attn_decode.hip", ("infv2::attn_decode_mfma", "infv2::attn_decode_topk_mfma")),
                 "select_logits": ("select.hip", ("infv2::sel_dec_logits_mfma",)),
                 "attn_prefill": ("attn_prefill.hip", ("infv2::attn_prefill_mfma",)),
                 "select_prefill": ("select.hip", ("infv2::sel_pre_mfma",)),
                 "bwd_row": ("attn_bwd_mfma.hip", ("infv2::bwd_row_mfma",)),
                 "bwd_col": ("attn_bwd_mfma.hip", ("infv2::bwd_col_mfma",))}


def source_digest(kernel: str) -> str:
    """SHA-256 over the kernel's source file and every shared header of csrc/."""
    import glob
    import hashlib
    csrc = os.path.join(ROOT, "trainable_block_sparse_amd", "csrc")
    h = hashlib.sha256()
    for path in [os.path.join(csrc, KERNEL_SOURCE[kernel][0])] + sorted(glob.glob(os.path.join(csrc, "*.hpp"))):
        h.update(os.path.basename(path).encode())
        h.update(open(path, "rb").read())
    return h.hexdigest()


def profiled(path: str, workload: str, kernel: str):
    """The committed profile record of `kernel` on `workload`, or None when there
    is none or the kernel's sources changed since it was taken."""
    try:
        rec = json.load(open(path))[workload][kernel]
    except (OSError, KeyError, ValueError, TypeError):
        return None
    if kernel not in KERNEL_SOURCE or rec.get("source_sha256") != source_digest(kernel):
        return None
    return rec


def _rocprof_name_family(name: str):
    base = name[5:] if name.startswith("void ") else name
    for fam, (_, prefixes) in KERNEL_SOURCE.items():
        if base.startswith(prefixes):
            return fam
    return None


def summarize_rocprof(kind: str, workload: str, paths, command: str) -> int:
    """Fold rocprofv3 CSV output into the committed profile records.
    kind "stats":   paths = [<name>_kernel_stats.csv, <name>_kernel_trace.csv]
                    -> kernel_durations.json: the average over every launch of the
                    run, and over the launches of the per-kernel timing passes
                    (those queued behind the spin kernel; what "kernels" and the
                    live roofline time)
    kind "traffic": paths = [FETCH_SIZE counter_collection.csv, WRITE_SIZE one]
                    -> traffic.json, each counter scaled by what it reads for the
                    device-to-device copies of known size (--copy-calibration)."""
    import csv
    out_path = DURATION_FILE if kind == "stats" else TRAFFIC_FILE
    try:
        db = json.load(open(out_path))
    except (OSError, ValueError):
        db = {}
    entry = db.setdefault(workload, {})
    if kind == "stats":
        # launches inside the timing passes: after a spin kernel, up to the next
        # spin kernel or the next pass's cache flush (copies of 50 us and more;
        # the small copies inside a step do not end a pass)
        passes = {}
        trace = sorted(csv.DictReader(open(paths[1])), key=lambda r: int(r["Start_Timestamp"]))
        inside = False
        for r in trace:
            name = r["Kernel_Name"]
            us = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
            if "sleep" in name or "spin" in name:
                inside = True
                continue
            fam = _rocprof_name_family(name)
            if fam is None:
                if us >= 50.0 and not name.startswith("void infv2") and not name.startswith("infv2"):
                    inside = False
                continue
            if inside:
                passes.setdefault(fam, []).append(us)
        seen = set()
        for row in csv.DictReader(open(paths[0])):
            fam = _rocprof_name_family(row["Name"])
            if fam is None:
                continue
            calls = int(row["Calls"])
            avg_us = float(row["AverageNs"]) / 1e3
            kname = row["Name"].split("(")[0]
            lo, hi = float(row["MinNs"]) / 1e3, float(row["MaxNs"]) / 1e3
            if fam in seen:
                # several instantiations of one family in this run: merge by call count
                prev = entry[fam]
                tot = prev["calls"] + calls
                avg_us = (prev["avg_us_all"] * prev["calls"] + avg_us * calls) / tot
                calls = tot
                kname = prev["kernel"] + "; " + kname
                lo, hi = min(lo, prev["min_us"]), max(hi, prev["max_us"])
            seen.add(fam)
            pv = passes.get(fam, [])
            entry[fam] = {"kernel": kname, "calls": calls, "avg_us_all": avg_us,
                          "min_us": lo, "max_us": hi,
                          "timing_pass_launches": len(pv),
                          "avg_us": float(np.mean(pv)) if pv else avg_us,
                          "command": command, "source_sha256": source_digest(fam)}
            print(f"{workload} {fam}: {calls} calls, average {avg_us:.2f} us; "
                  f"{len(pv)} in timing passes, average {entry[fam]['avg_us']:.2f} us")
    else:
        per = {}
        for counter, path in zip(("FETCH_SIZE", "WRITE_SIZE"), paths):
            vals, copies = {}, {}
            for row in csv.DictReader(open(path)):
                if row["Counter_Name"] != counter:
                    continue
                v = float(row["Counter_Value"])
                if row["Kernel_Name"].startswith("__amd_rocclr_copyBuffer"):
                    copies[int(row["Dispatch_Id"])] = v
                    continue
                fam = _rocprof_name_family(row["Kernel_Name"])
                if fam is not None:
                    vals.setdefault(fam, []).append(v)
            per[counter] = (vals, copies)
        (fv, fcopies), (wv, wcopies) = per["FETCH_SIZE"], per["WRITE_SIZE"]
        # the calibration copies (--copy-calibration) are the copyBuffer launches
        # whose WRITE_SIZE equals their size; FETCH_SIZE is read off the same
        # dispatches of the other pass (the program is deterministic)
        want = CALIBRATION_MIB * 1024.0
        ids = [i for i, v in wcopies.items() if abs(v / want - 1) < 0.01 and i in fcopies]
        if not ids:
            print(f"no {CALIBRATION_MIB} MiB calibration copy in the counter runs", file=sys.stderr)
            return 1
        fcopy = float(np.median([fcopies[i] for i in ids]))
        wcopy = float(np.median([wcopies[i] for i in ids]))
        # the calibration copy moves the same number of bytes in and out; its
        # write counter is exact (checked against its size), the fetch counter is not
        for fam in sorted(set(fv) & set(wv)):
            entry[fam] = {"launches": len(fv[fam]),
                          "fetch_kib_per_launch": sum(fv[fam]) / len(fv[fam]),
                          "write_kib_per_launch": sum(wv[fam]) / len(wv[fam]),
                          "fetch_scale": fcopy / wcopy, "write_scale": 1.0,
                          "calibration": f"device-to-device copy of {CALIBRATION_MIB} MiB: FETCH_SIZE "
                                         f"{fcopy:.1f} KiB, WRITE_SIZE {wcopy:.1f} KiB",
                          "command": command,
                          "source_sha256": source_digest(fam)}
            e = entry[fam]
            print(f"{workload} {fam}: {e['launches']} launches, FETCH {e['fetch_kib_per_launch']:.1f} KiB "
                  f"(scale {e['fetch_scale']:.4f}), WRITE {e['write_kib_per_launch']:.1f} KiB")
    json.dump(db, open(out_path, "w"), indent=1, sort_keys=True)
    open(out_path, "a").write("\n")
    return 0


# ----------------------------------------------------------------------------- decode
DECODE_FAMILIES = ("compress", "select_logits", "select_scores", "select_topk", "attn_decode",
                   "attn_merge")


def decode_bytes(wl, ck_bytes: int, n_list) -> dict:
    """Algorithmic HBM bytes of one decode step, per call of each entry point."""
    kb = decode_kernel_bytes(wl, ck_bytes, n_list)
    fused = kb["compress"] if wl.io_dtype == "bf16" else 0     # counted in the logits kernel too
    return {"compress": kb["compress"], "select": kb["select_logits"] - fused + kb["select_topk"],
            "attn": kb["attn_decode"] + kb["attn_merge"]}


def decode_kernel_bytes(wl, ck_bytes: int, n_list) -> dict:
    """Algorithmic HBM bytes per launch of each decode kernel: what the step must
    move, attributed to the kernel that moves it (intermediates between kernels
    are not counted)."""
    d, hq, hkv, m, k = wl.head_dim, wl.num_q_heads, wl.num_kv_heads, wl.block_size, wl.topk
    esz = 2 if wl.io_dtype == "bf16" else 4
    q_b = hq * d * esz
    sel_kv = sum(hkv * min(k * m, n) * d * esz * 2 for n in n_list)
    ck = sum(hkv * num_kernels(n, wl.kernel_size, wl.kernel_stride) * d * ck_bytes for n in n_list)
    B = len(n_list)
    new_ck = B * hkv * (wl.kernel_size * d * esz + d * ck_bytes)      # p keys in, one CK out
    return {
        "compress": new_ck,
        "select_logits": ck + B * q_b + (new_ck if esz == 2 else 0),     # every visible CK, q (and
                                                                          # the fused new CK, bf16)
        "select_topk": B * hkv * k * 4,                                   # block ids out
        "attn_decode": sel_kv + B * (q_b + hkv * k * 4),                  # selected K/V, q, ids
        "attn_merge": B * q_b,                                            # output rows
    }


def bench_decode(cfg_index: int, args, torch, tbs, gh, replicas: int = 0, ck_dtype=None) -> dict:
    """One decode step per replica of the cache.  The timed region holds exactly
    `steps` steps, replica (warmup + t) mod R at step t, after an Infinity-Cache
    flush; R is large enough that a replica is used again only after at least
    COLD_PASS_BYTES of other steps, so every step reads its compressed keys and
    selected K/V from HBM."""
    from synth import make_config, extra_decode_queries
    wl = make_config(cfg_index)
    ck_dtype = ck_dtype or args.ck_dtype
    ckb = 2 if ck_dtype == "bf16" else 4
    profile_name = wl.name if ck_dtype == "fp32" else wl.name + "/ck_bf16"
    lens = [int(n) for n in wl.lens]
    nb = decode_bytes(wl, ckb, lens)
    kb = decode_kernel_bytes(wl, ckb, lens)
    step_bytes = sum(nb.values())
    R = replicas if replicas > 0 else cold_replicas(step_bytes)
    dev = gh.DeviceWorkload(wl, ck_dtype)
    dev.compress()
    cfg = dev.cfg
    B, n_max = wl.batch, dev.max_len
    log(f"config {cfg_index}: {wl.name}, B={B}, replicas={R} ({R * step_bytes / 2**20:.0f} MiB per rotation)")
    qs = gh.to_device(extra_decode_queries(wl, R))                # [R][B][Hq][d]
    Ks = [dev.k] + [dev.k.clone() for _ in range(R - 1)]
    Vs = [dev.v] + [dev.v.clone() for _ in range(R - 1)]
    CKs = [dev.ck] + [dev.ck.clone() for _ in range(R - 1)]
    outs = torch.empty((R,) + tuple(dev.q.shape), dtype=dev.q.dtype, device="cuda")
    idx = torch.empty((B, wl.num_kv_heads, cfg.topk), dtype=torch.int32, device="cuda")
    ws_sel = dev.ws(tbs.OP_SELECT_DECODE, B, B, n_max)
    ws_att = dev.ws(tbs.OP_ATTN_DECODE, B, B, n_max)
    # the step's new token completes (at most) the last kernel of each sequence
    begin = torch.tensor([max(0, num_kernels(int(n), wl.kernel_size, wl.kernel_stride) - 1)
                          for n in wl.lens], dtype=torch.int64, device="cuda")

    def compress(r):
        tbs.infv2_compress_keys(cfg, Ks[r], dev.kv_offsets, dev.kv_lens, dev.ck_offsets, begin, B,
                                n_max, 1, CKs[r])

    def select(r):
        tbs.infv2_select_blocks(cfg, tbs.INFV2_MODE_DECODE, qs[r], B, 0, CKs[r], dev.ck_offsets,
                                dev.kv_offsets, dev.kv_lens, B, n_max, idx, None, ws_sel)

    def attn(r):
        tbs.infv2_sparse_attn_decode(cfg, qs[r], Ks[r], Vs[r], dev.kv_offsets, dev.kv_lens, B, n_max,
                                     idx, outs[r], ws_att)

    ws_step = dev.ws(tbs.OP_DECODE_STEP, B, B, n_max)

    def step(r):
        # one call: the newest token's compressed key, the selection and the attention
        tbs.infv2_decode_step(cfg, qs[r], Ks[r], Vs[r], dev.kv_offsets, dev.kv_lens, dev.ck_offsets,
                              CKs[r], B, n_max, idx, outs[r], ws_step)

    def step_separate(r):
        compress(r)
        select(r)
        attn(r)

    W, K = args.warmup, args.steps
    order = [(W + t) % R for t in range(K)]            # replicas of the timed steps
    T = Timer(torch)
    for t in range(W):
        step(t % R)
    torch.cuda.synchronize()
    # per-entry-point times, eager launches with events between the calls
    flush_mall(torch)
    ev = []
    for r in order:
        e0 = T.event(); compress(r); e1 = T.event(); select(r); e2 = T.event(); attn(r); e3 = T.event()
        ev.append((e0, e1, e2, e3))
    torch.cuda.synchronize()
    per = np.array([[a.elapsed_time(b) for a, b in zip(x[:-1], x[1:])] for x in ev]) * 1e3  # us
    per_us = dict(zip(["compress", "select", "attn"], per.mean(axis=0).tolist()))
    kt = kernel_times(tbs, torch, lambda t: step(order[t % K]), K, DECODE_FAMILIES)
    # whole steps, eager: the one-call step, and the three entry points in turn
    torch.cuda.synchronize()
    flush_mall(torch)
    s0 = T.event()
    for r in order:
        step(r)
    s1 = T.event()
    torch.cuda.synchronize()
    eager_ms = s0.elapsed_time(s1) / K
    flush_mall(torch)
    s0 = T.event()
    for r in order:
        step_separate(r)
    s1 = T.event()
    torch.cuda.synchronize()
    eager_sep_ms = s0.elapsed_time(s1) / K
    # whole steps, HIP-graph replay: one graph holds the K timed steps (K
    # "layers" of one decode token), captured once, warmed once, then replayed
    # after a cache flush
    graph_ms = None
    if args.graph:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                for r in order:
                    step(r)
        torch.cuda.current_stream().wait_stream(side)
        g.replay()
        torch.cuda.synchronize()
        flush_mall(torch)
        g0 = T.event()
        g.replay()
        g1 = T.event()
        torch.cuda.synchronize()
        graph_ms = g0.elapsed_time(g1) / K
    ms = graph_ms if graph_ms is not None else eager_ms
    for f, v in kt.items():
        if f in kb and v["us_per_launch"]:
            v["bytes_per_launch"] = kb[f]
            v["gbps"] = kb[f] / (v["us_per_launch"] * 1e-6) / 1e9
    distinct = len(set(order))
    res = {
        "workload": wl.name, "batch": B, "lens_min": int(wl.lens.min()), "lens_max": n_max,
        "step": "infv2_decode_step (newest token's compressed key + selection + attention)",
        "ms_per_step": ms, "ms_per_step_eager": eager_ms, "ms_per_step_graph": graph_ms,
        "ms_per_step_eager_separate_calls": eager_sep_ms,
        "tok_per_s": B / (ms * 1e-3), "per_call_us": per_us, "kernels": kt,
        "bytes_per_step": step_bytes,
        "bytes_per_call": nb, "hbm_gbps_step": step_bytes / (ms * 1e-3) / 1e9,
        "replicas": R,
        "cache_state": {
            "flushed_before_timing": True,
            "touched_mib_per_pass": distinct * step_bytes / 2**20,
            "reuse_distance_mib": (R * step_bytes / 2**20) if K > R else None,
            "note": "1 GiB read+write before each timed pass evicts the 256 MiB Infinity Cache; "
                    "inside a pass a replica recurs only after R steps"},
        "roofline": roofline_of(kt, {"select_logits": kb["select_logits"],
                                     "attn_decode": kb["attn_decode"]},
                                "hbm", HBM_PEAK_GBS, "GB/s", 1e9, profile_name),
    }
    # spot parity of the timed path: replica 0, oracle selection on the same query
    res["parity"] = decode_spot_parity(wl, dev, qs, outs, idx, lambda: step(0), ck_dtype, torch, gh)
    del Ks, Vs, CKs
    torch.cuda.empty_cache()
    return res


def bench_decode_loop(args, torch, tbs, gh) -> dict:
    """Decode loop at 128K: each step appends one token per sequence to its cache
    (infv2_append_kv: K/V rows and the compressed key the token completes), then
    selects and attends; and the same loop as one infv2_decode_step_append call
    per token (the append folded into the step's kernels).  The caches have room
    for every appended token; lengths advance on every step, graph replays
    included."""
    from synth import make_config, extra_decode_queries
    wl = make_config(2)
    dev = gh.DeviceWorkload(wl, args.ck_dtype)
    cfg = dev.cfg
    B, hkv, d = wl.batch, wl.num_kv_heads, wl.head_dim
    n_end = int(wl.lens[0])
    step_bytes = sum(decode_bytes(wl, 2 if args.ck_dtype == "bf16" else 4, [n_end]).values())
    R = args.replicas if args.replicas > 0 else cold_replicas(step_bytes)
    W, K = args.warmup, args.steps
    room = W + 12 * K + 64                        # every append of every timing pass fits
    # caches of capacity n_end (128K) holding an n0-token prefix: the loop ends
    # at most at 128K, so it runs the same kernel instantiations as the step
    # measured on the full 128K cache (a larger capacity would give more than
    # 2048 blocks, and the top-k 16 keys per thread instead of 8)
    cap, n0 = n_end, n_end - room
    def padded(t):
        x = torch.zeros((hkv, cap, d), dtype=t.dtype, device="cuda")
        x[:, :n0] = t.view(hkv, n_end, d)[:, :n0]
        return x.view(-1)
    Ks = [padded(dev.k) for _ in range(R)]
    Vs = [padded(dev.v) for _ in range(R)]
    nc_cap = num_kernels(cap, wl.kernel_size, wl.kernel_stride)
    ck_off = torch.tensor([0, nc_cap], dtype=torch.int64, device="cuda")
    kv_off = torch.tensor([0, cap], dtype=torch.int64, device="cuda")
    ck0 = torch.zeros(hkv * nc_cap * d, dtype=dev.ck.dtype, device="cuda")
    ncur = num_kernels(n0, wl.kernel_size, wl.kernel_stride)
    ck0.view(hkv, nc_cap, d)[:, :ncur] = dev.ck.view(hkv, -1, d)[:, :ncur]
    CKs = [ck0.clone() for _ in range(R)]
    lens = [torch.tensor([n0], dtype=torch.int64, device="cuda") for _ in range(R)]
    qs = gh.to_device(extra_decode_queries(wl, R))
    kn = qs[:, :, :hkv].contiguous()                     # any [B][Hkv][d] rows serve as new K/V
    vn = qs[:, :, hkv:2 * hkv].contiguous()
    idx = torch.empty((B, hkv, cfg.topk), dtype=torch.int32, device="cuda")
    out = torch.empty_like(dev.q)
    ws_sel = dev.ws(tbs.OP_SELECT_DECODE, B, B, cap)
    ws_att = dev.ws(tbs.OP_ATTN_DECODE, B, B, cap)

    def step(r):
        tbs.infv2_append_kv(cfg, kn[r], vn[r], Ks[r], Vs[r], kv_off, lens[r], ck_off, CKs[r], B)
        tbs.infv2_select_blocks(cfg, tbs.INFV2_MODE_DECODE, qs[r], B, 0, CKs[r], ck_off, kv_off,
                                lens[r], B, cap, idx, None, ws_sel)
        tbs.infv2_sparse_attn_decode(cfg, qs[r], Ks[r], Vs[r], kv_off, lens[r], B, cap, idx, out,
                                     ws_att)

    order = [(W + t) % R for t in range(K)]
    T = Timer(torch)
    for t in range(W):
        step(t % R)
    torch.cuda.synchronize()
    flush_mall(torch)
    s0 = T.event()
    for r in order:
        step(r)
    s1 = T.event()
    torch.cuda.synchronize()
    eager_ms = s0.elapsed_time(s1) / K
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            for r in order:
                step(r)
    torch.cuda.current_stream().wait_stream(side)
    g.replay()
    torch.cuda.synchronize()
    flush_mall(torch)
    g0 = T.event()
    g.replay()
    g1 = T.event()
    torch.cuda.synchronize()
    graph_ms = g0.elapsed_time(g1) / K
    kt = kernel_times(tbs, torch, lambda t: step(order[t % K]), K, ("append",))
    # the same loop with the append folded into the step
    ws_step = dev.ws(tbs.OP_DECODE_STEP, B, B, cap)

    def step_fused(r):
        tbs.infv2_decode_step_append(cfg, qs[r], kn[r], vn[r], Ks[r], Vs[r], kv_off, lens[r], ck_off,
                                     CKs[r], B, cap, idx, out, ws_step)

    def step_two(r):
        tbs.infv2_append_kv(cfg, kn[r], vn[r], Ks[r], Vs[r], kv_off, lens[r], ck_off, CKs[r], B)
        tbs.infv2_decode_step(cfg, qs[r], Ks[r], Vs[r], kv_off, lens[r], ck_off, CKs[r], B, cap, idx,
                              out, ws_step)

    def graph_time(fn):
        gx = torch.cuda.CUDAGraph()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            with torch.cuda.graph(gx, stream=side):
                for r in order:
                    fn(r)
        torch.cuda.current_stream().wait_stream(side)
        gx.replay()
        torch.cuda.synchronize()
        flush_mall(torch)
        a0 = T.event()
        gx.replay()
        a1 = T.event()
        torch.cuda.synchronize()
        return a0.elapsed_time(a1) / K

    two_ms = graph_time(step_two)
    fused_ms = graph_time(step_fused)
    final_len = int(lens[0].item())
    assert final_len < cap, "the caches ran out of room for the appended tokens"
    assert final_len - n0 <= room
    return {"workload": "decode_loop_bf16_128k", "batch": B, "start_len": n0, "final_len_replica0": final_len,
            "ms_per_step_eager": eager_ms, "ms_per_step_graph": graph_ms, "replicas": R,
            "tok_per_s": B / (graph_ms * 1e-3), "append_us_per_launch": kt["append"]["us_per_launch"],
            "ms_per_step_graph_append_then_step": two_ms,
            "ms_per_step_graph_step_append": fused_ms, "tok_per_s_step_append": B / (fused_ms * 1e-3),
            "note": "graph of the timed steps, replayed after a cache flush; lengths advance on "
                    "every replay"}


def decode_spot_parity(wl, dev, qs, outs, idx, run0, ck_dtype, torch, gh) -> str:
    from oracle import infv2_ref as ref
    from tests.parity import accept_selection, assert_close
    run0()
    torch.cuda.synchronize()
    gi = idx.cpu().numpy().astype(np.int64)
    go = gh.from_device(outs[0], wl.io_dtype)
    q = gh.from_device(qs[0], wl.io_dtype)
    prm = ref.Params(head_dim=wl.head_dim, num_q_heads=wl.num_q_heads, num_kv_heads=wl.num_kv_heads,
                     block_size=wl.block_size, kernel_size=wl.kernel_size,
                     kernel_stride=wl.kernel_stride, topk=wl.topk, init_blocks=wl.init_blocks,
                     local_blocks=wl.local_blocks, ck_dtype=ck_dtype)
    cks = dev.ck_host()
    verdicts = []
    for b in range(min(wl.batch, 2)):
        K = wl.k_f64(b)
        n = K.shape[1]
        for g in range(wl.num_kv_heads):
            rs = ref.select_row(q[b, 16 * g:16 * g + 16], cks[b][g], n - 1, prm)
            verdicts.append(accept_selection(gi[b, g], rs))
        want = ref.attend_with_selection(q[b:b + 1], K, wl.v_f64(b), [n - 1], gi[b:b + 1], prm)
        assert_close(go[b], want[0], wl.io_dtype, "bench decode spot check")
    bad = [v for v in verdicts if v.startswith("fail")]
    if bad:
        raise AssertionError(f"bench parity: {bad[0]}")
    return "ok (" + ", ".join(verdicts) + ")"


# ----------------------------------------------------------------------------- prefill
PREFILL_FAMILIES = ("compress", "select_prefill", "select_topk", "attn_prefill")


def prefill_spot_parity(wl, dev, gi, out, ck_dtype, rows, gh) -> str:
    """Sampled rows of the prefill against the float64 oracle, with compressed
    keys in ck_dtype (bf16: the oracle rounds the exact mean once too)."""
    from oracle import infv2_ref as ref
    from tests.parity import accept_selection, assert_close
    prm = ref.Params(head_dim=wl.head_dim, num_q_heads=wl.num_q_heads, num_kv_heads=wl.num_kv_heads,
                     block_size=wl.block_size, kernel_size=wl.kernel_size,
                     kernel_stride=wl.kernel_stride, topk=wl.topk, init_blocks=wl.init_blocks,
                     local_blocks=wl.local_blocks, ck_dtype=ck_dtype)
    K, V = wl.k_f64(0), wl.v_f64(0)
    ck = dev.ck_host()[0]
    if not np.array_equal(ck, ref.compress_keys(K, wl.kernel_size, wl.kernel_stride, ck_dtype)):
        raise AssertionError("bench parity: compressed keys differ from the oracle's")
    q = wl.decoded(wl.q[rows])                       # the sampled rows only, float64
    go = gh.from_device(out[rows], wl.io_dtype)
    verdicts = []
    for x, i in enumerate(rows):
        for g in range(wl.num_kv_heads):
            rs = ref.select_row(q[x, 16 * g:16 * g + 16], ck[g], i, prm)
            verdicts.append(accept_selection(gi[i, g].astype(np.int64), rs))
    want = ref.attend_with_selection(q, K, V, list(rows), gi[rows].astype(np.int64), prm)
    assert_close(go, want, wl.io_dtype, "bench prefill spot check")
    bad = [v for v in verdicts if v.startswith("fail")]
    if bad:
        raise AssertionError(f"bench parity: {bad[0]}")
    return f"ok: {len(rows)} rows x {wl.num_kv_heads} KV heads ({', '.join(sorted(set(verdicts)))})"


def bench_prefill(args, torch, tbs, gh, ck_dtype=None) -> dict:
    from synth import make_config
    wl = make_config(3)
    ck_dtype = ck_dtype or args.ck_dtype
    dev = gh.DeviceWorkload(wl, ck_dtype)
    L, C = int(wl.lens[0]), wl.chunk
    cfg = dev.cfg
    log(f"config 3: {wl.name}, L={L}, chunk={C}")
    T = Timer(torch)
    hkv, k, hq, d = wl.num_kv_heads, cfg.topk, wl.num_q_heads, wl.head_dim
    idx = torch.empty((L, hkv, k), dtype=torch.int32, device="cuda")
    out = torch.empty_like(dev.q)
    ws = dev.ws(tbs.OP_SELECT_PREFILL, C, 1, L)
    wsa = dev.ws(tbs.OP_ATTN_PREFILL, C, 1, L)
    p, s = wl.kernel_size, wl.kernel_stride

    def run(record):
        evs = []
        for q0 in range(0, L, C):
            q1 = min(L, q0 + C)
            lens = dev.kv_lens.new_tensor([q1])
            begin = dev.kv_lens.new_tensor([num_kernels(q0, p, s)])
            e0 = T.event() if record else None
            tbs.infv2_compress_keys(cfg, dev.k, dev.kv_offsets, lens, dev.ck_offsets, begin, 1, q1,
                                    num_kernels(q1, p, s) - num_kernels(q0, p, s), dev.ck)
            e1 = T.event() if record else None
            tbs.infv2_select_blocks(cfg, tbs.INFV2_MODE_PREFILL, dev.q[q0:q1], q1 - q0, q0, dev.ck,
                                    dev.ck_offsets, dev.kv_offsets, None, 1, q1, idx[q0:q1], None,
                                    ws)
            e2 = T.event() if record else None
            tbs.infv2_sparse_attn_prefill(cfg, dev.q[q0:q1], q1 - q0, q0, dev.k, dev.v,
                                          dev.kv_offsets, idx[q0:q1], out[q0:q1], wsa)
            e3 = T.event() if record else None
            evs.append((e0, e1, e2, e3))
        return evs

    side = torch.cuda.Stream()
    idx2 = torch.empty_like(idx)
    out2 = torch.empty_like(out)

    def run_two_streams():
        """The same calls with each chunk's attention on a second stream: the
        next chunk's compression and selection (which need neither its output
        nor its workspace) run on the first stream meanwhile, so their thread
        blocks fill the compute units the attention's last blocks leave idle."""
        main = torch.cuda.current_stream()
        side.wait_stream(main)
        for q0 in range(0, L, C):
            q1 = min(L, q0 + C)
            lens = dev.kv_lens.new_tensor([q1])
            begin = dev.kv_lens.new_tensor([num_kernels(q0, p, s)])
            tbs.infv2_compress_keys(cfg, dev.k, dev.kv_offsets, lens, dev.ck_offsets, begin, 1, q1,
                                    num_kernels(q1, p, s) - num_kernels(q0, p, s), dev.ck)
            tbs.infv2_select_blocks(cfg, tbs.INFV2_MODE_PREFILL, dev.q[q0:q1], q1 - q0, q0, dev.ck,
                                    dev.ck_offsets, dev.kv_offsets, None, 1, q1, idx2[q0:q1], None,
                                    ws)
            side.wait_stream(main)
            with torch.cuda.stream(side):
                tbs.infv2_sparse_attn_prefill(cfg, dev.q[q0:q1], q1 - q0, q0, dev.k, dev.v,
                                              dev.kv_offsets, idx2[q0:q1], out2[q0:q1], wsa)
        main.wait_stream(side)

    run(False)
    torch.cuda.synchronize()
    reps = []
    for _ in range(args.prefill_reps):
        evs = run(True)
        torch.cuda.synchronize()
        ph = np.array([[a.elapsed_time(b) for a, b in zip(x[:-1], x[1:])] for x in evs])  # ms
        reps.append(ph)
    ph = np.median(np.stack(reps), axis=0)          # [chunks][3]
    run_two_streams()
    torch.cuda.synchronize()
    two, one = [], []
    for _ in range(max(1, args.prefill_reps)):
        e0 = T.event()
        run(False)
        e1 = T.event()
        run_two_streams()
        e2 = T.event()
        torch.cuda.synchronize()
        one.append(e0.elapsed_time(e1))
        two.append(e1.elapsed_time(e2))
    two_ok = bool(torch.equal(idx, idx2) and torch.equal(out, out2))
    gi = idx.cpu().numpy()
    pos = np.arange(L)
    tok = attended_tokens(gi, pos, np.full(L, L), wl.block_size)       # [L][Hkv]
    useful = float(4 * d * (hq // hkv) * tok.sum())
    attn_ms = float(ph[:, 2].sum())
    total_ms = float(ph.sum())
    sel_ms = float(ph[:, 1].sum())
    # scoring GEMM work of one pass: Hq * d * 2 * sum_i n_vis(i)
    nvis = np.array([num_kernels(i + 1, p, s) for i in range(L)], dtype=np.int64)
    score_flops_pass = float(2 * d * hq * nvis.sum())
    # K/V reuse of the attention kernel: a thread block serves 16 consecutive rows
    # of one KV head and streams the union of their selected blocks once
    grp = gi[: (L // 16) * 16].reshape(L // 16, 16, hkv, k).transpose(0, 2, 1, 3).reshape(-1, 16 * k)
    union = np.array([np.unique(r[r >= 0]).size for r in grp])
    pairs = (grp >= 0).sum(axis=1)
    res = {
        "workload": wl.name, "rows": L, "chunk": C, "useful_attn_flops": useful,
        "union_blocks_per_16_rows": float(union.mean()),
        "kv_reuse_per_loaded_block": float(pairs.sum() / union.sum()),
        "attn_ms": attn_ms, "select_ms": sel_ms, "compress_ms": float(ph[:, 0].sum()),
        "total_ms": total_ms, "tflops_attn": useful / (attn_ms * 1e-3) / 1e12,
        "total_ms_endpoints": float(np.median(one)), "total_ms_two_streams": float(np.median(two)),
        "two_streams_equal": two_ok,
        "tflops_path": useful / (total_ms * 1e-3) / 1e12,
        "score_gemm_flops_per_pass": score_flops_pass,
        "last_chunk_attn_ms": float(ph[-1, 2]),
        "last_chunk_useful_flops": float(4 * d * (hq // hkv) * tok[L - C:].sum()),
        "mean_attended_tokens": float(tok.mean()),
    }
    reps_k = max(1, args.prefill_reps)
    kt = kernel_times(tbs, torch, lambda t: run(False), reps_k, PREFILL_FAMILIES)
    res["kernels"] = kt
    n_attn = kt["attn_prefill"]["launches_per_step"]
    res["tflops_attn_kernel"] = useful / (kt["attn_prefill"]["us_per_step"] * 1e-6) / 1e12
    res["roofline"] = roofline_of(kt, {"attn_prefill": useful / n_attn}, "mfma", BF16_PEAK_TFLOPS,
                                  "TFLOP/s", 1e12, wl.name if ck_dtype == "fp32" else wl.name + "/ck_bf16")
    res["ck_dtype"] = ck_dtype
    # spot parity: the first and last rows of the last chunk and 6 random rows
    rng = np.random.default_rng(3)
    rows = sorted({L - C, L - 1} | set(int(x) for x in rng.integers(0, L, 6)))
    res["parity"] = prefill_spot_parity(wl, dev, gi, out, ck_dtype, rows, gh)
    res["_idx"] = gi
    res["_wl"] = wl
    return res


def bench_varlen_prefill(args, torch, tbs, gh) -> dict:
    """Serving-style prefill: 8 sequences of 4K-16K tokens (lengths drawn by seed)
    prefilled whole in one varlen call each for compress, selection and attention."""
    from synth import make_workload, f32_to_bf16_bits
    rng = np.random.default_rng(12)
    lens = rng.integers(4096, 16384, size=8, endpoint=True).tolist()
    wl = make_workload(name="varlen_prefill_bf16_8x4k-16k", mode="decode", io_dtype="bf16", lens=lens,
                       num_q_heads=32, num_kv_heads=2, topk=64, init_blocks=1, local_blocks=4,
                       n_planted=32, seed=12)
    dev = gh.DeviceWorkload(wl, args.ck_dtype)
    cfg = dev.cfg
    rows = np.array(lens, dtype=np.int32)
    starts = np.zeros(len(lens), dtype=np.int64)
    T = int(rows.sum())
    q = gh.to_device(f32_to_bf16_bits(rng.standard_normal((T, 32, 128), dtype=np.float32)))
    idx = torch.empty((T, 2, 64), dtype=torch.int32, device="cuda")
    out = torch.empty_like(q)
    mx = int(rows.max())
    ws_s = dev.ws(tbs.OP_SELECT_PREFILL, T, len(lens), mx)        # all rows: one launch per kernel
    ws_a = dev.ws(tbs.OP_ATTN_PREFILL, mx, 1, mx)
    Timer_ = Timer(torch)

    def run():
        e0 = Timer_.event()
        tbs.infv2_compress_keys(cfg, dev.k, dev.kv_offsets, dev.kv_lens, dev.ck_offsets, None,
                                wl.batch, dev.max_len, -1, dev.ck)
        e1 = Timer_.event()
        tbs.infv2_select_blocks_varlen(cfg, q, rows, starts, dev.ck, dev.ck_offsets, dev.kv_offsets,
                                       idx, None, ws_s)
        e2 = Timer_.event()
        tbs.infv2_sparse_attn_prefill_varlen(cfg, q, rows, starts, dev.k, dev.v, dev.kv_offsets, idx,
                                             out, ws_a)
        e3 = Timer_.event()
        return e0, e1, e2, e3

    run()
    torch.cuda.synchronize()
    times = []
    for _ in range(max(1, args.prefill_reps)):
        ev = run()
        torch.cuda.synchronize()
        times.append([a.elapsed_time(b) for a, b in zip(ev[:-1], ev[1:])])
    tm = np.median(np.array(times), axis=0)
    gi = idx.cpu().numpy()
    pos = np.concatenate([np.arange(n) for n in lens])
    nn = np.concatenate([np.full(n, n) for n in lens])
    tok = attended_tokens(gi, pos, nn, 64)
    useful = float(4 * 128 * 16 * tok.sum())
    return {"workload": wl.name, "lens": lens, "rows": T, "compress_ms": float(tm[0]),
            "select_ms": float(tm[1]), "attn_ms": float(tm[2]), "total_ms": float(tm.sum()),
            "useful_attn_flops": useful, "tflops_attn": useful / (tm[2] * 1e-3) / 1e12,
            "tflops_path": useful / (tm.sum() * 1e-3) / 1e12}


BACKWARD_FAMILIES = ("bwd_row", "bwd_index", "bwd_col")


def bench_backward(args, torch, tbs, gh, pre: dict) -> dict:
    """Training backward of the 32K prefill: gradients of all 32768 rows in one
    call (dq, and dk / dv of the whole sequence), on the forward's selection and
    output.  Algorithmic FLOPs: the five products of an attention backward
    (S, dP, dQ, dK, dV), 10 d FLOPs per (head, attended token)."""
    from synth import upstream_grad
    wl = pre["_wl"]
    L = int(wl.lens[0])
    dev = gh.DeviceWorkload(wl, args.ck_dtype)
    idx, _, out = dev.prefill(wl.chunk)
    dout = gh.to_device(upstream_grad(wl))
    dq = torch.empty_like(dev.q)
    dk = torch.empty_like(dev.k)
    dv = torch.empty_like(dev.v)
    ws = dev.ws(tbs.OP_ATTN_PREFILL_BWD, L, 1, L)
    cfg = dev.cfg
    T = Timer(torch)

    def run(t=0):
        tbs.infv2_sparse_attn_prefill_bwd(cfg, dev.q, L, 0, dev.k, dev.v, dev.kv_offsets, idx, out,
                                          dout, dq, dk, dv, ws)

    run()
    torch.cuda.synchronize()
    times = []
    for _ in range(max(1, args.prefill_reps)):
        e0 = T.event()
        run()
        e1 = T.event()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    ms = float(np.median(times))
    gi = idx.cpu().numpy()
    G, d = wl.num_q_heads // wl.num_kv_heads, wl.head_dim
    tok = float(attended_tokens(gi, np.arange(L), np.full(L, L), wl.block_size).sum())
    algo = 10.0 * d * G * tok
    kt = kernel_times(tbs, torch, run, max(1, args.prefill_reps), BACKWARD_FAMILIES)
    # algorithmic products per kernel: row pass S, dP, dQ; column pass dK, dV
    # (it also recomputes S and dP, counted in "performed" only)
    work = {"bwd_row": 6.0 * d * G * tok / kt["bwd_row"]["launches_per_step"],
            "bwd_col": 4.0 * d * G * tok / kt["bwd_col"]["launches_per_step"]}
    roof = roofline_of(kt, work, "mfma", BF16_PEAK_TFLOPS, "TFLOP/s", 1e12, "prefill_backward_bf16_32k")
    if roof["kernel"] == "bwd_col":
        roof["performed_frac"] = roof["frac"] * 2.0
    per_kernel = {f: {"tflops_algorithmic": w / (kt[f]["us_per_launch"] * 1e-6) / 1e12,
                      "frac": w / (kt[f]["us_per_launch"] * 1e-6) / 1e12 / BF16_PEAK_TFLOPS}
                  for f, w in work.items()}
    # sampled parity: dq of a few rows against the oracle (float64)
    parity = backward_spot_parity(wl, gi, dq, dout, torch, gh)
    return {"workload": "prefill_backward_bf16_32k", "rows": L, "ms": ms,
            "algorithmic_flops": algo, "tflops": algo / (ms * 1e-3) / 1e12,
            "attended_tokens_per_row_head": tok / (L * wl.num_kv_heads),
            "kernels": kt, "per_kernel": per_kernel, "roofline": roof, "parity": parity}


def backward_spot_parity(wl, gi, dq_t, dout_t, torch, gh) -> str:
    from oracle import infv2_ref as ref
    prm = ref.Params(head_dim=128, num_q_heads=32, num_kv_heads=2, block_size=64, kernel_size=32,
                     kernel_stride=16, topk=64, init_blocks=1, local_blocks=4)
    K, V = wl.k_f64(0), wl.v_f64(0)
    q = wl.decoded(wl.q)
    dout = gh.from_device(dout_t, "bf16")
    dq = gh.from_device(dq_t, "bf16")
    L = q.shape[0]
    worst = 0.0
    for i in (0, 4095, L // 2, L - 1):
        for g in range(2):
            hs = slice(16 * g, 16 * g + 16)
            want = ref.attend_row_grad(q[i, hs], K[g], V[g], i, gi[i, g], prm, dout[i, hs])[0]
            s = max(1.0, float(np.abs(want).max()))
            err = np.abs(dq[i, hs] - want) / s - (2e-2 + 1e-2 * np.abs(want) / s)
            worst = max(worst, float(np.abs(dq[i, hs] - want).max() / s))
            if err.max() > 0:
                return f"FAIL dq row {i} head {g}: scaled err {worst:.2e}"
    return f"ok: dq of 4 rows x 2 heads vs the float64 oracle, scaled max err {worst:.1e}"


def _agreement(a: np.ndarray, e: np.ndarray):
    """(share of identical (row, KV head) selections, share of the exact selection's
    blocks also chosen) between approximate ids `a` and exact ids `e` [rows][Hkv][k]."""
    same = float(np.mean(np.all(a == e, axis=-1)))
    shared = total = 0
    for x, y in zip(a.reshape(-1, a.shape[-1]), e.reshape(-1, e.shape[-1])):
        yy = y[y >= 0]
        shared += np.intersect1d(x[x >= 0], yy).size
        total += yy.size
    return same, shared / max(1, total)


def bench_coarse(args, torch, tbs, gh) -> dict:
    """The coarse-kernel LogSumExp selection against the exact one: selection time
    per call and agreement of the selections, at 128K decode (cache replicas for 512 MiB between uses, a new
    query per step, as the main line) and over the 32K prefill (chunks of 4096)."""
    from synth import make_config, extra_decode_queries
    out = {}
    # ---- decode, 128K, batch 1
    wl = make_config(2)
    dev = gh.DeviceWorkload(wl, args.ck_dtype)
    dev.compress()
    cfg, B, n = dev.cfg, wl.batch, dev.max_len
    R = args.replicas if args.replicas > 0 else cold_replicas(dev.ck.numel() * dev.ck.element_size())
    qs = gh.to_device(extra_decode_queries(wl, R))
    CKs = [dev.ck] + [dev.ck.clone() for _ in range(R - 1)]
    T = Timer(torch)
    idx = torch.empty((B, wl.num_kv_heads, cfg.topk), dtype=torch.int32, device="cuda")
    ws_e = dev.ws(tbs.OP_SELECT_DECODE, B, B, n)
    ws_c = dev.ws(tbs.OP_SELECT_COARSE_DECODE, B, B, n)

    def time_calls(fn):
        for t in range(args.warmup):
            fn(t % R)
        torch.cuda.synchronize()
        flush_mall(torch)
        e0 = T.event()
        for t in range(args.steps):
            fn((args.warmup + t) % R)
        e1 = T.event()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / args.steps

    def exact(r, out_idx=idx):
        tbs.infv2_select_blocks(cfg, tbs.INFV2_MODE_DECODE, qs[r], B, 0, CKs[r], dev.ck_offsets,
                                dev.kv_offsets, dev.kv_lens, B, n, out_idx, None, ws_e)
    dec = {"workload": wl.name, "replicas": R, "exact_select_us": time_calls(exact)}
    ref_idx = []
    for r in range(R):
        e = torch.empty_like(idx)
        exact(r, e)
        ref_idx.append(e)
    ref_idx = torch.stack(ref_idx).cpu().numpy()
    for c in (64, 128, 256):
        ckc, ckc_off, _ = gh.coarse_ck(dev, c)
        CCs = [ckc] + [ckc.clone() for _ in range(R - 1)]

        def coarse(r, out_idx=idx, c=c, CCs=CCs, ckc_off=ckc_off):
            tbs.infv2_select_blocks_coarse(cfg, c, tbs.INFV2_MODE_DECODE, qs[r], B, 0, CKs[r],
                                           dev.ck_offsets, CCs[r], ckc_off, dev.kv_offsets,
                                           dev.kv_lens, B, n, out_idx, None, ws_c)
        us = time_calls(coarse)
        got = []
        for r in range(R):
            e = torch.empty_like(idx)
            coarse(r, e)
            got.append(e)
        same, shared = _agreement(torch.stack(got).cpu().numpy(), ref_idx)
        dec[f"coarse_{c}"] = {"select_us": us, "same_selection": same, "blocks_shared": shared}
        del CCs
    out["decode_128k"] = dec
    del CKs
    torch.cuda.empty_cache()
    # ---- prefill, 32K in 4096-row chunks (selection only; compressed keys built once)
    wp = make_config(3)
    devp = gh.DeviceWorkload(wp, args.ck_dtype)
    devp.compress()
    L, C = int(wp.lens[0]), wp.chunk
    hkv, k = wp.num_kv_heads, devp.cfg.topk
    idx_e = torch.empty((L, hkv, k), dtype=torch.int32, device="cuda")
    idx_c = torch.empty_like(idx_e)
    ws_p = devp.ws(tbs.OP_SELECT_COARSE_PREFILL, C, 1, L)

    def pre_exact():
        for q0 in range(0, L, C):
            q1 = min(L, q0 + C)
            tbs.infv2_select_blocks(devp.cfg, tbs.INFV2_MODE_PREFILL, devp.q[q0:q1], q1 - q0, q0,
                                    devp.ck, devp.ck_offsets, devp.kv_offsets, None, 1, q1,
                                    idx_e[q0:q1], None, ws_p)

    def time_once(fn):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(max(1, args.prefill_reps)):
            e0 = T.event(); fn(); e1 = T.event()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return float(np.median(ts))
    pre = {"workload": wp.name, "exact_select_ms": time_once(pre_exact)}
    ie = idx_e.cpu().numpy()
    scored = np.arange(L) // wp.block_size + 1 > k
    for c in (64, 128, 256):
        ckc, ckc_off, _ = gh.coarse_ck(devp, c)

        def pre_coarse(c=c, ckc=ckc, ckc_off=ckc_off):
            for q0 in range(0, L, C):
                q1 = min(L, q0 + C)
                tbs.infv2_select_blocks_coarse(devp.cfg, c, tbs.INFV2_MODE_PREFILL, devp.q[q0:q1],
                                               q1 - q0, q0, devp.ck, devp.ck_offsets, ckc, ckc_off,
                                               devp.kv_offsets, None, 1, q1, idx_c[q0:q1], None, ws_p)
        ms = time_once(pre_coarse)
        same, shared = _agreement(idx_c.cpu().numpy()[scored], ie[scored])
        pre[f"coarse_{c}"] = {"select_ms": ms, "same_selection": same, "blocks_shared": shared}
    out["prefill_32k"] = pre
    return out


def bench_batched(args, torch, tbs, gh, ck_dtype=None) -> dict:
    # one step reads ~170 MB: four replicas put 2x the Infinity Cache between two uses
    return bench_decode(4, args, torch, tbs, gh, replicas=args.replicas, ck_dtype=ck_dtype)


# ----------------------------------------------------------------------------- CPU oracle
def host_info() -> dict:
    """CPU model and the BLAS library NumPy uses, for the CPU-baseline record."""
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    blas = None
    try:
        cfg = np.show_config(mode="dicts")
        b = cfg.get("Build Dependencies", {}).get("blas", {})
        blas = " ".join(str(b.get(k)) for k in ("name", "version") if b.get(k))
    except Exception:  # pragma: no cover - reporting only
        pass
    try:
        import threadpoolctl
        apis = sorted({f"{x.get('internal_api')} ({x.get('threading_layer')})"
                       for x in threadpoolctl.threadpool_info() if x.get("user_api") == "blas"})
        if apis:
            blas = f"{blas}; runtime {', '.join(apis)}" if blas else ", ".join(apis)
    except Exception:  # pragma: no cover - reporting only
        pass
    return {"cpu_model": model, "blas": blas, "host_cpus": len(os.sched_getaffinity(0))}


def blas_threads() -> int:
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        return int(max([x.get("num_threads", 1) for x in info] + [1]))
    except Exception:  # pragma: no cover - reporting only
        return 1


def cpu_baseline_decode(seconds: float) -> dict:
    """Oracle decode steps at 128K (precomputed compressed keys as the cache state)."""
    from oracle import infv2_ref as ref
    from synth import make_config, extra_decode_queries, bf16_bits_to_f32
    wl = make_config(2)
    prm = ref.Params(head_dim=128, num_q_heads=32, num_kv_heads=2, block_size=64, kernel_size=32,
                     kernel_stride=16, topk=64, init_blocks=1, local_blocks=4)
    K, V = wl.k_f64(0), wl.v_f64(0)
    n = K.shape[1]
    ck = ref.compress_keys(K, 32, 16, "fp32")
    qs = bf16_bits_to_f32(extra_decode_queries(wl, 64)).astype(np.float64)
    t0 = time.perf_counter()
    steps = 0
    while True:
        q = qs[steps % qs.shape[0], 0]
        ref.compress_keys(K[:, n - 32:n], 32, 16, "fp32")           # the kernel the token completes
        for g in range(2):
            rs = ref.select_row(q[16 * g:16 * g + 16], ck[g], n - 1, prm)
            ref.attend_row(q[16 * g:16 * g + 16], K[g], V[g], n - 1, rs.sel, prm)
        steps += 1
        el = time.perf_counter() - t0
        if el >= seconds and steps >= 3:
            break
    return {"value": steps / el, "unit": "tok/s", "cores": blas_threads(), "kind": "oracle",
            **host_info(),
            "sample": f"{steps} decode steps of the 128K config (B=1), float64 NumPy, "
                      f"{el:.1f} s, cache state (compressed keys) precomputed"}


def cpu_baseline_prefill(seconds: float, pre: dict) -> dict:
    """Oracle prefill rows of the last 4096-row chunk of the 32K config."""
    from oracle import infv2_ref as ref
    wl = pre["_wl"]
    prm = ref.Params(head_dim=128, num_q_heads=32, num_kv_heads=2, block_size=64, kernel_size=32,
                     kernel_stride=16, topk=64, init_blocks=1, local_blocks=4)
    K, V = wl.k_f64(0), wl.v_f64(0)
    ck = ref.compress_keys(K, 32, 16, "fp32")
    q = wl.q_f64()
    L = q.shape[0]
    rng = np.random.default_rng(5)
    rows = rng.integers(L - wl.chunk, L, 4096)
    t0 = time.perf_counter()
    done = []
    for i in rows.tolist():
        for g in range(2):
            rs = ref.select_row(q[i, 16 * g:16 * g + 16], ck[g], i, prm)
            ref.attend_row(q[i, 16 * g:16 * g + 16], K[g], V[g], i, rs.sel, prm)
        done.append(i)
        if time.perf_counter() - t0 >= seconds and len(done) >= 4:
            break
    el = time.perf_counter() - t0
    gi = pre["_idx"][done]
    tok = attended_tokens(gi, np.array(done), np.full(len(done), L), 64)
    flops = float(4 * 128 * 16 * tok.sum())
    return {"value": flops / el / 1e12, "unit": "TFLOP/s", "cores": blas_threads(), "kind": "oracle",
            **host_info(),
            "sample": f"{len(done)} random rows of the last 4096-row chunk of the 32K prefill "
                      f"(selection + attention), {el:.1f} s; useful attention FLOPs / time"}


# ----------------------------------------------------------------------------- main
def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--replicas", type=int, default=0,
                    help="independent cache copies rotated per step; 0 (default): enough for "
                         "512 MiB between two uses of a copy (defeats the 256 MiB Infinity Cache)")
    ap.add_argument("--prefill-reps", type=int, default=3)
    ap.add_argument("--ck-dtype", default="fp32", choices=["fp32", "bf16"])
    ap.add_argument("--graph", type=int, default=1)
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-batched", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-loop", action="store_true", help="skip the append + select + attend loop record")
    ap.add_argument("--no-backward", action="store_true", help="skip the 32K training-backward record")
    ap.add_argument("--no-coarse", action="store_true", help="skip the coarse-kernel LSE selection record")
    ap.add_argument("--no-ck-bf16", action="store_true",
                    help="skip the extra decode records with bf16 compressed keys")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help=f"also run 8 device-to-device copies of {CALIBRATION_MIB} MiB (reference "
                         "kernel of known size for scaling the FETCH_SIZE / WRITE_SIZE counters)")
    ap.add_argument("--only", choices=["decode", "prefill", "batched", "backward", "coarse", "varlen",
                                       "loop"],
                    default=None,
                    help="run one workload only and print its record (for profiling)")
    ap.add_argument("--summarize-rocprof", nargs="+", metavar=("KIND", "CSV"), default=None,
                    help="fold rocprofv3 output into profiles/: 'stats <kernel_stats.csv> "
                         "<kernel_trace.csv>' or "
                         "'traffic <FETCH_SIZE counter_collection.csv> <WRITE_SIZE one>' "
                         "(no GPU; needs --workload and --command)")
    ap.add_argument("--workload", default=None, help="workload name for --summarize-rocprof")
    ap.add_argument("--command", default=None, help="the profiled command, recorded beside the figures")
    args = ap.parse_args()
    if args.summarize_rocprof:
        kind, paths = args.summarize_rocprof[0], args.summarize_rocprof[1:]
        if kind not in ("stats", "traffic") or len(paths) != 2 \
                or not args.workload or not args.command:
            ap.error("--summarize-rocprof stats STATS_CSV TRACE_CSV | traffic FETCH_CSV WRITE_CSV, "
                     "with --workload and --command")
        return summarize_rocprof(kind, args.workload, paths, args.command)
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path; "
              "run with --gpus 1.", file=sys.stderr)
        return 2

    import torch
    import trainable_block_sparse_amd as tbs
    from tests import gpu_harness as gh
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    tbs.load_library()
    torch.cuda.set_device(0)

    if args.copy_calibration:
        n = CALIBRATION_MIB * (1 << 20)
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(8):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log(f"copy calibration: 8 copies of {CALIBRATION_MIB} MiB")

    if args.only:
        if args.only == "decode":
            rec = bench_decode(2, args, torch, tbs, gh, replicas=args.replicas)
        elif args.only == "prefill":
            rec = {k: v for k, v in bench_prefill(args, torch, tbs, gh).items() if not k.startswith("_")}
        elif args.only == "coarse":
            rec = bench_coarse(args, torch, tbs, gh)
        elif args.only == "varlen":
            rec = bench_varlen_prefill(args, torch, tbs, gh)
        elif args.only == "loop":
            rec = bench_decode_loop(args, torch, tbs, gh)
        elif args.only == "backward":
            from synth import make_config
            rec = bench_backward(args, torch, tbs, gh, {"_wl": make_config(3)})
        else:
            rec = bench_batched(args, torch, tbs, gh)
        print(json.dumps({"only": args.only, "record": rec}))
        return 0

    main_res = bench_decode(2, args, torch, tbs, gh, replicas=args.replicas)
    log(f"decode 128K: {main_res['ms_per_step'] * 1e3:.1f} us/step, per call {main_res['per_call_us']}")
    pre = None if args.no_prefill else bench_prefill(args, torch, tbs, gh)
    if pre:
        log(f"prefill 32K: attn {pre['attn_ms']:.2f} ms, total {pre['total_ms']:.2f} ms "
            f"({pre['total_ms_endpoints']:.2f} ms between two events; two streams "
            f"{pre['total_ms_two_streams']:.2f} ms, equal: {pre['two_streams_equal']}), "
            f"{pre['tflops_attn']:.1f} TFLOPS")
    bat = None if args.no_batched else bench_batched(args, torch, tbs, gh)
    if bat:
        log(f"batched decode: {bat['ms_per_step'] * 1e3:.1f} us/step, per call {bat['per_call_us']}")
    varlen = None if args.no_prefill else bench_varlen_prefill(args, torch, tbs, gh)
    if varlen:
        log(f"varlen prefill 8 x 4K-16K: attn {varlen['attn_ms']:.2f} ms, total {varlen['total_ms']:.2f} ms, "
            f"{varlen['tflops_attn']:.1f} TFLOPS")
    bwd = None if (args.no_prefill or args.no_backward) else bench_backward(args, torch, tbs, gh, pre)
    if bwd:
        log(f"backward 32K (training, one call): {bwd['ms']:.2f} ms, {bwd['tflops']:.1f} TFLOPS "
            f"algorithmic; {bwd['parity']}")
    coarse = None if args.no_coarse else bench_coarse(args, torch, tbs, gh)
    if coarse:
        d2, p2 = coarse["decode_128k"], coarse["prefill_32k"]
        log(f"coarse LSE: decode select {d2['exact_select_us']:.1f} us exact vs "
            + ", ".join(f"{c}: {d2[f'coarse_{c}']['select_us']:.1f} us "
                        f"({d2[f'coarse_{c}']['blocks_shared']:.0%} shared)" for c in (64, 128, 256))
            + f"; prefill select {p2['exact_select_ms']:.2f} ms exact vs "
            + ", ".join(f"{c}: {p2[f'coarse_{c}']['select_ms']:.2f} ms" for c in (64, 128, 256)))
    loop = None if args.no_loop else bench_decode_loop(args, torch, tbs, gh)
    if loop:
        log(f"decode loop 128K (append + select + attend): {loop['ms_per_step_graph'] * 1e3:.1f} us/step; "
            f"one decode_step_append per token: {loop['ms_per_step_graph_step_append'] * 1e3:.1f} us/step")
    # the same decode workloads with bf16 compressed keys (the documented option)
    alt = {}
    out_pre_bf16 = None
    if not args.no_ck_bf16 and args.ck_dtype == "fp32":
        alt["decode_128k_ck_bf16"] = bench_decode(2, args, torch, tbs, gh, replicas=args.replicas,
                                                  ck_dtype="bf16")
        if not args.no_batched:
            alt["batched_decode_16x_ck_bf16"] = bench_batched(args, torch, tbs, gh, ck_dtype="bf16")
        if not args.no_prefill:
            pb = bench_prefill(args, torch, tbs, gh, ck_dtype="bf16")
            out_pre_bf16 = {k: v for k, v in pb.items() if not k.startswith("_")}
            log(f"prefill 32K, bf16 compressed keys: select {pb['select_ms']:.2f} ms, attn "
                f"{pb['attn_ms']:.2f} ms, total {pb['total_ms']:.2f} ms; {pb['parity']}")
        for k2, r2 in alt.items():
            log(f"{k2}: {r2['ms_per_step'] * 1e3:.1f} us/step")

    roof = main_res["roofline"]
    out = {
        "metric": METRIC,
        "value": main_res["tok_per_s"],
        "unit": "tok/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": main_res["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "decode_bf16_128k", "batch": 1, "context": 131072, "num_q_heads": 32,
                   "num_kv_heads": 2, "head_dim": 128, "block_size": 64, "kernel_size": 32,
                   "kernel_stride": 16, "topk": 64, "init_blocks": 1, "local_blocks": 4,
                   "ck_dtype": args.ck_dtype, "cache_replicas": main_res["replicas"],
                   "graph_replay": bool(args.graph)},
        "hbm_gbps": main_res["hbm_gbps_step"],
        "roofline": roof,
        "decode_128k": {k: v for k, v in main_res.items()},
    }
    if pre:
        out["prefill_32k"] = {k: v for k, v in pre.items() if not k.startswith("_")}
    if bat:
        out["batched_decode_16x"] = bat
    if loop:
        out["decode_loop_128k"] = loop
    if varlen:
        out["prefill_varlen_8x4k-16k"] = varlen
    if bwd:
        out["prefill_backward_32k"] = bwd
    if coarse:
        out["coarse_lse_selection"] = coarse
    for k2, r2 in alt.items():
        out[k2] = {x: r2[x] for x in ("workload", "batch", "ms_per_step", "tok_per_s", "hbm_gbps_step",
                                      "per_call_us", "kernels", "bytes_per_step", "roofline", "parity")}
    if out_pre_bf16:
        out["prefill_32k_ck_bf16"] = out_pre_bf16
    if not args.no_cpu_baseline:
        log("timing the CPU oracle")
        out["cpu_baseline"] = cpu_baseline_decode(args.cpu_seconds)
        if pre:
            out["prefill_32k"]["cpu_baseline"] = cpu_baseline_prefill(args.cpu_seconds, pre)
    print(json.dumps(out))
    return 0


if __name__ == "__main__":
    sys.exit(main())
