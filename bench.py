#!/usr/bin/env python3
"""Benchmark of the generalized paged-attention hot path on one MI355X.

One step = one pass of the whole path over one unified batch: plan the work
list (host) and upload it, append the step's new K/V rows into the paged
pools (kv_append), and run the attention of every query row over its
request's paged KV (attn_fwd).  The workload is the Llama-2-13B-shaped mixed
batch (40 heads, head_dim 128, fp16; 32 conversations with 16-128 new tokens
plus 32 decode requests, histories of 256-2048 tokens), generated from a
fixed seed and resident in HBM before the timed region starts.  Consecutive
steps alternate between two copies of the batch, so no step reads K/V or Q
left in the last-level cache by the step before.

Prints ONE JSON line with the headline metric (query tokens/s), a roofline
object for the dominant kernel (per-launch durations come from HIP events the
library records on its launch stream during the timed region; average, median
and shortest sampled launch), and the CPU oracle timed on this host (float32,
and float64) on a bounded sample of the same workload.

Beside the headline: the other workloads' attention calls, each timed as a
burst (40 calls after a short warm-up) and sustained (200 calls after 3 s of
back-to-back calls; their rooflines come from these), the long-context
workload also with a fixed 32-way split and unsplit, each with the oracle timed
on a bounded sample; the block swap; and the E4M3-pool lines.  `--only INDEX`
(with `--fp8`) measures one of these lines alone, exactly as the full run does,
for profiling runs.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import paged_kv_token_amd as pk  # noqa: E402
from workloads import config_batch  # noqa: E402

METRIC = "attn query-tokens/s + % HBM BW (decode) / % MFMA peak (prefill), 13B shape"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
MFMA_PEAK_TFLOPS = {"f16": 2500.0, "bf16": 2500.0, "f32": 157.3}   # dense MFMA (fp32: vector peak)
COUNTERS_FILE = os.path.join(ROOT, "profiles", "counters.json")
MIN_CPU_S = 10.0               # cpu_baseline times at least this much oracle work (within its budget)
KERNEL_SOURCES = {    # what a counter profile depends on: the kernel and the planner that orders its items
    "attn_mfma": ["attn_mfma.hip", "device_common.h", "api.cpp"],
    "attn_vector": ["attn_vector.hip", "device_common.h", "api.cpp"],
    "kv_append": ["kv_append.hip", "device_common.h"],
    "split_merge": ["split_merge.hip", "device_common.h"],
}


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def source_digest(kernel: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "paged_kv_token_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


# ---------------------------------------------------------------------------
# device-side batch
# ---------------------------------------------------------------------------
class DeviceBatch:
    """A seeded batch resident in HBM: pools filled with its cached history.

    `copies` independent copies of the pools, Q and O are kept and consecutive steps rotate
    through them, so a step's K/V and Q cannot still sit in the 256 MB last-level cache
    (MALL) from the step before (the working set of two copies exceeds it on every workload)."""

    def __init__(self, batch, copies: int = 2, kv_fp8=None):
        import torch
        self.b = b = batch
        td = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[b.dtype]
        self.td = td
        self.kv_fp8 = kv_fp8                      # (k_scale, v_scale): E4M3 pools
        self.kv_bytes = 1 if kv_fp8 else b.elem_bytes
        pd = torch.uint8 if kv_fp8 else td
        self.k_pool = torch.empty((b.num_blocks, b.num_kv_heads, 16, b.head_dim), dtype=pd, device="cuda")
        self.v_pool = torch.empty((b.num_blocks, b.num_kv_heads, 16, b.head_dim), dtype=pd, device="cuda")
        if kv_fp8:
            self.k_pool.fill_(0x7F)
            self.v_pool.fill_(0x7F)
        else:
            self.k_pool.fill_(float("nan"))
            self.v_pool.fill_(float("nan"))
        for r, k, v, slots, pos in b.iter_requests():
            if len(pos):
                self._append(self._dev(k[pos]), self._dev(v[pos]), self.k_pool, self.v_pool,
                             torch.from_numpy(slots.copy()).cuda())
        kn, vn = b.new_kv()
        self.k_new, self.v_new = self._dev(kn), self._dev(vn)
        self.new_slots = torch.from_numpy(b.new_slots.copy()).cuda()
        self.q = self._dev(b.q_all())
        self.o = torch.empty_like(self.q)
        self.bt = torch.from_numpy(b.block_tables.copy()).cuda()
        self.ctx = torch.from_numpy(b.context_lens.copy()).cuda()
        self.cu = torch.from_numpy(b.cu_q_lens.copy()).cuda()
        self.q_pos = None if b.has_default_positions else torch.from_numpy(b.q_pos.copy()).cuda()
        fp8 = {} if not kv_fp8 else dict(kv_dtype=pk.PENSIEVE_FP8_E4M3, k_scale=kv_fp8[0], v_scale=kv_fp8[1])
        self.desc = pk.make_desc(num_heads=b.num_heads, num_kv_heads=b.num_kv_heads, head_dim=b.head_dim,
                                 num_blocks=b.num_blocks, block_table_stride=b.block_table_stride,
                                 dtype={"f32": 0, "f16": 1, "bf16": 2}[b.dtype], softmax_scale=b.softmax_scale,
                                 context_lens_host=b.context_lens, cu_q_lens_host=b.cu_q_lens,
                                 q_pos_host=None if b.has_default_positions else b.q_pos, **fp8)
        self.ws = torch.empty(max(pk.pensieve_attn_workspace_size(self.desc), 256), dtype=torch.uint8, device="cuda")
        self.sets = [(self.k_pool, self.v_pool, self.q, self.o)]
        for _ in range(copies - 1):
            self.sets.append((self.k_pool.clone(), self.v_pool.clone(), self.q.clone(), torch.empty_like(self.o)))
        self.turn = 0
        torch.cuda.synchronize()

    def _next(self):
        s = self.sets[self.turn % len(self.sets)]
        self.turn += 1
        return s

    def _append(self, k, v, k_pool, v_pool, slots):
        if self.kv_fp8:
            pk.pensieve_kv_append_fp8(k, v, k_pool, v_pool, slots, self.kv_fp8[0], self.kv_fp8[1])
        else:
            pk.pensieve_kv_append(k, v, k_pool, v_pool, slots)

    def _dev(self, arr):
        import torch
        if self.b.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(np.ascontiguousarray(arr)).cuda()

    def step(self):
        """The whole path: append the step's new rows, then attention over the batch."""
        k_pool, v_pool, q, o = self._next()
        self._append(self.k_new, self.v_new, k_pool, v_pool, self.new_slots)
        pk.pensieve_attn_fwd(self.desc, q, k_pool, v_pool, self.bt, self.ctx, self.cu, self.q_pos, o, self.ws)

    def attn(self):
        k_pool, v_pool, q, o = self._next()
        pk.pensieve_attn_fwd(self.desc, q, k_pool, v_pool, self.bt, self.ctx, self.cu, self.q_pos, o, self.ws)

    def attn_no_split(self):
        """pensieve_attn_fwd with the adaptive split-KV turned off (every request whole)."""
        if not hasattr(self, "desc_ns"):
            b = self.b
            self.desc_ns = pk.make_desc(num_heads=b.num_heads, num_kv_heads=b.num_kv_heads, head_dim=b.head_dim,
                                        num_blocks=b.num_blocks, block_table_stride=b.block_table_stride,
                                        dtype={"f32": 0, "f16": 1, "bf16": 2}[b.dtype],
                                        softmax_scale=b.softmax_scale, context_lens_host=b.context_lens,
                                        cu_q_lens_host=b.cu_q_lens, flags=pk.PENSIEVE_FLAG_NO_SPLIT,
                                        q_pos_host=None if b.has_default_positions else b.q_pos)
        k_pool, v_pool, q, o = self._next()
        pk.pensieve_attn_fwd(self.desc_ns, q, k_pool, v_pool, self.bt, self.ctx, self.cu, self.q_pos, o, self.ws)

    def split_step(self, P, bufs):
        po, pm, pl, ws = bufs
        k_pool, v_pool, q, o = self._next()
        pk.pensieve_attn_split_partial(self.desc, P, q, k_pool, v_pool, self.bt, self.ctx, self.cu, self.q_pos,
                                       po, pm, pl, ws)
        pk.pensieve_attn_split_merge(po, pm, pl, o)

    def split_buffers(self, P):
        import torch
        b = self.b
        T = b.total_q
        return (torch.empty((T, b.num_heads, P, b.head_dim), dtype=torch.float32, device="cuda"),
                torch.empty((T, b.num_heads, P), dtype=torch.float32, device="cuda"),
                torch.empty((T, b.num_heads, P), dtype=torch.float32, device="cuda"),
                torch.empty(max(pk.pensieve_attn_workspace_size(self.desc, P), 256), dtype=torch.uint8,
                            device="cuda"))


# ---------------------------------------------------------------------------
# algorithmic work
# ---------------------------------------------------------------------------
def request_bytes(b, r: int, kv_bytes=None) -> int:
    """Bytes the method must move for request r: its K and V once per KV head (kv_bytes per
    element: the pools' type), its Q rows in and O rows out, its block-table entries, lengths
    and positions."""
    e = b.elem_bytes
    kb = e if kv_bytes is None else kv_bytes
    L, q = int(b.context_lens[r]), int(b.q_lens[r])
    nblk = -(-L // 16)
    kv = 2 * L * b.num_kv_heads * b.head_dim * kb
    qo = 2 * q * b.num_heads * b.head_dim * e
    meta = 4 * nblk + 8 + (0 if b.has_default_positions else 4 * q)
    return kv + qo + meta


PLAN_KERNELS = {0: "attn_vector", 1: "attn_mfma"}


def kernel_work(dev: DeviceBatch, kernel: str):
    """Algorithmic (bytes, flops) of the items one attention kernel serves, from the library's own plan.

    Bytes: each (request, KV head) the kernel touches reads its K and V once, up to the last key
    any of its rows may see, plus the Q and O rows of its items and the request's block-table
    entries, lengths and positions.  Flops: QK^T and PV over visible (row, key) pairs only."""
    b = dev.b
    e = b.elem_bytes
    plan = pk.pensieve_debug_plan(dev.desc, 0)
    keys, reqs = {}, set()
    nbytes = flops = 0
    pos_cache = {}
    for kern, r, g, q0, qc, part, nparts, cost, h0, hc in plan:
        if PLAN_KERNELS[int(kern)] != kernel or qc == 0:
            continue
        pos = pos_cache.setdefault(int(r), b.query_positions(int(r)))[q0:q0 + qc]
        keys[(r, g)] = max(keys.get((r, g), 0), int(pos.max()) + 1)
        reqs.add(int(r))
        nbytes += 2 * int(qc) * int(hc) * b.head_dim * e
        # keys of the item's partition (its share of the request's blocks) each row may see
        L = int(b.context_lens[r])
        per = -(-(-(-L // 16)) // int(nparts)) * 16
        k0, k1 = int(part) * per, min((int(part) + 1) * per, L)
        seen = np.clip(np.minimum(pos + 1, k1) - k0, 0, None)
        flops += 4 * b.head_dim * int(hc) * int(seen.sum())
    nbytes += sum(2 * k * b.head_dim * dev.kv_bytes for k in keys.values())
    for r in reqs:
        nbytes += 4 * (-(-int(b.context_lens[r]) // 16)) + 8 + (0 if b.has_default_positions else 4 * int(b.q_lens[r]))
    return nbytes, flops


def append_bytes(b, kv_bytes=None) -> int:
    """Read K/V new rows and write them into the pools (+ slot ids)."""
    kb = b.elem_bytes if kv_bytes is None else kv_bytes
    return 2 * b.total_q * b.num_kv_heads * b.head_dim * (b.elem_bytes + kb) + 4 * b.total_q


# ---------------------------------------------------------------------------
TRACE_EVERY = 4   # the library times every 4th launch of each kernel kind (a timed launch costs ~15 us)


def time_steps(fn, steps: int, warmup: int):
    """Warm up, then time exactly `steps` calls with library tracing on; returns (ms/step, trace).

    Tracing is already on during the warm-up (its events are then warm) and samples one launch in
    TRACE_EVERY of each kernel kind, so it adds about 1 % to a step."""
    import torch
    pk.pensieve_trace_enable(True, TRACE_EVERY)
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    pk.pensieve_trace_read()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    pk.pensieve_trace_enable(False)
    trace = pk.pensieve_trace_read()
    return (t1 - t0) * 1e3 / steps, trace


def summarize_trace(trace, steps: int):
    """Per kernel kind: sampled launches, their average, median and shortest duration, and the
    estimated time per step (each kind's launches are sampled one in TRACE_EVERY)."""
    per = {}
    for name, items, ms in trace:
        d = per.setdefault(name, {"launches": 0, "total_ms": 0.0, "items": items, "all": []})
        d["launches"] += 1
        d["total_ms"] += ms
        d["all"].append(ms)
    for d in per.values():
        d["avg_ms"] = d["total_ms"] / d["launches"]
        d["median_ms"] = float(np.median(d["all"]))
        d["min_ms"] = float(np.min(d["all"]))
        d["per_step_ms"] = d["total_ms"] * TRACE_EVERY / steps
        del d["all"]
    return per


def kernel_stats(per):
    """{kernel: {avg, median, min}} in ms, rounded, for the JSON line."""
    return {k: {"avg": round(v["avg_ms"], 4), "median": round(v["median_ms"], 4), "min": round(v["min_ms"], 4)}
            for k, v in per.items()}


SUSTAIN_S = 3.0    # seconds of back-to-back calls before a sustained measurement


def sustained(fn, steps: int, seconds: float):
    """Run fn back to back for `seconds` (the GPU settles at the clock it holds under continuous
    load), then time `steps` more calls as time_steps does."""
    import torch
    t_end = time.perf_counter() + seconds
    n = 0
    while time.perf_counter() < t_end:
        fn()
        n += 1
        if n % 64 == 0:
            torch.cuda.synchronize()
    ms, trace = time_steps(fn, steps, 5)
    return ms, trace, n


def roofline_for(b, dev, per, kernel: str, counters):
    if kernel in PLAN_KERNELS.values():
        nbytes, flops = kernel_work(dev, kernel)
    elif kernel == "kv_append":
        nbytes, flops = append_bytes(b, dev.kv_bytes), 0
    else:
        nbytes, flops = 0, 0
    avg_s = per[kernel]["avg_ms"] * 1e-3
    intensity = flops / nbytes if nbytes else 0.0
    ridge = MFMA_PEAK_TFLOPS[b.dtype] * 1e12 / (HBM_PEAK_GBS * 1e9)
    traffic = None
    if counters:
        c = counters.get(f"{kernel}@{b.name}" + ("" if dev.kv_fp8 is None else "@fp8"))
        if c and c.get("source_sha") == source_digest(kernel):
            traffic = c.get("traffic_bytes_per_launch")
    launches = {"avg_launch_ms": round(per[kernel]["avg_ms"], 4), "median_launch_ms": round(per[kernel]["median_ms"], 4),
                "min_launch_ms": round(per[kernel]["min_ms"], 4), "timed_launches": per[kernel]["launches"],
                "launch_sampling": f"1 in {TRACE_EVERY}"}
    if intensity < ridge:
        achieved = nbytes / avg_s / 1e9
        return {"kernel": kernel, "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "algorithmic_bytes": nbytes, "algorithmic_flops": flops, **launches}
    achieved = flops / avg_s / 1e12
    peak = MFMA_PEAK_TFLOPS[b.dtype]
    return {"kernel": kernel, "bound": "mfma", "achieved": round(achieved, 1), "peak": peak, "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4), "traffic": traffic, "algorithmic_bytes": nbytes,
            "algorithmic_flops": flops, **launches}


def load_counters():
    if not os.path.exists(COUNTERS_FILE):
        return {}
    with open(COUNTERS_FILE) as fh:
        return json.load(fh)


# ---------------------------------------------------------------------------
def copy_bandwidth(mib: int = 1024, reps: int = 10):
    """Achievable HBM bandwidth on this GPU: a device-to-device copy of `mib` MiB (read + write)."""
    import torch
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for _ in range(reps):
        dst.copy_(src)
    t1.record()
    torch.cuda.synchronize()
    gbs = 2 * n * reps / (t0.elapsed_time(t1) * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return {"gbs": round(gbs, 1), "frac_of_spec": round(gbs / HBM_PEAK_GBS, 4),
            "what": f"{mib} MiB device-to-device copy, bytes read + written"}


def swap_measure(index: int = 1, reps: int = 5, steps: int = 40):
    """Block swap with a pinned host tier on one workload: every block the batch uses goes out and
    comes back (GB/s each way over the host link); then attention steps run alone, and again with a
    swap-in on a second stream in every step (into spare device blocks) of as many blocks as the
    link carries in half a step: the swap should hide behind the attention."""
    import torch
    b = config_batch(index)
    dev = DeviceBatch(b, copies=1)
    used = b.used_blocks().astype(np.int32)
    n = len(used)
    k_host = torch.empty((n,) + tuple(dev.k_pool.shape[1:]), dtype=dev.k_pool.dtype).pin_memory()
    v_host = torch.empty((n,) + tuple(dev.v_pool.shape[1:]), dtype=dev.v_pool.dtype).pin_memory()
    host_ids = np.arange(n, dtype=np.int32)
    nbytes = 2 * n * b.num_kv_heads * 16 * b.head_dim * b.elem_bytes
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        t0.record()
        for _ in range(reps):
            fn()
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / reps

    out_ms = timed(lambda: pk.pensieve_kv_swap_out(dev.k_pool, dev.v_pool, k_host, v_host, used, host_ids))
    in_ms = timed(lambda: pk.pensieve_kv_swap_in(dev.k_pool, dev.v_pool, k_host, v_host, host_ids, used))
    spare = np.setdiff1d(np.arange(b.num_blocks), used).astype(np.int32)
    side = torch.cuda.Stream()
    block_bytes = 2 * b.num_kv_heads * 16 * b.head_dim * b.elem_bytes

    def steps_ms(m):
        """Wall time per step, both streams drained at the end."""
        torch.cuda.synchronize()
        w0 = time.perf_counter()
        for i in range(steps):
            if m:
                with torch.cuda.stream(side):
                    pk.pensieve_kv_swap_in(dev.k_pool, dev.v_pool, k_host, v_host, host_ids[:m], spare[:m],
                                           stream=side)
            dev.attn()
        torch.cuda.synchronize()
        return (time.perf_counter() - w0) * 1e3 / steps

    steps_ms(0)
    alone = steps_ms(0)
    m = int(min(len(spare), 0.5 * alone * 1e-3 * (nbytes / (in_ms * 1e-3)) / block_bytes))
    steps_ms(m)                                  # first use of the side stream and its launches
    beside = steps_ms(m)
    m_bytes = m * block_bytes
    out = {"workload": b.name, "blocks": n, "bytes": nbytes, "swap_out_ms": round(out_ms, 3),
           "swap_out_gbs": round(nbytes / (out_ms * 1e-3) / 1e9, 1), "swap_in_ms": round(in_ms, 3),
           "swap_in_gbs": round(nbytes / (in_ms * 1e-3) / 1e9, 1),
           "overlap": {"step_ms_alone": round(alone, 4), "step_ms_with_swap_in": round(beside, 4),
                       "swap_in_blocks_per_step": m, "swap_in_bytes_per_step": m_bytes}}
    del dev, k_host, v_host
    torch.cuda.empty_cache()
    return out


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown CPU"


def _blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        return 1


def cpu_baseline(b, budget_s: float, min_s: float = MIN_CPU_S, compute=np.float32):
    """The CPU oracle (as it stands) on this host: all requests, as many query heads as fit the budget,
    carried out in `compute` (float32, the precision the oracle is named in; float64 is the parity
    oracle's default)."""
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import oracle
    from oracle_helpers import oracle_pools
    threads = _blas_threads()
    pools = oracle_pools(b)
    q = b.q_all()
    qpos = None if b.has_default_positions else b.q_pos
    # Whole passes over the query heads, two heads at a time, until at least MIN_CPU_S of oracle
    # work (or the budget, if smaller) has been timed.
    done, elapsed = 0, 0.0
    chunk = 2
    min_s = min(min_s, budget_s)
    while elapsed < budget_s and (done < b.num_heads or elapsed < min_s):
        first = done % b.num_heads
        heads = list(range(first, min(first + chunk, b.num_heads)))
        t0 = time.perf_counter()
        oracle.paged_attention(q, pools[0], pools[1], b.block_tables, b.context_lens, b.cu_q_lens, qpos,
                               b.softmax_scale, b.dtype, heads=heads, compute=compute)
        elapsed += time.perf_counter() - t0
        done += len(heads)
    rate = b.total_q * (done / b.num_heads) / elapsed
    if done >= b.num_heads:
        what = f"all {b.num_reqs} requests x all {b.num_heads} query heads, {done / b.num_heads:.2f} passes"
    else:
        what = f"all {b.num_reqs} requests x query heads 0..{done - 1} of {b.num_heads} (rate scaled to all heads)"
    prec = "float32" if compute == np.float32 else "float64"
    return {"value": round(rate, 2), "unit": "query-tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{what} ({elapsed:.1f} s, {prec} NumPy on {cpu_model()})"}


def oracle_sample(b, reqs):
    """Pools and metadata holding only requests `reqs` of batch b (their own values, blocks renumbered
    0..n-1 in order), for timing the oracle on a bounded sample of a large workload."""
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import oracle
    from workloads import storage_dtype
    nblk = [b.num_logical_blocks(r) for r in reqs]
    sd = storage_dtype(b.dtype)
    kp = np.zeros((sum(nblk), b.num_kv_heads, 16, b.head_dim), sd)
    vp = np.zeros_like(kp)
    bt = np.zeros((len(reqs), max(nblk)), np.int32)
    qs, ctx, cu, qpos, off = [], [], [0], [], 0
    for i, r in enumerate(reqs):
        bt[i, :nblk[i]] = np.arange(off, off + nblk[i])
        off += nblk[i]
        k, v = b.request_kv(r)
        pos = np.arange(int(b.context_lens[r]))
        oracle.append_kv(kp, vp, k, v, (bt[i][pos // 16] * 16 + pos % 16).astype(np.int32), 16)
        qs.append(b.request_q(r))
        ctx.append(int(b.context_lens[r]))
        cu.append(cu[-1] + int(b.q_lens[r]))
        qpos.extend(b.query_positions(r).tolist())
    return (np.concatenate(qs), kp, vp, bt, np.array(ctx, np.int32), np.array(cu, np.int32),
            np.array(qpos, np.int32))


def cpu_baseline_sample(b, reqs, what: str, budget_s: float, split: int = 0):
    """The oracle (float32) on requests `reqs` of b, every query head, repeated until budget_s of
    oracle work; split > 0 times the split pair (partials over `split` partitions, then the merge)."""
    import oracle
    q, kp, vp, bt, ctx, cu, qpos = oracle_sample(b, reqs)
    rows = int(cu[-1])
    elapsed, passes = 0.0, 0
    while passes == 0 or elapsed < budget_s:
        t0 = time.perf_counter()
        if split:
            po, pm, pl = oracle.split_partial(q, kp, vp, bt, ctx, cu, qpos, b.softmax_scale, b.dtype, split,
                                              compute=np.float32)
            oracle.split_merge(po, pm, pl, compute=np.float32)
        else:
            oracle.paged_attention(q, kp, vp, bt, ctx, cu, qpos, b.softmax_scale, b.dtype, compute=np.float32)
        elapsed += time.perf_counter() - t0
        passes += 1
    how = f"split into {split} partitions + merge" if split else "unsplit"
    return {"value": round(rows * passes / elapsed, 2), "unit": "query-tokens/s", "cores": _blas_threads(),
            "kind": "oracle", "sample": f"{what}, all {b.num_heads} query heads, {how}: {passes} passes in "
                                        f"{elapsed:.1f} s (float32 NumPy on {cpu_model()})"}


def cpu_single_thread(budget_s: float = 3.0):
    """The oracle with its BLAS limited to one thread on bounded samples of the tiny, 13B mixed and
    decode-heavy workloads (their first requests, every query head), rates per query token."""
    from threadpoolctl import threadpool_limits
    out = []
    for index, cut, what in ((0, {}, "all 3 requests"), (1, dict(num_reqs=8), "first 8 conversations + first 8 decode requests"),
                             (2, dict(num_reqs=32), "first 32 of 256 requests")):
        b = config_batch(index, **cut)
        with threadpool_limits(limits=1):
            r = cpu_baseline(b, budget_s, min_s=budget_s)
        r["cores"] = 1
        r["workload"] = b.name
        r["sample"] = f"{what}: " + r["sample"]
        out.append(r)
    return out


# Bounded oracle samples of the other workloads: (requests, description).
CPU_SAMPLES = {2: (list(range(8)), "first 8 of 256 decode requests"),
               3: ([0, 1], "first 2 of 48 requests"),
               4: ([0, 2], "requests 0 (32768 history, 1 new row) and 2 (49152 history, 512 new rows)")}


def secondary(index: int, steps: int, warmup: int, counters, sustain_s: float = SUSTAIN_S, cpu_budget: float = 0.0,
              extras: bool = True):
    """Other workloads of the same path (attention calls alone), reported beside the headline.

    Each is timed twice: a burst of `steps` calls after a short warm-up, and `steps` calls after
    sustain_s seconds of back-to-back calls (the clock the chip holds under continuous load);
    the roofline is taken from the sustained calls."""
    import torch
    b = config_batch(index)
    dev = DeviceBatch(b)
    out = {"workload": b.name, "total_q": b.total_q}
    total_bytes = sum(request_bytes(b, r) for r in range(b.num_reqs))
    burst = min(steps, BURST_CALLS)
    ms_b, trace_b = time_steps(dev.attn, burst, warmup)
    per_b = summarize_trace(trace_b, burst)
    ms, trace, warm_calls = sustained(dev.attn, steps, sustain_s)
    per = summarize_trace(trace, steps)
    attn = {k: v for k, v in per.items() if k.startswith("attn")}
    dom = max(attn, key=lambda k: attn[k]["total_ms"])
    out["attn_ms"] = round(ms, 4)
    out["query_tokens_per_s"] = round(b.total_q / (ms * 1e-3), 1)
    out["kernels_ms"] = kernel_stats(per)
    out["timed"] = f"{steps} calls after {warm_calls} back-to-back calls ({sustain_s:g} s)"
    out["roofline"] = roofline_for(b, dev, per, dom, counters)
    # The whole call against HBM: every request's K/V, Q, O and metadata once, over the call's time.
    out["attn_hbm_frac"] = round(total_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
    out["burst"] = {"timed": f"{burst} calls after {warmup} warm-up calls", "attn_ms": round(ms_b, 4),
                    "kernels_ms": kernel_stats(per_b),
                    "roofline_frac": roofline_for(b, dev, per_b, dom, None)["frac"]}
    if index == 4 and extras:
        bufs = dev.split_buffers(32)
        ms2, trace2 = time_steps(lambda: dev.split_step(32, bufs), steps, warmup)
        per2 = summarize_trace(trace2, steps)
        out["split32_ms"] = round(ms2, 4)
        out["split32_kernels_ms"] = kernel_stats(per2)
        out["split32_hbm_frac"] = round(total_bytes / (ms2 * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
        del bufs
        ms3, trace3 = time_steps(dev.attn_no_split, steps, warmup)
        per3 = summarize_trace(trace3, steps)
        out["no_split_ms"] = round(ms3, 4)
        out["no_split_kernels_ms"] = kernel_stats(per3)
        out["no_split_hbm_frac"] = round(total_bytes / (ms3 * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
    del dev
    torch.cuda.empty_cache()
    if cpu_budget > 0 and index in CPU_SAMPLES:
        reqs, what = CPU_SAMPLES[index]
        log(f"cpu_baseline (oracle) on {b.name}: {what}")
        out["cpu_baseline"] = cpu_baseline_sample(b, reqs, what, cpu_budget)
        if index == 4:
            out["cpu_baseline_split32"] = cpu_baseline_sample(b, reqs, what, cpu_budget, split=32)
    return out


FP8_SCALES = (1 / 128, 1 / 128)   # the workloads' K/V (0.5 N(0,1)) stay below 3, i.e. codes below 384


def fp8_measure(index: int, steps: int, warmup: int, full_step: bool, counters=None):
    """The same workload with E4M3 pools: whole step (append + attention) or attention alone."""
    import torch
    b = config_batch(index)
    dev = DeviceBatch(b, kv_fp8=FP8_SCALES)
    ms, trace = time_steps(dev.step if full_step else dev.attn, steps, warmup)
    per = summarize_trace(trace, steps)
    attn = {k: v for k, v in per.items() if k.startswith("attn")}
    dom = max(attn, key=lambda k: attn[k]["total_ms"])
    out = {"workload": b.name, "kv_dtype": "fp8_e4m3", "scales": list(FP8_SCALES),
           "timed": "step (append + attention)" if full_step else "attention",
           "ms": round(ms, 4), "query_tokens_per_s": round(b.total_q / (ms * 1e-3), 1),
           "kernels_ms": kernel_stats(per),
           "roofline": roofline_for(b, dev, per, dom, counters)}
    attn_ms = sum(v["per_step_ms"] for v in attn.values())
    total_bytes = sum(request_bytes(b, r, 1) for r in range(b.num_reqs))
    out["attn_total"] = {"ms": round(attn_ms, 4), "bytes": total_bytes,
                         "hbm_frac": round(total_bytes / (attn_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    del dev
    torch.cuda.empty_cache()
    return out


def split_sweep(steps: int = 20, warmup: int = 3):
    """Split-KV crossover on long-context decode batches: the adaptive plan of pensieve_attn_fwd
    against never splitting and against a fixed 32-way split, as the number of long requests
    grows (timing only: pools hold device-side random values, 40/40 heads, d = 128, bf16)."""
    import torch
    H, heads, d = 32768, 40, 128
    cases = [(r, 0) for r in (1, 2, 4, 8, 16, 32)] + [(8, 24)]    # (long requests, short ones)
    rows = []
    for n_long, n_short in cases:
        ctx = np.array([H + 1] * n_long + [1024 + 1] * n_short, dtype=np.int32)
        R = len(ctx)
        cu = np.arange(R + 1, dtype=np.int32)
        nblk = -(-ctx // 16)
        NB = int(nblk.sum())
        gen = torch.Generator(device="cuda").manual_seed(7)
        perm = torch.randperm(NB, device="cuda", generator=gen).to(torch.int32)
        stride = int(nblk.max())
        bt = torch.zeros((R, stride), dtype=torch.int32, device="cuda")
        off = 0
        for r in range(R):
            bt[r, :nblk[r]] = perm[off:off + nblk[r]]
            off += int(nblk[r])
        kp = torch.randn((NB, heads, 16, d), device="cuda", dtype=torch.bfloat16, generator=gen) * 0.5
        vp = torch.randn((NB, heads, 16, d), device="cuda", dtype=torch.bfloat16, generator=gen) * 0.5
        q = torch.randn((R, heads, d), device="cuda", dtype=torch.bfloat16, generator=gen) * 0.5
        o = torch.empty_like(q)
        ctx_d, cu_d = torch.from_numpy(ctx).cuda(), torch.from_numpy(cu).cuda()
        mk = lambda flags: pk.make_desc(num_heads=heads, num_kv_heads=heads, head_dim=d, num_blocks=NB,
                                        block_table_stride=stride, dtype=pk.PENSIEVE_BF16,
                                        softmax_scale=1 / math.sqrt(d), context_lens_host=ctx, cu_q_lens_host=cu,
                                        flags=flags)
        d_ad, d_ns = mk(0), mk(pk.PENSIEVE_FLAG_NO_SPLIT)
        ws_bytes = max(pk.pensieve_attn_workspace_size(d_ad), pk.pensieve_attn_workspace_size(d_ad, 32), 256)
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
        po = torch.empty((R, heads, 32, d), dtype=torch.float32, device="cuda")
        pm = torch.empty((R, heads, 32), dtype=torch.float32, device="cuda")
        pl = torch.empty((R, heads, 32), dtype=torch.float32, device="cuda")
        plan = pk.pensieve_debug_plan(d_ad)
        parts = sorted({int(x[6]) for x in plan if x[4] > 0})

        def fixed32():
            pk.pensieve_attn_split_partial(d_ad, 32, q, kp, vp, bt, ctx_d, cu_d, None, po, pm, pl, ws)
            pk.pensieve_attn_split_merge(po, pm, pl, o)
        t_ad, _ = time_steps(lambda: pk.pensieve_attn_fwd(d_ad, q, kp, vp, bt, ctx_d, cu_d, None, o, ws), steps, warmup)
        t_ns, _ = time_steps(lambda: pk.pensieve_attn_fwd(d_ns, q, kp, vp, bt, ctx_d, cu_d, None, o, ws), steps, warmup)
        t_32, _ = time_steps(fixed32, steps, warmup)
        kv = 2 * int(ctx.sum()) * heads * d * 2
        row = {"long_requests": n_long, "short_requests": n_short, "adaptive_partitions": parts,
               "adaptive_ms": round(t_ad, 4), "no_split_ms": round(t_ns, 4), "split32_ms": round(t_32, 4),
               "adaptive_hbm_frac": round(kv / (t_ad * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        log(json.dumps(row))
        rows.append(row)
        del kp, vp, q, o, ws, po, pm, pl, bt
        torch.cuda.empty_cache()
    return rows


def routing_sweep(steps: int = 20, warmup: int = 3):
    """Decode rows of GQA groups on the two kernels: 128 decode requests of 2048 history tokens, 8
    KV heads of 1, 2, 4 or 8 query heads each, d = 128, bf16 (timing only: pools hold device-side
    random values).  pensieve_attn_fwd's default routing (the matrix cores from groups of 4) against
    PENSIEVE_FLAG_VECTOR_ONLY; K/V bytes over time as TB/s."""
    import torch
    R, hist, hkv, d = 128, 2048, 8, 128
    rows = []
    for G in (1, 2, 4, 8):
        heads = hkv * G
        ctx = np.full(R, hist + 1, dtype=np.int32)
        cu = np.arange(R + 1, dtype=np.int32)
        nblk = -(-ctx // 16)
        NB = int(nblk.sum())
        gen = torch.Generator(device="cuda").manual_seed(11)
        perm = torch.randperm(NB, device="cuda", generator=gen).to(torch.int32)
        stride = int(nblk.max())
        bt = perm.reshape(R, stride).contiguous()
        kp = torch.randn((NB, hkv, 16, d), device="cuda", dtype=torch.bfloat16, generator=gen) * 0.5
        vp = torch.randn((NB, hkv, 16, d), device="cuda", dtype=torch.bfloat16, generator=gen) * 0.5
        q = torch.randn((R, heads, d), device="cuda", dtype=torch.bfloat16, generator=gen) * 0.5
        o = torch.empty_like(q)
        ctx_d, cu_d = torch.from_numpy(ctx).cuda(), torch.from_numpy(cu).cuda()
        mk = lambda flags: pk.make_desc(num_heads=heads, num_kv_heads=hkv, head_dim=d, num_blocks=NB,
                                        block_table_stride=stride, dtype=pk.PENSIEVE_BF16,
                                        softmax_scale=1 / math.sqrt(d), context_lens_host=ctx, cu_q_lens_host=cu,
                                        flags=flags | pk.PENSIEVE_FLAG_NO_SPLIT)
        d_def, d_vec = mk(0), mk(pk.PENSIEVE_FLAG_VECTOR_ONLY)
        ws = torch.empty(max(pk.pensieve_attn_workspace_size(d_def), pk.pensieve_attn_workspace_size(d_vec), 256),
                         dtype=torch.uint8, device="cuda")
        kernel = "matrix" if any(int(x[0]) == 1 for x in pk.pensieve_debug_plan(d_def)) else "vector"
        t_def, _ = time_steps(lambda: pk.pensieve_attn_fwd(d_def, q, kp, vp, bt, ctx_d, cu_d, None, o, ws), steps, warmup)
        t_vec, _ = time_steps(lambda: pk.pensieve_attn_fwd(d_vec, q, kp, vp, bt, ctx_d, cu_d, None, o, ws), steps, warmup)
        kv = 2 * int(ctx.sum()) * hkv * d * 2
        row = {"group": G, "default_kernel": kernel, "default_ms": round(t_def, 4),
               "default_tbs": round(kv / (t_def * 1e-3) / 1e12, 2), "vector_only_ms": round(t_vec, 4),
               "vector_only_tbs": round(kv / (t_vec * 1e-3) / 1e12, 2)}
        log(json.dumps(row))
        rows.append(row)
        del kp, vp, q, o, ws, bt
        torch.cuda.empty_cache()
    return rows


def headline(b, steps: int, warmup: int, counters):
    """The headline bench line: whole steps (append + attention) on workload b."""
    import torch
    dev = DeviceBatch(b)
    ms, trace = time_steps(dev.step, steps, warmup)
    per = summarize_trace(trace, steps)
    dom = max(per, key=lambda k: per[k]["total_ms"])
    log(f"{ms:.4f} ms/step; kernels (one launch in {TRACE_EVERY} timed): " +
        ", ".join(f"{k} {v['avg_ms']:.4f} ms x{v['launches'] * TRACE_EVERY / steps:g}" for k, v in per.items()))
    result = {
        "metric": METRIC, "value": round(b.total_q / (ms * 1e-3), 1), "unit": "query-tokens/s",
        "n_gpus": 1, "steps": steps, "warmup": warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": b.dtype, "data": "synthetic",
        "config": {"workload": b.name, "requests": b.num_reqs, "decode_requests": int((b.new_lens == 1).sum()),
                   "total_q": b.total_q, "context_tokens": int(b.context_lens.sum()), "num_heads": b.num_heads,
                   "num_kv_heads": b.num_kv_heads, "head_dim": b.head_dim, "block_size": 16, "seed": b.seed},
        "roofline": roofline_for(b, dev, per, dom, counters),
        "kernels_ms": {k: round(v["avg_ms"], 4) for k, v in per.items()},
        "kernel_launch_stats_ms": kernel_stats(per),
    }
    if "kv_append" in per:
        ab = append_bytes(b)
        result["kv_append"] = {"bytes": ab, "avg_ms": round(per["kv_append"]["avg_ms"], 4),
                               "hbm_frac": round(ab / (per["kv_append"]["avg_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    # The attention as a whole (both kernels) against the HBM roofline.
    attn_ms = sum(v["per_step_ms"] for k, v in per.items() if k.startswith("attn"))
    total_bytes = sum(request_bytes(b, r) for r in range(b.num_reqs))
    result["attn_total"] = {"ms": round(attn_ms, 4), "bytes": total_bytes,
                            "hbm_frac": round(total_bytes / (attn_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    del dev
    torch.cuda.empty_cache()
    return result


BURST_CALLS = 40    # burst figure of the other workloads: the first calls after a short warm-up


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", type=int, default=1, help="index of the seeded workload to time (default: the "
                    "Llama-2-13B mixed batch); other indices are for profiling runs")
    ap.add_argument("--cpu-budget", type=float, default=20.0, help="seconds of oracle work for cpu_baseline")
    ap.add_argument("--secondary-cpu-budget", type=float, default=5.0,
                    help="seconds of oracle work for each other workload's cpu_baseline")
    ap.add_argument("--no-cpu", action="store_true", help="skip the cpu_baseline leg")
    ap.add_argument("--no-secondary", action="store_true", help="skip the other workloads")
    ap.add_argument("--no-hbm-copy", action="store_true", help="skip the device-copy bandwidth measurement")
    ap.add_argument("--sustain-s", type=float, default=SUSTAIN_S,
                    help="seconds of back-to-back calls before the other workloads' sustained measurement")
    ap.add_argument("--only", type=int, default=None, metavar="INDEX",
                    help="measure one bench line alone, exactly as the full run does (the headline line for the "
                         "headline workload, else that workload's secondary line without its extra unsplit and "
                         "32-way lines), print it and exit: for profiling runs")
    ap.add_argument("--fp8", action="store_true", help="with --only: the E4M3-pool line of that workload")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="first copy MIB MiB device-to-device (a reference kernel for HBM counters)")
    ap.add_argument("--split-sweep", action="store_true",
                    help="only measure the split-KV crossover on long-context decode batches and exit")
    ap.add_argument("--routing-sweep", action="store_true",
                    help="only measure GQA decode rows on the matrix cores against the vector kernel and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the path needs no collective); --gpus {args.gpus} is not run.",
              file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    pk.load_library()
    if args.split_sweep:
        print(json.dumps({"split_sweep": split_sweep()}), flush=True)
        return
    if args.routing_sweep:
        print(json.dumps({"routing_sweep": routing_sweep()}), flush=True)
        return
    counters = load_counters()
    if args.copy_calibration > 0:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(2):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"calibration copy: {args.copy_calibration} MiB x 2")
        del src, dst

    def fp8_line(idx):
        head = idx == args.workload
        return fp8_measure(idx, args.steps if head else BURST_CALLS, args.warmup if head else 5, full_step=head,
                           counters=counters)

    if args.only is not None:
        log(f"one bench line: workload {args.only}{' with E4M3 pools' if args.fp8 else ''}")
        if args.fp8:
            line = fp8_line(args.only)
        elif args.only == args.workload:
            line = headline(config_batch(args.only), args.steps, args.warmup, counters)
        else:
            line = secondary(args.only, args.steps, 5, counters, args.sustain_s, extras=False)
        print(json.dumps(line), flush=True)
        return

    b = config_batch(args.workload)
    log(f"workload {b.name}: R={b.num_reqs} T={b.total_q} context tokens={int(b.context_lens.sum())}")
    result = headline(b, args.steps, args.warmup, counters)
    result["hbm_copy"] = None if args.no_hbm_copy else copy_bandwidth()
    if not args.no_secondary:
        log("block swap with a pinned host tier")
        result["kv_swap"] = swap_measure()
        result["secondary"] = []
        for idx in (2, 3, 4):
            log(f"secondary workload {idx}")
            result["secondary"].append(secondary(idx, args.steps, 5, counters, args.sustain_s,
                                                 0.0 if args.no_cpu else args.secondary_cpu_budget))
        result["fp8_kv"] = []
        for idx in (1, 2, 3):
            log(f"fp8 KV pools, workload {idx}")
            result["fp8_kv"].append(fp8_line(idx))
    if not args.no_cpu:
        log("cpu_baseline (oracle, float32)")
        result["cpu_baseline"] = cpu_baseline(b, args.cpu_budget)
        log("cpu_baseline (oracle, float64)")
        result["cpu_baseline_f64"] = cpu_baseline(b, min(args.cpu_budget, 10.0), compute=np.float64)
        log("oracle on one thread (tiny, 13B mixed and decode-heavy samples)")
        result["cpu_single_thread"] = cpu_single_thread()
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
