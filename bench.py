"""Benchmark of paged varlen attention on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--secondary/--no-secondary]
                    [--no-cpu-baseline] [--copy-calibration]

Headline workload: the GQA decode batch -- 32 requests with one query token
each, context U[512, 4096], Hq=32 Hkv=8 D=128, 16-token pages shuffled over a
16,384-block pool, bf16.  One step is the whole decode hot path on that batch:
pa_reshape_and_cache of the 32 new K/V rows, pa_varlen_attention with 512-token
split-KV partitions, and pa_split_kv_reduce.  ``value`` is the step's
algorithmic HBM bytes (every visible KV row once per KV head, Q in, O out, the
cache write, table ints) divided by the step's wall time.

Inputs are resident in HBM before timing starts.  Each step is captured once
as a HIP graph and the timed region replays the graphs back to back, so host
launch overhead does not starve the GPU.  The steps cycle over several
identical copies of the KV pool so that no step finds the previous step's
pages in the 256 MB last-level cache (MALL); the "warm" figure (one copy) is
reported beside it.

``roofline`` times the dominant kernel (the decode attention launch) with HIP
events on the stream it runs on.  ``cpu_baseline`` times the fp64 oracle on
the same workload on this host's cores.  ``secondary`` holds the other
workloads of the metric: long-context split-KV decode, the two decode batches
over 8-bit E4M3 caches (half the KV bytes), the mixed prefill and
speculative-verify batches (MFMA TFLOP/s), a uniform long-prompt prefill batch
of the mixed batches' head shape that shows the tiled kernel's steady state
apart from the load imbalance of short ragged batches, and the KV block
offload rate.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0
METRIC = "paged-attn decode HBM GB/s (% of peak) + prefill TFLOP/s (% MFMA peak), 1 GPU"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


class Step:
    """One pass of the hot path over one batch, on the current stream,
    bracketed by events so each kernel's duration can be read back."""

    def __init__(self, w, partition_size, copies, device, write_cache, kv8=False):
        import torch
        import paged_varlen_attention_amd as pa
        self.w = w
        self.P = partition_size
        self.pa = pa
        self.device = device
        self.q = w.q.to(device)
        self.cu = w.cu_seqlens_q.to(device)
        self.sl = w.seq_lens.to(device)
        bt = w.block_tables.to(device)
        self.ratio = w.kernel_page_ratio
        self.bt_src = bt
        self.bt = pa.expand_block_tables(bt, self.ratio) if self.ratio > 1 else bt
        self.pools = []
        self.k_scale = self.v_scale = None
        if kv8:  # 8-bit pools: the workload's bf16 pool quantised by the library's cache write
            import workloads as W
            ks, vs = W.kv_scales(17, w.num_kv_heads)
            self.k_scale, self.v_scale = ks.to(device), vs.to(device)
            nb, bs, hkv, d = w.key_cache.shape
            all_slots = torch.arange(nb * bs, dtype=torch.int64, device=device)
        for _ in range(copies):
            kc = w.key_cache.to(device)
            vc = w.value_cache.to(device)
            if kv8:
                k8 = torch.empty(kc.shape, dtype=torch.uint8, device=device)
                v8 = torch.empty_like(k8)
                pa.reshape_and_cache(kc.view(nb * bs, hkv, d), vc.view(nb * bs, hkv, d), k8, v8,
                                     all_slots, k_scale=self.k_scale, v_scale=self.v_scale)
                torch.cuda.synchronize()
                del kc, vc
                kc, vc = k8, v8
            self.pools.append((kc, vc))
        self.write_cache = write_cache
        if self.write_cache:
            if w.slot_mapping is not None:
                nk, nv, sm = w.new_key, w.new_value, w.slot_mapping
            else:  # decode: the new tokens are already in the cache; write them again
                import workloads as W
                nk, nv, sm = W.last_token_rows(w)
            self.new_k, self.new_v, self.slots = nk.to(device), nv.to(device), sm.to(device)
            self.cache_write_rows = int(sm.numel())
        self.out = torch.empty_like(self.q)
        self.partials = None
        if self.P:
            mp = pa.max_partitions(w.max_seq_len, self.P)
            self.partials = pa.alloc_partials(w.total_q, w.num_q_heads, w.head_dim, mp, device)
        self.i = 0
        self.events = []

    def kernel_view(self, kc, vc):
        if self.ratio == 1:
            return kc, vc
        nb, bs, hkv, d = kc.shape
        return (kc.view(nb * self.ratio, bs // self.ratio, hkv, d),
                vc.view(nb * self.ratio, bs // self.ratio, hkv, d))

    def __call__(self, record=False, pool=None):
        """Enqueue one step on the current stream (pool: which KV-pool copy)."""
        import torch
        pa, w = self.pa, self.w
        if pool is None:
            pool = self.i % len(self.pools)
            self.i += 1
        kc, vc = self.pools[pool]
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(5)] if record else None
        if record:
            ev[0].record()
        if self.write_cache:
            pa.reshape_and_cache(self.new_k, self.new_v, kc, vc, self.slots,
                                 k_scale=self.k_scale, v_scale=self.v_scale)
        if record:
            ev[1].record()
        if self.ratio > 1:
            pa.expand_block_tables(self.bt_src, self.ratio, out=self.bt)
        if record:
            ev[2].record()
        kkc, kvc = self.kernel_view(kc, vc)
        pa.varlen_attention(self.q, kkc, kvc, self.cu, self.sl, self.bt, max_q_len=w.max_q_len,
                            max_seq_len=w.max_seq_len, scale=w.scale, partition_size=self.P,
                            out=self.out, partials=self.partials, reduce=False,
                            k_scale=self.k_scale, v_scale=self.v_scale)
        if record:
            ev[3].record()
        if self.P:
            pa.split_kv_reduce(self.out, self.partials, self.cu, self.sl, self.P)
        if record:
            ev[4].record()
            self.events.append(ev)

    def attention(self, pool):
        """Enqueue the attention launch alone (KV-pool copy `pool`)."""
        w = self.w
        kkc, kvc = self.kernel_view(*self.pools[pool])
        self.pa.varlen_attention(self.q, kkc, kvc, self.cu, self.sl, self.bt, max_q_len=w.max_q_len,
                                 max_seq_len=w.max_seq_len, scale=w.scale, partition_size=self.P,
                                 out=self.out, partials=self.partials, reduce=False,
                                 k_scale=self.k_scale, v_scale=self.v_scale)

    def capture(self):
        """One HIP graph per KV-pool copy, each holding a whole step."""
        import torch
        for i in range(len(self.pools)):  # warm the path before capture
            self(pool=i)
        torch.cuda.synchronize()
        self.graphs = []
        for i in range(len(self.pools)):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                self(pool=i)
            self.graphs.append(g)
        torch.cuda.synchronize()

    def replay(self, k):
        self.graphs[k % len(self.graphs)].replay()

    def kernel_ms(self):
        """Mean durations (ms) of: cache write, table view (only where the
        step launches one), attention, reduce."""
        n = len(self.events)
        if not n:
            return {}
        tot = [0.0] * 4
        for ev in self.events:
            for k in range(4):
                tot[k] += ev[k].elapsed_time(ev[k + 1])
        names = ("cache_write", "table_view", "attention", "reduce")
        return {k: t / n for k, t in zip(names, tot) if k != "table_view" or self.ratio > 1}


def step_bytes(w, include_cache_write, kv_elt_bytes=None):
    ke = w.elt_bytes if kv_elt_bytes is None else kv_elt_bytes
    b = w.algorithmic_bytes(ke)
    if include_cache_write:
        n = int((w.slot_mapping >= 0).sum()) if w.slot_mapping is not None else w.total_q
        # K and V rows: read at the row type, written at the cache type
        b += 2 * n * w.num_kv_heads * w.head_dim * (w.elt_bytes + ke)
    return b


def time_graph_steps(step, steps, warmup):
    """Wall time per step of `steps` graph replays, bracketed by synchronize."""
    import torch
    for k in range(warmup):
        step.replay(k)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        step.replay(k)
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps


def step_percentiles(step, reps):
    """p10 / p50 / p90 (ms) of single graph replays, each bracketed by its own
    events on the current stream."""
    import torch
    ts = []
    for k in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        step.replay(k)
        e1.record()
        ts.append((e0, e1))
    torch.cuda.synchronize()
    v = sorted(a.elapsed_time(b) for a, b in ts)
    pick = lambda q: v[min(len(v) - 1, int(q * (len(v) - 1) + 0.5))]  # noqa: E731
    return {"p10": round(pick(0.1), 5), "p50": round(pick(0.5), 5), "p90": round(pick(0.9), 5)}


def time_kernels(step, reps):
    """Per-kernel durations from HIP events on the launch stream (eager launches)."""
    import torch
    step.events.clear()
    for _ in range(reps):
        step(record=True)
    torch.cuda.synchronize()
    return step.kernel_ms()


def time_attention_b2b(step, reps):
    """Mean duration (ms) of the attention launch alone: `reps` launches back to
    back on the current stream (cycling the KV-pool copies, so every launch
    reads cold pages) between two HIP events.  Unlike the evented eager step,
    no launch waits for the host, so this matches the kernel's own duration
    plus the dispatch gap between consecutive kernels."""
    import torch
    for k in range(3):
        step.attention(k % len(step.pools))
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for k in range(reps):
        step.attention(k % len(step.pools))
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def measure(w, P, steps, warmup, copies, device, write_cache=True, kv8=False):
    step = Step(w, P, copies, device, write_cache, kv8)
    step.capture()
    sec = time_graph_steps(step, steps, warmup)
    pct = step_percentiles(step, max(10, steps))
    km = time_kernels(step, max(10, steps // 2))
    km["attention_back_to_back"] = time_attention_b2b(step, max(20, steps))
    km["step_ms_percentiles"] = pct
    step_warm = Step(w, P, 1, device, write_cache, kv8)
    step_warm.capture()
    sec_warm = time_graph_steps(step_warm, max(5, steps // 2), 2)
    km_warm = time_kernels(step_warm, 5)
    del step, step_warm
    return sec, km, sec_warm, km_warm


DECODE_SOURCES = ("paged_varlen_attention_amd/csrc/decode.hip",
                  "paged_varlen_attention_amd/csrc/decode_mfma.hip",
                  "paged_varlen_attention_amd/csrc/decode_rows.hip",
                  "paged_varlen_attention_amd/csrc/decode_rows8.hip",
                  "paged_varlen_attention_amd/csrc/pa_device.h",
                  "paged_varlen_attention_amd/csrc/pa_internal.h")
PMC_SUMMARY = "profiles/decode_gqa_decode_bf16_pmc.md"


def pmc_traffic():
    """HBM bytes per launch of the decode kernel from the committed rocprofv3
    FETCH_SIZE / WRITE_SIZE summary (each scaled by its copy-kernel
    calibration), or None when the kernel sources changed since it was taken."""
    kv = _summary_fields(PMC_SUMMARY, DECODE_SOURCES)
    if not kv:
        return None
    try:
        return int(round((float(kv["fetch_kib_per_dispatch"]) * float(kv["fetch_factor"]) +
                          float(kv["write_kib_per_dispatch"]) * float(kv["write_factor"])) * 1024))
    except (KeyError, ValueError):
        return None


PREFILL_SOURCES = ("paged_varlen_attention_amd/csrc/prefill.hip",
                   "paged_varlen_attention_amd/csrc/prefill_tile.h",
                   "paged_varlen_attention_amd/csrc/pa_device.h",
                   "paged_varlen_attention_amd/csrc/pa_internal.h")
PREFILL_PMC_SUMMARY = "profiles/prefill_tiles_pmc.md"


def _summary_fields(path, sources):
    """The machine-readable `key: value` lines of a committed rocprofv3
    summary, or None when the summary is missing or the kernel sources changed
    since it was taken (sha256 over `sources`)."""
    import hashlib
    path = os.path.join(ROOT, path)
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith(("#", "|", " ")):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    h = hashlib.sha256()
    for f in sources:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    return kv if kv.get("kernel_sources_sha256") == h.hexdigest() else None


def prefill_counters(name):
    """Counter-derived MFMA figures of the tile kernel on workload `name` from
    the committed rocprofv3 summary: executed MFMA flops (every MFMA issued) per
    trace-average duration against the bf16 peak, and MFMA-busy cycles per
    SIMD per 2.4 GHz cycle; None if the kernel changed since."""
    kv = _summary_fields(PREFILL_PMC_SUMMARY, PREFILL_SOURCES)
    if not kv or f"{name}.frac_mfma_counters" not in kv:
        return None
    return {"frac_mfma_counters": float(kv[f"{name}.frac_mfma_counters"]),
            "mfma_busy_frac": float(kv[f"{name}.mfma_busy_frac_2p4ghz"]),
            "rocprof_trace_avg_ms": round(float(kv[f"{name}.trace_avg_us"]) * 1e-3, 5),
            "source": PREFILL_PMC_SUMMARY}


def block_offload(device, n_blocks=4096, reps=10):
    """pa_copy_blocks between the GPU cache and a pinned host pool: 4,096
    blocks of 16 tokens x 8 KV heads x 128 bf16 (32 KiB each for K and for V,
    256 MiB per direction), evict (device -> host) and restore (host ->
    device), GB/s of block bytes moved."""
    import torch
    import paged_varlen_attention_amd as pa
    shape = (16, 8, 128)
    gk = torch.randn((n_blocks * 2,) + shape, device=device).to(torch.bfloat16)
    gv = torch.randn_like(gk)
    hk = torch.empty((n_blocks,) + shape, dtype=torch.bfloat16).pin_memory()
    hv = torch.empty_like(hk).pin_memory()
    g = torch.Generator().manual_seed(9)
    src = torch.randperm(n_blocks * 2, generator=g)[:n_blocks]
    out = torch.stack([src, torch.arange(n_blocks)], 1).to(torch.int64).to(device)
    back = out.flip(1).contiguous()
    nbytes = 2 * n_blocks * gk[0].numel() * 2
    res = {"blocks": n_blocks, "block_bytes_per_tensor": gk[0].numel() * 2}
    for name, args in (("evict_GB/s", (hk, hv, gk, gv, out)), ("restore_GB/s", (gk, gv, hk, hv, back))):
        pa.copy_blocks(*args)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            pa.copy_blocks(*args)
        e1.record()
        torch.cuda.synchronize()
        res[name] = round(nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9, 2)
    return res


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, pass_s=3.0):
    """The fp64 oracle, as it stands, timed on this host: the median of 3
    passes on all the threads OpenMP gives it (each pass repeats the whole
    batch for about pass_s seconds), then the median of 3 single-threaded
    passes.  Work unit: the workload's algorithmic bytes."""
    import oracle
    oracle.run_workload(w, rows=[(0, 0)])  # loads / builds the oracle library
    threads = oracle.num_threads()
    t0 = time.perf_counter()
    oracle.run_workload(w)
    reps = max(1, int(pass_s / max(time.perf_counter() - t0, 1e-3)))
    per = []
    for _ in range(3):
        t0 = time.perf_counter()
        for _ in range(reps):
            oracle.run_workload(w)
        per.append((time.perf_counter() - t0) / reps)
    per = sorted(per)[1]
    oracle.set_num_threads(1)
    one = []
    try:
        for _ in range(3):
            t0 = time.perf_counter()
            oracle.run_workload(w)
            one.append(time.perf_counter() - t0)
        one_threads = oracle.num_threads()
    finally:
        oracle.set_num_threads(threads)
    one = sorted(one)[1]
    nb = w.algorithmic_bytes()
    return {"value": round(nb / per / 1e9, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"median of 3 passes, each {reps} full runs of the {w.name} batch "
                      f"({w.num_seqs} requests, all {w.num_q_heads} heads; {per * 1e3:.1f} ms per "
                      f"batch), fp64 C oracle, OpenMP over (query row, head)",
            "cpu_model": cpu_model(), "host_logical_cpus": os.cpu_count(),
            "affinity_cpus": len(os.sched_getaffinity(0)),
            "single_thread": {"value": round(nb / one / 1e9, 3), "unit": "GB/s",
                              "ms_per_batch": round(one * 1e3, 1), "threads": one_threads,
                              "sample": "median of 3 full batches"}}


def gemm_reference(device, n=16384, reps=5):
    """The dense bf16 rate a plain library GEMM reaches on this GPU (torch.matmul,
    i.e. hipBLASLt; not the library's own kernels): an n x n x n product timed
    with HIP events, as the measured matrix-core reference beside the published
    2.5 PFLOP/s."""
    import torch
    g = torch.Generator(device=device).manual_seed(11)
    a = torch.randn((n, n), device=device, generator=g).to(torch.bfloat16)
    b = torch.randn((n, n), device=device, generator=g).to(torch.bfloat16)
    for _ in range(3):
        c = a @ b
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        c = a @ b
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    tf = 2 * n ** 3 / (ms * 1e-3) / 1e12
    del a, b, c
    return {"op": f"torch.matmul bf16 {n}x{n}x{n} (hipBLASLt)", "ms": round(ms, 4),
            "TFLOP/s": round(tf, 1), "frac_of_peak": round(tf / BF16_MFMA_PEAK_TFLOPS, 4)}


def copy_reference(device, mib=1024, reps=5):
    """The HBM rate a plain library copy reaches (torch's device-to-device copy,
    not the library's kernels): bytes read plus bytes written per HIP-event
    time, beside the published 8 TB/s."""
    import torch
    a = torch.empty(mib * 2 ** 20 // 4, dtype=torch.float32, device=device).fill_(1.0)
    b = torch.empty_like(a)
    for _ in range(2):
        b.copy_(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    gbs = 2 * mib * 2 ** 20 / (ms * 1e-3) / 1e9
    del a, b
    return {"op": f"torch copy_ of {mib} MiB (read + write)", "ms": round(ms, 4),
            "GB/s": round(gbs, 1), "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4)}


def copy_calibration(device, mib=512, reps=5):
    """A plain device copy of known size, for scaling rocprof FETCH/WRITE counters."""
    import torch
    a = torch.empty(mib * 2 ** 20 // 4, dtype=torch.float32, device=device).fill_(1.0)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    log(f"copy calibration: {reps} x copy of {mib} MiB (read {mib} MiB + write {mib} MiB each)")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--copies", type=int, default=3, help="KV pool copies cycled per step")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--secondary", dest="secondary", action="store_true", default=True)
    ap.add_argument("--no-secondary", dest="secondary", action="store_false")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--workloads", default="",
                    help="comma-separated secondary workloads to run (default: all)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import torch
    import workloads as W
    import paged_varlen_attention_amd  # noqa: F401  (fails loudly without libpa.so)

    device = torch.device("cuda:0")
    torch.cuda.set_device(device)

    # ---------------- headline: GQA decode batch ----------------
    w = W.gqa_decode_bf16()
    P = 512  # the workload's partition size
    import paged_varlen_attention_amd as pa
    P_policy = pa.pick_partition_size(w.seq_lens.tolist(), w.num_q_heads, w.num_kv_heads,
                                      w.head_dim, w.block_size, w.dtype)
    log(f"workload {w.name}: {w.description}; P={P} (partition policy picks {P_policy})")
    sec, km, sec_warm, km_warm = measure(w, P, args.steps, args.warmup, args.copies, device)
    nbytes = step_bytes(w, include_cache_write=True)
    value = nbytes / sec / 1e9
    attn_bytes = w.algorithmic_bytes()
    achieved = attn_bytes / (km["attention_back_to_back"] * 1e-3) / 1e9
    log(f"decode step {sec * 1e3:.4f} ms ({value:.1f} GB/s); kernels {km}; warm step "
        f"{sec_warm * 1e3:.4f} ms, kernels {km_warm}")
    policy_step_ms = sec * 1e3
    if P_policy != P:  # the policy's pick, timed the same way
        sec_p, _, _, _ = measure(w, P_policy, args.steps, args.warmup, args.copies, device)
        policy_step_ms = sec_p * 1e3

    result = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(sec * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "gqa_decode_bf16",
            "requests": w.num_seqs,
            "query_tokens": w.total_q,
            "context": "U[512,4096]",
            "heads_q_kv_dim": [w.num_q_heads, w.num_kv_heads, w.head_dim],
            "page_size": w.block_size,
            "pool_blocks": w.num_blocks,
            "partition_size": P,
            "partition_policy_pick": P_policy,
            "partition_policy_ms_per_step": round(policy_step_ms, 5),
            "step": "reshape_and_cache + varlen_attention + split_kv_reduce",
            "algorithmic_bytes_per_step": nbytes,
            "kv_pool_copies_cycled": args.copies,
            "warm_ms_per_step": round(sec_warm * 1e3, 5),
            "kernel_ms": {k: round(v, 5) for k, v in km.items() if k != "step_ms_percentiles"},
            "step_ms_percentiles": km["step_ms_percentiles"],
            "parallelism": "single GPU",
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "decode_rows_kernel (pa_varlen_attention, split 512)",
            "achieved": round(achieved, 3),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": pmc_traffic(),
            "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, "
                            "copy-calibrated; null if the kernel changed since)",
            "algorithmic_bytes_per_launch": attn_bytes,
            "avg_launch_ms": round(km["attention_back_to_back"], 5),
            "avg_launch_timing": "HIP events around back-to-back attention launches over the "
                                 "cycled KV-pool copies",
        },
    }

    # ---------------- secondary workloads ----------------
    only = {x for x in args.workloads.split(",") if x}

    def wanted(name):
        return not only or name in only

    if args.secondary:
        sec_out = {}
        steps2 = max(10, args.steps // 2)
        w4 = W.long_decode_bf16()
        # the workload's fixed sizes (256, 512) and the size the library's
        # partition policy picks for it on this GPU
        import paged_varlen_attention_amd as pa
        P4_policy = pa.pick_partition_size(w4.seq_lens.tolist(), w4.num_q_heads, w4.num_kv_heads,
                                           w4.head_dim, w4.block_size, w4.dtype)
        for P4 in sorted({256, 512, P4_policy}):
            if not wanted(f"long_decode_bf16_P{P4}"):
                continue
            s4, k4, s4w, _ = measure(w4, P4, steps2, 5, 2, device)
            b4 = w4.algorithmic_bytes()
            sec_out[f"long_decode_bf16_P{P4}"] = {
                "ms_per_step": round(s4 * 1e3, 5), "GB/s": round(b4 / s4 / 1e9, 2),
                "attention_ms": round(k4["attention_back_to_back"], 5),
                "attention_eager_ms": round(k4["attention"], 5), "reduce_ms": round(k4["reduce"], 5),
                "attention_GB/s": round(b4 / (k4["attention_back_to_back"] * 1e-3) / 1e9, 2),
                "frac_hbm": round(b4 / s4 / 1e9 / HBM_PEAK_GBS, 4),
                "step_ms_percentiles": k4["step_ms_percentiles"],
                "warm_ms_per_step": round(s4w * 1e3, 5),
                "partition_policy_pick": P4 == P4_policy}
            log(f"long decode P={P4}: {sec_out[f'long_decode_bf16_P{P4}']}")
        # 8-bit E4M3 caches (the library's KV quantisation): the same decode
        # batches with half the KV bytes
        for name8, w8, P8 in (("gqa_decode_fp8kv_P512", w, 512), ("gqa_decode_fp8kv_P1024", w, 1024),
                              ("long_decode_fp8kv_P2048", w4, 2048)):
            if not wanted(name8):
                continue
            s8, k8, s8w, _ = measure(w8, P8, steps2, 5, args.copies, device, kv8=True)
            b8 = step_bytes(w8, True, kv_elt_bytes=1)
            a8 = w8.algorithmic_bytes(1)
            sec_out[name8] = {
                "ms_per_step": round(s8 * 1e3, 5), "GB/s": round(b8 / s8 / 1e9, 2),
                "attention_ms": round(k8["attention_back_to_back"], 5),
                "attention_eager_ms": round(k8["attention"], 5), "reduce_ms": round(k8["reduce"], 5),
                "cache_write_ms": round(k8["cache_write"], 5),
                "attention_GB/s": round(a8 / (k8["attention_back_to_back"] * 1e-3) / 1e9, 2),
                "frac_hbm": round(a8 / (k8["attention_back_to_back"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                "algorithmic_bytes_per_launch": a8,
                "step_ms_percentiles": k8["step_ms_percentiles"],
                "warm_ms_per_step": round(s8w * 1e3, 5)}
            log(f"{name8}: {sec_out[name8]}")
        del w4
        # partition sizes: the mixed batches run unsplit (their rows are at
        # most 3,000 keys); the verify batch splits its long contexts so its
        # 164 q-tiles do not leave most of the GPU idle
        for name, P3 in (("mixed_prefill_bf16_A", 0), ("mixed_prefill_bf16_B", 0),
                         ("spec_verify_bf16", 1024), ("prefill_uniform_bf16", 0),
                         ("mixed_prefill_fp8kv_B", 0), ("prefill_uniform_fp8kv", 0)):
            kv8 = "fp8kv" in name
            if not wanted(name):
                continue
            try:
                w3 = W.CONFIGS[name.replace("fp8kv", "bf16")]()
                s3, k3, s3w, _ = measure(w3, P3, steps2, 5, 2, device, kv8=kv8)
            except Exception as e:  # report, do not hide: the line says what failed
                sec_out[name] = {"error": str(e)[:200]}
                log(f"{name}: {e}")
                continue
            f3 = w3.algorithmic_flops()
            b3 = step_bytes(w3, True, kv_elt_bytes=1 if kv8 else None)
            sec_out[name] = {
                "partition_size": P3,
                "ms_per_step": round(s3 * 1e3, 5),
                "TFLOP/s": round(f3 / s3 / 1e12, 2),
                "attention_ms": round(k3["attention_back_to_back"], 5),
                "attention_eager_ms": round(k3["attention"], 5),
                "attention_TFLOP/s": round(f3 / (k3["attention_back_to_back"] * 1e-3) / 1e12, 2),
                "frac_mfma": round(f3 / (k3["attention_back_to_back"] * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4),
                "GB/s": round(b3 / s3 / 1e9, 2),
                "algorithmic_flops": f3, "algorithmic_bytes": b3,
                "step_ms_percentiles": k3["step_ms_percentiles"],
                "warm_ms_per_step": round(s3w * 1e3, 5),
                "counters": prefill_counters(name)}
            log(f"{name}: {sec_out[name]}")
        if wanted("kv_block_offload_bf16"):
            sec_out["kv_block_offload_bf16"] = block_offload(device)
            log(f"kv block offload: {sec_out['kv_block_offload_bf16']}")
        if wanted("hbm_copy_reference"):
            sec_out["hbm_copy_reference"] = copy_reference(device)
            log(f"HBM copy reference: {sec_out['hbm_copy_reference']}")
        if wanted("bf16_gemm_reference"):
            sec_out["bf16_gemm_reference"] = gemm_reference(device)
            log(f"bf16 GEMM reference: {sec_out['bf16_gemm_reference']}")
        result["secondary"] = sec_out

    if args.copy_calibration:
        copy_calibration(device)

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w)
        log(f"cpu baseline: {result['cpu_baseline']}")

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
