"""Benchmark of the paged-attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--configs c1,c2,...]

A step is one pass of the decode hot path over one batch: every sequence's
newest K/V row is scattered into the block pool through its slot and the
sequences attend over their whole paged context, in one call
(pa_decode_append: the cache write fused with decode attention, split-K
chosen automatically).  All inputs are seeded synthetic data resident in HBM
before timing starts.

Every step is timed on its own: an untimed cache scrub runs first, then HIP
events on the launch stream bracket the call.  The scrub writes a 512 MiB
buffer and then reads another 512 MiB (each larger than the L2s and the 256
MB last-level cache together): the workload's data is evicted and the
caches hold clean lines, as after the other layers of a model have streamed
their weights through them.  (A write alone leaves ~256 MB of dirty lines
whose write-back would land inside the timed call; that variant is reported
beside the headline as ``step_cold_write_scrub``.)  The K timed steps are
bracketed by torch.cuda.synchronize() on both sides.  ``value`` is the KV
bytes of a step divided by the median scrubbed step time (GB/s) on the
Llama-3.1-8B-shaped layer; ``ms_per_step`` is that median.  The same calls
without the scrub ("hot") and a back-to-back loop are reported beside it.

``configs`` carries all five workloads, each with its KV bytes, tokens/s,
GB/s and fraction of the 8 TB/s HBM peak (or of the bf16 matrix-core peak
for prefill), scrubbed and hot, and its own CPU baseline: the fp64 oracle
run unchanged on the host on a bounded sample of the same workload.

Prints one JSON line.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.join(ROOT, "tests"))

METRIC = "paged decode attn: KV GB/s and % of MI355X HBM peak; decode tokens/s"
HBM_PEAK_GBS = 8000.0  # MI355X published HBM3E bandwidth
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X published dense bf16 matrix-core peak
SCRUB_BYTES = 512 << 20
CONFIGS = {
    "c1": "tiny_f32",
    "c2": "llama3_8b_b64",
    "c3": "llama2_70b_b256",
    "c4": "shared_prefix_32x4",
    "c5": "long_mixed",
}
PROFILES = os.path.join(ROOT, "profiles")


def _source_hash():
    h = hashlib.sha256()
    for f in ("decode.hip", "pa_device.h"):
        with open(os.path.join(ROOT, "paged_kv_cache_396_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _summary(name):
    """key: value pairs of a committed profile summary (comment lines skipped)."""
    path = os.path.join(PROFILES, name)
    d = {}
    if not os.path.exists(path):
        return d
    with open(path) as f:
        for line in f:
            if line.startswith("#") or ":" not in line:
                continue
            k, v = line.split(":", 1)
            d[k.strip()] = v.strip()
    return d


def _traffic(workload):
    """HBM bytes per step call from committed rocprofv3 counter passes, if they
    were taken on the current decode source; else None."""
    d = _summary(f"decode_{workload}_pmc.txt")
    if d.get("source_hash") != _source_hash() or "hbm_bytes_per_call" not in d:
        return None
    return int(float(d["hbm_bytes_per_call"]))


def _kernel_profile(workload, kv_bytes):
    """The dominant kernel's mean duration from the committed rocprofv3 kernel
    trace of the same source, as a roofline fraction; else None."""
    d = _summary(f"decode_{workload}_kernel_stats.txt")
    if d.get("source_hash") != _source_hash() or "dominant_kernel_avg_us" not in d:
        return None
    us = float(d["dominant_kernel_avg_us"])
    gbs = kv_bytes / (us * 1e-6) / 1e9
    return {"kernel": d.get("dominant_kernel"), "avg_us": us, "gbs": round(gbs, 1),
            "frac": round(gbs / HBM_PEAK_GBS, 4), "source": f"profiles/decode_{workload}_kernel_stats.txt"}


# ----------------------------------------------------------------------------
# timing


class Timer:
    """Per-call HIP event timing on the launch stream, with or without an
    untimed cache scrub before each call, and back-to-back loops."""

    def __init__(self):
        import torch

        self.torch = torch
        self.stream = torch.cuda.current_stream()
        self.scrub = torch.empty(SCRUB_BYTES, dtype=torch.uint8, device="cuda")
        self.scrub_read = torch.ones(SCRUB_BYTES // 4, dtype=torch.int32, device="cuda")

    def clean_scrub(self):
        """Evict everything, then leave clean lines: write 512 MiB, read 512 MiB."""
        self.scrub.fill_(7)
        self.scrub_read.sum()

    def calls(self, fn, n, cold, before=None, write_only=False):
        t = self.torch
        evs = []
        t.cuda.synchronize()
        for _ in range(n):
            if before is not None:
                before()
            if cold and write_only:
                self.scrub.fill_(7)
            elif cold:
                self.clean_scrub()
            a, b = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
            a.record(self.stream)
            fn()
            b.record(self.stream)
            evs.append((a, b))
        t.cuda.synchronize()
        return [a.elapsed_time(b) for a, b in evs]

    def loop(self, fn, n):
        t = self.torch
        t.cuda.synchronize()
        a, b = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
        a.record(self.stream)
        for _ in range(n):
            fn()
        b.record(self.stream)
        t.cuda.synchronize()
        return a.elapsed_time(b) / n


def dist(ms, nbytes=None, flops=None, tokens=None):
    """Median and p10/p90 of per-call times, with the rates of the median."""
    p10, p50, p90 = np.percentile(ms, [10, 50, 90])
    d = {"median_ms": round(float(p50), 5), "p10_ms": round(float(p10), 5),
         "p90_ms": round(float(p90), 5), "calls": len(ms)}
    if nbytes is not None:
        gbs = nbytes / (p50 * 1e-3) / 1e9
        d["gbs"] = round(gbs, 1)
        d["hbm_frac"] = round(gbs / HBM_PEAK_GBS, 4)
    if flops is not None:
        tf = flops / (p50 * 1e-3) / 1e12
        d["tflops"] = round(tf, 1)
        d["mfma_frac"] = round(tf / MFMA_BF16_PEAK_TFLOPS, 4)
    if tokens is not None:
        d["tokens_per_s"] = round(tokens / (p50 * 1e-3), 1)
    return d


# ----------------------------------------------------------------------------
# the oracle on the host (a reported baseline, not a target)


def _host_cores():
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _blas_one_thread():
    try:
        from threadpoolctl import threadpool_limits

        return threadpool_limits(1)
    except Exception:  # pragma: no cover
        return None


def cpu_oracle(units, run_unit, unit_bytes, unit_tokens, what, budget_s):
    """Runs ``run_unit(u)`` (the oracle unchanged on one unit of the workload:
    a sequence, or a group of query rows) over the units in order until
    ``budget_s / 2`` has passed on one core, then over a thread pool of every
    core this process may use (at most 16; NumPy's matrix products and
    exponentials release the GIL; BLAS one thread per worker) for the rest of
    the budget.  Rates are bytes (or tokens) of the units finished divided by
    the time taken."""
    from concurrent.futures import ThreadPoolExecutor

    lim = _blas_one_thread()
    try:
        t0 = time.perf_counter()
        n1 = 0
        while time.perf_counter() - t0 < budget_s / 2 or n1 == 0:
            run_unit(units[n1 % len(units)])
            n1 += 1
        el1 = time.perf_counter() - t0
        b1 = sum(unit_bytes(units[i % len(units)]) for i in range(n1))
        k1 = sum(unit_tokens(units[i % len(units)]) for i in range(n1))
        cores = _host_cores()
        t0 = time.perf_counter()
        nN = 0
        with ThreadPoolExecutor(max_workers=cores) as ex:
            while time.perf_counter() - t0 < budget_s / 2 or nN == 0:
                batch = [units[(nN + i) % len(units)] for i in range(cores)]
                list(ex.map(run_unit, batch))
                nN += cores
        elN = time.perf_counter() - t0
        bN = sum(unit_bytes(units[i % len(units)]) for i in range(nN))
        kN = sum(unit_tokens(units[i % len(units)]) for i in range(nN))
    finally:
        if lim is not None and hasattr(lim, "restore_original_limits"):
            lim.restore_original_limits()
    return {
        "value": round(bN / elN / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
        "sample": f"{nN} {what} on {cores} threads in {elN:.1f} s, then on one core {n1} in "
                  f"{el1:.1f} s (numpy fp64, BLAS 1 thread each)",
        "tokens_per_s": round(kN / elN, 2),
        "one_core": {"value": round(b1 / el1 / 1e9, 4), "unit": "GB/s",
                     "tokens_per_s": round(k1 / el1, 2)},
    }


def _oracle_pools(wl):
    import oracle
    from gpu_util import oracle_pools

    return oracle_pools(wl, oracle)


def cpu_decode(wl, budget_s, pools=None, what=None):
    """The oracle's decode of single sequences of ``wl`` (decode tokens =
    sequences)."""
    import oracle

    pk, pv = _oracle_pools(wl) if pools is None else pools
    per_tok = 2 * wl.num_kv_heads * wl.head_dim * (2 if wl.dtype == "bf16" else 4)
    order = list(np.argsort(-wl.context_lens.astype(np.int64), kind="stable"))

    def run(s):
        oracle.decode(wl.q, pk, pv, wl.block_tables, wl.context_lens, wl.scale, wl.dtype, seqs=[s])

    return cpu_oracle(order, run, lambda s: int(wl.context_lens[s]) * per_tok, lambda s: 1,
                      what or f"sequences of {wl.name}", budget_s)


def cpu_prefill(wl, budget_s, pools=None, rows_per_unit=16):
    """The oracle's prefill of groups of query rows of ``wl`` (rates in KV
    bytes of the keys each row sees and in query tokens)."""
    import oracle

    pk, pv = _oracle_pools(wl) if pools is None else pools
    per_tok = 2 * wl.num_kv_heads * wl.head_dim * 2
    pos = np.zeros(wl.total_q_tokens, dtype=np.int64)
    for r in range(wl.num_reqs):
        lo, hi = int(wl.query_start_loc[r]), int(wl.query_start_loc[r + 1])
        pos[lo:hi] = int(wl.context_lens[r]) - (hi - lo) + np.arange(hi - lo)
    units = [list(range(i, min(i + rows_per_unit, wl.total_q_tokens)))
             for i in range(0, wl.total_q_tokens, rows_per_unit)]
    rng = np.random.default_rng(0)
    units = [units[i] for i in rng.permutation(len(units))]

    def run(rows):
        oracle.prefill_chunk(wl.q, pk, pv, wl.block_tables, wl.query_start_loc, wl.context_lens,
                             wl.scale, wl.dtype, rows=rows)

    return cpu_oracle(units, run, lambda rows: int(sum(pos[r] + 1 for r in rows)) * per_tok,
                      lambda rows: len(rows), f"groups of {rows_per_unit} query rows of {wl.name}",
                      budget_s)


# ----------------------------------------------------------------------------
# the decode step of one decode workload


class DecodeBench:
    """Device state of one decode workload: the pool holds the history, the
    step appends every sequence's newest token and attends."""

    def __init__(self, wl):
        import torch

        import paged_kv_cache_396_amd as pa
        from gpu_util import GpuPool, to_dev

        self.wl = wl
        self.pa = pa
        self.pool = GpuPool(wl.num_blocks, wl.num_kv_heads, wl.head_dim, wl.dtype)
        self.pool.write(wl.hist_k, wl.hist_v, wl.hist_slots)
        self.new_k, self.new_v = to_dev(wl.new_k, wl.dtype), to_dev(wl.new_v, wl.dtype)
        self.new_slots = torch.from_numpy(wl.new_slots).cuda()
        self.q = to_dev(wl.q, wl.dtype)
        self.out = torch.empty_like(self.q)
        self.bt = torch.from_numpy(wl.block_tables).cuda()
        self.cl = torch.from_numpy(wl.context_lens).cuda()
        S, Hq, D = wl.q.shape
        self.max_ctx = int(wl.context_lens.max())
        self.part = pa.pa_decode_partition_size(S, wl.num_kv_heads, self.max_ctx, 0)
        ws_bytes = pa.pa_decode_workspace_bytes(S, Hq, wl.num_kv_heads, D, self.max_ctx, 0)
        self.ws = torch.empty(max(1, (ws_bytes + 3) // 4), dtype=torch.float32, device="cuda")

    def step(self):
        w = self.wl
        self.pa.pa_decode_append(self.out, self.q, self.new_k, self.new_v, self.new_slots,
                                 self.pool.k, self.pool.v, self.bt, self.cl, self.max_ctx,
                                 float(w.scale), self.pool.desc, workspace=self.ws)

    def write(self):
        self.pa.pa_reshape_and_cache(self.new_k, self.new_v, self.new_slots, self.pool.k,
                                     self.pool.v, self.pool.desc)

    def decode(self):
        w = self.wl
        self.pa.pa_decode(self.out, self.q, self.pool.k, self.pool.v, self.bt, self.cl,
                          self.max_ctx, float(w.scale), self.pool.desc, workspace=self.ws)

    def two_call(self):
        self.write()
        self.decode()

    def schedule(self):
        return ("work-balanced: equal block ranges, one per resident workgroup" if self.part == 0
                else f"partitions of {self.part} tokens")


def decode_section(db, timer, steps, warmup, cold_ms=None):
    """Step (pa_decode_append), two-call step and pa_decode alone on one
    decode workload, scrubbed and hot."""
    wl = db.wl
    kv = wl.kv_bytes
    S = wl.num_seqs
    for _ in range(warmup):
        db.step()
        db.two_call()
    if cold_ms is None:
        cold_ms = timer.calls(db.step, steps, cold=True)
    hot_ms = timer.calls(db.step, steps, cold=False)
    dec_cold = timer.calls(db.decode, steps, cold=True, before=db.write)
    dec_hot = timer.calls(db.decode, steps, cold=False, before=db.write)
    two_cold = timer.calls(db.two_call, steps, cold=True)
    loop_ms = timer.loop(db.step, steps)
    return {
        "workload": wl.name,
        "num_seqs": S, "num_q_heads": wl.num_q_heads, "num_kv_heads": wl.num_kv_heads,
        "head_dim": wl.head_dim, "dtype": wl.dtype, "ctx_sum": int(wl.context_lens.sum()),
        "num_blocks": wl.num_blocks, "kv_bytes_per_step": kv,
        "decode_schedule": db.schedule(),
        "step_call": "pa_decode_append (newest token of each sequence written, then decode)",
        "step_cold": dist(cold_ms, kv, tokens=S),
        "step_hot": dist(hot_ms, kv, tokens=S),
        "step_hot_loop_ms": round(loop_ms, 5),
        "decode_call_cold": dist(dec_cold, kv, tokens=S),
        "decode_call_hot": dist(dec_hot, kv, tokens=S),
        "two_call_step_cold": dist(two_cold, kv, tokens=S),
    }


# ----------------------------------------------------------------------------
# the five configurations


def bench_c1(timer, steps, warmup, budget):
    from workloads import make_decode

    wl = make_decode(1)
    db = DecodeBench(wl)
    sec = decode_section(db, timer, steps, warmup)
    sec["note"] = "latency-bound (121,856 KV bytes): read the step's median in microseconds"
    sec["step_cold_us"] = round(sec["step_cold"]["median_ms"] * 1e3, 2)
    sec["step_hot_us"] = round(sec["step_hot"]["median_ms"] * 1e3, 2)
    if budget > 0:
        sec["cpu_baseline"] = cpu_decode(wl, min(budget, 2.0))
    return sec


def bench_c2(timer, steps, warmup, budget):
    from workloads import make_decode

    wl = make_decode(2)
    db = DecodeBench(wl)
    for _ in range(warmup):
        db.step()
    # the timed steps: each scrubbed, each bracketed by its own events
    import torch

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    cold_ms = timer.calls(db.step, steps, cold=True)
    wall = time.perf_counter() - t0
    sec = decode_section(db, timer, steps, 0, cold_ms=cold_ms)
    sec["timed_region_wall_s"] = round(wall, 4)
    sec["step_cold_write_scrub"] = dist(timer.calls(db.step, steps, cold=True, write_only=True),
                                        wl.kv_bytes, tokens=wl.num_seqs)
    if budget > 0:
        sec["cpu_baseline"] = cpu_decode(wl, budget)
    return sec, db


def bench_c3(timer, steps, warmup, budget):
    from workloads import make_decode

    wl = make_decode(3)
    db = DecodeBench(wl)
    sec = decode_section(db, timer, steps, warmup)
    del db
    sec["cache_write_bulk"] = bench_bulk_write(wl, timer, min(steps, 10))
    if budget > 0:
        sec["cpu_baseline"] = cpu_decode(wl, budget)
    return sec


def bench_c4(timer, steps, warmup, budget):
    """pa_decode (every sample reads its own table: logical bytes) and
    pa_decode_shared_prefix (each shared block read once per group: unique
    bytes) on the same inputs."""
    import torch

    import paged_kv_cache_396_amd as pa
    from workloads import make_decode

    wl = make_decode(4)
    db = DecodeBench(wl)
    sec = decode_section(db, timer, steps, warmup)
    prompt_of = wl.extra["prompt_of"]
    group = int(np.sum(prompt_of == prompt_of[0]))
    n_groups = wl.num_seqs // group
    plen = int(wl.extra["prompt_len"])
    S, Hq, D = wl.q.shape
    prefix = torch.full((n_groups,), plen, dtype=torch.int32, device="cuda")
    ws_bytes = pa.pa_decode_shared_prefix_workspace_bytes(S, Hq, wl.num_kv_heads, D, db.max_ctx,
                                                          group, plen)
    ws = torch.empty((ws_bytes + 3) // 4, dtype=torch.float32, device="cuda")
    out = torch.empty_like(db.q)
    db.write()

    def shared():
        pa.pa_decode_shared_prefix(out, db.q, db.pool.k, db.pool.v, db.bt, db.cl, db.max_ctx,
                                   float(wl.scale), prefix, group, plen, db.pool.desc, ws)

    for _ in range(warmup):
        shared()
    cold = timer.calls(shared, steps, cold=True)
    hot = timer.calls(shared, steps, cold=False)
    unique = (n_groups * plen + int(wl.context_lens.sum()) - S * plen) * 2 * wl.num_kv_heads * D * 2
    sec["logical_kv_bytes"] = wl.kv_bytes
    sec["unique_kv_bytes"] = unique
    sec["shared_prefix_call"] = {
        "call": "pa_decode_shared_prefix (prefix blocks read once per group of 4 samples)",
        "group_size": group, "prefix_tokens": plen,
        "cold_unique": dist(cold, unique, tokens=S), "hot_unique": dist(hot, unique, tokens=S),
        "cold_logical_gbs": round(wl.kv_bytes / (np.median(cold) * 1e-3) / 1e9, 1),
    }
    med = sec["decode_call_cold"]["median_ms"]
    sec["decode_call_cold_unique_frac"] = round(unique / (med * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
    if budget > 0:
        sec["cpu_baseline"] = cpu_decode(wl, budget)
    return sec


def bench_c5(timer, steps, warmup, budget):
    """The long-context mixed batch over one pool: the decode half (8 x 32768,
    split-K) and the prefill half (4 x 512-token chunks over 4096 prior
    tokens) alone, back to back on one stream, and on two streams at once."""
    import torch

    from gpu_util import MixedStep
    from workloads import make_mixed

    dec, pre = make_mixed(0)
    st = MixedStep(dec, pre)
    fl = prefill_flops(pre)
    kv_dec = dec.kv_bytes

    def prefill_half():
        st.prefill_half(torch.cuda.current_stream())

    def decode_half():
        st.decode_half(torch.cuda.current_stream())

    for _ in range(warmup):
        st.run(False)
        st.run(True)
    d_cold = timer.calls(decode_half, steps, cold=True)
    d_hot = timer.calls(decode_half, steps, cold=False)
    p_cold = timer.calls(prefill_half, steps, cold=True)
    p_hot = timer.calls(prefill_half, steps, cold=False)
    seq_cold = timer.calls(lambda: st.run(False), steps, cold=True)
    conc_cold = timer.calls(lambda: st.run(True), steps, cold=True)
    seq_hot = timer.calls(lambda: st.run(False), steps, cold=False)
    conc_hot = timer.calls(lambda: st.run(True), steps, cold=False)
    sec = {
        "workload": "long_mixed: 8 x 32768 decode + 4 x 512-token chunks over 4096 prior tokens, one pool",
        "decode_kv_bytes": kv_dec,
        "decode_half": {"call": "pa_decode_append (8 new tokens, split-K decode)",
                        "cold": dist(d_cold, kv_dec, tokens=dec.num_seqs),
                        "hot": dist(d_hot, kv_dec, tokens=dec.num_seqs)},
        "prefill_half": {"calls": "pa_reshape_and_cache (2048 chunk tokens) + pa_prefill_chunk",
                         "causal_flops": fl,
                         "cold": dist(p_cold, flops=fl, tokens=pre.total_q_tokens),
                         "hot": dist(p_hot, flops=fl, tokens=pre.total_q_tokens)},
        "sequential_cold": dist(seq_cold), "concurrent_cold": dist(conc_cold),
        "sequential_hot": dist(seq_hot), "concurrent_hot": dist(conc_hot),
        "overlap_gain_cold": round(float(np.median(seq_cold) / np.median(conc_cold)), 3),
        "overlap_gain_hot": round(float(np.median(seq_hot) / np.median(conc_hot)), 3),
    }
    del st
    if budget > 0:
        pools = _oracle_pools_mixed(dec, pre)
        sec["cpu_baseline"] = cpu_decode(dec, budget / 2, pools=pools)
        sec["cpu_baseline_prefill"] = cpu_prefill(pre, budget / 2, pools=pools)
    return sec


def _oracle_pools_mixed(dec, pre):
    import oracle
    from workloads import poison_bits

    pk = oracle.new_pool(dec.num_blocks, dec.num_kv_heads, dec.head_dim, dec.dtype, poison_bits(dec.dtype))
    pv = oracle.new_pool(dec.num_blocks, dec.num_kv_heads, dec.head_dim, dec.dtype, poison_bits(dec.dtype))
    for wl in (dec, pre):
        oracle.reshape_and_cache_fast(pk, pv, wl.hist_k, wl.hist_v, wl.hist_slots)
        oracle.reshape_and_cache_fast(pk, pv, wl.new_k, wl.new_v, wl.new_slots)
    return pk, pv


def prefill_flops(wl):
    """Causal-useful FLOPs of one pa_prefill_chunk call: every query row does
    a 2-FLOP multiply-add per dim for Q.K and for P.V over the keys it sees."""
    tot = 0
    for r in range(wl.num_reqs):
        n_r = int(wl.query_start_loc[r + 1] - wl.query_start_loc[r])
        prior = int(wl.context_lens[r]) - n_r
        tot += n_r * prior + n_r * (n_r + 1) // 2  # sum over i of (prior + i + 1)
    return tot * wl.num_q_heads * 4 * wl.head_dim


def bench_bulk_write(wl, timer, steps):
    """pa_reshape_and_cache of the 70B layer's KV in one call (the shape of a
    prefill's cache fill), twice: every sequence's 2048 tokens (524,288 in
    all; each sequence's run starts at a block boundary) and the 2047-token
    histories alone (524,032; from the second sequence on, every run starts
    mid-block in the input's groups of 16)."""
    import torch

    import paged_kv_cache_396_amd as pa
    from gpu_util import GpuPool, to_dev

    pool = GpuPool(wl.num_blocks, wl.num_kv_heads, wl.head_dim, wl.dtype)
    S, Hkv, D = wl.num_seqs, wl.num_kv_heads, wl.head_dim
    n = int(wl.context_lens[0])
    whole_k = np.concatenate([wl.hist_k.reshape(S, n - 1, Hkv, D), wl.new_k.reshape(S, 1, Hkv, D)], 1)
    whole_v = np.concatenate([wl.hist_v.reshape(S, n - 1, Hkv, D), wl.new_v.reshape(S, 1, Hkv, D)], 1)
    whole_s = np.concatenate([wl.hist_slots.reshape(S, n - 1), wl.new_slots.reshape(S, 1)], 1)
    out = {}
    for name, (kr, vr, sr) in (("whole_contexts", (whole_k.reshape(-1, Hkv, D), whole_v.reshape(-1, Hkv, D),
                                                   whole_s.reshape(-1))),
                               ("histories_2047", (wl.hist_k, wl.hist_v, wl.hist_slots))):
        k, v = to_dev(kr, wl.dtype), to_dev(vr, wl.dtype)
        slots = torch.from_numpy(np.ascontiguousarray(sr)).cuda()

        def call():
            pa.pa_reshape_and_cache(k, v, slots, pool.k, pool.v, pool.desc)

        call()
        T = int(len(sr))
        moved = 4 * T * Hkv * D * 2  # K and V read once and written once
        out[name] = {"tokens": T, "bytes_moved": moved,
                     "cold": dist(timer.calls(call, steps, cold=True), moved)}
        del k, v, slots
    return out


# ----------------------------------------------------------------------------
# further rows: fp8 pools, speculative verification, block pool


class _Fp8Pool:
    """fp8 (E4M3) K and V pools filled through the library's quantizing write."""

    def __init__(self, wl):
        import torch

        import paged_kv_cache_396_amd as pa
        from workloads import FP8_K_SCALE, FP8_V_SCALE

        self.desc = pa.cache_desc(wl.num_blocks, wl.num_kv_heads, wl.head_dim, pa.PA_FP8_E4M3,
                                  float(FP8_K_SCALE), float(FP8_V_SCALE))
        n = pa.pa_cache_bytes(self.desc)
        self.k = torch.full((n,), 0x7F, dtype=torch.uint8, device="cuda")
        self.v = torch.full((n,), 0x7F, dtype=torch.uint8, device="cuda")

    def write(self, k_raw, v_raw, slots):
        import torch

        import paged_kv_cache_396_amd as pa
        from gpu_util import to_dev

        pa.pa_reshape_and_cache(to_dev(k_raw, "bf16"), to_dev(v_raw, "bf16"),
                                torch.from_numpy(slots).cuda(), self.k, self.v, self.desc)


def bench_prefill(timer, steps, warmup, fp8=False):
    """pa_prefill_chunk on the long-context mixed batch's prefill half (bf16
    pools, or fp8 pools holding the same rows quantized)."""
    import torch

    import paged_kv_cache_396_amd as pa
    from gpu_util import GpuPool, to_dev
    from workloads import make_prefill

    wl = make_prefill(5)
    pool = _Fp8Pool(wl) if fp8 else GpuPool(wl.num_blocks, wl.num_kv_heads, wl.head_dim, wl.dtype)
    pool.write(wl.hist_k, wl.hist_v, wl.hist_slots)
    pool.write(wl.new_k, wl.new_v, wl.new_slots)
    q = to_dev(wl.q, wl.dtype)
    out = torch.empty_like(q)
    bt = torch.from_numpy(wl.block_tables).cuda()
    qsl = torch.from_numpy(wl.query_start_loc).cuda()
    cl = torch.from_numpy(wl.context_lens).cuda()

    def call():
        pa.pa_prefill_chunk(out, q, pool.k, pool.v, bt, qsl, cl, wl.max_q_len, float(wl.scale),
                            pool.desc)

    for _ in range(warmup):
        call()
    fl = prefill_flops(wl)
    cold = timer.calls(call, steps, cold=True)
    hot = timer.calls(call, steps, cold=False)
    loop = timer.loop(call, steps)
    return {
        "workload": "long_mixed_prefill", "kv_dtype": "fp8_e4m3" if fp8 else "bf16",
        "num_reqs": wl.num_reqs, "chunk_tokens": int(wl.max_q_len),
        "prior_tokens": int(wl.context_lens[0]) - int(wl.max_q_len), "causal_flops": fl,
        "cold": dist(cold, flops=fl, tokens=wl.total_q_tokens),
        "hot": dist(hot, flops=fl, tokens=wl.total_q_tokens),
        "hot_loop_ms": round(loop, 5),
        "roofline": {"bound": "mfma", "kernel": "prefill_chunk_kernel",
                     "achieved": round(fl / (np.median(cold) * 1e-3) / 1e12, 2),
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(fl / (np.median(cold) * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)},
    }


def bench_fp8_decode(timer, steps, warmup):
    """The 8B layer's decode step with fp8 (E4M3) pools: the same bf16 K/V
    rows quantized with per-pool scales; attention reads half the bytes."""
    import torch

    import paged_kv_cache_396_amd as pa
    from gpu_util import to_dev
    from workloads import FP8_K_SCALE, FP8_V_SCALE, make_decode

    wl = make_decode(2)
    pool = _Fp8Pool(wl)
    pool.write(wl.hist_k, wl.hist_v, wl.hist_slots)
    new_k, new_v = to_dev(wl.new_k, "bf16"), to_dev(wl.new_v, "bf16")
    new_slots = torch.from_numpy(wl.new_slots).cuda()
    q = to_dev(wl.q, "bf16")
    out = torch.empty_like(q)
    bt = torch.from_numpy(wl.block_tables).cuda()
    cl = torch.from_numpy(wl.context_lens).cuda()
    S, Hq, D = wl.q.shape
    max_ctx = int(wl.context_lens.max())
    ws_bytes = pa.pa_decode_workspace_bytes(S, Hq, wl.num_kv_heads, D, max_ctx, 0)
    ws = torch.empty(max(1, (ws_bytes + 3) // 4), dtype=torch.float32, device="cuda")

    def step():
        pa.pa_decode_append(out, q, new_k, new_v, new_slots, pool.k, pool.v, bt, cl, max_ctx,
                            float(wl.scale), pool.desc, workspace=ws)

    for _ in range(warmup):
        step()
    kv = wl.kv_bytes // 2  # one byte per element instead of two
    cold = timer.calls(step, steps, cold=True)
    hot = timer.calls(step, steps, cold=False)
    return {"kv_dtype": "fp8_e4m3", "k_scale": float(FP8_K_SCALE), "v_scale": float(FP8_V_SCALE),
            "kv_bytes_per_step": kv, "step_cold": dist(cold, kv, tokens=S),
            "step_hot": dist(hot, kv, tokens=S)}


def bench_spec_verify(timer, steps, warmup):
    """One verification round of speculative decoding on the 64-sequence 8B
    batch (contexts U[128, 4096), k = 4 drafts, vocabulary 128256): write the
    k + 1 new tokens' K/V, the target's attention over those k + 1 rows
    (pa_prefill_chunk), and rejection sampling (pa_rejection_sample)."""
    import torch

    import paged_kv_cache_396_amd as pa
    from gpu_util import GpuPool, to_dev
    from workloads import make_spec_verify

    w = make_spec_verify()
    a = w.attn
    pool = GpuPool(a.num_blocks, a.num_kv_heads, a.head_dim, a.dtype)
    pool.write(a.hist_k, a.hist_v, a.hist_slots)
    nk, nv = to_dev(a.new_k, a.dtype), to_dev(a.new_v, a.dtype)
    ns = torch.from_numpy(a.new_slots).cuda()
    q = to_dev(a.q, a.dtype)
    out = torch.empty_like(q)
    bt = torch.from_numpy(a.block_tables).cuda()
    qsl = torch.from_numpy(a.query_start_loc).cuda()
    cl = torch.from_numpy(a.context_lens).cuda()
    k1 = int(w.target_probs.shape[1])
    tp = torch.from_numpy(w.target_probs).cuda()
    dp = torch.from_numpy(w.draft_probs).cuda()
    tk = torch.from_numpy(w.draft_tokens).cuda()
    uu = torch.from_numpy(w.uniforms).cuda()
    sws = torch.empty(pa.pa_rejection_sample_workspace_bytes(a.num_reqs, int(w.target_probs.shape[2])),
                      dtype=torch.uint8, device="cuda")
    ot = torch.empty((a.num_reqs, k1), dtype=torch.int32, device="cuda")
    on = torch.empty((a.num_reqs,), dtype=torch.int32, device="cuda")

    def write():
        pa.pa_reshape_and_cache(nk, nv, ns, pool.k, pool.v, pool.desc)

    max_ctx = int(a.context_lens.max())
    Tq, Hq, D = a.q.shape
    pws_bytes = pa.pa_prefill_chunk_workspace_bytes(a.num_reqs, Tq, k1, max_ctx, Hq, a.num_kv_heads,
                                                    D, 0)
    pws = torch.empty(max(1, (pws_bytes + 3) // 4), dtype=torch.float32, device="cuda")

    def attend():
        pa.pa_prefill_chunk(out, q, pool.k, pool.v, bt, qsl, cl, k1, float(a.scale), pool.desc,
                            max_context_len=max_ctx, workspace=pws)

    def attend_unsplit():
        pa.pa_prefill_chunk(out, q, pool.k, pool.v, bt, qsl, cl, k1, float(a.scale), pool.desc)

    def sample():
        pa.pa_rejection_sample(tp, dp, tk, uu, ot, on, workspace=sws)

    def step():
        write()
        attend()
        sample()

    for _ in range(warmup):
        step()
    round_cold = timer.calls(step, steps, cold=True)
    attn_cold = timer.calls(attend, steps, cold=True)
    attn_unsplit_cold = timer.calls(attend_unsplit, steps, cold=True)
    samp_cold = timer.calls(sample, steps, cold=True)
    n = on.cpu().numpy()
    V = int(w.target_probs.shape[2])
    samp_bytes = int(sum(V * 4 * (1 if int(c) == k1 else 2) for c in n))
    kv = int(a.context_lens.astype(np.int64).sum()) * 2 * a.num_kv_heads * a.head_dim * 2
    return {
        "batch": a.num_reqs, "k": k1 - 1, "vocab": V,
        "tokens_per_round_mean": round(float(n.mean()), 4),
        "round_cold": dist(round_cold),
        "tokens_per_s": round(float(n.sum()) / (np.median(round_cold) * 1e-3), 1),
        "verify_attention_call": "pa_prefill_chunk, k + 1 rows per request, automatic split-K over the keys",
        "verify_attention_cold": dist(attn_cold, kv),
        "verify_attention_unsplit_cold": dist(attn_unsplit_cold, kv),
        "rejection_sample_cold": dist(samp_cold, samp_bytes),
    }


def bench_block_pool(timer, steps=10):
    """Copy-on-write machinery: pa_copy_blocks of 4096 block pairs of an
    8B-layer pool, and the host pool's operation rate on a parallel-sampling
    pattern."""
    import torch

    import paged_kv_cache_396_amd as pa

    nb, Hkv, D, npairs = 16384, 8, 128, 4096
    desc = pa.cache_desc(nb, Hkv, D, pa.PA_BF16)
    nbytes = pa.pa_cache_bytes(desc)
    k = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    v = torch.empty_like(k)
    k.fill_(1)
    v.fill_(2)
    perm = np.random.default_rng(7).permutation(nb)[: 2 * npairs].astype(np.int32)
    pairs = torch.from_numpy(perm.reshape(npairs, 2).copy()).cuda()
    pa.pa_copy_blocks(k, v, pairs, desc)
    cold = timer.calls(lambda: pa.pa_copy_blocks(k, v, pairs, desc), steps, cold=True)
    moved = npairs * 2 * Hkv * 16 * D * 2 * 2  # K and V, read and written
    del k, v
    t0 = time.perf_counter()
    pool = pa.BlockPool(1 << 17)
    ops = 0
    rng = np.random.default_rng(3)
    for p in range(256):
        base = p * 8
        prompt = rng.integers(0, 32000, size=300).tolist()
        c = pool.add_request(base, prompt)
        pool.allocate_slots(base, prompt[c:])
        ops += 2
        for s in range(1, 4):
            pool.fork(base, base + s)
            ops += 1
        for _ in range(32):
            for s in range(4):
                pool.allocate_slots(base + s, [int(rng.integers(0, 32000))])
                ops += 1
        for s in range(4):
            pool.free_request(base + s)
            ops += 1
    host_s = time.perf_counter() - t0
    return {"copy_pairs": npairs, "copy_bytes_moved": moved, "copy_cold": dist(cold, moved),
            "host_pool_ops": ops, "host_pool_ops_per_s": round(ops / host_s, 1),
            "host_pool_note": "through the ctypes binding, one call per operation"}


def read_ceiling(timer, steps=10):
    """Read bandwidth of the streaming probe over 1 GiB of shuffled 4 KiB
    tiles: the practical ceiling for paged K/V reads on this device."""
    import torch

    import paged_kv_cache_396_amd as pa

    nbytes = 1 << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    buf.fill_(1)
    ntiles = nbytes // 4096
    order = torch.from_numpy(np.random.default_rng(396).permutation(ntiles).astype(np.int32)).cuda()
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    for _ in range(3):
        pa.pa_bw_probe(buf, order, sink)
    ms = timer.loop(lambda: pa.pa_bw_probe(buf, order, sink), steps)
    gbs = nbytes / (ms * 1e-3) / 1e9
    del buf
    return {"pattern": "1 GiB of 4 KiB tiles read once in shuffled order (pa_bw_probe)",
            "gbs": round(gbs, 1), "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4)}


# ----------------------------------------------------------------------------


def extras(timer, n):
    """The sections beside the five configurations: the read ceiling, fp8 pools
    (prefill and decode step), a speculative verification round and the host
    block pool."""
    return {"hbm_read_ceiling": read_ceiling(timer),
            "fp8_prefill_chunk": bench_prefill(timer, n, 3, fp8=True),
            "fp8_kv_step": bench_fp8_decode(timer, n, 5),
            "spec_verify_round": bench_spec_verify(timer, n, 3),
            "block_pool": bench_block_pool(timer)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--configs", default="c1,c2,c3,c4,c5",
                    help="comma list of c1..c5 (c2, the headline, always runs)")
    ap.add_argument("--no-headline", action="store_true",
                    help="skip the headline workload (profiling one configuration alone); "
                         "prints the configuration sections only")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip fp8 pools, speculative verification, block pool and the read probe")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=10.0,
                    help="seconds of oracle time for the headline workload (others get less)")
    ap.add_argument("--prefill-only", action="store_true",
                    help="time only pa_prefill_chunk on the long-context batch (for profiling)")
    ap.add_argument("--extras-only", action="store_true",
                    help="time only the extra sections (fp8 pools, speculative verification, "
                         "block pool, read probe; for profiling)")
    ap.add_argument("--calib-copy", type=int, default=0,
                    help="instead of the bench, run N plain 1 GiB device copies (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the paged-attention path has no multi-GPU part in this library)", file=sys.stderr)
        sys.exit(2)

    import torch

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.calib_copy:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        src.fill_(1)
        for _ in range(args.calib_copy):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calib_copy_bytes": n, "copies": args.calib_copy}))
        return

    timer = Timer()
    if args.prefill_only:
        print(json.dumps({"prefill_chunk": bench_prefill(timer, args.steps, args.warmup),
                          "fp8_prefill_chunk": bench_prefill(timer, args.steps, args.warmup, fp8=True)}),
              flush=True)
        return

    if args.extras_only:
        print(json.dumps(extras(timer, min(args.steps, 30))), flush=True)
        return

    want = [c.strip() for c in args.configs.split(",") if c.strip()]
    budget = 0.0 if args.no_cpu_baseline else args.cpu_budget

    def log(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    if args.no_headline:
        sections = {"c1": bench_c1, "c3": bench_c3, "c4": bench_c4, "c5": bench_c5}
        out = {}
        for c in want:
            if c in sections:
                log(f"{c} {CONFIGS[c]}")
                out[f"{c}_{CONFIGS[c]}"] = sections[c](timer, args.steps, args.warmup, budget / 2)
        if "c5" in want:
            out["prefill_chunk"] = bench_prefill(timer, min(args.steps, 30), 3)
        print(json.dumps({"configs": out}), flush=True)
        return

    log("c2 llama3_8b_b64")
    c2, db2 = bench_c2(timer, args.steps, args.warmup, budget)
    kv = db2.wl.kv_bytes
    S = db2.wl.num_seqs
    cold = c2["step_cold"]
    ms_step = cold["median_ms"]
    value = kv / (ms_step * 1e-3) / 1e9
    traffic = _traffic("llama3_8b_b64")
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "llama3_8b_b64",
            "num_seqs": S, "num_q_heads": 32, "num_kv_heads": 8, "head_dim": 128,
            "block_size": 16, "context_lens": "U[128,4096]", "ctx_sum": c2["ctx_sum"],
            "num_blocks": c2["num_blocks"], "decode_schedule": c2["decode_schedule"],
            "new_tokens_per_step": S, "parallelism": "single GPU",
            "timing": "median of per-step HIP-event times; before each step an untimed scrub "
                      "writes 512 MiB and reads another 512 MiB (caches evicted, left clean)",
        },
        "tokens_per_s": round(S / (ms_step * 1e-3), 1),
        "hbm_frac": round(value / HBM_PEAK_GBS, 4),
        "kv_bytes_per_step": kv,
        "cold_write_scrub": {k: c2["step_cold_write_scrub"][k] for k in ("median_ms", "gbs", "hbm_frac")},
        "hot": {"median_ms": c2["step_hot"]["median_ms"], "gbs": c2["step_hot"]["gbs"],
                "hbm_frac": c2["step_hot"]["hbm_frac"],
                "loop_ms_per_step": c2["step_hot_loop_ms"],
                "loop_hbm_frac": round(kv / (c2["step_hot_loop_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
        "roofline": {
            "bound": "hbm",
            "kernel": "pa_decode_append call (decode_balanced_kernel + decode_balanced_reduce_kernel)",
            "achieved": round(value, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(value / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "basis": "algorithmic KV bytes / median scrubbed call time (events on the launch stream)",
            "dominant_kernel_rocprof": _kernel_profile("llama3_8b_b64", kv),
        },
        "cpu_baseline": c2.get("cpu_baseline"),
        "configs": {},
    }
    del db2
    sections = {"c1": bench_c1, "c3": bench_c3, "c4": bench_c4, "c5": bench_c5}
    for c in ("c1", "c2", "c3", "c4", "c5"):
        if c not in want:
            continue
        if c == "c2":
            line["configs"]["c2_" + CONFIGS[c]] = c2
            continue
        log(f"{c} {CONFIGS[c]}")
        line["configs"][f"{c}_{CONFIGS[c]}"] = sections[c](timer, args.steps, args.warmup,
                                                          budget / 2 if c != "c1" else budget)
    if "c5" in want:
        log("prefill chunk (bf16)")
        line["prefill_chunk"] = bench_prefill(timer, min(args.steps, 30), 3)
    if not args.no_extras:
        log("extras")
        line.update(extras(timer, min(args.steps, 30)))
        line["roofline"]["frac_of_read_ceiling"] = round(value / line["hbm_read_ceiling"]["gbs"], 4)
        line["fp8_kv_step"]["speedup_vs_bf16_step_cold"] = round(
            ms_step / line["fp8_kv_step"]["step_cold"]["median_ms"], 3)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
