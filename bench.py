"""Benchmark of the paged-attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the decode hot path over one batch: scatter the step's
new K/V tokens into the block pool (pa_reshape_and_cache), then paged decode
attention over every sequence's full context (pa_decode, with automatic
split-K).  The default workload is one Llama-3.1-8B-shaped layer: 64
sequences, context lengths U[128, 4096], 32 q / 8 kv heads, head_dim 128,
bf16, 16-token blocks shuffled over a pool 1.25x the need.  All inputs are
seeded synthetic data resident in HBM before timing starts.

The same run also times pa_prefill_chunk on the prefill half of the
long-context mixed batch (4 requests, 512-token causal chunks against 4096
prior paged tokens, 32 q / 8 kv heads, head_dim 128, bf16) and reports it
under ``prefill_chunk`` against the bf16 matrix-core peak (skip with
--no-prefill).

Prints one JSON line.  ``value`` is KV GB/s over the timed steps (the K/V
bytes attention must read, one read per kv head, divided by step time);
tokens/s and the HBM fraction are reported beside it.  ``roofline`` refers
to the decode call (partition kernel + split-K merge), timed with HIP events
on the launch stream.  ``cpu_baseline`` times the fp64 CPU oracle on a
bounded sample of the same workload.
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

METRIC = "paged decode attn: KV GB/s and % of MI355X HBM peak; decode tokens/s"
HBM_PEAK_GBS = 8000.0  # MI355X published HBM3E bandwidth
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X published dense bf16 matrix-core peak
WORKLOADS = {
    "llama3_8b_b64": 2,
    "llama2_70b_b256": 3,
    "shared_prefix_32x4": 4,
    "long_mixed_decode": 5,
    "tiny_f32": 1,
}
PMC_SUMMARY = os.path.join(ROOT, "profiles", "decode_{name}_pmc.txt")


def _source_hash():
    h = hashlib.sha256()
    for f in ("decode.hip", "pa_device.h"):
        with open(os.path.join(ROOT, "paged_kv_cache_396_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _traffic(name, decode_launch_bytes):
    """HBM bytes per decode call from committed rocprofv3 counter runs, if
    they were taken on the current decode source; else None."""
    path = PMC_SUMMARY.format(name=name)
    if not os.path.exists(path):
        return None
    d = {}
    with open(path) as f:
        for line in f:
            if line.startswith("#") or ":" not in line:
                continue
            k, v = line.split(":", 1)
            d[k.strip()] = v.strip()
    if d.get("source_hash") != _source_hash():
        return None
    return int(float(d["hbm_bytes_per_call"]))


def cpu_baseline(wl, budget_s=10.0):
    """The oracle, untouched, on the host: whole batches until ``budget_s``,
    first on one core, then with the batch's sequences spread over a thread
    pool of every core this process may use (at most 16; NumPy's matrix
    products and exponentials release the GIL; BLAS one thread per worker)."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle
    from workloads import poison_bits

    try:
        from threadpoolctl import threadpool_limits

        limiter = threadpool_limits(1)
    except Exception:  # pragma: no cover
        limiter = None
    pk = oracle.new_pool(wl.num_blocks, wl.num_kv_heads, wl.head_dim, wl.dtype, poison_bits(wl.dtype))
    pv = pk.copy()
    oracle.reshape_and_cache_fast(pk, pv, wl.hist_k, wl.hist_v, wl.hist_slots)
    oracle.reshape_and_cache_fast(pk, pv, wl.new_k, wl.new_v, wl.new_slots)

    def timed(run):
        t0 = time.perf_counter()
        n = 0
        while True:
            run()
            n += 1
            el = time.perf_counter() - t0
            if el >= budget_s:
                return n, el

    def one_batch():
        oracle.decode(wl.q, pk, pv, wl.block_tables, wl.context_lens, wl.scale, wl.dtype)

    n1, el1 = timed(one_batch)
    cores = max(1, min(16, len(os.sched_getaffinity(0))))
    # longest sequences first, dealt round-robin, so the workers finish together
    order = np.argsort(-wl.context_lens.astype(np.int64), kind="stable")
    shares = [order[i::cores].tolist() for i in range(cores)]
    with ThreadPoolExecutor(max_workers=cores) as ex:
        def all_cores():
            list(ex.map(lambda sq: oracle.decode(wl.q, pk, pv, wl.block_tables, wl.context_lens,
                                                 wl.scale, wl.dtype, seqs=sq), shares))

        nN, elN = timed(all_cores)
    if limiter is not None:
        limiter.unregister() if hasattr(limiter, "unregister") else None
    return {
        "value": round(wl.kv_bytes * nN / elN / 1e9, 4),
        "unit": "GB/s",
        "cores": cores,
        "kind": "oracle",
        "sample": f"{nN} full decode batch(es) of {wl.name} ({wl.num_seqs} seqs, "
                  f"{int(wl.context_lens.sum())} tokens) in {elN:.1f} s on {cores} threads, numpy fp64, "
                  f"BLAS 1 thread each; one core: {n1} batch(es) in {el1:.1f} s",
        "tokens_per_s": round(wl.num_seqs * nN / elN, 2),
        "one_core": {"value": round(wl.kv_bytes * n1 / el1 / 1e9, 4), "unit": "GB/s",
                     "tokens_per_s": round(wl.num_seqs * n1 / el1, 2)},
    }


def prefill_flops(wl):
    """Causal-useful FLOPs of one pa_prefill_chunk call: every query row does
    a 2-FLOP multiply-add per dim for Q.K and for P.V over the keys it sees."""
    tot = 0
    for r in range(wl.num_reqs):
        n_r = int(wl.query_start_loc[r + 1] - wl.query_start_loc[r])
        prior = int(wl.context_lens[r]) - n_r
        tot += n_r * prior + n_r * (n_r + 1) // 2  # sum over i of (prior + i + 1)
    return tot * wl.num_q_heads * 4 * wl.head_dim


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


def bench_prefill(steps, warmup, fp8=False):
    """Time pa_prefill_chunk on the long-context mixed batch's prefill half
    (bf16 pools, or fp8 pools holding the same rows quantized)."""
    import torch

    import paged_kv_cache_396_amd as pa
    from workloads import make_prefill

    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from gpu_util import GpuPool, to_dev  # noqa: E402

    wl = make_prefill(5)
    pool = _Fp8Pool(wl) if fp8 else GpuPool(wl.num_blocks, wl.num_kv_heads, wl.head_dim, wl.dtype)
    pool.write(wl.hist_k, wl.hist_v, wl.hist_slots)
    pool.write(wl.new_k, wl.new_v, wl.new_slots)
    q = to_dev(wl.q, wl.dtype)
    out = torch.empty_like(q)
    bt = torch.from_numpy(wl.block_tables).cuda()
    qsl = torch.from_numpy(wl.query_start_loc).cuda()
    cl = torch.from_numpy(wl.context_lens).cuda()
    stream = torch.cuda.current_stream()

    def call():
        pa.pa_prefill_chunk(out, q, pool.k, pool.v, bt, qsl, cl, wl.max_q_len, float(wl.scale),
                            pool.desc)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    # back-to-back launches between two events: the average is the kernel's
    # own duration plus the small gap between consecutive launches
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(steps):
        call()
    b.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    fl = prefill_flops(wl)
    tf = fl / (ms * 1e-3) / 1e12
    return {
        "workload": "long_mixed_prefill", "kv_dtype": "fp8_e4m3" if fp8 else "bf16",
        "num_reqs": wl.num_reqs, "chunk_tokens": int(wl.max_q_len),
        "prior_tokens": int(wl.context_lens[0]) - int(wl.max_q_len),
        "num_q_heads": wl.num_q_heads, "num_kv_heads": wl.num_kv_heads, "head_dim": wl.head_dim,
        "calls": steps, "call_ms": round(ms, 5), "causal_flops": fl,
        "q_tokens_per_s": round(wl.total_q_tokens / (ms * 1e-3), 1),
        "roofline": {"bound": "mfma", "kernel": "prefill_chunk_kernel", "achieved": round(tf, 2),
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4)},
    }


def bench_mixed_concurrent(steps=10, warmup=3):
    """The long-context mixed batch as one step: its decode half (8 x 32768)
    and its prefill half (4 x 512-token chunks over 4096 prior tokens) read
    one shared pool.  Timed back to back on one stream, and concurrently on
    two streams (default priority) so the prefill's matrix work can overlap
    the decode's HBM reads."""
    import torch

    import paged_kv_cache_396_amd as pa
    from workloads import make_mixed

    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from gpu_util import GpuPool, to_dev  # noqa: E402

    dec, pre = make_mixed(0)
    pool = GpuPool(dec.num_blocks, dec.num_kv_heads, dec.head_dim, dec.dtype)
    for wl in (dec, pre):
        pool.write(wl.hist_k, wl.hist_v, wl.hist_slots)
        pool.write(wl.new_k, wl.new_v, wl.new_slots)
    dq = to_dev(dec.q, dec.dtype)
    dout = torch.empty_like(dq)
    dbt = torch.from_numpy(dec.block_tables).cuda()
    dcl = torch.from_numpy(dec.context_lens).cuda()
    S, Hq, D = dec.q.shape
    max_ctx = int(dec.context_lens.max())
    ws_bytes = pa.pa_decode_workspace_bytes(S, Hq, dec.num_kv_heads, D, max_ctx, 0)
    ws = torch.empty(max(1, (ws_bytes + 3) // 4), dtype=torch.float32, device="cuda")
    pq = to_dev(pre.q, pre.dtype)
    pout = torch.empty_like(pq)
    pbt = torch.from_numpy(pre.block_tables).cuda()
    pqsl = torch.from_numpy(pre.query_start_loc).cuda()
    pcl = torch.from_numpy(pre.context_lens).cuda()

    def decode(stream=None):
        pa.pa_decode(dout, dq, pool.k, pool.v, dbt, dcl, max_ctx, float(dec.scale), pool.desc,
                     workspace=ws, stream=stream)

    def prefill(stream=None):
        pa.pa_prefill_chunk(pout, pq, pool.k, pool.v, pbt, pqsl, pcl, pre.max_q_len,
                            float(pre.scale), pool.desc, stream=stream)

    main = torch.cuda.current_stream()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()

    def seq_step():
        decode(main)
        prefill(main)

    def conc_step():
        ev = torch.cuda.Event()
        ev.record(main)
        s1.wait_event(ev)
        s2.wait_event(ev)
        decode(s1)
        prefill(s2)
        e1, e2 = torch.cuda.Event(), torch.cuda.Event()
        e1.record(s1)
        e2.record(s2)
        main.wait_event(e1)
        main.wait_event(e2)

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(main)
        for _ in range(steps):
            fn()
        b.record(main)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / steps

    ms_dec = timed(lambda: decode(main))
    ms_pre = timed(lambda: prefill(main))
    ms_seq = timed(seq_step)
    ms_conc = timed(conc_step)
    return {
        "workload": "long_mixed (8 x 32768 decode + 4 x 512-token prefill chunks, one pool)",
        "decode_ms": round(ms_dec, 5), "prefill_ms": round(ms_pre, 5),
        "sequential_ms": round(ms_seq, 5), "concurrent_ms": round(ms_conc, 5),
        "overlap_gain": round(ms_seq / ms_conc, 3),
        "decode_kv_gbs_in_concurrent_step": round(dec.kv_bytes / (ms_conc * 1e-3) / 1e9, 1),
    }


def bench_shared_prefix(wl, pool, q, bt, cl, max_ctx, steps, warmup):
    """pa_decode_shared_prefix on a workload whose consecutive groups of
    samples share their prompt blocks, beside pa_decode on the same inputs."""
    import torch

    import paged_kv_cache_396_amd as pa

    prompt_of = wl.extra["prompt_of"]
    group = int(np.sum(prompt_of == prompt_of[0]))
    n_groups = wl.num_seqs // group
    plen = int(wl.extra["prompt_len"])
    S, Hq, D = wl.q.shape
    prefix = torch.full((n_groups,), plen, dtype=torch.int32, device="cuda")
    ws_bytes = pa.pa_decode_shared_prefix_workspace_bytes(S, Hq, wl.num_kv_heads, D, max_ctx, group,
                                                          plen)
    ws = torch.empty((ws_bytes + 3) // 4, dtype=torch.float32, device="cuda")
    out = torch.empty_like(q)

    def call():
        pa.pa_decode_shared_prefix(out, q, pool.k, pool.v, bt, cl, max_ctx, float(wl.scale), prefix,
                                   group, plen, pool.desc, ws)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    stream = torch.cuda.current_stream()
    a.record(stream)
    for _ in range(steps):
        call()
    b.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    unique = (n_groups * plen + int(wl.context_lens.sum()) - S * plen) * 2 * wl.num_kv_heads * D * 2
    return {
        "group_size": group, "prefix_tokens": plen, "call_ms": round(ms, 5),
        "logical_gbs": round(wl.kv_bytes / (ms * 1e-3) / 1e9, 1),
        "unique_kv_bytes": unique,
        "unique_gbs": round(unique / (ms * 1e-3) / 1e9, 1),
        "unique_hbm_frac": round(unique / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
    }


def bench_fp8_decode(wl, steps, warmup, partition=0):
    """The decode step (pa_decode_append: cache write fused with decode) of
    the same workload with fp8 (E4M3) pools: the same bf16 K/V rows are
    quantized into the pools with per-pool scales, and attention reads half
    the bytes.  The two-call step and pa_decode alone are timed beside it."""
    import torch

    import paged_kv_cache_396_amd as pa
    from gpu_util import to_dev
    from workloads import FP8_K_SCALE, FP8_V_SCALE

    dev = "cuda"
    desc = pa.cache_desc(wl.num_blocks, wl.num_kv_heads, wl.head_dim, pa.PA_FP8_E4M3,
                         float(FP8_K_SCALE), float(FP8_V_SCALE))
    nbytes = pa.pa_cache_bytes(desc)
    pk = torch.full((nbytes,), 0x7F, dtype=torch.uint8, device=dev)
    pv = torch.full((nbytes,), 0x7F, dtype=torch.uint8, device=dev)
    hs = torch.from_numpy(wl.hist_slots).to(dev)
    pa.pa_reshape_and_cache(to_dev(wl.hist_k, "bf16"), to_dev(wl.hist_v, "bf16"), hs, pk, pv, desc)
    new_k, new_v = to_dev(wl.new_k, "bf16"), to_dev(wl.new_v, "bf16")
    new_slots = torch.from_numpy(wl.new_slots).to(dev)
    q = to_dev(wl.q, "bf16")
    out = torch.empty_like(q)
    bt = torch.from_numpy(wl.block_tables).to(dev)
    cl = torch.from_numpy(wl.context_lens).to(dev)
    S, Hq, D = wl.q.shape
    max_ctx = int(wl.context_lens.max())
    ws_bytes = pa.pa_decode_workspace_bytes(S, Hq, wl.num_kv_heads, D, max_ctx, partition)
    ws = torch.empty(max(1, (ws_bytes + 3) // 4), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def decode():
        pa.pa_decode(out, q, pk, pv, bt, cl, max_ctx, float(wl.scale), desc,
                     partition_size=partition, workspace=ws)

    def step():
        pa.pa_decode_append(out, q, new_k, new_v, new_slots, pk, pv, bt, cl, max_ctx,
                            float(wl.scale), desc, partition_size=partition, workspace=ws)

    def two_call_step():
        pa.pa_reshape_and_cache(new_k, new_v, new_slots, pk, pv, desc)
        decode()

    def timed(fn):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(steps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / steps

    for _ in range(warmup):
        step()
        two_call_step()
    torch.cuda.synchronize()
    ms_step = timed(step)
    ms_two = timed(two_call_step)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for e0, e1 in evs:
        pa.pa_reshape_and_cache(new_k, new_v, new_slots, pk, pv, desc)
        e0.record(stream)
        decode()
        e1.record(stream)
    torch.cuda.synchronize()
    dec = float(np.median([e0.elapsed_time(e1) for e0, e1 in evs]))
    kv = wl.kv_bytes // 2  # one byte per element instead of two
    return {
        "kv_dtype": "fp8_e4m3", "k_scale": float(FP8_K_SCALE), "v_scale": float(FP8_V_SCALE),
        "ms_per_step": round(ms_step, 5), "tokens_per_s": round(S / (ms_step * 1e-3), 1),
        "kv_bytes_per_step": kv, "step_gbs": round(kv / (ms_step * 1e-3) / 1e9, 1),
        "two_call_ms_per_step": round(ms_two, 5),
        "decode_call_median_ms": round(dec, 5),
        "decode_call_gbs": round(kv / (dec * 1e-3) / 1e9, 1),
        "decode_call_hbm_frac": round(kv / (dec * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
    }


def bench_spec_verify(steps, warmup):
    """One verification round of speculative decoding on the 64-sequence 8B
    batch (contexts U[128, 4096), k = 4 drafts, Llama-3 vocabulary of 128256):
    write the k + 1 new tokens' K/V, the target's attention over those k + 1
    rows (pa_prefill_chunk), and rejection sampling (pa_rejection_sample)."""
    import torch

    import paged_kv_cache_396_amd as pa
    from gpu_util import GpuPool, to_dev
    from workloads import make_spec_verify

    dev = "cuda"
    w = make_spec_verify()
    a = w.attn
    pool = GpuPool(a.num_blocks, a.num_kv_heads, a.head_dim, a.dtype)
    pool.write(a.hist_k, a.hist_v, a.hist_slots)
    nk, nv = to_dev(a.new_k, a.dtype), to_dev(a.new_v, a.dtype)
    ns = torch.from_numpy(a.new_slots).to(dev)
    q = to_dev(a.q, a.dtype)
    out = torch.empty_like(q)
    bt = torch.from_numpy(a.block_tables).to(dev)
    qsl = torch.from_numpy(a.query_start_loc).to(dev)
    cl = torch.from_numpy(a.context_lens).to(dev)
    k1 = int(w.target_probs.shape[1])
    tp = torch.from_numpy(w.target_probs).to(dev)
    dp = torch.from_numpy(w.draft_probs).to(dev)
    tk = torch.from_numpy(w.draft_tokens).to(dev)
    uu = torch.from_numpy(w.uniforms).to(dev)
    sws = torch.empty(pa.pa_rejection_sample_workspace_bytes(a.num_reqs, int(w.target_probs.shape[2])),
                      dtype=torch.uint8, device=dev)
    ot = torch.empty((a.num_reqs, k1), dtype=torch.int32, device=dev)
    on = torch.empty((a.num_reqs,), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()

    # the same attention as shared-prefix decode: the k + 1 rows of a request
    # are a group of "sequences" with identical block tables whose contexts
    # end at their own positions; the blocks before the first row's position
    # are the group's shared prefix, read once per group
    ctx = a.context_lens.astype(np.int64)
    rows_ctx = (ctx[:, None] - (k1 - 1) + np.arange(k1)[None, :]).reshape(-1).astype(np.int32)
    rows_bt = torch.from_numpy(np.repeat(a.block_tables, k1, axis=0)).to(dev)
    rows_cl = torch.from_numpy(rows_ctx).to(dev)
    prefix_np = ((ctx - (k1 - 1)) // 16 * 16).astype(np.int32)
    prefix = torch.from_numpy(prefix_np).to(dev)
    max_ctx = int(ctx.max())
    max_prefix = int(prefix_np.max())
    sp_ws = torch.empty(pa.pa_decode_shared_prefix_workspace_bytes(
        a.num_reqs * k1, a.num_q_heads, a.num_kv_heads, a.head_dim, max_ctx, k1, max_prefix) // 4 + 1,
        dtype=torch.float32, device=dev)
    out_sp = torch.empty_like(q)

    def write():
        pa.pa_reshape_and_cache(nk, nv, ns, pool.k, pool.v, pool.desc)

    def attend():
        pa.pa_prefill_chunk(out, q, pool.k, pool.v, bt, qsl, cl, k1, float(a.scale), pool.desc)

    def attend_grouped():
        pa.pa_decode_shared_prefix(out_sp, q, pool.k, pool.v, rows_bt, rows_cl, max_ctx,
                                   float(a.scale), prefix, k1, max_prefix, pool.desc, sp_ws)

    def sample():
        pa.pa_rejection_sample(tp, dp, tk, uu, ot, on, workspace=sws)

    def step():
        write()
        attend()
        sample()

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / steps

    def per_call(fn):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(steps)]
        for x, y in evs:
            x.record(stream)
            fn()
            y.record(stream)
        torch.cuda.synchronize()
        return float(np.median([x.elapsed_time(y) for x, y in evs]))

    attn_ms = per_call(attend)
    grouped_ms = per_call(attend_grouped)
    samp_ms = per_call(sample)
    n = on.cpu().numpy()
    V = int(w.target_probs.shape[2])
    # rows the sampler streams: p_i and q_i after a rejection at i, p_k after k acceptances
    samp_bytes = int(sum(V * 4 * (1 if int(c) == k1 else 2) for c in n))
    kv = int(a.context_lens.astype(np.int64).sum()) * 2 * a.num_kv_heads * a.head_dim * 2
    return {
        "batch": a.num_reqs, "k": k1 - 1, "vocab": V,
        "ms_per_round": round(ms_step, 5),
        "tokens_per_round_mean": round(float(n.mean()), 4),
        "tokens_per_s": round(float(n.sum()) / (ms_step * 1e-3), 1),
        "verify_attention_ms": round(attn_ms, 5),
        "verify_attention_kv_gbs": round(kv / (attn_ms * 1e-3) / 1e9, 1),
        "verify_attention_hbm_frac": round(kv / (attn_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "verify_attention_grouped_ms": round(grouped_ms, 5),
        "verify_attention_grouped_kv_gbs": round(kv / (grouped_ms * 1e-3) / 1e9, 1),
        "rejection_sample_ms": round(samp_ms, 5),
        "rejection_sample_bytes": samp_bytes,
        "rejection_sample_gbs": round(samp_bytes / (samp_ms * 1e-3) / 1e9, 1),
    }


def bench_block_pool(steps=10):
    """Copy-on-write machinery: pa_copy_blocks of 4096 block pairs of an
    8B-layer pool (8 kv heads, d 128, bf16: 64 KiB per pair in K and V), and
    the host pool's operation rate on a parallel-sampling pattern."""
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
    for _ in range(2):
        pa.pa_copy_blocks(k, v, pairs, desc)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    stream = torch.cuda.current_stream()
    a.record(stream)
    for _ in range(steps):
        pa.pa_copy_blocks(k, v, pairs, desc)
    b.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    moved = npairs * 2 * Hkv * 16 * D * 2 * 2  # K and V, read and written
    del k, v
    # host pool: 256 prompts of 300 tokens, 4 samples each, 32 decode steps
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
    return {
        "copy_pairs": npairs, "copy_ms": round(ms, 5), "copy_bytes_moved": moved,
        "copy_gbs": round(moved / (ms * 1e-3) / 1e9, 1),
        "host_pool_ops": ops, "host_pool_ops_per_s": round(ops / host_s, 1),
        "host_pool_note": "through the ctypes binding, one call per operation",
    }


def bench_bulk_write(steps=5):
    """pa_reshape_and_cache of a whole Llama-2-70B-shaped layer history in one
    call: 256 sequences x 2048 tokens (524,288 tokens), 8 kv heads, d 128,
    bf16, each sequence's tokens in order into its shuffled blocks (the shape
    of a prefill's cache fill).  Random bits: the copy is value-blind."""
    import torch

    import paged_kv_cache_396_amd as pa

    S, ctx, Hkv, D = 256, 2048, 8, 128
    T = S * ctx
    num_blocks = int(1.25 * T // 16)
    g = torch.Generator(device="cuda")
    g.manual_seed(396_003)
    k = torch.randint(-2 ** 15, 2 ** 15, (T, Hkv, D), dtype=torch.int16, device="cuda",
                      generator=g).view(torch.bfloat16)
    v = torch.randint(-2 ** 15, 2 ** 15, (T, Hkv, D), dtype=torch.int16, device="cuda",
                      generator=g).view(torch.bfloat16)
    perm = torch.randperm(num_blocks, device="cuda", generator=g)[: T // 16].to(torch.int64)
    tok = torch.arange(T, device="cuda", dtype=torch.int64)
    slots = perm[tok // 16] * 16 + tok % 16
    desc = pa.cache_desc(num_blocks, Hkv, D, torch.bfloat16)
    nbytes = pa.pa_cache_bytes(desc)
    kc = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    vc = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    pa.pa_reshape_and_cache(k, v, slots, kc, vc, desc)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(steps):
        pa.pa_reshape_and_cache(k, v, slots, kc, vc, desc)
    b.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    moved = 4 * T * Hkv * D * 2  # K and V read once and written once
    return {"workload": "llama2_70b_layer_history_fill", "tokens": T, "bytes_moved": moved,
            "call_ms": round(ms, 4), "gbs": round(moved / (ms * 1e-3) / 1e9, 1),
            "hbm_frac": round(moved / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}


def read_ceiling(steps=10):
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
    stream = torch.cuda.current_stream()
    for _ in range(3):
        pa.pa_bw_probe(buf, order, sink)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(steps):
        pa.pa_bw_probe(buf, order, sink)
    b.record(stream)
    torch.cuda.synchronize()
    gbs = nbytes * steps / (a.elapsed_time(b) * 1e-3) / 1e9
    del buf
    return {"pattern": "1 GiB of 4 KiB tiles read once in shuffled order (pa_bw_probe)",
            "gbs": round(gbs, 1), "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="llama3_8b_b64", choices=sorted(WORKLOADS))
    ap.add_argument("--partition", type=int, default=0, help="0 auto, <0 no split, >0 tokens")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true", help="skip the prefill-chunk timing")
    ap.add_argument("--prefill-only", action="store_true",
                    help="time only pa_prefill_chunk (for profiling it alone)")
    ap.add_argument("--fp8-only", action="store_true",
                    help="time only the decode step over fp8 pools (for profiling)")
    ap.add_argument("--spec-only", action="store_true",
                    help="time only the speculative-decoding verification round (for profiling)")
    ap.add_argument("--cpu-budget", type=float, default=10.0)
    ap.add_argument("--calib-copy", type=int, default=0,
                    help="instead of the bench, run N plain 1 GiB device copies (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the paged-attention path has no multi-GPU part in this library)", file=sys.stderr)
        sys.exit(2)

    import torch

    import paged_kv_cache_396_amd as pa
    from workloads import make_decode

    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from gpu_util import GpuPool, to_dev  # noqa: E402

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

    if args.prefill_only:
        print(json.dumps({"prefill_chunk": bench_prefill(args.steps, args.warmup),
                          "fp8_prefill_chunk": bench_prefill(args.steps, args.warmup, fp8=True)}),
              flush=True)
        return

    cfg = WORKLOADS[args.workload]
    t_gen = time.perf_counter()
    wl = make_decode(cfg)
    print(f"[bench] workload {args.workload}: {wl.num_seqs} seqs, ctx sum {int(wl.context_lens.sum())}, "
          f"generated in {time.perf_counter() - t_gen:.1f} s", file=sys.stderr, flush=True)

    if args.spec_only:
        print(json.dumps({"spec_verify_round": bench_spec_verify(args.steps, args.warmup)}), flush=True)
        return
    if args.fp8_only:
        print(json.dumps({"fp8_kv_step": bench_fp8_decode(wl, args.steps, args.warmup, args.partition)}),
              flush=True)
        return

    pool = GpuPool(wl.num_blocks, wl.num_kv_heads, wl.head_dim, wl.dtype)
    pool.write(wl.hist_k, wl.hist_v, wl.hist_slots)
    new_k = to_dev(wl.new_k, wl.dtype)
    new_v = to_dev(wl.new_v, wl.dtype)
    new_slots = torch.from_numpy(wl.new_slots).to(dev)
    q = to_dev(wl.q, wl.dtype)
    out = torch.empty_like(q)
    bt = torch.from_numpy(wl.block_tables).to(dev)
    cl = torch.from_numpy(wl.context_lens).to(dev)
    S, Hq, D = wl.q.shape
    max_ctx = int(wl.context_lens.max())
    part = pa.pa_decode_partition_size(S, wl.num_kv_heads, max_ctx, args.partition)
    ws_bytes = pa.pa_decode_workspace_bytes(S, Hq, wl.num_kv_heads, D, max_ctx, args.partition)
    ws = torch.empty(max(1, (ws_bytes + 3) // 4), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    # one step of the layer: every sequence's newest K/V row goes into its
    # slot and the sequences attend over their whole context, in one launch
    # (pa_decode_append); the two-call form is timed beside it
    def step():
        pa.pa_decode_append(out, q, new_k, new_v, new_slots, pool.k, pool.v, bt, cl, max_ctx,
                            float(wl.scale), pool.desc, partition_size=args.partition,
                            workspace=ws)

    def two_call_step():
        pa.pa_reshape_and_cache(new_k, new_v, new_slots, pool.k, pool.v, pool.desc)
        decode()

    def decode():
        pa.pa_decode(out, q, pool.k, pool.v, bt, cl, max_ctx, float(wl.scale), pool.desc,
                     partition_size=args.partition, workspace=ws)

    for _ in range(args.warmup):
        step()
        two_call_step()
    torch.cuda.synchronize()

    # timed steps: nothing but the hot path between the two events
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(args.steps):
        step()
    stop.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_total = start.elapsed_time(stop)
    ms_step = ms_total / args.steps

    # the same steps as two calls (cache write, then decode)
    start2 = torch.cuda.Event(enable_timing=True)
    stop2 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start2.record(stream)
    for _ in range(args.steps):
        two_call_step()
    stop2.record(stream)
    torch.cuda.synchronize()
    ms_two = start2.elapsed_time(stop2) / args.steps

    def per_call(fn, before=None):
        """Each call bracketed by its own events on the launch stream (a
        separate pass, so the events do not pad the timed steps)."""
        evs = []
        for _ in range(args.steps):
            if before is not None:
                before()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            evs.append((a, b))
        torch.cuda.synchronize()
        return [a.elapsed_time(b) for a, b in evs]

    # roofline of the step's launch (pa_decode_append) and of pa_decode alone
    step_ms = per_call(step)
    step_avg_ms = float(np.mean(step_ms))
    dec_ms = per_call(decode, before=lambda: pa.pa_reshape_and_cache(
        new_k, new_v, new_slots, pool.k, pool.v, pool.desc))
    dec_avg_ms = float(np.mean(dec_ms))

    # the same call with the caches cold: an untimed 512 MiB write (larger
    # than the L2s and the 256 MB last-level cache together) before each one
    scrub = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    cold_ms = per_call(step, before=lambda: scrub.fill_(7))
    del scrub

    def dist(ms):
        p10, p50, p90 = np.percentile(ms, [10, 50, 90])
        return {"median_ms": round(float(p50), 5), "p10_ms": round(float(p10), 5),
                "p90_ms": round(float(p90), 5),
                "median_gbs": round(wl.kv_bytes / (p50 * 1e-3) / 1e9, 1)}

    kv = wl.kv_bytes
    value = kv / (ms_step * 1e-3) / 1e9
    achieved = kv / (step_avg_ms * 1e-3) / 1e9
    traffic = _traffic(args.workload, kv)
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
        "dtype": "bf16" if wl.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {
            "workload": args.workload,
            "num_seqs": S, "num_q_heads": Hq, "num_kv_heads": wl.num_kv_heads, "head_dim": D,
            "block_size": 16, "context_lens": "U[128,4096]" if cfg == 2 else "per config",
            "ctx_sum": int(wl.context_lens.sum()), "num_blocks": wl.num_blocks,
            "decode_schedule": ("work-balanced: equal block ranges, one per resident workgroup"
                                if part == 0 else f"partitions of {part} tokens"),
            "new_tokens_per_step": int(len(wl.new_slots)),
            "parallelism": "single GPU",
        },
        "tokens_per_s": round(S / (ms_step * 1e-3), 1),
        "hbm_frac": round(value / HBM_PEAK_GBS, 4),
        "kv_bytes_per_step": kv,
        "step_call": f"pa_decode_append (cache write of the {len(wl.new_slots)} new tokens fused with decode)",
        "step_call_hot": dist(step_ms),
        "step_call_cold": dist(cold_ms),
        "two_call_step": {"calls": "pa_reshape_and_cache + pa_decode", "ms_per_step": round(ms_two, 5),
                          "gbs": round(kv / (ms_two * 1e-3) / 1e9, 1),
                          "hbm_frac": round(kv / (ms_two * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
        "decode_call_ms": round(dec_avg_ms, 5),
        "decode_call_hot": dist(dec_ms),
        "wall_s": round(wall, 4),
        "roofline": {
            "bound": "hbm",
            "kernel": "pa_decode_append (decode_balanced_kernel + decode_balanced_reduce_kernel)",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
        },
        "cpu_baseline": None,
    }
    if "prompt_len" in wl.extra:
        line["shared_prefix_call"] = bench_shared_prefix(wl, pool, q, bt, cl, max_ctx, args.steps,
                                                         args.warmup)
    ceiling = read_ceiling()
    if not args.no_prefill:
        line["cache_write_bulk"] = bench_bulk_write()
    line["hbm_read_ceiling"] = ceiling
    line["roofline"]["frac_of_read_ceiling"] = round(achieved / ceiling["gbs"], 4)
    if not args.no_prefill:
        line["prefill_chunk"] = bench_prefill(min(args.steps, 20), min(args.warmup, 3))
        line["fp8_prefill_chunk"] = bench_prefill(min(args.steps, 20), min(args.warmup, 3), fp8=True)
        line["long_mixed_step"] = bench_mixed_concurrent()
        line["block_pool"] = bench_block_pool()
        line["spec_verify_round"] = bench_spec_verify(min(args.steps, 20), min(args.warmup, 3))
        if wl.dtype == "bf16" and D == 128:
            line["fp8_kv_step"] = bench_fp8_decode(wl, args.steps, args.warmup)
            line["fp8_kv_step"]["speedup_vs_bf16_step"] = round(
                ms_step / line["fp8_kv_step"]["ms_per_step"], 3)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl, args.cpu_budget)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
