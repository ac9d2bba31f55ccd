#!/usr/bin/env python3
"""Decode-phase PagedAttention benchmark on one MI355X.

A step is one layer of one decode step over one batch: the step's new K/V rows are
appended to the pool and the whole batch attends (pa_decode_append: one launch of the
partition kernel, plus the reduce when split; the same work as pa_cache_append followed
by pa_decode, which is timed beside it).  The headline workload is the Llama-70B-shaped GQA decode: 32 sequences x 4096
tokens, 64 q-heads / 8 kv-heads, head_dim 128, bf16 KV, 16-token blocks in a shuffled
pool.  Inputs are seeded and synthetic and already resident in HBM when timing starts.
The step cycles over four copies of the layer's pools at distinct addresses, as the
layers of a real step do, so K/V is not reused from the 256 MB last-level cache.

Printed: ONE JSON line on stdout.
  value      KV GB/s over the whole step (algorithmic K+V bytes / wall time per step)
  roofline   the step's launch, timed with HIP events on the launching stream around
             the K timed steps (also over a longer run of back-to-back launches), against
             the 8 TB/s HBM peak (unique K/V bytes; shared prefix blocks count once) and
             against the read rate a plain 16-byte-load kernel measures in the same run
             before the steps; traffic from the committed rocprofv3 counter passes when
             they match the current kernel source
  cpu_baseline  the fp64 oracle on the host cores, on the same workload
Progress goes to stderr.
"""
import argparse
import json
import os
import statistics
import sys
import time

import numpy as np
import torch

HBM_PEAK_GBS = 8000.0
ROOT = os.path.dirname(os.path.abspath(__file__))
LAYERS = 4
# Bytes a decode sweep reads between two uses of one layer pool at least: four times the
# MI355X's 256 MB last-level cache (MALL), so no step finds its K/V still cached there
MALL_SPAN_BYTES = 1 << 30
W_ELEM = {"f32": 4, "f16": 2, "bf16": 2, "fp8": 1}
CALIBRATION_BYTES = 256 << 20
HEADLINE = 3
PREFILL_HEADLINE = 7
MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 / f16


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=200,
                    help="untimed steps first; the GPU's clocks need some 20 ms of steady "
                         "work to settle, which 200 decode steps give")
    ap.add_argument("--config", type=int, default=None,
                    help="workload id 1..8 (default: the Llama-70B GQA decode headline for "
                         "step / copy_blocks, the 512-token chunked prefill (7) for "
                         "prefill; 6 is the decode shape with an FP8 E4M3 KV cache)")
    ap.add_argument("--partition-tokens", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sub-batches", action="store_true",
                    help="skip the sub-batch timings of a shared-prefix batch (profiler passes "
                         "then see only the whole batch's launches)")
    ap.add_argument("--ordinary-loads", action="store_true",
                    help="decode with PA_POOL_SHARED_BLOCKS set whatever the batch (ordinary "
                         "instead of non-temporal K/V loads), for an A/B of the load hint")
    ap.add_argument("--roofline-launches", type=int, default=100)
    ap.add_argument("--op", choices=["step", "copy_blocks", "prefill"], default="step",
                    help="step: the decode step (default); copy_blocks: the copy-on-write "
                         "block copy on the workload's pool; prefill: append + paged "
                         "prefill of prompt chunks")
    ap.add_argument("--sweep", choices=["decode-types", "decode-groups", "decode-batch",
                                        "decode-partitions", "prefill-types",
                                        "prefill-splits"],
                    default=None,
                    help="instead of the bench line, time one call per shape of a family "
                         "and print one JSON line of rows: decode pool types and head "
                         "sizes on the Llama-70B-shaped decode, decode GQA group sizes on "
                         "32 x 4096 tokens, decode batch sizes (1 .. 64 sequences of 4096 "
                         "tokens), decode partition lengths (the plan against forced ones "
                         "on small, ragged and wide-group batches), prefill pool types and "
                         "head sizes on the 512-token chunked prefill, or prefill launches "
                         "too small to fill the GPU with and without key splits")
    ap.add_argument("--torch-sdpa-reference", action="store_true",
                    help="instead of the bench line, time PyTorch's own fused attention "
                         "(flash and memory-efficient backends only) on contiguous dense "
                         "tensors of the prefill shapes, as a reference rate for the "
                         "prefill kernel on this GPU; one JSON line of rows")
    ap.add_argument("--sweep-launches", type=int, default=0,
                    help="with --sweep: launches per timed round and warm-up launches "
                         "(default 100 and 200 for decode, 30 and 20 for prefill); small "
                         "values keep a rocprofv3 counter pass over a sweep short")
    ap.add_argument("--calibrate", action="store_true",
                    help="also run one 256 MiB device copy (a kernel of known traffic for "
                         "scaling rocprofv3 FETCH_SIZE / WRITE_SIZE counters)")
    return ap.parse_args()


def kernel_source_digest():
    """sha256 of the decode kernel's sources (what the recorded counters describe)."""
    import hashlib
    h = hashlib.sha256()
    for f in ("pa_decode.hip", "pa_common.h"):
        with open(os.path.join(ROOT, "paged_kv_cache_161_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def recorded_traffic(workload, ptok):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE passes,
    scaled by the calibration copy; None unless they were taken on this exact kernel
    source, workload and partition length."""
    path = os.path.join(ROOT, "profiles", "pa_decode_counters.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except OSError:
        return None
    entry = rec.get("workloads", {}).get(workload)
    if (not entry or entry.get("partition_tokens") != ptok
            or rec.get("kernel_source_sha256") != kernel_source_digest()):
        return None
    return entry["traffic_bytes_per_launch"]


def cpu_baseline(w):
    """The fp64 oracle as it is, on the host cores, on the same workload (append then
    decode of the whole batch); median of 3 runs."""
    import oracle as O
    threads = O.default_threads()
    kp, vp, bt, sl = w.oracle_view()
    kp, vp = O.cache_append(kp, vp, w.k_new, w.v_new, sl, w.kv_dtype, act_dtype=w.dtype,
                            k_scale=w.k_scale, v_scale=w.v_scale)
    times = []
    for _ in range(3):
        t0 = time.perf_counter()
        O.decode_paged(w.q, kp, vp, w.kv_dtype, bt, w.context_lens, w.scale, threads=threads,
                       q_dtype=w.dtype, k_scale=w.k_scale, v_scale=w.v_scale)
        times.append(time.perf_counter() - t0)
    t = statistics.median(times)
    # the same on one host thread, once (the oracle's result does not depend on it)
    t0 = time.perf_counter()
    O.decode_paged(w.q, kp, vp, w.kv_dtype, bt, w.context_lens, w.scale, threads=1,
                   q_dtype=w.dtype, k_scale=w.k_scale, v_scale=w.v_scale)
    t1 = time.perf_counter() - t0
    return {"value": round(w.logical_kv_bytes() / t / 1e9, 4), "unit": "GB/s",
            "cores": threads, "kind": "oracle",
            "sample": f"whole workload ({w.spec.name}, {w.num_seqs} seqs), decode only, "
                      f"median of 3 runs: {t:.3f} s/step, "
                      f"{w.num_seqs / t:.1f} tokens/s",
            "one_thread_value": round(w.logical_kv_bytes() / t1 / 1e9, 4),
            "one_thread_s_per_step": round(t1, 3),
            "cpu_model": cpu_model()}


def cpu_model():
    """The host CPU's model name, as /proc/cpuinfo gives it (None elsewhere)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def bench_copy_blocks(args, w, PA, U, dev):
    """pa_copy_blocks on the workload's pool: 1024 (src, dst) pairs of distinct blocks
    per launch, launches back to back between two HIP events; bytes = read + write of
    both pools' blocks.  Consecutive launches cycle four disjoint sets of pairs, so no
    launch finds its blocks in the 256 MB MALL from the launch before (one set repeated
    would read as ~45 % faster)."""
    kp, vp = U.device_pools(w, dev)
    rng = np.random.Generator(np.random.PCG64(7))
    n_sets = 4
    n_pairs = min(1024, w.num_blocks // (2 * n_sets))
    perm = rng.permutation(w.num_blocks)
    sets = [torch.from_numpy(np.stack([perm[2 * n_pairs * j:2 * n_pairs * j + n_pairs],
                                       perm[2 * n_pairs * j + n_pairs:2 * n_pairs * (j + 1)]],
                                      1).astype(np.int32)).to(dev) for j in range(n_sets)]
    block_bytes = w.num_kv_heads * 16 * w.head_dim * W_ELEM[w.kv_dtype]
    moved = 2 * 2 * n_pairs * block_bytes          # K and V, read and write
    for i in range(args.warmup):
        PA.copy_blocks(kp, vp, sets[i % n_sets])
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(args.steps):
        PA.copy_blocks(kp, vp, sets[i % n_sets])
    e1.record(stream)
    torch.cuda.synchronize()
    dur = e0.elapsed_time(e1) * 1e-3 / args.steps
    gbs = moved / dur / 1e9
    log(f"[bench] copy_blocks: {n_pairs} pairs of {block_bytes} B blocks, {dur * 1e6:.1f} us "
        f"per launch -> {gbs:.0f} GB/s")
    print(json.dumps({
        "metric": "copy-on-write block copy GB/s (read + write), 1 MI355X",
        "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(dur * 1e3, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w.kv_dtype,
        "data": "synthetic", "config": {"workload": f"{w.spec.name} pool, {n_pairs} block pairs",
                                         "block_bytes_per_pool": block_bytes,
                                         "disjoint_pair_sets_cycled": n_sets},
        "roofline": {"bound": "hbm", "kernel": "pa_copy_blocks_kernel",
                     "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                     "launch_us_mean": round(dur * 1e6, 2), "bytes_per_launch": moved},
    }), flush=True)


def calibration_copy(dev):
    """One device copy of known size: rocprofv3's FETCH_SIZE / WRITE_SIZE readings of
    it scale the kernel's readings to bytes."""
    src = torch.ones(CALIBRATION_BYTES // 2, dtype=torch.int16, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    log(f"[bench] calibration copy: {CALIBRATION_BYTES} bytes read, {CALIBRATION_BYTES} "
        "written")
    del src, dst


READ_PROBE_BYTES = 2 << 30


def measured_read_ceiling(dev, launches=10, step_bytes=0):
    """The practical HBM read rate on this device: the benchmark's plain read kernel
    (16-byte loads, grid-stride, libpa_hbm_probe.so) over 2 GiB, median of `launches`
    launches timed with HIP events on the launching stream.  With step_bytes > 0, also
    the same kernel reading exactly step_bytes per launch, back to back over disjoint
    slices of the 2 GiB buffer (2 to 64 of them; for steps of 32 MB or more, every
    slice is evicted from the 256 MB MALL before its next turn): the time a plain read
    of one step's K/V takes.
    Returns (GB/s, µs per same-size read or None), or (None, None) if the probe library
    is not built."""
    import ctypes
    path = os.path.join(ROOT, "paged_kv_cache_161_amd", "libpa_hbm_probe.so")
    if not os.path.exists(path):
        log("[bench] read probe not built; no measured read ceiling")
        return None, None
    lib = ctypes.CDLL(path)
    lib.pa_probe_read.restype = ctypes.c_int32
    lib.pa_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                  ctypes.c_int32, ctypes.c_void_p]
    buf = torch.ones(READ_PROBE_BYTES, dtype=torch.uint8, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    groups = torch.cuda.get_device_properties(dev).multi_processor_count * 8
    stream = torch.cuda.current_stream(dev)
    times = []
    for r in range(launches + 2):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        rc = lib.pa_probe_read(buf.data_ptr(), READ_PROBE_BYTES, sink.data_ptr(), groups,
                               ctypes.c_void_p(stream.cuda_stream))
        e1.record(stream)
        if rc != 0:
            raise RuntimeError(f"pa_probe_read returned {rc}")
        torch.cuda.synchronize()
        if r >= 2:
            times.append(e0.elapsed_time(e1) * 1e-3)
    gbs = READ_PROBE_BYTES / statistics.median(times) / 1e9
    log(f"[bench] measured read ceiling: {gbs:.0f} GB/s (2 GiB plain read, median of "
        f"{launches})")
    same_us = None
    size = step_bytes // 16 * 16
    slices = min(READ_PROBE_BYTES // size, 64) if size > 0 else 0
    if slices >= 2:
        def sweep(n):
            for j in range(n):
                rc = lib.pa_probe_read(buf.data_ptr() + (j % slices) * size, size,
                                       sink.data_ptr(), groups,
                                       ctypes.c_void_p(stream.cuda_stream))
                if rc != 0:
                    raise RuntimeError(f"pa_probe_read returned {rc}")
        n = 10 * slices
        sweep(n)
        best = float("inf")
        for _ in range(3):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            sweep(n)
            e1.record(stream)
            torch.cuda.synchronize()
            best = min(best, e0.elapsed_time(e1) * 1e3 / n)
        same_us = best
        log(f"[bench] plain read of {size} bytes per launch ({slices} disjoint slices "
            f"cycled): {same_us:.2f} us")
    del buf, sink
    return gbs, same_us


def prefill_flops(w):
    """Algorithmic FLOPs of a prefill call: per (query row, q-head, attended key) one
    d-long dot product for the score and one d-long axpy into the output, 2 FLOPs per
    multiply-add."""
    return 4 * w.head_dim * w.num_q_heads * w.attended_keys()


def time_sub_batch(w, d, pools, k_rows, v_rows, idx, sc, n_launch, warmup, dev):
    """One sub-batch of a decode workload (sequences idx) stepped on its own through the
    fused decode_append: µs per launch over n_launch back-to-back launches (HIP events
    on the launching stream, cycling over the layers' pools), its unique-KV rate, and
    the step as one graph of the layers' steps, replayed."""
    from paged_kv_cache_161_amd import binding as PA
    sel = torch.tensor(idx, dtype=torch.long, device=dev)
    q = d["q"].index_select(0, sel).contiguous()
    bt = d["block_tables"].index_select(0, sel).contiguous()
    cl = d["context_lens"].index_select(0, sel).contiguous()
    kr = k_rows.index_select(0, sel).contiguous()
    vr = v_rows.index_select(0, sel).contiguous()
    ctx = w.context_lens[idx]
    max_ctx = int(ctx.max())
    ptok = PA.plan_partition_tokens(w.num_q_heads, w.num_kv_heads, w.head_dim, ctx, w.kv_dtype)
    ws = torch.empty(max(PA.workspace_bytes(len(idx), w.num_q_heads, w.num_kv_heads,
                                            w.head_dim, max_ctx, ptok, w.kv_dtype), 1),
                     dtype=torch.uint8, device=dev)
    out = torch.empty_like(q)
    layers = len(pools)
    shared = PA.tables_share_blocks(w.block_tables[idx], w.context_lens[idx])

    def step(i):
        kp, vp = pools[i % layers]
        PA.decode_append(q, kp, vp, kr, vr, bt, cl, float(w.scale), max_ctx, ptok, out=out,
                         workspace=ws, shared_blocks=shared, **sc)

    for i in range(warmup):
        step(i)
    stream = torch.cuda.current_stream(dev)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(n_launch):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    dur = e0.elapsed_time(e1) * 1e-3 / n_launch
    # distinct physical K/V rows of the sub-batch (shared prefix blocks once)
    seen = {}
    for b in idx:
        n = int(w.context_lens[b])
        for lb in range((n + 15) // 16):
            p = int(w.block_tables[b, lb])
            seen[p] = max(seen.get(p, 0), min(16, n - lb * 16))
    uniq = sum(seen.values()) * w.num_kv_heads * 2 * w.head_dim * W_ELEM[w.kv_dtype]
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream(dev)
    cap.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.graph(g, stream=cap):
        for i in range(layers):
            step(i)
    torch.cuda.current_stream(dev).wait_stream(cap)
    for _ in range(max(1, warmup // layers)):
        g.replay()
    reps = max(1, n_launch // layers)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        g.replay()
    torch.cuda.synchronize()
    graph4_us = (time.perf_counter() - t0) * 1e6 / (reps * layers)
    return {"num_seqs": len(idx), "partition_tokens": ptok,
            "launch_us_mean": round(dur * 1e6, 2),
            "unique_kv_bytes": int(uniq), "achieved_GBps": round(uniq / dur / 1e9, 1),
            "graph4_us_per_step": round(graph4_us, 2)}


def prefill_recorded_traffic(workload):
    """HBM bytes per prefill launch from committed rocprofv3 counter passes, or None
    unless they were taken on this exact kernel source."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "pa_prefill_counters.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except OSError:
        return None
    h = hashlib.sha256()
    for f in ("pa_prefill.hip", "pa_prefill.h", "pa_common.h"):
        with open(os.path.join(ROOT, "paged_kv_cache_161_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    entry = rec.get("workloads", {}).get(workload)
    if not entry or rec.get("kernel_source_sha256") != h.hexdigest():
        return None
    return entry["traffic_bytes_per_launch"]


def prefill_oracle_rows(w, rows, threads=None):
    """The oracle on the given q rows of a prefill workload, each as a one-row chunk
    over its own prefix (the causal definition); returns (out, seconds)."""
    import oracle as O
    kp, vp, bt, sl = w.oracle_view()
    kp, vp = O.cache_append(kp, vp, w.k_new, w.v_new, sl, w.kv_dtype, act_dtype=w.dtype,
                            k_scale=w.k_scale, v_scale=w.v_scale)
    owner = np.searchsorted(w.query_start, rows, side="right") - 1
    q_len = np.diff(w.query_start)[owner]
    pos = w.context_lens[owner] - q_len + (rows - w.query_start[owner])
    ctx = np.maximum(pos + 1, 0).astype(np.int32)
    q = np.ascontiguousarray(w.q[rows])
    t0 = time.perf_counter()
    out, _ = O.prefill_paged(q, kp, vp, w.kv_dtype, np.arange(rows.size + 1, dtype=np.int32),
                             np.ascontiguousarray(bt[owner]), ctx, w.scale,
                             threads=threads or O.default_threads(), q_dtype=w.dtype,
                             k_scale=w.k_scale, v_scale=w.v_scale)
    return out, time.perf_counter() - t0, int(ctx.astype(np.int64).sum())


def bench_prefill(args, w, PA, U, dev):
    """One step = pa_cache_append of the chunks' K/V rows + pa_prefill of the chunks'
    queries, one layer; four layer pools cycled as in the decode step."""
    assert w.is_prefill, "--op prefill needs a prefill workload (7 or 8)"
    pools = [U.device_pools(w, dev) for _ in range(LAYERS)]
    d = U.device_inputs(w, dev)
    qs = torch.from_numpy(w.query_start).to(dev)
    out = torch.empty_like(d["q"])
    sc = U.scales(w)
    scale, max_ctx, max_q = float(w.scale), w.max_context_len, w.max_query_len
    flops = prefill_flops(w)
    n_tok = w.num_query_tokens

    def prefill(i):
        kp, vp = pools[i % LAYERS]
        PA.prefill(d["q"], kp, vp, qs, d["block_tables"], d["context_lens"], scale, max_ctx,
                   max_q, out=out, **sc)

    def step(i):
        kp, vp = pools[i % LAYERS]
        PA.cache_append(kp, vp, d["k_new"], d["v_new"], d["slot_mapping"], **sc)
        prefill(i)

    if args.calibrate:
        calibration_copy(dev)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t_start) * 1e3 / args.steps
    log(f"[bench] {args.steps} prefill steps: {ms_per_step * 1e3:.1f} us/step")

    stream = torch.cuda.current_stream(dev)
    n_l = args.roofline_launches
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(n_l):
        prefill(i)
    e1.record(stream)
    torch.cuda.synchronize()
    dur = e0.elapsed_time(e1) * 1e-3 / n_l
    tflops = flops / dur / 1e12
    log(f"[bench] prefill call: {dur * 1e6:.1f} us per launch over {n_l} back-to-back "
        f"launches -> {tflops:.1f} TFLOP/s")

    parity = None
    try:
        rows = np.unique(np.random.Generator(np.random.PCG64(1)).integers(0, n_tok, size=32))
        ref, _, _ = prefill_oracle_rows(w, rows)
        got = U.widen(U.from_dev(out, w.dtype), w.dtype)[rows]
        ok, mx, mean = U.tolerance_ok(got, ref, w.dtype)
        parity = {"rows_checked": int(rows.size), "max_abs_err": mx, "mean_abs_err": mean,
                  "pass": bool(ok and np.isfinite(got).all())}
        log(f"[bench] parity on timed inputs: {parity}")
    except Exception as exc:
        parity = {"error": repr(exc)}

    cpu = None
    if not args.no_cpu_baseline:
        rows = np.sort(np.random.Generator(np.random.PCG64(2)).choice(n_tok, size=min(512, n_tok),
                                                                    replace=False))
        _, t, keys = prefill_oracle_rows(w, rows)
        import oracle as O
        f = 4 * w.head_dim * w.num_q_heads * keys
        cpu = {"value": round(f / t / 1e12, 6), "unit": "TFLOP/s",
               "cores": O.default_threads(), "kind": "oracle",
               "sample": f"{rows.size} of the {n_tok} query rows (all {w.num_q_heads} "
                         f"q-heads), each over its causal prefix: {t:.2f} s, "
                         f"{rows.size / t:.1f} query tokens/s"}
        log(f"[bench] cpu baseline: {cpu}")

    value = flops / (ms_per_step * 1e-3) / 1e12
    kv = w.logical_kv_bytes()
    print(json.dumps({
        "metric": "prefill-attention TFLOP/s (% of MFMA peak) and query tokens/s, 1 MI355X",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype if w.kv_dtype == w.dtype else f"{w.kv_dtype} KV, {w.dtype} q/out",
        "data": "synthetic (seeded PCG64 normals x0.5, NaN-poisoned paged pool)",
        "config": {"workload": f"{w.spec.name}: {w.num_seqs} seqs, {n_tok} query tokens "
                               f"(chunks up to {max_q}), contexts up to {max_ctx}, "
                               f"{w.num_q_heads} q / {w.num_kv_heads} kv heads, d "
                               f"{w.head_dim}, 16-token blocks; step = append + prefill "
                               f"of one layer",
                   "num_seqs": w.num_seqs, "query_tokens": n_tok, "max_query_len": max_q,
                   "max_context_len": max_ctx, "num_q_heads": w.num_q_heads,
                   "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim, "block_size": 16,
                   "parallelism": "none (1 GPU)"},
        "query_tokens_per_s": round(n_tok / (ms_per_step * 1e-3), 1),
        "flops_per_step": flops,
        "kv_bytes_attended": kv,
        "roofline": {"bound": "mfma", "kernel": "pa_prefill_kernel",
                     "achieved": round(tflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": prefill_recorded_traffic(w.spec.name),
                     "launch_us_mean": round(dur * 1e6, 2), "flops_per_launch": flops},
        "cpu_baseline": cpu,
        "parity": parity,
    }), flush=True)


def sweep_shapes(name, W):
    """(label, Spec, knob) of one shape family, each derived from a named workload; the
    knob is the prefill key splits, or the decode partition length (0 = the library's
    choice in both)."""
    import dataclasses
    import re
    fp8 = dict(kv_dtype="fp8", k_scale=0.0117, v_scale=0.0093)
    if name == "decode-partitions":
        # the partition planner's choice against forced lengths, where the choice is
        # not one pass per sequence: small batches of 4,096 tokens, one 32k sequence,
        # the ragged batch and the long + shared-prefix batch
        base = W.config_spec(HEADLINE)
        shapes = [(f"bf16 B={b} x 4096", dataclasses.replace(
                      base, name=f"{base.name}_B{b}", context_lens=[4096] * b))
                  for b in (1, 4, 16)]
        shapes.append(("bf16 B=1 x 32768", dataclasses.replace(
            base, name=f"{base.name}_B1_32k", context_lens=[32768])))
        shapes += [("ragged bf16 (config 4)", W.config_spec(4)),
                   ("long + shared prefix (config 5)", W.config_spec(5))]
        # groups above 16 q-heads on 32 x 4,096 tokens, where few kv-heads leave the
        # plan short partitions and a reduce
        for label, kw in (("bf16 G32 (64 q / 2 kv)", dict(num_kv_heads=2)),
                          ("bf16 G64 MQA (64 q / 1 kv)", dict(num_kv_heads=1)),
                          ("fp8/bf16 G32 (64 q / 2 kv)", dict(num_kv_heads=2, **fp8))):
            shapes.append((label, dataclasses.replace(
                base, name=base.name + "_" + re.sub(r"[^A-Za-z0-9]+", "_", label).strip("_"),
                **kw)))
        out = []
        for label, spec in shapes:
            for ptok in (0, 256, 512, 1024, 2048, 4096):
                out.append((f"{label}, {'plan' if ptok == 0 else ptok}", spec, ptok))
        return out
    if name == "prefill-splits":
        # one request's chunk over a long context, and a few long decode rows alone:
        # 64 q / 8 kv heads, d 128, bf16, each without a key split and with the
        # library's choice
        base = W.config_spec(PREFILL_HEADLINE)
        shapes = [("1 x 512-token chunk at 32k", dict(context_lens=[32768], query_lens=[512])),
                  ("1 x 256-token chunk at 32k", dict(context_lens=[32768], query_lens=[256])),
                  ("2 x 256-token chunks at 16k", dict(context_lens=[16384] * 2,
                                                       query_lens=[256] * 2)),
                  ("4 decode rows at 32k", dict(context_lens=[32768] * 4, query_lens=[1] * 4))]
        out = []
        for label, kw in shapes:
            for ks in (1, 0):
                tag = f"{label}, {'no split' if ks == 1 else 'auto split'}"
                spec = dataclasses.replace(base, name=base.name + "_" + re.sub(
                    r"[^A-Za-z0-9]+", "_", label).strip("_"), spare_blocks=1, **kw)
                out.append((tag, spec, ks))
        return out
    if name == "prefill-types":
        base = W.config_spec(PREFILL_HEADLINE)
        rows = [("bf16 d128", {}), ("f16 d128", dict(dtype="f16")),
                ("fp8/bf16 d128", fp8), ("fp8/f16 d128", dict(dtype="f16", **fp8)),
                ("bf16 d64", dict(head_dim=64)), ("fp8/bf16 d64", dict(head_dim=64, **fp8)),
                ("bf16 d256", dict(head_dim=256)), ("fp8/bf16 d256", dict(head_dim=256, **fp8))]
    elif name == "decode-batch":
        base = W.config_spec(HEADLINE)
        rows = [(f"bf16 B={b} x 4096", dict(context_lens=[4096] * b))
                for b in (1, 2, 4, 8, 16, 32, 64)]
        rows += [(f"bf16 B={b} x 32768", dict(context_lens=[32768] * b)) for b in (1, 4)]
    elif name == "decode-types":
        base = W.config_spec(HEADLINE)
        rows = [("bf16 d128", {}), ("f16 d128", dict(dtype="f16")),
                ("fp8/bf16 d128", fp8), ("bf16 d64", dict(head_dim=64)),
                ("fp8/bf16 d64", dict(head_dim=64, **fp8)), ("bf16 d256", dict(head_dim=256)),
                ("fp8/bf16 d256", dict(head_dim=256, **fp8)),
                ("f32 d64", dict(dtype="f32", head_dim=64))]
    else:
        base = W.config_spec(HEADLINE)
        rows = [("bf16 G8 (64 q / 8 kv)", {}),
                ("bf16 G16 (64 q / 4 kv)", dict(num_kv_heads=4)),
                ("bf16 G32 (64 q / 2 kv)", dict(num_kv_heads=2)),
                ("bf16 G64 MQA (64 q / 1 kv)", dict(num_kv_heads=1)),
                ("f16 G64 MQA (64 q / 1 kv)", dict(num_kv_heads=1, dtype="f16")),
                ("bf16 G48 (96 q / 2 kv)", dict(num_q_heads=96, num_kv_heads=2)),
                ("bf16 G64 (128 q / 2 kv)", dict(num_q_heads=128, num_kv_heads=2)),
                ("bf16 G32 (128 q / 4 kv)", dict(num_q_heads=128, num_kv_heads=4)),
                ("fp8/bf16 G32 (64 q / 2 kv)", dict(num_kv_heads=2, **fp8)),
                ("fp8/bf16 G64 MQA (64 q / 1 kv)", dict(num_kv_heads=1, **fp8))]
    return [(label, dataclasses.replace(base, name=base.name + "_" +
                                        re.sub(r"[^A-Za-z0-9]+", "_", label).strip("_"), **kw), 0)
            for label, kw in rows]


def pool_copies(w):
    """Layer pools a decode sweep cycles: four, as in the bench step, or more when a
    step reads so few bytes that four pools would fit in the 256 MB MALL (the copies
    then span MALL_SPAN_BYTES of K/V reads; at most 64)."""
    per_step = max(w.unique_kv_bytes(), 1)
    return int(min(64, max(LAYERS, -(-MALL_SPAN_BYTES // per_step))))


def bench_sweep(args, PA, W, U, dev):
    """One timed call per shape (decode: the fused step's launch at the planned
    partition, cycling layer pools whose reads together span 1 GiB, so K/V always comes
    from HBM; prefill: the prefill call), best of three rounds of back-to-back launches
    between HIP events on the launching stream."""
    rows = []
    if args.calibrate:
        calibration_copy(dev)
    for label, spec, key_splits in sweep_shapes(args.sweep, W):
        w = W.build(spec)
        sc = U.scales(w)
        d = U.device_inputs(w, dev)
        out = torch.empty_like(d["q"])
        if w.is_prefill:
            kp, vp = U.device_pools(w, dev)
            PA.cache_append(kp, vp, d["k_new"], d["v_new"], d["slot_mapping"], **sc)
            qs = torch.from_numpy(w.query_start).to(dev)

            ks_used = key_splits or PA.prefill_key_splits(
                w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim, w.num_query_tokens,
                w.max_query_len, w.max_context_len, w.kv_dtype)
            ws_bytes = PA.prefill_workspace_bytes(
                w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim, w.num_query_tokens,
                w.max_query_len, w.max_context_len, key_splits, w.kv_dtype)
            pws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)

            def call(i):
                PA.prefill(d["q"], kp, vp, qs, d["block_tables"], d["context_lens"],
                           float(w.scale), w.max_context_len, w.max_query_len, out=out,
                           key_splits=key_splits, workspace=pws, **sc)
            n_warm, n_launch = 20, 30
            if args.sweep_launches > 0:
                n_warm, n_launch = args.sweep_launches, args.sweep_launches
        else:
            n_pools = pool_copies(w)
            shared = PA.tables_share_blocks(w.block_tables, w.context_lens)
            pools = [U.device_pools(w, dev) for _ in range(n_pools)]
            plan = PA.plan_partition_tokens(w.num_q_heads, w.num_kv_heads, w.head_dim,
                                            w.context_lens, w.kv_dtype)
            ptok = key_splits or plan          # decode: a forced partition length
            try:
                ws_bytes = PA.workspace_bytes(w.num_seqs, w.num_q_heads, w.num_kv_heads,
                                              w.head_dim, w.max_context_len, ptok, w.kv_dtype)
            except PA.PaError:
                if not key_splits:
                    raise
                # a forced length longer than this kernel's partitions may be
                row = {"shape": label, "workload": spec.name, "partition_tokens": ptok,
                       "unsupported": True}
                log(f"[sweep] {json.dumps(row)}")
                rows.append(row)
                continue
            ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
            rows_new = np.zeros((w.num_seqs,) + w.k_new.shape[1:], w.k_new.dtype)
            rows_new[np.flatnonzero(w.context_lens > 0)] = w.k_new
            kr = U.to_dev(rows_new, w.dtype, dev)

            def call(i):
                kp, vp = pools[i % n_pools]
                PA.decode_append(d["q"], kp, vp, kr, kr, d["block_tables"], d["context_lens"],
                                 float(w.scale), w.max_context_len, ptok, out=out,
                                 workspace=ws, shared_blocks=shared, **sc)
            n_warm, n_launch = 200, 100
            if args.sweep_launches > 0:
                n_warm, n_launch = args.sweep_launches, args.sweep_launches
        for i in range(n_warm):
            call(i)
        torch.cuda.synchronize()
        s = torch.cuda.current_stream(dev)
        best = float("inf")
        for _ in range(3):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(s)
            for i in range(n_launch):
                call(i)
            e1.record(s)
            torch.cuda.synchronize()
            best = min(best, e0.elapsed_time(e1) * 1e3 / n_launch)
        finite = bool(torch.isfinite(out.float()).all().item())
        row = {"shape": label, "workload": spec.name, "us": round(best, 2), "finite": finite}
        if w.is_prefill:
            tf = prefill_flops(w) / best / 1e6
            row.update(tflops=round(tf, 1), pct_mfma_peak=round(100 * tf / MFMA_BF16_PEAK_TFLOPS, 1),
                       key_splits=int(ks_used))
        else:
            by = w.unique_kv_bytes()
            row.update(partition_tokens=ptok, planned=bool(ptok == plan), kv_bytes=int(by),
                       pools_cycled=n_pools,
                       GBps=round(by / best / 1e3, 1),
                       pct_hbm_peak=round(100 * by / best / 1e3 / HBM_PEAK_GBS, 1))
        log(f"[sweep] {json.dumps(row)}")
        rows.append(row)
        del out, d
        torch.cuda.empty_cache()
    print(json.dumps({"sweep": args.sweep, "rows": rows}), flush=True)


def torch_sdpa_reference(dev):
    """PyTorch's fused attention on contiguous tensors, the shapes of the prefill
    workloads without paging: 16 x 512 queries over 4,096 keys unmasked (the chunked
    prefill's size), and 2 x 4,096 causal, at 64 q-heads over 8 and over 64 kv-heads,
    d 128, bf16.  Only the flash and memory-efficient backends are allowed (a backend
    that cannot take a shape is reported unavailable, never replaced by the math
    path).  Best of three rounds of 20 launches between HIP events."""
    import torch.nn.functional as F
    from torch.nn.attention import SDPBackend, sdpa_kernel
    cases = [("512 q x 4096 k, no mask, 64 q / 8 kv heads, B 16", 16, 64, 8, 512, 4096, False),
             ("512 q x 4096 k, no mask, 64 q / 64 kv heads, B 16", 16, 64, 64, 512, 4096, False),
             ("4096 x 4096 causal, 64 q / 8 kv heads, B 2", 2, 64, 8, 4096, 4096, True),
             ("4096 x 4096 causal, 64 q / 64 kv heads, B 2", 2, 64, 64, 4096, 4096, True)]
    rows = []
    gen = torch.Generator(device=dev).manual_seed(0)
    for backend in (SDPBackend.FLASH_ATTENTION, SDPBackend.EFFICIENT_ATTENTION):
        for label, b, hq, hkv, lq, lk, causal in cases:
            q = torch.randn(b, hq, lq, 128, device=dev, dtype=torch.bfloat16, generator=gen)
            k = torch.randn(b, hkv, lk, 128, device=dev, dtype=torch.bfloat16, generator=gen)
            v = torch.randn(b, hkv, lk, 128, device=dev, dtype=torch.bfloat16, generator=gen)
            kw = {"enable_gqa": True} if hkv != hq else {}
            pairs = lq * (lq + 1) // 2 if causal else lq * lk
            flops = 4 * 128 * b * hq * pairs
            row = {"backend": backend.name, "shape": label}
            try:
                with sdpa_kernel([backend]):
                    def call():
                        return F.scaled_dot_product_attention(q, k, v, is_causal=causal, **kw)
                    for _ in range(3):
                        call()
                    torch.cuda.synchronize()
                    best = float("inf")
                    s = torch.cuda.current_stream(dev)
                    for _ in range(3):
                        e0 = torch.cuda.Event(enable_timing=True)
                        e1 = torch.cuda.Event(enable_timing=True)
                        e0.record(s)
                        for _ in range(20):
                            call()
                        e1.record(s)
                        torch.cuda.synchronize()
                        best = min(best, e0.elapsed_time(e1) * 1e3 / 20)
                tf = flops / best / 1e6
                row.update(us=round(best, 1), tflops=round(tf, 1),
                           pct_mfma_peak=round(100 * tf / MFMA_BF16_PEAK_TFLOPS, 1))
            except RuntimeError as exc:
                row.update(unavailable=str(exc).splitlines()[0][:120])
            log(f"[sdpa] {json.dumps(row)}")
            rows.append(row)
            del q, k, v
    print(json.dumps({"reference": "torch scaled_dot_product_attention",
                      "torch": torch.__version__, "rows": rows}), flush=True)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this decode path is not sharded across GPUs "
              "(how it would shard is described with the design); run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        sys.exit(2)

    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    from paged_kv_cache_161_amd import binding as PA
    from paged_kv_cache_161_amd import workloads as W
    from tests import devutil as U

    PA.load()
    dev = torch.device("cuda:0")
    if args.torch_sdpa_reference:
        return torch_sdpa_reference(dev)
    if args.sweep:
        return bench_sweep(args, PA, W, U, dev)
    t0 = time.time()
    if args.config is None:
        args.config = PREFILL_HEADLINE if args.op == "prefill" else HEADLINE
    w = W.make_config(args.config)
    log(f"[bench] built {w.spec.name} in {time.time() - t0:.1f}s: B={w.num_seqs} "
        f"Hq={w.num_q_heads} Hkv={w.num_kv_heads} d={w.head_dim} "
        f"max_ctx={w.max_context_len} pool={w.num_blocks} blocks")

    if args.op == "copy_blocks":
        return bench_copy_blocks(args, w, PA, U, dev)
    if args.op == "prefill":
        return bench_prefill(args, w, PA, U, dev)

    pools = [U.device_pools(w, dev) for _ in range(LAYERS)]
    d = U.device_inputs(w, dev)
    out = torch.empty_like(d["q"])
    # the partition length a serving loop would plan from the host's context lengths
    # (pa_decode_plan), unless one is forced
    ptok = args.partition_tokens or PA.plan_partition_tokens(
        w.num_q_heads, w.num_kv_heads, w.head_dim, w.context_lens, w.kv_dtype)
    ws_bytes = PA.workspace_bytes(w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim,
                                  w.max_context_len, ptok, w.kv_dtype)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    kv_bytes = w.logical_kv_bytes()
    uniq_bytes = w.unique_kv_bytes()
    scale = float(w.scale)
    max_ctx = w.max_context_len

    sc = U.scales(w)
    # each sequence's new row, laid out per sequence for the fused call
    appending = np.flatnonzero(w.context_lens > 0)
    rows_k = np.zeros((w.num_seqs,) + w.k_new.shape[1:], w.k_new.dtype)
    rows_v = np.zeros_like(rows_k)
    rows_k[appending] = w.k_new
    rows_v[appending] = w.v_new
    k_rows = U.to_dev(rows_k, w.dtype, dev)
    v_rows = U.to_dev(rows_v, w.dtype, dev)

    # a batch whose tables name a block for several sequences (config 5's beams) says
    # so (the library's host check of the tables, as a serving loop would run it)
    shared = PA.tables_share_blocks(w.block_tables, w.context_lens) or args.ordinary_loads

    def fused(i):
        kp, vp = pools[i % LAYERS]
        PA.decode_append(d["q"], kp, vp, k_rows, v_rows, d["block_tables"], d["context_lens"],
                         scale, max_ctx, ptok, out=out, workspace=ws, shared_blocks=shared, **sc)

    def two_calls(i):
        kp, vp = pools[i % LAYERS]
        PA.cache_append(kp, vp, d["k_new"], d["v_new"], d["slot_mapping"], **sc)
        PA.decode(d["q"], kp, vp, d["block_tables"], d["context_lens"], scale, max_ctx, ptok,
                  out=out, workspace=ws, shared_blocks=shared, **sc)

    # a step is one decode_append launch (the append fused into the attention); the
    # same work as two calls is timed beside it
    step = fused

    if args.calibrate:
        calibration_copy(dev)
    # the HBM read ceiling of this machine, measured before the steps (a plain 16-byte-load
    # read of 2 GiB, ten times)
    ceiling, plain_same_us = measured_read_ceiling(dev, step_bytes=uniq_bytes)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    log(f"[bench] warmup {args.warmup} steps done")

    # the timed steps: wall clock between two synchronisations, and HIP events on the
    # launching stream around the same launches (the roofline's launch duration)
    stream = torch.cuda.current_stream(dev)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    ms_per_step = wall * 1e3 / args.steps
    dur = ev0.elapsed_time(ev1) * 1e-3 / args.steps
    log(f"[bench] {args.steps} steps: {ms_per_step * 1e3:.1f} us/step "
        f"({dur * 1e6:.1f} us per launch by events)")
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        two_calls(i)
    torch.cuda.synchronize()
    two_call_ms = (time.perf_counter() - t_start) * 1e3 / args.steps
    log(f"[bench] {args.steps} steps as append + decode: {two_call_ms * 1e3:.1f} us/step")

    # the least HBM traffic the method must move is each physical K/V row once: shared
    # prefix blocks count once (the logical rate is reported beside it)
    achieved = uniq_bytes / dur / 1e9
    log(f"[bench] decode_append launches of the timed steps: {dur * 1e6:.1f} us each -> "
        f"{achieved:.0f} GB/s unique, {kv_bytes / dur / 1e9:.0f} logical")
    # a longer run of the same launches, back to back between HIP events on the stream,
    # cycling over the layers' pools so each launch's K/V is out of the caches (1.5 GiB
    # of other pools in between); reported beside the timed steps' figure
    n_l = args.roofline_launches
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(n_l):
        fused(i)
    e1.record(stream)
    torch.cuda.synchronize()
    dur_loop = e0.elapsed_time(e1) * 1e-3 / n_l
    log(f"[bench] {n_l} more back-to-back launches: {dur_loop * 1e6:.1f} us each")
    traffic = recorded_traffic(w.spec.name, ptok)

    # the same step captured as one HIP graph per layer pool and replayed (the
    # library enqueues only kernels, so the graphs hold exactly the eager launches)
    graphs = []
    cap = torch.cuda.Stream(dev)
    cap.wait_stream(torch.cuda.current_stream(dev))
    for i in range(LAYERS):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap):
            step(i)
        graphs.append(g)
    torch.cuda.current_stream(dev).wait_stream(cap)
    for i in range(args.warmup):
        graphs[i % LAYERS].replay()
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        graphs[i % LAYERS].replay()
    torch.cuda.synchronize()
    graph_ms = (time.perf_counter() - t_start) * 1e3 / args.steps
    log(f"[bench] {args.steps} graph-replayed steps: {graph_ms * 1e3:.1f} us/step")
    # as a serving loop captures a whole step: the four layers' steps in one graph
    g4 = torch.cuda.CUDAGraph()
    cap.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.graph(g4, stream=cap):
        for i in range(LAYERS):
            step(i)
    torch.cuda.current_stream(dev).wait_stream(cap)
    reps = max(1, args.steps // LAYERS)
    for _ in range(max(1, args.warmup // LAYERS)):
        g4.replay()
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for _ in range(reps):
        g4.replay()
    torch.cuda.synchronize()
    graph4_ms = (time.perf_counter() - t_start) * 1e3 / (reps * LAYERS)
    log(f"[bench] {reps} replays of one {LAYERS}-layer graph: {graph4_ms * 1e3:.1f} us per layer step")

    # a batch that shares a prefix (beams) is also timed as its two sub-batches, each
    # on its own: the long sequences, and the beams, whose step is µs-scale, eagerly
    # and as one graph of the four layers' steps
    sub_batches = None
    if w.spec.prefix_groups and not args.no_sub_batches:
        beams = sorted({b for grp, _ in w.spec.prefix_groups for b in grp})
        sub_batches = {}
        for name, idx in (("long", [b for b in range(w.num_seqs) if b not in beams]),
                          ("beams", beams)):
            if not idx:
                continue
            sub_batches[name] = time_sub_batch(w, d, pools, k_rows, v_rows, idx, sc, n_l,
                                               args.warmup, dev)
            log(f"[bench] sub-batch {name}: {sub_batches[name]}")

    # parity on the timed inputs (sampled rows against the oracle)
    parity = None
    try:
        import oracle as O
        rows = np.random.Generator(np.random.PCG64(0)).choice(
            w.num_seqs, size=min(4, w.num_seqs), replace=False)
        sub = {k: v for k, v in zip(("k", "v", "bt", "sl"), w.oracle_view())}
        kpo, vpo = O.cache_append(sub["k"], sub["v"], w.k_new, w.v_new, sub["sl"], w.kv_dtype,
                                  act_dtype=w.dtype, k_scale=w.k_scale, v_scale=w.v_scale)
        ref, _ = O.decode_paged(np.ascontiguousarray(w.q[rows]), kpo, vpo, w.kv_dtype,
                                np.ascontiguousarray(sub["bt"][rows]), w.context_lens[rows],
                                w.scale, q_dtype=w.dtype, k_scale=w.k_scale, v_scale=w.v_scale)
        got = U.widen(U.from_dev(out, w.dtype), w.dtype)[rows]
        ok, mx, mean = U.tolerance_ok(got, ref, w.dtype)
        parity = {"rows_checked": int(rows.size), "max_abs_err": mx, "mean_abs_err": mean,
                  "pass": bool(ok and np.isfinite(got).all())}
        log(f"[bench] parity on timed inputs: {parity}")
    except Exception as exc:  # parity is reported, never silently assumed
        parity = {"error": repr(exc)}

    cpu = None if args.no_cpu_baseline else cpu_baseline(w)
    if cpu:
        log(f"[bench] cpu baseline: {cpu}")

    value = kv_bytes / (ms_per_step * 1e-3) / 1e9
    tokens_per_s = w.num_seqs / (ms_per_step * 1e-3)
    result = {
        "metric": "decode-attention KV GB/s (% of HBM peak) and tokens/s, 1 MI355X",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype if w.kv_dtype == w.dtype else f"{w.kv_dtype} KV, {w.dtype} q/out",
        "data": "synthetic (seeded PCG64 normals x0.5, NaN-poisoned paged pool)",
        "config": {"workload": f"{w.spec.name}: {w.num_seqs} seqs x ctx {max_ctx}, "
                               f"{w.num_q_heads} q / {w.num_kv_heads} kv heads, d "
                               f"{w.head_dim}, 16-token blocks, {w.num_blocks}-block shuffled pool; "
                               f"step = append + decode of one layer (one fused launch)",
                   "num_seqs": w.num_seqs, "context_len": max_ctx,
                   "num_q_heads": w.num_q_heads, "num_kv_heads": w.num_kv_heads,
                   "head_dim": w.head_dim, "block_size": 16,
                   "partition_tokens": ptok,
                   "shared_blocks": shared,
                   "ordinary_loads_forced": bool(args.ordinary_loads),
                   "parallelism": "none (1 GPU)"},
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "tokens_per_s": round(tokens_per_s, 1),
        "context_tokens_per_s": round(float(w.context_lens.sum()) / (ms_per_step * 1e-3), 1),
        "kv_bytes_per_step": kv_bytes,
        "two_call_ms_per_step": round(two_call_ms, 5),
        "graph_ms_per_step": round(graph_ms, 5),
        "graph_tokens_per_s": round(w.num_seqs / (graph_ms * 1e-3), 1),
        "graph4_ms_per_step": round(graph4_ms, 5),
        "unique_kv_bytes_per_step": uniq_bytes,
        "sub_batches": sub_batches,
        "roofline": {"bound": "hbm", "kernel": "pa_decode_partition with the fused append "
                                               "(+ pa_decode_reduce when a sequence spans "
                                               "several partitions)",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "launch_us_mean": round(dur * 1e6, 2),
                     "launch_us_source": f"HIP events around the {args.steps} timed steps",
                     "bytes_per_launch": uniq_bytes,
                     "achieved_logical": round(kv_bytes / dur / 1e9, 1),
                     "launch_us_mean_longer_run": round(dur_loop * 1e6, 2),
                     "longer_run_launches": n_l,
                     "measured_read_ceiling": None if ceiling is None else round(ceiling, 1),
                     "frac_of_measured_read_ceiling":
                         None if ceiling is None else round(achieved / ceiling, 4),
                     "plain_read_same_bytes_us":
                         None if plain_same_us is None else round(plain_same_us, 2),
                     "frac_of_plain_read_same_bytes":
                         None if plain_same_us is None else round(plain_same_us / (dur * 1e6), 4)},
        "cpu_baseline": cpu,
        "parity": parity,
        "context_figures": {"A100_ridge_flop_per_byte": 156, "H100_hbm_TBps": 3.35},
    }
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
