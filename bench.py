#!/usr/bin/env python3
"""Benchmark of the KV compress -> quantise -> paged-store path on one MI355X.

One step is one pass of the whole path over one batch of synthetic inputs already
resident in HBM:
  1. the mixed decode/prefill step (V41_FP4): full -> SWA slot translation of the
     ragged batch's compressed rows, ratio-4 compression into the FP4 pool at the
     translated slots, dequant of every touched page into a bf16 workspace;
  2. C4A: 16384 output rows, ratio 4, fp32 kv/score [65536, 512], V41 pool;
  3. C128A: 16384 output rows, ratio 128, fp32 kv/score [2097152, 512], V41 pool.
Each step touches ~9.1 GB, far beyond the 256 MB last-level cache, so every kernel
reads cold inputs.  `value` is compressed rows per second over the whole step; every
kernel's duration (HIP events recorded by its own dispatch; mean, median, p10, p90),
algorithmic bytes and fraction of the 8 TB/s HBM peak are in `kernels`; `roofline` is
the dominant kernel (C128A).

    python bench.py [--gpus 1] [--steps 50] [--warmup 10] [--no-cpu-baseline] [--no-micro]
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "compressed KV rows/sec + achieved HBM GB/s (% of MI355X peak), C4A & C128A"
HBM_PEAK_GBS = 8000.0   # MI355X HBM3E, vendor figure
HEAD = 512
PROFILE = os.path.join(ROOT, "profiles", "compress_c128a_v41_pmc.txt")
def kernel_source_hash() -> str:
    """SHA-256 of the library's sources and build flags: the same value libkvq.so reports
    as kvq_build_id()."""
    from quantized_paged_kv_compress_amd import _build
    return _build.source_hash()


# ---------------------------------------------------------------- algorithmic bytes
# What the method must move, per launch: inputs read once, per-row metadata (position
# 4 B, slot 4 B, the gathered 64-float cos/sin row 256 B), the stored row.
def bytes_compress(R, ratio, token_bytes):
    return R * (ratio * HEAD * 4 * 2 + 4 + 4 + 64 * 4 + token_bytes)


def bytes_translate(n, cap):
    return n * (4 + 4 + 4) + (cap - n) * 4


def bytes_dequant(P, page_bytes):
    return P * (4 + page_bytes + 64 * HEAD * 2)


def read_traffic(duration_key_bytes):
    """HBM bytes per C128A launch from the committed rocprofv3 PMC summary: DRAM read and
    write sectors (32 bytes each), with FETCH_SIZE + WRITE_SIZE scaled by the copy-kernel
    calibration in the same file as a cross-check; None if the kernels changed since."""
    if not os.path.exists(PROFILE):
        return None
    kv = {}
    for line in open(PROFILE):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    try:
        if kv.get("kernel_source_sha256") != kernel_source_hash():
            return None
        copy_bytes = float(kv["copy_bytes_each_way"])
        fs = copy_bytes / (float(kv["copy_FETCH_SIZE_KiB_per_dispatch"]) * 1024)
        ws = copy_bytes / (float(kv["copy_WRITE_SIZE_KiB_per_dispatch"]) * 1024)
        fetch = float(kv["FETCH_SIZE_KiB_per_dispatch"]) * 1024 * fs
        write = float(kv["WRITE_SIZE_KiB_per_dispatch"]) * 1024 * ws
        dram = float(kv["DRAM_read_bytes_per_dispatch"]) + float(kv["DRAM_write_bytes_per_dispatch"])
        return {"bytes": dram, "dram_read_bytes": float(kv["DRAM_read_bytes_per_dispatch"]),
                "dram_write_bytes": float(kv["DRAM_write_bytes_per_dispatch"]),
                "fetch_write_scaled_bytes": fetch + write, "fetch_scale": fs, "write_scale": ws,
                "ratio_to_algorithmic": dram / duration_key_bytes}
    except (KeyError, ValueError, ZeroDivisionError):
        return None


def graph_us(fn, n_calls, reps=20):
    """Median per-call microseconds of `n_calls` back-to-back calls of fn captured in one
    HIP graph (torch.cuda.CUDAGraph), over `reps` replays."""
    import numpy as np
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(n_calls):
            fn()
    for _ in range(3):
        g.replay()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    times = []
    for _ in range(reps):
        e0.record()
        g.replay()
        e1.record()
        e1.synchronize()
        times.append(e0.elapsed_time(e1) * 1e3 / n_calls)
    return float(np.median(times))


def evict_caches(buf, mode):
    """Make the next kernel's inputs cold.  "read": read a 512 MiB buffer, so the caches
    hold none of the inputs and no dirty lines; "write": fill it, which evicts the inputs
    too but leaves the last-level cache full of dirty lines that the next kernel then pays
    to write back (reported beside the read figure as the after-a-large-write regime)."""
    if mode == "read":
        buf.sum()
    else:
        buf.fill_(1.0)


def store_configs(kvq, wl, dev, cs, reps=20, calls=50):
    """The two store workloads at their own sizes: V41 plain store (64 tokens, 16-page pool)
    and V41 store + RoPE (512 tokens, 4096-page pool).  Under 1 MB of data each, so the
    time is launch latency: graph-replayed per-launch time, tokens/s and algorithmic GB/s."""
    import numpy as np
    import torch

    def t(a):
        if a.dtype == np.uint16:
            a = a.view(np.int16)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    out = {"method": f"HIP graph of {calls} back-to-back launches, median of {reps} replays"}
    d1 = wl.store_v41(seed=1)
    pool1 = kvq.new_pool(kvq.V41, d1["num_pages"])
    k1, s1 = t(d1["k"]), t(d1["slots"])
    d2 = wl.store_rope(seed=2)
    pool2 = kvq.new_pool(kvq.V41, d2["num_pages"])
    k2, p2, s2 = t(d2["k"]), t(d2["pos"]), t(d2["slots"])
    cases = (("v41_plain_store", 64, 64 * (1024 + 4 + 528),
              lambda: kvq.kv_store(pool1, kvq.V41, k1, s1)),
             ("v41_store_rope", 512, 512 * (1024 + 4 + 4 + 256 + 528),
              lambda: kvq.kv_store_rope(pool2, kvq.V41, k2, p2, cs, s2)))
    for name, n, b, fn in cases:
        us = graph_us(fn, calls, reps)
        gbs = b / (us * 1e-6) / 1e9
        out[name] = {"tokens": n, "us_per_launch": round(us, 3), "tokens/s": round(n / (us * 1e-6), 1),
                     "alg_bytes": b, "GB/s": round(gbs, 1), "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4)}
    return out


def micro_bench(kvq, wl, dev, cs, layers=61, reps=20, calls=50):
    """Graph-replayed per-launch latency of the kernels in P1's latency table (store,
    store+RoPE, fused K norm+RoPE, c1, c2 at 1/8/64/512 tokens, V41, hot inputs), and the
    P2 hoisting case: 512 tokens stored into `layers` per-layer pools with one full->SWA
    translation per step (one store call per layer, or one kv_store_rope_layers launch for
    all layers) against a translation inside every layer."""
    import numpy as np
    import torch

    def t(a):
        if a.dtype == np.uint16:
            a = a.view(np.int16)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    rng = np.random.default_rng(123)
    num_pages = 4096
    pool = kvq.new_pool(kvq.V41, num_pages)
    w = t(wl.bf16_bits(rng.uniform(0.5, 1.5, HEAD).astype(np.float32)))
    table = {}
    for bs in (1, 8, 64, 512):
        k = t(wl.bf16_bits(rng.standard_normal((bs, HEAD)).astype(np.float32)))
        pos = t(rng.integers(0, 65536, bs).astype(np.int32))
        slots = t(wl.distinct_slots(rng, bs, 64, num_pages * 64))
        kv = t(rng.standard_normal((2 * bs, HEAD)).astype(np.float32))
        sc = t((2 * rng.standard_normal((2 * bs, HEAD))).astype(np.float32))
        fns = {
            "store": lambda: kvq.kv_store(pool, kvq.V41, k, slots),
            "store_rope": lambda: kvq.kv_store_rope(pool, kvq.V41, k, pos, cs, slots),
            "k_norm_rope": lambda: kvq.kv_store_norm_rope(pool, kvq.V41, k, w, 1e-6, pos, cs, slots),
            "c1": lambda: kvq.kv_compress_store(pool, kvq.V41, kv[:bs], None, 1, pos, cs, slots),
            "c2": lambda: kvq.kv_compress_store(pool, kvq.V41, kv, sc, 2, pos, cs, slots),
        }
        for name, fn in fns.items():
            table.setdefault(name, {})[f"bs{bs}"] = round(graph_us(fn, calls, reps), 3)

    # P2: translate once per step vs once per layer; 512 new tokens stored into `layers`
    # SWA pools, each layer with its own K rows
    n, cap = 512, 4096
    swa_pages = 64
    full = t((rng.permutation(swa_pages * 64)[:n] + 64 * 8).astype(np.int32))
    tab = np.full(64 * 8 + swa_pages * 64, -1, np.int32)
    tab[64 * 8:64 * 8 + swa_pages * 64] = rng.permutation(swa_pages * 64).astype(np.int32)
    tab = t(tab)
    buf = torch.empty(cap, dtype=torch.int32, device=dev)
    ks = [t(wl.bf16_bits(rng.standard_normal((n, HEAD)).astype(np.float32))) for _ in range(layers)]
    pos = t(rng.integers(0, 65536, n).astype(np.int32))
    pools = [kvq.new_pool(kvq.V41, swa_pages) for _ in range(layers)]

    def per_layer():
        for p, k in zip(pools, ks):
            loc = kvq.kv_translate_slots(tab, full, buf)
            kvq.kv_store_rope(p, kvq.V41, k, pos, cs, loc)

    def hoisted_calls():
        loc = kvq.kv_translate_slots(tab, full, buf)
        for p, k in zip(pools, ks):
            kvq.kv_store_rope(p, kvq.V41, k, pos, cs, loc)

    def hoisted_one_launch():
        loc = kvq.kv_translate_slots(tab, full, buf)
        kvq.kv_store_rope_layers(pools, kvq.V41, ks, pos, cs, loc)

    # the one-launch store's own duration (dispatch-recorded events), inputs cold: 512 MiB
    # read (or written) between repetitions evicts the 32 MB of K rows from the caches
    alg = layers * n * (2 * HEAD + 528) + n * (4 + 4 + 256)
    flush = torch.empty(1 << 27, dtype=torch.float32, device=dev)
    loc = kvq.kv_translate_slots(tab, full, buf)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(); e1.record()
    kern = {"read": [], "write": []}
    for r in range(2 * (reps + 3)):
        mode = ("read", "write")[r % 2]
        evict_caches(flush, mode)
        kvq.profile_next_launch(e0, e1)
        kvq.kv_store_rope_layers(pools, kvq.V41, ks, pos, cs, loc)
        e1.synchronize()
        if r >= 6:
            kern[mode].append(e0.elapsed_time(e1) * 1e3)
    del flush
    kus = float(np.median(kern["read"]))
    kus_w = float(np.median(kern["write"]))
    step = {"layers": layers, "tokens": n,
            "per_layer_translate_us_per_step": round(graph_us(per_layer, 1, reps), 2),
            "hoisted_per_layer_calls_us_per_step": round(graph_us(hoisted_calls, 1, reps), 2),
            "hoisted_one_launch_us_per_step": round(graph_us(hoisted_one_launch, 1, reps), 2),
            "one_launch_kernel_cold": {"us": round(kus, 2), "alg_bytes": alg,
                                       "GB/s": round(alg / (kus * 1e-6) / 1e9, 1),
                                       "frac_of_peak": round(alg / (kus * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                                       "after_512MiB_write_us": round(kus_w, 2),
                                       "after_512MiB_write_frac_of_peak":
                                           round(alg / (kus_w * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)},
            "note": "graph-replayed steps read hot inputs (32 MB of K rows stay in the 256 MB "
                    "last-level cache); the kernel line reads cold inputs, evicted by reading 512 MiB "
                    "(after_512MiB_write: evicted by writing it, which leaves dirty lines to write back)"}
    return {"method": f"HIP graph of {calls} back-to-back launches, median of {reps} replays, "
                      "per-launch microseconds, V41, hot inputs",
            "latency_us": table, "swa_hoisting": step}


def cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo), for the CPU-baseline record."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def mixed_graph(kvq, m, cs, fused=True, reps=20, flush_mode="read"):
    """The mixed FP4 step (full -> SWA translation, ratio-4 compress at the translated slots,
    dequant of the touched pages) captured as one HIP graph and replayed; each replay is
    timed by stream events around it, with 512 MiB read (flush_mode "read") or written
    ("write") before it so that its inputs are cold.  fused: the translation runs inside
    the compressor's launch (kv_compress_store_translate, two launches in all); otherwise
    kv_translate_slots is a launch of its own (three)."""
    import numpy as np
    import torch

    def seq():
        if fused:
            kvq.kv_compress_store_translate(m["pool"], kvq.V41_FP4, m["kv"], m["sc"], 4, m["pos"], cs,
                                            m["table"], m["full"], m["loc"])
        else:
            loc = kvq.kv_translate_slots(m["table"], m["full"], m["loc"])
            kvq.kv_compress_store(m["pool"], kvq.V41_FP4, m["kv"], m["sc"], 4, m["pos"], cs, loc)
        kvq.kv_dequant(m["pool"], kvq.V41_FP4, m["page_ids"], m["ws"])

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        seq()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        seq()
    flush = torch.empty(1 << 27, dtype=torch.float32, device=m["kv"].device)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ts = []
    for r in range(reps + 3):
        evict_caches(flush, flush_mode)
        e0.record()
        g.replay()
        e1.record()
        e1.synchronize()
        if r >= 3:
            ts.append(e0.elapsed_time(e1) * 1e3)
    del flush
    return float(np.median(ts)), float(np.percentile(ts, 10)), float(np.percentile(ts, 90))


def device_facts(torch):
    """What the runtime reports about the GPU the bench ran on."""
    p = torch.cuda.get_device_properties(0)
    facts = {"name": p.name, "compute_units": p.multi_processor_count,
             "memory_GiB": round(p.total_memory / 2 ** 30, 1)}
    for key, attr in (("arch", "gcnArchName"), ("l2_bytes", "L2_cache_size"),
                      ("max_shared_memory_per_block", "shared_memory_per_block")):
        if hasattr(p, attr):
            facts[key] = getattr(p, attr)
    return facts


class DispatchTimer:
    """Pairs of HIP events that a kernel's own dispatch records at its start and end
    (kvq_profile_next_launch), so elapsed times are kernel durations without the gaps
    between commands on the stream."""

    def __init__(self, kvq, n):
        import torch
        self.kvq = kvq
        self.ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(n)]
        for a, b in self.ev:      # a torch event gets its HIP handle when first recorded
            a.record()
            b.record()
        torch.cuda.synchronize()

    def arm(self, j):
        self.kvq.profile_next_launch(*self.ev[j])

    def us(self, j):
        a, b = self.ev[j]
        b.synchronize()
        return a.elapsed_time(b) * 1e3


def launch_floor(kvq, inputs, cs, reps=20):
    """The per-launch floor in the step's regime: a library launch that moves almost
    nothing (kv_store of one row whose slot is outside the pool: it loads the row and
    stores nothing), armed right after a C4A launch, so that it starts on a busy GPU as
    the mixed step's kernels do; dispatch-recorded events, median of `reps`."""
    import numpy as np
    import torch
    clock = DispatchTimer(kvq, 1)
    dev = inputs["c4a"]["kv"].device
    pool = kvq.new_pool(kvq.V41, 1, dev)
    k = torch.zeros((1, HEAD), dtype=torch.bfloat16, device=dev)
    slots = torch.full((1,), -1, dtype=torch.int32, device=dev)
    d = inputs["c4a"]
    ts = []
    for r in range(reps + 2):
        kvq.kv_compress_store(d["pool"], kvq.V41, d["kv"], d["sc"], d["ratio"], d["pos"], cs, d["slots"])
        clock.arm(0)
        kvq.kv_store(pool, kvq.V41, k, slots)
        if r >= 2:
            ts.append(clock.us(0))
    return {"us": round(float(np.median(ts)), 2), "us_p10": round(float(np.percentile(ts, 10)), 2),
            "us_p90": round(float(np.percentile(ts, 90)), 2),
            "method": "kv_store of one row with an out-of-pool slot (loads 1 KiB, stores nothing), "
                      "armed right after a C4A launch; HIP events recorded by its own dispatch, median"}


def fp4_configs(kvq, inputs, cs, reps=10):
    """C4A and C128A with the V41_FP4 layout: the same resident inputs, FP4 pools.  Each
    repetition runs C4A then C128A, so every C4A launch follows 8 GiB of other traffic and
    reads cold inputs.  Kernel durations from dispatch-recorded events, mean of `reps`."""
    import numpy as np
    clock = DispatchTimer(kvq, 1)
    pools = {n: kvq.new_pool(kvq.V41_FP4, inputs[n]["pool"].shape[0]) for n in ("c4a", "c128a")}
    times = {n: [] for n in pools}
    for k in range(reps + 1):
        for n in ("c4a", "c128a"):
            d = inputs[n]
            clock.arm(0)
            kvq.kv_compress_store(pools[n], kvq.V41_FP4, d["kv"], d["sc"], d["ratio"], d["pos"], cs, d["slots"])
            if k:
                times[n].append(clock.us(0))
    out = {"method": f"HIP events recorded by each launch's own dispatch, mean of {reps}"}
    for n, t in times.items():
        d = inputs[n]
        us = float(np.mean(t))
        b = bytes_compress(d["R"], d["ratio"], kvq.bytes_per_token(kvq.V41_FP4))
        out[n] = {"rows": d["R"], "ratio": d["ratio"], "us": round(us, 2), "alg_bytes": b,
                  "GB/s": round(b / us / 1e3, 1), "frac_of_peak": round(b / us / 1e3 / HBM_PEAK_GBS, 4),
                  "rows/s": round(d["R"] / (us * 1e-6), 1)}
    return out


def ratio_sweep(kvq, wl, dev, cs, kv, sc, c4_pool, c4_slots, reps=5):
    """NEXT-row measurements on the resident C128A inputs (2,097,152 fp32 rows of kv and
    score): every supported ratio r >= 2 compresses the same input rows into 2,097,152 / r
    output rows (V41); and the token-gather dequant of the 16,384 C4A rows."""
    import numpy as np
    import torch
    rng = np.random.default_rng(77)
    rows_in = kv.shape[0]
    num_pages = 20000          # room for 1,048,576 distinct slots (ratio 2)
    pool = kvq.new_pool(kvq.V41, num_pages)
    sweep = {}
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    clock = DispatchTimer(kvq, 1)
    for r in (2, 4, 8, 16, 32, 64, 128):
        R = rows_in // r
        pos = torch.from_numpy(rng.integers(0, 65536, R).astype(np.int32)).to(dev)
        slots = torch.from_numpy(wl.distinct_slots(rng, R, 64, num_pages * 64)).to(dev)
        times = []
        for k in range(reps + 1):
            clock.arm(0)
            kvq.kv_compress_store(pool, kvq.V41, kv[:R * r], sc[:R * r], r, pos, cs, slots)
            if k:
                times.append(clock.us(0))
        us = float(np.median(times))
        b = bytes_compress(R, r, kvq.bytes_per_token(kvq.V41))
        sweep[f"r{r}"] = {"rows": R, "us": round(us, 1), "GB/s": round(b / us / 1e3, 1),
                          "frac_of_peak": round(b / us / 1e3 / HBM_PEAK_GBS, 4)}
    # C4A- and C128A-shaped calls from a few rows (decode-time batches) to the benchmark's
    # size, each repetition on another region of the 8 GiB input so that it reads cold rows
    sizes = {}
    for r, Rs in ((4, (256, 1024, 4096, 16384, 65536)), (128, (64, 256, 1024, 4096, 16384))):
        for R in Rs:
            pos = torch.from_numpy(rng.integers(0, 65536, R).astype(np.int32)).to(dev)
            slots = torch.from_numpy(wl.distinct_slots(rng, R, 64, num_pages * 64)).to(dev)
            regions = rows_in // (R * r)
            times = []
            for k in range(reps + 1):
                o = (k * 7 % regions) * R * r
                clock.arm(0)
                kvq.kv_compress_store(pool, kvq.V41, kv[o:o + R * r], sc[o:o + R * r], r, pos, cs, slots)
                if k:
                    times.append(clock.us(0))
            us = float(np.median(times))
            b = bytes_compress(R, r, kvq.bytes_per_token(kvq.V41))
            sizes[f"r{r}_R{R}"] = {"us": round(us, 2), "GB/s": round(b / us / 1e3, 1),
                                   "frac_of_peak": round(b / us / 1e3 / HBM_PEAK_GBS, 4)}
    out = torch.empty((c4_slots.numel(), HEAD), dtype=torch.bfloat16, device=dev)
    times = []
    for k in range(reps + 1):
        clock.arm(0)
        kvq.kv_dequant_slots(c4_pool, kvq.V41, c4_slots, out)
        if k:
            times.append(clock.us(0))
    us = float(np.median(times))
    n = c4_slots.numel()
    b = n * (4 + kvq.bytes_per_token(kvq.V41) + HEAD * 2)
    gather = {"rows": n, "us": round(us, 2), "GB/s": round(b / us / 1e3, 1),
              "frac_of_peak": round(b / us / 1e3 / HBM_PEAK_GBS, 4)}
    # decode steps with the compressor state: 16,384 sequences add one row per call; one
    # full window (ratio calls) is timed, V41
    S = 16384
    state_pool = kvq.new_pool(kvq.V41, 4096)
    decode = {}
    for r in (4, 128):
        state, count = kvq.new_compress_state(S)
        ids = torch.randperm(S, device=dev, dtype=torch.int64).to(torch.int32)
        pos = torch.from_numpy(rng.integers(0, 65536, S).astype(np.int32)).to(dev)
        slots = torch.from_numpy(wl.distinct_slots(rng, S, 64, 4096 * 64)).to(dev)
        step_rows = [(kv[(k % 64) * S:(k % 64 + 1) * S], sc[(k % 64) * S:(k % 64 + 1) * S]) for k in range(r)]
        for k in range(r):      # one untimed window
            kvq.kv_compress_state_update(state_pool, kvq.V41, state, count, r, ids, step_rows[k][0],
                                         step_rows[k][1], pos, cs, slots)
        ev[0].record()
        for k in range(r):
            kvq.kv_compress_state_update(state_pool, kvq.V41, state, count, r, ids, step_rows[k][0],
                                         step_rows[k][1], pos, cs, slots)
        ev[1].record()
        ev[1].synchronize()
        us = ev[0].elapsed_time(ev[1]) * 1e3
        b = S * (r * (HEAD * 8 + 4 + 8) + 2 * (r - 1) * kvq.compress_state_bytes() + 4 + 4 + 256 +
                 kvq.bytes_per_token(kvq.V41))
        decode[f"r{r}"] = {"sequences": S, "us_per_step": round(us / r, 2), "GB/s": round(b / us / 1e3, 1),
                           "frac_of_peak": round(b / us / 1e3 / HBM_PEAK_GBS, 4)}
    return {"method": "HIP events recorded by each launch's own dispatch, median of %d launches "
                      "(decode steps: stream events around one full window); the ratio sweep reads the same 8 GiB "
                      "of cold inputs at every ratio; decode steps fold one row per sequence into "
                      "its 10 KiB float64 state per call (one full window timed); the size sweep "
                      "reads another region of the 8 GiB input at each repetition" % reps,
            "compress_ratio_sweep_v41": sweep, "compress_size_sweep_v41": sizes,
            "dequant_slots_c4a_rows": gather,
            "compress_state_decode_v41": decode}


# ---------------------------------------------------------------- rocprofv3 summaries
# `python bench.py --write-profiles RESULTS` condenses the CSV output of the three
# profiler runs below (written under RESULTS) into the text summaries in profiles/;
# bench.py reads `traffic` back from the PMC summary.
PROFILE_RUNS = {
    "trace": "rocprofv3 --kernel-trace --stats -f csv -d $RESULTS/prof_trace -o trace -- "
             "python3 bench.py --steps 10 --warmup 10 --no-cpu-baseline --no-micro",
    "fetch": "rocprofv3 --pmc FETCH_SIZE -f csv -d $RESULTS/pmc_fetch -o fetch -- "
             "python3 bench.py --steps 2 --warmup 1 --no-cpu-baseline --no-micro",
    "write": "rocprofv3 --pmc WRITE_SIZE -f csv -d $RESULTS/pmc_write -o write -- "
             "python3 bench.py --steps 2 --warmup 1 --no-cpu-baseline --no-micro",
    "dram": "rocprofv3 --pmc TCC_EA0_RDREQ_DRAM_32B_sum TCC_EA0_WRREQ_WRITE_DRAM_32B_sum "
            "TCC_EA0_RDREQ_128B_sum -f csv -d $RESULTS/pmc_dram -o dram -- "
            "python3 bench.py --steps 2 --warmup 1 --no-cpu-baseline --no-micro",
    "next": "rocprofv3 --kernel-trace --stats -f csv -d $RESULTS/prof_next -o next -- "
            "python3 bench.py --steps 1 --warmup 1 --no-cpu-baseline",
}
SHORT_NAMES = {
    "compress_long_kernel<(kvq::Layout)1, 128": "compress_long<V41, ratio 128> (C128A)",
    "compress_short_kernel<(kvq::Layout)1, 4, false>": "compress_short<V41, ratio 4> (C4A)",
    "compress_short_kernel<(kvq::Layout)2, 4, false>": "compress_short<V41_FP4, 4> (mixed, translating)",
    "dequant_kernel<(kvq::Layout)2": "dequant<V41_FP4> (mixed step)",
    "translate_kernel": "translate (three-launch mixed graph)",
    "__amd_rocclr_copyBuffer": "__amd_rocclr_copyBuffer (1 GiB device copy)",
}
COPY_KEY = SHORT_NAMES["__amd_rocclr_copyBuffer"]
DOM_KEY = SHORT_NAMES["compress_long_kernel<(kvq::Layout)1, 128"]
C4A_KEY = SHORT_NAMES["compress_short_kernel<(kvq::Layout)1, 4, false>"]


def _short_name(name):
    for k, v in SHORT_NAMES.items():
        if k in name:
            return v
    return None


def _find_csv(results, pattern):
    import glob
    found = glob.glob(os.path.join(results, pattern), recursive=True)
    if not found:
        raise SystemExit(f"bench.py --write-profiles: no {pattern} under {results}")
    return found[0]


def trace_summary(results, warmup=10):
    import csv
    import numpy as np
    rows = list(csv.DictReader(open(_find_csv(results, "prof_trace/**/trace_kernel_stats.csv"))))
    per = {}
    for r in csv.DictReader(open(_find_csv(results, "prof_trace/**/trace_kernel_trace.csv"))):
        name = _short_name(r["Kernel_Name"])
        if name is not None:
            per.setdefault(name, []).append((int(r["Start_Timestamp"]),
                                             (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3))
    lines = [
        "# rocprofv3 kernel-trace summary: one bench step (mixed V41_FP4 step + C4A + C128A), MI355X",
        f"# command: {PROFILE_RUNS['trace']}",
        "# (run from the repository root with TMPDIR=/tmp, RESULTS = the results directory;",
        "#  summarised by: python bench.py --write-profiles $RESULTS)",
        "# The bench launches every kernel on torch's current stream: 50 launches of each step",
        f"# kernel = {warmup} warmup steps + 10 timed steps + 3 passes of 10 steps that time the",
        "# kernels (plus the mixed step's graph replays).  avg_us covers every launch;",
        f"# after_warmup_us leaves out the first {warmup} launches of each kernel (the warmup",
        "# steps, during which the clocks settle), as the bench's own figures do.",
        "",
        f"{'kernel':<52} {'calls':>5} {'avg_us':>10} {'after_warmup_us':>16} {'min_us':>10} {'max_us':>10}",
    ]
    for r in rows:
        name = _short_name(r["Name"])
        if name is not None:
            d = [t for _, t in sorted(per.get(name, []))]
            aw = float(np.mean(d[warmup:])) if len(d) > warmup else float("nan")
            lines.append(f"{name:<52} {int(r['Calls']):>5} {float(r['AverageNs']) / 1e3:>10.2f} {aw:>16.2f} "
                         f"{float(r['MinNs']) / 1e3:>10.2f} {float(r['MaxNs']) / 1e3:>10.2f}")
    bench_json = os.path.join(results, "bench.json")
    if os.path.exists(bench_json):
        b = json.load(open(bench_json))
        lines += ["", "# bench.py (same build, separate run, default 50 timed steps; HIP events recorded by",
                  "# each kernel's own dispatch, so without the gaps between commands), mean us per launch:"]
        for k, v in b["kernels"].items():
            lines.append(f"#   {k:<22} {v['us']:>10.2f}  ({v['GB/s']} GB/s algorithmic, "
                         f"{100 * v['frac_of_peak']:.1f} % of 8 TB/s)")
    return "\n".join(lines) + "\n"


def _pmc_per_kernel(path, counter=None):
    import csv
    agg = {}
    for r in csv.DictReader(open(path)):
        name = _short_name(r["Kernel_Name"])
        if name is not None and (counter is None or r["Counter_Name"] == counter):
            agg.setdefault(name, []).append((int(r["Grid_Size"]), float(r["Counter_Value"])))
    return agg


def pmc_summary(results):
    import numpy as np
    f = _pmc_per_kernel(_find_csv(results, "pmc_fetch/**/fetch_counter_collection.csv"))
    w = _pmc_per_kernel(_find_csv(results, "pmc_write/**/write_counter_collection.csv"))
    # the calibration copies are the copyBuffer dispatches that write exactly 1 GiB
    big = {g for g, v in w[COPY_KEY] if abs(v - 1048576.0) < 1.0}
    copy_write = float(np.mean([v for g, v in w[COPY_KEY] if g in big]))
    copy_fetch = float(np.mean([v for g, v in f[COPY_KEY] if g in big]))
    fs = (1 << 30) / (copy_fetch * 1024)
    ws = (1 << 30) / (copy_write * 1024)
    fk = float(np.mean([v for _, v in f[DOM_KEY]]))
    wk = float(np.mean([v for _, v in w[DOM_KEY]]))
    dpath = _find_csv(results, "pmc_dram/**/dram_counter_collection.csv")
    dr = _pmc_per_kernel(dpath, "TCC_EA0_RDREQ_DRAM_32B_sum")
    dw = _pmc_per_kernel(dpath, "TCC_EA0_WRREQ_WRITE_DRAM_32B_sum")
    d128 = _pmc_per_kernel(dpath, "TCC_EA0_RDREQ_128B_sum")
    big_d = {g for g, v in dw[COPY_KEY] if abs(v * 32 - (1 << 30)) < (1 << 24)}
    copy_dr = float(np.mean([v for g, v in dr[COPY_KEY] if g in big_d])) * 32
    copy_dw = float(np.mean([v for g, v in dw[COPY_KEY] if g in big_d])) * 32
    dom_dr = float(np.mean([v for _, v in dr[DOM_KEY]])) * 32
    dom_dw = float(np.mean([v for _, v in dw[DOM_KEY]])) * 32
    dom_128 = float(np.mean([v for _, v in d128[DOM_KEY]]))
    lines = [
        "# rocprofv3 PMC summary: HBM traffic per dispatch, MI355X",
        f"# command (pass 1): {PROFILE_RUNS['fetch']}",
        f"# command (pass 2): {PROFILE_RUNS['write']}",
        "# (run from the repository root with TMPDIR=/tmp, RESULTS = the results directory;",
        "#  summarised by: python bench.py --write-profiles $RESULTS)",
        "# Counters are KiB per dispatch, averaged over the dispatches of each kernel.  Each is",
        "# scaled by what the same counter reads for a plain device copy of known size (the",
        "# bench's 1 GiB torch copy, __amd_rocclr_copyBuffer): on gfx950 FETCH_SIZE reports",
        f"# {1 / fs:.3f} of the copy's 1 GiB of reads (scale {fs:.1f}) and WRITE_SIZE {1 / ws:.3f} of its",
        f"# writes (scale {ws:.1f}).  kernel_source_sha256 identifies the kernel sources these",
        "# counters were taken on; bench.py reports `traffic` only while the sources still hash to it.",
        "",
        f"kernel_source_sha256: {kernel_source_hash()}",
        f"kernel: {DOM_KEY}",
        f"FETCH_SIZE_KiB_per_dispatch: {fk:.3f}",
        f"WRITE_SIZE_KiB_per_dispatch: {wk:.3f}",
        f"copy_bytes_each_way: {1 << 30}",
        f"copy_FETCH_SIZE_KiB_per_dispatch: {copy_fetch:.3f}",
        f"copy_WRITE_SIZE_KiB_per_dispatch: {copy_write:.3f}",
        "",
        f"# command (pass 3): {PROFILE_RUNS['dram']}",
        "# A second, uncalibrated count: DRAM read and write requests in 32-byte sectors",
        "# (TCC_EA0_RDREQ_DRAM_32B counts a 128-byte request as 4), times 32.  FETCH_SIZE's",
        "# formula counts every read request that is not 32 bytes as 64 bytes, while gfx950 reads",
        "# in 128-byte requests (TCC_EA0_RDREQ_128B), which is why the copy calibration finds 2.0.",
        f"DRAM_read_bytes_per_dispatch: {dom_dr:.0f}",
        f"DRAM_write_bytes_per_dispatch: {dom_dw:.0f}",
        f"RDREQ_128B_per_dispatch: {dom_128:.0f}",
        f"copy_DRAM_read_bytes_per_dispatch: {copy_dr:.0f}",
        f"copy_DRAM_write_bytes_per_dispatch: {copy_dw:.0f}",
        "",
        f"# all kernels of the step (raw KiB per dispatch; scaled bytes = fetch*1024*{fs:.1f} + "
        f"write*1024*{ws:.1f}):",
    ]
    alg = {DOM_KEY: bytes_compress(16384, 128, 528), C4A_KEY: bytes_compress(16384, 4, 528)}
    for k in f:
        if k == COPY_KEY:
            continue
        fa = float(np.mean([v for _, v in f[k]]))
        wa = float(np.mean([v for _, v in w[k]])) if k in w else 0.0
        tot = fa * 1024 * fs + wa * 1024 * ws
        dram = (float(np.mean([v for _, v in dr[k]])) + float(np.mean([v for _, v in dw.get(k, [(0, 0.0)])]))) * 32 \
            if k in dr else float("nan")
        extra = f"  ({tot / alg[k]:.3f} x algorithmic)" if k in alg else ""
        lines.append(f"#   {k:<48} fetch {fa:>14.1f}  write {wa:>12.1f}  -> {tot / 1e6:>10.2f} MB"
                     f"  (DRAM sectors {dram / 1e6:>10.2f} MB){extra}")
    return "\n".join(lines) + "\n"


def _kernel_label(name):
    """Readable label of a library kernel from its (demangled) name, e.g.
    compress_long_kernel<V41, 64, 8, 2>; None for kernels outside the library."""
    import re
    m = re.search(r"kvq::(\w+)(?:<([^>]*)>)?\(", name)
    if m is None:
        return None
    args = m.group(2)
    if args:
        args = args.replace("(kvq::Layout)1", "V41").replace("(kvq::Layout)2", "V41_FP4")
        return f"{m.group(1)}<{args}>"
    return m.group(1)


def all_kernels_summary(results):
    """Every library kernel of the run that includes the measurements beside the step,
    grouped by kernel and grid (one line per configuration), with its registers and LDS."""
    import csv
    import numpy as np
    groups = {}
    for r in csv.DictReader(open(_find_csv(results, "prof_next/**/next_kernel_trace.csv"))):
        label = _kernel_label(r["Kernel_Name"])
        if label is None:
            continue
        wg = int(r["Workgroup_Size_X"])
        key = (label, int(r["Grid_Size_X"]) // wg, wg, int(r["LDS_Block_Size"]))
        groups.setdefault(key, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    lines = [
        "# rocprofv3 kernel-trace summary: every library kernel of one full bench run (one timed",
        "# step plus the measurements beside it: FP4 C4A/C128A, store configs, graph-replayed",
        "# latency table, hoisting case, ratio sweep, token gather, decode state), MI355X,",
        "# one line per kernel and grid (workgroups x threads per workgroup), with the LDS bytes",
        "# per workgroup the trace reports",
        f"# command: {PROFILE_RUNS['next']}",
        "# (run from the repository root with TMPDIR=/tmp, RESULTS = the results directory;",
        "#  summarised by: python bench.py --write-profiles $RESULTS)",
        "",
        f"{'kernel':<44} {'workgroups':>10} {'thr':>5} {'lds':>6} {'calls':>6} "
        f"{'avg_us':>9} {'min_us':>9} {'max_us':>9}",
    ]
    for (label, nwg, wg, lds), t in sorted(groups.items()):
        t = np.array(t)
        lines.append(f"{label:<44} {nwg:>10} {wg:>5} {lds:>6} {t.size:>6} "
                     f"{t.mean():>9.2f} {t.min():>9.2f} {t.max():>9.2f}")
    return "\n".join(lines) + "\n"


def write_profiles(results):
    # the summaries are stamped with the hash of the sources in the tree; the library next
    # to them must have been built from those sources (load_library refuses a stale one)
    import quantized_paged_kv_compress_amd as kvq
    kvq.load_library()
    out = os.path.join(ROOT, "profiles")
    os.makedirs(out, exist_ok=True)
    outputs = [("bench_step_kernel_trace.txt", trace_summary(results)),
               ("compress_c128a_v41_pmc.txt", pmc_summary(results))]
    import glob
    if glob.glob(os.path.join(results, "prof_next/**/next_kernel_trace.csv"), recursive=True):
        outputs.append(("all_kernels_full_bench_trace.txt", all_kernels_summary(results)))
    for name, text in outputs:
        with open(os.path.join(out, name), "w") as fh:
            fh.write(text)
        print(text)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-micro", action="store_true",
                    help="skip the measurements beside the step: FP4 C4A/C128A, store configs, "
                         "latency table, hoisting case, ratio sweep")
    ap.add_argument("--write-profiles", metavar="RESULTS",
                    help="summarise rocprofv3 CSVs under RESULTS into profiles/ and exit (no GPU)")
    args = ap.parse_args()
    if args.write_profiles:
        write_profiles(args.write_profiles)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this path runs on one GPU; every output row depends only on its own "
              "window, so N GPUs would each run this same step on their own share "
              "(this library runs on one GPU; run one process per GPU).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import quantized_paged_kv_compress_amd as kvq
    from quantized_paged_kv_compress_amd import workloads as wl
    if not os.path.exists(kvq.LIB_PATH):
        from quantized_paged_kv_compress_amd import _build
        _build.build()
    kvq.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def log(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    def up(a):
        if a.dtype == np.uint16:
            a = a.view(np.int16)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    # ------------------------------------------------------------ inputs (HBM resident)
    t_gen = time.perf_counter()
    cs_host = wl.rope_cos_sin()
    cs = up(cs_host)
    inputs = {}
    cpu_rows_t = {}   # oracle seconds per workload (timed oracle calls only)
    cpu_1t = {}       # single-thread oracle: (rows, seconds) on the first chunk of each workload
    if not args.no_cpu_baseline:
        import oracle
        oracle.lib()
        all_threads = oracle.num_threads()

    def median_of_three(fn):
        """Median seconds of three runs of fn (the oracle on the same inputs)."""
        ts = []
        for _ in range(3):
            t = time.perf_counter()
            fn()
            ts.append(time.perf_counter() - t)
        return sorted(ts)[1]

    def oracle_one_thread(fn, rows, key):
        oracle.set_num_threads(1)
        cpu_1t[key] = (rows, median_of_three(fn))
        oracle.set_num_threads(all_threads)
    for name, seed, ratio in (("c4a", 3, 4), ("c128a", 4, 128)):
        R = 16384
        meta = wl.compressor_meta(seed, R)
        kv = torch.empty((R * ratio, HEAD), dtype=torch.float32, device=dev)
        sc = torch.empty_like(kv)
        step = max(1, (1 << 26) // (HEAD * ratio))
        orc_pool = None if args.no_cpu_baseline else oracle.new_pool(oracle.V41, meta["num_pages"])
        t_orc = 0.0
        for i0 in range(0, R, step):
            n = min(step, R - i0)
            a, b = wl.compressor_window(seed, ratio, i0, n)
            kv[i0 * ratio:(i0 + n) * ratio].copy_(torch.from_numpy(a))
            sc[i0 * ratio:(i0 + n) * ratio].copy_(torch.from_numpy(b))
            if orc_pool is not None:   # CPU baseline: the oracle on the same rows, chunk by chunk
                pos_c = np.ascontiguousarray(meta["pos"][i0:i0 + n])
                slots_c = np.ascontiguousarray(meta["slots"][i0:i0 + n])
                t_orc += median_of_three(lambda: oracle.kv_compress_store(oracle.V41, orc_pool, a, b, ratio,
                                                                          pos_c, cs_host, slots_c))
                if i0 == 0:
                    scratch = oracle.new_pool(oracle.V41, meta["num_pages"])
                    oracle_one_thread(lambda: oracle.kv_compress_store(
                        oracle.V41, scratch, a, b, ratio, pos_c, cs_host, slots_c), n, name)
                    del scratch
        cpu_rows_t[name] = t_orc
        del orc_pool
        inputs[name] = dict(R=R, ratio=ratio, kv=kv, sc=sc, pos=up(meta["pos"]),
                            slots=up(meta["slots"]), pool=kvq.new_pool(kvq.V41, meta["num_pages"]))
        log(f"{name}: inputs ready ({2 * kv.numel() * 4 / 2**30:.2f} GiB)")
    mx = wl.mixed_fp4(seed=5)
    m = dict(R=mx["R"], kv=up(mx["kv"]), sc=up(mx["score"]), pos=up(mx["pos"]),
             table=up(mx["table"]), full=up(mx["full"]),
             loc=torch.empty(mx["cap"], dtype=torch.int32, device=dev),
             page_ids=up(mx["page_ids"]), pool=kvq.new_pool(kvq.V41_FP4, mx["num_pages"]))
    m["ws"] = torch.empty((mx["page_ids"].size * 64, HEAD), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()
    log(f"mixed: R={m['R']}, pages={mx['page_ids'].size}; inputs generated in "
        f"{time.perf_counter() - t_gen:.1f} s")

    c4, c128 = inputs["c4a"], inputs["c128a"]
    # the mixed step's compressor translates its full-pool slots itself
    # (kv_compress_store_translate) and leaves them in m["loc"] for later consumers
    names = ["compress_mixed_fp4", "dequant_fp4", "compress_c4a", "compress_c128a"]

    # The timed region runs the steps alone, with nothing recorded between the launches.
    # Kernel durations come from events that a kernel's own dispatch records
    # (kvq_profile_next_launch) in passes of the same steps right after it; each armed
    # launch adds a few microseconds of gap on the stream, so one pass arms C4A and C128A
    # and another the mixed step's kernels.  A third pass brackets every kernel with events
    # recorded on the stream (these hold the gap between commands as well).
    timed_armed = {2, 3}

    def step(k=None, armed=(), clocks=None, ev=None):
        def arm(j):
            if j in armed:
                clocks[k].arm(j)
        if ev: ev[0].record()
        arm(0)
        kvq.kv_compress_store_translate(m["pool"], kvq.V41_FP4, m["kv"], m["sc"], 4, m["pos"], cs,
                                        m["table"], m["full"], m["loc"])
        if ev: ev[1].record()
        arm(1)
        kvq.kv_dequant(m["pool"], kvq.V41_FP4, m["page_ids"], m["ws"])
        if ev: ev[2].record()
        arm(2)
        kvq.kv_compress_store(c4["pool"], kvq.V41, c4["kv"], c4["sc"], 4, c4["pos"], cs, c4["slots"])
        if ev: ev[3].record()
        arm(3)
        kvq.kv_compress_store(c128["pool"], kvq.V41, c128["kv"], c128["sc"], 128, c128["pos"], cs,
                              c128["slots"])
        if ev: ev[4].record()

    for _ in range(args.warmup):
        step()
    stream_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(args.steps)]
    clocks = [DispatchTimer(kvq, len(names)) for _ in range(args.steps)]
    extra = [DispatchTimer(kvq, len(names)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    for k in range(args.steps):
        step(k, timed_armed, clocks)
    other = [j for j in range(len(names)) if j not in timed_armed]
    for k in range(args.steps):
        step(k, other, extra)
    for k in range(args.steps):
        step(k, ev=stream_ev[k])
    torch.cuda.synchronize()
    per = {n: [] for n in names}
    per_stream = {n: [] for n in names}
    for k in range(args.steps):
        for j, n in enumerate(names):
            per[n].append((clocks if j in timed_armed else extra)[k].us(j) * 1e-3)
            per_stream[n].append(stream_ev[k][j].elapsed_time(stream_ev[k][j + 1]))
    avg_ms = {n: float(np.mean(v)) for n, v in per.items()}
    avg_stream_ms = {n: float(np.mean(v)) for n, v in per_stream.items()}
    log("timed region done: " + ", ".join(f"{n} {avg_ms[n] * 1e3:.1f} us "
                                          f"({avg_stream_ms[n] * 1e3:.1f} between stream events)"
                                          for n in names))

    fp4 = None
    if not args.no_micro:
        fp4 = fp4_configs(kvq, inputs, cs)
        log(f"fp4 configs: c4a {fp4['c4a']['us']} us ({fp4['c4a']['frac_of_peak']}), "
            f"c128a {fp4['c128a']['us']} us ({fp4['c128a']['frac_of_peak']})")
    floor = launch_floor(kvq, inputs, cs)
    log(f"launch floor: {floor['us']} us")

    # achievable-bandwidth reference (context): a plain 1 GiB device copy
    src = torch.empty(1 << 28, dtype=torch.float32, device=dev).normal_()
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    ce = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ce[0].record()
    for _ in range(10):
        dst.copy_(src)
    ce[1].record()
    torch.cuda.synchronize()
    copy_gbs = 2 * src.numel() * 4 * 10 / (ce[0].elapsed_time(ce[1]) * 1e-3) / 1e9
    del src, dst

    pb_fp4, pb_v41 = kvq.page_bytes(kvq.V41_FP4), kvq.page_bytes(kvq.V41)
    alg = {
        "compress_mixed_fp4": (bytes_compress(m["R"], 4, kvq.bytes_per_token(kvq.V41_FP4))
                               + bytes_translate(m["R"], mx["cap"])),
        "dequant_fp4": bytes_dequant(mx["page_ids"].size, pb_fp4),
        "compress_c4a": bytes_compress(16384, 4, kvq.bytes_per_token(kvq.V41)),
        "compress_c128a": bytes_compress(16384, 128, kvq.bytes_per_token(kvq.V41)),
    }
    rows = {"compress_mixed_fp4": m["R"], "compress_c4a": 16384, "compress_c128a": 16384}
    kernels = {}
    for n in names:
        gbs = alg[n] / (avg_ms[n] * 1e-3) / 1e9
        p10, p50, p90 = (float(np.percentile(per[n], q)) * 1e3 for q in (10, 50, 90))
        kernels[n] = {"us": round(avg_ms[n] * 1e3, 2), "us_median": round(p50, 2),
                      "us_p10": round(p10, 2), "us_p90": round(p90, 2),
                      "us_between_stream_events": round(avg_stream_ms[n] * 1e3, 2),
                      "alg_bytes": alg[n], "GB/s": round(gbs, 1),
                      "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4)}
        if n in rows:
            kernels[n]["rows/s"] = round(rows[n] / (avg_ms[n] * 1e-3), 1)
    rows_per_step = sum(rows.values())
    dom = "compress_c128a"
    mixed_alg = alg["compress_mixed_fp4"] + alg["dequant_fp4"]
    g_us, g_p10, g_p90 = mixed_graph(kvq, m, cs, fused=True)
    s_us, _, _ = mixed_graph(kvq, m, cs, fused=False)
    w_us, _, _ = mixed_graph(kvq, m, cs, fused=True, flush_mode="write")
    mixed_graph_line = {"us": round(g_us, 2), "us_p10": round(g_p10, 2), "us_p90": round(g_p90, 2),
                  "alg_bytes": mixed_alg, "GB/s": round(mixed_alg / (g_us * 1e-6) / 1e9, 1),
                  "frac_of_peak": round(mixed_alg / (g_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                  "separate_translate_us": round(s_us, 2),
                  "separate_translate_frac_of_peak": round(mixed_alg / (s_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                  "after_512MiB_write_us": round(w_us, 2),
                  "after_512MiB_write_frac_of_peak": round(mixed_alg / (w_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                  "method": "compress with the translation fused in (kv_compress_store_translate) + dequant "
                            "replayed as one HIP graph, cold inputs (512 MiB read before each replay), "
                            "median of 20 replays timed by stream events around each; separate_translate: "
                            "the same step with kv_translate_slots as a launch of its own; "
                            "after_512MiB_write: inputs evicted by writing 512 MiB instead, which leaves "
                            "dirty lines in the last-level cache for the step to write back"}
    log(f"mixed step as one graph: {mixed_graph_line['us']} us, {mixed_graph_line['frac_of_peak']} of peak")
    traffic = read_traffic(alg[dom])

    micro = nxt = stores = None
    if not args.no_micro:
        stores = store_configs(kvq, wl, dev, cs)
        log(f"store configs: {stores}")
        micro = micro_bench(kvq, wl, dev, cs)
        log(f"micro: {micro['latency_us']}; hoisting {micro['swa_hoisting']}")
        nxt = ratio_sweep(kvq, wl, dev, cs, c128["kv"], c128["sc"], c4["pool"], c4["slots"])
        log(f"ratio sweep: {nxt['compress_ratio_sweep_v41']}; gather {nxt['dequant_slots_c4a_rows']}")

    # ------------------------------------------------------------ CPU oracle baseline
    cpu = None
    if not args.no_cpu_baseline:
        def mixed_step():
            rc, loc_h = oracle.translate_slots(mx["table"], mx["full"], mx["cap"])
            pool = oracle.new_pool(oracle.V41_FP4, mx["num_pages"])
            oracle.kv_compress_store(oracle.V41_FP4, pool, mx["kv"], mx["score"], 4, mx["pos"], cs_host,
                                     loc_h[: mx["R"]].copy())
            oracle.kv_dequant(oracle.V41_FP4, pool, mx["page_ids"])

        t_mixed = median_of_three(mixed_step)
        oracle_one_thread(mixed_step, m["R"], "mixed")
        cpu_step = t_mixed + cpu_rows_t["c4a"] + cpu_rows_t["c128a"]
        # single thread, projected to the whole step from the timed samples
        step_1t = cpu_1t["mixed"][1] + sum(cpu_1t[k][1] * 16384 / cpu_1t[k][0] for k in ("c4a", "c128a"))
        cpu = {"value": round(rows_per_step / cpu_step, 1), "unit": "rows/s",
               "cores": oracle.num_threads(), "kind": "oracle", "cpu_model": cpu_model(),
               "sample": ("the whole step: every row of the mixed FP4 step, C4A and C128A, each part "
                          "timed three times on the same inputs and the median kept, OpenMP over rows; "
                          "input generation excluded (C128A timed chunk by chunk as its inputs are "
                          "generated)"),
               "seconds": {"mixed_fp4": round(t_mixed, 3), "c4a": round(cpu_rows_t["c4a"], 3),
                           "c128a": round(cpu_rows_t["c128a"], 3)},
               "single_thread": {
                   "value": round(rows_per_step / step_1t, 1), "unit": "rows/s", "cores": 1,
                   "sample": ("one thread on the whole mixed FP4 step, all 16,384 C4A rows and the "
                              f"first {cpu_1t['c128a'][0]} C128A rows (median of three runs each), "
                              "projected to the whole step"),
                   "seconds": {k: round(v[1], 3) for k, v in cpu_1t.items()}}}
        log(f"cpu oracle: {cpu['value']} rows/s on {cpu['cores']} threads ({cpu_step:.2f} s per step)")

    out = {
        "metric": METRIC,
        "value": round(rows_per_step / (ms_per_step * 1e-3), 1),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": ("mixed V41_FP4 step (ratio-4 compress with the full->SWA slot translation "
                         "fused in + dequant) + C4A "
                         "(R=16384, ratio 4, V41) + C128A (R=16384, ratio 128, V41); fp32 kv/score "
                         "x 512 channels, 64-token pages"),
            "rows_per_step": rows_per_step,
            "mixed_rows": m["R"], "mixed_pages": int(mx["page_ids"].size),
            "c4a_rows": 16384, "c128a_rows": 16384,
        },
        "roofline": {
            "kernel": "compress_long_kernel<V41, ratio 128> (C128A)",
            "bound": "hbm",
            "achieved": kernels[dom]["GB/s"],
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": kernels[dom]["frac_of_peak"],
            "traffic": None if traffic is None else round(traffic["bytes"]),
        },
        "cpu_baseline": cpu,
        "library_build_id": kvq.load_library().kvq_build_id().decode(),
        "device": device_facts(torch),
        "mixed_fp4_step_graph": mixed_graph_line,
        "kernels": kernels,
        "kernel_timing": ("the timed region runs the steps with nothing recorded between launches; "
                          "us: HIP events recorded by the kernel's own dispatch (hipExtLaunchKernel), "
                          "mean over a pass of the same steps right after the timed region (one pass "
                          "for compress_c4a and compress_c128a, one for the mixed step's kernels); "
                          "us_between_stream_events: a third pass with events recorded on the stream "
                          "between the launches, which also hold the gap between commands"),
        "copy_1GiB_GB/s": round(copy_gbs, 1),
        "store_configs": stores,
        "micro": micro,
        "pages_context": {
            "note": "the pages' own figures, measured on other hardware: context, not targets",
            "store_bs512_us": "1.49 -> 1.39 (hardware not stated)",
            "c4a_us_gb200": 89.685, "c128a_us_gb200": 1606.181,
            "c4a_us_here": kernels["compress_c4a"]["us"], "c128a_us_here": kernels[dom]["us"],
        },
        "next_rows": nxt,
        "fp4_configs": fp4,
        "launch_floor": floor,
        "c4a": {"rows/s": kernels["compress_c4a"]["rows/s"], "GB/s": kernels["compress_c4a"]["GB/s"],
                "frac_of_peak": kernels["compress_c4a"]["frac_of_peak"]},
        "c128a": {"rows/s": kernels[dom]["rows/s"], "GB/s": kernels[dom]["GB/s"],
                  "frac_of_peak": kernels[dom]["frac_of_peak"]},
    }
    if traffic is not None:
        out["roofline"]["traffic_over_algorithmic"] = round(traffic["ratio_to_algorithmic"], 4)
        out["roofline"]["traffic_source"] = ("DRAM read + write sectors (TCC_EA0_RDREQ_DRAM_32B, "
                                             "TCC_EA0_WRREQ_WRITE_DRAM_32B) x 32 B per launch")
        out["roofline"]["traffic_fetch_write_scaled"] = round(traffic["fetch_write_scaled_bytes"])
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
