"""Edge cases on the GPU: boundary slots and positions for every writing entry point, and
compressor inputs at the edges of the domain (all-zero windows, fp32-denormal and very
large kv, score spreads wide enough for exp to underflow), against the CPU oracle."""
import numpy as np
import pytest

from helpers import FP4, V41, compare_compressed, gpu_lib, to_dev, to_host, untouched_equal
from quantized_paged_kv_compress_amd import workloads as wl

pytestmark = pytest.mark.gpu
LAYOUTS = [V41, FP4]
NUM_PAGES = 6
I32 = np.iinfo(np.int32)
EDGE_SLOTS = np.array([0, 63, 64, NUM_PAGES * 64 - 1, NUM_PAGES * 64, -1, I32.max, I32.min,
                       NUM_PAGES * 64 - 64, 1], np.int32)


@pytest.fixture(scope="module")
def kvq():
    return gpu_lib()


@pytest.fixture(scope="module")
def cs_small():
    return wl.rope_cos_sin(max_pos=100)


def canary(kvq, layout):
    pool = kvq.new_pool(layout, NUM_PAGES)
    pool.fill_(0x77)
    return pool, np.full((NUM_PAGES, kvq.page_bytes(layout)), 0x77, np.uint8)


@pytest.mark.parametrize("layout", LAYOUTS)
def test_boundary_slots_and_positions_store_paths(kvq, orc, cs_small, layout):
    rng = np.random.default_rng(61)
    n = EDGE_SLOTS.size
    k = wl.bf16_bits(rng.standard_normal((n, 512)).astype(np.float32))
    pos = np.array([0, 99, 50, 99, 3, 0, 1, 2, 100, -1], np.int32)   # 100 and -1 skip
    w = wl.bf16_bits(rng.uniform(0.5, 1.5, 512).astype(np.float32))
    for name in ("store", "rope", "norm"):
        pool, ref = canary(kvq, layout)
        if name == "store":
            kvq.kv_store(pool, layout, to_dev(k), to_dev(EDGE_SLOTS))
            orc.kv_store(layout, ref, k, EDGE_SLOTS)
        elif name == "rope":
            kvq.kv_store_rope(pool, layout, to_dev(k), to_dev(pos), to_dev(cs_small), to_dev(EDGE_SLOTS))
            orc.kv_store_rope(layout, ref, k, pos, cs_small, EDGE_SLOTS)
        else:
            kvq.kv_store_norm_rope(pool, layout, to_dev(k), to_dev(w), 1e-6, to_dev(pos), to_dev(cs_small),
                                   to_dev(EDGE_SLOTS))
            orc.kv_store_norm_rope(layout, ref, k, w, 1e-6, pos, cs_small, EDGE_SLOTS)
        got = to_host(pool)
        if name == "norm":
            valid = (EDGE_SLOTS >= 0) & (EDGE_SLOTS < NUM_PAGES * 64) & (pos >= 0) & (pos < 100)
            compare_compressed(got, ref, layout, EDGE_SLOTS[valid], label=f"edge norm L{layout}")
            assert untouched_equal(got, ref, layout, EDGE_SLOTS[valid])
        else:
            assert np.array_equal(got, ref), name


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("ratio", [1, 4, 128])
def test_boundary_slots_compress(kvq, orc, cs_small, layout, ratio):
    rng = np.random.default_rng(62 + ratio)
    R = EDGE_SLOTS.size
    kv = rng.standard_normal((R * ratio, 512)).astype(np.float32)
    sc = (2 * rng.standard_normal((R * ratio, 512))).astype(np.float32)
    pos = np.array([0, 99, 50, 99, 3, 0, 1, 2, 100, -1], np.int32)
    pool, ref = canary(kvq, layout)
    kvq.kv_compress_store(pool, layout, to_dev(kv), to_dev(sc) if ratio > 1 else None, ratio, to_dev(pos),
                          to_dev(cs_small), to_dev(EDGE_SLOTS))
    orc.kv_compress_store(layout, ref, kv, sc, ratio, pos, cs_small, EDGE_SLOTS)
    got = to_host(pool)
    valid = (EDGE_SLOTS >= 0) & (EDGE_SLOTS < NUM_PAGES * 64) & (pos >= 0) & (pos < 100)
    compare_compressed(got, ref, layout, EDGE_SLOTS[valid], label=f"edge slots r{ratio}")
    assert untouched_equal(got, ref, layout, EDGE_SLOTS[valid])


def extreme_windows(rng, ratio, R):
    """Window families: zeros, fp32-denormal kv, large kv, wide score spreads, ties."""
    kv = rng.standard_normal((R * ratio, 512)).astype(np.float32)
    sc = (2 * rng.standard_normal((R * ratio, 512))).astype(np.float32)
    fam = np.arange(R) % 6
    for i in range(R):
        rows = slice(i * ratio, (i + 1) * ratio)
        if fam[i] == 0:
            kv[rows] = 0.0                                         # all-zero window
        elif fam[i] == 1:
            kv[rows] *= np.float32(1e-40)                          # fp32 denormals
        elif fam[i] == 2:
            kv[rows] *= np.float32(1e36 / ratio)                   # large, sums stay finite
        elif fam[i] == 3:
            sc[rows] *= np.float32(60.0)                           # exp underflow for most rows
        elif fam[i] == 4:
            sc[rows] = np.float32(3.0)                             # equal scores: the mean
        else:
            kv[rows] *= np.float32(1e-20)                          # small normals
    return kv, sc


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("ratio", [2, 4, 128])
def test_compress_extreme_values(kvq, orc, layout, ratio):
    rng = np.random.default_rng(63 + ratio)
    R = 60 if ratio < 128 else 24
    kv, sc = extreme_windows(rng, ratio, R)
    cs = wl.rope_cos_sin(max_pos=4096)
    pos = rng.integers(0, 4096, R).astype(np.int32)
    slots = wl.distinct_slots(rng, R, 64, NUM_PAGES * 64)
    pool = kvq.new_pool(layout, NUM_PAGES)
    kvq.kv_compress_store(pool, layout, to_dev(kv), to_dev(sc), ratio, to_dev(pos), to_dev(cs), to_dev(slots))
    ref = orc.new_pool(layout, NUM_PAGES)
    orc.kv_compress_store(layout, ref, kv, sc, ratio, pos, cs, slots)
    compare_compressed(to_host(pool), ref, layout, slots, label=f"extreme r{ratio} L{layout}")


@pytest.mark.parametrize("layout", LAYOUTS)
def test_compress_state_edges(kvq, orc, layout):
    """Ratio 4: a window completed at an out-of-pool slot stores nothing but is consumed;
    out-of-range state ids are skipped; extreme values as in the batch test."""
    import torch
    rng = np.random.default_rng(64)
    ratio, S = 4, 12
    kv, sc = extreme_windows(rng, ratio, S)          # window of sequence s = rows [4s, 4s+4)
    cs = wl.rope_cos_sin(max_pos=4096)
    pos = rng.integers(0, 4096, S).astype(np.int32)
    slots = wl.distinct_slots(rng, S, 64, NUM_PAGES * 64)
    slots[5] = NUM_PAGES * 64                         # consumed, stores nothing
    pool = kvq.new_pool(layout, NUM_PAGES)
    state, count = kvq.new_compress_state(S)
    for t in range(ratio):
        ids = np.arange(S, dtype=np.int32)
        ids_call = np.concatenate([ids, [-1, S]]).astype(np.int32)   # two skipped rows
        kv_t = np.concatenate([kv[ids * ratio + t], kv[:2]])
        sc_t = np.concatenate([sc[ids * ratio + t], sc[:2]])
        kvq.kv_compress_state_update(pool, layout, state, count, ratio, to_dev(ids_call), to_dev(kv_t),
                                     to_dev(sc_t), to_dev(np.concatenate([pos, pos[:2]])), to_dev(cs),
                                     to_dev(np.concatenate([slots, slots[:2]])))
    torch.cuda.synchronize()
    assert np.all(to_host(count) == 0)
    ref = orc.new_pool(layout, NUM_PAGES)
    orc.kv_compress_store(layout, ref, kv, sc, ratio, pos, cs, slots)
    valid = slots < NUM_PAGES * 64
    got = to_host(pool)
    compare_compressed(got, ref, layout, slots[valid], label=f"state edges L{layout}")
    assert untouched_equal(got, ref, layout, slots[valid])


def test_binding_rejects_strided_index_arrays(kvq):
    """Index arrays are passed by pointer, so a strided view is refused, not misread."""
    import torch
    pool = kvq.new_pool(V41, 4)
    k = torch.zeros((8, 512), dtype=torch.bfloat16, device="cuda")
    idx = torch.arange(64, 80, dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError):
        kvq.kv_store(pool, V41, k, idx[::2])
    with pytest.raises(ValueError):
        kvq.kv_dequant(pool, V41, torch.zeros(8, dtype=torch.int32, device="cuda")[::2])
    table = torch.arange(128, dtype=torch.int32, device="cuda")
    out = torch.empty(16, dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError):
        kvq.kv_translate_slots(table, idx[::2], out)
    kvq.kv_store(pool, V41, k, idx[::2].contiguous())       # the same data, contiguous: fine
    torch.cuda.synchronize()


def test_pool_larger_than_4gib(kvq, orc, cs_small):
    """Byte offsets past 2^32: rows stored in the last pages of a 4.4 GB V41 pool (and
    around the 4 GiB mark) equal the oracle's rows, as do the page dequant and the gather."""
    import torch
    num_pages = (1 << 17) + 64                       # 131,136 pages x 33,792 B = 4.43 GB
    pool = kvq.new_pool(V41, num_pages)
    assert pool.numel() > 1 << 32
    boundary_page = (1 << 32) // 33792               # the page that straddles byte 2^32
    pages = np.array([boundary_page - 1, boundary_page, boundary_page + 1, num_pages - 2,
                      num_pages - 1], np.int64)
    rng = np.random.default_rng(66)
    slots = np.concatenate([p * 64 + rng.choice(64, 8, replace=False) for p in pages]).astype(np.int32)
    n = slots.size
    k = wl.bf16_bits(rng.standard_normal((n, 512)).astype(np.float32))
    pos = rng.integers(0, 100, n).astype(np.int32)
    kvq.kv_store_rope(pool, V41, to_dev(k), to_dev(pos), to_dev(cs_small), to_dev(slots))
    # the oracle works on a small pool holding the same pages in the same order
    local = {int(p): i for i, p in enumerate(pages)}
    small_slots = np.array([local[int(s) >> 6] * 64 + (int(s) & 63) for s in slots], np.int32)
    ref = orc.new_pool(V41, pages.size)
    orc.kv_store_rope(V41, ref, k, pos, cs_small, small_slots)
    got = to_host(pool[torch.from_numpy(pages).to("cuda")])
    assert np.array_equal(got, ref)
    # page dequant and token gather read the same far rows back
    out = kvq.kv_dequant(pool, V41, to_dev(pages.astype(np.int32)))
    assert np.array_equal(to_host(out).view(np.uint16), orc.kv_dequant(V41, ref, np.arange(pages.size, dtype=np.int32)))
    g = kvq.kv_dequant_slots(pool, V41, to_dev(slots))
    ref_g = np.zeros((n, 512), np.uint16)
    orc.kv_dequant_slots(V41, ref, small_slots, ref_g)
    assert np.array_equal(to_host(g).view(np.uint16), ref_g)
    # a ratio-4 compressor writing to the same far slots
    kv = rng.standard_normal((n * 4, 512)).astype(np.float32)
    sc = (2 * rng.standard_normal((n * 4, 512))).astype(np.float32)
    kvq.kv_compress_store(pool, V41, to_dev(kv), to_dev(sc), 4, to_dev(pos), to_dev(cs_small), to_dev(slots))
    ref2 = orc.new_pool(V41, pages.size)
    orc.kv_compress_store(V41, ref2, kv, sc, 4, pos, cs_small, small_slots)
    got2 = to_host(pool[torch.from_numpy(pages).to("cuda")])
    compare_compressed(got2, ref2, V41, small_slots, label="pool > 4 GiB")
    del pool
    torch.cuda.empty_cache()


def test_empty_inputs_through_the_binding(kvq, cs_small):
    """Zero rows is a no-op for every writer (the pool keeps its canary bytes), empty page or
    slot lists give empty workspaces, and translate with n = 0 still zeroes its buffer."""
    import torch
    dev = "cuda"
    for layout in LAYOUTS:
        pool, ref = canary(kvq, layout)
        k0 = torch.empty((0, 512), dtype=torch.bfloat16, device=dev)
        i0 = torch.empty(0, dtype=torch.int32, device=dev)
        f0 = torch.empty((0, 512), dtype=torch.float32, device=dev)
        w = torch.ones(512, dtype=torch.bfloat16, device=dev)
        cs = to_dev(cs_small)
        kvq.kv_store(pool, layout, k0, i0)
        kvq.kv_store_rope(pool, layout, k0, i0, cs, i0)
        kvq.kv_store_norm_rope(pool, layout, k0, w, 1e-6, i0, cs, i0)
        for ratio in (1, 4, 128):
            kvq.kv_compress_store(pool, layout, f0, f0 if ratio > 1 else None, ratio, i0, cs, i0)
            loc = torch.full((5,), 7, dtype=torch.int32, device=dev)
            got = kvq.kv_compress_store_translate(pool, layout, f0, f0, ratio, i0, cs,
                                                  torch.arange(64, dtype=torch.int32, device=dev), i0, loc)
            torch.cuda.synchronize()
            assert got.numel() == 0 and not to_host(loc).any()    # no rows: the buffer is zeroed
        state, count = kvq.new_compress_state(3)
        kvq.kv_compress_state_update(pool, layout, state, count, 4, i0, f0, f0, i0, cs, i0)
        torch.cuda.synchronize()
        assert np.array_equal(to_host(pool), ref)
        assert not to_host(state).any() and not to_host(count).any()
        assert tuple(kvq.kv_dequant(pool, layout, i0).shape) == (0, 512)
        assert tuple(kvq.kv_dequant_slots(pool, layout, i0).shape) == (0, 512)
    table = torch.arange(100, dtype=torch.int32, device=dev)
    out = torch.full((16,), 7, dtype=torch.int32, device=dev)
    got = kvq.kv_translate_slots(table, torch.empty(0, dtype=torch.int32, device=dev), out)
    torch.cuda.synchronize()
    assert got.numel() == 0 and np.all(to_host(out) == 0)
    out.fill_(7)
    assert kvq.kv_translate_slots(table, torch.arange(17, dtype=torch.int32, device=dev), out) is None
    torch.cuda.synchronize()
    assert np.all(to_host(out) == 7)                    # refused: nothing written


def test_concurrent_host_threads_on_separate_streams(kvq, cs_small):
    """Calls are thread-safe: four host threads (ctypes releases the GIL during each call)
    launch compressions and stores into their own pools on their own streams, repeatedly;
    every pool equals the result of the same calls made from one thread."""
    import threading
    import torch
    rng = np.random.default_rng(71)
    jobs = []
    for t in range(4):
        R, ratio = 300 + 37 * t, (4, 128, 2, 1)[t]
        kv = to_dev(rng.standard_normal((R * ratio, 512)).astype(np.float32))
        sc = to_dev((2 * rng.standard_normal((R * ratio, 512))).astype(np.float32))
        k = to_dev(wl.bf16_bits(rng.standard_normal((R, 512)).astype(np.float32)))
        pos = to_dev(rng.integers(0, 100, R).astype(np.int32))
        slots = to_dev(wl.distinct_slots(rng, R, 64, 40 * 64))
        slots2 = to_dev(wl.distinct_slots(rng, R, 64, 40 * 64))
        jobs.append((ratio, kv, sc, k, pos, slots, slots2))
    cs = to_dev(cs_small)

    def run(job, pool_a, pool_b, stream, reps):
        ratio, kv, sc, k, pos, slots, slots2 = job
        with torch.cuda.stream(stream):
            for _ in range(reps):
                kvq.kv_compress_store(pool_a, V41, kv, sc if ratio > 1 else None, ratio, pos, cs, slots)
                kvq.kv_store_rope(pool_b, FP4, k, pos, cs, slots2)

    want = []
    for job in jobs:
        a, b = kvq.new_pool(V41, 40), kvq.new_pool(FP4, 40)
        run(job, a, b, torch.cuda.current_stream(), 1)
        want.append((a, b))
    torch.cuda.synchronize()
    got = [(kvq.new_pool(V41, 40), kvq.new_pool(FP4, 40)) for _ in jobs]
    streams = [torch.cuda.Stream() for _ in jobs]
    torch.cuda.synchronize()
    errors = []

    def worker(i):
        try:
            run(jobs[i], got[i][0], got[i][1], streams[i], 20)
            streams[i].synchronize()
        except Exception as e:   # reported below, in the main thread
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(jobs))]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for (ga, gb), (wa, wb) in zip(got, want):
        assert torch.equal(ga, wa) and torch.equal(gb, wb)


@pytest.mark.parametrize("ratio", [4, 16, 128])
@pytest.mark.parametrize("sigma", [0.01, 10.0, 300.0])
def test_compress_score_spread(kvq, orc, ratio, sigma):
    """Score spreads far from the workload's sd 2: nearly uniform weights (0.01), sharp
    (10) and winner-take-all windows (300, where exp underflows for all but a few rows)."""
    rng = np.random.default_rng(int(80 + ratio + sigma))
    R = 64 if ratio < 128 else 24
    kv = rng.standard_normal((R * ratio, 512)).astype(np.float32)
    sc = (sigma * rng.standard_normal((R * ratio, 512))).astype(np.float32)
    cs = wl.rope_cos_sin(max_pos=4096)
    pos = rng.integers(0, 4096, R).astype(np.int32)
    slots = wl.distinct_slots(rng, R, 64, NUM_PAGES * 64)
    pool = kvq.new_pool(V41, NUM_PAGES)
    kvq.kv_compress_store(pool, V41, to_dev(kv), to_dev(sc), ratio, to_dev(pos), to_dev(cs), to_dev(slots))
    ref = orc.new_pool(V41, NUM_PAGES)
    orc.kv_compress_store(V41, ref, kv, sc, ratio, pos, cs, slots)
    compare_compressed(to_host(pool), ref, V41, slots, label=f"spread {sigma} r{ratio}")
