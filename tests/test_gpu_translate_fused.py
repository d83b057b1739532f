"""kv_compress_store_translate (the step's full -> SWA translation fused into the
compressor) against the oracle's translate followed by its compressor, through the C ABI.

Every case checks the whole translated buffer (and that nothing past it is written), the
whole pool (canary-filled, so untouched bytes are checked too) and covers: full slots
outside the table, table entries outside the pool, invalid positions, tails of every
length (including the long tails that the library hands to the separate translation
kernel), R == 0, the capacity refusal, the benchmark's mixed step, and graph replay.
"""
import numpy as np
import pytest

from helpers import (FP4, V41, check_step_dequant, compare_compressed, gpu_lib, to_dev, to_host,
                     untouched_equal)
from quantized_paged_kv_compress_amd import workloads as wl

pytestmark = pytest.mark.gpu
CANARY = 0x5A5A5A5A


@pytest.fixture(scope="module")
def kvq():
    return gpu_lib()


@pytest.fixture(scope="module")
def cos_sin():
    return wl.rope_cos_sin()


@pytest.fixture(scope="module")
def cos_sin_dev(kvq, cos_sin):
    return to_dev(cos_sin)


def log(msg):
    print(msg, flush=True)


def case(seed, R, ratio, num_pages):
    """Inputs of one call: a table that maps every full slot of [0, table_len) to a
    distinct SWA slot (a few negative or past the pool), distinct full slots with a few
    outside the table, and one invalid position."""
    rng = np.random.default_rng(seed)
    nslots = num_pages * 64
    table_len = max(4 * R, 256)
    table = rng.permutation(max(nslots, table_len))[:table_len].astype(np.int32)  # distinct SWA slots
    table[rng.choice(table_len, 4, replace=False)] = [-1, -5, nslots, nslots + 7]   # outside the pool
    full = rng.permutation(table_len + 64)[:R].astype(np.int32) - 32                # some outside the table
    kv = rng.standard_normal((R * ratio, 512)).astype(np.float32)
    sc = (2 * rng.standard_normal((R * ratio, 512))).astype(np.float32)
    pos = rng.integers(0, 65536, R).astype(np.int32)
    if R > 2:
        pos[2] = 65536
    return table, full, kv, sc, pos


def run_fused(kvq, layout, num_pages, table, full, kv, sc, pos, ratio, cap, cos_sin_dev):
    import torch
    pool = kvq.new_pool(layout, num_pages)
    pool.fill_(0xA5)
    buf = torch.full((cap + 64,), CANARY, dtype=torch.int32, device="cuda")
    res = kvq.kv_compress_store_translate(pool, layout, to_dev(kv), to_dev(sc), ratio, to_dev(pos),
                                          cos_sin_dev, to_dev(table), to_dev(full), buf[:cap])
    torch.cuda.synchronize()
    return res, to_host(pool), to_host(buf)


def oracle_ref(orc, layout, num_pages, table, full, kv, sc, pos, ratio, cap, cos_sin):
    rc, loc = orc.translate_slots(table, full, cap)
    assert rc == 0
    ref = np.full((num_pages, orc.page_bytes(layout)), 0xA5, np.uint8)
    slots = np.ascontiguousarray(loc[:full.size])
    orc.kv_compress_store(layout, ref, kv, sc, ratio, pos, cos_sin, slots)
    stored = (slots >= 0) & (slots < num_pages * 64) & (pos >= 0) & (pos < cos_sin.shape[0])
    return loc, ref, slots[stored]


@pytest.mark.parametrize("layout", [V41, FP4])
@pytest.mark.parametrize("ratio,R,extra", [(1, 300, 700), (2, 301, 0), (4, 1001, 5000), (4, 3, 61),
                                           (8, 130, 1), (8, 5, 3000), (16, 77, 2000), (32, 99, 64),
                                           (64, 45, 3000), (128, 37, 600), (128, 3, 2000), (128, 1, 5)])
def test_fused_equals_translate_then_compress(kvq, orc, cos_sin, cos_sin_dev, layout, ratio, R, extra):
    num_pages = max(4, (R + 63) // 64 * 2)
    cap = R + extra
    table, full, kv, sc, pos = case(100 * ratio + R, R, ratio, num_pages)
    log(f"[fused] ratio {ratio}, R {R}, cap {cap}, layout {layout}")
    res, got, buf = run_fused(kvq, layout, num_pages, table, full, kv, sc, pos, ratio, cap, cos_sin_dev)
    loc, ref, slots = oracle_ref(orc, layout, num_pages, table, full, kv, sc, pos, ratio, cap, cos_sin)
    assert res is not None and res.numel() == R
    assert np.array_equal(buf[:cap], loc) and np.all(buf[cap:] == CANARY)
    compare_compressed(got, ref, layout, slots, label=f"fused r{ratio} R{R} L{layout}")
    assert untouched_equal(got, ref, layout, slots)


@pytest.mark.parametrize("ratio,R", [(4, 3), (128, 2), (1, 1), (32, 5)])
def test_fused_long_tail(kvq, orc, cos_sin, cos_sin_dev, ratio, R):
    """A tail far longer than the grid: the library translates in a launch of its own."""
    num_pages, cap = 4, 70000
    table, full, kv, sc, pos = case(7 + ratio, R, ratio, num_pages)
    res, got, buf = run_fused(kvq, V41, num_pages, table, full, kv, sc, pos, ratio, cap, cos_sin_dev)
    loc, ref, slots = oracle_ref(orc, V41, num_pages, table, full, kv, sc, pos, ratio, cap, cos_sin)
    assert res is not None
    assert np.array_equal(buf[:cap], loc) and np.all(buf[cap:] == CANARY)
    compare_compressed(got, ref, V41, slots, label=f"fused long tail r{ratio}")
    assert untouched_equal(got, ref, V41, slots)


def test_fused_no_rows_zeroes_the_buffer(kvq, cos_sin_dev):
    import torch
    pool = kvq.new_pool(V41, 4)
    buf = torch.full((300,), CANARY, dtype=torch.int32, device="cuda")
    empty_f = torch.empty((0, 512), dtype=torch.float32, device="cuda")
    none = torch.empty(0, dtype=torch.int32, device="cuda")
    table = to_dev(np.arange(64, dtype=np.int32))
    res = kvq.kv_compress_store_translate(pool, V41, empty_f, empty_f, 4, none, cos_sin_dev, table, none,
                                          buf[:200])
    torch.cuda.synchronize()
    got = to_host(buf)
    assert res is not None and res.numel() == 0
    assert np.all(got[:200] == 0) and np.all(got[200:] == CANARY)
    assert not to_host(pool).any()


def test_fused_capacity_refusal_writes_nothing(kvq, cos_sin_dev):
    import torch
    R, ratio, num_pages = 20, 4, 4
    table, full, kv, sc, pos = case(3, R, ratio, num_pages)
    pool = kvq.new_pool(V41, num_pages)
    buf = torch.full((19,), CANARY, dtype=torch.int32, device="cuda")
    res = kvq.kv_compress_store_translate(pool, V41, to_dev(kv), to_dev(sc), ratio, to_dev(pos), cos_sin_dev,
                                          to_dev(table), to_dev(full), buf)
    torch.cuda.synchronize()
    assert res is None
    assert np.all(to_host(buf) == CANARY) and not to_host(pool).any()


def test_fused_mixed_fp4_step(kvq, orc, cos_sin, cos_sin_dev):
    """The benchmark's mixed step with the translation fused into the compressor, then the
    dequant of the touched pages."""
    import torch
    d = wl.mixed_fp4(seed=5)
    R = d["R"]
    log(f"[fused mixed] R {R}, cap {d['cap']}, pages {d['page_ids'].size}")
    pool = kvq.new_pool(FP4, d["num_pages"])
    buf = torch.full((d["cap"] + 64,), CANARY, dtype=torch.int32, device="cuda")
    kvq.kv_compress_store_translate(pool, FP4, to_dev(d["kv"]), to_dev(d["score"]), 4, to_dev(d["pos"]),
                                    cos_sin_dev, to_dev(d["table"]), to_dev(d["full"]), buf[:d["cap"]])
    ws = kvq.kv_dequant(pool, FP4, to_dev(d["page_ids"]))
    got_pool, got_buf = to_host(pool), to_host(buf)
    rc, loc = orc.translate_slots(d["table"], d["full"], d["cap"])
    assert rc == 0 and np.array_equal(got_buf[:d["cap"]], loc) and np.all(got_buf[d["cap"]:] == CANARY)
    slots = np.ascontiguousarray(loc[:R])
    ref_pool = orc.new_pool(FP4, d["num_pages"])
    orc.kv_compress_store(FP4, ref_pool, d["kv"], d["score"], 4, d["pos"], cos_sin, slots)
    compare_compressed(got_pool, ref_pool, FP4, slots, label="fused mixed fp4")
    assert untouched_equal(got_pool, ref_pool, FP4, slots)
    check_step_dequant(orc, FP4, to_host(ws), got_pool, ref_pool, d["page_ids"])


def test_fused_graph_replay_matches_eager(kvq, cos_sin_dev):
    import torch
    R, ratio, num_pages, cap = 500, 4, 16, 4096
    table, full, kv, sc, pos = case(77, R, ratio, num_pages)
    args = [to_dev(x) for x in (kv, sc, pos, table, full)]
    pool = kvq.new_pool(FP4, num_pages)
    buf = torch.empty(cap, dtype=torch.int32, device="cuda")
    pages = to_dev(np.arange(num_pages, dtype=np.int32))
    ws = torch.empty((num_pages * 64, 512), dtype=torch.bfloat16, device="cuda")

    def seq():
        kvq.kv_compress_store_translate(pool, FP4, args[0], args[1], ratio, args[2], cos_sin_dev, args[3],
                                        args[4], buf)
        kvq.kv_dequant(pool, FP4, pages, ws)

    seq()
    torch.cuda.synchronize()
    want = [to_host(x).copy() for x in (buf, pool, ws)]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        seq()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        seq()
    for rep in range(4):
        buf.fill_(CANARY)
        pool.zero_()
        ws.fill_(1.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for w, x in zip(want, (buf, pool, ws)):
            assert np.array_equal(to_host(x), w), rep
