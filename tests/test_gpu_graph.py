"""The entry points are capture-safe: no allocation, no synchronisation, no memset nodes.

A translate + store + compress + dequant sequence is captured once into a HIP graph (via
torch.cuda.CUDAGraph on the library's launch stream) and replayed several times, with the
program's own eager work and synchronisations in between; every replay must reproduce
the eager result byte for byte.
"""
import numpy as np
import pytest

from helpers import FP4, V41, gpu_lib, to_dev, to_host
from quantized_paged_kv_compress_amd import workloads as wl

pytestmark = pytest.mark.gpu


def test_graph_replay_matches_eager():
    import torch
    kvq = gpu_lib()
    rng = np.random.default_rng(41)
    cs = to_dev(wl.rope_cos_sin(max_pos=4096))
    n, R, num_pages = 300, 200, 16
    table = to_dev(rng.permutation(num_pages * 64).astype(np.int32))
    full = to_dev(rng.permutation(num_pages * 64)[:R].astype(np.int32))
    k = to_dev(wl.bf16_bits(rng.standard_normal((n, 512)).astype(np.float32)))
    kpos = to_dev(rng.integers(0, 4096, n).astype(np.int32))
    kslots = to_dev(wl.distinct_slots(rng, n, 0, num_pages * 64))
    kv = to_dev(rng.standard_normal((R * 4, 512)).astype(np.float32))
    sc = to_dev((2 * rng.standard_normal((R * 4, 512))).astype(np.float32))
    cpos = to_dev(rng.integers(0, 4096, R).astype(np.int32))
    pages = to_dev(np.arange(num_pages, dtype=np.int32))
    loc = torch.empty(512, dtype=torch.int32, device="cuda")
    pool_a = kvq.new_pool(V41, num_pages)
    pool_b = kvq.new_pool(FP4, num_pages)
    ws = torch.empty((num_pages * 64, 512), dtype=torch.bfloat16, device="cuda")

    def seq():
        swa = kvq.kv_translate_slots(table, full, loc)
        kvq.kv_store_rope(pool_a, V41, k, kpos, cs, kslots)
        kvq.kv_compress_store(pool_b, FP4, kv, sc, 4, cpos, cs, swa)
        kvq.kv_dequant(pool_b, FP4, pages, ws)

    seq()
    torch.cuda.synchronize()
    want = [to_host(x).copy() for x in (loc, pool_a, pool_b, ws)]

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        seq()                                     # warm the stream before capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        seq()
    for rep in range(4):
        for x in (loc, ws):
            x.fill_(0x55 if x.dtype != torch.bfloat16 else 1.0)
        pool_a.zero_()
        pool_b.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [to_host(x) for x in (loc, pool_a, pool_b, ws)]
        for name, a, b in zip(("translate", "store_rope", "compress", "dequant"), got, want):
            assert np.array_equal(a, b), (rep, name)


def test_graph_replay_of_norm_gather_and_decode_state():
    """The remaining entry points in one graph: K-norm store, token-gather dequant and the
    decode-step compressor state.  Each replay is one decode step whose new rows are copied
    into the captured input buffers first; after every replay the pools, state, counts and
    gathered rows must equal the same steps run eagerly."""
    import torch
    kvq = gpu_lib()
    rng = np.random.default_rng(42)
    cs = to_dev(wl.rope_cos_sin(max_pos=4096))
    S, ratio, num_pages, steps = 48, 4, 8, 6
    w = to_dev(wl.bf16_bits(rng.uniform(0.5, 1.5, 512).astype(np.float32)))
    step_kv = [rng.standard_normal((S, 512)).astype(np.float32) for _ in range(steps)]
    step_sc = [(2 * rng.standard_normal((S, 512))).astype(np.float32) for _ in range(steps)]
    step_k = [wl.bf16_bits(rng.standard_normal((S, 512)).astype(np.float32)) for _ in range(steps)]
    ids = to_dev(rng.permutation(S).astype(np.int32))
    pos = to_dev(rng.integers(0, 4096, S).astype(np.int32))
    slots_c = to_dev(wl.distinct_slots(rng, S, 64, num_pages * 64))
    slots_k = to_dev(wl.distinct_slots(rng, S, 64, num_pages * 64))

    def make():
        st, cnt = kvq.new_compress_state(S)
        return dict(pool_c=kvq.new_pool(V41, num_pages), pool_k=kvq.new_pool(FP4, num_pages),
                    state=st, count=cnt,
                    gathered=torch.zeros((S, 512), dtype=torch.bfloat16, device="cuda"),
                    kv=torch.empty((S, 512), dtype=torch.float32, device="cuda"),
                    sc=torch.empty((S, 512), dtype=torch.float32, device="cuda"),
                    k=torch.empty((S, 512), dtype=torch.int16, device="cuda"))

    def seq(b):
        kvq.kv_store_norm_rope(b["pool_k"], FP4, b["k"], w, 1e-6, pos, cs, slots_k)
        kvq.kv_compress_state_update(b["pool_c"], V41, b["state"], b["count"], ratio, ids, b["kv"], b["sc"],
                                     pos, cs, slots_c)
        kvq.kv_dequant_slots(b["pool_c"], V41, slots_c, b["gathered"])

    def feed(b, t):
        b["kv"].copy_(torch.from_numpy(step_kv[t]))
        b["sc"].copy_(torch.from_numpy(step_sc[t]))
        b["k"].copy_(torch.from_numpy(step_k[t].view(np.int16)))

    eager, graphed = make(), make()
    # capture on a side stream after a warm-up call on a scratch set of buffers
    warm = make()
    feed(warm, 0)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        seq(warm)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        seq(graphed)
    keys = ("pool_k", "pool_c", "state", "count", "gathered")
    for t in range(steps):
        feed(eager, t)
        seq(eager)
        feed(graphed, t)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for key in keys:
            assert np.array_equal(to_host(graphed[key]), to_host(eager[key])), (t, key)
    assert np.all(to_host(eager["count"]) == steps % ratio)
