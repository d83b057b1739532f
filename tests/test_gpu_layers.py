"""The multi-layer hoisted store (kv_store_rope_layers) against the oracle, layer by layer.

The step of the SWA hoisting page: translate the step's full-pool slots once, then store
every layer's K rows at the translated slots of that layer's pool.  Each layer's pool must
equal the oracle's kv_store_rope of that layer's rows at the same slots, byte for byte.
"""
import numpy as np
import pytest

from helpers import FP4, V41, gpu_lib, to_dev, to_host
from quantized_paged_kv_compress_amd import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kvq():
    return gpu_lib()


def layer_inputs(rng, L, n, ld=512):
    return [wl.bf16_bits((rng.standard_normal((n, ld)) * np.exp(rng.uniform(-3, 3, (1, ld)))).astype(np.float32))
            for _ in range(L)]


def check_layers(kvq, orc, layout, pools, ks_host, pos, cs, slots):
    import torch
    torch.cuda.synchronize()
    num_pages = pools[0].shape[0]
    for l, (pool, k) in enumerate(zip(pools, ks_host)):
        ref = orc.new_pool(layout, num_pages)
        orc.kv_store_rope(layout, ref, np.ascontiguousarray(k[:, :512]), pos, cs, slots)
        got = to_host(pool)
        assert np.array_equal(got, ref), f"layer {l}: {int((got != ref).sum())} bytes differ"


@pytest.mark.parametrize("layout", [V41, FP4])
def test_hoisted_step_61_layers(kvq, orc, layout):
    """61 layers x 512 tokens: translate once, one store call for every layer."""
    import torch
    rng = np.random.default_rng(61)
    L, n, num_pages = 61, 512, 16
    cs = wl.rope_cos_sin()
    pos = rng.integers(0, 65536, n).astype(np.int32)
    table = (rng.permutation(num_pages * 64 - 64) + 64).astype(np.int32)    # full slot -> SWA slot
    full = rng.permutation(table.size)[:n].astype(np.int32)
    ks = layer_inputs(rng, L, n)
    loc = torch.empty(1024, dtype=torch.int32, device="cuda")
    swa = kvq.kv_translate_slots(to_dev(table), to_dev(full), loc)
    pools = [kvq.new_pool(layout, num_pages) for _ in range(L)]
    kvq.kv_store_rope_layers(pools, layout, [to_dev(k) for k in ks], to_dev(pos), to_dev(cs), swa)
    print(f"[layers] {L} layers x {n} tokens, layout {layout}", flush=True)
    check_layers(kvq, orc, layout, pools, ks, pos, cs, table[full])


@pytest.mark.parametrize("L,n", [(1, 1), (2, 77), (3, 9), (4, 64), (7, 3), (64, 33), (65, 130), (130, 5)])
def test_layer_counts_strides_and_skipped_rows(kvq, orc, L, n):
    """Layer counts across the 64-per-launch boundary and the 4-layer groups of a
    wavefront, ragged rows, a row stride above 512, and rows skipped for out-of-pool slots
    and out-of-range positions."""
    rng = np.random.default_rng(1000 + L * 7 + n)
    num_pages, ld, max_pos = 4, 640, 3000
    cs = np.ascontiguousarray(wl.rope_cos_sin()[:max_pos])
    pos = rng.integers(0, max_pos, n).astype(np.int32)
    slots = wl.distinct_slots(rng, n, 0, num_pages * 64 + 40)
    if n > 4:
        pos[1], pos[2] = -1, max_pos
        slots[3] = -5
    ks = layer_inputs(rng, L, n, ld)
    pools = [kvq.new_pool(V41, num_pages) for _ in range(L)]
    for p in pools:
        p.fill_(0x5A)
    kd = [to_dev(k) for k in ks]
    kvq.kv_store_rope_layers(pools, V41, [k[:, :512] for k in kd], to_dev(pos), to_dev(cs), to_dev(slots))
    import torch
    torch.cuda.synchronize()
    for l, (pool, k) in enumerate(zip(pools, ks)):
        ref = np.full((num_pages, kvq.page_bytes(V41)), 0x5A, np.uint8)
        orc.kv_store_rope(V41, ref, np.ascontiguousarray(k[:, :512]), pos, cs, slots)
        assert np.array_equal(to_host(pool), ref), f"layer {l}"


def test_hoisted_step_graph_replay(kvq, orc):
    """translate + the multi-layer store captured in one HIP graph; each replay, with new K
    rows copied in eagerly beforehand, equals the oracle on every layer."""
    import torch
    rng = np.random.default_rng(62)
    L, n, num_pages = 12, 200, 8
    cs = wl.rope_cos_sin()
    cs_d = to_dev(cs)
    pos = rng.integers(0, 65536, n).astype(np.int32)
    table = (rng.permutation(num_pages * 64 - 64) + 64).astype(np.int32)
    full = rng.permutation(table.size)[:n].astype(np.int32)
    table_d, full_d, pos_d = to_dev(table), to_dev(full), to_dev(pos)
    loc = torch.empty(256, dtype=torch.int32, device="cuda")
    kd = [torch.empty((n, 512), dtype=torch.int16, device="cuda") for _ in range(L)]
    pools = [kvq.new_pool(FP4, num_pages) for _ in range(L)]

    def step():
        swa = kvq.kv_translate_slots(table_d, full_d, loc)
        kvq.kv_store_rope_layers(pools, FP4, kd, pos_d, cs_d, swa)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        ks = layer_inputs(rng, L, n)
        for d, h in zip(kd, ks):
            d.copy_(to_dev(h))
        for p in pools:
            p.zero_()
        loc.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        check_layers(kvq, orc, FP4, pools, ks, pos, cs, table[full])
        assert np.array_equal(to_host(loc)[:n], table[full]), rep
