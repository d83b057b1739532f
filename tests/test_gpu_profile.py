"""kvq_profile_next_launch: the armed launch records its own start/stop events, results
are unchanged, and the request is consumed by that one launch."""
import numpy as np
import pytest

from helpers import V41, gpu_lib, to_dev, to_host
from quantized_paged_kv_compress_amd import workloads as wl

pytestmark = pytest.mark.gpu


def test_profiled_launch_times_the_kernel_and_changes_nothing():
    import torch
    kvq = gpu_lib()
    rng = np.random.default_rng(91)
    R, ratio, num_pages = 2048, 4, 64
    cs = to_dev(wl.rope_cos_sin(max_pos=4096))
    kv = to_dev(rng.standard_normal((R * ratio, 512)).astype(np.float32))
    sc = to_dev((2 * rng.standard_normal((R * ratio, 512))).astype(np.float32))
    pos = to_dev(rng.integers(0, 4096, R).astype(np.int32))
    slots = to_dev(wl.distinct_slots(rng, R, 0, num_pages * 64))
    plain = kvq.new_pool(V41, num_pages)
    kvq.kv_compress_store(plain, V41, kv, sc, ratio, pos, cs, slots)

    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    for e in ev:
        e.record()
    torch.cuda.synchronize()
    with pytest.raises(ValueError):
        kvq.profile_next_launch(torch.cuda.Event(enable_timing=True), ev[1])   # never recorded

    profiled = kvq.new_pool(V41, num_pages)
    torch.cuda.synchronize()
    ev[0].record()                                  # stream event before the launch
    kvq.profile_next_launch(ev[1], ev[2])
    kvq.kv_compress_store(profiled, V41, kv, sc, ratio, pos, cs, slots)
    ev[3].record()                                  # stream event after it
    torch.cuda.synchronize()
    assert np.array_equal(to_host(profiled), to_host(plain))
    kernel_ms = ev[1].elapsed_time(ev[2])
    assert kernel_ms > 0
    assert ev[0].elapsed_time(ev[1]) >= 0 and ev[2].elapsed_time(ev[3]) >= 0
    assert kernel_ms <= ev[0].elapsed_time(ev[3])

    # consumed: a later unarmed launch leaves the events where they were
    stop_before = ev[0].elapsed_time(ev[2])
    kvq.kv_compress_store(profiled, V41, kv, sc, ratio, pos, cs, slots)
    torch.cuda.synchronize()
    assert ev[0].elapsed_time(ev[2]) == stop_before
