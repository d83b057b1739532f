"""Parity at bf16 rounding ties: windows whose exact pooled value is a bf16 midpoint, or
sits one float32 step (divided by the ratio) beside one.

With equal scores in a window every softmax weight is 1/r, so the pooled value is the mean
of the window's kv values.  r is a power of two and the values are chosen so that the mean
is exactly a bf16 midpoint m, or m + k ulp32(m) / r with k = +-1 -- all exact in float64.
The pooled bf16 is then fixed by the definition alone: the even neighbour for a tie, the
neighbour on its side otherwise.  This drives the short-window kernels' float32 fast path
into its float64 fallback on almost every channel and checks how the float64 kernels round
ties.  No tolerance applies: the values are exact, so the whole pool must equal the
oracle's, and the oracle itself is checked against the construction on the CPU.
"""
import numpy as np
import pytest

from helpers import FP4, V41, gpu_lib, to_dev, to_host
from quantized_paged_kv_compress_amd import workloads as wl


def tie_windows(rng, R, ratio):
    """kv, score fp32 [R*ratio, 512] and k [R, 512]: per channel a random bf16 b (normal
    range, random sign), its midpoint m with the next bf16 up in magnitude, and kv values
    whose mean is exactly m + k * ulp32(m) / ratio; scores are equal within each window."""
    b = rng.integers(0x3000, 0x4F00, (R, 512)).astype(np.uint32)
    b |= rng.integers(0, 2, (R, 512)).astype(np.uint32) << 15
    mid = ((b << 16) | 0x8000).view(np.float32)
    amid = np.abs(mid).astype(np.float64)
    ulp = np.spacing(np.abs(mid)).astype(np.float64)
    lower = 2.0 ** np.floor(np.log2(amid))
    room = np.minimum(amid - lower, 2 * lower - amid) - 2 * ulp     # keep every value in m's binade
    k = rng.integers(-1, 2, (R, 512))
    d = np.round(rng.uniform(-0.9, 0.9, (R, ratio // 2, 512)) * room[:, None, :] / ulp[:, None, :]) * ulp[:, None, :]
    x = np.empty((R, ratio, 512), np.float64)
    x[:, 0::2, :] = mid[:, None, :] + d
    x[:, 1::2, :] = mid[:, None, :] - d
    x[:, 0, :] += k * ulp * np.sign(mid)
    x32 = x.astype(np.float32)
    assert np.array_equal(x32.astype(np.float64), x), "every kv value is a float32"
    mean = x.sum(axis=1) / ratio
    assert np.array_equal(mean, mid + k * ulp * np.sign(mid) / ratio), "the mean is exact"
    sc = np.repeat(rng.normal(0, 2, (R, 1, 512)).astype(np.float32), ratio, axis=1)
    return (np.ascontiguousarray(x32.reshape(R * ratio, 512)), np.ascontiguousarray(sc.reshape(R * ratio, 512)),
            b.astype(np.uint16), k)


def expected_bf16(b, k):
    """k = 0: the even of b and its successor; k = 1 (farther from zero): the successor;
    k = -1: b."""
    even = np.where(b & 1, b + 1, b)
    return np.where(k == 0, even, np.where(k > 0, b + 1, b)).astype(np.uint16)


@pytest.mark.parametrize("ratio", [2, 4, 8, 128])
def test_tie_construction_and_oracle(orc, ratio):
    """The oracle's pooled bf16 is what the construction fixes."""
    rng = np.random.default_rng(5 + ratio)
    kv, sc, b, k = tie_windows(rng, 64, ratio)
    _, pooled = orc.pool_rows(kv, sc, ratio)
    assert (k == 0).any() and (k != 0).any()
    assert np.array_equal(pooled, expected_bf16(b, k))


@pytest.fixture(scope="module")
def kvq():
    return gpu_lib()


@pytest.mark.gpu
@pytest.mark.parametrize("layout", [V41, FP4])
@pytest.mark.parametrize("ratio,R", [(2, 2048), (4, 2048), (8, 1024), (16, 512), (32, 256), (64, 128),
                                     (128, 64)])
def test_pooled_ties_round_exactly(kvq, orc, layout, ratio, R):
    import torch
    rng = np.random.default_rng(900 + ratio)
    kv, sc, b, k = tie_windows(rng, R, ratio)
    cs = wl.rope_cos_sin()
    pos = rng.integers(0, 65536, R).astype(np.int32)
    num_pages = (R + 63) // 64 * 2 + 2
    slots = wl.distinct_slots(rng, R, 64, num_pages * 64)
    print(f"[ties] ratio {ratio}, R {R}, layout {layout}: {(k == 0).mean() * 100:.1f} % exact ties", flush=True)
    pool = kvq.new_pool(layout, num_pages)
    kvq.kv_compress_store(pool, layout, to_dev(kv), to_dev(sc), ratio, to_dev(pos), to_dev(cs), to_dev(slots))
    ref = orc.new_pool(layout, num_pages)
    orc.kv_compress_store(layout, ref, kv, sc, ratio, pos, cs, slots)
    torch.cuda.synchronize()
    got = to_host(pool)
    assert np.array_equal(got, ref), f"ratio {ratio}: {int((got != ref).sum())} pool bytes differ"
