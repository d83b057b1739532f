"""GPU parity: libkvq.so (through its C ABI) against the CPU oracle on seeded inputs.

Small cases span several workgroups and a ragged tail and are compared on the whole
pool; the full-size workloads run in the same launch configuration as the benchmark and
are compared on every row, with the oracle run chunk by chunk as the inputs are generated.
"""
import numpy as np
import pytest

from helpers import (FP4, V41, check_step_dequant, compare_compressed, gpu_lib, rows_of, to_dev, to_host,
                     untouched_equal)
from quantized_paged_kv_compress_amd import workloads as wl

pytestmark = pytest.mark.gpu
LAYOUTS = [V41, FP4]


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


def canary_pool(kvq, layout, num_pages):
    import torch
    pool = kvq.new_pool(layout, num_pages)
    pool.fill_(0xA5)
    host = np.full((num_pages, kvq.page_bytes(layout)), 0xA5, np.uint8)
    torch.cuda.synchronize()
    return pool, host


# ------------------------------------------------------------------ plain store
@pytest.mark.parametrize("layout", LAYOUTS)
def test_store_v41_workload_bit_exact(kvq, orc, layout):
    d = wl.store_v41(seed=1)
    log(f"[store] 64 rows, layout {layout}")
    pool, ref = canary_pool(kvq, layout, d["num_pages"])
    kvq.kv_store(pool, layout, to_dev(d["k"]), to_dev(d["slots"]))
    orc.kv_store(layout, ref, d["k"], d["slots"])
    assert np.array_equal(to_host(pool), ref)


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("n", [1, 3, 5, 63, 257, 1001])
def test_store_ragged_sizes_bit_exact(kvq, orc, layout, n):
    rng = np.random.default_rng(100 + n)
    num_pages = 40
    k = wl.bf16_bits(rng.standard_normal((n, 512)).astype(np.float32)
                     * np.exp(rng.uniform(-8, 8, (1, 512))).astype(np.float32))
    slots = wl.distinct_slots(rng, n, 0, num_pages * 64)
    pool, ref = canary_pool(kvq, layout, num_pages)
    kvq.kv_store(pool, layout, to_dev(k), to_dev(slots))
    orc.kv_store(layout, ref, k, slots)
    assert np.array_equal(to_host(pool), ref)


@pytest.mark.parametrize("layout", LAYOUTS)
def test_store_strided_rows_and_invalid_slots(kvq, orc, layout):
    import torch
    rng = np.random.default_rng(5)
    n, ld, num_pages = 300, 640, 8
    kfull = wl.bf16_bits(rng.standard_normal((n, ld)).astype(np.float32))
    slots = wl.distinct_slots(rng, n, 0, num_pages * 64 + 100)   # some beyond the pool
    slots[::17] = -1
    slots[5] = np.iinfo(np.int32).min
    slots[6] = np.iinfo(np.int32).max
    pool, ref = canary_pool(kvq, layout, num_pages)
    kd = to_dev(kfull)
    kvq.kv_store(pool, layout, kd[:, :512], to_dev(slots))   # stride 640 elements
    orc.kv_store(layout, ref, np.ascontiguousarray(kfull[:, :512]), slots)
    assert np.array_equal(to_host(pool), ref)
    # n == 0 is a no-op
    before = to_host(pool).copy()
    kvq.kv_store(pool, layout, kd[:0, :512], torch.zeros(0, dtype=torch.int32, device="cuda"))
    assert np.array_equal(to_host(pool), before)


def exhaustive_rows(orc_mod, layout):
    """Rows whose blocks put every finite bf16 value (V41) or every bf16 magnitude in
    [s/16, 6s] for every positive e4m3 scale s (FP4) next to a block maximum that fixes
    the scale; same construction as the oracle's own exhaustive pins."""
    b = np.arange(65536, dtype=np.uint32)
    v = (b << 16).view(np.float32)
    v = v[np.isfinite(v)]
    blocks = []
    if layout == V41:
        for amax in (448.0, 1.0, 3.0, 2.0 ** -100, 1.5 * 2.0 ** 100, 2.0 ** -126):
            vals = v[np.abs(v) <= amax]
            for s in range(0, vals.size, 31):
                blocks.append(np.concatenate([[np.float32(amax)], vals[s:s + 31]]))
    else:
        vpos = v[v > 0]
        for sc in range(1, 0x7F):
            s = np.float32(orc_mod.e4m3_decode(sc))
            xs = vpos[(vpos >= s / 16) & (vpos <= 6 * s)]
            xs = np.concatenate([xs, -xs, [0.0, -0.0]]).astype(np.float32)
            for q in range(0, xs.size, 31):
                blocks.append(np.concatenate([[6 * s], xs[q:q + 31]]))
    while len(blocks) % 16:
        blocks.append(np.zeros(1, np.float32))
    rows = np.zeros((len(blocks) // 16, 512), np.float32)
    for i, blk in enumerate(blocks):
        r, q = divmod(i, 16)
        rows[r, q * 32:q * 32 + blk.size] = blk
    bits = rows.view(np.uint32)
    assert np.all((bits & 0xFFFF) == 0)
    return (bits >> 16).astype(np.uint16)


@pytest.mark.parametrize("layout", LAYOUTS)
def test_store_exhaustive_encoder_bit_exact(kvq, orc, layout):
    k = exhaustive_rows(orc, layout)
    n = k.shape[0]
    num_pages = (n + 63) // 64
    log(f"[store exhaustive] layout {layout}: {n} rows")
    slots = np.arange(n, dtype=np.int32)
    pool = kvq.new_pool(layout, num_pages)
    ref = orc.new_pool(layout, num_pages)
    kvq.kv_store(pool, layout, to_dev(k), to_dev(slots))
    orc.kv_store(layout, ref, k, slots)
    got = to_host(pool)
    if not np.array_equal(got, ref):
        gc, gs = rows_of(got, layout, slots)
        rc, rs = rows_of(ref, layout, slots)
        bad = np.nonzero((gc != rc).any(1) | (gs != rs).any(1))[0]
        r = bad[0]
        raise AssertionError(f"{bad.size} rows differ; first row {r}: "
                             f"scales {gs[r][:16]} vs {rs[r][:16]}")


def every_amax_rows(seed):
    """One 32-value block per positive finite bf16 amax (0x0001..0x7F7F, 32,639 values) and
    one all-zero block: the block maximum sits on a rotating channel, with either sign;
    the other 31 values are bf16 roundings of random fractions of it (random signs), so
    every block exercises the scale encoder at its amax and the code encoder at that
    scale.  16 blocks per row."""
    rng = np.random.default_rng(seed)
    amax = np.concatenate([np.arange(1, 0x7F80, dtype=np.uint32), [0]]).astype(np.uint32)
    nb = amax.size
    av = (amax << 16).view(np.float32)
    frac = rng.uniform(0, 1, (nb, 32)).astype(np.float32)
    vals = wl.bf16_bits(frac * av[:, None] * np.where(rng.integers(0, 2, (nb, 32)) == 1, 1, -1))
    vbits = (vals.astype(np.uint32) << 16).view(np.float32)
    vals[np.abs(vbits) > av[:, None]] = 0          # rounding up past amax: drop to zero
    at = np.arange(nb) % 32
    sign = np.where(rng.integers(0, 2, nb) == 1, 0x8000, 0).astype(np.uint32)
    vals[np.arange(nb), at] = (amax | sign).astype(np.uint16)
    pad = (-nb) % 16
    vals = np.concatenate([vals, np.zeros((pad, 32), np.uint16)])
    return np.ascontiguousarray(vals.reshape(-1, 512)), nb


@pytest.mark.parametrize("layout", LAYOUTS)
def test_store_every_bf16_amax_bit_exact(kvq, orc, layout):
    """The scale byte (ue8m0 from the amax bits for V41, e4m3 RNE of fl32(amax / 6) for
    V41_FP4) at every positive bf16 amax, and the codes at that scale, bit-exact."""
    k, nb = every_amax_rows(31 + layout)
    bits = (k.astype(np.uint32) << 16).view(np.float32).reshape(-1, 32)
    got_amax = np.abs(bits).max(axis=1).view(np.uint32) >> 16
    assert set(range(1, 0x7F80)) <= set(got_amax.tolist())
    n = k.shape[0]
    num_pages = (n + 63) // 64
    log(f"[every amax] layout {layout}: {nb} blocks in {n} rows")
    slots = np.arange(n, dtype=np.int32)
    pool = kvq.new_pool(layout, num_pages)
    ref = orc.new_pool(layout, num_pages)
    kvq.kv_store(pool, layout, to_dev(k), to_dev(slots))
    orc.kv_store(layout, ref, k, slots)
    got = to_host(pool)
    gc, gs = rows_of(got, layout, slots)
    rc, rs = rows_of(ref, layout, slots)
    bad = np.argwhere(gs[:, :16] != rs[:, :16])
    assert bad.size == 0, (f"{len(bad)} scale bytes differ; first row {bad[0][0]} block {bad[0][1]}: "
                           f"{gs[bad[0][0], bad[0][1]]} vs {rs[bad[0][0], bad[0][1]]}")
    assert np.array_equal(got, ref)


# ------------------------------------------------------------------ store + RoPE
@pytest.mark.parametrize("layout", LAYOUTS)
def test_store_rope_workload_bit_exact(kvq, orc, cos_sin, cos_sin_dev, layout):
    d = wl.store_rope(seed=2)
    log(f"[store_rope] 512 rows, layout {layout}")
    pool, ref = canary_pool(kvq, layout, d["num_pages"])
    kvq.kv_store_rope(pool, layout, to_dev(d["k"]), to_dev(d["pos"]), cos_sin_dev, to_dev(d["slots"]))
    orc.kv_store_rope(layout, ref, d["k"], d["pos"], cos_sin, d["slots"])
    assert np.array_equal(to_host(pool), ref)


@pytest.mark.parametrize("layout", LAYOUTS)
def test_store_rope_edges(kvq, orc, cos_sin, cos_sin_dev, layout):
    """Position 0 equals the plain store; positions outside [0, max_pos) skip the row;
    a short table (max_pos) is honoured; ragged n."""
    rng = np.random.default_rng(9)
    n, num_pages = 77, 4
    k = wl.bf16_bits(rng.standard_normal((n, 512)).astype(np.float32))
    slots = wl.distinct_slots(rng, n, 0, num_pages * 64)
    pos0 = np.zeros(n, np.int32)
    a = kvq.new_pool(layout, num_pages)
    b = kvq.new_pool(layout, num_pages)
    kvq.kv_store_rope(a, layout, to_dev(k), to_dev(pos0), cos_sin_dev, to_dev(slots))
    kvq.kv_store(b, layout, to_dev(k), to_dev(slots))
    assert np.array_equal(to_host(a), to_host(b))
    pos = rng.integers(0, 1000, n).astype(np.int32)
    pos[[0, 10, 20]] = [1000, -1, 5000]
    short = np.ascontiguousarray(cos_sin[:1000])
    pool, ref = canary_pool(kvq, layout, num_pages)
    kvq.kv_store_rope(pool, layout, to_dev(k), to_dev(pos), to_dev(short), to_dev(slots))
    orc.kv_store_rope(layout, ref, k, pos, short, slots)
    assert np.array_equal(to_host(pool), ref)


# ------------------------------------------------------------------ K norm + RoPE
@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("n,eps", [(1, 1e-6), (130, 1e-6), (512, 0.0), (1001, 0.25), (65536, 1e-6)])
def test_store_norm_rope_within_tolerance(kvq, orc, cos_sin, cos_sin_dev, layout, n, eps):
    import torch
    rng = np.random.default_rng(200 + n)
    num_pages = max(8, (n + 63) // 64 * 2)
    k = wl.bf16_bits((rng.standard_normal((n, 512)) * np.exp(rng.uniform(-4, 4, (n, 1)))).astype(np.float32))
    w = wl.bf16_bits(rng.uniform(0.25, 2.0, 512).astype(np.float32))
    pos = rng.integers(0, 65536, n).astype(np.int32)
    slots = wl.distinct_slots(rng, n, 64, num_pages * 64)
    pool, ref = canary_pool(kvq, layout, num_pages)
    kvq.kv_store_norm_rope(pool, layout, to_dev(k), to_dev(w), eps, to_dev(pos), cos_sin_dev, to_dev(slots))
    orc.kv_store_norm_rope(layout, ref, k, w, eps, pos, cos_sin, slots)
    got = to_host(pool)
    compare_compressed(got, ref, layout, slots, label=f"norm n{n} L{layout}")
    assert untouched_equal(got, ref, layout, slots)


# ------------------------------------------------------------------ compressors
def run_compress(kvq, orc, layout, ratio, kv, sc, pos, slots, num_pages, cos_sin, cos_sin_dev):
    pool = kvq.new_pool(layout, num_pages)
    kvq.kv_compress_store(pool, layout, to_dev(kv), to_dev(sc) if ratio > 1 else None, ratio,
                          to_dev(pos), cos_sin_dev, to_dev(slots))
    got = to_host(pool)
    ref = orc.new_pool(layout, num_pages)
    orc.kv_compress_store(layout, ref, kv, sc, ratio, pos, cos_sin, slots)
    return got, ref


@pytest.mark.parametrize("layout", LAYOUTS)
def test_compress_ratio1_is_bit_exact(kvq, orc, cos_sin, cos_sin_dev, layout):
    """c1: pooling a one-row window is the identity, so the whole pool is bit-exact."""
    rng = np.random.default_rng(11)
    R, num_pages = 1003, 20
    kv = rng.standard_normal((R, 512)).astype(np.float32)
    sc = (2 * rng.standard_normal((R, 512))).astype(np.float32)
    pos = rng.integers(0, 65536, R).astype(np.int32)
    slots = wl.distinct_slots(rng, R, 64, num_pages * 64)
    got, ref = run_compress(kvq, orc, layout, 1, kv, sc, pos, slots, num_pages, cos_sin, cos_sin_dev)
    assert np.array_equal(got, ref)
    # and equals store+RoPE of bf16(kv)
    pool = kvq.new_pool(layout, num_pages)
    kvq.kv_store_rope(pool, layout, to_dev(wl.bf16_bits(kv)), to_dev(pos), cos_sin_dev, to_dev(slots))
    assert np.array_equal(to_host(pool), got)


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("ratio,R", [(2, 515), (4, 1001), (4, 3), (8, 301), (16, 150), (32, 99),
                                     (64, 45), (128, 37), (128, 1)])
def test_compress_small_within_tolerance(kvq, orc, cos_sin, cos_sin_dev, layout, ratio, R):
    rng = np.random.default_rng(1000 * ratio + R)
    num_pages = max(4, (R + 63) // 64 * 2)
    kv = rng.standard_normal((R * ratio, 512)).astype(np.float32)
    sc = (2 * rng.standard_normal((R * ratio, 512))).astype(np.float32)
    pos = rng.integers(0, 65536, R).astype(np.int32)
    slots = wl.distinct_slots(rng, R, 64, num_pages * 64)
    log(f"[compress] ratio {ratio}, R {R}, layout {layout}")
    got, ref = run_compress(kvq, orc, layout, ratio, kv, sc, pos, slots, num_pages, cos_sin, cos_sin_dev)
    compare_compressed(got, ref, layout, slots, label=f"r{ratio} R{R} L{layout}")
    assert untouched_equal(got, ref, layout, slots)


@pytest.mark.parametrize("layout", LAYOUTS)
def test_compress_skips_invalid_rows_and_honours_stride(kvq, orc, cos_sin, cos_sin_dev, layout):
    import torch
    rng = np.random.default_rng(12)
    R, ratio, ld, num_pages = 200, 4, 520, 6
    kvw = rng.standard_normal((R * ratio, ld)).astype(np.float32)
    scw = (2 * rng.standard_normal((R * ratio, ld))).astype(np.float32)
    pos = rng.integers(0, 4000, R).astype(np.int32)
    pos[[1, 2]] = [-7, 4000]
    slots = wl.distinct_slots(rng, R, 0, num_pages * 64 + 50)
    slots[3] = -1
    short = np.ascontiguousarray(cos_sin[:4000])
    pool = kvq.new_pool(layout, num_pages)
    pool.fill_(0x3C)
    kd, sd = to_dev(kvw), to_dev(scw)
    kvq.kv_compress_store(pool, layout, kd[:, :512], sd[:, :512], ratio, to_dev(pos),
                          to_dev(short), to_dev(slots))
    got = to_host(pool)
    ref = np.full_like(got, 0x3C)
    kv, sc = np.ascontiguousarray(kvw[:, :512]), np.ascontiguousarray(scw[:, :512])
    orc.kv_compress_store(layout, ref, kv, sc, ratio, pos, short, slots)
    valid = (slots >= 0) & (slots < num_pages * 64) & (pos >= 0) & (pos < 4000)
    compare_compressed(got, ref, layout, slots[valid], label="stride/skip")
    assert untouched_equal(got, ref, layout, slots[valid])
    torch.cuda.synchronize()


def full_compressor_check(kvq, orc, layout, ratio, R, seed, cos_sin, cos_sin_dev, num_pages=4096):
    """Full-size workload, launched as the benchmark launches it, compared on every output
    row.  The inputs are generated chunk by chunk, uploaded, and the oracle writes its pool
    from each chunk, so no full-size host copy of the inputs is ever held."""
    import torch
    meta = wl.compressor_meta(seed, R, num_pages)
    log(f"[full] ratio {ratio} R {R}: generating inputs, oracle on every row")
    kv = torch.empty((R * ratio, 512), dtype=torch.float32, device="cuda")
    sc = torch.empty_like(kv)
    ref = orc.new_pool(layout, num_pages)
    step = max(1, (1 << 26) // (512 * ratio))      # output rows per chunk
    chunks = [(i0, min(step, R - i0)) for i0 in range(0, R, step)]
    for i0, n in chunks:
        a, b = wl.compressor_window(seed, ratio, i0, n)
        kv[i0 * ratio:(i0 + n) * ratio].copy_(torch.from_numpy(a))
        sc[i0 * ratio:(i0 + n) * ratio].copy_(torch.from_numpy(b))
        orc.kv_compress_store(layout, ref, a, b, ratio, np.ascontiguousarray(meta["pos"][i0:i0 + n]),
                              cos_sin, np.ascontiguousarray(meta["slots"][i0:i0 + n]))
    pool = kvq.new_pool(layout, num_pages)
    log(f"[full] ratio {ratio}: launching")
    kvq.kv_compress_store(pool, layout, kv, sc, ratio, to_dev(meta["pos"]), cos_sin_dev,
                          to_dev(meta["slots"]))
    torch.cuda.synchronize()
    got = to_host(pool)
    del kv, sc, pool
    compare_compressed(got, ref, layout, meta["slots"], label=f"full r{ratio} L{layout} R {R}")
    assert untouched_equal(got, ref, layout, meta["slots"])   # nothing outside the slots


@pytest.mark.slow
@pytest.mark.parametrize("layout", LAYOUTS)
def test_c4a_full_size_every_row(kvq, orc, cos_sin, cos_sin_dev, layout):
    full_compressor_check(kvq, orc, layout, 4, 16384, 3, cos_sin, cos_sin_dev)


@pytest.mark.slow
@pytest.mark.parametrize("layout", LAYOUTS)
def test_c128a_full_size_every_row(kvq, orc, cos_sin, cos_sin_dev, layout):
    full_compressor_check(kvq, orc, layout, 128, 16384, 4, cos_sin, cos_sin_dev)


@pytest.mark.slow
@pytest.mark.parametrize("ratio", [2, 4, 8, 16, 32, 64])
def test_ratio_sweep_size_every_row(kvq, orc, cos_sin, cos_sin_dev, ratio):
    """The benchmark's ratio sweep shape: 2,097,152 input rows (8 GiB of kv and score)
    compressed at each ratio, V41, every output row compared.  At ratios 2 and 4 this
    size takes the non-temporal-store build of the short-window kernel (C4A the plain one)."""
    R = 2097152 // ratio
    full_compressor_check(kvq, orc, V41, ratio, R, 40 + ratio, cos_sin, cos_sin_dev,
                          num_pages=max(4096, (R * 5 // 4) // 64 + 1))


# ------------------------------------------------------------------ decode-step state
@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("ratio,S,T", [(1, 40, 5), (4, 96, 41), (7, 30, 40), (128, 24, 300), (200, 8, 450)])
def test_compress_state_decode_steps(kvq, orc, cos_sin, cos_sin_dev, layout, ratio, S, T):
    """S sequences add one row per step (sequence s joins at step t0[s]); every completed
    window must equal the batch compressor's result on the same rows (tolerance rule),
    incomplete windows store nothing, and the counts end at (rows seen) mod ratio."""
    import torch
    rng = np.random.default_rng(1000 * ratio + S)
    num_pages = 64
    t0 = rng.integers(0, max(1, T // 3), S)
    nrows = np.maximum(T - t0, 0)
    nwin = nrows // ratio
    rows = [rng.standard_normal((nrows[s_], 512)).astype(np.float32) for s_ in range(S)]
    scs = [(2 * rng.standard_normal((nrows[s_], 512))).astype(np.float32) for s_ in range(S)]
    wslots = wl.distinct_slots(rng, int(nwin.sum()) + S, 64, num_pages * 64)
    win_slot, win_pos, k_ = [], [], 0
    for s_ in range(S):
        win_slot.append(wslots[k_:k_ + nwin[s_] + 1]); k_ += nwin[s_] + 1
        win_pos.append(rng.integers(0, 65536, nwin[s_] + 1).astype(np.int32))
    pool = kvq.new_pool(layout, num_pages)
    state, count = kvq.new_compress_state(S + 3)
    sid_of = rng.permutation(S + 3)[:S].astype(np.int32)       # states need not be dense
    for t in range(T):
        act = [s_ for s_ in range(S) if t >= t0[s_]]
        rng.shuffle(act)
        if not act:
            continue
        r_idx = [t - t0[s_] for s_ in act]
        kv = np.stack([rows[s_][r] for s_, r in zip(act, r_idx)])
        sc = np.stack([scs[s_][r] for s_, r in zip(act, r_idx)])
        w_idx = [r // ratio for r in r_idx]
        pos = np.array([win_pos[s_][w] for s_, w in zip(act, w_idx)], np.int32)
        slots = np.array([win_slot[s_][w] for s_, w in zip(act, w_idx)], np.int32)
        kvq.kv_compress_state_update(pool, layout, state, count, ratio, to_dev(sid_of[act]), to_dev(kv),
                                     to_dev(sc), to_dev(pos), cos_sin_dev, to_dev(slots))
    torch.cuda.synchronize()
    got = to_host(pool)
    assert np.array_equal(to_host(count)[sid_of], (nrows % ratio).astype(np.int32))
    ref = orc.new_pool(layout, num_pages)
    done_slots = []
    for s_ in range(S):
        if nwin[s_] == 0:
            continue
        kvw = np.ascontiguousarray(rows[s_][:nwin[s_] * ratio])
        scw = np.ascontiguousarray(scs[s_][:nwin[s_] * ratio])
        sl = np.ascontiguousarray(win_slot[s_][:nwin[s_]])
        orc.kv_compress_store(layout, ref, kvw, scw, ratio, np.ascontiguousarray(win_pos[s_][:nwin[s_]]),
                              cos_sin, sl)
        done_slots.append(sl)
    done = np.concatenate(done_slots)
    log(f"[state] ratio {ratio}: {done.size} windows completed over {T} steps")
    compare_compressed(got, ref, layout, done, label=f"state r{ratio} L{layout}")
    assert untouched_equal(got, ref, layout, done)   # incomplete windows wrote nothing


# ------------------------------------------------------------------ dequant
@pytest.mark.parametrize("layout", LAYOUTS)
def test_dequant_exhaustive_bit_exact(kvq, orc, layout):
    """Every (code, scale byte) pair, including NaN codes, NaN scales and under/overflow."""
    if layout == V41:
        pool = np.zeros((2, kvq.page_bytes(V41)), np.uint8)
        for r in range(128):
            page, row = divmod(r, 64)
            for b in range(16):
                pool[page, 64 * 512 + row * 16 + b] = 2 * r + (b // 8)
                pool[page, row * 512 + b * 32: row * 512 + b * 32 + 32] = (b % 8) * 32 + np.arange(32)
        pages = np.array([1, 0, 1, 7, -2], np.int32)
    else:
        pool = np.zeros((1, kvq.page_bytes(FP4)), np.uint8)
        nib = np.arange(32) % 16
        for r in range(16):
            for b in range(16):
                pool[0, 64 * 256 + r * 32 + b] = r * 16 + b
            pool[0, r * 256:(r + 1) * 256] = np.tile((nib[0::2] | (nib[1::2] << 4)).astype(np.uint8), 16)
        pool[0, 16 * 256:64 * 256] = np.random.default_rng(3).integers(0, 256, 48 * 256)
        pages = np.array([0, 0, 3], np.int32)
    import torch
    out = torch.full((pages.size * 64, 512), 0x1357, dtype=torch.int16, device="cuda")
    kvq.kv_dequant(to_dev(pool), layout, to_dev(pages), out)
    ref = np.full((pages.size * 64, 512), 0x1357, np.uint16)
    orc.kv_dequant(layout, pool, pages, ref)
    assert np.array_equal(to_host(out), ref)


@pytest.mark.parametrize("layout", LAYOUTS)
def test_dequant_after_store_bit_exact(kvq, orc, layout):
    rng = np.random.default_rng(14)
    n, num_pages = 900, 20
    k = wl.bf16_bits(rng.standard_normal((n, 512)).astype(np.float32))
    slots = wl.distinct_slots(rng, n, 64, num_pages * 64)
    pool = kvq.new_pool(layout, num_pages)
    kvq.kv_store(pool, layout, to_dev(k), to_dev(slots))
    pages = np.unique(slots >> 6).astype(np.int32)[::-1].copy()     # any order
    out = kvq.kv_dequant(pool, layout, to_dev(pages))
    ref_pool = orc.new_pool(layout, num_pages)
    orc.kv_store(layout, ref_pool, k, slots)
    assert np.array_equal(to_host(pool), ref_pool)
    ref = orc.kv_dequant(layout, ref_pool, pages)
    assert np.array_equal(to_host(out), ref)


@pytest.mark.parametrize("layout", LAYOUTS)
def test_dequant_long_page_list_bit_exact(kvq, orc, layout):
    """Lists of 1024 pages or more use four rows per wavefront; random pool bytes (NaN
    codes and scales included), repeated and out-of-pool page ids."""
    rng = np.random.default_rng(16)
    num_pages = 1500
    pool = rng.integers(0, 256, (num_pages, kvq.page_bytes(layout))).astype(np.uint8)
    pages = rng.integers(0, num_pages, 1100).astype(np.int32)
    pages[[3, 500, 1099]] = [-1, num_pages, 7]
    import torch
    out = torch.full((pages.size * 64, 512), 0x2468, dtype=torch.int16, device="cuda")
    kvq.kv_dequant(to_dev(pool), layout, to_dev(pages), out)
    ref = np.full((pages.size * 64, 512), 0x2468, np.uint16)
    orc.kv_dequant(layout, pool, pages, ref)
    assert np.array_equal(to_host(out), ref)


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("n", [1, 77, 2049])
def test_dequant_slots_bit_exact(kvq, orc, layout, n):
    import torch
    rng = np.random.default_rng(17 + n)
    num_pages = 40
    pool = rng.integers(0, 256, (num_pages, kvq.page_bytes(layout))).astype(np.uint8)
    slots = rng.integers(0, num_pages * 64, n).astype(np.int32)
    if n > 3:
        slots[[0, 1, 2]] = [-5, num_pages * 64, 3]
    out = torch.full((n, 512), 0x3579, dtype=torch.int16, device="cuda")
    kvq.kv_dequant_slots(to_dev(pool), layout, to_dev(slots), out)
    ref = np.full((n, 512), 0x3579, np.uint16)
    orc.kv_dequant_slots(layout, pool, slots, ref)
    assert np.array_equal(to_host(out), ref)


# ------------------------------------------------------------------ translate
def test_translate_semantics(kvq, orc):
    import torch
    rng = np.random.default_rng(15)
    table = rng.integers(0, 1 << 20, 5000).astype(np.int32)
    for n, cap in ((0, 0), (0, 77), (1, 1), (300, 300), (300, 1025), (4097, 5000)):
        full = rng.integers(-3, 5003, n).astype(np.int32)
        out = torch.full((cap,), 0x5A5A5A5A, dtype=torch.int32, device="cuda")
        res = kvq.kv_translate_slots(to_dev(table), to_dev(full), out)
        rc, ref = orc.translate_slots(table, full, cap)
        assert rc == 0 and res is not None and res.numel() == n
        assert np.array_equal(to_host(out), ref), (n, cap)
    full = rng.integers(0, 5000, 10).astype(np.int32)
    out = torch.full((9,), 0x5A5A5A5A, dtype=torch.int32, device="cuda")
    assert kvq.kv_translate_slots(to_dev(table), to_dev(full), out) is None   # n > cap
    assert np.all(to_host(out) == 0x5A5A5A5A)


# ------------------------------------------------------------------ mixed step (FP4)
def test_mixed_fp4_step(kvq, orc, cos_sin, cos_sin_dev):
    """Ragged decode/prefill batch: translate once, compress (ratio 4, V41_FP4) at the
    translated slots, dequantise the touched pages."""
    import torch
    d = wl.mixed_fp4(seed=5)
    R = d["R"]
    log(f"[mixed] R {R}, pages {d['page_ids'].size}")
    out = torch.empty(d["cap"], dtype=torch.int32, device="cuda")
    swa = kvq.kv_translate_slots(to_dev(d["table"]), to_dev(d["full"]), out)
    rc, ref_loc = orc.translate_slots(d["table"], d["full"], d["cap"])
    assert rc == 0 and np.array_equal(to_host(out), ref_loc)
    pool = kvq.new_pool(FP4, d["num_pages"])
    kvq.kv_compress_store(pool, FP4, to_dev(d["kv"]), to_dev(d["score"]), 4, to_dev(d["pos"]),
                          cos_sin_dev, swa)
    ws = kvq.kv_dequant(pool, FP4, to_dev(d["page_ids"]))
    got_pool = to_host(pool)
    slots = ref_loc[:R].copy()
    ref_pool = orc.new_pool(FP4, d["num_pages"])
    orc.kv_compress_store(FP4, ref_pool, d["kv"], d["score"], 4, d["pos"], cos_sin, slots)
    compare_compressed(got_pool, ref_pool, FP4, slots, label="mixed fp4")
    assert untouched_equal(got_pool, ref_pool, FP4, slots)
    check_step_dequant(orc, FP4, to_host(ws), got_pool, ref_pool, d["page_ids"])


@pytest.mark.slow
@pytest.mark.parametrize("layout", LAYOUTS)
def test_compress_state_bench_shape(kvq, orc, cos_sin, cos_sin_dev, layout):
    """The benchmark's decode shape: 16,384 sequences, ratio 4, one row per sequence per
    call in a shuffled order, one full window each; every window compared."""
    import torch
    S, ratio, num_pages = 16384, 4, 4096
    rng = np.random.default_rng(77)
    kv = rng.standard_normal((S * ratio, 512)).astype(np.float32)     # window of s: rows [4s, 4s+4)
    sc = (2 * rng.standard_normal((S * ratio, 512))).astype(np.float32)
    pos = rng.integers(0, 65536, S).astype(np.int32)
    slots = wl.distinct_slots(rng, S, 64, num_pages * 64)
    pool = kvq.new_pool(layout, num_pages)
    state, count = kvq.new_compress_state(S)
    for t in range(ratio):
        order = rng.permutation(S).astype(np.int32)
        rows = order * ratio + t
        kvq.kv_compress_state_update(pool, layout, state, count, ratio, to_dev(order), to_dev(kv[rows]),
                                     to_dev(sc[rows]), to_dev(pos[order]), cos_sin_dev, to_dev(slots[order]))
    torch.cuda.synchronize()
    assert not to_host(count).any()
    ref = orc.new_pool(layout, num_pages)
    orc.kv_compress_store(layout, ref, kv, sc, ratio, pos, cos_sin, slots)
    got = to_host(pool)
    compare_compressed(got, ref, layout, slots, label=f"state bench shape L{layout}")
    assert untouched_equal(got, ref, layout, slots)
