"""Seeded random configurations through the C ABI, against the oracle.

Each compressor case draws from its seed a layout, a ratio, the number of output rows, a
row stride (the channels past 512 hold NaN, so a read of them would show), a value
family, a pool size, slots and positions with some outside the pool or the table, and the
entry point (kv_compress_store, or kv_compress_store_translate with a table).  The whole
pool is canary-filled and compared with the oracle's (compressor rule on the stored rows,
every other byte equal), and the translated buffer bit for bit.  The oracle's pool is
then dequantised on the GPU, page list with ids outside the pool included, and compared
with the oracle's dequant bit for bit.  The store cases do the same for kv_store,
kv_store_rope and kv_store_norm_rope, and the decode-state cases fold rows of the same
value families one call at a time (kv_compress_state_update) against the batch oracle.

Value families beyond the benchmark's normal rows: per-channel scales spread over 2^+-60,
fp32 denormals, magnitudes near 1e38, equal scores (the window mean; with bf16 inputs at
ratio 2 the mean of two neighbours is an exact bf16 midpoint), one dominant score per
window, windows of exact zeros, and rows that cancel.
"""
import os

import numpy as np
import pytest

from helpers import FP4, V41, compare_compressed, gpu_lib, to_dev, to_host, untouched_equal
from quantized_paged_kv_compress_amd import workloads as wl

pytestmark = pytest.mark.gpu
RATIOS = (1, 2, 4, 8, 16, 32, 64, 128)
FAMILIES = ("normal", "channel_scales", "denormal", "large", "equal_scores", "dominant",
            "zeros", "cancel", "midpoints")
# KVQ_RANDOM_CASES widens the sweep (more seeds of both kinds) for a longer numerics run
N_COMPRESS = int(os.environ.get("KVQ_RANDOM_CASES", 64))
N_STORE = max(24, N_COMPRESS * 3 // 8)
CANARY8 = 0xA5
CANARY16 = 0x5A5A


@pytest.fixture(scope="module")
def kvq():
    return gpu_lib()


def log(msg):
    print(msg, flush=True)


def padded(rows, ld):
    """fp32 [rows, ld] whose channels past 512 are NaN."""
    return np.full((rows, ld), np.nan, np.float32)


def family_values(rng, family, rows, ratio, ld):
    """kv and score rows (fp32 [rows, ld]) of one value family."""
    kv, sc = padded(rows, ld), padded(rows, ld)
    x = rng.standard_normal((rows, 512))
    s = 2.0 * rng.standard_normal((rows, 512))
    if family == "channel_scales":
        x = x * np.exp2(rng.uniform(-60, 60, 512))[None, :]
        s = s * np.exp2(rng.uniform(-3, 3, 512))[None, :]
    elif family == "denormal":
        x = x * 1e-40
    elif family == "large":
        x = rng.uniform(-1.0, 1.0, (rows, 512)) * 1e38
    elif family == "equal_scores":
        s = np.repeat(rng.standard_normal((rows // ratio, 512)), ratio, axis=0)
    elif family == "dominant":
        s = rng.standard_normal((rows, 512))
        top = rng.integers(0, ratio, (rows // ratio, 512))
        s[(np.arange(rows // ratio)[:, None] * ratio + top), np.arange(512)[None, :]] += 80.0
    elif family == "zeros":
        x[rng.random(rows) < 0.5] = 0.0
        w = rng.random(rows // ratio) < 0.3
        x[np.repeat(w, ratio)] = 0.0
    elif family == "cancel":
        x = x.reshape(rows // ratio, ratio, 512)
        if ratio > 1:
            x[:, 1::2] = -x[:, 0:ratio - 1:2] * (1 + 2.0 ** -20 * rng.standard_normal(x[:, 1::2].shape))
        x = x.reshape(rows, 512)
        s = np.repeat(rng.standard_normal((rows // ratio, 512)), ratio, axis=0)
    elif family == "midpoints":
        # bf16 inputs and equal scores: at ratio 2 the pooled value of two bf16 neighbours
        # is the exact midpoint between them, so its rounding is a tie
        xb = wl.bf16_bits(x.astype(np.float32)).astype(np.uint32)
        if ratio == 2:
            xb = xb.reshape(rows // 2, 2, 512)
            xb[:, 1] = xb[:, 0] + 1
            xb = xb.reshape(rows, 512)
        x = (xb << 16).astype(np.uint32).view(np.float32)
        s = np.repeat(rng.standard_normal((rows // ratio, 512)), ratio, axis=0)
    kv[:, :512] = x
    sc[:, :512] = s
    return kv, sc


def slot_source(rng, R, nslots):
    """R distinct slots drawn from [-8, nslots + 8): a few are outside the pool."""
    return (rng.choice(nslots + 16, R, replace=False) - 8).astype(np.int32)


def positions(rng, n, max_pos):
    pos = rng.integers(0, max_pos, n).astype(np.int32)
    bad = rng.random(n) < 0.02
    pos[bad] = rng.choice(np.array([-1, max_pos, max_pos + 100], np.int32), int(bad.sum()))
    return pos


def draw_compress(seed):
    rng = np.random.default_rng(7100 + seed)
    layout = (V41, FP4)[seed % 2]
    ratio = RATIOS[(seed // 2) % len(RATIOS)]
    ld = int(rng.choice([512, 516, 528, 640, 1024]))
    max_in = min(1 << 15, (1 << 24) // ld)
    R = int(rng.integers(1, min(max_in // ratio, 3000) + 1))
    family = FAMILIES[int(rng.integers(0, len(FAMILIES)))]
    fused = bool(rng.integers(0, 2))
    num_pages = (R + 63) // 64 + int(rng.integers(0, 8))
    max_pos = int(rng.choice([65536, 5000]))
    return rng, dict(layout=layout, ratio=ratio, ld=ld, R=R, family=family, fused=fused,
                     num_pages=num_pages, max_pos=max_pos)


def dequant_check(kvq, orc, layout, ref_pool, pages, rng):
    """The oracle's pool dequantised on the GPU equals the oracle's dequant, bit for bit."""
    import torch
    num_pages = ref_pool.shape[0]
    ids = np.concatenate([pages, np.array([-1, num_pages, num_pages + 9], np.int64)])
    ids = rng.permutation(ids).astype(np.int32)
    want = orc.kv_dequant(layout, ref_pool, ids, np.full((ids.size * 64, 512), CANARY16, np.uint16))
    dpool = to_dev(ref_pool)
    out = torch.full((ids.size * 64, 512), CANARY16, dtype=torch.int16, device="cuda")
    kvq.kv_dequant(dpool, layout, to_dev(ids), out)
    torch.cuda.synchronize()
    got = to_host(out)
    assert np.array_equal(got, want), f"dequant: {int((got != want).sum())} values differ"


@pytest.mark.parametrize("seed", range(N_COMPRESS))
def test_random_compressor_config(kvq, orc, seed):
    import torch
    rng, c = draw_compress(seed)
    log(f"[random compress {seed}] {c}")
    layout, ratio, R, ld, num_pages = c["layout"], c["ratio"], c["R"], c["ld"], c["num_pages"]
    nslots = num_pages * 64
    kv, sc = family_values(rng, c["family"], R * ratio, ratio, ld)
    cs = wl.rope_cos_sin(max_pos=c["max_pos"])
    pos = positions(rng, R, c["max_pos"])
    pool = kvq.new_pool(layout, num_pages)
    pool.fill_(CANARY8)
    ref = np.full((num_pages, orc.page_bytes(layout)), CANARY8, np.uint8)
    kv_d, sc_d = to_dev(kv), to_dev(sc)
    score_d = sc_d if ratio > 1 else None
    if c["fused"]:
        table_len = int(rng.integers(R, 3 * R + 64))
        table = (rng.permutation(max(table_len, nslots + 16))[:table_len] - 8).astype(np.int32)
        full = (rng.choice(table_len + 32, R, replace=False) - 16).astype(np.int32)
        cap = R + int(rng.integers(0, 4 * R + 100))
        buf = torch.full((cap + 64,), -77, dtype=torch.int32, device="cuda")
        res = kvq.kv_compress_store_translate(pool, layout, kv_d, score_d, ratio, to_dev(pos), to_dev(cs),
                                              to_dev(table), to_dev(full), buf[:cap])
        assert res is not None
        rc, loc = orc.translate_slots(table, full, cap)
        assert rc == 0
        slots = np.ascontiguousarray(loc[:R])
    else:
        slots = slot_source(rng, R, nslots)
        kvq.kv_compress_store(pool, layout, kv_d, score_d, ratio, to_dev(pos), to_dev(cs), to_dev(slots))
    torch.cuda.synchronize()
    orc.kv_compress_store(layout, ref, kv, sc, ratio, pos, cs, slots)
    got = to_host(pool)
    if c["fused"]:
        got_buf = to_host(buf)
        assert np.array_equal(got_buf[:cap], loc), "translated slots"
        assert np.all(got_buf[cap:] == -77), "written past the buffer"
    stored = slots[(slots >= 0) & (slots < nslots) & (pos >= 0) & (pos < c["max_pos"])]
    compare_compressed(got, ref, layout, stored, label=f"random {seed}")
    assert untouched_equal(got, ref, layout, stored), "bytes outside the stored rows"
    dequant_check(kvq, orc, layout, ref, np.unique(stored >> 6), rng)


def draw_store(seed):
    rng = np.random.default_rng(7300 + seed)
    layout = (V41, FP4)[seed % 2]
    mode = ("store", "store_rope", "norm_rope")[(seed // 2) % 3]
    ld = int(rng.choice([512, 520, 640, 1024]))
    n = int(rng.integers(1, 5000))
    family = ("normal", "channel_scales", "denormal", "large", "zeros")[int(rng.integers(0, 5))]
    num_pages = (n + 63) // 64 + int(rng.integers(0, 8))
    max_pos = int(rng.choice([65536, 3000]))
    return rng, dict(layout=layout, mode=mode, ld=ld, n=n, family=family, num_pages=num_pages,
                     max_pos=max_pos)


@pytest.mark.parametrize("seed", range(N_STORE))
def test_random_store_config(kvq, orc, seed):
    import torch
    rng, c = draw_store(seed)
    log(f"[random store {seed}] {c}")
    layout, mode, n, ld, num_pages = c["layout"], c["mode"], c["n"], c["ld"], c["num_pages"]
    nslots = num_pages * 64
    x, _ = family_values(rng, c["family"], n, 1, ld)
    k = np.full((n, ld), 0x7FC0, np.uint16)                 # bf16 NaN past channel 512
    k[:, :512] = wl.bf16_bits(np.ascontiguousarray(x[:, :512]))
    slots = slot_source(rng, n, nslots)
    cs = wl.rope_cos_sin(max_pos=c["max_pos"])
    pos = positions(rng, n, c["max_pos"])
    weight = wl.bf16_bits(rng.uniform(0.25, 2.0, 512).astype(np.float32))
    # eps 0 is drawn only where no row is all zeros (0 / 0 has no defined value)
    eps = 1e-6 if c["family"] == "zeros" else float(rng.choice([0.0, 1e-6]))
    pool = kvq.new_pool(layout, num_pages)
    pool.fill_(CANARY8)
    ref = np.full((num_pages, orc.page_bytes(layout)), CANARY8, np.uint8)
    k_d = to_dev(k)
    if mode == "store":
        kvq.kv_store(pool, layout, k_d, to_dev(slots))
        orc.kv_store(layout, ref, np.ascontiguousarray(k[:, :512]), slots)
        ok = (slots >= 0) & (slots < nslots)
    elif mode == "store_rope":
        kvq.kv_store_rope(pool, layout, k_d, to_dev(pos), to_dev(cs), to_dev(slots))
        orc.kv_store_rope(layout, ref, np.ascontiguousarray(k[:, :512]), pos, cs, slots)
        ok = (slots >= 0) & (slots < nslots) & (pos >= 0) & (pos < c["max_pos"])
    else:
        kvq.kv_store_norm_rope(pool, layout, k_d, to_dev(weight), eps, to_dev(pos), to_dev(cs), to_dev(slots))
        orc.kv_store_norm_rope(layout, ref, np.ascontiguousarray(k[:, :512]), weight, eps, pos, cs, slots)
        ok = (slots >= 0) & (slots < nslots) & (pos >= 0) & (pos < c["max_pos"])
    torch.cuda.synchronize()
    got = to_host(pool)
    stored = slots[ok]
    if mode == "norm_rope":
        compare_compressed(got, ref, layout, stored, label=f"random store {seed}")
        assert untouched_equal(got, ref, layout, stored)
    else:
        assert np.array_equal(got, ref), f"{int((got != ref).sum())} pool bytes differ"
    dequant_check(kvq, orc, layout, ref, np.unique(stored >> 6), rng)


N_STATE = max(24, N_COMPRESS * 3 // 8)


def draw_state(seed):
    rng = np.random.default_rng(7500 + seed)
    layout = (V41, FP4)[seed % 2]
    ratio = int(rng.choice([1, 2, 3, 4, 7, 16, 64, 128, 200]))
    S = int(rng.integers(1, 300))
    T = int(rng.integers(1, 3 * ratio + 3))
    family = FAMILIES[int(rng.integers(0, len(FAMILIES)))]
    return rng, dict(layout=layout, ratio=ratio, S=S, T=T, family=family)


@pytest.mark.parametrize("seed", range(N_STATE))
def test_random_state_config(kvq, orc, seed):
    """The decode-step state: S sequences join at random steps and add one row per call in a
    shuffled order, rows drawn from a value family; every completed window must equal the
    batch compressor on the same rows, incomplete windows store nothing, a few windows end
    at slots outside the pool, and the counts end at (rows seen) mod ratio."""
    import torch
    rng, c = draw_state(seed)
    log(f"[random state {seed}] {c}")
    layout, ratio, S, T = c["layout"], c["ratio"], c["S"], c["T"]
    num_pages, max_pos = 64, 65536
    nslots = num_pages * 64
    cs = wl.rope_cos_sin()
    t0 = rng.integers(0, max(1, T // 3), S)
    nrows = np.maximum(T - t0, 0)
    nwin = nrows // ratio
    rows, scs = [], []
    for s_ in range(S):
        x, sc_ = family_values(rng, c["family"], (nwin[s_] + 1) * ratio, ratio, 512)
        rows.append(np.ascontiguousarray(x[:nrows[s_]]))
        scs.append(np.ascontiguousarray(sc_[:nrows[s_]]))
    wslots = (rng.choice(nslots + 16, int(nwin.sum()) + S, replace=False) - 8).astype(np.int32)
    win_slot, win_pos, k_ = [], [], 0
    for s_ in range(S):
        win_slot.append(wslots[k_:k_ + nwin[s_] + 1])
        k_ += nwin[s_] + 1
        win_pos.append(rng.integers(0, max_pos, nwin[s_] + 1).astype(np.int32))
    pool = kvq.new_pool(layout, num_pages)
    pool.fill_(CANARY8)
    state, count = kvq.new_compress_state(S + 5)
    sid_of = rng.permutation(S + 5)[:S].astype(np.int32)
    cs_d = to_dev(cs)
    for t in range(T):
        act = [s_ for s_ in range(S) if t >= t0[s_]]
        if not act:
            continue
        rng.shuffle(act)
        r_idx = [t - t0[s_] for s_ in act]
        kv = np.stack([rows[s_][r] for s_, r in zip(act, r_idx)])
        sc = np.stack([scs[s_][r] for s_, r in zip(act, r_idx)])
        w_idx = [r // ratio for r in r_idx]
        pos = np.array([win_pos[s_][w] for s_, w in zip(act, w_idx)], np.int32)
        slots = np.array([win_slot[s_][w] for s_, w in zip(act, w_idx)], np.int32)
        kvq.kv_compress_state_update(pool, layout, state, count, ratio, to_dev(sid_of[act]), to_dev(kv),
                                     to_dev(sc), to_dev(pos), cs_d, to_dev(slots))
    torch.cuda.synchronize()
    got = to_host(pool)
    assert np.array_equal(to_host(count)[sid_of], (nrows % ratio).astype(np.int32)), "counts"
    ref = np.full((num_pages, orc.page_bytes(layout)), CANARY8, np.uint8)
    stored = []
    for s_ in range(S):
        if nwin[s_] == 0:
            continue
        sl = np.ascontiguousarray(win_slot[s_][:nwin[s_]])
        orc.kv_compress_store(layout, ref, np.ascontiguousarray(rows[s_][:nwin[s_] * ratio]),
                              np.ascontiguousarray(scs[s_][:nwin[s_] * ratio]), ratio,
                              np.ascontiguousarray(win_pos[s_][:nwin[s_]]), cs, sl)
        stored.append(sl[(sl >= 0) & (sl < nslots)])
    stored = np.concatenate(stored) if stored else np.zeros(0, np.int32)
    compare_compressed(got, ref, layout, stored, label=f"random state {seed}")
    assert untouched_equal(got, ref, layout, stored), "bytes outside the completed windows"
