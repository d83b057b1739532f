"""Shared test helpers: GPU library loading, tensor marshalling and the comparison rules.

Comparison rules (the parity bar):
* store paths, dequant, translate, addressing and untouched bytes: bit-exact;
* compressor rows: scale bytes bit-exact; codes within one code step (ordinal distance
  <= 1, +0 and -0 equal) and at least 99.9 % identical.  A block whose scale differs is
  admitted only if its scale is one step away and the exact (float64) pooled value of a
  channel feeding that block lies within 2^-16 relative of a bf16 rounding midpoint (the
  only way an fp32 pooled value can round to another bf16 than the exact one, and so move
  the block maximum across a scale boundary); at most 2 such blocks per call.
* RoPE channels (448..511): the rotation can turn a one-ulp bf16 difference of an input
  into several code steps when its two products nearly cancel.  A code there more than
  one step from the oracle's is admitted only if an input of its rotation pair sits at a
  bf16 near-tie and the code is within one step of the oracle's own result (its RoPE and
  encoders) with that input rounded to the other neighbouring bf16.
"""
import math
import os

import numpy as np

V41, FP4 = 1, 2
CR = {V41: 512, FP4: 256}
SR = {V41: 16, FP4: 32}


def gpu_lib():
    import torch
    if not torch.cuda.is_available():
        import pytest
        pytest.skip("no GPU")
    import quantized_paged_kv_compress_amd as kvq
    if not os.path.exists(kvq.LIB_PATH):
        from quantized_paged_kv_compress_amd import _build
        _build.build()
    kvq.load_library()
    return kvq


def to_dev(a, dev="cuda"):
    import torch
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def to_host(t):
    import torch
    t = t.cpu()
    if t.dtype in (torch.bfloat16, torch.int16, torch.uint16):
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def rows_of(pool, layout, slots):
    """(codes [n, CR], scales [n, SR]) of the given slots."""
    slots = np.asarray(slots, np.int64)
    page, row = slots >> 6, slots & 63
    cr, sr = CR[layout], SR[layout]
    ci = row[:, None] * cr + np.arange(cr)[None, :]
    si = 64 * cr + row[:, None] * sr + np.arange(sr)[None, :]
    return pool[page[:, None], ci], pool[page[:, None], si]


def code_ords(codes, layout):
    codes = codes.astype(np.int64)
    if layout == V41:
        return np.where(codes & 0x80, -(codes & 0x7F), codes & 0x7F)
    n = np.stack([codes & 15, codes >> 4], axis=-1).reshape(codes.shape[0], -1)
    return np.where(n & 8, -(n & 7), n & 7)


def near_bf16_midpoint(x, rel=2.0 ** -16):
    """True where float64 x is within rel (relative) of a midpoint between two bf16."""
    x = np.abs(np.asarray(x, np.float64))
    with np.errstate(divide="ignore", invalid="ignore"):
        e = np.floor(np.log2(np.where(x > 0, x, 1.0)))
    e = np.maximum(e, -126)
    q = 2.0 ** (e - 7)                     # bf16 spacing in this binade
    frac = x / q - np.floor(x / q)
    return np.abs(frac - 0.5) * q <= rel * np.maximum(x, 2.0 ** -133)


def _bf16_neighbours(x):
    """bf16 bit patterns of the two bf16 values around float64 x (same sign)."""
    ax = abs(float(x))
    if ax == 0.0:
        return [0]
    e = max(math.floor(math.log2(ax)), -126)
    q = 2.0 ** (e - 7)                       # bf16 spacing in this binade
    lo = math.floor(ax / q) * q
    vals = np.array([lo, lo + q], np.float64) * (-1.0 if x < 0 else 1.0)
    return [int(b) for b in (vals.astype(np.float32).view(np.uint32) >> 16)]


def _ord(code, layout):
    if layout == V41:
        return -(code & 0x7F) if code & 0x80 else code & 0x7F
    return -(code & 7) if code & 8 else code & 7


def rope_alternative_ok(layout, got_ord, scale_byte, pooled_row, c, pos_i, cos_sin):
    """The RoPE-channel rule: True if got_ord is within one code step of the oracle's code
    for channel c computed with some admissible bf16 rounding of the rotation pair's
    inputs (the exact RNE, or the other neighbour where the exact value is at a near-tie)."""
    import oracle
    p = (c - 448) % 32
    pair = (448 + p, 480 + p)
    options = []
    for q in pair:
        x = pooled_row[q]
        opts = {oracle.bf16_from_double(x)}
        if near_bf16_midpoint(x):
            opts |= set(_bf16_neighbours(x))
        options.append(sorted(opts))
    if len(options[0]) * len(options[1]) == 1:
        return False                          # no near-tie: nothing to excuse
    cs_row = np.ascontiguousarray(cos_sin[pos_i])
    for b1 in options[0]:
        for b2 in options[1]:
            v = np.zeros(512, np.uint16)
            v[pair[0]], v[pair[1]] = b1, b2
            val = oracle.bf16_to_f32(int(oracle.rope_row(v, cs_row)[c]))
            if layout == V41:
                code = oracle.e4m3_encode(math.ldexp(val, -(int(scale_byte) - 127)))
            else:
                s = oracle.e4m3_decode(int(scale_byte))
                code = 0 if s == 0 else oracle.e2m1_encode(float(np.float32(val) / np.float32(s)))
            if abs(got_ord - _ord(code, layout)) <= 1:
                return True
    return False


def compare_compressed(got_pool, ref_pool, layout, slots, pooled_f64=None, min_equal=0.999,
                       label="", rope=None):
    """Apply the compressor comparison rule on the rows at `slots`.  pooled_f64: [n, 512]
    exact pooled values (before RoPE) of the same rows, for the scale-escape and RoPE
    rules; rope = (pos, cos_sin): positions of the same rows and the table, for the RoPE
    rule."""
    gc, gs = rows_of(got_pool, layout, slots)
    rc, rs = rows_of(ref_pool, layout, slots)
    if layout == FP4:
        assert np.all(gs[:, 16:] == 0) and np.all(rs[:, 16:] == 0), "FP4 pad bytes"
    gs, rs = gs[:, :16].astype(np.int64), rs[:, :16].astype(np.int64)
    bad_scale = gs != rs
    n_bad = int(bad_scale.sum())
    if n_bad:
        assert pooled_f64 is not None, f"{label}: {n_bad} scale bytes differ"
        assert n_bad <= 2, f"{label}: {n_bad} scale bytes differ"
        for r, b in zip(*np.nonzero(bad_scale)):
            assert abs(gs[r, b] - rs[r, b]) == 1, f"{label}: scale off by more than one step"
            blocks = [b] + ([14, 15] if b in (14, 15) else [])
            ch = np.concatenate([np.arange(32 * q, 32 * q + 32) for q in blocks])
            assert near_bf16_midpoint(pooled_f64[r, ch]).any(), \
                f"{label}: scale mismatch at row {r} block {b} not explained by a bf16 tie"
        print(f"[{label}] {n_bad} scale byte(s) one step apart at bf16 near-ties", flush=True)
    og, orf = code_ords(gc, layout), code_ords(rc, layout)
    keep = np.repeat(~bad_scale, 32, axis=1)
    far = (np.abs(og - orf) > 1) & keep
    excused = np.zeros_like(far)
    for r, c in zip(*np.nonzero(far)):
        ok = (c >= 448 and pooled_f64 is not None and rope is not None and
              rope_alternative_ok(layout, og[r, c], rs[r, c // 32], pooled_f64[r], c, rope[0][r], rope[1]))
        excused[r, c] = ok
        print(f"[{label}] code {og[r, c]} vs {orf[r, c]} at row {r} (slot {slots[r]}) channel {c}: "
              f"{'a RoPE input at a bf16 near-tie, within one step of the other rounding' if ok else 'NOT EXPLAINED'}",
              flush=True)
    keep_codes = keep & ~excused
    d = np.abs(og - orf)[keep_codes]
    frac = float((np.abs(og - orf)[keep] == 0).mean()) if keep.any() else 1.0
    print(f"[{label}] codes identical {frac * 100:.5f} %, max step {int(d.max()) if d.size else 0}, "
          f"rows {len(slots)}", flush=True)
    assert d.size == 0 or d.max() <= 1, f"{label}: a code differs by more than one step"
    assert frac >= min_equal, f"{label}: only {frac * 100:.4f} % of codes identical"
    return frac


def untouched_equal(got_pool, ref_pool, layout, slots):
    """Every byte outside the rows at `slots` is equal in both pools."""
    mask = np.ones(got_pool.shape, bool)
    slots = np.asarray(slots, np.int64)
    page, row = slots >> 6, slots & 63
    cr, sr = CR[layout], SR[layout]
    mask[page[:, None], row[:, None] * cr + np.arange(cr)[None, :]] = False
    mask[page[:, None], 64 * cr + row[:, None] * sr + np.arange(sr)[None, :]] = False
    return np.array_equal(got_pool[mask], ref_pool[mask])
