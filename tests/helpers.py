"""Shared test helpers: GPU library loading, tensor marshalling and the comparison rules.

Comparison rules (the parity bar):
* store paths, dequant, translate, addressing and untouched bytes: bit-exact;
* compressor rows: scale bytes bit-exact; codes within one code step (ordinal distance
  <= 1, +0 and -0 equal) and at least 99.9 % identical.  No code or scale is excused: the
  kernels pool in float64 and round the pooled value once to bf16, so their bytes equal
  the oracle's unless an exact pooled value sits within about 1e-15 of a bf16 midpoint.
"""
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


def compare_compressed(got_pool, ref_pool, layout, slots, min_equal=0.999, label=""):
    """Apply the compressor comparison rule on the rows at `slots`; returns the fraction of
    identical codes and prints how many codes differ."""
    if len(slots) == 0:
        return 1.0
    gc, gs = rows_of(got_pool, layout, slots)
    rc, rs = rows_of(ref_pool, layout, slots)
    if layout == FP4:
        assert np.all(gs[:, 16:] == 0) and np.all(rs[:, 16:] == 0), f"{label}: FP4 pad bytes"
    bad_scale = gs[:, :16] != rs[:, :16]
    if bad_scale.any():
        r, b = np.argwhere(bad_scale)[0]
        raise AssertionError(f"{label}: {int(bad_scale.sum())} scale bytes differ; first at row {r} "
                             f"(slot {slots[r]}) block {b}: {gs[r, b]} vs {rs[r, b]}")
    og, orf = code_ords(gc, layout), code_ords(rc, layout)
    d = np.abs(og - orf)
    n_diff = int((d != 0).sum())
    frac = 1.0 - n_diff / d.size if d.size else 1.0
    print(f"[{label}] rows {len(slots)}: {n_diff} of {d.size} codes differ "
          f"(identical {frac * 100:.6f} %), max step {int(d.max()) if d.size else 0}", flush=True)
    if d.size and d.max() > 1:
        r, c = np.argwhere(d > 1)[0]
        raise AssertionError(f"{label}: code {og[r, c]} vs {orf[r, c]} at row {r} (slot {slots[r]}) "
                             f"channel {c}: more than one step")
    assert frac >= min_equal, f"{label}: only {frac * 100:.4f} % of codes identical"
    return frac


def code_differs(got_pool, ref_pool, layout, page_ids):
    """[P*64, 512] mask of the dequant outputs of the listed pages whose code or scale byte
    differs between two pools (False for page ids outside the pool)."""
    ids = np.asarray(page_ids, np.int64)
    valid = (ids >= 0) & (ids < got_pool.shape[0])
    safe = np.where(valid, ids, 0)
    cr, sr = CR[layout], SR[layout]

    def parts(pool):
        pg = pool[safe]
        codes = pg[:, :64 * cr].reshape(-1, 64, cr)
        if layout == FP4:
            codes = np.stack([codes & 15, codes >> 4], axis=-1).reshape(-1, 64, 512)
        scales = np.repeat(pg[:, 64 * cr:].reshape(-1, 64, sr)[:, :, :16], 32, axis=-1)
        return codes, scales

    gc, gs = parts(got_pool)
    rc, rs = parts(ref_pool)
    return (((gc != rc) | (gs != rs)) & valid[:, None, None]).reshape(-1, 512)


def check_step_dequant(orc, layout, ws_host, got_pool, ref_pool, page_ids):
    """A step's dequant of the GPU's pool against the oracle's dequant of the oracle's pool:
    equal wherever the two pools hold the same code and scale (everywhere when the
    compressor's bytes are identical); a code that differs by the one step the compressor
    rule allows may give another value.  Returns the number of such values."""
    want = orc.kv_dequant(layout, ref_pool, np.ascontiguousarray(page_ids, np.int32))
    differs = code_differs(got_pool, ref_pool, layout, page_ids)
    assert np.array_equal(ws_host[~differs], want[~differs]), "dequant differs where the codes agree"
    return int(differs.sum())


def untouched_equal(got_pool, ref_pool, layout, slots):
    """Every byte outside the rows at `slots` is equal in both pools."""
    mask = np.ones(got_pool.shape, bool)
    slots = np.asarray(slots, np.int64)
    page, row = slots >> 6, slots & 63
    cr, sr = CR[layout], SR[layout]
    mask[page[:, None], row[:, None] * cr + np.arange(cr)[None, :]] = False
    mask[page[:, None], 64 * cr + row[:, None] * sr + np.arange(sr)[None, :]] = False
    return np.array_equal(got_pool[mask], ref_pool[mask])
