"""CPU oracle for the KV compress -> quantise -> paged-store path.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU-baseline
leg may import this package; the library in ``quantized_paged_kv_compress_amd`` never
does.  The arithmetic lives in ``kvq_oracle.c`` (plain C, built by ``oracle/build.py``);
this module only marshals numpy arrays through ctypes.

What each oracle function follows, and what pins it (tests/test_oracle_pins.py):

================  ========================================  ==============================
function          source                                    pinned by
================  ========================================  ==============================
layout sizes      P1 s.1, "memory usage reduction"          printed 528 / 288 / 584 B and
                                                            9.6 % / 50.7 % savings
bf16 rounding     bfloat16 definition                       brute force on neighbours;
                                                            torch f32 -> bf16 casts
e4m3 enc/dec      OCP e4m3fn definition                     exhaustive vs brute-force
                                                            nearest; torch float8 casts
ue8m0             P1 s.1 (exponent from amax bits)          exhaustive vs exact rational
                                                            ceil(log2(amax/448)) and the
                                                            amax-bits closed form
e2m1 / fp4 scale  P1 s.1-2 (e2m1 codes, e4m3 scale per 32)  exhaustive vs brute force
                                                            with exact rational ties
RoPE              P3 s.3; NeoX half rotation                pos 0 identity; hand-computed
                                                            angles; norm preservation;
                                                            a worked row whose float32
                                                            rounding order decides its bf16
K norm (RMS)      P1 latency table "fused K norm + RoPE"    hand-computed row (eps 0);
                  (formula is a reading)                    power-of-two scale invariance;
                                                            weight channel mapping;
                                                            Python fsum brute force
pooling           P3 s.2 (per-channel online softmax)       r = 1 identity; equal scores
                                                            give the mean; dominance;
                                                            permutation and shift
                                                            invariance; Fraction brute
                                                            force on tiny windows
addressing        P1 s.1 (PagedKV page/row/scale row)       brute-force tagged rows and
                                                            canaries on a 4-page pool
dequant           P1 s.4                                    decode tables; quant(dequant)
                                                            idempotence; round-trip bound
dequant by slot   P1 s.4 (per-token form)                   equals the matching rows of the
                                                            page dequant; skips out-of-pool
translate         P2 s.1                                    buffer semantics printed on
                                                            the page (zero tail, refusal)
composition       P1 s.2-3, P3 s.1-3 (pool, bf16, RoPE,    compress at ratio 1 equals
                  quantise, store)                          store_rope of the bf16 rows;
                                                            compress equals the pool then
                                                            store_rope; norm + RoPE + store
                                                            equals its parts
================  ========================================  ==============================
"""
import ctypes
import os

import numpy as np

from . import build as _build

V41 = 1
V41_FP4 = 2
HEAD = 512
ROPE_DIM = 64
PAGE_ROWS = 64

_lib = None


def lib():
    """Load oracle/liboracle.so, building it first if it is not there."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_build.LIB):
        _build.build()
    _lib = _load(_build.LIB)
    return _lib


def use_library(path):
    """Swap in another build of the oracle (the mutation tests plant mistakes in copies
    of kvq_oracle.c); returns the previous handle, which use_handle() restores."""
    global _lib
    prev = _lib
    _lib = _load(path)
    return prev


def use_handle(handle):
    global _lib
    _lib = handle


def _load(path):
    L = ctypes.CDLL(path)
    i32, i64, u8, u16, f32, f64 = (ctypes.c_int32, ctypes.c_int64, ctypes.c_uint8,
                                   ctypes.c_uint16, ctypes.c_float, ctypes.c_double)
    vp = ctypes.c_void_p
    sig = {
        "orc_num_threads": (ctypes.c_int, []),
        "orc_set_num_threads": (None, [ctypes.c_int]),
        "orc_code_row_bytes": (i64, [i32]),
        "orc_scale_row_bytes": (i64, [i32]),
        "orc_bytes_per_token": (i64, [i32]),
        "orc_page_bytes": (i64, [i32]),
        "orc_bf16_to_f32": (f32, [u16]),
        "orc_bf16_from_double": (u16, [f64]),
        "orc_e4m3_decode": (f64, [u8]),
        "orc_e4m3_encode": (u8, [f64]),
        "orc_ue8m0_exponent": (ctypes.c_int, [f32]),
        "orc_ue8m0_byte": (u8, [f32]),
        "orc_e2m1_decode": (f64, [u8]),
        "orc_e2m1_encode": (u8, [f32]),
        "orc_fp4_scale_code": (u8, [f32]),
        "orc_quant_row": (ctypes.c_int, [i32, vp, vp, vp]),
        "orc_rope_row": (ctypes.c_int, [vp, vp]),
        "orc_kv_store": (ctypes.c_int, [i32, vp, i64, vp, i64, vp, i64]),
        "orc_kv_store_rope": (ctypes.c_int, [i32, vp, i64, vp, i64, vp, vp, i64, vp, i64]),
        "orc_pool_rows": (ctypes.c_int, [vp, vp, i64, i32, i64, vp, vp]),
        "orc_kv_store_norm_rope": (ctypes.c_int, [i32, vp, i64, vp, i64, vp, f32, vp, vp, i64, vp, i64]),
        "orc_norm_row": (ctypes.c_int, [vp, vp, f32]),
        "orc_kv_compress_store": (ctypes.c_int,
                                  [i32, vp, i64, vp, vp, i64, i32, vp, vp, i64, vp, i64]),
        "orc_kv_dequant": (ctypes.c_int, [i32, vp, i64, vp, i64, vp]),
        "orc_kv_dequant_slots": (ctypes.c_int, [i32, vp, i64, vp, i64, vp]),
        "orc_translate_slots": (ctypes.c_int, [vp, i64, vp, i64, vp, i64]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    return L


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(a, dtype, name):
    if not isinstance(a, np.ndarray) or a.dtype != dtype or not a.flags.c_contiguous:
        raise TypeError(f"{name}: need a C-contiguous numpy array of {np.dtype(dtype)}")
    return a


def _ok(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what} returned {rc}")


# ------------------------------------------------------------------ scalar helpers
def num_threads():
    return int(lib().orc_num_threads())


def set_num_threads(n):
    lib().orc_set_num_threads(int(n))


def code_row_bytes(layout):
    return int(lib().orc_code_row_bytes(layout))


def scale_row_bytes(layout):
    return int(lib().orc_scale_row_bytes(layout))


def bytes_per_token(layout):
    return int(lib().orc_bytes_per_token(layout))


def page_bytes(layout):
    return int(lib().orc_page_bytes(layout))


def bf16_from_double(x):
    return int(lib().orc_bf16_from_double(float(x)))


def bf16_to_f32(h):
    return float(lib().orc_bf16_to_f32(int(h)))


def e4m3_encode(q):
    return int(lib().orc_e4m3_encode(float(q)))


def e4m3_decode(c):
    return float(lib().orc_e4m3_decode(int(c)))


def ue8m0_exponent(amax):
    return int(lib().orc_ue8m0_exponent(float(amax)))


def ue8m0_byte(amax):
    return int(lib().orc_ue8m0_byte(float(amax)))


def e2m1_encode(q):
    return int(lib().orc_e2m1_encode(float(q)))


def e2m1_decode(n):
    return float(lib().orc_e2m1_decode(int(n)))


def fp4_scale_code(amax):
    return int(lib().orc_fp4_scale_code(float(amax)))


# ------------------------------------------------------------------ row helpers
def quant_row(layout, v_bf16):
    """Quantise one 512-channel bf16 row (uint16 bits) -> (code row, scale row) bytes."""
    v = np.ascontiguousarray(v_bf16, dtype=np.uint16)
    assert v.shape == (HEAD,)
    code = np.zeros(code_row_bytes(layout), np.uint8)
    scale = np.zeros(scale_row_bytes(layout), np.uint8)
    _ok(lib().orc_quant_row(layout, _p(v), _p(code), _p(scale)), "quant_row")
    return code, scale


def rope_row(v_bf16, cos_sin_row):
    v = np.array(v_bf16, dtype=np.uint16, copy=True)
    cs = np.ascontiguousarray(cos_sin_row, dtype=np.float32)
    assert v.shape == (HEAD,) and cs.shape == (ROPE_DIM,)
    _ok(lib().orc_rope_row(_p(v), _p(cs)), "rope_row")
    return v


# ------------------------------------------------------------------ the path
def new_pool(layout, num_pages):
    return np.zeros((num_pages, page_bytes(layout)), np.uint8)


def _distinct_stored(slots, num_pages, pos=None, max_pos=None):
    """Two rows of one call stored at the same slot is a caller error (which row wins is
    unspecified), so a comparison on such inputs would not be defined: refuse them."""
    keep = (slots >= 0) & (slots < num_pages * PAGE_ROWS)
    if pos is not None:
        keep &= (pos >= 0) & (pos < max_pos)
    s = slots[keep]
    if np.unique(s).size != s.size:
        raise ValueError("duplicate slots among the rows of one call")


def kv_store(layout, pool, k_bf16, slots):
    _check(pool, np.uint8, "pool")
    _check(k_bf16, np.uint16, "k")
    _check(slots, np.int32, "slots")
    n = slots.shape[0]
    assert k_bf16.ndim == 2 and k_bf16.shape[0] >= n and k_bf16.shape[1] >= HEAD
    _distinct_stored(slots, pool.shape[0])
    _ok(lib().orc_kv_store(layout, _p(pool), pool.shape[0], _p(k_bf16), k_bf16.shape[1],
                           _p(slots), n), "kv_store")


def kv_store_rope(layout, pool, k_bf16, pos, cos_sin, slots):
    _check(pool, np.uint8, "pool")
    _check(k_bf16, np.uint16, "k")
    _check(pos, np.int32, "pos")
    _check(cos_sin, np.float32, "cos_sin")
    _check(slots, np.int32, "slots")
    n = slots.shape[0]
    assert pos.shape[0] == n and cos_sin.shape[1] == ROPE_DIM
    _distinct_stored(slots, pool.shape[0], pos, cos_sin.shape[0])
    _ok(lib().orc_kv_store_rope(layout, _p(pool), pool.shape[0], _p(k_bf16), k_bf16.shape[1],
                                _p(pos), _p(cos_sin), cos_sin.shape[0], _p(slots), n),
        "kv_store_rope")


def norm_row(v_bf16, weight_bf16, eps):
    v = np.array(v_bf16, dtype=np.uint16, copy=True)
    w = np.ascontiguousarray(weight_bf16, dtype=np.uint16)
    assert v.shape == (HEAD,) and w.shape == (HEAD,)
    _ok(lib().orc_norm_row(_p(v), _p(w), float(eps)), "norm_row")
    return v


def kv_store_norm_rope(layout, pool, k_bf16, weight_bf16, eps, pos, cos_sin, slots):
    _check(pool, np.uint8, "pool")
    _check(k_bf16, np.uint16, "k")
    _check(weight_bf16, np.uint16, "weight")
    _check(pos, np.int32, "pos")
    _check(cos_sin, np.float32, "cos_sin")
    _check(slots, np.int32, "slots")
    n = slots.shape[0]
    assert pos.shape[0] == n and weight_bf16.shape == (HEAD,)
    _distinct_stored(slots, pool.shape[0], pos, cos_sin.shape[0])
    _ok(lib().orc_kv_store_norm_rope(layout, _p(pool), pool.shape[0], _p(k_bf16), k_bf16.shape[1],
                                     _p(weight_bf16), float(eps), _p(pos), _p(cos_sin),
                                     cos_sin.shape[0], _p(slots), n), "kv_store_norm_rope")


def pool_rows(kv, score, ratio):
    """Pooled rows before RoPE: (float64 exact values, bf16 bits), each [R, 512]."""
    _check(kv, np.float32, "kv")
    _check(score, np.float32, "score")
    assert kv.shape == score.shape and kv.shape[0] % ratio == 0
    R = kv.shape[0] // ratio
    f64 = np.zeros((R, HEAD), np.float64)
    b16 = np.zeros((R, HEAD), np.uint16)
    _ok(lib().orc_pool_rows(_p(kv), _p(score), kv.shape[1], ratio, R, _p(f64), _p(b16)),
        "pool_rows")
    return f64, b16


def kv_compress_store(layout, pool, kv, score, ratio, pos, cos_sin, slots):
    _check(pool, np.uint8, "pool")
    _check(kv, np.float32, "kv")
    _check(score, np.float32, "score")
    _check(pos, np.int32, "pos")
    _check(cos_sin, np.float32, "cos_sin")
    _check(slots, np.int32, "slots")
    R = slots.shape[0]
    assert kv.shape == score.shape and kv.shape[0] >= R * ratio and pos.shape[0] == R
    _distinct_stored(slots, pool.shape[0], pos, cos_sin.shape[0])
    _ok(lib().orc_kv_compress_store(layout, _p(pool), pool.shape[0], _p(kv), _p(score),
                                    kv.shape[1], ratio, _p(pos), _p(cos_sin),
                                    cos_sin.shape[0], _p(slots), R), "kv_compress_store")


def kv_dequant(layout, pool, page_ids, out=None):
    _check(pool, np.uint8, "pool")
    _check(page_ids, np.int32, "page_ids")
    P = page_ids.shape[0]
    if out is None:
        out = np.zeros((P * PAGE_ROWS, HEAD), np.uint16)
    _check(out, np.uint16, "out")
    _ok(lib().orc_kv_dequant(layout, _p(pool), pool.shape[0], _p(page_ids), P, _p(out)),
        "kv_dequant")
    return out


def kv_dequant_slots(layout, pool, slots, out=None):
    _check(pool, np.uint8, "pool")
    _check(slots, np.int32, "slots")
    n = slots.shape[0]
    if out is None:
        out = np.zeros((n, HEAD), np.uint16)
    _check(out, np.uint16, "out")
    _ok(lib().orc_kv_dequant_slots(layout, _p(pool), pool.shape[0], _p(slots), n, _p(out)),
        "kv_dequant_slots")
    return out


def translate_slots(table, full, cap):
    """Returns (status, out[cap]); status -4 means n > cap and nothing was written."""
    _check(table, np.int32, "table")
    _check(full, np.int32, "full")
    out = np.full(cap, 0x5A5A5A5A, np.int32)
    rc = lib().orc_translate_slots(_p(table), table.shape[0], _p(full), full.shape[0],
                                   _p(out), cap)
    return int(rc), out
