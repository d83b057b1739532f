"""MI355X-native KV-cache compress -> quantise -> paged store.

Thin Python binding of libkvq.so (declared in include/kvq.h): argument marshalling only.
Every step of the path runs in the library's HIP kernels; torch provides device memory
and the current stream.  The library must have been built (``__graft_entry__.build()``
or ``python -m quantized_paged_kv_compress_amd._build``); importing the ops without it
raises instead of falling back to anything else.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "V41", "V41_FP4", "KVQError", "load_library", "profile_next_launch", "bytes_per_token", "page_bytes",
    "code_row_bytes", "scale_row_bytes", "new_pool", "kv_store", "kv_store_rope", "kv_store_rope_layers", "kv_store_norm_rope",
    "kv_compress_store", "kv_compress_store_translate", "kv_compress_state_update", "new_compress_state", "compress_state_bytes", "kv_dequant", "kv_dequant_slots", "kv_translate_slots", "SUPPORTED_RATIOS",
]

V41 = 1
V41_FP4 = 2
HEAD_DIM = 512
ROPE_DIM = 64
PAGE_ROWS = 64
SUPPORTED_RATIOS = (1, 2, 4, 8, 16, 32, 64, 128)

KVQ_OK, KVQ_EINVAL, KVQ_ELAYOUT, KVQ_ERATIO, KVQ_ECAPACITY, KVQ_ELAUNCH = 0, -1, -2, -3, -4, -5

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkvq.so")
_lib = None


class KVQError(RuntimeError):
    def __init__(self, fn: str, status: int, message: str):
        super().__init__(f"{fn}: {message} (status {status})")
        self.status = status


def load_library() -> ctypes.CDLL:
    """Load libkvq.so; raises if it has not been built, or if it was built from other
    sources than the ones next to it (its kvq_build_id differs from their hash)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m quantized_paged_kv_compress_amd._build`")
    from . import _build
    L = ctypes.CDLL(LIB_PATH)
    L.kvq_build_id.restype = ctypes.c_char_p
    L.kvq_build_id.argtypes = []
    built, want = L.kvq_build_id().decode(), _build.source_hash()
    if built != want:
        raise ImportError(f"{LIB_PATH} is stale (built from sources {built[:12]}, current {want[:12]}): "
                          "rebuild it with `python -m quantized_paged_kv_compress_amd._build`")
    i32, i64, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
    L.kvq_status_string.restype = ctypes.c_char_p
    L.kvq_status_string.argtypes = [ctypes.c_int]
    L.kvq_compress_state_bytes.restype = i64
    L.kvq_compress_state_bytes.argtypes = []
    L.kvq_profile_next_launch.restype = ctypes.c_int
    L.kvq_profile_next_launch.argtypes = [vp, vp]
    for q in ("kvq_bytes_per_token", "kvq_page_bytes", "kvq_code_row_bytes", "kvq_scale_row_bytes"):
        getattr(L, q).restype = i64
        getattr(L, q).argtypes = [i32]
    sigs = {
        "kv_store": [i32, vp, i64, vp, i64, vp, i64, vp],
        "kv_store_rope": [i32, vp, i64, vp, i64, vp, vp, i64, vp, i64, vp],
        "kv_store_norm_rope": [i32, vp, i64, vp, i64, vp, ctypes.c_float, vp, vp, i64, vp, i64, vp],
        "kv_store_rope_layers": [i32, vp, i64, vp, i64, i32, vp, vp, i64, vp, i64, vp],
        "kv_compress_store": [i32, vp, i64, vp, vp, i64, i32, vp, vp, i64, vp, i64, vp],
        "kv_compress_store_translate": [i32, vp, i64, vp, vp, i64, i32, vp, vp, i64, vp, i64, vp, vp, i64,
                                        i64, vp],
        "kv_compress_state_update": [i32, vp, i64, vp, vp, i64, i32, vp, vp, vp, i64, vp, vp, i64, vp,
                                     i64, vp],
        "kv_dequant": [i32, vp, i64, vp, i64, vp, vp],
        "kv_dequant_slots": [i32, vp, i64, vp, i64, vp, vp],
        "kv_translate_slots": [vp, i64, vp, i64, vp, i64, vp],
    }
    for name, args in sigs.items():
        fn = getattr(L, name)
        fn.restype = ctypes.c_int
        fn.argtypes = args
    _lib = L
    return L


def profile_next_launch(start_event, stop_event):
    """Make the next kernel launched from this thread record the two torch.cuda.Event
    objects at its own start and end (they must have been recorded once already, so their
    handles exist)."""
    handles = (start_event.cuda_event, stop_event.cuda_event)
    if not all(handles):
        raise ValueError("profile_next_launch: record each event once before arming it")
    load_library().kvq_profile_next_launch(*handles)


def _raise(fn: str, status: int):
    if status != KVQ_OK:
        msg = load_library().kvq_status_string(status).decode()
        raise KVQError(fn, status, msg)


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _ptr(t: torch.Tensor | None):
    return None if t is None else t.data_ptr()


def _dev(t: torch.Tensor, name: str, dtypes) -> torch.Tensor:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name}: expected a CUDA tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not in {dtypes}")
    return t


def _vec(t: torch.Tensor, name: str, dtypes=(torch.int32,)) -> torch.Tensor:
    """A device array passed by pointer: elements must be contiguous."""
    _dev(t, name, dtypes)
    if not t.is_contiguous():
        raise ValueError(f"{name}: need a contiguous tensor (pass .contiguous())")
    return t


def _rows(t: torch.Tensor, name: str) -> int:
    """Row stride (elements) of a [rows, >=512] tensor whose channels are contiguous."""
    if t.dim() != 2 or t.shape[1] < HEAD_DIM or t.stride(1) != 1:
        raise ValueError(f"{name}: need a [rows, >=512] tensor with contiguous channels")
    return t.stride(0)


# ------------------------------------------------------------------ layout queries
def bytes_per_token(layout: int) -> int:
    return int(load_library().kvq_bytes_per_token(layout))


def page_bytes(layout: int) -> int:
    return int(load_library().kvq_page_bytes(layout))


def code_row_bytes(layout: int) -> int:
    return int(load_library().kvq_code_row_bytes(layout))


def scale_row_bytes(layout: int) -> int:
    return int(load_library().kvq_scale_row_bytes(layout))


def new_pool(layout: int, num_pages: int, device="cuda") -> torch.Tensor:
    """A zeroed pool: uint8 [num_pages, page_bytes(layout)]."""
    pb = page_bytes(layout)
    if pb < 0:
        _raise("new_pool", pb)
    return torch.zeros((num_pages, pb), dtype=torch.uint8, device=device)


def _pool(pool: torch.Tensor, layout: int) -> int:
    _dev(pool, "pool", (torch.uint8,))
    if not pool.is_contiguous() or pool.dim() != 2 or pool.shape[1] != page_bytes(layout):
        raise ValueError("pool: need a contiguous uint8 [num_pages, page_bytes(layout)] tensor")
    return pool.shape[0]


_BF16 = (torch.bfloat16, torch.int16, torch.uint16)
_I32 = (torch.int32,)
_F32 = (torch.float32,)


# ------------------------------------------------------------------ the path
def kv_store(pool, layout, k, slots, stream=None):
    """Quantise bf16 rows k[i, :512] into pool slots slots[i]."""
    num_pages = _pool(pool, layout)
    ld = _rows(_dev(k, "k", _BF16), "k")
    _vec(slots, "slots")
    n = slots.numel()
    if k.shape[0] < n:
        raise ValueError("k has fewer rows than slots")
    _raise("kv_store", load_library().kv_store(layout, _ptr(pool), num_pages, _ptr(k), ld,
                                               _ptr(slots), n, _stream(stream)))


def kv_store_rope(pool, layout, k, pos, cos_sin, slots, stream=None):
    """RoPE on the last 64 channels at pos[i], then quantise into slots[i]."""
    num_pages = _pool(pool, layout)
    ld = _rows(_dev(k, "k", _BF16), "k")
    _vec(pos, "pos")
    _vec(slots, "slots")
    _dev(cos_sin, "cos_sin", _F32)
    if not cos_sin.is_contiguous() or cos_sin.dim() != 2 or cos_sin.shape[1] != ROPE_DIM:
        raise ValueError("cos_sin: need a contiguous fp32 [max_pos, 64] tensor")
    n = slots.numel()
    if k.shape[0] < n or pos.numel() != n:
        raise ValueError("k / pos / slots sizes disagree")
    _raise("kv_store_rope", load_library().kv_store_rope(
        layout, _ptr(pool), num_pages, _ptr(k), ld, _ptr(pos), _ptr(cos_sin), cos_sin.shape[0],
        _ptr(slots), n, _stream(stream)))


def kv_store_rope_layers(pools, layout, ks, pos, cos_sin, slots, stream=None):
    """kv_store_rope for every layer l: row i of ks[l] is rotated at pos[i] and stored at
    slots[i] of pools[l].  pools and ks are equal-length sequences; every K tensor has the
    same row stride.  One launch per 64 layers."""
    pools, ks = list(pools), list(ks)
    if not pools or len(pools) != len(ks):
        raise ValueError("pools and ks: one pool and one K tensor per layer")
    num_pages = _pool(pools[0], layout)
    for p in pools[1:]:
        if _pool(p, layout) != num_pages:
            raise ValueError("pools: every layer's pool has the same number of pages")
    ld = _rows(_dev(ks[0], "ks[0]", _BF16), "ks[0]")
    for j, k in enumerate(ks[1:], 1):
        if _rows(_dev(k, f"ks[{j}]", _BF16), f"ks[{j}]") != ld:
            raise ValueError("ks: every layer's K has the same row stride")
    _vec(pos, "pos")
    _vec(slots, "slots")
    _dev(cos_sin, "cos_sin", _F32)
    if not cos_sin.is_contiguous() or cos_sin.dim() != 2 or cos_sin.shape[1] != ROPE_DIM:
        raise ValueError("cos_sin: need a contiguous fp32 [max_pos, 64] tensor")
    n = slots.numel()
    if pos.numel() != n or any(k.shape[0] < n for k in ks):
        raise ValueError("ks / pos / slots sizes disagree")
    L = len(pools)
    pool_ptrs = (ctypes.c_void_p * L)(*[p.data_ptr() for p in pools])
    k_ptrs = (ctypes.c_void_p * L)(*[k.data_ptr() for k in ks])
    _raise("kv_store_rope_layers", load_library().kv_store_rope_layers(
        layout, pool_ptrs, num_pages, k_ptrs, ld, L, _ptr(pos), _ptr(cos_sin), cos_sin.shape[0], _ptr(slots), n,
        _stream(stream)))


def kv_store_norm_rope(pool, layout, k, weight, eps, pos, cos_sin, slots, stream=None):
    """RMS-normalise each row with a per-channel bf16 weight, RoPE at pos[i], quantise into
    slots[i]."""
    num_pages = _pool(pool, layout)
    ld = _rows(_dev(k, "k", _BF16), "k")
    _dev(weight, "weight", _BF16)
    if not weight.is_contiguous() or weight.numel() != HEAD_DIM:
        raise ValueError("weight: need a contiguous bf16 [512] tensor")
    _vec(pos, "pos")
    _vec(slots, "slots")
    _dev(cos_sin, "cos_sin", _F32)
    if not cos_sin.is_contiguous() or cos_sin.dim() != 2 or cos_sin.shape[1] != ROPE_DIM:
        raise ValueError("cos_sin: need a contiguous fp32 [max_pos, 64] tensor")
    n = slots.numel()
    if k.shape[0] < n or pos.numel() != n:
        raise ValueError("k / pos / slots sizes disagree")
    _raise("kv_store_norm_rope", load_library().kv_store_norm_rope(
        layout, _ptr(pool), num_pages, _ptr(k), ld, _ptr(weight), float(eps), _ptr(pos),
        _ptr(cos_sin), cos_sin.shape[0], _ptr(slots), n, _stream(stream)))


def kv_compress_store(pool, layout, kv, score, ratio, pos, cos_sin, slots, stream=None):
    """Pool each ratio-row window of kv by the per-channel softmax of score, RoPE, quantise
    and store at slots[i].  kv and score: fp32 [R*ratio, >=512] with equal strides."""
    num_pages = _pool(pool, layout)
    ld = _rows(_dev(kv, "kv", _F32), "kv")
    if score is not None:
        if _rows(_dev(score, "score", _F32), "score") != ld or score.shape[0] != kv.shape[0]:
            raise ValueError("score must match kv in shape and stride")
    _vec(pos, "pos")
    _vec(slots, "slots")
    _dev(cos_sin, "cos_sin", _F32)
    if not cos_sin.is_contiguous() or cos_sin.dim() != 2 or cos_sin.shape[1] != ROPE_DIM:
        raise ValueError("cos_sin: need a contiguous fp32 [max_pos, 64] tensor")
    R = slots.numel()
    if pos.numel() != R or kv.shape[0] < R * ratio:
        raise ValueError("kv / pos / slots sizes disagree")
    _raise("kv_compress_store", load_library().kv_compress_store(
        layout, _ptr(pool), num_pages, _ptr(kv), _ptr(score), ld, ratio, _ptr(pos),
        _ptr(cos_sin), cos_sin.shape[0], _ptr(slots), R, _stream(stream)))


def kv_compress_store_translate(pool, layout, kv, score, ratio, pos, cos_sin, table, full_loc, out,
                                stream=None):
    """kv_translate_slots(table, full_loc, out) and kv_compress_store(..., slots=out[:R]) in
    one launch: row i is stored at table[full_loc[i]], which is also left in out[i]
    (out[R:] zeroed).  Returns out[:R], or None when full_loc is longer than out (nothing
    is written)."""
    num_pages = _pool(pool, layout)
    ld = _rows(_dev(kv, "kv", _F32), "kv")
    if score is not None:
        if _rows(_dev(score, "score", _F32), "score") != ld or score.shape[0] != kv.shape[0]:
            raise ValueError("score must match kv in shape and stride")
    _vec(pos, "pos")
    _vec(table, "table")
    _vec(full_loc, "full_loc")
    _vec(out, "out")
    _dev(cos_sin, "cos_sin", _F32)
    if not cos_sin.is_contiguous() or cos_sin.dim() != 2 or cos_sin.shape[1] != ROPE_DIM:
        raise ValueError("cos_sin: need a contiguous fp32 [max_pos, 64] tensor")
    R = full_loc.numel()
    if pos.numel() != R or kv.shape[0] < R * ratio:
        raise ValueError("kv / pos / full_loc sizes disagree")
    st = load_library().kv_compress_store_translate(
        layout, _ptr(pool), num_pages, _ptr(kv), _ptr(score), ld, ratio, _ptr(pos), _ptr(cos_sin),
        cos_sin.shape[0], _ptr(table), table.numel(), _ptr(full_loc), _ptr(out), out.numel(), R,
        _stream(stream))
    if st == KVQ_ECAPACITY:
        return None
    _raise("kv_compress_store_translate", st)
    return out[:R]


def compress_state_bytes() -> int:
    """Bytes of one sequence's decode-step compressor state."""
    return int(load_library().kvq_compress_state_bytes())


def new_compress_state(num_states: int, device="cuda"):
    """An empty decode-step compressor state: (uint8 [num_states, compress_state_bytes()]
    opaque states, int32 counts)."""
    return (torch.zeros((num_states, compress_state_bytes()), dtype=torch.uint8, device=device),
            torch.zeros(num_states, dtype=torch.int32, device=device))


def kv_compress_state_update(pool, layout, state, count, ratio, state_ids, kv, score, pos,
                             cos_sin, slots, stream=None):
    """Fold row j of kv/score into state state_ids[j]; a window completed by row j is
    stored at slots[j] with RoPE at pos[j].  At most one row per state per call."""
    num_pages = _pool(pool, layout)
    _dev(state, "state", (torch.uint8,))
    _vec(count, "count")
    if not state.is_contiguous() or state.dim() != 2 or state.shape[1] != compress_state_bytes():
        raise ValueError("state: need a contiguous uint8 [num_states, compress_state_bytes()] tensor")
    if count.numel() != state.shape[0]:
        raise ValueError("count: one int32 per state")
    ld = _rows(_dev(kv, "kv", _F32), "kv")
    if _rows(_dev(score, "score", _F32), "score") != ld or score.shape[0] != kv.shape[0]:
        raise ValueError("score must match kv in shape and stride")
    for t, nm in ((state_ids, "state_ids"), (pos, "pos"), (slots, "slots")):
        _vec(t, nm)
    _dev(cos_sin, "cos_sin", _F32)
    if not cos_sin.is_contiguous() or cos_sin.dim() != 2 or cos_sin.shape[1] != ROPE_DIM:
        raise ValueError("cos_sin: need a contiguous fp32 [max_pos, 64] tensor")
    n = state_ids.numel()
    if kv.shape[0] < n or pos.numel() != n or slots.numel() != n:
        raise ValueError("kv / state_ids / pos / slots sizes disagree")
    _raise("kv_compress_state_update", load_library().kv_compress_state_update(
        layout, _ptr(pool), num_pages, _ptr(state), _ptr(count), state.shape[0], ratio,
        _ptr(state_ids), _ptr(kv), _ptr(score), ld, _ptr(pos), _ptr(cos_sin), cos_sin.shape[0],
        _ptr(slots), n, _stream(stream)))


def kv_dequant(pool, layout, page_ids, out=None, stream=None):
    """bf16 [P*64, 512] workspace of the listed pages (list order)."""
    num_pages = _pool(pool, layout)
    _vec(page_ids, "page_ids")
    P = page_ids.numel()
    if out is None:
        out = torch.empty((P * PAGE_ROWS, HEAD_DIM), dtype=torch.bfloat16, device=pool.device)
    _dev(out, "out", _BF16)
    if not out.is_contiguous() or out.numel() < P * PAGE_ROWS * HEAD_DIM:
        raise ValueError("out: need a contiguous [P*64, 512] bf16 tensor")
    _raise("kv_dequant", load_library().kv_dequant(layout, _ptr(pool), num_pages, _ptr(page_ids),
                                                   P, _ptr(out), _stream(stream)))
    return out


def kv_dequant_slots(pool, layout, slots, out=None, stream=None):
    """bf16 [n, 512]: the dequantised rows at slots[i] (rows of out-of-pool slots untouched)."""
    num_pages = _pool(pool, layout)
    _vec(slots, "slots")
    n = slots.numel()
    if out is None:
        out = torch.empty((n, HEAD_DIM), dtype=torch.bfloat16, device=pool.device)
    _dev(out, "out", _BF16)
    if not out.is_contiguous() or out.numel() < n * HEAD_DIM:
        raise ValueError("out: need a contiguous [n, 512] bf16 tensor")
    _raise("kv_dequant_slots", load_library().kv_dequant_slots(layout, _ptr(pool), num_pages,
                                                               _ptr(slots), n, _ptr(out), _stream(stream)))
    return out


def kv_translate_slots(table, full_loc, out, stream=None):
    """Fill out[:n] with table[full_loc] (-1 outside the table) and zero out[n:].

    Returns out[:n], or None when full_loc is longer than out (nothing is written; the
    caller then translates into a buffer of its own, still once per step)."""
    _vec(table, "table")
    _vec(full_loc, "full_loc")
    _vec(out, "out")
    n = full_loc.numel()
    st = load_library().kv_translate_slots(_ptr(table), table.numel(), _ptr(full_loc), n,
                                           _ptr(out), out.numel(), _stream(stream))
    if st == KVQ_ECAPACITY:
        return None
    _raise("kv_translate_slots", st)
    return out[:n]
