"""Seeded synthetic inputs for the compress / quantise / paged-store path.

This module only draws inputs; it holds none of the method's arithmetic.  Both the HIP
library's tests and the CPU oracle's tests take their inputs from here.

Large normal tensors are drawn in fixed chunks of ``CHUNK`` elements; chunk ``c`` of
stream ``s`` under seed ``seed`` comes from ``PCG64(SeedSequence([seed, s, c]))``.  Any
row range can therefore be regenerated on its own (the full-size parity tests rebuild
only the windows they sample), and the values do not depend on the thread count.

Workloads (all synthetic; shapes and distributions of the pages' workloads):

* ``store_v41``     64 bf16 rows x 512, N(0,1) times a per-channel LogUniform[0.1,10]
                    scale; 16-page pool; distinct random slots.
* ``store_rope``    512 bf16 rows x 512, N(0,1); positions U[0,65536); 4096-page pool.
* ``c4a``           16384 output rows, ratio 4: fp32 kv N(0,1) and scores N(0, sd 2),
                    [65536, 512] each; positions U[0,65536); 4096-page pool.
* ``c128a``         as c4a with ratio 128: [2097152, 512] each (4 GiB per tensor).
* ``mixed_fp4``     ragged batch of 256 sequences (1 new token with p = 0.8, else
                    U[64, 2048]); the ratio-4 windows completed this step; full-pool
                    slots, a full -> SWA int32 table, and the pages to dequantise.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

HEAD = 512
ROPE_DIM = 64
PAGE_ROWS = 64
MAX_POS = 65536
ROPE_THETA = 10000.0
CHUNK = 1 << 20  # elements per generator chunk (2048 rows of 512)

# stream ids inside one seed
S_K, S_KV, S_SCORE, S_SCALE = 1, 2, 3, 4


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _fill_chunk(seed: int, stream: int, c: int, out: np.ndarray, lo: int, hi: int) -> None:
    """Write elements [lo, hi) of chunk c (chunk-relative offsets) into out."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, stream, c])))
    if lo == 0 and hi == CHUNK and out.shape[0] == CHUNK:
        g.standard_normal(out=out, dtype=np.float32)
        return
    buf = g.standard_normal(hi, dtype=np.float32)
    out[:] = buf[lo:hi]


def normal_f32(seed: int, stream: int, start: int, count: int, sd: float = 1.0,
               out: np.ndarray | None = None) -> np.ndarray:
    """Elements [start, start+count) of the standard-normal stream, times sd (fp32)."""
    if out is None:
        out = np.empty(count, np.float32)
    assert out.shape == (count,) and out.dtype == np.float32
    jobs = []
    e = start
    while e < start + count:
        c = e // CHUNK
        lo = e - c * CHUNK
        hi = min(CHUNK, start + count - c * CHUNK)
        jobs.append((c, lo, hi, e - start))
        e = c * CHUNK + hi
    def run(job):
        c, lo, hi, off = job
        _fill_chunk(seed, stream, c, out[off:off + hi - lo], lo, hi)
    if len(jobs) == 1:
        run(jobs[0])
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(run, jobs))
    if sd != 1.0:
        np.multiply(out, np.float32(sd), out=out)
    return out


def normal_rows(seed: int, stream: int, row0: int, nrows: int, sd: float = 1.0,
                width: int = HEAD) -> np.ndarray:
    """Rows [row0, row0+nrows) of a [*, width] fp32 tensor drawn from the stream."""
    return normal_f32(seed, stream, row0 * width, nrows * width, sd).reshape(nrows, width)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 (round to nearest even, via torch) as uint16 bit patterns."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def rope_cos_sin(max_pos: int = MAX_POS, theta: float = ROPE_THETA,
                 rot_dim: int = ROPE_DIM) -> np.ndarray:
    """Caller-side RoPE table [max_pos, rot_dim] fp32: cos of the angles in the first half,
    sin in the second; angle(p, i) = p * theta^(-2i/rot_dim); built in float64."""
    half = rot_dim // 2
    inv = theta ** (-np.arange(half, dtype=np.float64) * 2.0 / rot_dim)
    ang = np.arange(max_pos, dtype=np.float64)[:, None] * inv[None, :]
    return np.concatenate([np.cos(ang), np.sin(ang)], axis=1).astype(np.float32)


def distinct_slots(rng: np.random.Generator, n: int, lo: int, hi: int) -> np.ndarray:
    """n distinct int32 slots drawn uniformly from [lo, hi), in random order."""
    return (rng.choice(hi - lo, size=n, replace=False) + lo).astype(np.int32)


# ---------------------------------------------------------------------------- configs
def store_v41(seed: int = 1, n: int = 64, num_pages: int = 16) -> dict:
    rng = np.random.default_rng(seed)
    sigma = np.exp(rng.uniform(np.log(0.1), np.log(10.0), HEAD)).astype(np.float32)
    k = normal_rows(seed, S_K, 0, n) * sigma[None, :]
    return dict(k=bf16_bits(k), slots=distinct_slots(rng, n, PAGE_ROWS, num_pages * PAGE_ROWS),
                num_pages=num_pages)


def store_rope(seed: int = 2, n: int = 512, num_pages: int = 4096) -> dict:
    rng = np.random.default_rng(seed)
    k = normal_rows(seed, S_K, 0, n)
    pos = rng.integers(0, MAX_POS, n).astype(np.int32)
    return dict(k=bf16_bits(k), pos=pos,
                slots=distinct_slots(rng, n, PAGE_ROWS, num_pages * PAGE_ROWS),
                num_pages=num_pages)


def compressor_meta(seed: int, R: int, num_pages: int = 4096) -> dict:
    """Positions and slots of R compressed rows (c4a / c128a)."""
    rng = np.random.default_rng(seed)
    pos = rng.integers(0, MAX_POS, R).astype(np.int32)
    slots = distinct_slots(rng, R, PAGE_ROWS, num_pages * PAGE_ROWS)
    return dict(pos=pos, slots=slots, num_pages=num_pages)


def compressor_window(seed: int, ratio: int, i0: int, nrows_out: int) -> tuple:
    """kv and score rows of output rows [i0, i0+nrows_out): [nrows_out*ratio, 512] each."""
    kv = normal_rows(seed, S_KV, i0 * ratio, nrows_out * ratio)
    sc = normal_rows(seed, S_SCORE, i0 * ratio, nrows_out * ratio, sd=2.0)
    return kv, sc


def compressor(seed: int, ratio: int, R: int, num_pages: int = 4096) -> dict:
    d = compressor_meta(seed, R, num_pages)
    d["kv"], d["score"] = compressor_window(seed, ratio, 0, R)
    d["ratio"] = ratio
    return d


def c4a(seed: int = 3, R: int = 16384) -> dict:
    return compressor(seed, 4, R)


def c128a(seed: int = 4, R: int = 16384) -> dict:
    return compressor(seed, 128, R)


def mixed_fp4(seed: int = 5, n_seq: int = 256, ratio: int = 4, num_pages: int = 8192,
              cap: int = 65536, with_rows: bool = True) -> dict:
    """Mixed decode/prefill step.

    Sequence s has `prior` cached tokens and `new` tokens this step; the ratio-4 windows
    w with prior//4 <= w < (prior+new)//4 complete now and are compressed (their rows are
    supplied whole).  Full slot of window w of sequence s: (s*256 + w//64)*64 + w%64.
    The full -> SWA table sends each touched full page to a distinct physical page in
    [1, num_pages) with the row offset kept; every other entry is 0.
    """
    rng = np.random.default_rng(seed)
    full, pos = [], []
    for s in range(n_seq):
        new = 1 if rng.random() < 0.8 else int(rng.integers(64, 2049))
        prior = int(rng.integers(0, MAX_POS - new + 1))
        w = np.arange(prior // ratio, (prior + new) // ratio, dtype=np.int64)
        full.append((s * 256 + (w >> 6)) * PAGE_ROWS + (w & 63))
        pos.append(w * ratio)
    full = np.concatenate(full).astype(np.int32)
    pos = np.concatenate(pos).astype(np.int32)
    R = full.shape[0]
    table_len = n_seq * 256 * PAGE_ROWS
    table = np.zeros(table_len, np.int32)
    fpages = np.unique(full >> 6)
    phys = rng.choice(np.arange(1, num_pages), size=fpages.shape[0], replace=False)
    for fp, pp in zip(fpages, phys):
        table[fp * PAGE_ROWS:(fp + 1) * PAGE_ROWS] = pp * PAGE_ROWS + np.arange(PAGE_ROWS)
    swa_pages = np.unique(phys).astype(np.int32)  # pages touched, ascending
    d = dict(full=full, pos=pos, table=table, R=R, ratio=ratio, num_pages=num_pages,
             cap=cap, page_ids=swa_pages)
    if with_rows:
        d["kv"], d["score"] = compressor_window(seed, ratio, 0, R)
    return d
