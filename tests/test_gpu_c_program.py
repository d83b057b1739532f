"""The boundary end to end from C: a C99 program built with gcc (no Python and no torch in
it) allocates device memory through the HIP runtime, calls kv_store_rope,
kv_compress_store_translate (including a call refused for capacity) and kv_dequant through
include/kvq.h on the null stream, and writes the results back.  They are compared with
the oracle's: the store pool byte for byte, the translated slots exactly, the compressed
pool by the compressor rule, and the dequantised pages where the pools agree."""
import os
import shutil
import subprocess

import numpy as np
import pytest

from helpers import FP4, V41, check_step_dequant, compare_compressed, gpu_lib, untouched_equal
from quantized_paged_kv_compress_amd import workloads as wl

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

PROGRAM = r"""
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <hip/hip_runtime_api.h>
#include "kvq.h"

static const char* dir;

static void* load(const char* name, size_t bytes) {
    char path[4096];
    snprintf(path, sizeof path, "%s/%s", dir, name);
    FILE* f = fopen(path, "rb");
    void* p = malloc(bytes ? bytes : 1);
    if (!f || !p || fread(p, 1, bytes, f) != bytes) { fprintf(stderr, "cannot read %s\n", path); exit(2); }
    fclose(f);
    return p;
}

static void save(const char* name, const void* p, size_t bytes) {
    char path[4096];
    snprintf(path, sizeof path, "%s/%s", dir, name);
    FILE* f = fopen(path, "wb");
    if (!f || fwrite(p, 1, bytes, f) != bytes) { fprintf(stderr, "cannot write %s\n", path); exit(2); }
    fclose(f);
}

static void check(hipError_t e, const char* what) {
    if (e != hipSuccess) { fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e)); exit(3); }
}

static void* dev_copy(const void* h, size_t bytes) {
    void* d = NULL;
    check(hipMalloc(&d, bytes ? bytes : 16), "hipMalloc");
    if (bytes) check(hipMemcpy(d, h, bytes, hipMemcpyHostToDevice), "hipMemcpy to device");
    return d;
}

int main(int argc, char** argv) {
    long long n, R, num_pages, max_pos, cap, table_len, P;
    int bad = 0, st;
    if (argc != 2) return 2;
    dir = argv[1];
    {
        char path[4096];
        FILE* f;
        snprintf(path, sizeof path, "%s/meta.txt", dir);
        f = fopen(path, "r");
        if (!f || fscanf(f, "%lld %lld %lld %lld %lld %lld %lld", &n, &R, &num_pages, &max_pos, &cap,
                         &table_len, &P) != 7) return 2;
        fclose(f);
    }
    {
        const size_t pb1 = (size_t)kvq_page_bytes(KVQ_LAYOUT_V41), pb2 = (size_t)kvq_page_bytes(KVQ_LAYOUT_V41_FP4);
        void* k = dev_copy(load("k.bin", (size_t)n * 512 * 2), (size_t)n * 512 * 2);
        void* pos = dev_copy(load("pos.bin", (size_t)n * 4), (size_t)n * 4);
        void* slots = dev_copy(load("slots.bin", (size_t)n * 4), (size_t)n * 4);
        void* cs = dev_copy(load("cs.bin", (size_t)max_pos * 64 * 4), (size_t)max_pos * 64 * 4);
        void* kv = dev_copy(load("kv.bin", (size_t)R * 4 * 512 * 4), (size_t)R * 4 * 512 * 4);
        void* sc = dev_copy(load("sc.bin", (size_t)R * 4 * 512 * 4), (size_t)R * 4 * 512 * 4);
        void* pos_c = dev_copy(load("pos_c.bin", (size_t)R * 4), (size_t)R * 4);
        void* table = dev_copy(load("table.bin", (size_t)table_len * 4), (size_t)table_len * 4);
        void* full = dev_copy(load("full.bin", (size_t)R * 4), (size_t)R * 4);
        void* pages = dev_copy(load("pages.bin", (size_t)P * 4), (size_t)P * 4);
        void *pool1 = NULL, *pool2 = NULL, *loc = NULL, *ws = NULL;
        void* h;
        check(hipMalloc(&pool1, (size_t)num_pages * pb1), "hipMalloc pool1");
        check(hipMalloc(&pool2, (size_t)num_pages * pb2), "hipMalloc pool2");
        check(hipMalloc(&loc, (size_t)cap * 4), "hipMalloc loc");
        check(hipMalloc(&ws, (size_t)P * 64 * 512 * 2), "hipMalloc ws");
        check(hipMemset(pool1, 0, (size_t)num_pages * pb1), "hipMemset");
        check(hipMemset(pool2, 0, (size_t)num_pages * pb2), "hipMemset");
        check(hipDeviceSynchronize(), "sync");

        st = kv_store_rope(KVQ_LAYOUT_V41, pool1, num_pages, (const uint16_t*)k, 512, (const int32_t*)pos,
                           (const float*)cs, max_pos, (const int32_t*)slots, n, NULL);
        if (st != KVQ_OK) { fprintf(stderr, "kv_store_rope: %s\n", kvq_status_string(st)); bad |= 1; }
        /* more rows than the buffer holds: refused, nothing enqueued */
        st = kv_compress_store_translate(KVQ_LAYOUT_V41_FP4, pool2, num_pages, (const float*)kv,
                                         (const float*)sc, 512, 4, (const int32_t*)pos_c, (const float*)cs,
                                         max_pos, (const int32_t*)table, table_len, (const int32_t*)full,
                                         (int32_t*)loc, R - 1, R, NULL);
        if (st != KVQ_ECAPACITY) { fprintf(stderr, "capacity refusal: %s\n", kvq_status_string(st)); bad |= 2; }
        st = kv_compress_store_translate(KVQ_LAYOUT_V41_FP4, pool2, num_pages, (const float*)kv,
                                         (const float*)sc, 512, 4, (const int32_t*)pos_c, (const float*)cs,
                                         max_pos, (const int32_t*)table, table_len, (const int32_t*)full,
                                         (int32_t*)loc, cap, R, NULL);
        if (st != KVQ_OK) { fprintf(stderr, "kv_compress_store_translate: %s\n", kvq_status_string(st)); bad |= 4; }
        st = kv_dequant(KVQ_LAYOUT_V41_FP4, pool2, num_pages, (const int32_t*)pages, P, (uint16_t*)ws, NULL);
        if (st != KVQ_OK) { fprintf(stderr, "kv_dequant: %s\n", kvq_status_string(st)); bad |= 8; }
        check(hipDeviceSynchronize(), "sync");

        h = malloc((size_t)num_pages * pb1 + (size_t)P * 64 * 512 * 2 + (size_t)cap * 4);
        if (!h) return 2;
        check(hipMemcpy(h, pool1, (size_t)num_pages * pb1, hipMemcpyDeviceToHost), "copy pool1");
        save("pool1.bin", h, (size_t)num_pages * pb1);
        check(hipMemcpy(h, pool2, (size_t)num_pages * pb2, hipMemcpyDeviceToHost), "copy pool2");
        save("pool2.bin", h, (size_t)num_pages * pb2);
        check(hipMemcpy(h, loc, (size_t)cap * 4, hipMemcpyDeviceToHost), "copy loc");
        save("loc.bin", h, (size_t)cap * 4);
        check(hipMemcpy(h, ws, (size_t)P * 64 * 512 * 2, hipMemcpyDeviceToHost), "copy ws");
        save("ws.bin", h, (size_t)P * 64 * 512 * 2);
    }
    printf("kvq C program on the GPU: %s (%d)\n", bad ? "FAILED" : "ok", bad);
    return bad != 0;
}
"""


def test_c_program_drives_the_path(tmp_path, orc):
    gcc = shutil.which("gcc")
    if gcc is None or not os.path.exists(os.path.join(ROCM, "include", "hip", "hip_runtime_api.h")):
        pytest.skip("no gcc or HIP headers")
    kvq = gpu_lib()   # skips without a GPU
    rng = np.random.default_rng(77)
    n, R, num_pages, max_pos, cap = 700, 500, 64, 4096, 1024
    nslots = num_pages * 64
    k = wl.bf16_bits(rng.standard_normal((n, 512)).astype(np.float32))
    pos = rng.integers(0, max_pos, n).astype(np.int32)
    pos[[3, 9]] = [-1, max_pos]
    slots = (rng.choice(nslots + 16, n, replace=False) - 8).astype(np.int32)   # a few outside
    cs = wl.rope_cos_sin(max_pos=max_pos)
    kv = rng.standard_normal((R * 4, 512)).astype(np.float32)
    sc = (2 * rng.standard_normal((R * 4, 512))).astype(np.float32)
    pos_c = rng.integers(0, max_pos, R).astype(np.int32)
    table_len = 3000
    table = (rng.permutation(max(table_len, nslots + 16))[:table_len] - 8).astype(np.int32)
    full = (rng.choice(table_len + 32, R, replace=False) - 16).astype(np.int32)
    rc, loc = orc.translate_slots(table, full, cap)
    assert rc == 0
    slots_c = np.ascontiguousarray(loc[:R])
    pages = np.unique(slots_c[(slots_c >= 0) & (slots_c < nslots)] >> 6).astype(np.int32)
    for name, a in (("k", k), ("pos", pos), ("slots", slots), ("cs", cs), ("kv", kv), ("sc", sc),
                    ("pos_c", pos_c), ("table", table), ("full", full), ("pages", pages)):
        np.ascontiguousarray(a).tofile(tmp_path / f"{name}.bin")
    (tmp_path / "meta.txt").write_text(f"{n} {R} {num_pages} {max_pos} {cap} {table_len} {pages.size}\n")

    src = tmp_path / "program.c"
    src.write_text(PROGRAM)
    exe = tmp_path / "program"
    libdir = os.path.dirname(kvq.LIB_PATH)
    subprocess.run([gcc, "-std=c99", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
                    "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"), str(src),
                    "-o", str(exe), "-L", libdir, "-lkvq", f"-Wl,-rpath,{libdir}",
                    "-L", os.path.join(ROCM, "lib"), "-lamdhip64", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}"],
                   check=True)
    print(f"[c program] n {n}, R {R}, pages {num_pages}, cap {cap}", flush=True)
    r = subprocess.run([str(exe), str(tmp_path)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "ok" in r.stdout

    pool1 = np.fromfile(tmp_path / "pool1.bin", np.uint8).reshape(num_pages, -1)
    ref1 = orc.new_pool(V41, num_pages)
    orc.kv_store_rope(V41, ref1, k, pos, cs, slots)
    assert np.array_equal(pool1, ref1), f"{int((pool1 != ref1).sum())} store bytes differ"

    got_loc = np.fromfile(tmp_path / "loc.bin", np.int32)
    assert np.array_equal(got_loc, loc), "translated slots"

    pool2 = np.fromfile(tmp_path / "pool2.bin", np.uint8).reshape(num_pages, -1)
    ref2 = orc.new_pool(FP4, num_pages)
    orc.kv_compress_store(FP4, ref2, kv, sc, 4, pos_c, cs, slots_c)
    stored = slots_c[(slots_c >= 0) & (slots_c < nslots)]
    compare_compressed(pool2, ref2, FP4, stored, label="C program")
    assert untouched_equal(pool2, ref2, FP4, stored)

    ws = np.fromfile(tmp_path / "ws.bin", np.uint16).reshape(-1, 512)
    check_step_dequant(orc, FP4, ws, pool2, ref2, pages)
