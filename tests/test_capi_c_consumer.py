"""The boundary as a C program sees it: include/kvq.h compiles as strict C99, a program
links against libkvq.so, and the host-only calls (layout queries, status strings,
argument errors) behave as the header states.  No GPU needed: nothing here launches."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

PROGRAM = r"""
#include <stdio.h>
#include <string.h>
#include "kvq.h"

int main(void) {
    int bad = 0;
    if (kvq_bytes_per_token(KVQ_LAYOUT_V41) != 528) bad |= 1;
    if (kvq_bytes_per_token(KVQ_LAYOUT_V41_FP4) != 288) bad |= 2;
    if (kvq_page_bytes(KVQ_LAYOUT_V41) != 64 * 528) bad |= 4;
    if (kvq_page_bytes(KVQ_LAYOUT_V41_FP4) != 64 * 288) bad |= 8;
    if (kvq_code_row_bytes(KVQ_LAYOUT_V41) != 512 || kvq_scale_row_bytes(KVQ_LAYOUT_V41_FP4) != 32) bad |= 16;
    if (kvq_bytes_per_token(3) != KVQ_ELAYOUT) bad |= 32;
    if (strcmp(kvq_status_string(KVQ_OK), "ok") != 0) bad |= 64;
    /* errors are reported before anything is launched */
    if (kv_store(KVQ_LAYOUT_V41, NULL, 4, NULL, 512, NULL, 1, NULL) != KVQ_EINVAL) bad |= 128;
    if (kv_compress_store(KVQ_LAYOUT_V41, NULL, 4, NULL, NULL, 512, 3, NULL, NULL, 10, NULL, 1, NULL)
        != KVQ_ERATIO) bad |= 256;
    if (kv_translate_slots(NULL, 0, NULL, 11, NULL, 10, NULL) != KVQ_ECAPACITY) bad |= 512;
    if (kv_dequant(KVQ_LAYOUT_V41_FP4, NULL, 4, NULL, 0, NULL, NULL) != KVQ_OK) bad |= 1024;
    if (kvq_profile_next_launch(NULL, NULL) != KVQ_OK) bad |= 2048;
    printf("kvq C consumer: %s (%d)\n", bad ? "FAILED" : "ok", bad);
    return bad != 0;
}
"""


def test_header_compiles_as_c99_and_links(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no gcc")
    import quantized_paged_kv_compress_amd as kvq
    if not os.path.exists(kvq.LIB_PATH):
        from quantized_paged_kv_compress_amd import _build
        _build.build()
    src = tmp_path / "consumer.c"
    src.write_text(PROGRAM)
    exe = tmp_path / "consumer"
    libdir = os.path.dirname(kvq.LIB_PATH)
    subprocess.run([gcc, "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror",
                    "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe),
                    "-L", libdir, "-lkvq", f"-Wl,-rpath,{libdir}"], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "ok" in r.stdout
