"""The hardware approximations the short-window compressor's float32 error bound relies on,
measured on the GPU the tests run on (see tests/test_short_window_bound.py for the bound).

The ratio-2 and ratio-4 kernels keep a float32 pooled value only where it is certified to
round to the same bf16 as the exact pool; the certificate assumes that v_exp_f32 is within
1 ulp of 2^a wherever 2^a >= 2^-126 (for every a the kernel can produce) and that
v_rcp_f32 is within 1 ulp of 1/l.  A different chip, firmware or compiler lowering that
broke either would silently void the certificate, so both are swept exhaustively here
(every float32 input in the ranges that matter) with tests/hw_probe/libhwprobe.so.
"""
import ctypes
import os

import pytest

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def probe():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sys_path = os.path.join(HERE, "hw_probe")
    lib_path = os.path.join(sys_path, "libhwprobe.so")
    if not os.path.exists(lib_path):
        import importlib.util
        spec = importlib.util.spec_from_file_location("hwprobe_build", os.path.join(sys_path, "build.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build()
    lib = ctypes.CDLL(lib_path)
    for fn in (lib.hwprobe_exp2, lib.hwprobe_rcp):
        fn.restype = ctypes.c_int
        fn.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    return lib


def run(fn, label):
    import torch
    out = torch.zeros(4, dtype=torch.int64, device="cuda")
    print(f"[hw] sweeping {label}", flush=True)
    assert fn(out.data_ptr(), torch.cuda.current_stream().cuda_stream) == 0
    torch.cuda.synchronize()
    max_q, flushed, worst, checked = (int(v) for v in out.cpu().tolist())
    max_ulp = max_q / 2.0 ** 32
    print(f"[hw] {label}: {checked} inputs, largest error {max_ulp:.4f} ulp, {flushed} flushed", flush=True)
    return max_ulp, flushed, worst, checked


def test_exp2_within_one_ulp_over_the_kernels_range(probe):
    max_ulp, flushed, worst, checked = run(probe.hwprobe_exp2, "v_exp_f32 over [-160, 1]")
    assert checked == (0x43200000 + 1) + (0x3F800000 + 1)
    assert flushed == 0, "a result of at least 2^-126 was flushed"
    assert worst == 0 and max_ulp <= 1.0, f"v_exp_f32 error {max_ulp:.4f} ulp (input bits 0x{worst:08x})"


def test_reciprocal_within_one_ulp_over_weight_sums(probe):
    max_ulp, flushed, worst, checked = run(probe.hwprobe_rcp, "v_rcp_f32 over [1/2, 256)")
    assert checked == 0x437FFFFF - 0x3F000000 + 1
    assert flushed == 0
    assert worst == 0 and max_ulp <= 1.0, f"v_rcp_f32 error {max_ulp:.4f} ulp (input bits 0x{worst:08x})"
