"""The compressor comparison rule itself, pinned on the CPU with constructed pools: it
passes identical pools and one-step code differences under 0.1 %, and rejects any scale
byte difference, any code two or more steps away, and one-step differences above 0.1 %."""
import numpy as np
import pytest

from helpers import CR, FP4, SR, V41, compare_compressed


def _pools(layout, n=64, seed=0):
    rng = np.random.default_rng(seed)
    pb = 64 * (CR[layout] + SR[layout])
    pool = np.zeros((2, pb), np.uint8)
    slots = np.arange(64, 64 + n, dtype=np.int32)
    for s in slots:
        page, row = divmod(int(s), 64)
        codes = rng.integers(0, 256, CR[layout]).astype(np.uint8)
        if layout == V41:
            codes[(codes & 0x7F) == 0x7F] = 0x10          # no NaN codes
        pool[page, row * CR[layout]:(row + 1) * CR[layout]] = codes
        pool[page, 64 * CR[layout] + row * SR[layout]:64 * CR[layout] + row * SR[layout] + 16] = \
            rng.integers(100, 140, 16)
    return pool, slots


def _code_offset(layout, row, byte):
    return row * CR[layout] + byte


@pytest.mark.parametrize("layout", [V41, FP4])
def test_identical_pools_pass(layout):
    pool, slots = _pools(layout)
    assert compare_compressed(pool, pool.copy(), layout, slots) == 1.0


def test_signed_zero_codes_are_equal():
    pool, slots = _pools(V41)
    a, b = pool.copy(), pool.copy()
    a[1, _code_offset(V41, 0, 5)] = 0x00
    b[1, _code_offset(V41, 0, 5)] = 0x80
    assert compare_compressed(a, b, V41, slots) == 1.0


@pytest.mark.parametrize("layout", [V41, FP4])
def test_a_scale_byte_difference_fails(layout):
    pool, slots = _pools(layout)
    b = pool.copy()
    b[1, 64 * CR[layout] + 3 * SR[layout] + 7] ^= 1
    with pytest.raises(AssertionError, match="scale bytes differ"):
        compare_compressed(pool, b, layout, slots)


def test_two_code_steps_fail_and_one_passes():
    pool, slots = _pools(V41)
    a, b = pool.copy(), pool.copy()
    a[1, _code_offset(V41, 2, 9)] = 0x20
    b[1, _code_offset(V41, 2, 9)] = 0x21
    assert compare_compressed(a, b, V41, slots) < 1.0          # one step: admitted
    b[1, _code_offset(V41, 2, 9)] = 0x22
    with pytest.raises(AssertionError, match="more than one step"):
        compare_compressed(a, b, V41, slots)
    b[1, _code_offset(V41, 2, 9)] = 0xA1                      # -1 vs +0x20: far apart
    with pytest.raises(AssertionError, match="more than one step"):
        compare_compressed(a, b, V41, slots)


def test_fp4_nibbles_are_compared_one_by_one():
    pool, slots = _pools(FP4)
    a, b = pool.copy(), pool.copy()
    a[1, _code_offset(FP4, 4, 0)] = 0x32        # low nibble 2, high nibble 3
    b[1, _code_offset(FP4, 4, 0)] = 0x23        # low 3 (one step), high 2 (one step)
    assert compare_compressed(a, b, FP4, slots) < 1.0
    b[1, _code_offset(FP4, 4, 0)] = 0x34        # low nibble 4: two steps
    with pytest.raises(AssertionError, match="more than one step"):
        compare_compressed(a, b, FP4, slots)
    b[1, _code_offset(FP4, 4, 0)] = 0xB2        # high nibble -3 vs 3
    with pytest.raises(AssertionError, match="more than one step"):
        compare_compressed(a, b, FP4, slots)


def test_too_many_one_step_differences_fail():
    pool, slots = _pools(V41, n=4)               # 2048 codes: 0.1 % is 2 codes
    a, b = pool.copy(), pool.copy()
    for j in range(3):
        a[1, _code_offset(V41, 1, j)] = 0x30
        b[1, _code_offset(V41, 1, j)] = 0x31
    with pytest.raises(AssertionError, match="identical"):
        compare_compressed(a, b, V41, slots)
    b[1, _code_offset(V41, 1, 2)] = 0x30
    compare_compressed(a, b, V41, slots)
