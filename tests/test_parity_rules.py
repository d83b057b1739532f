"""The parity rules themselves, pinned on the CPU with constructed cases: the RoPE-channel
rule must admit exactly the codes that the other admissible bf16 rounding of a rotation
input produces, and nothing else."""
import math

import numpy as np

import oracle
from helpers import V41, _bf16_neighbours, _ord, near_bf16_midpoint, rope_alternative_ok
from quantized_paged_kv_compress_amd import workloads as wl

SCALE_BYTE = 119          # ue8m0 k = -8: blocks whose largest value is near 1


def _setup():
    """Rotation pair 0 at position 1 (angle 1 rad): x1 (channel 448) just above the
    midpoint of two bf16 neighbours, x2 (channel 480) the bf16 value that nearly cancels
    x1 in o2 = x2*c + x1*s."""
    cs = wl.rope_cos_sin(max_pos=4)
    pos = 1
    c, s = float(cs[pos, 0]), float(cs[pos, 32])
    lo, q = 103 / 256, 2.0 ** -9                     # a bf16 value in [0.25, 0.5) and its spacing
    x1 = lo + 0.5 * q * (1 + 2.0 ** -30)
    x2 = oracle.bf16_to_f32(oracle.bf16_from_double(-x1 * s / c))
    row = np.zeros(512)
    row[448], row[480] = x1, x2
    return cs, pos, row


def _code(b1, b2, cs, pos, ch):
    v = np.zeros(512, np.uint16)
    v[448], v[480] = b1, b2
    val = oracle.bf16_to_f32(int(oracle.rope_row(v, cs[pos])[ch]))
    return _ord(oracle.e4m3_encode(math.ldexp(val, -(SCALE_BYTE - 127))), V41)


def test_bf16_neighbours_bracket_the_value():
    for x in (0.3, -0.3, 1e-3, 123.456, 2.0 ** -130):
        a, b = (oracle.bf16_to_f32(n) for n in _bf16_neighbours(x))
        assert min(a, b) <= x <= max(a, b) and a != b


def test_rope_rule_admits_the_other_rounding_and_nothing_else():
    cs, pos, row = _setup()
    assert near_bf16_midpoint(row[448]) and not near_bf16_midpoint(row[480])
    b2 = oracle.bf16_from_double(row[480])
    b_rne = oracle.bf16_from_double(row[448])
    b_alt = [b for b in _bf16_neighbours(row[448]) if b != b_rne][0]
    o_rne, o_alt = _code(b_rne, b2, cs, pos, 480), _code(b_alt, b2, cs, pos, 480)
    assert abs(o_rne - o_alt) > 1          # the rotation amplifies one bf16 ulp (precondition)
    for got in (o_rne, o_alt, o_alt + 1 if o_alt > o_rne else o_alt - 1):
        assert rope_alternative_ok(V41, got, SCALE_BYTE, row, 480, pos, cs)
    far = max(o_rne, o_alt) + 3
    assert not rope_alternative_ok(V41, far, SCALE_BYTE, row, 480, pos, cs)
    # the same code with no input at a near-tie is not excused
    row2 = row.copy()
    row2[448] = 103 / 256 + 0.25 * 2.0 ** -9
    assert not rope_alternative_ok(V41, o_alt, SCALE_BYTE, row2, 480, pos, cs)
