"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test checks one oracle function against what the pages print (tests/golden/), a
closed form, an exhaustive brute force written independently here, a library routine
(torch's float8 / bfloat16 casts), or an invariant of the mathematics.  They are chosen
so that a plausible slip in the oracle (a dropped term, a wrong sign, index or operand
order, a wrong tie rule, a wrong byte or nibble order) fails at least one of them.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

from quantized_paged_kv_compress_amd import workloads as wl

V41, FP4 = 1, 2


# ---------------------------------------------------------------- independent helpers
def bf16_vals(bits):
    return (np.asarray(bits, np.uint32) << 16).view(np.float32)


def all_bf16_finite():
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = bf16_vals(b)
    keep = np.isfinite(v)
    return b[keep], v[keep]


def torch_e4m3_table():
    """Decode table of the 256 e4m3fn codes from torch's float8 dtype (library routine)."""
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float32).numpy().astype(np.float64)


def formula_e4m3(c):
    s = -1.0 if c & 0x80 else 1.0
    e, m = (c >> 3) & 15, c & 7
    if e == 15 and m == 7:
        return math.nan
    if e == 0:
        return s * m / 8.0 * 2.0 ** -6
    return s * (1 + m / 8.0) * 2.0 ** (e - 7)


def nearest_even(q, table_codes, table_vals):
    """Brute-force nearest of |q| among non-negative table values; ties -> even code."""
    a = np.abs(q)[:, None]
    d = np.abs(a - table_vals[None, :])
    dmin = d.min(axis=1, keepdims=True)
    cand = d == dmin
    even = cand & ((table_codes[None, :] & 1) == 0)
    pick = np.where(even.any(axis=1), even.argmax(axis=1), cand.argmax(axis=1))
    return table_codes[pick]


E4M3_POS_CODES = np.arange(0, 0x7F, dtype=np.int64)          # 0x00..0x7E (finite, >= 0)
E4M3_POS_VALS = np.array([formula_e4m3(c) for c in range(0x7F)])
E2M1_MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
E2M1_CODES = np.arange(8, dtype=np.int64)


def row_from_blocks(blocks):
    """16 blocks of up to 32 float values -> one bf16 row (uint16 bits); missing = 0."""
    v = np.zeros(512, np.float32)
    for b, vals in enumerate(blocks):
        v[b * 32:b * 32 + len(vals)] = vals
    bits = v.view(np.uint32)
    assert np.all((bits & 0xFFFF) == 0), "fixture values must be exact bf16"
    return (bits >> 16).astype(np.uint16)


# ---------------------------------------------------------------- layout facts (pages)
def test_layout_sizes_match_pages(orc, golden):
    g = golden("layout_sizes.json")
    assert orc.bytes_per_token(V41) == g["v41_bytes_per_token"] == 528
    assert orc.bytes_per_token(FP4) == g["v41_fp4_bytes_per_token"] == 288
    for lay, key in ((V41, "v41_saving_percent_1dp"), (FP4, "v41_fp4_saving_percent_1dp")):
        saving = 100.0 * (g["v4_bytes_per_token"] - orc.bytes_per_token(lay)) / g["v4_bytes_per_token"]
        assert round(saving, 1) == g[key]
    # V41: one byte per code, one scale per 32 values
    assert orc.code_row_bytes(V41) == g["head_dim"]
    assert orc.scale_row_bytes(V41) == g["head_dim"] // g["values_per_scale"] == g["v41_scales_per_token"]
    # FP4: two codes per byte, one e4m3 byte per 32 values, rest padding
    assert orc.code_row_bytes(FP4) == g["head_dim"] // 2
    assert orc.code_row_bytes(FP4) + g["head_dim"] // g["values_per_scale"] < 288
    for lay in (V41, FP4):
        assert orc.page_bytes(lay) == 64 * orc.bytes_per_token(lay)
    assert orc.bytes_per_token(7) < 0 and orc.page_bytes(0) < 0


def test_compressor_mapping_constants_consistent(golden):
    g = golden("compressor_mapping.json")
    assert g["copy_elems"] * 32 == g["copy_bits"]
    assert g["quant_block"] // g["elems_per_lane"] == g["lanes_per_group"]
    assert g["nvidia_warp_lanes"] // g["lanes_per_group"] == g["groups_per_warp"]
    assert (g["head_size"] // g["quant_block"]) // g["groups_per_warp"] == g["warps_per_row"]
    # one 64-lane wavefront covers a whole row at 8 elements per lane
    assert 64 * g["elems_per_lane"] == g["head_size"]


# ---------------------------------------------------------------- bfloat16 rounding
def test_bf16_rounding_matches_torch_on_float32(orc):
    rng = np.random.default_rng(11)
    bits = rng.integers(0, 2 ** 32, 200_000, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    f = f[np.isfinite(f)]
    # include exact ties and near-ties
    base = bf16_vals(rng.integers(0, 0x7F7F, 2000).astype(np.uint16)).view(np.uint32)
    ties = np.concatenate([base | 0x8000, (base | 0x8000) + 1, (base | 0x8000) - 1]).view(np.float32)
    f = np.concatenate([f, ties, -ties])
    want = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([orc.bf16_from_double(float(x)) for x in f], np.uint16)
    assert np.array_equal(got, want)


def test_bf16_rounding_from_double_brute_force(orc):
    rng = np.random.default_rng(12)
    xs = rng.standard_normal(20000) * np.exp(rng.uniform(-80, 80, 20000))
    for x in xs:
        h = orc.bf16_from_double(x)
        v = Fraction(float(bf16_vals(h)))
        # neighbours of the chosen value must not be nearer (ties -> even significand)
        for nb in ((h + 1) & 0xFFFF, (h - 1) & 0xFFFF):
            w = float(bf16_vals(nb))
            if not math.isfinite(w) or (nb ^ h) & 0x8000:
                continue
            dx, dn = abs(Fraction(x) - v), abs(Fraction(x) - Fraction(w))
            assert dx < dn or (dx == dn and h % 2 == 0)
    assert orc.bf16_from_double(-0.0) == 0x8000
    assert orc.bf16_from_double(1e300) == 0x7F80
    assert orc.bf16_from_double(2.0 ** -134) == 0x0000       # tie 0 | 2^-133 -> even (0)
    assert orc.bf16_from_double(2.0 ** -134 * 1.5) == 0x0001


# ---------------------------------------------------------------- e4m3
def test_e4m3_decode_table(orc):
    tt = torch_e4m3_table()
    for c in range(256):
        want = formula_e4m3(c)
        got = orc.e4m3_decode(c)
        if math.isnan(want):
            assert math.isnan(got) and math.isnan(tt[c])
        else:
            assert got == want == tt[c], c
            assert math.copysign(1, got) == math.copysign(1, want)


def test_e4m3_encode_exhaustive_bf16_inputs(orc):
    _, v = all_bf16_finite()
    v = v[np.abs(v) <= 448].astype(np.float64)
    # exact midpoints between neighbouring codes, and one float32 ulp either side
    mids = (E4M3_POS_VALS[1:] + E4M3_POS_VALS[:-1]) / 2
    mids32 = mids.astype(np.float32)
    near = np.concatenate([mids32, np.nextafter(mids32, np.float32(0)),
                           np.nextafter(mids32, np.float32(1e9))]).astype(np.float64)
    q = np.concatenate([v, near, -near, [0.0, -0.0, 448.0, -448.0]])
    mag = nearest_even(q, E4M3_POS_CODES, E4M3_POS_VALS)
    want = mag | np.where(np.signbit(q), 0x80, 0)
    got = np.array([orc.e4m3_encode(x) for x in q], np.int64)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(q[i], got[i], want[i]) for i in bad[:5]]


def test_e4m3_encode_matches_torch_cast(orc):
    rng = np.random.default_rng(13)
    q = (rng.standard_normal(100_000) * np.exp(rng.uniform(-12, 5.5, 100_000))).astype(np.float32)
    q = q[np.abs(q) <= 448]
    want = torch.from_numpy(q).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([orc.e4m3_encode(float(x)) for x in q], np.uint8)
    # torch drops the sign of values that round to zero in some builds; compare magnitude
    # codes everywhere and the full byte where torch's result is non-zero
    assert np.array_equal(got & 0x7F, want & 0x7F)
    nz = (want & 0x7F) != 0
    assert np.array_equal(got[nz], want[nz])


# ---------------------------------------------------------------- ue8m0
def exact_k(amax):
    """smallest integer k >= -127 with amax <= 448 * 2^k, by exact rational search"""
    a = Fraction(float(amax))
    k = -127
    while a > 448 * Fraction(2) ** k:
        k += 1
    return k


def test_ue8m0_exhaustive_bf16_amax(orc):
    bits, v = all_bf16_finite()
    pos = v[(v > 0)]
    assert pos.size == 32639
    got = np.array([orc.ue8m0_byte(float(a)) for a in pos], np.int64)
    # closed form on the float32 bits of amax (the "exponent from amax bits" route)
    u = pos.view(np.uint32).astype(np.int64)
    closed = np.maximum(0, (u >> 23) - 8 + ((u & 0x7FFFFF) > 0x600000))
    assert np.array_equal(got, closed)
    # exact rational definition on a spread of values (all binades, all mantissas of 3)
    for a in pos[::7]:
        assert orc.ue8m0_exponent(float(a)) == exact_k(a)
    # invariants: amax / s <= 448, and one power of two lower would not fit (byte > 0)
    k = got - 127
    s = np.ldexp(1.0, k)
    assert np.all(pos / s <= 448)
    assert np.all((pos / (s / 2) > 448) | (got == 0))
    assert orc.ue8m0_byte(0.0) == 0


def test_ue8m0_random_float32_amax(orc):
    rng = np.random.default_rng(14)
    a = np.abs(rng.standard_normal(20000) * np.exp(rng.uniform(-90, 87, 20000))).astype(np.float32)
    a = a[np.isfinite(a) & (a > 0)]
    for x in a[:4000]:
        assert orc.ue8m0_exponent(float(x)) == exact_k(x)


# ---------------------------------------------------------------- V41 rows (worked examples)
def test_v41_worked_examples(orc, golden):
    g = golden("worked_examples.json")
    blocks = [[float.fromhex(h) for h in b["values"]] for b in g["v41_blocks"]]
    code, scale = orc.quant_row(V41, row_from_blocks(blocks))
    for b, blk in enumerate(g["v41_blocks"]):
        assert scale[b] == blk["scale_byte"], (b, blk["why"])
        want = blk["codes"] + [0] * (32 - len(blk["codes"]))
        assert list(code[b * 32:(b + 1) * 32]) == want, (b, blk["why"])
    assert np.all(scale[len(blocks):] == 0) and np.all(code[len(blocks) * 32:] == 0)


def test_v41_row_exhaustive_bf16_codes(orc):
    """Every finite bf16 value, in a block whose amax sets k, encodes to the brute-force
    nearest code of x * 2^-k (ties to even), sign kept."""
    _, v = all_bf16_finite()
    rng = np.random.default_rng(15)
    rows = []
    expect = []
    for amax in (448.0, 1.0, 3.0, 2.0 ** -100, 1.5 * 2.0 ** 100, 2.0 ** -126):
        vals = v[np.abs(v) <= amax]
        vals = vals[rng.permutation(vals.size)]
        k = exact_k(amax)
        for start in range(0, vals.size, 31 * 16):
            chunk = vals[start:start + 31 * 16]
            blocks = []
            for b in range(0, chunk.size, 31):
                blk = np.concatenate([[np.float32(amax)], chunk[b:b + 31]]).astype(np.float32)
                blocks.append(blk)
                q = np.ldexp(blk.astype(np.float64), -k)
                exp = nearest_even(q, E4M3_POS_CODES, E4M3_POS_VALS) | np.where(np.signbit(q), 0x80, 0)
                expect.append((k + 127, np.pad(exp, (0, 32 - exp.size))))
            rows.append(row_from_blocks(blocks))
            while len(expect) % 16:                  # empty blocks of a partial row
                expect.append((0, np.zeros(32, np.int64)))
    k_in = np.stack(rows)
    pool = orc.new_pool(V41, (k_in.shape[0] + 63) // 64)
    slots = np.arange(k_in.shape[0], dtype=np.int32)
    orc.kv_store(V41, pool, k_in, slots)
    flat = []
    for r in range(k_in.shape[0]):
        page, row = divmod(r, 64)
        codes = pool[page, row * 512:(row + 1) * 512]
        scales = pool[page, 64 * 512 + row * 16: 64 * 512 + row * 16 + 16]
        for b in range(16):
            flat.append((scales[b], codes[b * 32:(b + 1) * 32]))
    for (s_got, c_got), (s_want, c_want) in zip(flat, expect):
        assert s_got == s_want
        assert np.array_equal(c_got.astype(np.int64), c_want)


# ---------------------------------------------------------------- FP4
def e4m3_rne_positive(t):
    """Independent: nearest non-negative e4m3 code to t (ties even), held at 0x7E."""
    t = np.asarray(t, np.float64)
    c = nearest_even(t, E4M3_POS_CODES, E4M3_POS_VALS)
    return np.where(t > 448, 0x7E, c)


def test_fp4_scale_exhaustive_bf16_amax(orc):
    _, v = all_bf16_finite()
    pos = v[~np.signbit(v)]                              # amax is never -0
    t = (pos / np.float32(6)).astype(np.float32)         # IEEE single division (numpy)
    want = e4m3_rne_positive(t.astype(np.float64))
    got = np.array([orc.fp4_scale_code(float(a)) for a in pos], np.int64)
    assert np.array_equal(got, want)
    tin = t[t <= 448]
    tc = torch.from_numpy(tin).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got[t <= 448], tc.astype(np.int64))


def e2m1_from_quotient(q):
    mag = nearest_even(np.minimum(np.abs(q), 6.0), E2M1_CODES, E2M1_MAG)
    mag = np.where(np.abs(q) > 6, 7, mag)
    return mag | np.where(np.signbit(q), 8, 0)


def e2m1_exact_compare(x, s):
    """Code from exact comparisons |x| vs t*s (products exact in float64), ties to even."""
    a = np.abs(x.astype(np.float64))
    s = np.float64(s)
    c = ((a > 0.25 * s).astype(np.int64) + (a >= 0.75 * s) + (a > 1.25 * s) + (a >= 1.75 * s)
         + (a > 2.5 * s) + (a >= 3.5 * s) + (a > 5.0 * s))
    return c | np.where(np.signbit(x), 8, 0)


def test_fp4_worked_examples(orc, golden):
    g = golden("worked_examples.json")
    blocks = [[float.fromhex(h) for h in b["values"]] for b in g["fp4_blocks"]]
    code, scale = orc.quant_row(FP4, row_from_blocks(blocks))
    for b, blk in enumerate(g["fp4_blocks"]):
        assert scale[b] == blk["scale_code"], blk["why"]
        want = blk["bytes"] + [0] * (16 - len(blk["bytes"]))
        assert list(code[b * 16:(b + 1) * 16]) == want, blk["why"]
        nib = [(code[b * 16 + j // 2] >> (4 * (j % 2))) & 15 for j in range(len(blk["nibbles"]))]
        assert nib == blk["nibbles"]
    assert np.all(scale[16:] == 0)   # padding bytes


def test_fp4_codes_exhaustive_pairs(orc):
    """All 126 positive e4m3 scales x all bf16 magnitudes in [s/16, 6s] (both signs): the
    codes equal the brute-force nearest of fl32(x / s), and also the exact comparison
    codes (fl32 rounding of the quotient never lands on a tie it did not start on)."""
    _, v = all_bf16_finite()
    vpos = v[v > 0]
    rows, expect = [], []
    blocks = []
    for sc in range(1, 0x7F):
        s = np.float32(formula_e4m3(sc))
        amax = np.float32(6) * s
        xs = vpos[(vpos >= s / 16) & (vpos <= amax)]
        xs = np.concatenate([xs, -xs, [np.float32(0), np.float32(-0.0)]]).astype(np.float32)
        for b in range(0, xs.size, 31):
            blk = np.concatenate([[amax], xs[b:b + 31]]).astype(np.float32)
            q = (blk / s).astype(np.float32)
            want = e2m1_from_quotient(q.astype(np.float64))
            assert np.array_equal(want, e2m1_exact_compare(blk, s))
            blocks.append(blk)
            expect.append((sc, np.pad(want, (0, 32 - want.size))))
            if len(blocks) == 16:
                rows.append(row_from_blocks(blocks))
                blocks = []
    if blocks:
        rows.append(row_from_blocks(blocks))
        while len(expect) % 16:
            expect.append((0, np.zeros(32, np.int64)))
    k_in = np.stack(rows)
    pool = orc.new_pool(FP4, (k_in.shape[0] + 63) // 64)
    orc.kv_store(FP4, pool, k_in, np.arange(k_in.shape[0], dtype=np.int32))
    n_checked = 0
    for r in range(k_in.shape[0]):
        page, row = divmod(r, 64)
        codes = pool[page, row * 256:(row + 1) * 256]
        scales = pool[page, 64 * 256 + row * 32: 64 * 256 + row * 32 + 32]
        assert np.all(scales[16:] == 0)
        nib = np.stack([codes & 15, codes >> 4], axis=1).reshape(-1).astype(np.int64)
        for b in range(16):
            s_want, c_want = expect[r * 16 + b]
            assert scales[b] == s_want
            assert np.array_equal(nib[b * 32:(b + 1) * 32], c_want), (r, b)
            n_checked += 1
    assert n_checked > 100_000 // 32


# ---------------------------------------------------------------- RoPE
def test_rope_table_closed_form():
    cs = wl.rope_cos_sin()
    assert cs.shape == (65536, 64) and cs.dtype == np.float32
    rng = np.random.default_rng(16)
    for p in rng.integers(0, 65536, 200):
        for i in range(32):
            ang = float(p) * 10000.0 ** (-2.0 * i / 64)
            for got, ref in ((cs[p, i], math.cos(ang)), (cs[p, 32 + i], math.sin(ang))):
                ulp = np.spacing(np.float32(abs(ref)))
                assert abs(float(got) - ref) <= 0.5 * ulp + 1e-15


def test_rope_position_zero_is_identity(orc):
    rng = np.random.default_rng(17)
    cs = wl.rope_cos_sin(max_pos=4)
    for _ in range(20):
        v = wl.bf16_bits(rng.standard_normal(512).astype(np.float32))
        assert np.array_equal(orc.rope_row(v, cs[0]), v)


def test_rope_pairs_and_rotation_direction(orc):
    """A unit vector on channel 448+i turns into (cos a, sin a) on (448+i, 480+i), and one
    on 480+i into (-sin a, cos a): pins the NeoX half pairing, the angle index, the table
    halves and the rotation sign.  Other channels are untouched."""
    cs = wl.rope_cos_sin()
    rng = np.random.default_rng(18)
    for p in rng.integers(1, 65536, 6):
        for i in range(32):
            ang = float(p) * 10000.0 ** (-2.0 * i / 64)
            c32, s32 = np.float32(math.cos(ang)), np.float32(math.sin(ang))
            for on_first in (True, False):
                v = np.zeros(512, np.float32)
                v[:448] = rng.standard_normal(448)
                v = wl.bf16_bits(v)
                v[448 + i if on_first else 480 + i] = 0x3F80  # 1.0
                out = orc.rope_row(v, cs[p])
                if on_first:
                    want1, want2 = wl.bf16_bits(np.array([c32, s32]))
                else:
                    want1, want2 = wl.bf16_bits(np.array([-s32, c32]))
                assert out[448 + i] == want1 and out[480 + i] == want2, (p, i, on_first)
                assert np.array_equal(out[:448], v[:448])
                # the other rope pairs are zero and stay zero (a negative cosine or sine
                # can give -0, which is the correctly rounded result)
                others = np.ones(64, bool)
                others[[i, 32 + i]] = False
                assert np.all(bf16_vals(out[448:][others]) == 0)


def test_rope_rounding_order_worked_example(orc, golden):
    """Hand-derived row (tests/golden/worked_examples.json, 'rope') where rounding each
    float32 product and the difference on its own gives a different bf16 than both a
    float64 evaluation and a fused multiply-add -- pins the rounding order of the rotation,
    at every pair index."""
    ex = golden("worked_examples.json")["rope"]
    for e in ex:
        x1, x2 = int(e["x1_bf16"], 16), int(e["x2_bf16"], 16)
        c, s = np.float32(float.fromhex(e["cos"])), np.float32(float.fromhex(e["sin"]))
        assert int(e["o1_bf16"], 16) not in (int(e["o1_if_float64"], 16), int(e["o1_if_fused"], 16))
        for i in (0, 17, 31):
            v = np.zeros(512, np.uint16)
            v[448 + i], v[480 + i] = x1, x2
            cs = np.zeros(64, np.float32)
            cs[i], cs[32 + i] = c, s
            out = orc.rope_row(v, cs)
            assert out[448 + i] == int(e["o1_bf16"], 16), (i, hex(out[448 + i]))
            assert out[480 + i] == int(e["o2_bf16"], 16), (i, hex(out[480 + i]))


def test_rope_preserves_pair_norm(orc):
    cs = wl.rope_cos_sin()
    rng = np.random.default_rng(19)
    for _ in range(50):
        v = wl.bf16_bits(rng.standard_normal(512).astype(np.float32))
        p = int(rng.integers(0, 65536))
        out = bf16_vals(orc.rope_row(v, cs[p])).astype(np.float64)
        vin = bf16_vals(v).astype(np.float64)
        n_in = np.hypot(vin[448:480], vin[480:])
        n_out = np.hypot(out[448:480], out[480:])
        assert np.all(np.abs(n_out - n_in) <= 2 * 2.0 ** -8 * n_in + 1e-30)


# ---------------------------------------------------------------- pooling
def py_pool(kv, sc, ratio, i, c):
    """Brute force in Python floats: softmax over the window's scores in channel c."""
    s = [float(sc[i * ratio + j, c]) for j in range(ratio)]
    m = max(s)
    w = [math.exp(x - m) for x in s]
    den = math.fsum(w)
    return math.fsum(w[j] * float(kv[i * ratio + j, c]) for j in range(ratio)) / den


@pytest.mark.parametrize("ratio,R", [(1, 3), (2, 3), (4, 3), (128, 2)])
def test_pool_brute_force_tiny(orc, ratio, R):
    rng = np.random.default_rng(20 + ratio)
    kv = rng.standard_normal((R * ratio, 512)).astype(np.float32)
    sc = (2 * rng.standard_normal((R * ratio, 512))).astype(np.float32)
    f64, b16 = orc.pool_rows(kv, sc, ratio)
    for i in range(R):
        for c in range(0, 512, 7):
            ref = py_pool(kv, sc, ratio, i, c)
            assert abs(f64[i, c] - ref) <= 1e-12 * (abs(ref) + 1e-3)
    # bf16 outputs are the single rounding of the float64 values
    for i in range(R):
        for c in range(0, 512, 5):
            assert b16[i, c] == orc.bf16_from_double(f64[i, c])


def test_pool_ratio_one_is_identity(orc):
    rng = np.random.default_rng(21)
    kv = rng.standard_normal((300, 512)).astype(np.float32)
    sc = (2 * rng.standard_normal((300, 512))).astype(np.float32)
    f64, b16 = orc.pool_rows(kv, sc, 1)
    assert np.array_equal(f64, kv.astype(np.float64))
    assert np.array_equal(b16, wl.bf16_bits(kv))


def test_pool_two_rows_closed_form(orc):
    """r = 2: the softmax weight of row 0 is the logistic function of s0 - s1."""
    rng = np.random.default_rng(22)
    kv = rng.standard_normal((40, 512)).astype(np.float32)
    sc = (2 * rng.standard_normal((40, 512))).astype(np.float32)
    f64, _ = orc.pool_rows(kv, sc, 2)
    d = sc[0::2].astype(np.float64) - sc[1::2].astype(np.float64)
    w0 = 1.0 / (1.0 + np.exp(-d))
    ref = kv[1::2] + w0 * (kv[0::2].astype(np.float64) - kv[1::2])
    assert np.allclose(f64, ref, rtol=1e-12, atol=1e-13)


def test_pool_equal_scores_give_mean_and_dominant_row_wins(orc):
    rng = np.random.default_rng(23)
    for ratio in (4, 128):
        kv = rng.standard_normal((3 * ratio, 512)).astype(np.float32)
        sc = np.full((3 * ratio, 512), 0.75, np.float32)
        f64, _ = orc.pool_rows(kv, sc, ratio)
        mean = kv.astype(np.float64).reshape(3, ratio, 512).mean(axis=1)
        assert np.allclose(f64, mean, rtol=1e-13, atol=1e-14)
        sc = (2 * rng.standard_normal((3 * ratio, 512))).astype(np.float32)
        win = rng.integers(0, ratio, (3, 512))
        for i in range(3):
            sc[i * ratio + win[i], np.arange(512)] += 1000.0
        f64, b16 = orc.pool_rows(kv, sc, ratio)
        want = kv[np.arange(3)[:, None] * ratio + win, np.arange(512)[None, :]]
        assert np.array_equal(f64, want.astype(np.float64))


def test_pool_permutation_and_shift_invariance(orc):
    rng = np.random.default_rng(24)
    ratio, R = 128, 3
    kv = rng.standard_normal((R * ratio, 512)).astype(np.float32)
    sc = (2 * rng.standard_normal((R * ratio, 512))).astype(np.float32)
    f64, _ = orc.pool_rows(kv, sc, ratio)
    perm = np.concatenate([i * ratio + rng.permutation(ratio) for i in range(R)])
    f64p, _ = orc.pool_rows(np.ascontiguousarray(kv[perm]), np.ascontiguousarray(sc[perm]), ratio)
    assert np.allclose(f64p, f64, rtol=1e-12, atol=1e-14)
    shift = rng.uniform(-20, 20, 512).astype(np.float32)
    # shift by values that keep every score exact in float32 (multiples of 2^-4, |s| < 64)
    shift = np.round(shift * 16) / 16
    sc_q = np.round(sc * 2 ** 12) / 2 ** 12
    f_a, _ = orc.pool_rows(kv, sc_q.astype(np.float32), ratio)
    f_b, _ = orc.pool_rows(kv, (sc_q + shift[None, :]).astype(np.float32), ratio)
    assert np.allclose(f_a, f_b, rtol=1e-12, atol=1e-14)


def test_pool_window_indexing(orc):
    """Window i is rows [i*r, i*r + r): a kv row tagged with its index and a dominant
    score on exactly one row per window gives back that row's tag."""
    ratio, R = 4, 50
    kv = np.repeat(np.arange(R * ratio, dtype=np.float32)[:, None], 512, axis=1)
    sc = np.zeros((R * ratio, 512), np.float32)
    rng = np.random.default_rng(25)
    pick = rng.integers(0, ratio, R)
    sc[np.arange(R) * ratio + pick, :] = 500.0
    f64, _ = orc.pool_rows(kv, sc, ratio)
    assert np.array_equal(f64[:, 0], (np.arange(R) * ratio + pick).astype(np.float64))


# ---------------------------------------------------------------- addressing
@pytest.mark.parametrize("layout", [V41, FP4])
def test_addressing_brute_force_with_canaries(orc, layout):
    """Each slot of a 4-page pool gets a row whose block b holds the value 2^(b-8) in every
    element (so block b's scale byte and codes identify the block); the bytes must land at
    page*PB + row*CR (codes) and page*PB + 64*CR + row*SR (scales), nothing else changes,
    and out-of-pool slots write nothing."""
    num_pages = 4
    PB = orc.page_bytes(layout)
    CR, SR = (512, 16) if layout == V41 else (256, 32)
    rng = np.random.default_rng(26)
    slots = rng.permutation(num_pages * 64)[:150].astype(np.int32)
    slots = np.concatenate([slots, np.array([-1, num_pages * 64, -(2 ** 31), 2 ** 31 - 1], np.int32)])
    blocks = [[2.0 ** (b - 8)] * 32 for b in range(16)]
    row = row_from_blocks(blocks)
    k = np.tile(row, (slots.size, 1))
    pool = np.full((num_pages, PB), 0xA5, np.uint8)
    orc.kv_store(layout, pool, k, slots)
    flat = pool.reshape(-1)
    touched = np.zeros(flat.size, bool)
    for s in slots[:150]:
        page, r = divmod(int(s), 64)
        c0 = page * PB + r * CR
        s0 = page * PB + 64 * CR + r * SR
        touched[c0:c0 + CR] = True
        touched[s0:s0 + SR] = True
        codes, scales = flat[c0:c0 + CR], flat[s0:s0 + SR]
        for b in range(16):
            x = 2.0 ** (b - 8)
            if layout == V41:
                k_ = exact_k(x)
                assert scales[b] == k_ + 127
                want = nearest_even(np.array([x * 2.0 ** -k_]), E4M3_POS_CODES, E4M3_POS_VALS)[0]
                assert np.all(codes[b * 32:(b + 1) * 32] == want)
            else:
                sc = e4m3_rne_positive([np.float32(x) / np.float32(6)])[0]
                assert scales[b] == sc
                sv = E4M3_POS_VALS[sc]
                n = 0 if sv == 0 else e2m1_from_quotient(np.array([np.float32(x) / np.float32(sv)]))[0]
                assert np.all(codes[b * 16:(b + 1) * 16] == n | (n << 4))
        if layout == FP4:
            assert np.all(scales[16:] == 0)
    assert np.all(flat[~touched] == 0xA5)


def test_store_layout_byte_and_nibble_order(orc):
    """V41 code c sits at byte c of the code row; FP4 element 2j is the low nibble of byte j;
    scale byte b belongs to block b."""
    v = np.zeros(512, np.float32)
    v[5] = 1.0
    v[32 * 3 + 1] = -2.0
    row = wl.bf16_bits(v)
    code, scale = orc.quant_row(V41, row)
    assert np.nonzero(code)[0].tolist() == [5, 97]
    assert scale[0] == exact_k(1.0) + 127 and scale[3] == exact_k(2.0) + 127
    assert scale[1] == 0 and scale[2] == 0
    code, scale = orc.quant_row(FP4, row)
    assert code[2] == 0x70     # element 5 is the high nibble of byte 2: 1.0 -> 6 -> code 7
    assert code[48] == 0xF0    # element 97 (block 3) high nibble of byte 48: -2 -> -6 -> 0xF


# ---------------------------------------------------------------- dequant
def test_dequant_worked_examples(orc, golden):
    g = golden("worked_examples.json")
    for ex in g["dequant"]:
        layout = V41 if ex["layout"] == "V41" else FP4
        pool = orc.new_pool(layout, 1)
        CR = 512 if layout == V41 else 256
        if layout == V41:
            pool[0, 0] = ex["code"]
        else:
            pool[0, 0] = ex["code"]       # element 0 = low nibble
        pool[0, 64 * CR] = ex["scale"]
        out = orc.kv_dequant(layout, pool, np.array([0], np.int32))
        assert out[0, 0] == int(ex["bf16"], 16), ex["why"]


def test_dequant_exhaustive_v41(orc):
    """All 256 codes x all 256 scale bytes against torch's e4m3 decode times 2^(byte-127),
    formed in float32 and cast to bf16 by torch."""
    pool = orc.new_pool(V41, 2)
    for r in range(128):
        page, row = divmod(r, 64)
        for b in range(16):
            pool[page, 64 * 512 + row * 16 + b] = 2 * r + (b // 8)
            pool[page, row * 512 + b * 32: row * 512 + b * 32 + 32] = (b % 8) * 32 + np.arange(32)
    out = orc.kv_dequant(V41, pool, np.array([0, 1], np.int32))
    tt = torch_e4m3_table()
    for r in range(128):
        for b in range(16):
            sbyte = 2 * r + (b // 8)
            codes = (b % 8) * 32 + np.arange(32)
            val = tt[codes]
            if sbyte == 255:
                want = np.full(32, 0x7FC0, np.uint16)
            else:
                with np.errstate(over="ignore"):
                    prod = (val * 2.0 ** (sbyte - 127)).astype(np.float32)
                want = torch.from_numpy(prod).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
                want = np.where(np.isnan(val), 0x7FC0, want)
            got = out[r, b * 32:(b + 1) * 32]
            assert np.array_equal(got, want), (r, b)


def test_dequant_exhaustive_fp4(orc):
    pool = orc.new_pool(FP4, 1)
    for r in range(16):
        for b in range(16):
            pool[0, 64 * 256 + r * 32 + b] = r * 16 + b
        nib = np.arange(32) % 16
        pool[0, r * 256:(r + 1) * 256] = np.tile((nib[0::2] | (nib[1::2] << 4)).astype(np.uint8), 16)
    out = orc.kv_dequant(FP4, pool, np.array([0], np.int32))
    tt = torch_e4m3_table()
    for r in range(16):
        for b in range(16):
            s = tt[r * 16 + b]
            vals = np.array([(-1.0 if n & 8 else 1.0) * E2M1_MAG[n & 7] for n in np.arange(32) % 16])
            if math.isnan(s):
                want = np.full(32, 0x7FC0, np.uint16)
            else:
                want = torch.from_numpy((vals * s).astype(np.float32)).to(torch.bfloat16) \
                    .view(torch.int16).numpy().view(np.uint16)
            assert np.array_equal(out[r, b * 32:(b + 1) * 32], want), (r, b)


@pytest.mark.parametrize("layout", [V41, FP4])
def test_dequant_roundtrip_bound_and_idempotence(orc, layout):
    d = wl.store_v41(seed=31, n=128, num_pages=4)
    k, slots = d["k"], np.arange(128, dtype=np.int32) + 64
    pool = orc.new_pool(layout, 4)
    orc.kv_store(layout, pool, k, slots)
    out = orc.kv_dequant(layout, pool, np.array([1, 2], np.int32))
    x = bf16_vals(k).astype(np.float64)
    y = bf16_vals(out).astype(np.float64)
    # round-trip error within half a code step times the scale
    for i in range(128):
        for b in range(16):
            xb, yb = x[i, b * 32:(b + 1) * 32], y[i, b * 32:(b + 1) * 32]
            amax = np.abs(xb).max()
            if layout == V41:
                s = 2.0 ** exact_k(amax)
                q = np.abs(xb) / s
                e = np.maximum(np.floor(np.log2(np.maximum(q, 2.0 ** -30))), -6)
                bound = 0.5 * 2.0 ** (e - 3) * s
            else:
                s = E4M3_POS_VALS[e4m3_rne_positive([np.float32(amax) / np.float32(6)])[0]]
                q = np.abs(xb) / s
                gap = np.where(q < 2, 0.5, np.where(q < 4, 1.0, 2.0))
                bound = np.where(q <= 6, 0.5 * gap, q - 6) * s
            err = np.abs(xb - yb)
            assert np.all(err <= bound * (1 + 2.0 ** -8) + 1e-40), (i, b)
    # quantising the dequantised rows reproduces the same values
    pool2 = orc.new_pool(layout, 4)
    orc.kv_store(layout, pool2, out, np.arange(128, dtype=np.int32) + 64)
    out2 = orc.kv_dequant(layout, pool2, np.array([1, 2], np.int32))
    assert np.array_equal(out2, out)
    if layout == FP4:
        assert np.array_equal(pool2, pool)


def test_dequant_skips_out_of_pool_pages(orc):
    pool = orc.new_pool(V41, 2)
    out = np.full((3 * 64, 512), 0x1234, np.uint16)
    orc.kv_dequant(V41, pool, np.array([1, 5, -1], np.int32), out)
    assert np.all(out[:64] == 0) and np.all(out[64:] == 0x1234)


# ---------------------------------------------------------------- translate
def test_translate_semantics(orc, golden):
    g = golden("translate_semantics.json")
    rng = np.random.default_rng(27)
    table = rng.integers(0, 10 ** 6, 1000).astype(np.int32)
    full = rng.integers(0, 1000, 300).astype(np.int32)
    full[:3] = [-1, 1000, 999]
    rc, out = orc.translate_slots(table, full, 512)
    assert rc == 0 and out.dtype == np.dtype(g["dtype"])
    assert out[0] == -1 and out[1] == -1 and out[2] == table[999]
    assert np.array_equal(out[3:300], table[full[3:]])
    assert np.all(out[300:] == g["tail_value"])
    rc, out = orc.translate_slots(table, full, 299)            # n > capacity: refused
    assert rc == -4 and np.all(out == 0x5A5A5A5A)
    rc, out = orc.translate_slots(table, full[:0], 8)
    assert rc == 0 and np.all(out == 0)


# ---------------------------------------------------------------- compressor assembly
def test_compress_ratio_one_equals_store_rope_of_bf16(orc):
    rng = np.random.default_rng(28)
    R = 200
    kv = rng.standard_normal((R, 512)).astype(np.float32)
    sc = rng.standard_normal((R, 512)).astype(np.float32)
    cs = wl.rope_cos_sin()
    pos = rng.integers(0, 65536, R).astype(np.int32)
    slots = wl.distinct_slots(rng, R, 64, 8 * 64)
    for layout in (V41, FP4):
        a = orc.new_pool(layout, 8)
        b = orc.new_pool(layout, 8)
        orc.kv_compress_store(layout, a, kv, sc, 1, pos, cs, slots)
        orc.kv_store_rope(layout, b, wl.bf16_bits(kv), pos, cs, slots)
        assert np.array_equal(a, b)


def test_compress_equals_pool_then_store_rope(orc):
    """The compressor is pooling (rounded to bf16) followed by the store+RoPE path, and
    rows with an out-of-range position or slot are skipped."""
    rng = np.random.default_rng(29)
    R, ratio = 60, 4
    kv = rng.standard_normal((R * ratio, 512)).astype(np.float32)
    sc = (2 * rng.standard_normal((R * ratio, 512))).astype(np.float32)
    cs = wl.rope_cos_sin(max_pos=1024)
    pos = rng.integers(0, 1024, R).astype(np.int32)
    pos[3] = 1024
    pos[4] = -5
    slots = wl.distinct_slots(rng, R, 64, 4 * 64)
    slots[7] = -1
    _, pooled = orc.pool_rows(kv, sc, ratio)
    for layout in (V41, FP4):
        a = orc.new_pool(layout, 4)
        b = orc.new_pool(layout, 4)
        orc.kv_compress_store(layout, a, kv, sc, ratio, pos, cs, slots)
        orc.kv_store_rope(layout, b, pooled, pos, cs, slots)
        assert np.array_equal(a, b)
        CR = 512 if layout == V41 else 256
        for i in (3, 4):
            page, r = divmod(int(slots[i]), 64)
            assert np.all(a[page, r * CR:(r + 1) * CR] == 0)

# ---------------------------------------------------------------- K norm (RMS)
def _row_from_spec(spec, default):
    v = np.full(512, default, np.float32)
    for k_, h in spec.items():
        if k_ == "all":
            v[:] = float.fromhex(h)
        else:
            v[int(k_)] = float.fromhex(h)
    return wl.bf16_bits(v)


def test_norm_worked_examples(orc, golden):
    for ex in golden("worked_examples.json")["k_norm"]:
        x = _row_from_spec(ex["x"], 0.0)
        w = _row_from_spec(ex["weight"], 1.0)
        y = orc.norm_row(x, w, ex["eps"])
        for c, h in ex["y_bf16"].items():
            assert y[int(c)] == int(h, 16), ex["why"]
        if "all" not in ex["x"]:
            others = np.ones(512, bool)
            others[[int(c) for c in ex["x"]]] = False
            assert np.all(bf16_vals(y[others]) == 0)


def test_norm_is_nearest_bf16_of_exact_value(orc):
    rng = np.random.default_rng(51)
    for _ in range(40):
        x = wl.bf16_bits((rng.standard_normal(512) * np.exp(rng.uniform(-3, 3))).astype(np.float32))
        w = wl.bf16_bits(rng.uniform(0.5, 2.0, 512).astype(np.float32))
        eps = float(rng.choice([0.0, 1e-6, 0.5]))
        y = bf16_vals(orc.norm_row(x, w, eps)).astype(np.float64)
        xv = bf16_vals(x).astype(np.float64)
        wv = bf16_vals(w).astype(np.float64)
        r = 1.0 / math.sqrt(math.fsum(xv * xv) / 512 + eps)
        exact = xv * wv * r
        ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(exact), 1e-300))) - 7)
        assert np.all(np.abs(y - exact) <= 0.5 * ulp * (1 + 1e-12))


def test_norm_scale_invariance_and_weight_mapping(orc):
    rng = np.random.default_rng(52)
    x = rng.standard_normal(512).astype(np.float32)
    w = wl.bf16_bits(np.ones(512, np.float32))
    y = orc.norm_row(wl.bf16_bits(x), w, 0.0)
    for k in (-20, -3, 1, 7):        # a power-of-two scale of the row cancels exactly (eps 0)
        assert np.array_equal(orc.norm_row(wl.bf16_bits(x * np.float32(2.0 ** k)), w, 0.0), y)
    for j in (0, 255, 256, 447, 448, 511):
        wj = np.zeros(512, np.float32)
        wj[j] = 1.0
        yj = orc.norm_row(wl.bf16_bits(x), wl.bf16_bits(wj), 0.0)
        nz = np.nonzero(bf16_vals(yj))[0]
        assert nz.tolist() == ([j] if x[j] != 0 else [])
        assert yj[j] == y[j]


def test_norm_rope_store_composes(orc):
    rng = np.random.default_rng(53)
    n, num_pages = 70, 4
    k = wl.bf16_bits(rng.standard_normal((n, 512)).astype(np.float32))
    w = wl.bf16_bits(rng.uniform(0.5, 1.5, 512).astype(np.float32))
    cs = wl.rope_cos_sin(max_pos=512)
    pos = rng.integers(0, 512, n).astype(np.int32)
    pos[3] = 600                                         # skipped
    slots = wl.distinct_slots(rng, n, 0, num_pages * 64)
    normed = np.stack([orc.norm_row(k[i], w, 1e-6) for i in range(n)])
    for layout in (V41, FP4):
        a = orc.new_pool(layout, num_pages)
        b = orc.new_pool(layout, num_pages)
        orc.kv_store_norm_rope(layout, a, k, w, 1e-6, pos, cs, slots)
        orc.kv_store_rope(layout, b, normed, pos, cs, slots)
        assert np.array_equal(a, b)


# ---------------------------------------------------------------- token-gather dequant
@pytest.mark.parametrize("layout", [V41, FP4])
def test_dequant_slots_matches_page_dequant(orc, layout):
    """Row i of the token gather equals row (slot & 63) of page (slot >> 6) of the page
    dequant (pinned exhaustively above); out-of-pool slots leave their rows untouched."""
    rng = np.random.default_rng(54)
    num_pages = 6
    pool = rng.integers(0, 256, (num_pages, orc.page_bytes(layout))).astype(np.uint8)
    pages = orc.kv_dequant(layout, pool, np.arange(num_pages, dtype=np.int32))
    slots = rng.integers(0, num_pages * 64, 300).astype(np.int32)
    slots[[5, 6, 7]] = [-1, num_pages * 64, 2 ** 31 - 1]
    out = np.full((300, 512), 0x1234, np.uint16)
    orc.kv_dequant_slots(layout, pool, slots, out)
    for i, sl in enumerate(slots):
        if 0 <= sl < num_pages * 64:
            assert np.array_equal(out[i], pages[sl])
        else:
            assert np.all(out[i] == 0x1234)


def test_duplicate_stored_slots_are_refused(orc):
    """Two rows of one call stored at the same slot is a caller error; the oracle refuses
    such inputs (a comparison on them would not be defined), but a duplicate among rows
    that are skipped (slot outside the pool, position outside the table) is allowed."""
    import pytest
    rng = np.random.default_rng(5)
    k = rng.integers(0, 1 << 15, (4, 512)).astype(np.uint16)
    cs = np.zeros((8, 64), np.float32)
    pool = orc.new_pool(orc.V41, 2)
    with pytest.raises(ValueError):
        orc.kv_store(orc.V41, pool, k, np.array([3, 7, 3, 9], np.int32))
    with pytest.raises(ValueError):
        orc.kv_store_rope(orc.V41, pool, k, np.array([1, 2, 3, 4], np.int32), cs, np.array([5, 5, 6, 7], np.int32))
    kv = rng.standard_normal((8, 512)).astype(np.float32)
    with pytest.raises(ValueError):
        orc.kv_compress_store(orc.V41, pool, kv, kv, 2, np.zeros(4, np.int32), cs, np.array([0, 1, 1, 2], np.int32))
    # skipped rows may share a slot: out of the pool, or with an out-of-range position
    orc.kv_store(orc.V41, pool, k, np.array([-1, -1, 200, 200], np.int32))
    orc.kv_store_rope(orc.V41, pool, k, np.array([1, 9, 9, 2], np.int32), cs, np.array([5, 6, 6, 7], np.int32))
