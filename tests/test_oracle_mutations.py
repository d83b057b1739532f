"""Planted mistakes: each plausible slip in the oracle must fail at least one pin.

Every case copies oracle/kvq_oracle.c, changes one expression, builds the copy with the
oracle's own gcc command into a temporary directory, swaps it in, and runs the pins that
cover that part.  The test passes only if some pin rejects the mutant; the real oracle is
restored afterwards.  Nothing here touches the GPU.
"""
import json
import os
import subprocess

import pytest

import oracle
from oracle import build as oracle_build
import test_oracle_pins as pins

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def golden(name):
    with open(os.path.join(ROOT, "tests", "golden", name)) as f:
        return json.load(f)


# (name, original text, mutated text, pins that must catch it)
MUTATIONS = [
    ("rope sign flipped", "float o1 = a - b, o2 = d + e;", "float o1 = a + b, o2 = d - e;",
     ["rope_pairs"]),
    ("cos and sin swapped", "float c = cs[i], s = cs[half + i];", "float c = cs[half + i], s = cs[i];",
     ["rope_pos0", "rope_pairs"]),
    ("ue8m0 one power too high", "(double)amax > ldexp(448.0, k)) k++;",
     "(double)amax > ldexp(448.0, k + 1)) k++;", ["ue8m0", "v41_worked"]),
    ("e4m3 ties rounded up", "double n = nearbyint(a / quantum);", "double n = floor(a / quantum + 0.5);",
     ["e4m3_exhaustive", "v41_worked"]),
    ("e2m1 ties to odd", "(d == bestd && (i % 2) == 0)", "(d == bestd && (i % 2) == 1)",
     ["fp4_worked", "fp4_pairs"]),
    ("fp4 scale amax/4", "float t = amax / 6.0f;", "float t = amax / 4.0f;",
     ["fp4_scale", "fp4_worked"]),
    ("nibbles swapped", "(uint8_t)(lo | (hi << 4))", "(uint8_t)(hi | (lo << 4))",
     ["fp4_worked", "byte_order"]),
    ("window rows transposed", "(i * ratio + j) * ld", "(i + j * ratio) * ld",
     ["pool_tiny", "pool_window"]),
    ("softmax not normalised", "out[c] = num / den;", "out[c] = num;",
     ["pool_tiny", "pool_mean"]),
    ("scale rows reversed in the page", "*scale = pg + kPageRows * cr + row * sr;",
     "*scale = pg + kPageRows * cr + (kPageRows - 1 - row) * sr;", ["addressing"]),
    ("bf16 truncates", "double r = nearbyint(m);", "double r = trunc(m);",
     ["bf16_torch", "bf16_brute"]),
    ("dequant exponent shifted", "s = ldexp(1.0, (int)scale - 127);", "s = ldexp(1.0, (int)scale - 128);",
     ["dequant_worked", "dequant_v41"]),
    ("translate tail not zeroed", "for (int64_t i = n; i < cap; i++) out[i] = 0;",
     "for (int64_t i = n; i < cap; i++) out[i] = -1;", ["translate"]),
    ("rms over 448 channels", "double r = 1.0 / sqrt(ss / kHead + (double)eps);",
     "double r = 1.0 / sqrt(ss / 448 + (double)eps);", ["norm_worked", "norm_exact"]),
    ("norm weight shifted a channel", "(double)orc_bf16_to_f32(w_bf16[c]) * r", "(double)orc_bf16_to_f32(w_bf16[(c + 1) % kHead]) * r",
     ["norm_worked", "norm_mapping"]),
    ("fp4 padding not written", "memset(scale + kHead / kBlock, 0, 16); /* documented padding */",
     "(void)0; /* padding left as it was */", ["addressing"]),
    ("rope pairs offset by one channel", "float x1 = v[base + i], x2 = v[base + half + i];",
     "float x1 = v[base + i], x2 = v[base + half + (i + 1) % half];", ["rope_pairs"]),
    ("softmax max not subtracted", "double w = exp((double)score[(i * ratio + j) * ld + c] - m);",
     "double w = exp((double)score[(i * ratio + j) * ld + c]); (void)m;", ["pool_mean"]),
    ("pooled row not rounded to bf16", "v[c] = orc_bf16_to_f32(orc_bf16_from_double(p[c]));",
     "v[c] = (float)p[c];", ["compress_r1", "compress_pool_rope"]),
    ("gather row from the wrong slot bits", "int64_t r = slot % kPageRows;", "int64_t r = slot % 32;",
     ["dequant_slots"]),
    ("fp4 code sign dropped in dequant", "(code[c / 2] & 15) : (code[c / 2] >> 4)",
     "(code[c / 2] & 7) : ((code[c / 2] >> 4) & 7)", ["dequant_fp4"]),
    ("dequant scale rows 16 bytes apart", "const uint8_t* scale = pg + kPageRows * cr + r * sr;",
     "const uint8_t* scale = pg + kPageRows * cr + r * 16;", ["dequant_fp4", "dequant_slots"]),
    ("translate maps unknown full slots to 0", "? table[f] : -1;", "? table[f] : 0;", ["translate"]),
    ("rope evaluated in double", "float a = x1 * c, b = x2 * s, d = x2 * c, e = x1 * s;\n        float o1 = a - b, o2 = d + e;",
     "double a = (double)x1 * c, b = (double)x2 * s, d = (double)x2 * c, e = (double)x1 * s;\n"
     "        double o1 = a - b, o2 = d + e;", ["rope_order"]),
    ("rope with fused multiply-add", "float o1 = a - b, o2 = d + e;",
     "float o1 = fmaf(x1, c, -b), o2 = fmaf(x2, c, e); (void)a; (void)d;", ["rope_order"]),
]

PINS = {
    "rope_pairs": lambda o: pins.test_rope_pairs_and_rotation_direction(o),
    "rope_pos0": lambda o: pins.test_rope_position_zero_is_identity(o),
    "rope_order": lambda o: pins.test_rope_rounding_order_worked_example(o, golden),
    "ue8m0": lambda o: pins.test_ue8m0_exhaustive_bf16_amax(o),
    "v41_worked": lambda o: pins.test_v41_worked_examples(o, golden),
    "e4m3_exhaustive": lambda o: pins.test_e4m3_encode_exhaustive_bf16_inputs(o),
    "fp4_worked": lambda o: pins.test_fp4_worked_examples(o, golden),
    "fp4_pairs": lambda o: pins.test_fp4_codes_exhaustive_pairs(o),
    "fp4_scale": lambda o: pins.test_fp4_scale_exhaustive_bf16_amax(o),
    "byte_order": lambda o: pins.test_store_layout_byte_and_nibble_order(o),
    "pool_tiny": lambda o: pins.test_pool_brute_force_tiny(o, 4, 3),
    "pool_window": lambda o: pins.test_pool_window_indexing(o),
    "pool_mean": lambda o: pins.test_pool_equal_scores_give_mean_and_dominant_row_wins(o),
    "addressing": lambda o: (pins.test_addressing_brute_force_with_canaries(o, 1),
                             pins.test_addressing_brute_force_with_canaries(o, 2)),
    "bf16_torch": lambda o: pins.test_bf16_rounding_matches_torch_on_float32(o),
    "bf16_brute": lambda o: pins.test_bf16_rounding_from_double_brute_force(o),
    "dequant_worked": lambda o: pins.test_dequant_worked_examples(o, golden),
    "dequant_v41": lambda o: pins.test_dequant_exhaustive_v41(o),
    "translate": lambda o: pins.test_translate_semantics(o, golden),
    "norm_worked": lambda o: pins.test_norm_worked_examples(o, golden),
    "norm_exact": lambda o: pins.test_norm_is_nearest_bf16_of_exact_value(o),
    "norm_mapping": lambda o: pins.test_norm_scale_invariance_and_weight_mapping(o),
    "compress_r1": lambda o: pins.test_compress_ratio_one_equals_store_rope_of_bf16(o),
    "compress_pool_rope": lambda o: pins.test_compress_equals_pool_then_store_rope(o),
    "dequant_slots": lambda o: (pins.test_dequant_slots_matches_page_dequant(o, 1),
                                pins.test_dequant_slots_matches_page_dequant(o, 2)),
    "dequant_fp4": lambda o: pins.test_dequant_exhaustive_fp4(o),
}


def test_every_pin_name_exists():
    for _, _, _, names in MUTATIONS:
        for n in names:
            assert n in PINS


@pytest.mark.parametrize("name,old,new,pin_names", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(tmp_path, name, old, new, pin_names):
    src = open(oracle_build.SRC).read()
    assert src.count(old) >= 1, f"mutation anchor not found: {old}"
    mutant = tmp_path / "kvq_oracle_mutant.c"
    mutant.write_text(src.replace(old, new))
    lib = tmp_path / "liboracle_mutant.so"
    subprocess.run(oracle_build.command(str(mutant), str(lib)), check=True,
                   stdout=subprocess.DEVNULL, stderr=subprocess.DEVNULL)
    prev = oracle.use_library(str(lib))
    caught = []
    try:
        for pn in pin_names:
            try:
                PINS[pn](oracle)
            except (AssertionError, ValueError) as e:
                caught.append((pn, type(e).__name__))
    finally:
        oracle.use_handle(prev)
    assert caught, f"no pin caught the planted mistake '{name}'"


def test_real_oracle_passes_the_same_pins():
    oracle.lib()
    for fn in PINS.values():
        fn(oracle)
