"""Plants one plausible mistake at a time in a copy of the C oracle, builds the
copy, and checks that the pins in test_oracle_pins.py reject it.  This shows
the pins are tied to the pages and to mathematics rather than to the oracle's
own code.  Everything here runs on the CPU."""
import os

import numpy as np
import pytest

import oracle
import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "mrr_oracle.c")

# (name, original text, planted mistake)
MUTANTS = [
    ("rank order reversed",
     "float a = (float)load_value(in[0], i, tin);",
     "float a = (float)load_value(in[nranks - 1], i, tin);"),
    ("rank order: peers reversed",
     "float x = (float)load_value(in[r], i, tin);",
     "float x = (float)load_value(in[nranks - r], i, tin);"),
    ("accumulator starts at +0",
     "float a = (float)load_value(in[0], i, tin);",
     "float a = 0.0f + (float)load_value(in[0], i, tin);"),
    ("last rank dropped",
     "for (int r = 1; r < nranks; ++r) {",
     "for (int r = 1; r < nranks - 1; ++r) {"),
    ("native accumulation not rounded",
     "for (int r = 1; r < nranks; ++r) a = round_to(acc, a + load_value(in[r], i, tin));",
     "for (int r = 1; r < nranks; ++r) a = a + load_value(in[r], i, tin);\n  a = round_to(acc, a);"),
    ("fp8 bias 14", "else v = ldexp(1.0 + (double)m / 8.0, e - 15);",
     "else v = ldexp(1.0 + (double)m / 8.0, e - 14);"),
    ("fp8 subnormal scale", "else if (e == 0) v = ldexp((double)m / 8.0, -14);",
     "else if (e == 0) v = ldexp((double)m / 8.0, -15);"),
    ("fp8 saturation lost",
     "if (a >= fp8_tab[FP8_NFIN - 1]) return s | (uint8_t)(FP8_NFIN - 1);",
     "if (a >= fp8_tab[FP8_NFIN - 1]) return s | (uint8_t)0x78;"),
    ("f16 subnormal scale", "else if (e == 0) v = ldexp((double)m, -24);",
     "else if (e == 0) v = ldexp((double)m, -25);"),
    ("f16 bias 16", "else v = ldexp(1.0 + (double)m / 1024.0, e - 15);",
     "else v = ldexp(1.0 + (double)m / 1024.0, e - 16);"),
    ("ties away from zero", "return (lo % 2 == 0) ? lo : hi;", "return hi;"),
    ("ties toward zero", "return (lo % 2 == 0) ? lo : hi;", "return lo;"),
    ("bf16 overflow threshold", "bf16_tab[BF16_NFIN] = ldexp(1.0, 128);",
     "bf16_tab[BF16_NFIN] = ldexp(1.0, 129);"),
    ("packet flag in the low word", "return ((uint64_t)flag << 32) | (uint64_t)word;",
     "return ((uint64_t)word << 32) | (uint64_t)flag;"),
    ("packet tail not zero-padded", "uint32_t byte = at < nbytes ? src[at] : 0;",
     "uint32_t byte = at < nbytes ? src[at] : 0xFF;"),
    ("scratch indexed [src][dst]", "((size_t)d * nranks + s) * npkt;",
     "((size_t)s * nranks + d) * npkt;"),
    ("e4m3fn bias 8", "else v = ldexp(1.0 + (double)m / 8.0, e - 7);",
     "else v = ldexp(1.0 + (double)m / 8.0, e - 8);"),
    ("e4m3fn NaN code finite", "if (e == 0xF && m == 7) v = NAN;", "if (e == 0xF && m == 8) v = NAN;"),
    ("two-phase scratch indexed [src][dst]", "rs[((size_t)c * nranks + d) * cw + k] =",
     "rs[((size_t)d * nranks + c) * cw + k] ="),
    ("two-phase all-gather of the input", "make_packet(word_at((const uint8_t*)outputs[0], nbytes, w), flag);",
     "make_packet(word_at((const uint8_t*)inputs[c], nbytes, w), flag);"),
    ("fp8 encode rounds twice, through f16", "case ORC_FP8: b[0] = narrow_fp8(v); break;",
     "case ORC_FP8: b[0] = narrow_fp8(f16_value(narrow_f16(v))); break;"),
    ("full-mesh inbox indexed [src][dst]",
     "uint8_t* slot = inbox + (dst * n + src) * chunk * (size_t)e;",
     "uint8_t* slot = inbox + (src * n + dst) * chunk * (size_t)e;"),
    ("full-mesh inbox holds the receiver's own chunk",
     "const uint8_t* in = (const uint8_t*)inputs[src];",
     "const uint8_t* in = (const uint8_t*)inputs[dst];"),
    ("full-mesh semaphore flag in the low word",
     "sem[(dst * n + src) * 1024 + (size_t)b] = (uint64_t)flag << 32;",
     "sem[(dst * n + src) * 1024 + (size_t)b] = (uint64_t)flag;"),
    ("full-mesh last block not signalled", "for (int b = 0; b < nblocks; ++b) sem[",
     "for (int b = 0; b + 1 < nblocks; ++b) sem["),
]


def _checks():
    """The pins, bound to fixed parameters, cheapest first."""
    return [
        pins.test_fp8_format_facts_from_pages,
        pins.test_fp8_decode_matches_fp16_route,
        pins.test_fp8_worked_values,
        pins.test_fp8_encode_ties_and_saturation,
        pins.test_fp8_encode_all_f16_inputs_brute_force,
        pins.test_fp8_encode_f32_midpoints_and_random,
        pins.test_f16_decode_all_codes,
        pins.test_bf16_decode_all_codes,
        pins.test_f16_narrow_from_f64_vs_numpy,
        pins.test_bf16_narrow_from_f32_vs_torch,
        pins.test_rank_order_pin_f32,
        pins.test_signed_zero_and_cancellation,
        lambda o: pins.test_constant_buffers_sum_to_n_times_c(o, 8, "f16", 0.5),
        lambda o: pins.test_constant_fp8_buffers(o, 32),
        lambda o: pins.test_f32_sum_vs_numpy_sequential(o, 8),
        lambda o: pins.test_f16_sum_vs_numpy(o, 4),
        lambda o: pins.test_fp8_native_and_f16_accumulation(o),
        pins.test_pack_layout_worked_example,
        pins.test_pack_unpack_roundtrip,
        lambda o: pins.test_allreduce_packet_expectation(o, "f16", 1001),
        lambda o: pins.test_packet_rsag_expectation(o, "f16", 1001, 4),
        lambda o: pins.test_fullmesh_expectation(o, "f16", 1001, 4, 3),
        pins.test_fp8fn_decode_vs_torch,
        pins.test_fp8fn_encode_all_f16_brute_force_and_torch,
    ]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_reject_planted_mistake(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, "mutation site for %r not unique" % name
    mutant_src = tmp_path / "mutant.c"
    mutant_src.write_text(src.replace(old, new))
    lib = oracle.build(force=True, src=str(mutant_src), out=str(tmp_path / "mutant.so"))
    orc = oracle.load(lib)
    for check in _checks():
        try:
            check(orc)
        except (AssertionError, ValueError):
            return  # a pin caught it
    pytest.fail("no pin rejected the planted mistake: %s" % name)


def test_unmutated_oracle_passes_every_check(orc):
    for check in _checks():
        check(orc)
