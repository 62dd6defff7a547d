"""Mutation tests for the oracle's pins (host only).

Each case plants one plausible mistake in a copy of the oracle's C source
(on the CPU, never in the GPU path), builds it, and requires that at least
one pin in ``pins.ALL_PINS`` rejects the mutated build.  Several mutants are
the very mistakes the pages record (round-half-up E2M1, the 1/1024 subnormal,
the 480 maximum, a missing mantissa carry).
"""
import os
import subprocess

import pytest

import oracle
import pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "nvfp4_oracle.c")

MUTANTS = {
    "e2m1_round_half_up": [("int hs = (int)nearbyintf(twice);", "int hs = (int)(twice + 0.5f);")],
    "e4m3_subnormal_1024": [("v = (double)m * ldexp(1.0, -9);", "v = (double)m * ldexp(1.0, -10);")],
    "e4m3_bias_8": [("(1.0 + (double)m / 8.0, (int)e - 7)", "(1.0 + (double)m / 8.0, (int)e - 8)")],
    "e4m3_max_480": [("if (e == 15 && m == 7) return NAN;", ""),
                     ("if (a >= 448.0) return 0x7e;", "if (a >= 480.0) return 0x7f;"),
                     ("for (uint32_t c = 0; c <= 0x7e; ++c)", "for (uint32_t c = 0; c <= 0x7f; ++c)")],
    "e4m3_exp15_reserved": [("if (a >= 448.0) return 0x7e;", "if (a >= 240.0) return 0x77;"),
                            ("for (uint32_t c = 0; c <= 0x7e; ++c)", "for (uint32_t c = 0; c <= 0x77; ++c)")],
    "e4m3_ties_to_odd": [("(c & 1u) == 0 && (best & 1u) == 1", "(c & 1u) == 1 && (best & 1u) == 0")],
    "nibble_order_swapped": [("qb[i] = (uint8_t)(nib[2 * i] | (nib[2 * i + 1] << 4));",
                              "qb[i] = (uint8_t)((nib[2 * i] << 4) | nib[2 * i + 1]);")],
    "step_table_10_to_7": [("{0, 1, 2, 3, 4, 4, 5, 6, 6, 6, 6, 7, 7}", "{0, 1, 2, 3, 4, 4, 5, 6, 6, 6, 7, 7, 7}")],
    "step_table_5_to_5": [("{0, 1, 2, 3, 4, 4, 5, 6, 6, 6, 6, 7, 7}", "{0, 1, 2, 3, 4, 5, 5, 6, 6, 6, 6, 7, 7}")],
    "block_scale_over_448": [("float bsf = (bmax / 6.0f) * E;", "float bsf = (bmax / 448.0f) * E;")],
    "global_scale_over_448": [("if (amax > 0.0f) return amax / 2688.0f;", "if (amax > 0.0f) return amax / 448.0f;")],
    "nibble_sign_dropped": [("nib[i] = orc_e2m1_nibble(s, signbit(xb[i]) != 0);", "nib[i] = orc_e2m1_nibble(s, 0);")],
    "multiplier_inverted": [("float r = (sfd == 0.0f) ? 0.0f : E / sfd;", "float r = (sfd == 0.0f) ? 0.0f : sfd / E;")],
    "gate_up_swapped": [("silu(h[gate_col(j)]) * h[up_col(j)]", "silu(h[up_col(j)]) * h[gate_col(j)]")],
    "interleave_group_wrong": [("static int64_t gate_col(int64_t j) { return 16 * (j / 8) + (j % 8); }",
                                "static int64_t gate_col(int64_t j) { return 16 * (j / 8) + ((j + 1) % 8); }")],
    "l1_alpha_dropped": [("h[n] = acc * alpha;", "h[n] = acc;")],
    "l2_alpha_dropped": [("yacc[n] += wt * (acc * alpha2);", "yacc[n] += wt * acc;")],
    "routing_weight_dropped": [("yacc[n] += wt * (acc * alpha2);", "yacc[n] += acc * alpha2;")],
    "dequant_global_scale_dropped": [("out[r * K + c] = v * g;", "out[r * K + c] = v;")],
}


def _build_mutant(tmp_path, name, edits):
    src = open(SRC).read()
    for old, new in edits:
        assert old in src, f"mutant {name}: pattern no longer in the oracle source: {old!r}"
        src = src.replace(old, new)
    cpath = tmp_path / f"{name}.c"
    cpath.write_text(src)
    lib = tmp_path / f"lib_{name}.so"
    inc = os.path.dirname(SRC)
    subprocess.run(["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fPIC", "-shared", "-pthread",
                    "-I", inc, "-o", str(lib), str(cpath), os.path.join(inc, "mxfp4_oracle.c"), "-lm"],
                   check=True)
    return str(lib)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_reject_mutant(tmp_path, name):
    lib = _build_mutant(tmp_path, name, MUTANTS[name])
    o = oracle.Oracle(lib)
    caught = None
    for pin in pins.ALL_PINS:
        try:
            pin(o)
        except AssertionError:
            caught = pin.__name__
            break
    assert caught is not None, f"no pin rejects the planted mistake {name}"
    print(f"{name}: rejected by {caught}")
