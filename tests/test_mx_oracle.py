"""The MXFP4 CPU oracle against the OCP MX v1.0 definitions (host only), and
mutation tests: each case plants one plausible mistake in a copy of
``oracle/mxfp4_oracle.c`` (on the CPU, never in the GPU path) and requires
that at least one pin rejects the mutated build."""
import os
import subprocess

import pytest

import mx_pins
import oracle

HERE = os.path.dirname(oracle.__file__)
SRC = os.path.join(HERE, "mxfp4_oracle.c")


@pytest.mark.parametrize("pin", mx_pins.MX_PINS, ids=lambda f: f.__name__)
def test_mx_oracle_pin(orc, pin):
    pin(orc)


MUTANTS = {
    "emax_1": [("int code = (e - 1) - 2 + 127;", "int code = (e - 1) - 1 + 127;")],
    "log2_rounded_up": [("int code = (e - 1) - 2 + 127;", "int code = e - 2 + 127;")],
    "no_low_clamp": [("if (code < 0) code = 0;", "if (code < 0) code = 254;")],
    "scale_bias_126": [("return ldexp(1.0, (int)code - 127);", "return ldexp(1.0, (int)code - 126);")],
    "ties_to_odd": [("(d == bd && (c & 1) == 0)", "(d == bd && (c & 1) == 1)")],
    "ties_away": [("if (d < bd || (d == bd && (c & 1) == 0))", "if (d <= bd)")],
    "no_saturation": [("uint32_t best = 7;", "uint32_t best = 0;")],
    "sign_dropped": [("return best | (signbit(v) ? 8u : 0u);", "return best | (v < 0.0 ? 8u : 0u);")],
    "nibble_order_swapped": [("qb[i] = (uint8_t)(lo | (hi << 4));", "qb[i] = (uint8_t)((lo << 4) | hi);")],
    "zero_block_code_127": [("if (!(amax > 0.0)) return 0;", "if (!(amax > 0.0)) return 127;")],
    "linear_operand_transposed": [("s += arow[k] * mx_elem(j->wq, j->wsc, j->K, n, k);",
                                   "s += arow[k] * mx_elem(j->wq, j->wsc, j->K, k % j->N, n % j->K);")],
    "block_scale_per_16": [("return orc_mx_e2m1_value(nib) * orc_mx_scale_value(sc[r * (K / 32) + k / 32]);",
                            "return orc_mx_e2m1_value(nib) * orc_mx_scale_value(sc[r * (K / 32) + (k / 16) % (K / 32)]);")],
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mx_pins_reject_mutant(tmp_path, name):
    src = open(SRC).read()
    for old, new in MUTANTS[name]:
        assert old in src, f"mutant {name}: pattern no longer in the oracle source: {old!r}"
        src = src.replace(old, new)
    cpath = tmp_path / f"{name}.c"
    cpath.write_text(src)
    lib = tmp_path / f"lib_{name}.so"
    subprocess.run(["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fPIC", "-shared", "-pthread", "-I", HERE,
                    "-o", str(lib), str(cpath), os.path.join(HERE, "nvfp4_oracle.c"), "-lm"], check=True)
    o = oracle.Oracle(str(lib))
    caught = None
    for pin in mx_pins.MX_PINS:
        try:
            pin(o)
        except AssertionError:
            caught = pin.__name__
            break
    assert caught is not None, f"no pin rejects the planted mistake {name}"
    print(f"{name}: rejected by {caught}")
