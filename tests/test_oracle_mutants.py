"""Plausible mistakes planted in copies of the oracle must each fail a pin.

Each mutant is oracle.c with one small edit (a dropped term, a wrong sign or
index, a transposed operand), built with gcc into a temporary directory. Every
mutant keeps its memory accesses inside the arrays, so a failing pin is an
assertion, never a crash. The
real oracle passes every pin (test_oracle.py); here every mutant must fail at
least one, which shows the pins can tell a wrong oracle from the right one.
"""
import os
import subprocess

import pytest

import oracle
import oracle_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

# (name, text to replace, replacement) -- each must occur in oracle.c.
MUTANTS = [
    ("flipped_filter", "w[(size_t)(((k * C + c) * R + u) * S + v)]",
     "w[(size_t)(((k * C + c) * R + (R - 1 - u)) * S + (S - 1 - v))]"),
    ("transposed_taps", "w[(size_t)(((k * C + c) * R + u) * S + v)]",
     "w[(size_t)(((k * C + c) * S + v) * R + u)]"),
    ("row_offset_off_by_one", "const int64_t ii = i + u - ph;", "const int64_t ii = i + u - ph + 1;"),
    ("col_pad_from_rows", "pw = (S - 1) / 2;", "pw = (R - 1) / 2;"),
    ("dropped_bias", "double out = sum + bias;", "double out = sum;"),
    ("bias_sign", "double out = sum + bias;", "double out = sum - bias;"),
    ("replicate_border", "if (ii < 0 || ii >= H || jj < 0 || jj >= W) continue; /* zero padding */",
     "const int64_t ic = ii < 0 ? 0 : (ii >= H ? H - 1 : ii); const int64_t jc = jj < 0 ? 0 : (jj >= W ? W - 1 : jj); (void)ic; (void)jc; if (ii < 0 || ii >= H) continue;"),
    ("dropped_last_channel", "for (int64_t c = 0; c < C; ++c) {", "for (int64_t c = 0; c < (C > 1 ? C - 1 : C); ++c) {"),
    ("dropped_last_tap", "for (int64_t v = 0; v < S; ++v) {", "for (int64_t v = 0; v < (S > 1 ? S - 1 : S); ++v) {"),
    ("relu_inverted", "if (relu && out < 0.0) out = 0.0;", "if (relu && out > 0.0) out = 0.0;"),
    ("relu_before_bias", "double out = sum + bias;\n  if (relu && out < 0.0) out = 0.0;",
     "double out = sum;\n  if (relu && out < 0.0) out = 0.0;\n  out += bias;"),
    ("scale_without_abs", "mag += fabs(p);", "mag += p;"),
    ("scale_without_bias", "*m_out = mag + fabs(bias);", "*m_out = mag;"),
    ("nhwc_read_as_nchw", "return (size_t)(((n * H + i) * W + j) * C + c);", "return (size_t)(((n * C + c) * H + i) * W + j);"),
    ("product_as_sum", "const double p = wv * xv;", "const double p = wv + xv;"),
]


def _build(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) >= 1, "mutation %s does not apply" % name
    msrc = src.replace(old, new, 1)
    cpath = tmp_path / (name + ".c")
    cpath.write_text(msrc)
    lib = tmp_path / ("lib" + name + ".so")
    subprocess.run(["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared",
                    "-w", "-o", str(lib), str(cpath), "-lm"], check=True)
    return oracle.load_library(str(lib))


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_fails_a_pin(tmp_path, name, old, new):
    lib = _build(tmp_path, name, old, new)

    def conv(x, w, b, relu, layout):
        return oracle.conv2d(x, w, b, relu, layout, lib=lib)

    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(conv)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, "mutant %s passed every pin" % name
