"""The pins are strong enough: planted mistakes in the oracle are caught.

Each case below edits one line of a private copy of oracle/attn_oracle.c (a
dropped term, a wrong sign, a wrong index, an off-by-one in a mask bound, a
transposed operand ...), compiles it on the CPU, binds it in place of the
real oracle and runs the pin battery of test_oracle_pins.py.  Every mutant
must fail at least one pin; the unmodified source must pass all of them.
"""
import os
import subprocess

import pytest

import oracle
from tests import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "attn_oracle.c")

MUTANTS = {
    "scale_dropped": ("s_row[j] = scale * dot;", "s_row[j] = dot;"),
    "causal_excludes_diagonal": ("    *lo = 0;\n    *hi = i + 1 < N ? i + 1 : N;",
                                 "    *lo = 0;\n    *hi = i < N ? i : N;"),
    "window_off_by_one": ("long long first = i - window + 1;",
                          "long long first = i - window;"),
    "window_not_causal": ("*lo = first > 0 ? first : 0;\n    *hi = i + 1 < N ? i + 1 : N;",
                          "*lo = first > 0 ? first : 0;\n    *hi = N;"),
    "key_channels_transposed": ("dot += qi[c] * kj[c];", "dot += qi[c] * kj[d - 1 - c];"),
    "lse_missing_max": ("*lse_i = m + log(l);", "*lse_i = log(l);"),
    "lse_log2": ("*lse_i = m + log(l);", "*lse_i = m + log2(l);"),
    "no_normalisation": ("for (c = 0; c < d; ++c) oi[c] /= l;", ""),
    "value_row_fixed": ("const double *vj = v + j * d;", "const double *vj = v + lo * d;"),
    "min_instead_of_max": ("if (s_row[j] > m) m = s_row[j];", "if (s_row[j] < m) m = s_row[j];"),
    "exp_sign_flipped": ("double e = exp(s_row[j] - m);", "double e = exp(m - s_row[j]);"),
    "first_key_dropped": ("for (j = lo; j < hi; ++j) {\n    double e",
                          "for (j = lo + 1; j < hi; ++j) {\n    double e"),
    "heads_share_keys": ("const double *kb = k + bh * N * d", "const double *kb = k + 0 * N * d"),
    "value_weight_squared": ("oi[c] += e * vj[c];", "oi[c] += e * e * vj[c];"),
}


def battery():
    """Run a representative subset of the pins; return the names that fail."""
    cases = [
        ("hand", pins.test_hand_worked_example, {}),
        ("mp_none", pins.test_matches_mpmath_bruteforce, dict(N=7, d=4, mask="none", window=0)),
        ("mp_causal", pins.test_matches_mpmath_bruteforce, dict(N=7, d=4, mask="causal", window=0)),
        ("mp_sliding", pins.test_matches_mpmath_bruteforce, dict(N=7, d=4, mask="sliding", window=3)),
        ("const_v", pins.test_constant_values_give_that_constant, dict(mask="causal", window=0)),
        ("zero_scale_w", pins.test_zero_scale_gives_uniform_average, dict(mask="sliding", window=3)),
        ("dominant", pins.test_dominant_logit_selects_its_value, dict(mask="causal", window=0)),
        ("window_one", pins.test_window_one_is_self_attention, {}),
        ("slices", pins.test_slices_are_independent, dict(mask="none", window=0)),
        ("key_shift", pins.test_key_shift_moves_lse_only, dict(mask="none", window=0)),
        ("large_logits", pins.test_large_logits_stay_finite, {}),
    ]
    failed = []
    for name, fn, kw in cases:
        try:
            fn(**kw)
        except Exception:  # assertion or a NaN/inf-driven error
            failed.append(name)
    return failed


def _compile(tmp_path, text, tag):
    src = tmp_path / ("m_%s.c" % tag)
    lib = tmp_path / ("m_%s.so" % tag)
    src.write_text(text)
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
                    "-o", str(lib), str(src), "-lm"], check=True)
    return str(lib)


@pytest.fixture
def swap_oracle():
    saved = oracle._lib
    yield
    oracle._lib = saved


def test_unmodified_source_passes_battery(tmp_path, swap_oracle):
    oracle._lib = oracle.bind(_compile(tmp_path, open(SRC).read(), "orig"))
    assert battery() == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path, swap_oracle):
    old, new = MUTANTS[name]
    text = open(SRC).read()
    assert text.count(old) == 1, "mutation site not unique: %s" % name
    oracle._lib = oracle.bind(_compile(tmp_path, text.replace(old, new), name))
    failed = battery()
    assert failed, "mutant %s passed every pin" % name
