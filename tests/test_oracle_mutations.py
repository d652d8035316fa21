"""The pins catch plausible mistakes: each case plants one slip in a private
copy of the oracle source (CPU only), rebuilds it, and requires at least one
pin of tests/test_oracle_pins.py to fail against that build."""

import ctypes
import os
import subprocess

import pytest

import oracle
from oracle.build import SRC
from tests import test_oracle_pins as pins

# (name, text in lora_oracle.cpp, replacement)
MUTATIONS = [
    ("scale dropped",
     "buf[(static_cast<int64_t>(s) * num_tokens + t) * rank + k] = scale * acc;",
     "buf[(static_cast<int64_t>(s) * num_tokens + t) * rank + k] = acc;"),
    ("expand sign flipped",
     "delta += brow[k] * widen_bf16(wrow[k]);",
     "delta -= brow[k] * widen_bf16(wrow[k]);"),
    ("last rank term dropped",
     "for (int32_t k = 0; k < rank; ++k) delta +=",
     "for (int32_t k = 0; k + 1 < rank; ++k) delta +="),
    ("A indexed transposed",
     "lora_a[s] + (static_cast<int64_t>(l) * rank + k) * hidden",
     "lora_a[s] + (static_cast<int64_t>(k) * max_loras + l) * hidden"),
    ("B indexed transposed",
     "lora_b[s] + (static_cast<int64_t>(l) * n_s + n) * rank",
     "lora_b[s] + (static_cast<int64_t>(n) * max_loras + l) * rank"),
    ("slice offset not advanced",
     "        off += n_s;\n",
     "\n"),
    ("unstable grouping (reverse visit)",
     "  for (int64_t t = 0; t < num_tokens; ++t) {\n    const int g = adapter_of(mapping, t, max_loras) + 1;",
     "  for (int64_t t = num_tokens - 1; t >= 0; --t) {\n    const int g = adapter_of(mapping, t, max_loras) + 1;"),
    ("rounding through float32 first",
     "  const double a = std::fabs(v);\n  if (a == 0.0) return sign;",
     "  const double a = std::fabs(static_cast<double>(static_cast<float>(v)));\n  if (a == 0.0) return sign;"),
    ("ties rounded away from zero",
     "const double r = std::nearbyint(std::ldexp(a, -q));",
     "const double r = std::round(std::ldexp(a, -q));"),
    ("padding start zero",
     "    lora_token_start[i] = num_tokens;",
     "    lora_token_start[i] = 0;"),
    ("out-of-range ids sent to adapter 0",
     "return (m >= -1 && m < max_loras) ? m : -1;",
     "return (m >= -1 && m < max_loras) ? m : 0;"),
    ("y0 not added",
     "const double v = widen_bf16(yin[off + n]) + delta;",
     "const double v = delta;"),
]

PIN_FUNCS = [
    lambda: pins.test_round_bf16_ieee_values(1 + 2**-8 + 2**-40, 0x3F81),
    lambda: pins.test_round_bf16_ieee_values(1 + 2**-8, 0x3F80),
    pins.test_round_bf16_matches_exact_rational_rounding,
    pins.test_metadata_worked_example,
    pins.test_metadata_padding_slots,
    lambda: pins.test_metadata_matches_library_routines("wild", 1000, 16),
    pins.test_single_adapter_equals_dense_product,
    pins.test_per_adapter_dense_loop_equals_oracle,
    pins.test_rows_without_adapter_are_untouched,
    pins.test_rank_one_closed_form,
    pins.test_exact_rational_brute_force_tiny,
    lambda: pins.test_integer_exact_mode_matches_integer_arithmetic(8, 1.0),
    pins.test_golden_tiny_exact_values,
]


def _build_variant(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name!r} not found exactly once"
    path = tmp_path / "mut.cpp"
    path.write_text(src.replace(old, new))
    so = tmp_path / "libmut.so"
    subprocess.run(["g++", "-O1", "-std=c++17", "-fPIC", "-shared", "-pthread",
                    "-ffp-contract=off", str(path), "-o", str(so)], check=True)
    return oracle.configure(ctypes.CDLL(str(so)))


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_planted_mistake(tmp_path, monkeypatch, name, old, new):
    mutant = _build_variant(tmp_path, name, old, new)
    monkeypatch.setattr(oracle, "_lib", mutant)
    caught = []
    for f in PIN_FUNCS:
        try:
            f()
        except (AssertionError, ValueError, IndexError):
            caught.append(f)
    assert caught, f"no pin failed with the planted mistake: {name}"


def test_unmutated_source_passes_every_pin(tmp_path, monkeypatch):
    monkeypatch.setattr(oracle, "_lib", _build_variant(tmp_path, "none", "extern \"C\" {",
                                                       "extern \"C\" {"))
    for f in PIN_FUNCS:
        f()
