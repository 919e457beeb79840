"""Planted mistakes in the oracle: the pins must reject each one.

Each mutant is oracle.c with one plausible error written into a copy (a
dropped K block, a wrong scale or row index, a wrong rounding rule, a
routing slip), compiled with gcc into a library of its own and loaded
through a second instance of the oracle's Python module.  The pins named
next to each mutant must fail on it.  This shows the pins would catch such
a mistake in the oracle itself, not only that the oracle passes them.

Every mutant stays within the arrays the oracle is handed, so no mutant can
fault the test process.  CPU only."""
import importlib.util
import itertools
import os

import pytest

from tests import test_oracle_e8m0 as pe8
from tests import test_oracle_formats as pf
from tests import test_oracle_gemm as pg
from tests import test_oracle_quantize as pq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE_C = os.path.join(ROOT, "oracle", "oracle.c")
ORACLE_PY = os.path.join(ROOT, "oracle", "__init__.py")

# name: (text in oracle.c, its replacement, pins that must fail)
MUTANTS = {
    "last_k_block_dropped": (
        "for (int64_t kb = 0; kb < KB; ++kb) {\n            double block = 0.0;",
        "for (int64_t kb = 0; kb < KB - 1; ++kb) {\n            double block = 0.0;",
        [pg.test_unit_scales_equal_fp64_matmul, pg.test_handworked_fixture]),
    "row_scale_of_first_k_block_only": (
        "double scale = (double)sa_row[kb] * (double)sb_row[kb];",
        "double scale = (double)sa_row[0] * (double)sb_row[kb];",
        [pg.test_brute_force_rational_tiny, pg.test_scale_linearity]),
    "column_scale_row_off_at_block_edge": (
        "const float* sb_row = sb + (n / 128) * KB;",
        "const float* sb_row = sb + (n / 129) * KB;",
        [pg.test_sb_row_selection_partial_block]),
    "b_row_shifted_by_one": (
        "const uint8_t* b_row = b + n * K;",
        "const uint8_t* b_row = b + (n > 0 ? n - 1 : 0) * K;",
        [pg.test_unit_scales_equal_fp64_matmul, pg.test_identity_b]),
    "b_reversed_within_a_block": (
        "block += dec[a_row[k]] * dec[b_row[k]];",
        "block += dec[a_row[k]] * dec[b_row[kb * 128 + 127 - (k - kb * 128)]];",
        [pg.test_unit_scales_equal_fp64_matmul, pg.test_exact_integer_case]),
    "addend_joins_after_rounding": (
        "        if (c_row)\n            v += (double)c_row[n];\n        d_row[n] = orc_bf16_from_double(v);",
        "        if (c_row)\n            v = (double)orc_bf16_value(orc_bf16_from_double(v)) + (double)c_row[n];\n"
        "        d_row[n] = orc_bf16_from_double(v);",
        [pg.test_acc_brute_force_rational]),
    "bf16_truncates": (
        "double r = nearbyint(scaled);",
        "double r = trunc(scaled);",
        [pf.test_bf16_exhaustive_exact_midpoints_and_neighbours, pf.test_bf16_matches_torch_on_fp32_inputs]),
    "bf16_ties_away_from_zero": (
        "double r = nearbyint(scaled);",
        "double r = round(scaled);",
        [pf.test_bf16_exhaustive_exact_midpoints_and_neighbours]),
    "e4m3_ties_to_larger_magnitude": (
        "best = (lo & 1) == 0 ? lo : hi;",
        "best = hi;",
        [pf.test_e4m3_rounding_edge_cases, pf.test_e4m3_rounding_matches_torch]),
    "e4m3_overflow_to_nan": (
        "if (a >= 448.0)\n        return (uint8_t)(sign | 0x7E);",
        "if (a > 448.0)\n        return (uint8_t)(sign | 0x7F);",
        [pf.test_e4m3_rounding_edge_cases]),
    "e4m3_subnormal_exponent": (
        "mag = ldexp((double)m / 8.0, -6);",
        "mag = ldexp((double)m / 8.0, -7);",
        [pf.test_e4m3_decode_matches_torch_all_codes]),
    "fnuz_range_in_per_token_scale": (
        "float scale = amax / 448.0f;\n            s[m * KB + kb] = scale;",
        "float scale = amax / 240.0f;\n            s[m * KB + kb] = scale;",
        [pq.test_per_token_against_torch_cast]),
    "per_block_amax_of_first_row_only": (
        "            for (int64_t n = nb * 128; n < n_end; ++n)\n                for (int k = 0; k < 128; ++k) {\n"
        "                    float a = fabsf(",
        "            for (int64_t n = nb * 128; n < nb * 128 + 1; ++n)\n                for (int k = 0; k < 128; ++k) {\n"
        "                    float a = fabsf(",
        [pq.test_per_block_against_torch_cast]),
    "masked_count_one_short": (
        "    if (v > M_max)\n        v = M_max;\n    return v;",
        "    if (v > M_max)\n        v = M_max;\n    return v > 0 ? v - 1 : 0;",
        [pg.test_masked_composes_from_dense]),
    "negative_group_id_read_as_group_0": (
        "        int64_t g = layout[r];\n        if (g < 0 || g >= G)\n            continue;\n"
        "        oracle_row(A + r * K, sa + r * KB, B + g * N * K, sb + g * NB * KB, N, K, D + r * N);",
        "        int64_t g = layout[r];\n        if (g >= G)\n            continue;\n        if (g < 0)\n            g = 0;\n"
        "        oracle_row(A + r * K, sa + r * KB, B + g * N * K, sb + g * NB * KB, N, K, D + r * N);",
        [pg.test_contiguous_composes_from_dense, pg.test_untouched_rows_keep_prefill]),
    "e8m0_exponent_one_high_at_powers": (
        "while ((double)amax > ldexp(448.0, e))",
        "while ((double)amax >= ldexp(448.0, e))",
        [pe8.test_exponent_hand_table]),
}


def _build_mutant(tmp_path_factory, name, old, new):
    src = open(ORACLE_C).read()
    assert src.count(old) >= 1, f"{name}: the text it mutates is no longer in oracle.c"
    d = tmp_path_factory.mktemp(name)
    c_path = d / "oracle.c"
    c_path.write_text(src.replace(old, new, 1))
    spec = importlib.util.spec_from_file_location(f"oracle_mutant_{name}", ORACLE_PY)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    mod._SRC, mod._LIB, mod._lib = str(c_path), str(d / "liborc.so"), None
    mod.build()
    mod._load()
    return mod


def _cases(fn):
    """Every parametrization of a pin, as keyword dicts (one empty dict when
    it has none)."""
    axes = []
    for mark in getattr(fn, "pytestmark", []):
        if mark.name != "parametrize":
            continue
        names, values = mark.args[0], mark.args[1]
        names = [s.strip() for s in names.split(",")] if isinstance(names, str) else list(names)
        axes.append([dict(zip(names, v if len(names) > 1 else (v,))) for v in values])
    if not axes:
        return [{}]
    return [dict(kv for part in combo for kv in part.items()) for combo in itertools.product(*axes)]


def _fails(fn, orc):
    for kw in _cases(fn):
        try:
            fn(orc, **kw)
        except AssertionError:
            return True
    return False


def test_unmutated_copy_passes_the_pins(tmp_path_factory):
    # the harness itself: a copy built and loaded the same way, with nothing
    # changed, passes every pin the mutants are held to
    same = "double r = nearbyint(scaled);"
    mod = _build_mutant(tmp_path_factory, "unmutated", same, same)
    pins = {p for _, _, ps in MUTANTS.values() for p in ps}
    for pin in sorted(pins, key=lambda p: p.__name__):
        assert not _fails(pin, mod), pin.__name__


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_reject_mutant(tmp_path_factory, name):
    old, new, pins = MUTANTS[name]
    mod = _build_mutant(tmp_path_factory, name, old, new)
    survived = [p.__name__ for p in pins if not _fails(p, mod)]
    assert not survived, f"mutant {name} passed {survived}"
