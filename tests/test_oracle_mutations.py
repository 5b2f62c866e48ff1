"""The oracle's pins catch plausible mistakes (CPU only).

Each case plants one mistake in a copy of oracle/mx_oracle.cpp, builds it, and
runs the named pin tests against that build (through MX_ORACLE_LIB) in a
subprocess; the pins must fail.  A control build of the unchanged source must
pass the same tests.  The mistakes: a wrong rounding rule, a wrong
saturation bound, a dropped sign, a wrong subnormal grid, wrong exponent
biases, a strict instead of a non-strict scale bound, a signed amax, a
reversed block, a dropped scale in the GEMM, a block that reaches past its
group, groups sharing columns, the E4M3 limit used for E5M2 scales, and the
MoE backward's E5M2 paths falling back to E4M3 or mixing up the operands'
element types.
"""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "mx_oracle.cpp")
F = "tests/test_oracle_formats.py"
Q = "tests/test_oracle_quant.py"
G = "tests/test_oracle_gemm.py"
MB = "tests/test_oracle_moe_backward.py"
E5 = "tests/test_oracle_e5m2.py"

MUTATIONS = [
    ("rounding ties away from zero",
     "double k = nearbyint(ldexp(a, -p)); /* default rounding mode: ties to even */",
     "double k = round(ldexp(a, -p));",
     [F + "::test_e4m3_round_brute_force"]),
    ("saturation above 448",
     "if (a >= 448.0)\n        return sign | 0x7E;",
     "if (a >= 480.0)\n        return sign | 0x7E;",
     [F + "::test_e4m3_round_brute_force"]),
    ("sign of zero dropped",
     "double r = ldexp(k, p);             /* the rounded magnitude, <= 448 here */\n    if (r == 0.0)\n        return sign;",
     "double r = ldexp(k, p);             /* the rounded magnitude, <= 448 here */\n    if (r == 0.0)\n        return 0;",
     [F + "::test_e4m3_round_spot_values"]),
    ("subnormal grid 2^-10",
     "p = -9;", "p = -10;",
     [F + "::test_e4m3_round_brute_force"]),
    ("E4M3 subnormal decode",
     "mag = ldexp(M / 8.0, -6);", "mag = ldexp(M / 8.0, -7);",
     [F + "::test_e4m3_decode_matches_torch_and_spot_values"]),
    ("BF16 exponent bias",
     "mag = ldexp(1.0 + m / 128.0, E - 127);", "mag = ldexp(1.0 + m / 128.0, E - 126);",
     [F + "::test_bf16_decode_matches_torch"]),
    ("E8M0 bias",
     "return ldexp(1.0, (int)b - 127);", "return ldexp(1.0, (int)b - 128);",
     [F + "::test_e8m0_decode_matches_torch"]),
    ("strict scale bound",
     "while (e < 127 && amax > ldexp(emax_value, e))",
     "while (e < 127 && amax >= ldexp(emax_value, e))",
     [F + "::test_rceil_spot_values"]),
    ("signed amax",
     "if (fabs(v[i]) > amax)\n            amax = fabs(v[i]);",
     "if (v[i] > amax)\n            amax = v[i];",
     [Q + "::test_row_matches_library_quantiser"]),
    ("column block reversed",
     "v[k] = orc_bf16_value(x[(32 * i + k) * C + c]);",
     "v[k] = orc_bf16_value(x[(32 * i + 31 - k) * C + c]);",
     [Q + "::test_col_is_row_of_transpose"]),
    ("GEMM drops the B scale",
     "return elem_value(elem, b[n * K + k]) * orc_e8m0_value(sb[n * (K / 32) + k / 32]);",
     "return elem_value(elem, b[n * K + k]);",
     [G + "::test_gemm_matches_numpy_float64"]),
    ("group block reaches past its group",
     "const int n = (int)((rows - 32 * j) < 32 ? (rows - 32 * j) : 32);",
     "const int n = (int)((T - o - 32 * j) < 32 ? (T - o - 32 * j) : 32);",
     [MB + "::test_partial_blocks_hand_values"]),
    ("groups share columns",
     "return 128 * (o_g / 128 + g);", "return 128 * (o_g / 128);",
     [MB + "::test_grouped_col_equals_col_of_padded_matrix"]),
    ("E5M2 scaled against 448",
     "return rceil_for(amax, 57344.0);", "return rceil_for(amax, 448.0);",
     [E5 + "::test_e5m2_layouts"]),
    ("grouped column blocks ignore the element type",
     "s_t[c * nbc + P / 32 + j] = quant_block_elem(elem, n, v, codes);",
     "s_t[c * nbc + P / 32 + j] = quant_block_elem(ELEM_E4M3, n, v, codes);",
     [MB + "::test_grouped_col_e5m2_equals_col_of_padded_matrix"]),
    ("weight gradient decodes B with A's element type",
     "elem_value(b_elem, b[n * cap + k])", "elem_value(a_elem, b[n * cap + k])",
     [MB + "::test_wgrad_elem_matches_numpy_per_group"]),
]


def _build(tmp_path, name, text):
    src = tmp_path / f"{name}.cpp"
    src.write_text(text)
    lib = tmp_path / f"{name}.so"
    subprocess.check_call([oracle.CXX, *oracle.CFLAGS, "-o", str(lib), str(src), "-lm"])
    return str(lib)


def _run_pins(lib, tests):
    env = dict(os.environ, MX_ORACLE_LIB=lib)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", *tests],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    return r.returncode, r.stdout[-2000:]


@pytest.fixture(scope="module")
def source():
    return open(SRC).read()


def test_control_build_passes_every_selected_pin(tmp_path, source):
    lib = _build(tmp_path, "control", source)
    tests = sorted({t for *_, ts in MUTATIONS for t in ts})
    rc, out = _run_pins(lib, tests)
    assert rc == 0, out


@pytest.mark.parametrize("name,old,new,tests", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_mutation_is_caught(tmp_path, source, name, old, new, tests):
    assert source.count(old) == 1, f"mutation site not unique: {name}"
    lib = _build(tmp_path, "mutant", source.replace(old, new))
    rc, out = _run_pins(lib, tests)
    assert rc == 1 and " failed" in out, f"{name} was not caught:\n{out}"
