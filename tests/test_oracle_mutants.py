"""Planted mistakes in the CPU oracle must be caught by its pins.

Each case copies ``oracle/mxfp8_oracle.c``, applies one plausible mistake
(a dropped term, a wrong sign, index or rounding rule), builds the copy with
gcc in a temporary directory and runs the quick pin battery from
``oracle_pins`` on it in a child process.  The child must fail.  Nothing here
touches the GPU.
"""
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTANTS = {
    "scale_off_by_one": ("floor_log2(amax) - E4M3_EMAX + E8M0_BIAS",
                         "floor_log2(amax) - E4M3_EMAX + E8M0_BIAS + 1"),
    "ties_away_from_zero": ("(frac == 0.5 && fmod(m, 2.0) == 1.0)", "(frac == 0.5)"),
    "truncate": ("if (frac > 0.5 || (frac == 0.5 && fmod(m, 2.0) == 1.0)) m += 1.0;", ""),
    "subnormal_grid": ("if (e < -6) e = -6;", "if (e < -7) e = -7;"),
    "overflow_to_nan": ("if (a >= E4M3_MAX) return sign | 0x7E;",
                        "if (a >= E4M3_MAX) return sign | 0x7F;"),
    "no_low_clamp": ("if (s < 0) s = 0;", ""),
    "scale_applied_backwards": ("ldexp(v[i], E8M0_BIAS - sb)", "ldexp(v[i], sb - E8M0_BIAS)"),
    "exponent_bias": ("((er + 7) << 3)", "((er + 8) << 3)"),
    "zero_sign_lost": ("uint8_t sign = signbit(v) ? 0x80 : 0x00;",
                       "uint8_t sign = v < 0 ? 0x80 : 0x00;"),
    "colwise_scale_transposed": ("s + i * cols + c);", "s + c * nb + i);"),
    "nan_block_sign_lost": ("b = (signbit(v[i]) ? 0x80 : 0x00) | 0x7F;", "b = 0x7F;"),
    "amax_signed": ("double a = fabs(v[i]);", "double a = v[i];"),
    "subnormal_code": ("r / ldexp(1.0, -9)", "r / ldexp(1.0, -10)"),
    "rms_eps_dropped": ("ss / (double)cols + (double)eps", "ss / (double)cols"),
    "rms_sum_not_mean": ("ss / (double)cols + (double)eps", "ss + (double)eps"),
    # float32 accumulation of the squares: overflows for rows near 2^64 and
    # flushes rows below 2^-75
    "rms_sum_in_float32": ("double ss = 0.0;\n    for (int64_t c = 0; c < cols; ++c) {\n        double v = bf16_value(x_row[c]);\n        ss += v * v;\n    }",
                           "float ss = 0.0f;\n    for (int64_t c = 0; c < cols; ++c) {\n        float v = (float)bf16_value(x_row[c]);\n        ss += v * v;\n    }"),
    "rms_offset_sign": ("(bf16_value(gamma[c]) + (double)weight_offset)",
                        "(bf16_value(gamma[c]) - (double)weight_offset)"),
    "dequant_exponent": ("ldexp(1.0 + m / 8.0, ef - 7)", "ldexp(1.0 + m / 8.0, ef - 8)"),
    "dequant_col_index": ("s[(r / MX_BLOCK) * cols + c]", "s[(r / MX_BLOCK) * cols + (cols - 1 - c)]"),
    "bf16_precision": ("round_half_even_to(a, ldexp(1.0, e - 7))",
                       "round_half_even_to(a, ldexp(1.0, e - 8))"),
    "gemm_b_scale_index": ("e8m0_value(sb[n * (K / MX_BLOCK) + k / MX_BLOCK])",
                           "e8m0_value(sb[m * (K / MX_BLOCK) + k / MX_BLOCK])"),
    "gemm_reversed_k": ("e4m3_value(qb[n * K + k])", "e4m3_value(qb[n * K + (K - 1 - k)])"),
    "f32_through_bf16": ("for (int i = 0; i < n; ++i) v[i] = (double)x[(int64_t)i * stride];",
                         "for (int i = 0; i < n; ++i) { uint32_t u; memcpy(&u, &x[(int64_t)i * stride], 4);"
                         " v[i] = bf16_value((uint16_t)(u >> 16)); }"),
}

_CHILD = r"""
import sys
sys.path.insert(0, {root!r})
import oracle
from tests import oracle_pins as P
o = oracle.Oracle({lib!r})
failed = []
for name, fn in P.QUICK_CHECKS:
    try:
        fn(o)
    except Exception as e:
        failed.append(name)
print("FAILED_CHECKS", failed)
sys.exit(3 if failed else 0)
"""


def _run_mutant(name, tmp):
    old, new = MUTANTS[name]
    src = open(oracle.SOURCE).read()
    assert src.count(old) >= 1, "mutation site for %s not found" % name
    path = os.path.join(tmp, name + ".c")
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    lib = oracle.build(force=True, src=path, out=os.path.join(tmp, name + ".so"))
    env = dict(os.environ, OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-c", _CHILD.format(root=ROOT, lib=lib)],
                       capture_output=True, text=True, timeout=600, env=env)
    return name, r.returncode, r.stdout[-400:] + r.stderr[-400:]


@pytest.mark.slow
def test_every_planted_mistake_is_caught():
    with tempfile.TemporaryDirectory() as tmp:
        with ThreadPoolExecutor(max_workers=4) as ex:
            results = list(ex.map(lambda n: _run_mutant(n, tmp), sorted(MUTANTS)))
    survivors = [(n, out) for n, rc, out in results if rc == 0]
    assert not survivors, "mistakes the pins did not catch: %s" % survivors


def test_unmutated_copy_passes_the_battery():
    with tempfile.TemporaryDirectory() as tmp:
        lib = oracle.build(force=True, src=oracle.SOURCE, out=os.path.join(tmp, "same.so"))
        r = subprocess.run([sys.executable, "-c", _CHILD.format(root=ROOT, lib=lib)],
                           capture_output=True, text=True, timeout=600)
        assert r.returncode == 0, r.stdout[-800:] + r.stderr[-800:]
