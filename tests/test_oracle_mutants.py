"""Plant plausible mistakes in copies of oracle.c and check that the pins catch
each one (CPU only).  A mutant that every pin accepts would mean the pins do not
constrain that part of the oracle."""
import os
import subprocess
import sys

import pytest

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
from oracle_pins import ALL_PINS  # noqa: E402

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

# (name, text in oracle.c, replacement): one mistake each
MUTANTS = [
    ("causal_off_by_one", "return !causal || j <= i;", "return !causal || j < i;"),
    ("k_v_swapped_in_logits", "e[j] = scale * dot(qi, kh + j * d, d);",
     "e[j] = scale * dot(qi, vh + j * d, d);"),
    ("no_normalisation", "for (int64_t t = 0; t < d; ++t) oi[t] /= l;", ""),
    ("lse_sign", "lse[r] = m + log(l);", "lse[r] = m - log(l);"),
    ("exact_drops_max_shift", "e[j] = key_valid(i, j, causal) ? exp(e[j] - m) : 0.0;",
     "e[j] = key_valid(i, j, causal) ? exp(e[j]) : 0.0;"),
    ("alpha_not_applied_to_l", "                            l[a] *= alpha;\n                            for",
     "                            for"),
    ("alpha_not_applied_to_O",
     "                            for (int64_t u = 0; u < d; ++u) O[a * d + u] *= alpha;\n                        }\n                        mhat = mhat_new;",
     "                        }\n                        mhat = mhat_new;"),
    ("alpha_inverted", "exp2(c * (mhat - mhat_new))", "exp2(c * (mhat_new - mhat))"),
    ("z_sign", "double z = c * x - c * mhat;", "double z = c * x + c * mhat;"),
    ("natural_exp_for_exp2", "round_p(exp2(z), p_round, p_shift);\n                            }\n                    }",
     "round_p(exp(z), p_round, p_shift);\n                            }\n                    }"),
    ("tilemax_is_min", "if (m[a] > mhat_new) mhat_new = m[a];", "if (m[a] < mhat_new || mhat_new == -INFINITY) mhat_new = m[a];"),
    ("tilemax_skips_last_row", "if (m[a] > mhat_new) mhat_new = m[a];",
     "if (a + 1 < nt && m[a] > mhat_new) mhat_new = m[a];"),
    ("per_row_ref_not_updated", "                        ref[a] = m[a];\n", ""),
    ("fallback_trigger_inverted", "c * (mhat_new - mmin) > tau", "c * (mhat_new - mmin) < tau"),
    ("lse_shift_sign", "- p_shift * 0.69314718055994530941723212145818", "+ p_shift * 0.69314718055994530941723212145818"),
    ("bf16_one_bit_short", "r = ldexp(nearbyint(ldexp(f, 8)), e - 8);", "r = ldexp(nearbyint(ldexp(f, 7)), e - 7);"),
    ("e4m3_no_subnormals", "r = ldexp(nearbyint(ldexp(ax, 9)), -9);", "r = 0.0;"),
    ("f16_bf16_precision", "r = ldexp(nearbyint(ldexp(f, 11)), e - 11);",
     "r = ldexp(nearbyint(ldexp(f, 8)), e - 8);"),
    ("f16_no_overflow", "if (r > 65504.0) r = INFINITY;", ""),
    ("f16_model_is_bf16", "case 3: return oracle_round_f16(ldexp(p, p_shift));",
     "case 3: return oracle_round_bf16(ldexp(p, p_shift));"),
    ("flushed_row_gets_nan", "for (int64_t u = 0; u < d; ++u) oi[u] = 0.0;\n                    lse[row] = -INFINITY;",
     "for (int64_t u = 0; u < d; ++u) oi[u] = O[a * d + u] / l[a];\n                    lse[row] = -INFINITY;"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    import oracle
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not unique/found"
    path = tmp_path / "mutant.c"
    path.write_text(src.replace(old, new))
    lib = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", str(path),
                    "-o", str(lib), "-lm"], check=True)
    orc = oracle.Oracle(str(lib))
    caught = []
    for pin in ALL_PINS:
        try:
            pin(orc)
        except (AssertionError, ValueError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passes every pin"
