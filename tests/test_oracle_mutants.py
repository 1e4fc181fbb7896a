"""Plants plausible mistakes in a copy of the oracle's C source (on the CPU)
and checks that the oracle pins in test_oracle.py catch every one of them."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "vm_oracle.c")

# (name, original text, planted mistake)
MUTANTS = [
    ("drop_D_skip", "y[t] = acc + D * u[t];", "y[t] = acc;"),
    ("exp_sign", "double retain = exp(dt * A[n]);", "double retain = exp(-dt * A[n]);"),
    ("B_C_swapped", "double write = write_coef(dt, A[n], zoh) * B[n * L + t] * u[t];",
     "double write = write_coef(dt, A[n], zoh) * C[n * L + t] * u[t];"),
    ("bias_dropped", "double x = delta[t] + bias;", "double x = delta[t];"),
    ("read_before_update", "      h[n] = retain * h[n] + write;\n      acc += C[n * L + t] * h[n];",
     "      acc += C[n * L + t] * h[n];\n      h[n] = retain * h[n] + write;"),
    ("no_softplus", "return (x > 0.0 ? x : 0.0) + log1p(exp(-fabs(x)));", "return x;"),
    ("reverse_keeps_B_order", "flip_rows(Bb, Bf, N, L);", "memcpy(Bf, Bb, sizeof(double) * (size_t)(N * L));"),
    ("gate_is_sigmoid", "return z / (1.0 + exp(-z));", "return 1.0 / (1.0 + exp(-z));"),
    ("bidir_no_scale", "double y = (yf[i] + yb[i]) * scale;", "double y = (yf[i] + yb[i]);"),
    ("bidir_bwd_not_reversed", "N, delta_softplus, zoh, 1, yb);\n  if (s == 0)\n    for",
     "N, delta_softplus, zoh, 0, yb);\n  if (s == 0)\n    for"),
    ("odd_groups_row_major", "if (group % 2 == 0) {", "if (1) {"),
    ("offsets_swapped", "static const int off_row[4] = {0, 1, 0, 1};", "static const int off_row[4] = {0, 0, 1, 1};"),
    ("pad_not_zero", "? plane[rr[t] * W + cc[t]] : 0.0;", "? plane[rr[t] * W + cc[t]] : 1.0;"),
    ("pool_wrong_extent", "pooled[r * H + i] = s / (double)W;", "pooled[r * H + i] = s / (double)H;"),
    ("repeat_wrong_axis", "int64_t p = axis == 0 ? i : j;", "int64_t p = axis == 0 ? (j % Lp) : (i % Lp);"),
    ("ss2d_columns_as_rows", "pos[t] = k < 2 ? t : (t % H) * W + t / H;", "pos[t] = t;"),
    ("ss2d_no_reverse", "N, delta_softplus, zoh, k % 2, yk);", "N, delta_softplus, zoh, 0, yk);"),
    ("zoh_ignored", "if (!zoh) return dt;", "return dt;"),
    ("zoh_no_divide", "return a != 0.0 ? expm1(dt * a) / a : dt;", "return a != 0.0 ? expm1(dt * a) : dt;"),
    ("zoh_exp_minus_one", "return a != 0.0 ? expm1(dt * a) / a : dt;",
     "return a != 0.0 ? (exp(dt * a) - 1.0) / a : dt;"),
    ("zoh_dropped_in_bidir", "N, delta_softplus, zoh, 1, yb);\n  if (s == 0)\n    for",
     "N, delta_softplus, 0, 1, yb);\n  if (s == 0)\n    for"),
    ("zoh_dropped_in_pool", "Lp,\n                           N, delta_softplus, zoh, 0, yf);",
     "Lp,\n                           N, delta_softplus, 0, 0, yf);"),
    ("zoh_dropped_in_ss2d", "N, delta_softplus, zoh, k % 2, yk);", "N, delta_softplus, 0, k % 2, yk);"),
    ("conv_taps_reversed", "if (s >= 0) v += w[d * 4 + k] * src[s];", "if (s >= 0) v += w[d * 4 + 3 - k] * src[s];"),
    ("conv_no_silu", "dst[t] = silu(v);", "dst[t] = v;"),
    ("conv_shifted_window", "const int64_t s = t - 3 + k;", "const int64_t s = t - 4 + k;"),
    ("conv_reverse_not_flipped_back", "if (reverse) flip_rows(dst, out + row * L, 1, L);",
     "if (0) flip_rows(dst, out + row * L, 1, L);"),
    ("conv_bias_dropped", "double v = bias ? bias[d] : 0.0;", "double v = 0.0;"),
    ("ss2d_overwrite_not_sum", "out[r * L + pos[t]] += yk[r * L + t];", "out[r * L + pos[t]] = yk[r * L + t];"),
]


def test_mutant_list_applies():
    src = open(SRC).read()
    for name, old, new in MUTANTS:
        assert src.count(old) == 1, name


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(tmp_path, name, old, new):
    src = open(SRC).read().replace(old, new)
    c = tmp_path / "mutant.c"
    c.write_text(src)
    so = tmp_path / "libmutant.so"
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", str(c), "-o", str(so), "-lm"])
    env = dict(os.environ, VM_ORACLE_LIB=str(so), OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, f"mutant {name} survived the oracle pins:\n{r.stdout[-2000:]}"
