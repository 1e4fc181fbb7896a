"""Plants plausible mistakes in a copy of the gradient oracle (oracle/grad.py,
on the CPU) and checks that the finite-difference pins in
test_oracle_grad.py catch every one of them."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "grad.py")

# (name, original text, planted mistake, -k expression selecting the pins
# that must catch it)
MUTANTS = [
    ("zoh_dropped_in_pool_fwd", "y = _direction_y(pooled(lf), delta_softplus, False, zoh)",
     "y = _direction_y(pooled(lf), delta_softplus, False)", "zoh and pool"),
    ("zoh_dropped_in_pool_bwd", "y = y + _direction_y(pooled(lb), delta_softplus, True, zoh)",
     "y = y + _direction_y(pooled(lb), delta_softplus, True)", "zoh and pool"),
    ("zoh_dropped_in_ss2d", "y = _direction_y([seq] + lv, delta_softplus, k % 2 == 1, zoh)",
     "y = _direction_y([seq] + lv, delta_softplus, k % 2 == 1)", "zoh and ss2d"),
    ("zoh_dropped_in_bidir_bwd", "_direction_y(lb, delta_softplus, True, zoh))",
     "_direction_y(lb, delta_softplus, True))", "zoh and bidir"),
    ("zoh_series_wrong_term", "1 + x * (1 / 2 + x * (1 / 6", "1 + x * (1 / 3 + x * (1 / 6", "zoh"),
    ("zoh_no_divide", "torch.expm1(xs) / xs)", "torch.expm1(xs))", "zoh"),
    ("write_uses_C", "h = a * h + k * B[:, None, :, t] * u[:, :, t, None]",
     "h = a * h + k * C[:, None, :, t] * u[:, :, t, None]", "single"),
    ("read_before_update",
     "        h = a * h + k * B[:, None, :, t] * u[:, :, t, None]\n"
     "        ys.append((C[:, None, :, t] * h).sum(-1) + D[None, :] * u[:, :, t])",
     "        ys.append((C[:, None, :, t] * h).sum(-1) + D[None, :] * u[:, :, t])\n"
     "        h = a * h + k * B[:, None, :, t] * u[:, :, t, None]", "single"),
    ("skip_dropped", "ys.append((C[:, None, :, t] * h).sum(-1) + D[None, :] * u[:, :, t])",
     "ys.append((C[:, None, :, t] * h).sum(-1))", "single"),
    ("reverse_not_flipped_back", "return f(_scan_loop(f(u), f(dl), A, f(B), f(C), D, bias, delta_softplus, zoh))",
     "return _scan_loop(f(u), f(dl), A, f(B), f(C), D, bias, delta_softplus, zoh)", "single"),
    ("pool_extent_swapped", "w = u.shape[3] if pool_axis == 0 else u.shape[2]",
     "w = u.shape[2] if pool_axis == 0 else u.shape[3]", "pool"),
    ("pool_repeat_axis_swapped", "rep = y[:, :, :, None] if pool_axis == 0 else y[:, :, None, :]",
     "rep = y[:, :, None, :] if pool_axis == 0 else y[:, :, :, None]", "pool"),
    ("ss2d_columns_not_transposed", "seq = (ut if k < 2 else ut.transpose(2, 3)).reshape(batch, dim, H * W)",
     "seq = ut.reshape(batch, dim, H * W)", "ss2d"),
    ("ss2d_no_reverse", "y = _direction_y([seq] + lv, delta_softplus, k % 2 == 1, zoh)",
     "y = _direction_y([seq] + lv, delta_softplus, False, zoh)", "ss2d"),
    ("bidir_no_scale", "y = combine_scale * (_direction_y(lf, delta_softplus, False, zoh) +",
     "y = (_direction_y(lf, delta_softplus, False, zoh) +", "bidir"),
    ("conv_taps_reversed", "shift = 3 - k                     # tap k reads x[t - shift]",
     "shift = k", "conv"),
]


def test_mutant_list_applies():
    src = open(SRC).read()
    for name, old, new, _ in MUTANTS:
        assert src.count(old) == 1, name


@pytest.mark.parametrize("name,old,new,sel", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_grad_mutant(tmp_path, name, old, new, sel):
    src = open(SRC).read().replace(old, new)
    mut = tmp_path / "grad_mutant.py"
    mut.write_text(src)
    env = dict(os.environ, VM_GRAD_ORACLE=str(mut), OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-k", sel,
                        os.path.join(ROOT, "tests", "test_oracle_grad.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert "passed" in r.stdout or "failed" in r.stdout, r.stdout[-2000:] + r.stderr[-2000:]
    assert r.returncode == 1, f"grad mutant {name} survived the pins ({sel}):\n{r.stdout[-2000:]}"
