"""Plant one mistake at a time in a copy of the oracle and require that the
pins catch it (CPU only; the real oracle source is never modified)."""
import os
import subprocess

import pytest

import oracle
import pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "ssd_oracle.c")

UPDATE = "hs[n] = decay * hs[n] + d * xv * Bt[n];"
READ = "acc += Ct[n] * hs[n];"

# (name, text in ssd_oracle.c, replacement)
MUTANTS = [
    ("dropped_decay", "hs[n] = decay * hs[n]", "hs[n] = hs[n]"),
    ("decay_sign", "exp(d * A[h])", "exp(-d * A[h])"),
    ("dropped_dt_on_input", "d * xv * Bt[n]", "xv * Bt[n]"),
    ("output_before_update", UPDATE + "\n                    " + READ,
     READ + "\n                    " + UPDATE),
    ("B_C_swapped", "const double *Bt = B +", "const double *Bt = C +"),
    ("group_index", "const int64_t g = h / heads_per_group;", "const int64_t g = h % G;"),
    ("dropped_D", "(D ? D[h] * xv : 0.0)", "0.0"),
    ("D_scaled_by_dt", "(D ? D[h] * xv : 0.0)", "(D ? D[h] * d * xv : 0.0)"),
    ("init_ignored", "hs[n] = init_state ? init_state[state_off + n] : 0.0;", "hs[n] = 0.0;"),
    ("state_out_off_by_one", "if (state_out && t == j)", "if (state_out && t + 1 == j)"),
    ("chunk_state_after_update", "if (chunk_states && t % chunk == 0) {",
     "if (chunk_states && (t + 1) % chunk == 0) {"),
    ("x_transposed_index", "x[((b * T + t) * H + h) * P + p]", "x[((b * T + t) * H + (p % H)) * P + (h % P)]"),
    ("decay_uses_next_dt", "const double decay = exp(d * A[h]);",
     "const double decay = exp((t + 1 < T ? dt[(b * T + t + 1) * H + h] : d) * A[h]);"),
]


def _compile(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation {name}: pattern must occur exactly once"
    mutated = tmp_path / f"{name}.c"
    mutated.write_text(src.replace(old, new))
    lib = tmp_path / f"lib{name}.so"
    subprocess.run(["gcc", "-O1", "-std=c11", "-fopenmp", "-fPIC", "-shared", str(mutated), "-o", str(lib), "-lm"],
                   check=True)
    return oracle.bind(str(lib))


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(tmp_path, name, old, new):
    lib = _compile(tmp_path, name, old, new)

    def fwd(*args, **kw):
        return oracle.ssd_forward(*args, lib=lib, **kw)

    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin(fwd)
        except (AssertionError, ValueError):
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake '{name}'"
