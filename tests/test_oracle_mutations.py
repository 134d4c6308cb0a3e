"""Each plausible mistake planted in a copy of the oracle source must fail at least one
pin: proof that the pins have teeth. The mutation is applied to a temporary copy on the
CPU; the committed oracle is never modified."""
import os
import shutil

import pytest

import oracle
from tests.pins import ALL_PINS

SRC = os.path.join(os.path.dirname(oracle.__file__), "kda_oracle.c")

MUTATIONS = {
    "swap_state_axes": ("S[i * D + j] = sin[(size_t)j * D + i];",
                        "S[i * D + j] = sin[(size_t)i * D + j];"),
    "reverse_conv_taps": ("conv_w[(size_t)cf * K + j]", "conv_w[(size_t)cf * K + (K - 1 - j)]"),
    "drop_decay": ("S[i * D + j] *= decay;", "S[i * D + j] *= 1.0;"),
    "l2_eps_outside_sqrt": ("1.0 / sqrt(ss + 1e-6)", "1.0 / (sqrt(ss) + 1e-6)"),
    "gdn_gate_sigmoid": ("gdn ? silu(zz) : sigmoid(zz)", "sigmoid(zz)"),
    "update_sign": ("S[i * D + j] += bt * kt[i] * u[j];", "S[i * D + j] -= bt * kt[i] * u[j];"),
    "ring_roll_off_by_one": ("ring_out[IDX3(b, cf, m, rows, pad)] = xt[T + m];",
                             "ring_out[IDX3(b, cf, m, rows, pad)] = xt[T + m - 1];"),
    "chunk_P_strict": ("P[s * C + j] = (j <= s) ? p : 0.0;", "P[s * C + j] = (j < s) ? p : 0.0;"),
    "chunk_solve_drops_beta": ("acc -= bet[s] * L[s * C + j] * Tm[j * C + col];",
                               "acc -= L[s * C + j] * Tm[j * C + col];"),
    "chunk_state_no_decay": ("double acc = dec * S[i * D + jv];", "double acc = S[i * D + jv];"),
    "rms_sum_not_mean": ("sqrt(ss / D + eps)", "sqrt(ss + eps)"),
    "decay_on_value_axis": ("const double gi = gdn ? g[IDX3(b, t, h, T, H)] : g[row + i];\n"
                            "                    const double decay = exp(gi);\n"
                            "                    for (int j = 0; j < D; ++j) S[i * D + j] *= decay;",
                            "for (int j = 0; j < D; ++j) S[i * D + j] *= "
                            "exp(gdn ? g[IDX3(b, t, h, T, H)] : g[row + j]);"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, tmp_path):
    old, new = MUTATIONS[name]
    text = open(SRC).read()
    assert old in text, f"mutation anchor for {name} not found in the oracle source"
    src = tmp_path / "mutant.c"
    src.write_text(text.replace(old, new))
    lib = oracle.load(oracle.build(str(src), str(tmp_path / "libmutant.so")))
    failed = []
    for pin_name, pin in ALL_PINS.items():
        try:
            pin(lib)
        except AssertionError:
            failed.append(pin_name)
    assert failed, f"mutation {name} passed every pin"
