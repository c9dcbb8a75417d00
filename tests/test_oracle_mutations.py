"""Plant a plausible mistake in a copy of the C oracle and check that at
least one pin catches it. The mistakes are planted in the oracle only, on
the CPU; each mutated copy is compiled into a temporary directory."""
import os

import pytest

from oracle import oracle as orc_mod
from pins import LIMITS, PINS

SRC = os.path.join(os.path.dirname(orc_mod.__file__), "ssd_oracle.c")

# name -> list of (exact text, replacement); every text must occur in the source.
MUTATIONS = {
    "drop_D_skip": [("yt[p] = acc + (D ? D[h] * xt[p] : 0.0);", "yt[p] = acc;")],
    "decay_sign": [("exp(d * A[h])", "exp(-d * A[h])")],
    "output_before_update": [(
        "            S[p * N + n] = s;\n            acc += s * Ct[n];",
        "            acc += S[p * N + n] * Ct[n];\n            S[p * N + n] = s;")],
    "input_without_dt": [("+ d * xt[p] * Bt[n]", "+ xt[p] * Bt[n]")],
    "initial_state_ignored": [("S[i] = s_in ? s_in[((b * H + h) * P) * N + i] : 0.0;",
                               "S[i] = 0.0;")],
    "conv_taps_reversed": [("acc += w[c * W + k] * v;", "acc += w[c * W + (W - 1 - k)] * v;")],
    "conv_bias_dropped": [("double acc = bias ? bias[c] : 0.0;", "double acc = 0.0;")],
    "conv_state_rows_shifted": [("int64_t e = L + r;", "int64_t e = L + r - 1;")],
    "silu_sign": [("return u / (1.0 + exp(-u));", "return u / (1.0 + exp(u));")],
    "norm_without_gate": [("double q = y[c0 + c] * silu(z[c0 + c]);", "double q = y[c0 + c];")],
    "norm_without_eps": [("sqrt(ss / (double)S + eps)", "sqrt(ss / (double)S)")],
    "norm_sum_not_mean": [("sqrt(ss / (double)S + eps)", "sqrt(ss + eps)")],
    "norm_weight_index": [("q * w[j * S + c] * inv", "q * w[c] * inv")],
    "split_B_C_swapped": [
        ("memcpy(Bm + i * GN, v + i * C + HP, ", "memcpy(Bm + i * GN, v + i * C + HP + GN, "),
        ("memcpy(Cm + i * GN, v + i * C + HP + GN, ", "memcpy(Cm + i * GN, v + i * C + HP, ")],
    "decode_conv_state_not_kept": [
        ("memcpy(conv_state, cs_new, (size_t)(Bn * R * C) * sizeof(double));", "(void)cs_new;")],
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, tmp_path):
    src = open(SRC).read()
    for old, new in MUTATIONS[name]:
        assert src.count(old) >= 1, f"mutation {name}: pattern not found: {old!r}"
        src = src.replace(old, new)
    path = tmp_path / "mut.c"
    path.write_text(src)
    lib = orc_mod.build(force=True, src=str(path), out=str(tmp_path / "libmut.so"))
    orc = orc_mod.Oracle(lib)
    caught = []
    for pin, fn in PINS.items():
        if fn(orc) > LIMITS[pin]:
            caught.append(pin)
    assert caught, f"no pin caught the planted mistake {name}"
