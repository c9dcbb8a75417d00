"""Plant a plausible mistake in a copy of the C oracle (or of the backward
oracle) and check that at least one pin catches it. The mistakes are planted
in the oracle only, on the CPU; each mutated copy is compiled (or loaded)
from a temporary directory."""
import importlib.util
import os

import pytest

from oracle import oracle as orc_mod
from pins import LIMITS, PINS, pin_backward

SRC = os.path.join(os.path.dirname(orc_mod.__file__), "ssd_oracle.c")
BWD_SRC = os.path.join(os.path.dirname(orc_mod.__file__), "backward.py")

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
    "softplus_dropped": [("dt[i * H + h] = softplus(dt_raw[i * H + h] + dt_bias[h]);",
                          "dt[i * H + h] = dt_raw[i * H + h] + dt_bias[h];")],
    "dt_bias_dropped": [("softplus(dt_raw[i * H + h] + dt_bias[h])", "softplus(dt_raw[i * H + h])")],
    "softplus_large_branch": [("v + log1p(exp(-v))", "v + log1p(exp(v))")],
    "A_log_sign": [("A[h] = -exp(A_log[h]);", "A[h] = exp(A_log[h]);")],
    "A_log_not_exponentiated": [("A[h] = -exp(A_log[h]);", "A[h] = -A_log[h];")],
    "packed_z_xbc_swapped": [
        ("memcpy(z + i * HP, r, (size_t)HP * sizeof(double));",
         "memcpy(z + i * HP, r + C, (size_t)HP * sizeof(double));"),
        ("memcpy(xbc + i * C, r + HP, (size_t)C * sizeof(double));",
         "memcpy(xbc + i * C, r, (size_t)C * sizeof(double));")],
    "packed_dt_offset": [("memcpy(dt_raw + i * H, r + HP + C, ", "memcpy(dt_raw + i * H, r + C, ")],
    "varlen_slot_ignored": [("double* sslot = ssm_pool + (int64_t)slots[i] * SN;",
                             "double* sslot = ssm_pool + i * SN;")],
    "varlen_fresh_not_zero": [("const int resume = has_state ? has_state[i] != 0 : 1;",
                               "const int resume = 1;")],
    "varlen_state_not_written": [("memcpy(sslot, ss, (size_t)SN * sizeof(double));",
                                  "(void)ss;")],
    "varlen_token_offset": [("oracle_mixer_prefill(1, L, H, P, G, N, W, xbc + t0 * C,",
                             "oracle_mixer_prefill(1, L, H, P, G, N, W, xbc + i * C,")],
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


# Mistakes in the backward oracle's forward (its gradients come from
# autograd of that forward): the backward pin compares the forward with the
# C oracle and the gradients with central differences of the C oracle. A
# dropped term keeps its tensor in the graph with weight zero, since autograd
# refuses inputs that take no part in the result.
BWD_MUTATIONS = {
    "bwd_conv_bias_dropped": [("u = u + conv_b", "u = u + 0.0 * conv_b")],
    "bwd_gate_without_z": [("q = y * z * torch.sigmoid(z)", "q = y * torch.sigmoid(z)")],
    "bwd_decay_without_dt": [("torch.exp(dt[:, t] * A)", "torch.exp(A + 0.0 * dt[:, t])")],
    "bwd_D_dropped": [("+ D[:, None] * x[:, t])", "+ 0.0 * D[:, None] * x[:, t])")],
    "bwd_norm_sum_not_mean": [("(qg * qg).mean(-1, keepdim=True)",
                               "(qg * qg).sum(-1, keepdim=True)")],
    "bwd_conv_taps_reversed": [("conv_w[:, k] * ext[:, k:k + L]",
                                "conv_w[:, W - 1 - k] * ext[:, k:k + L]")],
    "bwd_initial_state_ignored": [("S = s_in if s_in is not None else",
                                   "S = 0.0 * s_in if s_in is not None else")],
    "bwd_final_state_gradient_dropped": [("loss = loss + (s_out * _t(d_s_out)).sum()",
                                          "loss = loss")],
}


@pytest.fixture(scope="module")
def c_oracle():
    return orc_mod.Oracle()


@pytest.mark.parametrize("name", sorted(BWD_MUTATIONS))
def test_planted_backward_mistake_is_caught(name, tmp_path, c_oracle):
    src = open(BWD_SRC).read()
    for old, new in BWD_MUTATIONS[name]:
        assert src.count(old) >= 1, f"mutation {name}: pattern not found: {old!r}"
        src = src.replace(old, new)
    path = tmp_path / "bwd_mut.py"
    path.write_text(src)
    spec = importlib.util.spec_from_file_location("bwd_mut", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    assert pin_backward(c_oracle, bwd=mod) > LIMITS["backward"], (
        f"the backward pin did not catch the planted mistake {name}")
