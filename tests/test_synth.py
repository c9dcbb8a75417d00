"""The seeded input generators: deterministic, shaped as stated, and rounded
to the I/O dtype."""
import numpy as np

from mamba_ssd_selective_mixer_amd import synth


def test_round_bf16_ties_to_even():
    # 1 + 2^-8 is halfway between bf16 neighbours 1 and 1 + 2^-7: rounds to even (1).
    v = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 0.0], dtype=np.float32)
    r = synth.round_bf16(v)
    assert r[0] == 1.0 and r[1] == 1.0 + 2 ** -6 and r[2] == -2.5 and r[3] == 0.0
    assert np.all((r.view(np.uint32) & 0xFFFF) == 0)


def test_deterministic_and_shaped():
    cfg = synth.replace(synth.CONFIGS["tiny_layer"], batch=2, seqlen=33)
    a = synth.prefill_inputs(cfg)
    b = synth.prefill_inputs(cfg)
    for k in a:
        assert np.array_equal(a[k], b[k])
    assert a["xbc"].shape == (2, 33, cfg.channels)
    assert a["z"].shape == (2, 33, cfg.hp) and a["dt"].shape == (2, 33, cfg.nheads)
    assert np.all(a["dt"] > 0)
    assert np.all((a["xbc"].view(np.uint32) & 0xFFFF) == 0)      # bf16-representable
    p = synth.layer_params(cfg)
    assert np.all(p["A"] < 0) and np.all(p["A"] >= -16.0) and np.all(p["A"] <= -1.0)
    assert p["conv_w"].shape == (cfg.channels, cfg.conv_width) and p["conv_b"] is None


def test_streams_differ_and_pieces_concatenate():
    cfg = synth.replace(synth.CONFIGS["long_context"], seqlen=16)
    p0 = synth.prefill_inputs(cfg, piece=0)
    p1 = synth.prefill_inputs(cfg, piece=1)
    assert not np.array_equal(p0["xbc"], p1["xbc"])
    st = synth.initial_states(synth.replace(synth.CONFIGS["decode_loop"], batch=3))
    assert st["conv_state"].shape == (3, 3, 18432) and st["ssm_state"].shape == (3, 256, 64, 128)
    assert abs(float(st["ssm_state"].std()) - np.sqrt(0.1)) < 0.01


def test_distributions():
    cfg = synth.replace(synth.CONFIGS["tiny_layer"], batch=1, seqlen=512)
    t = synth.prefill_inputs(cfg, dtype="f32")
    x, Bm, Cm = synth.split_channels(cfg, t["xbc"])
    assert abs(x.std() - 1.0) < 0.02
    assert abs(Bm.std() * np.sqrt(cfg.dstate) - 1.0) < 0.02
    assert abs(Cm.std() * np.sqrt(cfg.dstate) - 1.0) < 0.02
    w = synth.layer_params(cfg, dtype="f32")["conv_w"]
    assert abs(w.std() - 0.5) < 0.02
