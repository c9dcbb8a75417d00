"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times. The oracle computes what it can in seconds: the whole
tiny-model layer prefill; for the large layer, the long-context chain and
the decode loop it computes sampled norm groups / sampled sequences exactly
(norm groups and B/C groups are independent of each other, and so are
sequences), so every compared element is checked against the fp64
recurrence itself."""
import numpy as np
import pytest

from gpu_util import TOL, check, dev, host
from mamba_ssd_selective_mixer_amd import synth
from oracle import oracle

pytestmark = pytest.mark.gpu
TOLB = TOL["bf16"]


@pytest.fixture(scope="module")
def env():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from mamba_ssd_selective_mixer_amd import ops
    return torch, ops


def dims(ops, torch, cfg, **kw):
    d = ops.SSDDims(cfg.batch, cfg.seqlen, cfg.nheads, cfg.headdim, cfg.ngroups, cfg.dstate,
                    cfg.conv_width, cfg.chunk or 128, torch.bfloat16)
    return d.replace(**kw) if kw else d


def group_problem(cfg, g, xbc, z, dt, prm, conv_state=None, ssm_state=None):
    """The sub-problem of norm/BC group g: heads g*hpg.. of the group, its x
    channels and its B and C channels, as a one-group layer."""
    hpg = cfg.nheads // cfg.ngroups
    S, HP, GN, N = hpg * cfg.headdim, cfg.hp, cfg.gn, cfg.dstate
    chans = np.r_[g * S:(g + 1) * S, HP + g * N:HP + (g + 1) * N, HP + GN + g * N:HP + GN + (g + 1) * N]
    heads = slice(g * hpg, (g + 1) * hpg)
    sub = dict(xbc=xbc[..., chans], z=None if z is None else z[..., g * S:(g + 1) * S],
               dt=dt[..., heads], A=prm["A"][heads], D=prm["D"][heads],
               conv_w=prm["conv_w"][chans], norm_w=prm["norm_w"][g * S:(g + 1) * S],
               conv_b=None if prm["conv_b"] is None else prm["conv_b"][chans],
               conv_in=None if conv_state is None else conv_state[..., chans],
               s_in=None if ssm_state is None else ssm_state[:, heads])
    return sub, chans, heads


def test_tiny_model_layer_prefill_full(env):
    """4 x 2048 tokens, 32 heads x 64, 8 groups, state 128: every output."""
    torch, ops = env
    cfg = synth.CONFIGS["tiny_layer"]
    prm, inp = synth.layer_params(cfg), synth.prefill_inputs(cfg)
    bf = torch.bfloat16
    out = ops.ssd_mixer_prefill(dims(ops, torch, cfg), dev(inp["xbc"], bf), dev(inp["z"], bf),
                                dev(inp["dt"], bf), dev(prm["A"]), dev(prm["D"]),
                                dev(prm["conv_w"], bf), None, dev(prm["norm_w"], bf), prm["eps"])
    ref = oracle.mixer_prefill(inp["xbc"], inp["z"], inp["dt"], prm["A"], prm["D"], prm["conv_w"],
                               None, prm["norm_w"], prm["eps"], cfg.nheads, cfg.headdim,
                               cfg.ngroups, cfg.dstate)
    check("tiny layer out", host(out), ref["out"], TOLB)


def cb_dev(prm, bf):
    return None if prm["conv_b"] is None else dev(prm["conv_b"], bf)


@pytest.mark.parametrize("bias_slow", [False, True])
def test_large_layer_prefill_full(env, bias_slow):
    """1 x 8192 tokens, 256 heads x 64 (32 heads per norm group), chunk 256,
    final conv and SSM state returned; groups 0 and 7 checked exactly. With
    bias_slow, a conv bias and slowly decaying heads (A ~ -U(0.005, 0.05)):
    the state grows along the B offset over thousands of tokens, the case the
    fused kernels' state split is for."""
    torch, ops = env
    cfg = synth.CONFIGS["large_layer"]
    prm = synth.layer_params(cfg, slow_decay=bias_slow, with_bias=bias_slow)
    inp = synth.prefill_inputs(cfg)
    bf = torch.bfloat16
    cs = torch.empty(1, cfg.conv_width - 1, cfg.channels, dtype=bf, device="cuda")
    ss = torch.empty(1, cfg.nheads, cfg.headdim, cfg.dstate, device="cuda")
    out = ops.ssd_mixer_prefill(dims(ops, torch, cfg), dev(inp["xbc"], bf), dev(inp["z"], bf),
                                dev(inp["dt"], bf), dev(prm["A"]), dev(prm["D"]),
                                dev(prm["conv_w"], bf), cb_dev(prm, bf),
                                dev(prm["norm_w"], bf), prm["eps"], None, cs, None, ss)
    out_h, ss_h, cs_h = host(out), host(ss), host(cs)
    hpg = cfg.nheads // cfg.ngroups
    S = hpg * cfg.headdim
    for g in (0, 7):
        sub, chans, heads = group_problem(cfg, g, inp["xbc"], inp["z"], inp["dt"], prm)
        ref = oracle.mixer_prefill(sub["xbc"], sub["z"], sub["dt"], sub["A"], sub["D"],
                                   sub["conv_w"], sub["conv_b"], sub["norm_w"], prm["eps"], hpg,
                                   cfg.headdim, 1, cfg.dstate)
        check(f"large layer out group {g}", out_h[..., g * S:(g + 1) * S], ref["out"], TOLB)
        check(f"large layer final state group {g}", ss_h[:, heads], ref["s_out"], TOLB)
        assert np.array_equal(cs_h[..., chans], ref["conv_out"])


def test_general_layer_prefill_full(env):
    """4 x 2048 tokens, 32 heads x 64, 8 groups, state 64 (outside the fused
    kernels' envelope), with states in and out: every output and final state.
    At this size the general output kernel applies the gated norm itself
    (1024 (chunk, group) workgroups), as the benchmark runs it."""
    torch, ops = env
    cfg = synth.replace(synth.CONFIGS["tiny_layer"], dstate=64)
    prm, inp = synth.layer_params(cfg), synth.prefill_inputs(cfg)
    st = synth.initial_states(cfg)
    bf = torch.bfloat16
    cs_in, ss_in = dev(st["conv_state"], bf), dev(st["ssm_state"])
    cs_out, ss_out = torch.empty_like(cs_in), torch.empty_like(ss_in)
    out = ops.ssd_mixer_prefill(dims(ops, torch, cfg), dev(inp["xbc"], bf), dev(inp["z"], bf),
                                dev(inp["dt"], bf), dev(prm["A"]), dev(prm["D"]),
                                dev(prm["conv_w"], bf), None, dev(prm["norm_w"], bf), prm["eps"],
                                cs_in, cs_out, ss_in, ss_out)
    ref = oracle.mixer_prefill(inp["xbc"], inp["z"], inp["dt"], prm["A"], prm["D"], prm["conv_w"],
                               None, prm["norm_w"], prm["eps"], cfg.nheads, cfg.headdim,
                               cfg.ngroups, cfg.dstate, conv_in=st["conv_state"],
                               s_in=st["ssm_state"])
    check("general layer out", host(out), ref["out"], TOLB)
    check("general layer final state", host(ss_out), ref["s_out"], TOLB)
    assert np.array_equal(host(cs_out), ref["conv_out"])


def test_one_long_sequence_full(env):
    """One sequence of 32768 tokens in a single call (tiny-layer heads,
    slowly decaying, from a nonzero state): 256 chunks per head walked by the
    state pass with its narrowest vectors and deepest look-ahead (2 elements,
    32 chunks in flight, as a call this size runs it); groups 0 and 7
    against one fp64 run, outputs and final states."""
    torch, ops = env
    cfg = synth.replace(synth.CONFIGS["tiny_layer"], batch=1, seqlen=32768)
    prm = synth.layer_params(cfg, slow_decay=True)
    inp = synth.prefill_inputs(cfg)
    st = synth.initial_states(cfg)
    bf = torch.bfloat16
    cs = dev(st["conv_state"], bf)
    ss = dev(st["ssm_state"])
    out = ops.ssd_mixer_prefill(dims(ops, torch, cfg), dev(inp["xbc"], bf), dev(inp["z"], bf),
                                dev(inp["dt"], bf), dev(prm["A"]), dev(prm["D"]),
                                dev(prm["conv_w"], bf), None, dev(prm["norm_w"], bf), prm["eps"],
                                cs, cs, ss, ss)
    oh, ss_h, cs_h = host(out), host(ss), host(cs)
    S = cfg.nheads // cfg.ngroups * cfg.headdim
    for g in (0, 7):
        sub, chans, heads = group_problem(cfg, g, inp["xbc"], inp["z"], inp["dt"], prm,
                                          st["conv_state"], st["ssm_state"])
        ref = oracle.mixer_prefill(sub["xbc"], sub["z"], sub["dt"], sub["A"], sub["D"],
                                   sub["conv_w"], None, sub["norm_w"], prm["eps"],
                                   cfg.nheads // cfg.ngroups, cfg.headdim, 1, cfg.dstate,
                                   conv_in=sub["conv_in"], s_in=sub["s_in"])
        check(f"long sequence out group {g}", oh[..., g * S:(g + 1) * S], ref["out"], TOLB)
        check(f"long sequence final state group {g}", ss_h[:, heads], ref["s_out"], TOLB)
        assert np.array_equal(cs_h[..., chans], ref["conv_out"])


@pytest.mark.parametrize("bias_slow", [False, True])
def test_long_context_chain_full(env, bias_slow):
    """16 pieces of 8192 tokens (131072 in all), each resuming from the
    previous piece's states, against ONE single-shot fp64 run over all the
    tokens (groups 0 and 5). With bias_slow, a conv bias and slowly decaying
    heads: every piece's carried-in state already holds the large part along
    the B offset, which the fused kernels split off by projection."""
    torch, ops = env
    cfg = synth.CONFIGS["long_context"]
    prm = synth.layer_params(cfg, slow_decay=bias_slow, with_bias=bias_slow)
    bf = torch.bfloat16
    d = dims(ops, torch, cfg)
    cs = torch.zeros(1, cfg.conv_width - 1, cfg.channels, dtype=bf, device="cuda")
    ss = torch.zeros(1, cfg.nheads, cfg.headdim, cfg.dstate, device="cuda")
    hpg = cfg.nheads // cfg.ngroups
    S = hpg * cfg.headdim
    groups = (0, 5)
    got = {g: [] for g in groups}
    parts = {g: {"xbc": [], "z": [], "dt": []} for g in groups}
    for k in range(cfg.pieces):
        inp = synth.prefill_inputs(cfg, piece=k)
        out = ops.ssd_mixer_prefill(d, dev(inp["xbc"], bf), dev(inp["z"], bf), dev(inp["dt"], bf),
                                    dev(prm["A"]), dev(prm["D"]), dev(prm["conv_w"], bf),
                                    cb_dev(prm, bf), dev(prm["norm_w"], bf), prm["eps"], cs, cs,
                                    ss, ss)
        oh = host(out)
        for g in groups:
            got[g].append(oh[..., g * S:(g + 1) * S])
            sub, _, _ = group_problem(cfg, g, inp["xbc"], inp["z"], inp["dt"], prm)
            for key in ("xbc", "z", "dt"):
                parts[g][key].append(sub[key])
    ss_h, cs_h = host(ss), host(cs)
    for g in groups:
        sub, chans, heads = group_problem(cfg, g, np.zeros((1, 1, cfg.channels)), None,
                                          np.zeros((1, 1, cfg.nheads)), prm)
        xbc = np.concatenate(parts[g]["xbc"], axis=1)
        ref = oracle.mixer_prefill(xbc, np.concatenate(parts[g]["z"], axis=1),
                                   np.concatenate(parts[g]["dt"], axis=1), sub["A"], sub["D"],
                                   sub["conv_w"], sub["conv_b"], sub["norm_w"], prm["eps"], hpg,
                                   cfg.headdim, 1, cfg.dstate)
        check(f"chain out group {g}", np.concatenate(got[g], axis=1), ref["out"], TOLB)
        check(f"chain final state group {g}", ss_h[:, heads], ref["s_out"], TOLB)
        assert np.array_equal(cs_h[..., chans], ref["conv_out"])


def test_decode_loop_full(env):
    """256 sequences x 64 single-token steps, 256 heads; states ~ N(0, 0.1)
    updated in place. Sequences 0, 77 and 255 are followed step by step by
    the fp64 decode."""
    torch, ops = env
    cfg = synth.CONFIGS["decode_loop"]
    prm = synth.layer_params(cfg)
    st = synth.initial_states(cfg)
    bf = torch.bfloat16
    d = dims(ops, torch, cfg, seqlen=1)
    cs, ss = dev(st["conv_state"], bf), dev(st["ssm_state"])
    seqs = [0, 77, 255]
    rcs = st["conv_state"][seqs].astype(np.float64)
    rss = st["ssm_state"][seqs].astype(np.float64)
    A, D, cw, nw = dev(prm["A"]), dev(prm["D"]), dev(prm["conv_w"], bf), dev(prm["norm_w"], bf)
    for k in range(cfg.steps):
        inp = synth.decode_inputs(cfg, k)
        y = ops.ssd_decode_step(d, dev(inp["xbc_t"], bf), dev(inp["z_t"], bf), dev(inp["dt_t"], bf),
                                A, D, cw, None, nw, prm["eps"], cs, ss)
        ro, rcs, rss = oracle.decode_step(inp["xbc_t"][seqs], inp["z_t"][seqs], inp["dt_t"][seqs],
                                          prm["A"], prm["D"], prm["conv_w"], None, prm["norm_w"],
                                          prm["eps"], cfg.nheads, cfg.headdim, cfg.ngroups,
                                          cfg.dstate, rcs, rss)
        if k % 8 == 0 or k == cfg.steps - 1:
            check(f"decode out step {k}", host(y[seqs]), ro, TOLB)
    check("decode final SSM state", host(ss[seqs]), rss, TOLB)
    assert np.array_equal(host(cs[seqs]), rcs)


def test_prefill_many_sequences(env):
    """Maximum-size edge: the large-layer shape with 1024 short sequences, so
    batch x 4-head blocks (65 536) exceeds one grid dimension's limit (the
    kernels put the batch in its own dimension), with the norm spanning 8
    blocks per group in 8 ticket partitions. Sampled sequences, outputs and
    final states, against the fp64 oracle on those sequences alone."""
    torch, ops = env
    cfg = synth.replace(synth.CONFIGS["large_layer"], batch=1024, seqlen=5)
    assert cfg.batch * cfg.nheads // 4 > 65535
    prm, inp = synth.layer_params(cfg), synth.prefill_inputs(cfg)
    bf = torch.bfloat16
    so = torch.empty(cfg.batch, cfg.nheads, cfg.headdim, cfg.dstate, device="cuda")
    out = ops.ssd_mixer_prefill(dims(ops, torch, cfg), dev(inp["xbc"], bf), dev(inp["z"], bf),
                                dev(inp["dt"], bf), dev(prm["A"]), dev(prm["D"]),
                                dev(prm["conv_w"], bf), None, dev(prm["norm_w"], bf), prm["eps"],
                                ssm_state_out=so)
    for b in (0, 517, cfg.batch - 1):
        sl = slice(b, b + 1)
        ref = oracle.mixer_prefill(inp["xbc"][sl], inp["z"][sl], inp["dt"][sl], prm["A"],
                                   prm["D"], prm["conv_w"], None, prm["norm_w"], prm["eps"],
                                   cfg.nheads, cfg.headdim, cfg.ngroups, cfg.dstate)
        check(f"out, sequence {b}", host(out[sl]), ref["out"], TOLB)
        check(f"final state, sequence {b}", host(so[sl]), ref["s_out"], TOLB)
