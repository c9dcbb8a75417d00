"""GPU parity of the backward pass (ssd_mixer_backward) against the fp64
autograd oracle (oracle/backward.py, itself pinned to finite differences of
the C oracle) on the same seeded inputs and upstream gradients.

The kernels recompute the forward and form every gradient in fp32, so each
gradient is compared with a tolerance relative to that gradient's largest
magnitude: |gpu - ref| <= tol * max|ref| with tol 2e-4 for fp32 I/O. For
bf16 I/O the inputs are bf16 (the oracle sees the same rounded values) and
d_xbc, d_z, d_dt are rounded to bf16 on output (relative 2^-8), so tol is
1e-2 there and 2e-3 for the fp32 parameter and state gradients."""
import numpy as np
import pytest

from gpu_util import dev, host, torch_dtype
from mamba_ssd_selective_mixer_amd import synth
from oracle import backward as bwd_oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ops():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from mamba_ssd_selective_mixer_amd import ops as _ops
    return _ops


def close(name, got, ref, tol):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64).reshape(got.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    scale = float(np.abs(ref).max()) if ref.size else 0.0
    err = float(np.abs(got - ref).max()) if ref.size else 0.0
    assert err <= tol * max(scale, 1e-30), (
        f"{name}: max |gpu-ref| {err:.3e} beyond {tol} x max|ref| {scale:.3e} "
        f"(at flat index {int(np.argmax(np.abs(got - ref)))})")
    return err / max(scale, 1e-30)


def run_case(ops, cfg, with_bias=True, with_state=True, with_d_state=True, with_D=True,
             slow_decay=False):
    import torch
    td = torch_dtype(cfg.dtype)
    B, L, H, P, G, N = cfg.batch, cfg.seqlen, cfg.nheads, cfg.headdim, cfg.ngroups, cfg.dstate
    print(f"backward case B={B} L={L} H={H} P={P} G={G} N={N} W={cfg.conv_width} "
          f"{cfg.dtype} bias={with_bias} state={with_state} d_state={with_d_state} "
          f"D={with_D}", flush=True)
    prm = synth.layer_params(cfg, slow_decay=slow_decay, with_bias=with_bias)
    inp = synth.prefill_inputs(cfg)
    seeds = synth.backward_seeds(cfg)
    st = synth.initial_states(cfg) if with_state else {"conv_state": None, "ssm_state": None}
    d_s = seeds["d_ssm_state_out"] if with_d_state else None
    D = prm["D"] if with_D else None
    d = ops.SSDDims(B, L, H, P, G, N, cfg.conv_width, cfg.chunk or 128, td)
    g = ops.ssd_mixer_backward(
        d, dev(inp["xbc"], td), dev(inp["z"], td), dev(inp["dt"], td), dev(prm["A"]), dev(D),
        dev(prm["conv_w"], td), dev(prm["conv_b"], td), dev(seeds["norm_w"], td),
        dev(seeds["d_out"], td), eps=prm["eps"], conv_state_in=dev(st["conv_state"], td),
        ssm_state_in=dev(st["ssm_state"]), d_ssm_state_out=dev(d_s))
    torch.cuda.synchronize()
    ref = bwd_oracle.mixer_backward(
        inp["xbc"], inp["z"], inp["dt"], prm["A"], D if with_D else np.zeros(H), prm["conv_w"],
        prm["conv_b"], seeds["norm_w"], prm["eps"], H, P, G, N, seeds["d_out"],
        conv_in=st["conv_state"], s_in=st["ssm_state"], d_s_out=d_s)
    act = 1e-2 if cfg.dtype == "bf16" else 2e-4
    par = 2e-3 if cfg.dtype == "bf16" else 2e-4
    worst = {}
    for k in ("xbc", "z", "dt"):
        worst[k] = close("d_" + k, host(g[k]), ref[k], act)
    for k in ("A", "conv_w", "norm_w"):
        worst[k] = close("d_" + k, host(g[k]), ref[k], par)
    if with_D:
        worst["D"] = close("d_D", host(g["D"]), ref["D"], par)
    else:
        assert "D" not in g
    if with_bias:
        worst["conv_b"] = close("d_conv_b", host(g["conv_b"]), ref["conv_b"], par)
    if with_state:
        worst["conv_in"] = close("d_conv_state_in", host(g["conv_state_in"]), ref["conv_in"],
                                 par)
        worst["s_in"] = close("d_ssm_state_in", host(g["ssm_state_in"]), ref["s_in"], par)
    print("  worst relative error per gradient:",
          {k: f"{v:.1e}" for k, v in worst.items()}, flush=True)
    return g


CASES = [
    # several 64-token chunks and a ragged tail, two groups of two heads
    ("f32_ragged", dict(batch=2, seqlen=150, nheads=4, headdim=16, ngroups=2, dstate=16), {}),
    ("f32_plain", dict(batch=1, seqlen=130, nheads=4, headdim=16, ngroups=1, dstate=32),
     dict(with_bias=False, with_state=False, with_d_state=False, with_D=False)),
    ("f32_one_token", dict(batch=2, seqlen=1), {}),
    ("f32_exact_chunk", dict(batch=1, seqlen=64, conv_width=2), {}),
    ("f32_slow_decay", dict(batch=1, seqlen=200, nheads=4, headdim=32, ngroups=2, dstate=64),
     dict(slow_decay=True)),
    ("f32_w3", dict(batch=1, seqlen=97, conv_width=3, nheads=8, ngroups=4), {}),
    ("f32_layer_shape", dict(batch=1, seqlen=160, nheads=8, headdim=64, ngroups=2, dstate=128),
     {}),
    # the widest head and state: head_dim 128 with state 256, and with state 16
    ("f32_p128_n256", dict(batch=1, seqlen=100, nheads=4, headdim=128, ngroups=2, dstate=256),
     {}),
    ("f32_p128_n16", dict(batch=2, seqlen=70, nheads=4, headdim=128, ngroups=1, dstate=16),
     dict(with_bias=False)),
]


@pytest.mark.parametrize("name,shape,opts", CASES, ids=[c[0] for c in CASES])
def test_backward_f32(ops, name, shape, opts):
    cfg = synth.replace(synth.CONFIGS["tiny_fp32"], **shape)
    run_case(ops, cfg, **opts)


def test_backward_bf16_layer_shape(ops):
    """bf16 I/O at the layer's head size (64 x 128 state, 8 heads, 2 groups)."""
    cfg = synth.replace(synth.CONFIGS["tiny_layer"], batch=1, seqlen=160, nheads=8, ngroups=2)
    run_case(ops, cfg)


HEADS_CASES = [
    # bf16 I/O at the layer's head size, 4 heads per group: 2 and 4 per workgroup
    ("bf16_layer_h2", "tiny_layer", dict(batch=1, seqlen=160, nheads=8, ngroups=2), 2),
    ("bf16_layer_h4", "tiny_layer", dict(batch=1, seqlen=160, nheads=8, ngroups=2), 4),
    # fp32, head sizes 16 and 32, 2 heads per group, ragged tails
    ("f32_p16_h2", "tiny_fp32", dict(batch=2, seqlen=150, nheads=4, headdim=16, ngroups=2,
                                     dstate=16), 2),
    ("f32_p32_h2", "tiny_fp32", dict(batch=1, seqlen=200, nheads=4, headdim=32, ngroups=2,
                                     dstate=64), 2),
]


@pytest.mark.parametrize("name,base,shape,heads", HEADS_CASES, ids=[c[0] for c in HEADS_CASES])
def test_backward_heads_per_workgroup(ops, name, base, shape, heads):
    """Several heads of a group per workgroup of the per-chunk kernels, one
    after the other: the gradient kernel sums their dB and dC rows in place,
    the state-gradient-term kernel stages C once for them (the large layer
    takes 32 and 8; small shapes keep one unless the diagnostic asks): every
    gradient against the oracle."""
    cfg = synth.replace(synth.CONFIGS[base], **shape)
    prev = ops.ssd_set_backward_chunk_heads(heads)
    try:
        run_case(ops, cfg)
    finally:
        ops.ssd_set_backward_chunk_heads(prev)


def test_backward_state_grad_chains(ops):
    """The initial-state gradient of a two-piece prefill chains: feeding the
    second piece's d_ssm_state_in as the first piece's d_ssm_state_out gives
    the gradient of the whole sequence (checked against the oracle on the
    joined sequence)."""
    import torch
    cfg = synth.replace(synth.CONFIGS["tiny_fp32"], batch=1, seqlen=192, nheads=4, headdim=16,
                        ngroups=2, dstate=16)
    td = torch.float32
    H, P, G, N, W = cfg.nheads, cfg.headdim, cfg.ngroups, cfg.dstate, cfg.conv_width
    prm = synth.layer_params(cfg, slow_decay=True)
    inp = synth.prefill_inputs(cfg)
    seeds = synth.backward_seeds(cfg)
    cut = 100
    ref = bwd_oracle.mixer_backward(inp["xbc"], inp["z"], inp["dt"], prm["A"], prm["D"],
                                    prm["conv_w"], None, seeds["norm_w"], prm["eps"], H, P, G, N,
                                    seeds["d_out"])
    # forward of the first piece for the second piece's initial states
    from oracle import oracle as fwd_oracle
    f1 = fwd_oracle.mixer_prefill(inp["xbc"][:, :cut], inp["z"][:, :cut], inp["dt"][:, :cut],
                                  prm["A"], prm["D"], prm["conv_w"], None, seeds["norm_w"],
                                  prm["eps"], H, P, G, N)
    sl = [slice(None, cut), slice(cut, None)]
    lens = [cut, cfg.seqlen - cut]

    def piece(i, cs, ss, d_s):
        d = ops.SSDDims(1, lens[i], H, P, G, N, W, 64, td)
        return ops.ssd_mixer_backward(
            d, dev(inp["xbc"][:, sl[i]]), dev(inp["z"][:, sl[i]]), dev(inp["dt"][:, sl[i]]),
            dev(prm["A"]), dev(prm["D"]), dev(prm["conv_w"]), None, dev(seeds["norm_w"]),
            dev(seeds["d_out"][:, sl[i]]), eps=prm["eps"], conv_state_in=cs,
            ssm_state_in=ss, d_ssm_state_out=d_s)
    g2 = piece(1, dev(f1["conv_out"]), dev(f1["s_out"]), None)
    zero_cs = torch.zeros(1, W - 1, cfg.channels, device="cuda")
    zero_ss = torch.zeros(1, H, P, N, device="cuda")
    g1 = piece(0, zero_cs, zero_ss, g2["ssm_state_in"])
    torch.cuda.synchronize()
    got_x = np.concatenate([host(g1["xbc"]), host(g2["xbc"])], axis=1)
    # the conv taps reaching back into the first piece add into its last rows
    got_x[:, cut - (W - 1):cut] += host(g2["conv_state_in"])
    close("joined d_xbc", got_x, ref["xbc"], 2e-4)
    close("joined d_dt", np.concatenate([host(g1["dt"]), host(g2["dt"])], axis=1), ref["dt"],
          2e-4)
    for k in ("A", "D", "conv_w", "norm_w"):
        close("joined d_" + k, host(g1[k]) + host(g2[k]), ref[k], 2e-4)


def test_backward_rejects(ops):
    import torch
    cfg = synth.replace(synth.CONFIGS["tiny_fp32"], batch=1, seqlen=8)
    d = ops.SSDDims(1, 8, cfg.nheads, cfg.headdim, cfg.ngroups, cfg.dstate, 4, 64,
                    torch.float32)
    t = lambda *s: torch.zeros(*s, device="cuda")
    C, HP, H = cfg.channels, cfg.hp, cfg.nheads
    args = (t(1, 8, C), t(1, 8, HP), t(1, 8, H), t(H), t(H), t(C, 4), None, t(HP), t(1, 8, HP))
    with pytest.raises(ValueError):  # z is required
        ops.ssd_mixer_backward(d, args[0], None, *args[2:])
    with pytest.raises(ops.SSDError) as e:  # d_xbc aliasing the input
        ops.ssd_mixer_backward(d, *args, grads={"xbc": args[0]})
    assert e.value.rc == -5


def test_backward_deterministic_and_graph_replay(ops):
    """Every sum of the backward is taken in a fixed order (no atomics): two
    calls give bit-identical gradients, and the call captured into a HIP graph
    and replayed several times (the outputs and the workspace scribbled over
    between replays, with eager work and synchronisation in between) gives
    the same bits on every replay."""
    import torch
    bf = torch.bfloat16
    cfg = synth.replace(synth.CONFIGS["tiny_layer"], batch=2, seqlen=300, nheads=8, ngroups=2)
    prm = synth.layer_params(cfg, with_bias=True)
    inp = synth.prefill_inputs(cfg)
    seeds = synth.backward_seeds(cfg)
    st = synth.initial_states(cfg)
    d = ops.SSDDims(cfg.batch, cfg.seqlen, cfg.nheads, cfg.headdim, cfg.ngroups, cfg.dstate,
                    cfg.conv_width, cfg.chunk, bf)
    args = (dev(inp["xbc"], bf), dev(inp["z"], bf), dev(inp["dt"], bf), dev(prm["A"]),
            dev(prm["D"]), dev(prm["conv_w"], bf), dev(prm["conv_b"], bf),
            dev(seeds["norm_w"], bf), dev(seeds["d_out"], bf))
    kw = dict(eps=prm["eps"], conv_state_in=dev(st["conv_state"], bf),
              ssm_state_in=dev(st["ssm_state"]),
              d_ssm_state_out=dev(seeds["d_ssm_state_out"]))
    ref = {k: host(v) for k, v in ops.ssd_mixer_backward(d, *args, **kw).items()}
    again = {k: host(v) for k, v in ops.ssd_mixer_backward(d, *args, **kw).items()}
    for k in ref:
        assert np.array_equal(again[k], ref[k]), f"d{k} differs between two calls"
    ws = ops.workspace(ops.ssd_mixer_backward_workspace_bytes(d))
    grads = ops.ssd_mixer_backward(d, *args, ws=ws, **kw)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        ops.ssd_mixer_backward(d, *args, grads=grads, ws=ws, **kw)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ops.ssd_mixer_backward(d, *args, grads=grads, ws=ws, **kw)
    for i in range(4):
        for t in grads.values():
            t.fill_(float("nan"))
        ws.fill_(7)
        g.replay()
        torch.cuda.synchronize()
        for k in ref:
            assert np.array_equal(host(grads[k]), ref[k]), f"replay {i}: d{k}"
