"""GPU parity: every C-ABI entry against the fp64 oracle on the same seeded
inputs, at sizes the oracle finishes in seconds that still span several
chunks/tiles and a ragged tail. Tolerance per element: |gpu - ref| <= tol +
tol*|ref| with tol 1e-4 for fp32 I/O and 2e-2 for bf16 I/O (fp32 accumulate).
Conv states are exact copies and must match bit for bit."""
import numpy as np
import pytest

from gpu_util import TOL, check, dev, host, torch_dtype
from mamba_ssd_selective_mixer_amd import synth
from oracle import oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ops():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from mamba_ssd_selective_mixer_amd import ops as _ops
    return _ops


def make_dims(ops, cfg, **kw):
    d = ops.SSDDims(cfg.batch, cfg.seqlen, cfg.nheads, cfg.headdim, cfg.ngroups, cfg.dstate,
                    cfg.conv_width, cfg.chunk or 128, torch_dtype(cfg.dtype))
    return d.replace(**kw) if kw else d


def small(name, **kw):
    return synth.replace(synth.CONFIGS[name], **kw)


# --------------------------------------------------------------------- conv
@pytest.mark.parametrize("name,kw,with_state,with_bias", [
    ("tiny_fp32", {}, False, False),
    ("tiny_fp32", {}, True, True),
    ("tiny_layer", dict(batch=2, seqlen=77), True, False),
    ("tiny_layer", dict(batch=3, seqlen=2), True, True),      # shorter than W-1
    ("tiny_layer", dict(batch=1, seqlen=1, conv_width=2), True, False),
    ("large_layer", dict(seqlen=40, conv_width=3), False, True),
])
def test_conv1d(ops, name, kw, with_state, with_bias):
    import torch
    cfg = small(name, **kw)
    d = make_dims(ops, cfg)
    td = torch_dtype(cfg.dtype)
    prm = synth.layer_params(cfg, with_bias=with_bias)
    inp = synth.prefill_inputs(cfg)
    st = synth.initial_states(cfg) if with_state else {"conv_state": None}
    cs_out = torch.empty(cfg.batch, cfg.conv_width - 1, cfg.channels, dtype=td, device="cuda")
    out = ops.ssd_conv1d(d, dev(inp["xbc"], td), dev(prm["conv_w"], td), dev(prm["conv_b"], td),
                         dev(st["conv_state"], td), cs_out)
    ref, ref_cs = oracle.conv1d_silu(inp["xbc"], prm["conv_w"], prm["conv_b"], st["conv_state"])
    check("conv out", host(out), ref, TOL[cfg.dtype])
    assert np.array_equal(host(cs_out), ref_cs), "conv state out must be an exact copy"


def test_conv1d_state_in_place(ops):
    cfg = small("tiny_layer", batch=2, seqlen=2)
    d = make_dims(ops, cfg)
    td = torch_dtype(cfg.dtype)
    prm = synth.layer_params(cfg)
    inp = synth.prefill_inputs(cfg)
    st = synth.initial_states(cfg)
    cs = dev(st["conv_state"], td)
    ops.ssd_conv1d(d, dev(inp["xbc"], td), dev(prm["conv_w"], td), None, cs, cs)
    _, ref_cs = oracle.conv1d_silu(inp["xbc"], prm["conv_w"], None, st["conv_state"])
    assert np.array_equal(host(cs), ref_cs)


def test_conv1d_strided_views(ops):
    import torch
    cfg = small("tiny_layer", batch=2, seqlen=33)
    d = make_dims(ops, cfg)
    td = torch_dtype(cfg.dtype)
    prm = synth.layer_params(cfg)
    inp = synth.prefill_inputs(cfg)
    C = cfg.channels
    big = torch.zeros(cfg.batch, cfg.seqlen, C + 64, dtype=td, device="cuda")
    big[..., 32:32 + C] = dev(inp["xbc"], td)
    obig = torch.zeros(cfg.batch, cfg.seqlen, C + 128, dtype=td, device="cuda")
    ops.ssd_conv1d(d, big[..., 32:32 + C], dev(prm["conv_w"], td), out=obig[..., 64:64 + C])
    ref, _ = oracle.conv1d_silu(inp["xbc"], prm["conv_w"])
    check("conv strided", host(obig[..., 64:64 + C]), ref, TOL[cfg.dtype])
    assert float(obig[..., :64].abs().max()) == 0.0


# --------------------------------------------------------------------- norm
@pytest.mark.parametrize("io,rows,H,P,G", [("f32", 37, 4, 16, 1), ("bf16", 50, 32, 64, 8),
                                           ("bf16", 9, 256, 64, 8), ("f32", 5, 8, 32, 4)])
def test_gated_rmsnorm(ops, io, rows, H, P, G):
    r = np.random.default_rng(3)
    td = torch_dtype(io)
    y = synth.to_io(r.standard_normal((1, rows, H * P)), io)
    y[0, 0] *= 1e-3
    z = synth.to_io(r.standard_normal((1, rows, H * P)), io)
    w = synth.to_io(1 + 0.2 * r.standard_normal(H * P), io)
    d = ops.SSDDims(1, rows, H, P, G, 16, 4, 64, td)
    out = ops.ssd_gated_rmsnorm(d, dev(y, td), dev(z, td), dev(w, td), 1e-5)
    ref = oracle.gated_rmsnorm(y, z, w, G, 1e-5)
    check("norm", host(out), ref, TOL[io])


# --------------------------------------------------------------------- scan
def scan_case(ops, cfg, with_state, with_norm, slow=False, Q=None):
    import torch
    td = torch_dtype(cfg.dtype)
    Q = Q or cfg.chunk
    d = make_dims(ops, cfg, chunk=Q)
    prm = synth.layer_params(cfg, slow_decay=slow)
    inp = synth.prefill_inputs(cfg)
    x, Bm, Cm = synth.split_channels(cfg, inp["xbc"])
    s0 = synth.initial_states(cfg)["ssm_state"] if with_state else None
    s_out = torch.empty(cfg.batch, cfg.nheads, cfg.headdim, cfg.dstate, device="cuda")
    y = ops.ssd_chunk_scan(d, dev(x, td), dev(inp["dt"], td), dev(prm["A"]), dev(prm["D"]),
                           dev(Bm, td), dev(Cm, td),
                           z=dev(inp["z"], td) if with_norm else None,
                           norm_w=dev(prm["norm_w"], td) if with_norm else None, eps=prm["eps"],
                           ssm_state_in=dev(s0), ssm_state_out=s_out)
    ry, rs = oracle.ssm_scan(x, inp["dt"], prm["A"], Bm, Cm, prm["D"], s0)
    ry = ry.reshape(cfg.batch, cfg.seqlen, cfg.hp)
    if with_norm:
        ry = oracle.gated_rmsnorm(ry, inp["z"], prm["norm_w"], cfg.ngroups, prm["eps"])
    tol = TOL[cfg.dtype]
    check("scan y", host(y), ry, tol)
    check("final state", host(s_out), rs, tol)
    return host(y), host(s_out)


@pytest.mark.parametrize("with_state", [False, True])
@pytest.mark.parametrize("with_norm", [False, True])
def test_chunk_scan_fp32_tiny(ops, with_state, with_norm):
    scan_case(ops, synth.CONFIGS["tiny_fp32"], with_state, with_norm)


@pytest.mark.parametrize("kw", [dict(batch=2, seqlen=300), dict(batch=1, seqlen=128),
                                dict(batch=1, seqlen=1), dict(batch=2, seqlen=17)])
def test_chunk_scan_bf16(ops, kw):
    scan_case(ops, small("tiny_layer", **kw), True, True)


@pytest.mark.parametrize("Q", [32, 64, 128, 256])
@pytest.mark.parametrize("dstate,dtype", [(64, "bf16"), (128, "f32"), (16, "f32")])
def test_chunk_scan_chunk_invariance(ops, Q, dstate, dtype):
    """Every chunk length gives the oracle's answer (the SSD identity on the
    GPU), each run by the generic kernels at the requested chunk length: bf16
    I/O with d_state 64, and fp32 I/O (1e-4) with the layer's d_state 128 and
    with 16. (bf16 I/O at head_dim 64 / d_state 128 takes the fused path,
    whose chunk length is fixed at 128 tokens.)"""
    scan_case(ops, small("tiny_layer", batch=1, seqlen=520, dstate=dstate, dtype=dtype), True, False, Q=Q)


@pytest.mark.parametrize("name,kw", [("tiny_fp32", {}), ("tiny_layer", dict(batch=1, seqlen=700))])
def test_chunk_scan_slow_decay(ops, name, kw):
    """Slow decay: the state carries signal across many chunks, so a broken
    inter-chunk state passing cannot hide behind fast forgetting."""
    scan_case(ops, small(name, **kw), True, False, slow=True)


def test_chunk_scan_large_heads_group(ops):
    scan_case(ops, small("large_layer", seqlen=300), True, True)


@pytest.mark.parametrize("Q,with_norm", [(64, True), (32, False), (128, True)])
def test_chunk_scan_bf16_small_state(ops, Q, with_norm):
    """d_state 16 with bf16 operands (generic kernels): the C.B^T and C.S_in
    contractions run 32 deep, so the k-slices past d_state must read nothing
    and count as zero."""
    scan_case(ops, small("tiny_layer", nheads=2, ngroups=1, headdim=32, dstate=16, batch=1, seqlen=100),
              True, with_norm, Q=Q)


def test_chunk_scan_bf16_generic_norm(ops):
    """Generic kernels, bf16 I/O, d_state 16 and head_dim 64 with norm groups
    of 128 channels whose RMS is small: the norm amplifies the scan's operand
    rounding, which stays inside the tolerance with fp16 MFMA operands (bf16
    operands reached 1.7x the tolerance on this case)."""
    scan_case(ops, small("tiny_layer", nheads=4, ngroups=2, headdim=64, dstate=16, batch=1, seqlen=257),
              True, True, Q=128)


@pytest.mark.parametrize("P,N,W", [(128, 16, 2), (64, 64, 4)])
def test_prefill_generic_bias_normed(ops, P, N, W):
    """Generic kernels with a conv bias and the gated norm (bf16 I/O): the
    bias shifts B and C by a shared offset whose C.B products cancel, and the
    norm amplifies what remains, so the conv output must not be rounded to
    bf16 between the conv and the scan (it reached 1.1-2.5x the tolerance)."""
    prefill_case(ops, small("tiny_layer", nheads=64, ngroups=8, headdim=P, dstate=N, conv_width=W,
                            batch=1, seqlen=129), with_state=False, with_bias=True)


_NORM_FUSE = [
    ("tiny_fp32", dict(batch=2, seqlen=200), "scan"),            # 4 heads x 16: one 64-channel piece
    ("tiny_layer", dict(nheads=2, ngroups=1, headdim=32, dstate=16, batch=1, seqlen=100), "scan"),
    ("tiny_layer", dict(nheads=4, ngroups=2, headdim=64, dstate=16, batch=1, seqlen=257), "scan"),
    ("tiny_layer", dict(dstate=64, batch=2, seqlen=200), "prefill"),            # 4 x 64: two pieces
    ("tiny_layer", dict(nheads=4, ngroups=2, headdim=128, dstate=64, batch=1, seqlen=150), "prefill"),
    ("tiny_layer", dict(nheads=8, ngroups=8, headdim=64, dstate=32, batch=1, seqlen=77), "prefill"),
    ("tiny_fp32", dict(nheads=16, ngroups=2, headdim=32, dstate=32, batch=1, seqlen=130), "prefill"),
]


@pytest.mark.parametrize("name,kw,entry", _NORM_FUSE)
@pytest.mark.parametrize("mode", [1, 2])
def test_general_norm_fusion(ops, name, kw, entry, mode):
    """General kernels with the gated norm inside the chunk-output kernel
    (mode 1: wherever the group fits; here 1, 2, 4 and 8 heads per group,
    64 to 256 channels, one and two LDS pieces) and after it (mode 2), both
    against the oracle, with states and ragged chunk tails."""
    prev = ops.ssd_set_output_norm_fusion(mode)
    try:
        cfg = small(name, **kw)
        if entry == "scan":
            scan_case(ops, cfg, True, True)
        else:
            prefill_case(ops, cfg, with_state=True)
    finally:
        ops.ssd_set_output_norm_fusion(prev)


def test_prefill_bf16_small_state(ops):
    prefill_case(ops, small("tiny_layer", nheads=4, ngroups=1, headdim=32, dstate=16, batch=2,
                            seqlen=100), with_state=True)


@pytest.mark.parametrize("kw", [dict(batch=2, seqlen=200),                      # fast path
                                dict(batch=2, seqlen=128, headdim=32, dstate=64)])  # generic
def test_chunk_scan_strided_views(ops, kw):
    """x, B and C passed as strided views into one padded xBC tensor (token
    stride > row width), the way a caller hands over slices of a projection."""
    import torch
    cfg = small("tiny_layer", **kw)
    td = torch_dtype(cfg.dtype)
    d = make_dims(ops, cfg)
    prm = synth.layer_params(cfg)
    inp = synth.prefill_inputs(cfg)
    x, Bm, Cm = synth.split_channels(cfg, inp["xbc"])
    HP, GN, C = cfg.hp, cfg.gn, cfg.channels
    big = torch.zeros(cfg.batch, cfg.seqlen, C + 64, dtype=td, device="cuda")
    big[..., :C] = dev(inp["xbc"], td)
    s0 = synth.initial_states(cfg)["ssm_state"]
    so = torch.empty(cfg.batch, cfg.nheads, cfg.headdim, cfg.dstate, device="cuda")
    y = ops.ssd_chunk_scan(d, big[..., :HP], dev(inp["dt"], td), dev(prm["A"]), dev(prm["D"]),
                           big[..., HP:HP + GN], big[..., HP + GN:C], z=dev(inp["z"], td),
                           norm_w=dev(prm["norm_w"], td), eps=prm["eps"], ssm_state_in=dev(s0),
                           ssm_state_out=so)
    ry, rs = oracle.ssm_scan(x, inp["dt"], prm["A"], Bm, Cm, prm["D"], s0)
    ry = oracle.gated_rmsnorm(ry.reshape(cfg.batch, cfg.seqlen, HP), inp["z"], prm["norm_w"],
                              cfg.ngroups, prm["eps"])
    check("scan y (strided)", host(y), ry, TOL[cfg.dtype])
    check("final state (strided)", host(so), rs, TOL[cfg.dtype])


@pytest.mark.parametrize("kw", [
    dict(dtype="f32", nheads=64, headdim=16, ngroups=4, dstate=16),   # 16 heads per group
    dict(dtype="bf16", nheads=64, headdim=32, ngroups=8, dstate=64),  # fp16 operands
])
def test_chunk_scan_state_heads_per_workgroup(ops, kw):
    """Long enough (2 x 2048 tokens, 64 heads) that the chunk-state kernel
    takes two heads of a group per workgroup, staging the chunk's B once for
    both."""
    scan_case(ops, small("tiny_layer", batch=2, seqlen=2048, **kw), True, True)


def test_chunk_scan_fp32_shapes(ops):
    scan_case(ops, small("tiny_fp32", nheads=8, headdim=32, ngroups=2, dstate=64, seqlen=130,
                         batch=2), True, True)


def test_chunk_scan_state_in_place(ops):
    import torch
    cfg = small("tiny_layer", batch=2, seqlen=150)
    td = torch_dtype(cfg.dtype)
    d = make_dims(ops, cfg)
    prm = synth.layer_params(cfg)
    inp = synth.prefill_inputs(cfg)
    x, Bm, Cm = synth.split_channels(cfg, inp["xbc"])
    s0 = synth.initial_states(cfg)["ssm_state"]
    st = dev(s0)
    ops.ssd_chunk_scan(d, dev(x, td), dev(inp["dt"], td), dev(prm["A"]), dev(prm["D"]),
                       dev(Bm, td), dev(Cm, td), ssm_state_in=st, ssm_state_out=st)
    _, rs = oracle.ssm_scan(x, inp["dt"], prm["A"], Bm, Cm, prm["D"], s0)
    check("in-place state", host(st), rs, TOL[cfg.dtype])


# ------------------------------------------------------------------- decode
def decode_case(ops, cfg, steps, with_norm=True, with_bias=False):
    td = torch_dtype(cfg.dtype)
    d = make_dims(ops, cfg, seqlen=1)
    prm = synth.layer_params(cfg, with_bias=with_bias)
    st = synth.initial_states(cfg)
    cs, ss = dev(st["conv_state"], td), dev(st["ssm_state"])
    rcs, rss = st["conv_state"].astype(np.float64), st["ssm_state"].astype(np.float64)
    tol = TOL[cfg.dtype]
    for k in range(steps):
        inp = synth.decode_inputs(cfg, k)
        y = ops.ssd_decode_step(d, dev(inp["xbc_t"], td),
                                dev(inp["z_t"], td) if with_norm else None,
                                dev(inp["dt_t"], td), dev(prm["A"]), dev(prm["D"]),
                                dev(prm["conv_w"], td), dev(prm["conv_b"], td),
                                dev(prm["norm_w"], td), prm["eps"], cs, ss)
        ro, rcs, rss = oracle.decode_step(inp["xbc_t"], inp["z_t"] if with_norm else None,
                                          inp["dt_t"], prm["A"], prm["D"], prm["conv_w"],
                                          prm["conv_b"],
                                          prm["norm_w"], prm["eps"], cfg.nheads, cfg.headdim,
                                          cfg.ngroups, cfg.dstate, rcs, rss)
        check(f"decode out step {k}", host(y), ro, tol)
        # the GPU keeps its conv state in the I/O dtype: compare what it holds
        assert np.array_equal(host(cs), rcs), f"conv state differs at step {k}"
        check(f"decode state step {k}", host(ss), rss, tol)
        rss = host(ss)   # continue from the GPU's own fp32 state (its rounding, not drift)


def test_decode_fp32_tiny(ops):
    decode_case(ops, synth.replace(synth.CONFIGS["tiny_fp32"], batch=3), steps=5)


def test_decode_fp32_no_norm(ops):
    decode_case(ops, synth.replace(synth.CONFIGS["tiny_fp32"], batch=2), steps=2, with_norm=False)


# Decode with a conv bias: fp32 tiny shapes and bf16 shapes of the decode
# loop's layer (256 heads in 8 groups, state 128), gate on and off.
@pytest.mark.parametrize("base,kw,norm", [
    ("tiny_fp32", dict(batch=3), True),
    ("tiny_fp32", dict(batch=2, nheads=8, ngroups=2, headdim=32, dstate=64, conv_width=3), False),
    ("decode_loop", dict(batch=4), True),
    ("decode_loop", dict(batch=3), False),
    ("decode_loop", dict(batch=2, nheads=32, dstate=64, conv_width=2), True)])
def test_decode_conv_bias(ops, base, kw, norm):
    decode_case(ops, synth.replace(synth.CONFIGS[base], **kw), steps=4, with_norm=norm,
                with_bias=True)


@pytest.mark.parametrize("kw", [dict(batch=4), dict(batch=2, nheads=32, dstate=64),
                                dict(batch=2, nheads=16, ngroups=4, headdim=32, dstate=16,
                                     conv_width=3)])
def test_decode_bf16(ops, kw):
    decode_case(ops, synth.replace(synth.CONFIGS["decode_loop"], **kw), steps=3)


# Decode shapes across the envelope (head_dim, d_state, conv width, heads per
# group, I/O type, gate on or off), each stepped three times.
@pytest.mark.parametrize("base,kw,norm", [
    ("decode_loop", dict(batch=3, nheads=8, ngroups=1, headdim=128, dstate=128, conv_width=2), True),
    ("decode_loop", dict(batch=5, nheads=4, ngroups=4, headdim=16, dstate=32, conv_width=3), True),
    ("tiny_fp32", dict(batch=2, nheads=8, ngroups=2, headdim=64, dstate=16), True),
    ("decode_loop", dict(batch=2, nheads=16, ngroups=8, headdim=32, dstate=64, conv_width=2), False)])
def test_decode_envelope(ops, base, kw, norm):
    decode_case(ops, synth.replace(synth.CONFIGS[base], **kw), steps=3, with_norm=norm)


# -------------------------------------------------------------- full prefill
def prefill_case(ops, cfg, with_state, pieces=None, slow=False, with_bias=False, inplace=False,
                 with_norm=True, A=None, flags=0):
    """Whole path (conv -> scan -> norm) with state in/out; optional chaining
    over `pieces` (token boundaries) each resuming from the previous state.
    A, when given, replaces the drawn per-head decay rates."""
    import torch
    td = torch_dtype(cfg.dtype)
    prm = synth.layer_params(cfg, slow_decay=slow, with_bias=with_bias)
    if A is not None:
        prm["A"] = np.full(cfg.nheads, A, dtype=np.float32)
    inp = synth.prefill_inputs(cfg)
    st = synth.initial_states(cfg) if with_state else {"conv_state": None, "ssm_state": None}
    zz = inp["z"] if with_norm else None
    ref = oracle.mixer_prefill(inp["xbc"], zz, inp["dt"], prm["A"], prm["D"],
                               prm["conv_w"], prm["conv_b"], prm["norm_w"], prm["eps"],
                               cfg.nheads, cfg.headdim, cfg.ngroups, cfg.dstate,
                               conv_in=st["conv_state"], s_in=st["ssm_state"])
    bounds = [0] + list(pieces or []) + [cfg.seqlen]
    cs = dev(st["conv_state"], td) if with_state else torch.zeros(
        cfg.batch, cfg.conv_width - 1, cfg.channels, dtype=td, device="cuda")
    ss = dev(st["ssm_state"]) if with_state else torch.zeros(
        cfg.batch, cfg.nheads, cfg.headdim, cfg.dstate, device="cuda")
    outs = []
    for a, b in zip(bounds[:-1], bounds[1:]):
        d = make_dims(ops, cfg, seqlen=b - a, flags=flags)
        cs2 = cs if inplace else torch.empty_like(cs)
        ss2 = ss if inplace else torch.empty_like(ss)
        out = ops.ssd_mixer_prefill(d, dev(inp["xbc"][:, a:b], td),
                                    dev(zz[:, a:b], td) if with_norm else None,
                                    dev(inp["dt"][:, a:b], td), dev(prm["A"]), dev(prm["D"]),
                                    dev(prm["conv_w"], td), dev(prm["conv_b"], td),
                                    dev(prm["norm_w"], td), prm["eps"], cs, cs2, ss, ss2)
        outs.append(host(out))
        cs, ss = cs2, ss2
    tol = TOL[cfg.dtype]
    check("prefill out", np.concatenate(outs, axis=1), ref["out"], tol)
    check("prefill final state", host(ss), ref["s_out"], tol)
    assert np.array_equal(host(cs), ref["conv_out"])


def test_prefill_fp32_tiny(ops):
    prefill_case(ops, synth.CONFIGS["tiny_fp32"], with_state=False)


def test_prefill_fp32_tiny_state_bias(ops):
    prefill_case(ops, synth.CONFIGS["tiny_fp32"], with_state=True, with_bias=True)


def test_prefill_bf16(ops):
    prefill_case(ops, small("tiny_layer", batch=2, seqlen=400), with_state=True)


@pytest.mark.parametrize("kw", [dict(nheads=64, batch=1, seqlen=333),   # 8 heads per group
                                dict(batch=3, seqlen=129),
                                dict(batch=1, seqlen=5, nheads=16, ngroups=4)])
def test_prefill_bf16_shapes(ops, kw):
    prefill_case(ops, small("tiny_layer", **kw), with_state=True)


@pytest.mark.parametrize("kw", [dict(nheads=64, batch=1, seqlen=333), dict(batch=3, seqlen=129)])
def test_prefill_bf16_conv_bias(ops, kw):
    """With a conv bias the whole prefill is checked before the norm (z = None):
    every element of y within 2e-2 + 2e-2 |ref|. The bias shifts B and C by a
    shared offset, so C.B^T sums of O(16) partly cancel; the fp16 operands and
    the fp32 conv intermediate keep that within the tolerance."""
    prefill_case(ops, small("tiny_layer", **kw), with_state=True, with_bias=True, with_norm=False)


@pytest.mark.parametrize("kw", [dict(nheads=64, batch=1, seqlen=333), dict(batch=3, seqlen=129)])
def test_prefill_bf16_conv_bias_normed(ops, kw):
    """Conv bias with the gated norm, every output element within 2e-2 (the
    fp16 MFMA operands keep the shared-offset C.B^T sums precise enough)."""
    prefill_case(ops, small("tiny_layer", **kw), with_state=True, with_bias=True, with_norm=True)


_BIAS_SLOW = [(dict(batch=1, seqlen=600), [2, 130, 257]),
              (dict(nheads=64, batch=2, seqlen=300), None),
              (dict(batch=2, seqlen=400, dstate=64), None),
              (dict(nheads=64, batch=1, seqlen=700), [300])]


@pytest.mark.parametrize("kw,pieces", _BIAS_SLOW)
@pytest.mark.parametrize("flags", [0, 1])
def test_prefill_bias_slow_decay(ops, kw, pieces, flags):
    """Conv bias with slow decay: B and C share large channel offsets, x has
    one too, and the state grows over hundreds of tokens along the B offset,
    while C . bbar is small for some groups, so C . S is a small sum of large
    terms. The fused path carries the state split into S' + a bbar^T (fp16
    MFMA operands only for the small parts), the general path has fp32
    carried-in states and output operands; with fp32 operands
    (SSD_FLAG_FP32_OPERANDS) too, every element is within 2e-2. Shapes: 4 and
    8 heads per group (the chunk-state kernel keeping B and C rows), state 64
    (general path), chained pieces resuming from the final state."""
    prefill_case(ops, small("tiny_layer", **kw), with_state=True, pieces=pieces, slow=True,
                 with_bias=True, flags=flags)


@pytest.mark.parametrize("name,kw", [("tiny_fp32", {}), ("tiny_layer", dict(batch=2, seqlen=300))])
def test_prefill_no_decay(ops, name, kw):
    """A = 0: no forgetting, the scan is a running sum over the whole
    sequence (states carried across every chunk and the initial state)."""
    prefill_case(ops, small(name, **kw), with_state=True, A=0.0)


@pytest.mark.parametrize("name,kw", [("tiny_fp32", {}), ("tiny_layer", dict(batch=2, seqlen=300))])
def test_prefill_memoryless(ops, name, kw):
    """A = -1e4: every decay underflows to 0, y_t = dt_t (C_t . B_t) x_t + D x_t."""
    prefill_case(ops, small(name, **kw), with_state=True, A=-1e4)


@pytest.mark.parametrize("name,L", [("tiny_fp32", 1), ("tiny_layer", 1), ("tiny_layer", 2), ("tiny_layer", 129)])
def test_prefill_short(ops, name, L):
    """One- and two-token calls (shorter than the conv window) and a chunk
    plus one token, resuming from nonzero conv and SSM states."""
    prefill_case(ops, small(name, batch=2, seqlen=L), with_state=True)


@pytest.mark.parametrize("kw,pieces", [(dict(batch=3, seqlen=200), None),
                                       (dict(batch=2, seqlen=2), None),
                                       (dict(batch=2, seqlen=300), [2, 150])])
def test_prefill_grouped_heads(ops, kw, pieces):
    """8 heads per group, so the chunk-state kernel writes the convolved B and
    C rows once for the output kernel's two 4-head blocks: several sequences
    (per-sequence row indexing), calls shorter than the conv window (conv
    state rows feed the stored C), and pieces chained through both states."""
    prefill_case(ops, small("tiny_layer", nheads=64, **kw), with_state=True, pieces=pieces)


@pytest.mark.parametrize("kw", [
    dict(nheads=32, ngroups=1, batch=1, seqlen=300),  # 8 blocks per group; 3 groups: one partition
    dict(nheads=24, ngroups=2, batch=2, seqlen=200),  # 3 blocks per group; 8 groups: 8 partitions
    dict(nheads=16, ngroups=2, batch=1, seqlen=260),  # 2 blocks per group; 6 groups, ragged tail
    dict(nheads=144, ngroups=1, batch=1, seqlen=130),  # 36 blocks: y, then the grouped norm
])
def test_prefill_norm_across_blocks(ops, kw):
    """Norm groups wider than the output kernel's 4-head block: each block
    publishes its per-token sums of squares and gathers its partners', with
    the tickets split over 8 partitions (group count a multiple of 8) or not;
    beyond 32 blocks per group the norm runs after the scan instead."""
    prefill_case(ops, small("tiny_layer", **kw), with_state=True)


def test_chunk_scan_norm_across_blocks(ops):
    """The same exchange in the chunk-scan entry point (no conv), one partition."""
    scan_case(ops, small("tiny_layer", nheads=32, ngroups=1, batch=1, seqlen=300), True, True)


# Fast-path shapes from a seeded sweep (random.Random(7) and (11) over heads
# per group 4..64, groups 1..8, batch 1..3, lengths 1..383, states and conv
# bias on or off); 70 cases passed with a worst margin of 0.40 of the
# tolerance, these 14 are kept: (H, G, batch, seqlen, states, bias).
@pytest.mark.parametrize("H,G,B,L,st,bias", [
    (12, 1, 2, 2, True, False), (12, 3, 2, 127, False, False), (128, 2, 2, 200, True, False),
    (16, 1, 3, 128, True, True), (16, 4, 1, 129, True, True), (24, 2, 1, 2, True, True),
    (32, 2, 1, 256, True, True), (32, 4, 3, 128, False, False), (32, 8, 2, 5, False, True),
    (4, 1, 1, 128, False, False), (4, 1, 3, 300, True, False), (64, 2, 3, 128, True, False),
    (64, 8, 3, 256, True, False), (8, 2, 3, 64, True, False)])
def test_prefill_fast_path_shapes(ops, H, G, B, L, st, bias):
    prefill_case(ops, small("tiny_layer", nheads=H, ngroups=G, batch=B, seqlen=L), with_state=st,
                 with_bias=bias)


# d_state 256 (the top of the envelope): the general kernels with 32 output
# tiles per wave in the chunk-state kernel at head_dim 128, and the decode
# kernel with one wave per state row.
@pytest.mark.parametrize("P,io", [(64, "bf16"), (128, "bf16"), (32, "f32")])
def test_prefill_dstate256(ops, P, io):
    prefill_case(ops, small("tiny_layer", nheads=8, ngroups=2, headdim=P, dstate=256, batch=2,
                            seqlen=200, dtype=io), with_state=True)


def test_chunk_scan_dstate256_fp32(ops):
    scan_case(ops, small("tiny_fp32", nheads=4, headdim=64, ngroups=1, dstate=256, seqlen=150,
                         batch=2), True, True)


@pytest.mark.parametrize("kw", [dict(batch=3, nheads=8, ngroups=2, headdim=64, dstate=256),
                                dict(batch=2, nheads=4, ngroups=1, headdim=128, dstate=256,
                                     conv_width=2)])
def test_decode_dstate256(ops, kw):
    decode_case(ops, synth.replace(synth.CONFIGS["decode_loop"], **kw), steps=3)


def test_prefill_generic_shapes(ops):
    """Shapes outside the fast path (d_state 64, head_dim 32) on the generic kernels."""
    prefill_case(ops, small("tiny_layer", batch=2, seqlen=300, dstate=64, headdim=32), with_state=True)


def test_prefill_pieces_uneven(ops):
    """Piecewise == single shot, including pieces shorter than W-1."""
    prefill_case(ops, small("long_context", seqlen=600), with_state=True, pieces=[1, 3, 130, 256, 257],
                 slow=True)


def test_prefill_pieces_in_place(ops):
    prefill_case(ops, small("long_context", seqlen=300), with_state=True, pieces=[2, 128], inplace=True)


def test_concurrent_streams(ops):
    """Two prefill calls in flight at once on two streams, each with its own
    workspace (one of them normalising across blocks, whose tickets live in
    the workspace), give bit-identical results to the same calls run one
    after the other: the library keeps no state between calls."""
    import torch
    bf = torch.bfloat16
    cases = []
    for cfg in (small("tiny_layer", batch=2, seqlen=300), small("tiny_layer", nheads=64, ngroups=2, batch=2,
                                                         seqlen=300)):
        d = make_dims(ops, cfg)
        prm = synth.layer_params(cfg)
        inp = synth.prefill_inputs(cfg)
        args = (dev(inp["xbc"], bf), dev(inp["z"], bf), dev(inp["dt"], bf), dev(prm["A"]),
                dev(prm["D"]), dev(prm["conv_w"], bf), None, dev(prm["norm_w"], bf), prm["eps"])
        cases.append((d, args))
    ref = [host(ops.ssd_mixer_prefill(d, *a)) for d, a in cases]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]  # default priority
    outs = []
    for (d, a), st in zip(cases, streams):
        ws = ops.workspace(ops.ssd_mixer_prefill_workspace_bytes(d))
        outs.append((torch.empty(d.batch, d.seqlen, d.hp, dtype=bf, device="cuda"), ws))
    for _ in range(3):
        for (d, a), st, (o, ws) in zip(cases, streams, outs):
            st.wait_stream(torch.cuda.current_stream())
            ops.ssd_mixer_prefill(d, *a, out=o, ws=ws, stream=st)
        torch.cuda.synchronize()
        for r, (o, _) in zip(ref, outs):
            assert np.array_equal(host(o), r)


@pytest.mark.parametrize("kw", [dict(batch=2, seqlen=300),                 # norm in the block
                                dict(nheads=64, ngroups=2, batch=2, seqlen=300)])  # across blocks
def test_graph_replay(ops, kw):
    """The fused prefill captured into a HIP graph and replayed several times,
    with eager work and synchronisation between replays, matches the eager
    call on every replay (its only per-call state, the cross-block norm's
    tickets and slots, is reset by a kernel, not a memset)."""
    import torch
    bf = torch.bfloat16
    cfg = small("tiny_layer", **kw)
    d = make_dims(ops, cfg)
    prm = synth.layer_params(cfg)
    inp = synth.prefill_inputs(cfg)
    args = (dev(inp["xbc"], bf), dev(inp["z"], bf), dev(inp["dt"], bf), dev(prm["A"]),
            dev(prm["D"]), dev(prm["conv_w"], bf), None, dev(prm["norm_w"], bf), prm["eps"])
    ref = host(ops.ssd_mixer_prefill(d, *args))
    ws = ops.workspace(ops.ssd_mixer_prefill_workspace_bytes(d))
    out = torch.empty(cfg.batch, cfg.seqlen, cfg.hp, dtype=bf, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        ops.ssd_mixer_prefill(d, *args, out=out, ws=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ops.ssd_mixer_prefill(d, *args, out=out, ws=ws)
    for i in range(4):
        out.fill_(float("nan"))
        ws.fill_(7)                      # scribble over the workspace between replays
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(out), ref), f"replay {i}"


def test_causality_gpu(ops):
    """Perturbing token t leaves every earlier output of the GPU path unchanged."""
    cfg = small("tiny_layer", batch=1, seqlen=256)
    td = torch_dtype(cfg.dtype)
    d = make_dims(ops, cfg)
    prm = synth.layer_params(cfg)
    inp = synth.prefill_inputs(cfg)
    args = lambda xbc: ops.ssd_mixer_prefill(d, dev(xbc, td), dev(inp["z"], td),
                                             dev(inp["dt"], td), dev(prm["A"]), dev(prm["D"]),
                                             dev(prm["conv_w"], td), None,
                                             dev(prm["norm_w"], td), prm["eps"])
    base = host(args(inp["xbc"]))
    for t in (5, 130):
        xbc = inp["xbc"].copy()
        xbc[:, t] += 1.0
        out = host(args(xbc))
        assert np.array_equal(out[:, :t], base[:, :t]), f"output before {t} changed"
        assert not np.array_equal(out[:, t], base[:, t])


@pytest.mark.parametrize("kw", [dict(batch=2, seqlen=300),
                                dict(nheads=64, ngroups=2, batch=2, seqlen=300)])
def test_determinism(ops, kw):
    """Repeated runs on the same inputs give bit-identical outputs and states;
    the second shape normalises across 8 blocks per group, whose tickets (and
    so the order in which partners finish) change from run to run."""
    import torch
    cfg = small("tiny_layer", **kw)
    td = torch_dtype(cfg.dtype)
    d = make_dims(ops, cfg)
    prm = synth.layer_params(cfg)
    inp = synth.prefill_inputs(cfg)
    res = []
    for _ in range(3):
        so = torch.empty(cfg.batch, cfg.nheads, cfg.headdim, cfg.dstate, device="cuda")
        out = ops.ssd_mixer_prefill(d, dev(inp["xbc"], td), dev(inp["z"], td), dev(inp["dt"], td),
                                    dev(prm["A"]), dev(prm["D"]), dev(prm["conv_w"], td), None,
                                    dev(prm["norm_w"], td), prm["eps"], ssm_state_out=so)
        res.append((host(out), host(so)))
    for r in res[1:]:
        assert np.array_equal(res[0][0], r[0]) and np.array_equal(res[0][1], r[1])
