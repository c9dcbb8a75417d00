"""GPU parity of the packed-projection entry points: the kernels read the
input projection's rows [z | xBC | dt_raw] through one row stride and form
dt = softplus(dt_raw + dt_bias) and A = -exp(A_log) themselves; compared
with the fp64 oracle's packed entry points on the same rows, elementwise at
2e-2 (bf16) / 1e-4 (fp32), conv states bit for bit. Rows carry padding
columns past the row (never read) in most cases."""
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


def dims(ops, cfg, **kw):
    d = ops.SSDDims(cfg.batch, cfg.seqlen, cfg.nheads, cfg.headdim, cfg.ngroups, cfg.dstate,
                    cfg.conv_width, cfg.chunk or 128, torch_dtype(cfg.dtype))
    return d.replace(**kw) if kw else d


def packed_case(ops, cfg, pad=8, with_state=True, pieces=None, slow=False, with_bias=False,
                flags=0):
    import torch
    td = torch_dtype(cfg.dtype)
    prm = synth.packed_params(cfg, slow_decay=slow, with_bias=with_bias)
    rows = synth.packed_prefill_inputs(cfg, pad=pad)
    st = synth.initial_states(cfg) if with_state else {"conv_state": None, "ssm_state": None}
    ref = oracle.mixer_prefill_packed(rows, prm["dt_bias"], prm["A_log"], prm["D"],
                                      prm["conv_w"], prm["conv_b"], prm["norm_w"], prm["eps"],
                                      cfg.nheads, cfg.headdim, cfg.ngroups, cfg.dstate,
                                      conv_in=st["conv_state"], s_in=st["ssm_state"])
    bounds = [0] + list(pieces or []) + [cfg.seqlen]
    drow = dev(rows, td)
    cs = dev(st["conv_state"], td) if with_state else None
    ss = dev(st["ssm_state"]) if with_state else None
    outs = []
    for a, b in zip(bounds[:-1], bounds[1:]):
        d = dims(ops, cfg, seqlen=b - a, flags=flags)
        cs2 = torch.empty(cfg.batch, cfg.conv_width - 1, cfg.channels, dtype=td, device="cuda")
        ss2 = torch.empty(cfg.batch, cfg.nheads, cfg.headdim, cfg.dstate, device="cuda")
        ws = ops.workspace(ops.ssd_mixer_prefill_workspace_bytes(d))
        out = ops.ssd_mixer_prefill_packed(d, drow[:, a:b], dev(prm["dt_bias"]), dev(prm["A_log"]),
                                           dev(prm["D"]), dev(prm["conv_w"], td),
                                           dev(prm["conv_b"], td), dev(prm["norm_w"], td),
                                           prm["eps"], cs, cs2, ss, ss2, ws=ws)
        assert ops.ssd_workspace_status(ws) == 0
        outs.append(host(out))
        cs, ss = cs2, ss2
    tol = TOL[cfg.dtype]
    check("packed out", np.concatenate(outs, axis=1), ref["out"], tol)
    check("packed final state", host(ss), ref["s_out"], tol)
    assert np.array_equal(host(cs), ref["conv_out"])


@pytest.mark.parametrize("kw,pad", [
    (dict(batch=2, seqlen=300), 8),                      # fused, norm in the block
    (dict(batch=2, seqlen=300), 0),                      # row stride == row width
    (dict(nheads=64, batch=1, seqlen=333), 8),           # fused, norm across 2 blocks
    (dict(nheads=64, ngroups=2, batch=2, seqlen=200), 24),  # 8 blocks per group
    (dict(batch=1, seqlen=5), 8),                        # shorter than a chunk
    (dict(batch=2, seqlen=200, dstate=64), 8),           # general kernels
    (dict(batch=1, seqlen=130, headdim=32, dstate=256, nheads=8, ngroups=2), 8),
])
def test_prefill_packed_bf16(ops, kw, pad):
    packed_case(ops, synth.replace(synth.CONFIGS["tiny_layer"], **kw), pad=pad)


def test_prefill_packed_fp32_tiny(ops):
    packed_case(ops, synth.CONFIGS["tiny_fp32"], pad=4)


@pytest.mark.parametrize("flags", [1, 0])
def test_prefill_packed_bias_slow_pieces(ops, flags):
    """Conv bias, slow decay (A_log from U(log 0.005, log 0.05)) and uneven
    pieces (one shorter than the conv window) chained through both states;
    with fp32 MFMA operands (general kernels) and on the fused path (its
    state split keeps the cancelling sums in fp32)."""
    packed_case(ops, synth.replace(synth.CONFIGS["long_context"], seqlen=600), pieces=[2, 130, 257],
                slow=True, with_bias=True, flags=flags)


@pytest.mark.parametrize("base,kw,pad", [("decode_loop", dict(batch=4), 8), ("tiny_fp32", dict(batch=3), 4),
                                         ("decode_loop", dict(batch=2, nheads=32, dstate=64,
                                                     conv_width=3), 0)])
def test_decode_packed(ops, base, kw, pad):
    cfg = synth.replace(synth.CONFIGS[base], **kw)
    td = torch_dtype(cfg.dtype)
    d = dims(ops, cfg, seqlen=1)
    prm = synth.packed_params(cfg, with_bias=True)
    st = synth.initial_states(cfg)
    cs, ss = dev(st["conv_state"], td), dev(st["ssm_state"])
    rcs, rss = st["conv_state"].astype(np.float64), st["ssm_state"].astype(np.float64)
    tol = TOL[cfg.dtype]
    for k in range(4):
        row = synth.packed_decode_inputs(cfg, k, pad=pad)
        y = ops.ssd_decode_step_packed(d, dev(row, td), dev(prm["dt_bias"]), dev(prm["A_log"]),
                                       dev(prm["D"]), dev(prm["conv_w"], td),
                                       dev(prm["conv_b"], td), dev(prm["norm_w"], td),
                                       prm["eps"], cs, ss)
        ro, rcs, rss = oracle.decode_step_packed(row, prm["dt_bias"], prm["A_log"], prm["D"],
                                                 prm["conv_w"], prm["conv_b"], prm["norm_w"],
                                                 prm["eps"], cfg.nheads, cfg.headdim,
                                                 cfg.ngroups, cfg.dstate, rcs, rss)
        check(f"packed decode out step {k}", host(y), ro, tol)
        assert np.array_equal(host(cs), rcs)
        check(f"packed decode state step {k}", host(ss), rss, tol)
        rss = host(ss)


def test_large_layer_prefill_packed_full(ops):
    """The large-model layer (1 x 8192 tokens, 256 heads) from packed rows in
    the benchmark's launch configuration; groups 0 and 7 against the oracle's
    packed prefill of that group's columns alone."""
    import torch
    cfg = synth.CONFIGS["large_layer"]
    prm = synth.packed_params(cfg)
    rows = synth.packed_prefill_inputs(cfg)
    bf = torch.bfloat16
    cs = torch.empty(1, cfg.conv_width - 1, cfg.channels, dtype=bf, device="cuda")
    ss = torch.empty(1, cfg.nheads, cfg.headdim, cfg.dstate, device="cuda")
    d = dims(ops, cfg)
    out = ops.ssd_mixer_prefill_packed(d, dev(rows, bf), dev(prm["dt_bias"]), dev(prm["A_log"]),
                                       dev(prm["D"]), dev(prm["conv_w"], bf), None,
                                       dev(prm["norm_w"], bf), prm["eps"], None, cs, None, ss)
    out_h, ss_h, cs_h = host(out), host(ss), host(cs)
    HP, GN, C, H = cfg.hp, cfg.gn, cfg.channels, cfg.nheads
    hpg, N = H // cfg.ngroups, cfg.dstate
    S = hpg * cfg.headdim
    for g in (0, 7):
        zc = np.r_[g * S:(g + 1) * S]
        xc = np.r_[g * S:(g + 1) * S, HP + g * N:HP + (g + 1) * N,
                   HP + GN + g * N:HP + GN + (g + 1) * N]
        heads = np.r_[g * hpg:(g + 1) * hpg]
        sub = np.concatenate([rows[..., zc], rows[..., HP + xc], rows[..., HP + C + heads]], -1)
        ref = oracle.mixer_prefill_packed(sub, prm["dt_bias"][heads], prm["A_log"][heads],
                                          prm["D"][heads], prm["conv_w"][xc], None,
                                          prm["norm_w"][zc], prm["eps"], hpg, cfg.headdim, 1, N)
        check(f"packed large layer out group {g}", out_h[..., g * S:(g + 1) * S], ref["out"], TOL["bf16"])
        check(f"packed large layer state group {g}", ss_h[:, heads], ref["s_out"], TOL["bf16"])
        assert np.array_equal(cs_h[..., xc], ref["conv_out"])
