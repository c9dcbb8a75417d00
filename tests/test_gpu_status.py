"""Conditions that depend on the data and so can only be seen on the GPU
are recorded in the call's workspace and reported by ssd_workspace_status:
a cross-block norm exchange that gives up (forced here from the host with a
poll bound of 0, so every kernel still exits normally), and outputs or final
states that are not finite. Activations far outside the usual range (xBC
scaled by 256, exact in bf16, with slow decay so states grow) are computed
exactly enough with SSD_FLAG_FP32_OPERANDS, and with the fused fp16 path
either within tolerance or reported."""
import numpy as np
import pytest

from gpu_util import TOL, check, dev, host
from mamba_ssd_selective_mixer_amd import synth
from oracle import oracle

pytestmark = pytest.mark.gpu
TIMEOUT, NONFINITE = -9, -10


@pytest.fixture(scope="module")
def ops():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from mamba_ssd_selective_mixer_amd import ops as _ops
    return _ops


def run(ops, cfg, prm, inp, flags=0, st=None):
    import torch
    bf = torch.bfloat16
    d = ops.SSDDims(cfg.batch, cfg.seqlen, cfg.nheads, cfg.headdim, cfg.ngroups, cfg.dstate,
                    cfg.conv_width, cfg.chunk, bf, flags)
    ws = ops.workspace(ops.ssd_mixer_prefill_workspace_bytes(d))
    so = torch.empty(cfg.batch, cfg.nheads, cfg.headdim, cfg.dstate, device="cuda")
    out = ops.ssd_mixer_prefill(d, dev(inp["xbc"], bf), dev(inp["z"], bf), dev(inp["dt"], bf),
                                dev(prm["A"]), dev(prm["D"]), dev(prm["conv_w"], bf), None,
                                dev(prm["norm_w"], bf), prm["eps"],
                                ssm_state_in=None if st is None else dev(st), ssm_state_out=so,
                                ws=ws)
    return host(out), host(so), ops.ssd_workspace_status(ws)


def reference(cfg, prm, inp):
    return oracle.mixer_prefill(inp["xbc"], inp["z"], inp["dt"], prm["A"], prm["D"],
                                prm["conv_w"], None, prm["norm_w"], prm["eps"], cfg.nheads,
                                cfg.headdim, cfg.ngroups, cfg.dstate)


def test_exchange_timeout_is_reported(ops):
    """Norm groups of 8 heads (two 4-head blocks exchanging row sums): with
    a poll bound of 0 every wait gives up at once, the rows are NaN and the
    call reports SSD_ERR_TIMEOUT; with the bound restored the same workspace
    reports SSD_OK and the output matches the oracle."""
    cfg = synth.replace(synth.CONFIGS["tiny_layer"], nheads=64, ngroups=8, batch=1, seqlen=300)
    prm, inp = synth.layer_params(cfg), synth.prefill_inputs(cfg)
    prev = ops.ssd_set_exchange_spin_limit(0)
    try:
        out, _, rc = run(ops, cfg, prm, inp)
    finally:
        ops.ssd_set_exchange_spin_limit(prev)
    assert rc == TIMEOUT
    assert np.isnan(out).any()
    out, so, rc = run(ops, cfg, prm, inp)
    assert rc == 0
    ref = reference(cfg, prm, inp)
    check("out after restore", out, ref["out"], TOL["bf16"])


@pytest.mark.parametrize("kw,flags", [(dict(batch=2, seqlen=300), 0),        # fused path
                                      (dict(batch=2, seqlen=300), 1),        # fp32 operands
                                      (dict(batch=1, seqlen=200, dstate=64), 0)])  # general
def test_nonfinite_input_is_reported(ops, kw, flags):
    cfg = synth.replace(synth.CONFIGS["tiny_layer"], **kw)
    prm, inp = synth.layer_params(cfg), synth.prefill_inputs(cfg)
    out, so, rc = run(ops, cfg, prm, inp, flags)
    assert rc == 0
    bad = dict(inp)
    bad["xbc"] = inp["xbc"].copy()
    bad["xbc"][0, 150, 3] = np.inf
    out, so, rc = run(ops, cfg, prm, bad, flags)
    assert rc == NONFINITE
    assert not np.isfinite(out).all() or not np.isfinite(so).all()


@pytest.mark.parametrize("kw", [dict(batch=2, seqlen=300), dict(nheads=64, batch=1, seqlen=333)])
def test_fp32_operands_parity(ops, kw):
    """SSD_FLAG_FP32_OPERANDS on bf16 I/O (general kernels, fp32 MFMA
    operands): elementwise parity at the bf16 tolerance, final state too."""
    cfg = synth.replace(synth.CONFIGS["tiny_layer"], **kw)
    prm, inp = synth.layer_params(cfg), synth.prefill_inputs(cfg)
    st = synth.initial_states(cfg)["ssm_state"]
    out, so, rc = run(ops, cfg, prm, inp, flags=1, st=st)
    assert rc == 0
    ref = oracle.mixer_prefill(inp["xbc"], inp["z"], inp["dt"], prm["A"], prm["D"],
                               prm["conv_w"], None, prm["norm_w"], prm["eps"], cfg.nheads,
                               cfg.headdim, cfg.ngroups, cfg.dstate, s_in=st)
    check("out (fp32 operands)", out, ref["out"], TOL["bf16"])
    check("state (fp32 operands)", so, ref["s_out"], TOL["bf16"])


def test_large_activations(ops):
    """xBC scaled by 256 (exact in bf16) with slow decay, so chunk states,
    carried states and the scan output reach magnitudes beyond fp16's range.
    The fused path either stays within tolerance or reports
    SSD_ERR_NONFINITE; with SSD_FLAG_FP32_OPERANDS the call is within
    tolerance elementwise, output and final state."""
    cfg = synth.replace(synth.CONFIGS["tiny_layer"], batch=1, seqlen=700)
    prm = synth.layer_params(cfg, slow_decay=True)
    inp = synth.prefill_inputs(cfg)
    inp = dict(inp, xbc=inp["xbc"] * np.float32(256.0))
    ref = reference(cfg, prm, inp)
    out, so, rc = run(ops, cfg, prm, inp)
    if rc == 0:
        check("out (fused)", out, ref["out"], TOL["bf16"])
        check("state (fused)", so, ref["s_out"], TOL["bf16"])
    else:
        assert rc == NONFINITE
        assert not np.isfinite(out).all() or not np.isfinite(so).all()
    out, so, rc = run(ops, cfg, prm, inp, flags=1)
    assert rc == 0
    check("out (fp32 operands)", out, ref["out"], TOL["bf16"])
    check("state (fp32 operands)", so, ref["s_out"], TOL["bf16"])
