"""The allocation-free prefill entry point (the library's fixed per-GPU
scratch instead of a workspace) against the workspace entry point on the
same inputs, through the C ABI: two calls in a row, the second smaller, on
the fused path with the norm inside one block and across blocks (whose
tickets and exchange slots live in the scratch), and on the general path.
Both run the same kernels, so the results must be bit-identical. A call that
needs more than the fixed scratch is refused before any launch."""
import numpy as np
import pytest

from gpu_util import dev, host
from mamba_ssd_selective_mixer_amd import synth

pytestmark = pytest.mark.gpu
SCRATCH = -11


@pytest.fixture(scope="module")
def ops():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from mamba_ssd_selective_mixer_amd import ops as _ops
    return _ops


def both(ops, cfg):
    import torch
    bf = torch.bfloat16
    d = ops.SSDDims(cfg.batch, cfg.seqlen, cfg.nheads, cfg.headdim, cfg.ngroups, cfg.dstate,
                    cfg.conv_width, cfg.chunk, bf)
    prm, inp = synth.layer_params(cfg), synth.prefill_inputs(cfg)
    st = synth.initial_states(cfg)
    args = (dev(inp["xbc"], bf), dev(inp["z"], bf), dev(inp["dt"], bf), dev(prm["A"]),
            dev(prm["D"]), dev(prm["conv_w"], bf), None, dev(prm["norm_w"], bf))
    res = []
    for noalloc in (False, True):
        cs_out = torch.empty(cfg.batch, cfg.conv_width - 1, cfg.channels, dtype=bf, device="cuda")
        ss_out = torch.empty(cfg.batch, cfg.nheads, cfg.headdim, cfg.dstate, device="cuda")
        out = torch.full((cfg.batch, cfg.seqlen, cfg.hp), float("nan"), dtype=bf, device="cuda")
        kw = dict(conv_state_in=dev(st["conv_state"], bf), conv_state_out=cs_out,
                  ssm_state_in=dev(st["ssm_state"]), ssm_state_out=ss_out)
        if noalloc:
            ops.ssd_mixer_prefill_noalloc(d, *args, out, prm["eps"], **kw)
        else:
            ops.ssd_mixer_prefill(d, *args, prm["eps"], out=out, **kw)
        torch.cuda.synchronize()
        res.append((host(out), host(cs_out), host(ss_out)))
    for a, b, what in zip(res[0], res[1], ("out", "conv state", "ssm state")):
        assert np.array_equal(a, b), f"{what} differs from the workspace entry point"
        assert np.isfinite(a).all()


@pytest.mark.parametrize("first,second", [
    (dict(batch=4, seqlen=2048), dict(batch=1, seqlen=130)),               # norm in the block
    (dict(nheads=64, ngroups=2, batch=2, seqlen=700), dict(nheads=64, ngroups=2, batch=1,
                                                           seqlen=200)),   # across blocks
    (dict(batch=2, seqlen=300, dstate=64), dict(batch=1, seqlen=77, dstate=64)),  # general
])
def test_noalloc_matches_workspace_entry(ops, first, second):
    both(ops, synth.replace(synth.CONFIGS["tiny_layer"], **first))
    both(ops, synth.replace(synth.CONFIGS["tiny_layer"], **second))


def test_noalloc_refuses_beyond_scratch(ops):
    """The large-model layer (1 x 8192 tokens, 256 heads) needs more scratch
    than the fixed buffer: refused on the host, nothing launched."""
    import ctypes
    from mamba_ssd_selective_mixer_amd import _lib
    large = synth.CONFIGS["large_layer"]
    d = _lib.Dims(large.batch, large.seqlen, large.nheads, large.headdim, large.ngroups,
                  large.dstate, large.conv_width, large.chunk, _lib.SSD_BF16)
    lib = _lib.load()
    assert lib.ssd_mixer_prefill_workspace_bytes(ctypes.byref(d)) > 64 << 20
    V = ctypes.c_void_p
    rc = lib.ssd_mixer_prefill_noalloc(ctypes.byref(d), *(V(k << 36) for k in range(1, 9)), 1e-5,
                                       *(V(k << 36) for k in range(9, 14)), None)
    assert rc == SCRATCH
