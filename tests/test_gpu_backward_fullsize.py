"""The backward pass at the benchmark's full size (the large-model layer
prefill: 1 x 8192 tokens, 256 heads x 64, 8 groups, state 128), where the
fp64 autograd oracle is out of reach, checked through properties that hold
at any size:

1. With fp32 I/O, for directions v of every input and parameter (random,
   and along the gradient's signs for dt and A), <grad, v> equals the
   central finite difference of L = sum(out * d_out)
   computed by the library's own forward (fp32 I/O, fp32 MFMA operands),
   within 1e-2 (the difference quotient's rounding and curvature error at
   the step used is far below that; a wrong term in any gradient is not).
2. The bf16-I/O backward (the configuration the benchmark times) equals the
   fp32-I/O backward on the same bf16 values: the activation gradients to
   bf16 rounding, the parameter gradients to 1e-4 of their largest entry.

The small-size parity against the oracle is in test_gpu_backward.py."""
import numpy as np
import pytest

from mamba_ssd_selective_mixer_amd import _lib, synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from mamba_ssd_selective_mixer_amd import ops
    cfg = synth.CONFIGS["large_layer"]
    f32 = torch.float32
    prm = synth.layer_params(cfg)
    inp = synth.prefill_inputs(cfg)
    seeds = synth.backward_seeds(cfg)
    t = lambda a, dt=f32: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda", dt)
    # bf16-rounded values (the benchmark's inputs), held in fp32 and bf16
    args32 = {"xbc": t(inp["xbc"]), "z": t(inp["z"]), "dt": t(inp["dt"]), "A": t(prm["A"]),
              "D": t(prm["D"]), "conv_w": t(prm["conv_w"]), "norm_w": t(seeds["norm_w"]),
              "d_out": t(seeds["d_out"])}
    return torch, ops, cfg, prm, args32


def dims(ops, cfg, dt, flags=0):
    return ops.SSDDims(cfg.batch, cfg.seqlen, cfg.nheads, cfg.headdim, cfg.ngroups, cfg.dstate,
                       cfg.conv_width, cfg.chunk, dt, flags=flags)


def test_directional_derivatives_full_size(env):
    torch, ops, cfg, prm, a = env
    f32 = torch.float32
    print("backward full size: fp32 I/O, finite differences of the forward", flush=True)
    d = dims(ops, cfg, f32)
    df = dims(ops, cfg, f32, flags=_lib.SSD_FLAG_FP32_OPERANDS)
    ws = ops.workspace(ops.ssd_mixer_prefill_workspace_bytes(df))
    out = torch.empty(cfg.batch, cfg.seqlen, cfg.hp, device="cuda")

    def loss(p):
        ops.ssd_mixer_prefill(df, p["xbc"], p["z"], p["dt"], p["A"], p["D"], p["conv_w"], None,
                              p["norm_w"], prm["eps"], out=out, ws=ws)
        return float((out.double() * p["d_out"].double()).sum())

    g = ops.ssd_mixer_backward(d, a["xbc"], a["z"], a["dt"], a["A"], a["D"], a["conv_w"], None,
                               a["norm_w"], a["d_out"], eps=prm["eps"])
    torch.cuda.synchronize()
    gen = torch.Generator(device="cuda").manual_seed(11)
    HP, GN = cfg.hp, cfg.gn
    # (tensor, direction support, step): every input and parameter, the x, B
    # and C channels of xBC apart, and late tokens alone. The step keeps the
    # loss difference far above the fp32 forward's rounding noise on a loss
    # of order 1e4; a central difference has no second-order error.
    cases = [("xbc", (slice(None), slice(None), slice(0, HP)), 1e-3),
             ("xbc", (slice(None), slice(None), slice(HP, HP + GN)), 1e-3),
             ("xbc", (slice(None), slice(None), slice(HP + GN, None)), 1e-3),
             ("xbc", (slice(None), slice(8000, None), slice(None)), 1e-3),
             ("z", None, 1e-3), ("dt", None, 1e-3), ("A", None, 1e-3), ("D", None, 1e-3),
             ("conv_w", None, 1e-3), ("norm_w", None, 1e-3)]
    worst = 0.0
    for name, sup, eps in cases:
        v = torch.zeros_like(a[name])
        r = torch.randn(v.shape, generator=gen, device="cuda")
        if sup is None:
            v = r
        else:
            v[sup] = r[sup]
        if name in ("dt", "A"):
            # these directional derivatives are small sums of many signed
            # terms; along sign(grad) the difference quotient adds them all
            # up (the check stays independent: the quotient does not use the
            # gradient). dt moves by a relative step and stays positive.
            v = torch.sign(g[name]).float()
            if name == "dt":
                v = v * a["dt"]
        pp, pm = dict(a), dict(a)
        pp[name] = a[name] + eps * v
        pm[name] = a[name] - eps * v
        fd = (loss(pp) - loss(pm)) / (2 * eps)
        ad = float((g[name].double() * v.double()).sum())
        rel = abs(fd - ad) / max(abs(ad), 1e-30)
        worst = max(worst, rel)
        print(f"  d{name} {'' if sup is None else 'part '}: <grad, v> {ad:.6e} finite "
              f"difference {fd:.6e} rel {rel:.1e}", flush=True)
        assert rel < 1e-2, name
    print(f"  worst relative difference {worst:.1e}", flush=True)


def test_bf16_backward_matches_fp32_full_size(env):
    torch, ops, cfg, prm, a = env
    bf = torch.bfloat16
    print("backward full size: bf16 I/O against fp32 I/O on the same values", flush=True)
    g32 = ops.ssd_mixer_backward(dims(ops, cfg, torch.float32), a["xbc"], a["z"], a["dt"],
                                 a["A"], a["D"], a["conv_w"], None, a["norm_w"], a["d_out"],
                                 eps=prm["eps"])
    b = {k: (v.to(bf) if k not in ("A", "D") else v) for k, v in a.items()}
    g16 = ops.ssd_mixer_backward(dims(ops, cfg, bf), b["xbc"], b["z"], b["dt"], b["A"], b["D"],
                                 b["conv_w"], None, b["norm_w"], b["d_out"], eps=prm["eps"])
    torch.cuda.synchronize()
    for k in ("xbc", "z", "dt"):
        ref = g32[k].float()
        got = g16[k].float()
        err = (got - ref).abs()
        # bf16 rounding of the fp32 value (relative 2^-8) plus a sliver of
        # its scale for the slightly different fp32 arithmetic order
        bound = ref.abs() * 2.0 ** -8 + 1e-5 * float(ref.abs().max())
        excess = float((err - bound).max())
        print(f"  d{k}: max |bf16 - fp32| {float(err.max()):.3e} (max |grad| "
              f"{float(ref.abs().max()):.3e})", flush=True)
        assert excess <= 0, k
    for k in ("A", "D", "conv_w", "norm_w"):
        ref, got = g32[k].double(), g16[k].double()
        rel = float((got - ref).abs().max() / ref.abs().max())
        print(f"  d{k}: max |bf16 - fp32| / max |grad| {rel:.1e}", flush=True)
        assert rel < 1e-4, k
