"""The torch binding checks every tensor before it reaches the C ABI:
dtype against the dims' I/O type (A, D and SSM states fp32), element count,
dense layout (token views only where the C ABI takes a token stride) and
device. These run on CPU tensors, so each wrong argument must be refused
before the device check, and a call whose only fault is the device is
refused for that."""
import pytest
import torch

from mamba_ssd_selective_mixer_amd import ops

D0 = ops.SSDDims(batch=2, seqlen=5, nheads=8, headdim=64, ngroups=2, dstate=128,
                 conv_width=4, chunk=128, io_dtype=torch.bfloat16)


def prefill_args(d=D0):
    bf, f32 = d.io_dtype, torch.float32
    B, L, H, C = d.batch, d.seqlen, d.nheads, d.channels
    return dict(xbc=torch.zeros(B, L, C, dtype=bf), z=torch.zeros(B, L, d.hp, dtype=bf),
                dt=torch.zeros(B, L, H, dtype=bf), A=torch.zeros(H, dtype=f32),
                D=torch.zeros(H, dtype=f32), conv_w=torch.zeros(C, d.conv_width, dtype=bf),
                conv_b=None, norm_w=torch.zeros(d.hp, dtype=bf),
                conv_state_in=torch.zeros(B, d.conv_width - 1, C, dtype=bf),
                ssm_state_in=torch.zeros(B, H, d.headdim, d.dstate, dtype=f32),
                out=torch.zeros(B, L, d.hp, dtype=bf))


def call_prefill(**kw):
    a = prefill_args()
    a.update(kw)
    return ops.ssd_mixer_prefill(D0, a.pop("xbc"), a.pop("z"), a.pop("dt"), a.pop("A"),
                                 a.pop("D"), a.pop("conv_w"), a.pop("conv_b"), a.pop("norm_w"),
                                 **a)


def test_prefill_valid_but_host_tensors():
    with pytest.raises(ValueError, match="device"):
        call_prefill()


@pytest.mark.parametrize("kw,match", [
    (dict(A=torch.zeros(8, dtype=torch.bfloat16)), "A: dtype"),
    (dict(D=torch.zeros(8, dtype=torch.float64)), "D: dtype"),
    (dict(ssm_state_in=torch.zeros(2, 8, 64, 128, dtype=torch.bfloat16)), "ssm_state_in: dtype"),
    (dict(xbc=torch.zeros(2, 5, 1024 + 512, dtype=torch.float32)), "xbc: dtype"),
    (dict(out=torch.zeros(2, 4, 512, dtype=torch.bfloat16)), "out: .* elements"),
    (dict(conv_state_in=torch.zeros(2, 2, 1024, dtype=torch.bfloat16)), "conv_state_in: .* elements"),
    (dict(z=torch.zeros(2, 512, 5, dtype=torch.bfloat16).transpose(1, 2)), "z must be contiguous"),
    (dict(xbc=torch.zeros(2, 5, 2048, dtype=torch.bfloat16)[..., :1024 + 512]), "xbc"),
    (dict(norm_w=None), "norm_w is required"),
    (dict(A=None), "A is required"),
])
def test_prefill_refuses(kw, match):
    with pytest.raises(ValueError, match=match):
        call_prefill(**kw)


def test_prefill_short_workspace():
    with pytest.raises(ValueError, match="workspace"):
        call_prefill(ws=torch.zeros(256, dtype=torch.uint8))


def test_chunk_scan_views_and_strides():
    d = D0
    bf, f32 = d.io_dtype, torch.float32
    B, L, H = d.batch, d.seqlen, d.nheads
    big = torch.zeros(B, L, d.channels + 64, dtype=bf)
    HP, GN = d.hp, d.ngroups * d.dstate
    x, Bm, Cm = big[..., :HP], big[..., HP:HP + GN], big[..., HP + GN:HP + 2 * GN]
    args = (torch.zeros(B, L, H, dtype=bf), torch.zeros(H, dtype=f32), None)
    # token views into one padded row are accepted up to the device check
    with pytest.raises(ValueError, match="device"):
        ops.ssd_chunk_scan(d, x, args[0], args[1], args[2], Bm, Cm)
    # B and C with different token strides
    other = torch.zeros(B, L, GN, dtype=bf)
    with pytest.raises(ValueError, match="share one token stride"):
        ops.ssd_chunk_scan(d, x, args[0], args[1], args[2], Bm, other)
    # a view whose rows are not dense
    with pytest.raises(ValueError, match="contiguous"):
        ops.ssd_chunk_scan(d, big[..., :2 * HP:2], args[0], args[1], args[2], Bm, Cm)
    # the wrong number of channels per row
    with pytest.raises(ValueError, match="rows of"):
        ops.ssd_chunk_scan(d, big[..., :HP + 8], args[0], args[1], args[2], Bm, Cm)


def test_decode_refuses():
    d = D0.replace(seqlen=1)
    bf, f32 = d.io_dtype, torch.float32
    B, H, C = d.batch, d.nheads, d.channels
    a = [torch.zeros(B, C, dtype=bf), torch.zeros(B, d.hp, dtype=bf), torch.zeros(B, H, dtype=bf),
         torch.zeros(H, dtype=f32), torch.zeros(H, dtype=f32), torch.zeros(C, 4, dtype=bf), None,
         torch.zeros(d.hp, dtype=bf), 1e-5, torch.zeros(B, 3, C, dtype=bf),
         torch.zeros(B, H, d.headdim, d.dstate, dtype=f32)]
    with pytest.raises(ValueError, match="device"):
        ops.ssd_decode_step(d, *a)
    bad = list(a)
    bad[10] = torch.zeros(B, H, d.headdim, d.dstate, dtype=bf)
    with pytest.raises(ValueError, match="ssm_state: dtype"):
        ops.ssd_decode_step(d, *bad)
    bad = list(a)
    bad[0] = torch.zeros(B + 1, C, dtype=bf)
    with pytest.raises(ValueError, match="xbc_t: .* elements"):
        ops.ssd_decode_step(d, *bad)


def test_norm_and_conv_refuse():
    d = D0
    bf = d.io_dtype
    n = (d.batch, d.seqlen, d.hp)
    with pytest.raises(ValueError, match="w: .* elements"):
        ops.ssd_gated_rmsnorm(d, torch.zeros(n, dtype=bf), torch.zeros(n, dtype=bf),
                              torch.zeros(d.hp + 1, dtype=bf))
    with pytest.raises(ValueError, match="w: dtype"):
        ops.ssd_conv1d(d, torch.zeros(d.batch, d.seqlen, d.channels, dtype=bf),
                       torch.zeros(d.channels, 4, dtype=torch.float32))
