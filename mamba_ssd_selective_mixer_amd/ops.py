"""Thin torch binding of the C ABI: the functions carry the C names and only
marshal arguments (device pointers, token strides, the current HIP stream).
Every step runs in the HIP kernels of libssd_mi355x.so; there is no CPU or
PyTorch fallback, and a missing library raises.

Tensors are torch device tensors. A, D and SSM states are float32; all
other tensors use the I/O dtype (torch.float32 or torch.bfloat16).
"""
from __future__ import annotations

import ctypes
import dataclasses

import torch

from . import _lib


@dataclasses.dataclass(frozen=True)
class SSDDims:
    batch: int
    seqlen: int
    nheads: int
    headdim: int
    ngroups: int
    dstate: int
    conv_width: int = 4
    chunk: int = 128
    io_dtype: torch.dtype = torch.bfloat16

    @property
    def hp(self):
        return self.nheads * self.headdim

    @property
    def channels(self):
        return self.hp + 2 * self.ngroups * self.dstate

    def c(self) -> _lib.Dims:
        code = {torch.float32: _lib.SSD_F32, torch.bfloat16: _lib.SSD_BF16}.get(self.io_dtype, 99)
        return _lib.Dims(self.batch, self.seqlen, self.nheads, self.headdim, self.ngroups,
                         self.dstate, self.conv_width, self.chunk, code)

    def replace(self, **kw) -> "SSDDims":
        return dataclasses.replace(self, **kw)


class SSDError(RuntimeError):
    def __init__(self, rc: int, where: str):
        super().__init__(f"{where}: {_lib.STATUS.get(rc, rc)} ({_lib.status_str(rc)})")
        self.rc = rc


def _check(rc: int, where: str):
    if rc != 0:
        raise SSDError(rc, where)


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _tok_stride(t, inner: int, name: str) -> int:
    """Token stride (elements) of a [B, L, ...inner...] view whose trailing
    `inner` elements are contiguous and whose batch stride is L * token stride."""
    if t.dim() < 2:
        raise ValueError(f"{name}: expected [B, L, ...]")
    B, L = t.shape[0], t.shape[1]
    flat = t.reshape(B, L, -1) if t.is_contiguous() else None
    if flat is None:
        # strided view: inner dims must still be dense
        expect = 1
        for d in range(t.dim() - 1, 1, -1):
            if t.stride(d) != expect and t.shape[d] != 1:
                raise ValueError(f"{name}: inner dimensions must be contiguous")
            expect *= t.shape[d]
        ts = t.stride(1)
    else:
        ts = flat.stride(1)
    if flat is None and B > 1 and t.stride(0) != L * ts:
        raise ValueError(f"{name}: batch stride must equal seqlen * token stride")
    if ts < inner:
        raise ValueError(f"{name}: token stride {ts} < row width {inner}")
    return ts


def _need_cuda(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("all tensors must be device (HIP) tensors")


# ---------------------------------------------------------------- host logic

def ssd_validate(entry: str, d: SSDDims) -> int:
    return int(_lib.load().ssd_validate(_lib.ENTRY[entry], ctypes.byref(d.c())))


def ssd_ssm_state_bytes(d: SSDDims) -> int:
    return int(_lib.load().ssd_ssm_state_bytes(ctypes.byref(d.c())))


def ssd_conv_state_bytes(d: SSDDims, as_fp32: bool = False) -> int:
    return int(_lib.load().ssd_conv_state_bytes(ctypes.byref(d.c()), int(as_fp32)))


def ssd_chunk_scan_workspace_bytes(d: SSDDims) -> int:
    return int(_lib.load().ssd_chunk_scan_workspace_bytes(ctypes.byref(d.c())))


def ssd_mixer_prefill_workspace_bytes(d: SSDDims) -> int:
    return int(_lib.load().ssd_mixer_prefill_workspace_bytes(ctypes.byref(d.c())))


def workspace(nbytes: int, device="cuda") -> torch.Tensor:
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


# ---------------------------------------------------------------- compute

def ssd_conv1d(d: SSDDims, xbc, w, bias=None, conv_state_in=None, conv_state_out=None,
               out=None, stream=None):
    _need_cuda(xbc, w, bias, conv_state_in, conv_state_out, out)
    C = d.channels
    if out is None:
        out = torch.empty(d.batch, d.seqlen, C, dtype=d.io_dtype, device=xbc.device)
    rc = _lib.load().ssd_conv1d(ctypes.byref(d.c()), _p(xbc), _tok_stride(xbc, C, "xbc"), _p(w),
                                _p(bias), _p(conv_state_in), _p(conv_state_out), _p(out),
                                _tok_stride(out, C, "out"), _stream(stream))
    _check(rc, "ssd_conv1d")
    return out


def ssd_chunk_scan(d: SSDDims, x, dt, A, D, Bm, Cm, z=None, norm_w=None, eps=1e-5,
                   ssm_state_in=None, ssm_state_out=None, y=None, ws=None, stream=None):
    _need_cuda(x, dt, A, D, Bm, Cm, z, norm_w, ssm_state_in, ssm_state_out, y, ws)
    xs = _tok_stride(x, d.hp, "x")
    bs = _tok_stride(Bm, d.ngroups * d.dstate, "Bm")
    if _tok_stride(Cm, d.ngroups * d.dstate, "Cm") != bs:
        raise ValueError("Bm and Cm must share one token stride")
    if y is None:
        y = torch.empty(d.batch, d.seqlen, d.hp, dtype=d.io_dtype, device=x.device)
    need = ssd_chunk_scan_workspace_bytes(d)
    if ws is None:
        ws = workspace(need, x.device)
    rc = _lib.load().ssd_chunk_scan(ctypes.byref(d.c()), _p(x), xs, _p(dt), _p(A), _p(D), _p(Bm),
                                    _p(Cm), bs, _p(z), _p(norm_w), float(eps), _p(ssm_state_in),
                                    _p(ssm_state_out), _p(y), _p(ws), ws.numel(), _stream(stream))
    _check(rc, "ssd_chunk_scan")
    return y


def ssd_gated_rmsnorm(d: SSDDims, y, z, w, eps=1e-5, out=None, stream=None):
    _need_cuda(y, z, w, out)
    if out is None:
        out = torch.empty_like(y)
    rc = _lib.load().ssd_gated_rmsnorm(ctypes.byref(d.c()), _p(y), _p(z), _p(w), float(eps),
                                       _p(out), _stream(stream))
    _check(rc, "ssd_gated_rmsnorm")
    return out


def ssd_decode_step(d: SSDDims, xbc_t, z_t, dt_t, A, D, conv_w, conv_b, norm_w, eps,
                    conv_state, ssm_state, y_t=None, stream=None):
    _need_cuda(xbc_t, z_t, dt_t, A, D, conv_w, conv_b, norm_w, conv_state, ssm_state, y_t)
    if y_t is None:
        y_t = torch.empty(d.batch, d.hp, dtype=d.io_dtype, device=xbc_t.device)
    rc = _lib.load().ssd_decode_step(ctypes.byref(d.c()), _p(xbc_t), _p(z_t), _p(dt_t), _p(A),
                                     _p(D), _p(conv_w), _p(conv_b), _p(norm_w), float(eps),
                                     _p(conv_state), _p(ssm_state), _p(y_t), _stream(stream))
    _check(rc, "ssd_decode_step")
    return y_t


def ssd_mixer_prefill(d: SSDDims, xbc, z, dt, A, D, conv_w, conv_b, norm_w, eps=1e-5,
                      conv_state_in=None, conv_state_out=None, ssm_state_in=None,
                      ssm_state_out=None, out=None, ws=None, stream=None):
    _need_cuda(xbc, z, dt, A, D, conv_w, conv_b, norm_w, conv_state_in, conv_state_out,
               ssm_state_in, ssm_state_out, out, ws)
    if out is None:
        out = torch.empty(d.batch, d.seqlen, d.hp, dtype=d.io_dtype, device=xbc.device)
    need = ssd_mixer_prefill_workspace_bytes(d)
    if ws is None:
        ws = workspace(need, xbc.device)
    rc = _lib.load().ssd_mixer_prefill(ctypes.byref(d.c()), _p(xbc), _p(z), _p(dt), _p(A), _p(D),
                                       _p(conv_w), _p(conv_b), _p(norm_w), float(eps),
                                       _p(conv_state_in), _p(conv_state_out), _p(ssm_state_in),
                                       _p(ssm_state_out), _p(out), _p(ws), ws.numel(),
                                       _stream(stream))
    _check(rc, "ssd_mixer_prefill")
    return out


def profile_start(capacity: int) -> None:
    """Time every kernel launch of the library with a pair of HIP events on
    the launch stream, for the next `capacity` launches."""
    _check(_lib.load().ssd_profile_start(int(capacity)), "ssd_profile_start")


def profile_stop() -> None:
    _check(_lib.load().ssd_profile_stop(), "ssd_profile_stop")


def profile_read(kernel: str) -> tuple[int, float]:
    """(timed launches, summed milliseconds) of one kernel since profile_start."""
    n = ctypes.c_int64(0)
    ms = ctypes.c_double(0.0)
    _check(_lib.load().ssd_profile_read(_lib.KERNELS.index(kernel), ctypes.byref(n),
                                        ctypes.byref(ms)), "ssd_profile_read")
    return int(n.value), float(ms.value)
