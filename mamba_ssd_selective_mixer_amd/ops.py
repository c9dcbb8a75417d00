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

import numpy as np
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
    flags: int = 0      # SSD_FLAG_* bits (1: fp32 MFMA operands for bf16 I/O)

    @property
    def hp(self):
        return self.nheads * self.headdim

    @property
    def channels(self):
        return self.hp + 2 * self.ngroups * self.dstate

    def c(self) -> _lib.Dims:
        code = {torch.float32: _lib.SSD_F32, torch.bfloat16: _lib.SSD_BF16}.get(self.io_dtype, 99)
        return _lib.Dims(self.batch, self.seqlen, self.nheads, self.headdim, self.ngroups,
                         self.dstate, self.conv_width, self.chunk, code, self.flags)

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
    dev = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("all tensors must be device (HIP) tensors")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"tensors on different devices: {dev} and {t.device}")


def _want(t, name: str, dtype, numel: int, contiguous: bool = True, optional: bool = False):
    """Check a tensor argument: dtype, element count and (by default) dense
    layout; the C ABI reads exactly numel elements from the base pointer."""
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if t.numel() != numel:
        raise ValueError(f"{name}: {t.numel()} elements, expected {numel}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _want_rows(t, name: str, dtype, B: int, L: int, width: int) -> int:
    """A [B, L, ...] token view whose trailing `width` elements are dense;
    returns its token stride."""
    if t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if t.dim() < 3 or t.shape[0] != B or t.shape[1] != L:
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected [{B}, {L}, ...]")
    n = 1
    for k in t.shape[2:]:
        n *= k
    if n != width:
        raise ValueError(f"{name}: rows of {n} elements, expected {width}")
    return _tok_stride(t, width, name)


def _want_ws(ws, need: int):
    if ws.dtype != torch.uint8 or not ws.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 tensor")
    if ws.numel() < need:
        raise ValueError(f"workspace of {ws.numel()} bytes, {need} needed")


def _alloc(stream, fn):
    """Allocate on the stream the call runs on, so the caching allocator
    never hands the memory to other work while the call's kernels run."""
    if stream is None:
        return fn()
    with torch.cuda.stream(stream):
        return fn()


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
    C, io = d.channels, d.io_dtype
    xs = _want_rows(xbc, "xbc", io, d.batch, d.seqlen, C)
    _want(w, "w", io, C * d.conv_width)
    _want(bias, "bias", io, C, optional=True)
    ns = d.batch * (d.conv_width - 1) * C
    _want(conv_state_in, "conv_state_in", io, ns, optional=True)
    _want(conv_state_out, "conv_state_out", io, ns, optional=True)
    if out is None:
        out = _alloc(stream, lambda: torch.empty(d.batch, d.seqlen, C, dtype=io,
                                                 device=xbc.device))
    os_ = _want_rows(out, "out", io, d.batch, d.seqlen, C)
    _need_cuda(xbc, w, bias, conv_state_in, conv_state_out, out)
    rc = _lib.load().ssd_conv1d(ctypes.byref(d.c()), _p(xbc), xs, _p(w), _p(bias),
                                _p(conv_state_in), _p(conv_state_out), _p(out), os_,
                                _stream(stream))
    _check(rc, "ssd_conv1d")
    return out


def ssd_chunk_scan(d: SSDDims, x, dt, A, D, Bm, Cm, z=None, norm_w=None, eps=1e-5,
                   ssm_state_in=None, ssm_state_out=None, y=None, ws=None, stream=None):
    io, f32 = d.io_dtype, torch.float32
    B, L, H = d.batch, d.seqlen, d.nheads
    xs = _want_rows(x, "x", io, B, L, d.hp)
    bs = _want_rows(Bm, "Bm", io, B, L, d.ngroups * d.dstate)
    if _want_rows(Cm, "Cm", io, B, L, d.ngroups * d.dstate) != bs:
        raise ValueError("Bm and Cm must share one token stride")
    _want(dt, "dt", io, B * L * H)
    _want(A, "A", f32, H)
    _want(D, "D", f32, H, optional=True)
    _want(z, "z", io, B * L * d.hp, optional=True)
    _want(norm_w, "norm_w", io, d.hp, optional=z is None)
    ns = B * H * d.headdim * d.dstate
    _want(ssm_state_in, "ssm_state_in", f32, ns, optional=True)
    _want(ssm_state_out, "ssm_state_out", f32, ns, optional=True)
    if y is None:
        y = _alloc(stream, lambda: torch.empty(B, L, d.hp, dtype=io, device=x.device))
    _want(y, "y", io, B * L * d.hp)
    need = ssd_chunk_scan_workspace_bytes(d)
    if ws is None:
        ws = _alloc(stream, lambda: workspace(need, x.device))
    _want_ws(ws, need)
    _need_cuda(x, dt, A, D, Bm, Cm, z, norm_w, ssm_state_in, ssm_state_out, y, ws)
    rc = _lib.load().ssd_chunk_scan(ctypes.byref(d.c()), _p(x), xs, _p(dt), _p(A), _p(D), _p(Bm),
                                    _p(Cm), bs, _p(z), _p(norm_w), float(eps), _p(ssm_state_in),
                                    _p(ssm_state_out), _p(y), _p(ws), ws.numel(), _stream(stream))
    _check(rc, "ssd_chunk_scan")
    return y


def ssd_gated_rmsnorm(d: SSDDims, y, z, w, eps=1e-5, out=None, stream=None):
    io, n = d.io_dtype, d.batch * d.seqlen * d.hp
    _want(y, "y", io, n)
    _want(z, "z", io, n)
    _want(w, "w", io, d.hp)
    if out is None:
        out = _alloc(stream, lambda: torch.empty_like(y))
    _want(out, "out", io, n)
    _need_cuda(y, z, w, out)
    rc = _lib.load().ssd_gated_rmsnorm(ctypes.byref(d.c()), _p(y), _p(z), _p(w), float(eps),
                                       _p(out), _stream(stream))
    _check(rc, "ssd_gated_rmsnorm")
    return out


def ssd_decode_step(d: SSDDims, xbc_t, z_t, dt_t, A, D, conv_w, conv_b, norm_w, eps,
                    conv_state, ssm_state, y_t=None, stream=None):
    io, f32 = d.io_dtype, torch.float32
    B, H, C = d.batch, d.nheads, d.channels
    _want(xbc_t, "xbc_t", io, B * C)
    _want(z_t, "z_t", io, B * d.hp, optional=True)
    _want(dt_t, "dt_t", io, B * H)
    _want(A, "A", f32, H)
    _want(D, "D", f32, H, optional=True)
    _want(conv_w, "conv_w", io, C * d.conv_width)
    _want(conv_b, "conv_b", io, C, optional=True)
    _want(norm_w, "norm_w", io, d.hp, optional=z_t is None)
    _want(conv_state, "conv_state", io, B * (d.conv_width - 1) * C)
    _want(ssm_state, "ssm_state", f32, B * H * d.headdim * d.dstate)
    if y_t is None:
        y_t = _alloc(stream, lambda: torch.empty(B, d.hp, dtype=io, device=xbc_t.device))
    _want(y_t, "y_t", io, B * d.hp)
    _need_cuda(xbc_t, z_t, dt_t, A, D, conv_w, conv_b, norm_w, conv_state, ssm_state, y_t)
    rc = _lib.load().ssd_decode_step(ctypes.byref(d.c()), _p(xbc_t), _p(z_t), _p(dt_t), _p(A),
                                     _p(D), _p(conv_w), _p(conv_b), _p(norm_w), float(eps),
                                     _p(conv_state), _p(ssm_state), _p(y_t), _stream(stream))
    _check(rc, "ssd_decode_step")
    return y_t


def ssd_mixer_prefill(d: SSDDims, xbc, z, dt, A, D, conv_w, conv_b, norm_w, eps=1e-5,
                      conv_state_in=None, conv_state_out=None, ssm_state_in=None,
                      ssm_state_out=None, out=None, ws=None, stream=None):
    io, f32 = d.io_dtype, torch.float32
    B, L, H, C = d.batch, d.seqlen, d.nheads, d.channels
    _want(xbc, "xbc", io, B * L * C)
    _want(z, "z", io, B * L * d.hp, optional=True)
    _want(dt, "dt", io, B * L * H)
    _want(A, "A", f32, H)
    _want(D, "D", f32, H, optional=True)
    _want(conv_w, "conv_w", io, C * d.conv_width)
    _want(conv_b, "conv_b", io, C, optional=True)
    _want(norm_w, "norm_w", io, d.hp, optional=z is None)
    ncs, nss = B * (d.conv_width - 1) * C, B * H * d.headdim * d.dstate
    _want(conv_state_in, "conv_state_in", io, ncs, optional=True)
    _want(conv_state_out, "conv_state_out", io, ncs, optional=True)
    _want(ssm_state_in, "ssm_state_in", f32, nss, optional=True)
    _want(ssm_state_out, "ssm_state_out", f32, nss, optional=True)
    if out is None:
        out = _alloc(stream, lambda: torch.empty(B, L, d.hp, dtype=io, device=xbc.device))
    _want(out, "out", io, B * L * d.hp)
    need = ssd_mixer_prefill_workspace_bytes(d)
    if ws is None:
        ws = _alloc(stream, lambda: workspace(need, xbc.device))
    _want_ws(ws, need)
    _need_cuda(xbc, z, dt, A, D, conv_w, conv_b, norm_w, conv_state_in, conv_state_out,
               ssm_state_in, ssm_state_out, out, ws)
    rc = _lib.load().ssd_mixer_prefill(ctypes.byref(d.c()), _p(xbc), _p(z), _p(dt), _p(A), _p(D),
                                       _p(conv_w), _p(conv_b), _p(norm_w), float(eps),
                                       _p(conv_state_in), _p(conv_state_out), _p(ssm_state_in),
                                       _p(ssm_state_out), _p(out), _p(ws), ws.numel(),
                                       _stream(stream))
    _check(rc, "ssd_mixer_prefill")
    return out


def _want_packed(t, name: str, d: SSDDims, lead: tuple) -> int:
    """Packed projection rows [..., row] with row >= 2HP + 2GN + H, the row
    dense; returns the row stride (elements between tokens)."""
    width = 2 * d.hp + 2 * d.ngroups * d.dstate + d.nheads
    if t.dtype != d.io_dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {d.io_dtype}")
    if tuple(t.shape[:-1]) != lead or t.shape[-1] < width:
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {list(lead)} + [>= {width}]")
    if t.stride(-1) != 1:
        raise ValueError(f"{name}: rows must be dense")
    rs = t.stride(-2)
    for i in range(len(lead) - 1):   # outer dims stack rows evenly
        if lead[i] > 1 and t.stride(i) != rs * int(np.prod(lead[i + 1:])):
            raise ValueError(f"{name}: outer strides must be multiples of the row stride")
    return rs


def ssd_mixer_prefill_packed(d: SSDDims, zxbcdt, dt_bias, A_log, D, conv_w, conv_b, norm_w,
                             eps=1e-5, conv_state_in=None, conv_state_out=None,
                             ssm_state_in=None, ssm_state_out=None, out=None, ws=None,
                             stream=None):
    """Prefill on the projection's packed rows [z | xBC | dt_raw] ([B, L, row]),
    with dt = softplus(dt_raw + dt_bias) and A = -exp(A_log) formed in the
    kernels."""
    io, f32 = d.io_dtype, torch.float32
    B, L, H, C = d.batch, d.seqlen, d.nheads, d.channels
    rs = _want_packed(zxbcdt, "zxbcdt", d, (B, L))
    _want(dt_bias, "dt_bias", f32, H)
    _want(A_log, "A_log", f32, H)
    _want(D, "D", f32, H, optional=True)
    _want(conv_w, "conv_w", io, C * d.conv_width)
    _want(conv_b, "conv_b", io, C, optional=True)
    _want(norm_w, "norm_w", io, d.hp)
    ncs, nss = B * (d.conv_width - 1) * C, B * H * d.headdim * d.dstate
    _want(conv_state_in, "conv_state_in", io, ncs, optional=True)
    _want(conv_state_out, "conv_state_out", io, ncs, optional=True)
    _want(ssm_state_in, "ssm_state_in", f32, nss, optional=True)
    _want(ssm_state_out, "ssm_state_out", f32, nss, optional=True)
    if out is None:
        out = _alloc(stream, lambda: torch.empty(B, L, d.hp, dtype=io, device=zxbcdt.device))
    _want(out, "out", io, B * L * d.hp)
    need = ssd_mixer_prefill_workspace_bytes(d)
    if ws is None:
        ws = _alloc(stream, lambda: workspace(need, zxbcdt.device))
    _want_ws(ws, need)
    _need_cuda(zxbcdt, dt_bias, A_log, D, conv_w, conv_b, norm_w, conv_state_in, conv_state_out,
               ssm_state_in, ssm_state_out, out, ws)
    rc = _lib.load().ssd_mixer_prefill_packed(
        ctypes.byref(d.c()), _p(zxbcdt), rs, _p(dt_bias), _p(A_log), _p(D), _p(conv_w),
        _p(conv_b), _p(norm_w), float(eps), _p(conv_state_in), _p(conv_state_out),
        _p(ssm_state_in), _p(ssm_state_out), _p(out), _p(ws), ws.numel(), _stream(stream))
    _check(rc, "ssd_mixer_prefill_packed")
    return out


def ssd_decode_step_packed(d: SSDDims, zxbcdt_t, dt_bias, A_log, D, conv_w, conv_b, norm_w, eps,
                           conv_state, ssm_state, y_t=None, stream=None):
    """One decode token per sequence from packed rows [B, row]."""
    io, f32 = d.io_dtype, torch.float32
    B, H, C = d.batch, d.nheads, d.channels
    rs = _want_packed(zxbcdt_t, "zxbcdt_t", d, (B,))
    _want(dt_bias, "dt_bias", f32, H)
    _want(A_log, "A_log", f32, H)
    _want(D, "D", f32, H, optional=True)
    _want(conv_w, "conv_w", io, C * d.conv_width)
    _want(conv_b, "conv_b", io, C, optional=True)
    _want(norm_w, "norm_w", io, d.hp)
    _want(conv_state, "conv_state", io, B * (d.conv_width - 1) * C)
    _want(ssm_state, "ssm_state", f32, B * H * d.headdim * d.dstate)
    if y_t is None:
        y_t = _alloc(stream, lambda: torch.empty(B, d.hp, dtype=io, device=zxbcdt_t.device))
    _want(y_t, "y_t", io, B * d.hp)
    _need_cuda(zxbcdt_t, dt_bias, A_log, D, conv_w, conv_b, norm_w, conv_state, ssm_state, y_t)
    rc = _lib.load().ssd_decode_step_packed(
        ctypes.byref(d.c()), _p(zxbcdt_t), rs, _p(dt_bias), _p(A_log), _p(D), _p(conv_w),
        _p(conv_b), _p(norm_w), float(eps), _p(conv_state), _p(ssm_state), _p(y_t),
        _stream(stream))
    _check(rc, "ssd_decode_step_packed")
    return y_t


def ssd_mixer_varlen_workspace_bytes(d: SSDDims, num_slots: int) -> int:
    return int(_lib.load().ssd_mixer_varlen_workspace_bytes(ctypes.byref(d.c()), int(num_slots)))


def ssd_mixer_varlen(d: SSDDims, cu_seqlens, slots, xbc, z, dt, A, D, conv_w, conv_b, norm_w,
                     conv_pool, ssm_pool, eps=1e-5, has_state=None, out=None, ws=None,
                     stream=None):
    """Ragged sequences (d.batch of them, d.seqlen tokens in all) packed back
    to back, each resuming from and writing back its state slot in the
    pools; cu_seqlens [batch+1] and slots [batch] int32 device tensors,
    has_state [batch] uint8 or None. Check the call's validity with
    ssd_workspace_status(ws) (SSD_ERR_VARLEN when offsets or slots are bad)."""
    io, f32 = d.io_dtype, torch.float32
    B, T, H, C = d.batch, d.seqlen, d.nheads, d.channels
    _want(cu_seqlens, "cu_seqlens", torch.int32, B + 1)
    _want(slots, "slots", torch.int32, B)
    _want(has_state, "has_state", torch.uint8, B, optional=True)
    _want(xbc, "xbc", io, T * C)
    _want(z, "z", io, T * d.hp, optional=True)
    _want(dt, "dt", io, T * H)
    _want(A, "A", f32, H)
    _want(D, "D", f32, H, optional=True)
    _want(conv_w, "conv_w", io, C * d.conv_width)
    _want(conv_b, "conv_b", io, C, optional=True)
    _want(norm_w, "norm_w", io, d.hp, optional=z is None)
    if conv_pool.dtype != io or not conv_pool.is_contiguous() or conv_pool.dim() != 3 or \
            tuple(conv_pool.shape[1:]) != (d.conv_width - 1, C):
        raise ValueError(f"conv_pool: expected contiguous [slots, {d.conv_width - 1}, {C}] {io}")
    S = conv_pool.shape[0]
    _want(ssm_pool, "ssm_pool", f32, S * H * d.headdim * d.dstate)
    if out is None:
        out = _alloc(stream, lambda: torch.empty(T, d.hp, dtype=io, device=xbc.device))
    _want(out, "out", io, T * d.hp)
    need = ssd_mixer_varlen_workspace_bytes(d, S)
    if need == 0:
        raise SSDError(-3, "ssd_mixer_varlen_workspace_bytes")
    if ws is None:
        ws = _alloc(stream, lambda: workspace(need, xbc.device))
    _want_ws(ws, need)
    _need_cuda(cu_seqlens, slots, has_state, xbc, z, dt, A, D, conv_w, conv_b, norm_w,
               conv_pool, ssm_pool, out, ws)
    rc = _lib.load().ssd_mixer_varlen(
        ctypes.byref(d.c()), _p(cu_seqlens), _p(slots), _p(has_state), S, _p(xbc), _p(z),
        _p(dt), _p(A), _p(D), _p(conv_w), _p(conv_b), _p(norm_w), float(eps), _p(conv_pool),
        _p(ssm_pool), _p(out), _p(ws), ws.numel(), _stream(stream))
    _check(rc, "ssd_mixer_varlen")
    return out


def ssd_mixer_prefill_noalloc(d: SSDDims, xbc, z, dt, A, D, conv_w, conv_b, norm_w, out,
                              eps=1e-5, conv_state_in=None, conv_state_out=None,
                              ssm_state_in=None, ssm_state_out=None, stream=None):
    """ssd_mixer_prefill with the library's fixed per-GPU scratch buffer
    instead of a workspace; `out` is required, so nothing is allocated."""
    io, f32 = d.io_dtype, torch.float32
    B, L, H, C = d.batch, d.seqlen, d.nheads, d.channels
    _want(xbc, "xbc", io, B * L * C)
    _want(z, "z", io, B * L * d.hp, optional=True)
    _want(dt, "dt", io, B * L * H)
    _want(A, "A", f32, H)
    _want(D, "D", f32, H, optional=True)
    _want(conv_w, "conv_w", io, C * d.conv_width)
    _want(conv_b, "conv_b", io, C, optional=True)
    _want(norm_w, "norm_w", io, d.hp, optional=z is None)
    ncs, nss = B * (d.conv_width - 1) * C, B * H * d.headdim * d.dstate
    _want(conv_state_in, "conv_state_in", io, ncs, optional=True)
    _want(conv_state_out, "conv_state_out", io, ncs, optional=True)
    _want(ssm_state_in, "ssm_state_in", f32, nss, optional=True)
    _want(ssm_state_out, "ssm_state_out", f32, nss, optional=True)
    _want(out, "out", io, B * L * d.hp)
    _need_cuda(xbc, z, dt, A, D, conv_w, conv_b, norm_w, conv_state_in, conv_state_out,
               ssm_state_in, ssm_state_out, out)
    rc = _lib.load().ssd_mixer_prefill_noalloc(
        ctypes.byref(d.c()), _p(xbc), _p(z), _p(dt), _p(A), _p(D), _p(conv_w), _p(conv_b),
        _p(norm_w), float(eps), _p(conv_state_in), _p(conv_state_out), _p(ssm_state_in),
        _p(ssm_state_out), _p(out), _stream(stream))
    _check(rc, "ssd_mixer_prefill_noalloc")
    return out


def ssd_mixer_backward_workspace_bytes(d: SSDDims) -> int:
    return int(_lib.load().ssd_mixer_backward_workspace_bytes(ctypes.byref(d.c())))


BACKWARD_GRADS = ("xbc", "z", "dt", "A", "D", "conv_w", "conv_b", "norm_w", "conv_state_in",
                  "ssm_state_in")


def ssd_mixer_backward(d: SSDDims, xbc, z, dt, A, D, conv_w, conv_b, norm_w, d_out, eps=1e-5,
                       conv_state_in=None, ssm_state_in=None, d_ssm_state_out=None,
                       grads=None, ws=None, stream=None):
    """Gradients of the mixer prefill (conv + SiLU, chunked scan, gated
    norm) for upstream gradient d_out (and d_ssm_state_out of the final
    state). Returns a dict keyed by BACKWARD_GRADS: xbc, z, dt in the I/O
    dtype; A, D, conv_w, conv_b, norm_w and the two initial states in fp32
    (D, conv_b and the states only when the forward had them). `grads` may
    supply any of these output tensors."""
    io, f32 = d.io_dtype, torch.float32
    B, L, H, C, W = d.batch, d.seqlen, d.nheads, d.channels, d.conv_width
    _want(xbc, "xbc", io, B * L * C)
    _want(z, "z", io, B * L * d.hp)
    _want(dt, "dt", io, B * L * H)
    _want(A, "A", f32, H)
    _want(D, "D", f32, H, optional=True)
    _want(conv_w, "conv_w", io, C * W)
    _want(conv_b, "conv_b", io, C, optional=True)
    _want(norm_w, "norm_w", io, d.hp)
    _want(d_out, "d_out", io, B * L * d.hp)
    ncs, nss = B * (W - 1) * C, B * H * d.headdim * d.dstate
    _want(conv_state_in, "conv_state_in", io, ncs, optional=True)
    _want(ssm_state_in, "ssm_state_in", f32, nss, optional=True)
    _want(d_ssm_state_out, "d_ssm_state_out", f32, nss, optional=True)
    dev = xbc.device
    spec = {"xbc": ((B, L, C), io), "z": ((B, L, d.hp), io), "dt": ((B, L, H), io),
            "A": ((H,), f32), "D": ((H,), f32), "conv_w": ((C, W), f32), "conv_b": ((C,), f32),
            "norm_w": ((d.hp,), f32), "conv_state_in": ((B, W - 1, C), f32),
            "ssm_state_in": ((B, H, d.headdim, d.dstate), f32)}
    present = {"D": D is not None, "conv_b": conv_b is not None,
               "conv_state_in": conv_state_in is not None,
               "ssm_state_in": ssm_state_in is not None}
    g = dict(grads or {})
    for k in BACKWARD_GRADS:
        if not present.get(k, True):
            g.pop(k, None)
            continue
        shape, dtype = spec[k]
        if g.get(k) is None:
            g[k] = _alloc(stream, lambda: torch.empty(shape, dtype=dtype, device=dev))
        n = 1
        for s in shape:
            n *= s
        _want(g[k], "grad " + k, dtype, n)
    need = ssd_mixer_backward_workspace_bytes(d)
    if need == 0:
        raise SSDError(-3, "ssd_mixer_backward_workspace_bytes")
    if ws is None:
        ws = _alloc(stream, lambda: workspace(need, dev))
    _want_ws(ws, need)
    _need_cuda(xbc, z, dt, A, D, conv_w, conv_b, norm_w, d_out, conv_state_in, ssm_state_in,
               d_ssm_state_out, ws, *g.values())
    rc = _lib.load().ssd_mixer_backward(
        ctypes.byref(d.c()), _p(xbc), _p(z), _p(dt), _p(A), _p(D), _p(conv_w), _p(conv_b),
        _p(norm_w), float(eps), _p(conv_state_in), _p(ssm_state_in), _p(d_out),
        _p(d_ssm_state_out), _p(g["xbc"]), _p(g["z"]), _p(g["dt"]), _p(g["A"]), _p(g.get("D")),
        _p(g["conv_w"]), _p(g.get("conv_b")), _p(g["norm_w"]), _p(g.get("conv_state_in")),
        _p(g.get("ssm_state_in")), _p(ws), ws.numel(), _stream(stream))
    _check(rc, "ssd_mixer_backward")
    return g


def ssd_workspace_status(ws, stream=None) -> int:
    """Status code of the scan / prefill call that last used workspace `ws`
    (waits for `stream`): 0, SSD_ERR_TIMEOUT (-9) or SSD_ERR_NONFINITE (-10)."""
    _need_cuda(ws)
    return int(_lib.load().ssd_workspace_status(_p(ws), _stream(stream)))


def ssd_set_exchange_spin_limit(polls: int) -> int:
    """Diagnostic: bound on the fused path's cross-block norm polls; returns
    the previous bound."""
    rc = int(_lib.load().ssd_set_exchange_spin_limit(int(polls)))
    if rc < 0:
        raise SSDError(rc, "ssd_set_exchange_spin_limit")
    return rc


def ssd_set_backward_chunk_heads(heads: int) -> int:
    """Diagnostic: heads per workgroup of the backward's per-chunk kernels
    (0: chosen from the shape); returns the previous setting."""
    rc = int(_lib.load().ssd_set_backward_chunk_heads(int(heads)))
    if rc < 0:
        raise SSDError(rc, "ssd_set_backward_chunk_heads")
    return rc


def ssd_set_output_norm_fusion(mode: int) -> int:
    """Diagnostic: the general kernels' gated norm inside the output kernel
    (0: chosen from the shape, 1: wherever the group fits, 2: never);
    returns the previous mode."""
    rc = int(_lib.load().ssd_set_output_norm_fusion(int(mode)))
    if rc < 0:
        raise SSDError(rc, "ssd_set_output_norm_fusion")
    return rc


def profile_start(capacity: int) -> None:
    """Time every kernel launch of the library with a pair of HIP events on
    the launch stream, for the next `capacity` launches."""
    _check(_lib.load().ssd_profile_start(int(capacity)), "ssd_profile_start")


def profile_stop() -> None:
    _check(_lib.load().ssd_profile_stop(), "ssd_profile_stop")


def profile_only(kernels=None) -> None:
    """Time only the named kernels from now on (None: every kernel)."""
    mask = (1 << 64) - 1 if kernels is None else sum(1 << _lib.KERNELS.index(k) for k in kernels)
    _lib.load().ssd_profile_set_mask(mask)


def profile_read(kernel: str) -> tuple[int, float]:
    """(timed launches, summed milliseconds) of one kernel since profile_start."""
    n = ctypes.c_int64(0)
    ms = ctypes.c_double(0.0)
    _check(_lib.load().ssd_profile_read(_lib.KERNELS.index(kernel), ctypes.byref(n),
                                        ctypes.byref(ms)), "ssd_profile_read")
    return int(n.value), float(ms.value)
