"""The C ABI on the host: the library loads without a GPU, exports every
symbol the header declares, and its host-only logic (validation, state
sizing, argument checks that return before any launch) behaves as
documented. No test here launches a kernel."""
import ctypes
import json
import os
import re

import pytest

from mamba_ssd_selective_mixer_amd import _lib, synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssd_mi355x.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return _lib.load()


def dims(cfg, **kw):
    base = dict(batch=cfg.batch, seqlen=cfg.seqlen, nheads=cfg.nheads, headdim=cfg.headdim,
                ngroups=cfg.ngroups, dstate=cfg.dstate, conv_width=cfg.conv_width,
                chunk=cfg.chunk or 128,
                io_dtype=_lib.SSD_BF16 if cfg.dtype == "bf16" else _lib.SSD_F32)
    base.update(kw)
    return _lib.Dims(**base)


def test_exports_every_declared_symbol(lib):
    text = open(HEADER).read()
    declared = set(re.findall(r"\b(ssd_[a-z0-9_]+)\s*\(", text))
    assert declared, "no declarations parsed"
    assert declared == set(_lib.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name


def test_validate_configs(lib):
    for name, entry in [("tiny_fp32", 4), ("tiny_layer", 4), ("large_layer", 4), ("long_context", 4), ("tiny_layer", 1), ("tiny_fp32", 0)]:
        assert lib.ssd_validate(entry, ctypes.byref(dims(synth.CONFIGS[name]))) == 0, name
    dec = synth.CONFIGS["decode_loop"]
    assert lib.ssd_validate(3, ctypes.byref(dims(dec, chunk=128))) == 0


@pytest.mark.parametrize("kw,entry,rc", [
    (dict(nheads=30), 1, -2),          # n_groups must divide the heads
    (dict(headdim=48), 1, -3),
    (dict(dstate=512), 1, -3),
    (dict(dstate=256), 1, 0),
    (dict(dstate=256, seqlen=1), 3, 0),
    (dict(flags=2), 1, -3),            # unknown flag bits
    (dict(io_dtype=7), 1, -4),
    (dict(seqlen=0), 1, -2),
    (dict(batch=0), 0, -2),
    (dict(chunk=100), 1, -3),
    (dict(conv_width=5), 0, -3),
    (dict(conv_width=5), 1, 0),        # the scan alone has no conv
    (dict(seqlen=2), 3, -2),           # decode is one token
    (dict(), 9, -3),
])
def test_validate_errors(lib, kw, entry, rc):
    assert lib.ssd_validate(entry, ctypes.byref(dims(synth.CONFIGS["tiny_layer"], **kw))) == rc


def test_envelope_fits_lds(lib):
    """The general kernels run 64-token chunks whatever the caller's chunk, so
    every head size, state size and chunk of the envelope fits one CU's LDS,
    fp32 I/O and fp32 operands included (the widest: head 128, state 256)."""
    for io in (_lib.SSD_F32, _lib.SSD_BF16):
        for P in (16, 32, 64, 128):
            for N in (16, 32, 64, 128, 256):
                for Q in (32, 64, 128, 256):
                    for flags in (0, _lib.SSD_FLAG_FP32_OPERANDS):
                        d = dims(synth.CONFIGS["tiny_fp32"], headdim=P, dstate=N, chunk=Q, io_dtype=io,
                                 flags=flags)
                        assert lib.ssd_validate(1, ctypes.byref(d)) == 0, (io, P, N, Q, flags)


def test_status_strings(lib):
    for rc in _lib.STATUS:
        assert lib.ssd_status_str(rc)
    assert lib.ssd_status_str(-99) == b"unknown status"


def test_null_and_alignment_checks_return_before_launch(lib):
    d = dims(synth.CONFIGS["tiny_layer"])
    V = ctypes.c_void_p
    # NULL required pointer
    assert lib.ssd_conv1d(ctypes.byref(d), None, 4096, V(4096), None, None, None, V(8192), 4096,
                          None) == -1
    # misaligned pointer (never dereferenced: the check returns first)
    assert lib.ssd_conv1d(ctypes.byref(d), V(0x1008), 4096, V(4096), None, None, None,
                          V(1 << 40), 4096, None) == -8
    # token stride narrower than a row
    assert lib.ssd_conv1d(ctypes.byref(d), V(1 << 36), 100, V(4096), None, None, None,
                          V(1 << 40), 4096, None) == -2
    # output overlapping the input
    assert lib.ssd_conv1d(ctypes.byref(d), V(1 << 36), 4096, V(4096), None, None, None,
                          V((1 << 36) + 4096), 4096, None) == -5
    # workspace too small
    need = lib.ssd_chunk_scan_workspace_bytes(ctypes.byref(d))
    assert need > 0
    assert lib.ssd_chunk_scan(ctypes.byref(d), V(1 << 36), 4096, V(1 << 37), V(4096), None,
                              V(1 << 38), V(1 << 39), 4096, None, None, 1e-5, None, None,
                              V(1 << 40), V(1 << 41), need - 1, None) == -6
    # z without a norm weight
    assert lib.ssd_chunk_scan(ctypes.byref(d), V(1 << 36), 4096, V(1 << 37), V(4096), None,
                              V(1 << 38), V(1 << 39), 4096, V(1 << 42), None, 1e-5, None, None,
                              V(1 << 40), V(1 << 41), need, None) == -1
    # partially overlapping in/out SSM state
    S = 4 * 32 * 64 * 128 * 4
    assert lib.ssd_chunk_scan(ctypes.byref(d), V(1 << 36), 4096, V(1 << 37), V(4096), None,
                              V(1 << 38), V(1 << 39), 4096, None, None, 1e-5, V(1 << 43),
                              V((1 << 43) + S // 2), V(1 << 40), V(1 << 41), need, None) == -5


def test_prefill_decode_norm_refuse_before_launch(lib):
    """The mixer prefill, decode step and standalone norm refuse NULLs,
    misalignment, a short workspace, a wrong shape and aliasing with their
    documented codes, before any launch (addresses are never dereferenced)."""
    V = ctypes.c_void_p
    NULL, SHAPE, ALIAS, WORKSPACE, ALIGN = -1, -2, -5, -6, -8
    d = dims(synth.CONFIGS["tiny_layer"])
    need = lib.ssd_mixer_prefill_workspace_bytes(ctypes.byref(d))
    assert need > 0
    xbc, z, dt, A, D, cw, nw = (V(k << 36) for k in (1, 2, 3, 4, 5, 6, 7))
    cs_in, cs_out, ss_in, ss_out, out, ws = (V(k << 36) for k in (8, 9, 10, 11, 12, 13))

    def prefill(**kw):
        a = dict(xbc=xbc, z=z, dt=dt, A=A, D=D, cw=cw, cb=None, nw=nw, cs_in=cs_in,
                 cs_out=cs_out, ss_in=ss_in, ss_out=ss_out, out=out, ws=ws, n=need)
        a.update(kw)
        return lib.ssd_mixer_prefill(ctypes.byref(d), a["xbc"], a["z"], a["dt"], a["A"], a["D"],
                                     a["cw"], a["cb"], a["nw"], 1e-5, a["cs_in"], a["cs_out"],
                                     a["ss_in"], a["ss_out"], a["out"], a["ws"], a["n"], None)

    assert prefill(xbc=None) == NULL
    assert prefill(nw=None) == NULL                      # z given without a norm weight
    assert prefill(out=V((12 << 36) + 8)) == ALIGN
    assert prefill(n=need - 1) == WORKSPACE
    assert prefill(ws=None) == WORKSPACE
    assert prefill(cs_out=V((1 << 36) + 4096)) == ALIAS  # new conv state inside xBC
    assert prefill(cs_out=V((8 << 36) + 16)) == ALIAS    # conv states partly overlapping
    assert prefill(ss_out=V((10 << 36) + 64)) == ALIAS   # SSM states partly overlapping
    assert prefill(ws=V((12 << 36) + 256)) == ALIAS      # workspace over the output

    dd = dims(synth.CONFIGS["decode_loop"], seqlen=1)
    st, y = V(14 << 36), V(15 << 36)

    def decode(d_=dd, **kw):
        a = dict(x=xbc, z=z, dt=dt, cs=cs_in, ss=st, y=y, nw=nw)
        a.update(kw)
        return lib.ssd_decode_step(ctypes.byref(d_), a["x"], a["z"], a["dt"], A, D, cw, None,
                                   a["nw"], 1e-5, a["cs"], a["ss"], a["y"], None)

    assert decode(d_=dims(synth.CONFIGS["decode_loop"], seqlen=2)) == SHAPE
    assert decode(ss=None) == NULL
    assert decode(nw=None) == NULL
    assert decode(y=V((15 << 36) + 4)) == ALIGN
    assert decode(cs=V((14 << 36) + 4096)) == ALIAS      # conv state inside the SSM state

    n = 4 * 2048 * 32 * 64 * 2
    assert lib.ssd_gated_rmsnorm(ctypes.byref(d), None, z, nw, 1e-5, out, None) == NULL
    assert lib.ssd_gated_rmsnorm(ctypes.byref(d), y, z, nw, 1e-5, V((12 << 36) + 2), None) == ALIGN
    assert lib.ssd_gated_rmsnorm(ctypes.byref(d), y, z, nw, 1e-5, V((15 << 36) + n // 2),
                                 None) == ALIAS          # out partly over y
    assert lib.ssd_gated_rmsnorm(ctypes.byref(d), y, z, nw, 1e-5, z, None) == ALIAS


def test_workspace_sizes(lib):
    tiny = synth.CONFIGS["tiny_layer"]
    d = dims(tiny)
    ws = lib.ssd_chunk_scan_workspace_bytes(ctypes.byref(d))
    nc = tiny.seqlen // 128
    assert ws >= tiny.batch * nc * tiny.nheads * tiny.headdim * tiny.dstate * 2  # fp16 chunk states
    # the general path (state 64 here): fp32 states of 64-token chunks, fp32 y
    g = dims(tiny, dstate=64)
    wg = lib.ssd_chunk_scan_workspace_bytes(ctypes.byref(g))
    assert wg >= (tiny.batch * (tiny.seqlen // 64) * tiny.nheads * tiny.headdim * 64 * 4
                  + tiny.batch * tiny.seqlen * tiny.hp * 4)
    assert lib.ssd_mixer_prefill_workspace_bytes(ctypes.byref(d)) >= ws
    bad = dims(tiny, headdim=48)
    assert lib.ssd_chunk_scan_workspace_bytes(ctypes.byref(bad)) == 0


def test_workspace_covers_wide_norm_groups(lib):
    """Large-layer shape (32 heads per norm group): the prefill workspace holds
    the fp16 chunk increments (overwritten in place by the carried-in states),
    the convolved B and C rows the output kernel reads, and the per-row sums
    its blocks exchange."""
    large = synth.CONFIGS["large_layer"]
    d = dims(large)
    ws = lib.ssd_mixer_prefill_workspace_bytes(ctypes.byref(d))
    nc = -(-large.seqlen // 128)
    states = large.batch * nc * large.nheads * large.headdim * large.dstate * 2
    rows = 2 * large.batch * large.seqlen * large.ngroups * large.dstate * 2
    sums = nc * large.batch * (large.nheads // 4) * 128 * 4
    assert ws >= states + rows + sums


def test_state_slot_size_matches_page_figure(lib):
    """A sequence slot of Nemotron 3 Nano (23 Mamba-2 layers of 64 x 64 heads)
    holds 47.6 MiB of fp32 recurrent state (tests/golden/nano_recurrent_state.json)."""
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "nano_recurrent_state.json")))
    d = _lib.Dims(1, 1, g["nheads"], g["headdim"], g["ngroups"], g["dstate"], g["conv_width"],
                  128, _lib.SSD_BF16)
    per_layer = lib.ssd_ssm_state_bytes(ctypes.byref(d)) + lib.ssd_conv_state_bytes(ctypes.byref(d), 1)
    mib = g["mamba_layers"] * per_layer / 2 ** 20
    assert round(mib, 1) == g["mib_per_slot"]
    assert lib.ssd_conv_channels(ctypes.byref(d)) == 64 * 64 + 2 * 8 * 128


def test_kernel_names_and_profile_arguments(lib):
    """Kernel identifiers of the timing aid match the binding's table, and
    reading checks its arguments before touching any event."""
    for i, name in enumerate(_lib.KERNELS):
        assert lib.ssd_kernel_name(i).decode() == name
    assert lib.ssd_kernel_name(len(_lib.KERNELS)) == b"unknown"
    n, ms = ctypes.c_int64(0), ctypes.c_double(0)
    assert lib.ssd_profile_read(len(_lib.KERNELS), ctypes.byref(n), ctypes.byref(ms)) == -2
    assert lib.ssd_profile_read(0, None, ctypes.byref(ms)) == -1
    assert lib.ssd_profile_read(0, ctypes.byref(n), ctypes.byref(ms)) == 0 and n.value == 0
    assert lib.ssd_profile_start(0) == -2
    # the kernel mask: all kernels timed by default, the previous mask returned
    assert lib.ssd_profile_set_mask(5) == 2 ** 64 - 1
    assert lib.ssd_profile_set_mask(2 ** 64 - 1) == 5


# Every buffer a call writes against every other buffer it touches: placed
# at the same address (or, for its in-place twin, 256 bytes into it) the
# call must return SSD_ERR_ALIAS before any launch. Addresses are fake and
# never dereferenced.
_ALIAS = -5


def _alias_cases(buffers, written, twins):
    cases = []
    for w in written:
        for o in buffers:
            if o == w:
                continue
            cases.append((w, o, 256 if twins.get(w) == o else 0))
    return cases


_PREFILL_BUFS = ("xbc", "z", "dt", "A", "D", "cw", "cb", "nw", "cs_in", "cs_out", "ss_in",
                 "ss_out", "out", "ws")
_PREFILL_W = ("cs_out", "ss_out", "out", "ws")
_PREFILL_TWINS = {"cs_out": "cs_in", "ss_out": "ss_in"}


@pytest.mark.parametrize("w,o,off", _alias_cases(_PREFILL_BUFS, _PREFILL_W, _PREFILL_TWINS))
def test_prefill_alias_every_pair(lib, w, o, off):
    V = ctypes.c_void_p
    d = dims(synth.CONFIGS["tiny_layer"])
    need = lib.ssd_mixer_prefill_workspace_bytes(ctypes.byref(d))
    a = {k: (i + 1) << 36 for i, k in enumerate(_PREFILL_BUFS)}
    a[w] = a[o] + off
    rc = lib.ssd_mixer_prefill(ctypes.byref(d), *(V(a[k]) for k in _PREFILL_BUFS[:8]), 1e-5,
                               *(V(a[k]) for k in _PREFILL_BUFS[8:]), need, None)
    assert rc == _ALIAS


_SCAN_BUFS = ("x", "dt", "A", "D", "Bm", "Cm", "z", "nw", "ss_in", "ss_out", "y", "ws")
_SCAN_W = ("ss_out", "y", "ws")


@pytest.mark.parametrize("w,o,off", _alias_cases(_SCAN_BUFS, _SCAN_W, {"ss_out": "ss_in"}))
def test_chunk_scan_alias_every_pair(lib, w, o, off):
    V = ctypes.c_void_p
    d = dims(synth.CONFIGS["tiny_layer"])
    need = lib.ssd_chunk_scan_workspace_bytes(ctypes.byref(d))
    a = {k: (i + 1) << 36 for i, k in enumerate(_SCAN_BUFS)}
    a[w] = a[o] + off
    rc = lib.ssd_chunk_scan(ctypes.byref(d), V(a["x"]), 4096, V(a["dt"]), V(a["A"]), V(a["D"]),
                            V(a["Bm"]), V(a["Cm"]), 4096, V(a["z"]), V(a["nw"]), 1e-5,
                            V(a["ss_in"]), V(a["ss_out"]), V(a["y"]), V(a["ws"]), need, None)
    assert rc == _ALIAS


_DEC_BUFS = ("x", "z", "dt", "A", "D", "cw", "cb", "nw", "cs", "ss", "y")
_DEC_W = ("cs", "ss", "y")


@pytest.mark.parametrize("w,o,off", _alias_cases(_DEC_BUFS, _DEC_W, {}))
def test_decode_alias_every_pair(lib, w, o, off):
    V = ctypes.c_void_p
    d = dims(synth.CONFIGS["decode_loop"], seqlen=1)
    a = {k: (i + 1) << 36 for i, k in enumerate(_DEC_BUFS)}
    a[w] = a[o] + off
    rc = lib.ssd_decode_step(ctypes.byref(d), *(V(a[k]) for k in _DEC_BUFS[:8]), 1e-5,
                             *(V(a[k]) for k in _DEC_BUFS[8:]), None)
    assert rc == _ALIAS


_CONV_BUFS = ("xbc", "w", "bias", "cs_in", "cs_out", "out")


@pytest.mark.parametrize("w,o,off", _alias_cases(_CONV_BUFS, ("cs_out", "out"),
                                                 {"cs_out": "cs_in"}))
def test_conv1d_alias_every_pair(lib, w, o, off):
    V = ctypes.c_void_p
    d = dims(synth.CONFIGS["tiny_layer"])
    a = {k: (i + 1) << 36 for i, k in enumerate(_CONV_BUFS)}
    a[w] = a[o] + off
    rc = lib.ssd_conv1d(ctypes.byref(d), V(a["xbc"]), 4096, V(a["w"]), V(a["bias"]),
                        V(a["cs_in"]), V(a["cs_out"]), V(a["out"]), 4096, None)
    assert rc == _ALIAS


@pytest.mark.parametrize("o", ["z", "w"])
def test_gated_rmsnorm_alias_every_pair(lib, o):
    V = ctypes.c_void_p
    d = dims(synth.CONFIGS["tiny_layer"])
    a = {"y": 1 << 36, "z": 2 << 36, "w": 3 << 36}
    assert lib.ssd_gated_rmsnorm(ctypes.byref(d), V(a["y"]), V(a["z"]), V(a["w"]), 1e-5,
                                 V(a[o]), None) == _ALIAS
    # out may equal y (in place) but not sit partly over it
    assert lib.ssd_gated_rmsnorm(ctypes.byref(d), V(a["y"]), V(a["z"]), V(a["w"]), 1e-5,
                                 V(a["y"] + 256), None) == _ALIAS


_PK_BUFS = ("row", "dtb", "alog", "D", "cw", "cb", "nw", "cs_in", "cs_out", "ss_in", "ss_out",
            "out", "ws")
_PK_W = ("cs_out", "ss_out", "out", "ws")


@pytest.mark.parametrize("w,o,off", _alias_cases(_PK_BUFS, _PK_W,
                                                 {"cs_out": "cs_in", "ss_out": "ss_in"}))
def test_prefill_packed_alias_every_pair(lib, w, o, off):
    V = ctypes.c_void_p
    d = dims(synth.CONFIGS["tiny_layer"])
    need = lib.ssd_mixer_prefill_workspace_bytes(ctypes.byref(d))
    a = {k: (i + 1) << 36 for i, k in enumerate(_PK_BUFS)}
    a[w] = a[o] + off
    rs = 2 * 2048 + 2 * 1024 + 32
    rc = lib.ssd_mixer_prefill_packed(ctypes.byref(d), V(a["row"]), rs,
                                      *(V(a[k]) for k in _PK_BUFS[1:7]), 1e-5,
                                      *(V(a[k]) for k in _PK_BUFS[7:]), need, None)
    assert rc == _ALIAS


def test_packed_entries_refuse_before_launch(lib):
    """Row stride narrower than [z | xBC | dt] or breaking the 16-byte rule,
    missing dt_bias / A_log / norm weight: refused before any launch."""
    V = ctypes.c_void_p
    d = dims(synth.CONFIGS["tiny_layer"])
    need = lib.ssd_mixer_prefill_workspace_bytes(ctypes.byref(d))
    width = 2 * 2048 + 2 * 1024 + 32
    a = [V(k << 36) for k in range(1, 14)]

    def pre(rs=width + 8, **kw):
        args = list(a)
        for i, v in kw.items():
            args[int(i[1:])] = v
        return lib.ssd_mixer_prefill_packed(ctypes.byref(d), args[0], rs, *args[1:7], 1e-5,
                                            *args[7:], need, None)

    assert pre(rs=width - 1) == -2
    assert pre(rs=width + 1) == -8                 # (width + 1) * 2 bytes is not 16-aligned
    assert pre(a1=None) == -1                      # dt_bias
    assert pre(a2=None) == -1                      # A_log
    assert pre(a6=None) == -1                      # norm weight
    dd = dims(synth.CONFIGS["decode_loop"], seqlen=1)
    wdec = 2 * 16384 + 2 * 1024 + 256
    assert lib.ssd_decode_step_packed(ctypes.byref(dd), a[0], wdec - 8, *a[1:7], 1e-5, *a[7:10],
                                      None) == -2
    assert lib.ssd_decode_step_packed(ctypes.byref(dd), a[0], wdec, None, *a[2:7], 1e-5,
                                      *a[7:10], None) == -1
    # y_t over the packed rows
    assert lib.ssd_decode_step_packed(ctypes.byref(dd), a[0], wdec, *a[1:7], 1e-5, a[7], a[8],
                                      V((1 << 36) + 4096), None) == -5


_VL_BUFS = ("xbc", "z", "dt", "A", "D", "cw", "cb", "nw", "cu", "slots", "has", "cpool",
            "spool", "out", "ws")
_VL_W = ("cpool", "spool", "out", "ws")


@pytest.mark.parametrize("w,o,off", _alias_cases(_VL_BUFS, _VL_W, {}))
def test_varlen_alias_every_pair(lib, w, o, off):
    V = ctypes.c_void_p
    d = dims(synth.CONFIGS["tiny_layer"], batch=3, seqlen=500)
    need = lib.ssd_mixer_varlen_workspace_bytes(ctypes.byref(d), 8)
    a = {k: (i + 1) << 36 for i, k in enumerate(_VL_BUFS)}
    a[w] = a[o] + off
    rc = lib.ssd_mixer_varlen(ctypes.byref(d), V(a["cu"]), V(a["slots"]), V(a["has"]), 8,
                              *(V(a[k]) for k in _VL_BUFS[:8]), 1e-5, V(a["cpool"]),
                              V(a["spool"]), V(a["out"]), V(a["ws"]), need, None)
    assert rc == _ALIAS


def test_varlen_envelope_and_refusals(lib):
    """The batched entry runs on the fused kernels only: other shapes, flags
    or a missing pool are refused before any launch."""
    V = ctypes.c_void_p
    d = dims(synth.CONFIGS["tiny_layer"], batch=3, seqlen=500)
    assert lib.ssd_mixer_varlen_workspace_bytes(ctypes.byref(d), 8) > 0
    assert lib.ssd_mixer_varlen_workspace_bytes(ctypes.byref(d), 0) == 0
    for bad in (dict(dstate=64), dict(io_dtype=_lib.SSD_F32), dict(flags=1),
                dict(nheads=288, ngroups=1)):  # 288 heads per norm group: beyond the fused norm
        dd = dims(synth.CONFIGS["tiny_layer"], batch=3, seqlen=500, **bad)
        assert lib.ssd_mixer_varlen_workspace_bytes(ctypes.byref(dd), 8) == 0, bad
        a = [V(k << 36) for k in range(1, 16)]
        rc = lib.ssd_mixer_varlen(ctypes.byref(dd), a[0], a[1], None, 8, *a[2:10], 1e-5, *a[10:14],
                                  1 << 30, None)
        assert rc == -3, bad
    a = [V(k << 36) for k in range(1, 16)]
    need = lib.ssd_mixer_varlen_workspace_bytes(ctypes.byref(d), 8)
    assert lib.ssd_mixer_varlen(ctypes.byref(d), None, a[1], None, 8, *a[2:10], 1e-5,
                                *a[10:14], need, None) == -1
    assert lib.ssd_mixer_varlen(ctypes.byref(d), a[0], a[1], None, 8, *a[2:10], 1e-5, None,
                                *a[11:14], need, None) == -1
    assert lib.ssd_mixer_varlen(ctypes.byref(d), a[0], a[1], None, 0, *a[2:10], 1e-5,
                                *a[10:14], need, None) == -2
    assert lib.ssd_mixer_varlen(ctypes.byref(d), a[0], a[1], None, 8, *a[2:10], 1e-5,
                                *a[10:14], need - 1, None) == -6


def test_argtypes_match_header_arity(lib):
    """Every prototype in the header has as many parameters as the binding
    passes (a missing or extra argument would shift every later one)."""
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    protos = re.findall(r"\b(ssd_[a-z0-9_]+)\s*\(([^)]*)\)\s*;", text)
    assert len(protos) == len(_lib.EXPORTS)
    for name, params in protos:
        params = params.strip()
        n = 0 if params in ("", "void") else params.count(",") + 1
        assert len(getattr(lib, name).argtypes) == n, name


_BWD_BUFS = ("xbc", "z", "dt", "A", "D", "cw", "cb", "nw", "cs_in", "ss_in", "d_out", "d_ss_out",
             "g_xbc", "g_z", "g_dt", "g_A", "g_D", "g_cw", "g_cb", "g_nw", "g_cs_in", "g_ss_in",
             "ws")
_BWD_W = ("g_xbc", "g_z", "g_dt", "g_A", "g_D", "g_cw", "g_cb", "g_nw", "g_cs_in", "g_ss_in",
          "ws")


def _bwd_call(lib, d, a, need):
    V = ctypes.c_void_p
    return lib.ssd_mixer_backward(ctypes.byref(d), *(V(a[k]) for k in _BWD_BUFS[:8]), 1e-5,
                                  *(V(a[k]) for k in _BWD_BUFS[8:]), need, None)


@pytest.mark.parametrize("w,o,off", _alias_cases(_BWD_BUFS, _BWD_W, {}))
def test_backward_alias_every_pair(lib, w, o, off):
    d = dims(synth.CONFIGS["tiny_layer"])
    need = lib.ssd_mixer_backward_workspace_bytes(ctypes.byref(d))
    a = {k: (i + 1) << 36 for i, k in enumerate(_BWD_BUFS)}
    a[w] = a[o] + off
    assert _bwd_call(lib, d, a, need) == _ALIAS


def test_backward_refuses_before_launch(lib):
    d = dims(synth.CONFIGS["tiny_layer"])
    need = lib.ssd_mixer_backward_workspace_bytes(ctypes.byref(d))
    # workspace: the status word, fp32 conv output / its gradient, y, chunk
    # states and their gradients (64-token chunks), per-head dB / dC, 1024
    # partial norm-weight gradients, the conv gradients' partial sums per
    # 64-token range, each chunk's parts of dA and dD, and each chunk's
    # C B^T per group (64 x 64 fp32)
    cfg = synth.CONFIGS["tiny_layer"]
    T, C, HP = cfg.batch * cfg.seqlen, cfg.channels, cfg.hp
    nc = -(-cfg.seqlen // 64)
    st = cfg.batch * nc * HP * cfg.dstate * 4
    r = lambda b: -(-b // 256) * 256
    assert need == (256 + 2 * r(T * C * 4) + r(T * HP * 4) + 2 * r(st)
                    + r(cfg.batch * cfg.nheads * nc * 4) + 2 * r(T * cfg.nheads * cfg.dstate * 4)
                    + r(1024 * HP * 4) + r(cfg.batch * nc * C * 5 * 4)
                    + r(2 * cfg.batch * nc * cfg.nheads * 4)
                    + r(cfg.batch * nc * cfg.ngroups * 64 * 64 * 4))
    base = {k: (i + 1) << 36 for i, k in enumerate(_BWD_BUFS)}
    for k in ("xbc", "z", "dt", "A", "cw", "nw", "d_out", "g_xbc", "g_z", "g_dt", "g_A", "g_cw",
              "g_nw", "ws"):
        a = dict(base)
        a[k] = 0
        assert _bwd_call(lib, d, a, need) == (-6 if k == "ws" else -1), k
    for k in ("D", "cb", "cs_in", "ss_in", "d_ss_out", "g_D", "g_cb", "g_cs_in", "g_ss_in"):
        a = dict(base)
        a[k] += 4
        assert _bwd_call(lib, d, a, need) == -8, k
    assert _bwd_call(lib, d, base, need - 1) == -6
    wide = dims(cfg, nheads=512)  # H*P = 32768 channels in a norm row
    assert lib.ssd_mixer_backward_workspace_bytes(ctypes.byref(wide)) == 0
    assert _bwd_call(lib, wide, base, need) == -3
    assert _bwd_call(lib, dims(cfg, flags=4), base, need) == -3


def test_output_norm_fusion_setting(lib):
    """The general path's norm-fusion diagnostic takes 0, 1 or 2, returns
    the previous mode, and refuses anything else."""
    prev = lib.ssd_set_output_norm_fusion(1)
    try:
        assert prev == 0
        for bad in (-1, 3, 100):
            assert lib.ssd_set_output_norm_fusion(bad) == -2, bad
        assert lib.ssd_set_output_norm_fusion(2) == 1
        assert lib.ssd_set_output_norm_fusion(0) == 2
    finally:
        lib.ssd_set_output_norm_fusion(0)


def test_backward_chunk_heads_setting(lib):
    """The per-chunk workgroup heads diagnostic takes 0 or a power of two up
    to 32, returns the previous setting, and refuses anything else."""
    prev = lib.ssd_set_backward_chunk_heads(4)
    try:
        assert prev == 0
        for bad in (-1, 3, 6, 64):
            assert lib.ssd_set_backward_chunk_heads(bad) == -2, bad
        assert lib.ssd_set_backward_chunk_heads(32) == 4
        assert lib.ssd_set_backward_chunk_heads(1) == 32
    finally:
        lib.ssd_set_backward_chunk_heads(0)
