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
    for name, entry in [("c0", 4), ("c1", 4), ("c2", 4), ("c3", 4), ("c1", 1), ("c0", 0)]:
        assert lib.ssd_validate(entry, ctypes.byref(dims(synth.CONFIGS[name]))) == 0, name
    c4 = synth.CONFIGS["c4"]
    assert lib.ssd_validate(3, ctypes.byref(dims(c4, chunk=128))) == 0


@pytest.mark.parametrize("kw,entry,rc", [
    (dict(nheads=30), 1, -2),          # n_groups must divide the heads
    (dict(headdim=48), 1, -3),
    (dict(dstate=256), 1, -3),
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
    assert lib.ssd_validate(entry, ctypes.byref(dims(synth.CONFIGS["c1"], **kw))) == rc


def test_fp32_envelope_limits_lds(lib):
    d = dims(synth.CONFIGS["c0"], headdim=128, dstate=128, chunk=256)
    assert lib.ssd_validate(1, ctypes.byref(d)) == -3
    d = dims(synth.CONFIGS["c0"], headdim=64, dstate=128, chunk=256)
    assert lib.ssd_validate(1, ctypes.byref(d)) == 0


def test_status_strings(lib):
    for rc in _lib.STATUS:
        assert lib.ssd_status_str(rc)
    assert lib.ssd_status_str(-99) == b"unknown status"


def test_null_and_alignment_checks_return_before_launch(lib):
    d = dims(synth.CONFIGS["c1"])
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
    d = dims(synth.CONFIGS["c1"])
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

    dd = dims(synth.CONFIGS["c4"], seqlen=1)
    st, y = V(14 << 36), V(15 << 36)

    def decode(d_=dd, **kw):
        a = dict(x=xbc, z=z, dt=dt, cs=cs_in, ss=st, y=y, nw=nw)
        a.update(kw)
        return lib.ssd_decode_step(ctypes.byref(d_), a["x"], a["z"], a["dt"], A, D, cw, None,
                                   a["nw"], 1e-5, a["cs"], a["ss"], a["y"], None)

    assert decode(d_=dims(synth.CONFIGS["c4"], seqlen=2)) == SHAPE
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
    c1 = synth.CONFIGS["c1"]
    d = dims(c1)
    ws = lib.ssd_chunk_scan_workspace_bytes(ctypes.byref(d))
    nc = c1.seqlen // c1.chunk
    assert ws >= c1.batch * nc * c1.nheads * c1.headdim * c1.dstate * 4
    assert lib.ssd_mixer_prefill_workspace_bytes(ctypes.byref(d)) >= ws
    bad = dims(c1, headdim=48)
    assert lib.ssd_chunk_scan_workspace_bytes(ctypes.byref(bad)) == 0


def test_workspace_covers_wide_norm_groups(lib):
    """Large-layer shape (32 heads per norm group): the prefill workspace holds
    the fp16 chunk increments and carried-in states, the convolved B and C
    rows the output kernel reads, and the per-row sums its blocks exchange."""
    c2 = synth.CONFIGS["c2"]
    d = dims(c2)
    ws = lib.ssd_mixer_prefill_workspace_bytes(ctypes.byref(d))
    nc = -(-c2.seqlen // 128)
    states = 2 * c2.batch * nc * c2.nheads * c2.headdim * c2.dstate * 2
    rows = 2 * c2.batch * c2.seqlen * c2.ngroups * c2.dstate * 2
    sums = nc * c2.batch * (c2.nheads // 4) * 128 * 4
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
