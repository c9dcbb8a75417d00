"""Benchmark of the Mamba-2 mixer core on one MI355X.

A step is one pass of the whole prefill hot path (dt = softplus(dt_raw +
dt_bias) and A = -exp(A_log), conv + SiLU over xBC, the chunked SSD scan,
the gated RMSNorm, the final conv and SSM states written out) over one batch
of synthetic input of the large-model layer shape: 1 x 8192 tokens, 256
heads x 64, 8 groups, state 128, conv width 4, chunk 256, bf16 I/O, zero
initial state, the input projection's packed rows [z | xBC | dt_raw]
already resident in HBM. Two input/output buffer sets alternate across
steps (each set, 0.85 GB, is larger than the 256 MB Infinity Cache).

Also measured (reported under "workloads"): the same layer from separate
x | B | C, z, dt tensors, the same layer with a conv bias (the fused kernels
then carry the state split), a serving-style mixed batch (ragged prefills and
decode steps over a state pool in one call), the tiny-model layer prefill
(4 x 2048 tokens, 32 heads), the long-context chained prefill (16 pieces of
8192 tokens, each resuming from the previous piece's states, per piece and
per chain), the decode loop (256 sequences x 64 single-token steps, 256
heads), the tiny fp32 layer and a bf16 shape outside the fused kernels'
envelope (both on the general kernels), and the backward pass of the
large-model layer prefill (every gradient, fp32 MFMA); under "ceilings": a streaming copy
and an MFMA-only loop on this GPU; under "cpu_baseline": the fp64 oracle on
the host cores.

Prints one JSON line. Only one GPU is used: --gpus above 1 exits.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
MFMA_F16_PEAK_TFS = 2500.0   # dense fp16 / bf16 MFMA, TFLOP/s
MFMA_F32_PEAK_TFS = 157.3    # dense fp32 MFMA, TFLOP/s

KERNEL_NAMES = ("conv1d_silu", "conv_state", "gated_rmsnorm", "decode_step", "chunk_state",
                "state_pass", "chunk_out", "fused_chunk_state", "fused_state_pass",
                "fused_chunk_out_norm", "bwd_gated_norm", "bwd_chunk_z", "bwd_rev_pass",
                "bwd_chunk", "bwd_group_sum", "bwd_conv_du", "bwd_conv_dx", "bwd_y",
                "chunk_cb")
DOMINANT = "fused_chunk_out_norm"
FUSED = ("fused_chunk_state", "fused_state_pass", "fused_chunk_out_norm")
# Counter-measured HBM bytes per launch (rocprofv3 FETCH_SIZE / WRITE_SIZE,
# scaled by a copy of known size), kept with the hash of the kernel sources
# they were taken on.
TRAFFIC_FILE = "{kernel}.large_layer_prefill.traffic.txt"
KERNEL_SOURCES = ("mamba_ssd_selective_mixer_amd/csrc/scan_fast.hip",
                  "mamba_ssd_selective_mixer_amd/csrc/common.hpp")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(kernel: str):
    """HBM bytes per launch of `kernel` on the large-model layer from the
    counter summary under profiles/, or None when there is none or the kernel
    sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", TRAFFIC_FILE.format(kernel=kernel))
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    if fields.get("kernel_source_sha256") != kernel_source_hash():
        return None
    try:
        return int(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--quick", action="store_true", help="headline workload only")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--sets", type=int, default=2, help="alternating input/output buffer sets")
    ap.add_argument("--no-kernel-events", action="store_true",
                    help="time the steps without the per-kernel HIP events")
    ap.add_argument("--only", choices=("tiny", "chain", "decode", "general", "serving", "backward",
                                       "unpacked", "bias"),
                    help="time only one of the secondary workloads (for profiling)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 512 MiB device copy (for the HBM counter scale)")
    return ap.parse_args()


# ------------------------------------------------------------ byte / flop counts
def token_bytes(cfg):
    """Algorithmic bytes per token of a prefill call: xBC, z, dt read once and
    the output written once."""
    e = 2 if cfg.dtype == "bf16" else 4
    return e * (cfg.channels + 2 * cfg.hp + cfg.nheads)


def state_bytes(cfg):
    """One sequence's SSM state (fp32) and conv state (I/O dtype)."""
    e = 2 if cfg.dtype == "bf16" else 4
    return cfg.hp * cfg.dstate * 4 + (cfg.conv_width - 1) * cfg.channels * e


def prefill_bytes(cfg, states_in, states_out):
    b = token_bytes(cfg) * cfg.batch * cfg.seqlen
    return b + cfg.batch * state_bytes(cfg) * (int(states_in) + int(states_out))


def prefill_flops(cfg):
    """Dense contractions of the chunked scan at the configuration's chunk
    length (causal half of the Q x Q products): C B^T per group, the masked
    (C B^T) X, C S_in^T and B^T X per head."""
    Q = cfg.chunk
    tok = cfg.batch * cfg.seqlen
    per_tok_group = Q * cfg.dstate
    per_tok_head = Q * cfg.headdim + 2 * cfg.headdim * cfg.dstate * 2
    return tok * (cfg.ngroups * per_tok_group + cfg.nheads * per_tok_head)


def decode_bytes(cfg):
    e = 2
    B = cfg.batch
    return (8 * B * cfg.hp * cfg.dstate + 2 * e * B * (cfg.conv_width - 1) * cfg.channels
            + e * B * (cfg.channels + 2 * cfg.hp + cfg.nheads))


# ------------------------------------------------------------------ timing
class Timer:
    """HIP events on the stream the library launches on (torch's current
    stream, which the binding passes to every call)."""

    def __init__(self, torch):
        self.torch = torch
        self.s = torch.cuda.Event(enable_timing=True)
        self.e = torch.cuda.Event(enable_timing=True)

    def start(self):
        self.s.record(self.torch.cuda.current_stream())

    def stop_ms(self):
        self.e.record(self.torch.cuda.current_stream())
        self.e.synchronize()
        return self.s.elapsed_time(self.e)


def to_dev(torch, a, dt):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda", dt)


def kernel_times(ops, run, steps, launches_per_step=8, only=None):
    """{kernel: mean ms per launch} from the library's per-kernel HIP events
    (recorded on the stream each kernel runs on) over `steps` calls of run().
    only: time just these kernels (the others launch with no events around
    them, so the stream keeps its ordinary spacing)."""
    ops.profile_only(only)
    ops.profile_start(launches_per_step * steps)
    for i in range(steps):
        run(i)
    ops.profile_stop()
    ops.profile_only(None)
    out = {}
    for name in KERNEL_NAMES:
        n, t = ops.profile_read(name)
        if n:
            out[name] = t / n
    return out


def prefill_workload(torch, ops, synth, cfg, steps, warmup, nsets, states_in, states_out,
                     kernel_events=True, packed=False, breakdown=True, bias=False):
    """Mean ms per prefill call over `steps` timed calls (HIP events around the
    whole timed region), and the output kernel's mean ms over the same calls
    (only that kernel is bracketed by the library's events, on its own
    stream; the other launches keep their ordinary spacing). With breakdown,
    the other kernels' mean ms from a second pass in which every launch is
    bracketed. packed: the call takes the input projection's rows
    [z | xBC | dt_raw] with dt_bias and A_log (dt and A formed in the
    kernels). bias: the conv carries a bias (drawn as in the parity tests)."""
    td = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    prm = (synth.packed_params(cfg, with_bias=bias) if packed
           else synth.layer_params(cfg, with_bias=bias))
    d = ops.SSDDims(cfg.batch, cfg.seqlen, cfg.nheads, cfg.headdim, cfg.ngroups, cfg.dstate,
                    cfg.conv_width, cfg.chunk, td)
    D = to_dev(torch, prm["D"], torch.float32)
    if packed:
        dtb = to_dev(torch, prm["dt_bias"], torch.float32)
        alog = to_dev(torch, prm["A_log"], torch.float32)
    else:
        A = to_dev(torch, prm["A"], torch.float32)
    cw, nw = to_dev(torch, prm["conv_w"], td), to_dev(torch, prm["norm_w"], td)
    cb = to_dev(torch, prm["conv_b"], td) if bias else None
    base = {"row": synth.packed_prefill_inputs(cfg)} if packed else synth.prefill_inputs(cfg)
    st0 = synth.initial_states(cfg) if states_in else None
    sets = []
    for _ in range(nsets):
        s = {k: to_dev(torch, v, td) for k, v in base.items()}
        s["out"] = torch.empty(cfg.batch, cfg.seqlen, cfg.hp, dtype=td, device="cuda")
        if states_in:
            s["cs_in"] = to_dev(torch, st0["conv_state"], td)
            s["ss_in"] = to_dev(torch, st0["ssm_state"], torch.float32)
        if states_out:
            s["cs_out"] = torch.empty(cfg.batch, cfg.conv_width - 1, cfg.channels, dtype=td,
                                      device="cuda")
            s["ss_out"] = torch.empty(cfg.batch, cfg.nheads, cfg.headdim, cfg.dstate,
                                      device="cuda")
        sets.append(s)
    ws = ops.workspace(ops.ssd_mixer_prefill_workspace_bytes(d))

    def step(i):
        s = sets[i % nsets]
        if packed:
            ops.ssd_mixer_prefill_packed(d, s["row"], dtb, alog, D, cw, cb, nw, prm["eps"],
                                         s.get("cs_in"), s.get("cs_out"), s.get("ss_in"),
                                         s.get("ss_out"), s["out"], ws)
        else:
            ops.ssd_mixer_prefill(d, s["xbc"], s["z"], s["dt"], A, D, cw, cb, nw, prm["eps"],
                                  s.get("cs_in"), s.get("cs_out"), s.get("ss_in"),
                                  s.get("ss_out"), s["out"], ws)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    # the output kernel (fused or general, whichever the shape runs) is
    # bracketed by events inside the timed steps themselves
    out_ks = [DOMINANT, "chunk_out"]
    if kernel_events:
        ops.profile_only(out_ks)
        ops.profile_start(2 * steps)
    tm = Timer(torch)
    tm.start()
    for i in range(steps):
        step(i)
    ms = tm.stop_ms() / steps
    torch.cuda.synchronize()
    kern = {}
    if kernel_events:
        ops.profile_stop()
        ops.profile_only(None)
        for name in out_ks:
            n, t = ops.profile_read(name)
            if n:
                kern[name] = t / n
        if breakdown:
            for k, v in kernel_times(ops, step, steps).items():
                kern.setdefault(k, v)
    status = ops.ssd_workspace_status(ws)
    del sets, ws
    torch.cuda.empty_cache()
    return ms, kern, status


def summarize_prefill(cfg, ms, kern, states_in, states_out):
    tokens = cfg.batch * cfg.seqlen
    nb = prefill_bytes(cfg, states_in, states_out)
    kb = token_bytes(cfg) * tokens
    r = {"tokens_per_s": tokens / (ms * 1e-3), "us_per_call": ms * 1e3,
         "algorithmic_bytes": nb, "hbm_frac": nb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
         "mfma_frac": prefill_flops(cfg) / (ms * 1e-3) / 1e12 / MFMA_F16_PEAK_TFS,
         "kernels_us": {k: v * 1e3 for k, v in kern.items()}}
    out_k = DOMINANT if DOMINANT in kern else ("chunk_out" if "chunk_out" in kern else None)
    if out_k:
        r["dominant_kernel"] = out_k
        r["dominant_kernel_bytes"] = kb
        r["dominant_kernel_hbm_frac"] = kb / (kern[out_k] * 1e-3) / 1e9 / HBM_PEAK_GBS
    return r


def run_chain(torch, ops, synth, cfg, reps, kernel_events=True):
    """Long-context prefill: cfg.pieces pieces chained through conv/SSM state
    (each call reads the previous piece's states and writes its own)."""
    bf = torch.bfloat16
    prm = synth.layer_params(cfg)
    d = ops.SSDDims(cfg.batch, cfg.seqlen, cfg.nheads, cfg.headdim, cfg.ngroups, cfg.dstate,
                    cfg.conv_width, cfg.chunk, bf)
    A, D = to_dev(torch, prm["A"], torch.float32), to_dev(torch, prm["D"], torch.float32)
    cw, nw = to_dev(torch, prm["conv_w"], bf), to_dev(torch, prm["norm_w"], bf)
    pieces = []
    for k in range(cfg.pieces):
        p = synth.prefill_inputs(cfg, piece=k)
        pieces.append({kk: to_dev(torch, v, bf) for kk, v in p.items()})
    out = torch.empty(cfg.batch, cfg.seqlen, cfg.hp, dtype=bf, device="cuda")
    cs = torch.zeros(cfg.batch, cfg.conv_width - 1, cfg.channels, dtype=bf, device="cuda")
    ss = torch.zeros(cfg.batch, cfg.nheads, cfg.headdim, cfg.dstate, device="cuda")
    ws = ops.workspace(ops.ssd_mixer_prefill_workspace_bytes(d))

    def piece(i):
        p = pieces[i % cfg.pieces]
        ops.ssd_mixer_prefill(d, p["xbc"], p["z"], p["dt"], A, D, cw, None, nw, prm["eps"],
                              cs, cs, ss, ss, out, ws)

    def chain():
        cs.zero_()
        ss.zero_()
        for i in range(cfg.pieces):
            piece(i)

    chain()
    torch.cuda.synchronize()
    tm = Timer(torch)
    tm.start()
    for _ in range(reps):
        chain()
    ms = tm.stop_ms() / reps
    kern = kernel_times(ops, piece, cfg.pieces) if kernel_events else {}
    return ms, kern


def run_decode(torch, ops, synth, cfg, reps, kernel_events=True):
    bf = torch.bfloat16
    prm = synth.layer_params(cfg)
    d = ops.SSDDims(cfg.batch, 1, cfg.nheads, cfg.headdim, cfg.ngroups, cfg.dstate,
                    cfg.conv_width, 128, bf)
    A, D = to_dev(torch, prm["A"], torch.float32), to_dev(torch, prm["D"], torch.float32)
    cw, nw = to_dev(torch, prm["conv_w"], bf), to_dev(torch, prm["norm_w"], bf)
    st = synth.initial_states(cfg)
    cs = to_dev(torch, st["conv_state"], bf)
    ss = to_dev(torch, st["ssm_state"], torch.float32)
    steps = []
    for k in range(cfg.steps):
        t = synth.decode_inputs(cfg, k)
        steps.append({kk: to_dev(torch, v, bf) for kk, v in t.items()})
    y = torch.empty(cfg.batch, cfg.hp, dtype=bf, device="cuda")

    def one(i):
        t = steps[i % cfg.steps]
        ops.ssd_decode_step(d, t["xbc_t"], t["z_t"], t["dt_t"], A, D, cw, None, nw, prm["eps"],
                            cs, ss, y)

    def loop():
        for i in range(cfg.steps):
            one(i)

    loop()
    torch.cuda.synchronize()
    tm = Timer(torch)
    tm.start()
    for _ in range(reps):
        loop()
    ms = tm.stop_ms() / reps  # per 64-step loop
    kern = kernel_times(ops, one, cfg.steps, 2) if kernel_events else {}
    return ms, kern


def run_serving(torch, ops, synth, reps, kernel_events=True):
    """Continuous batching on the large-model layer (256 heads x 64, 8 groups,
    state 128) over a pool of 512 state slots: one call takes 16 fresh
    prefills (lengths drawn from 64..1024 tokens) and 240 decode steps (one
    token each, resuming from their slots), every sequence on its own slot."""
    bf = torch.bfloat16
    cfg = synth.replace(synth.CONFIGS["large_layer"], chunk=128)
    r = np.random.default_rng(2024)
    lens = np.concatenate([r.integers(64, 1025, 16), np.ones(240, dtype=np.int64)])
    T, nseq, S = int(lens.sum()), len(lens), 512
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    slots = r.permutation(S)[:nseq].astype(np.int32)
    has = np.concatenate([np.zeros(16), np.ones(240)]).astype(np.uint8)
    prm = synth.layer_params(cfg)
    inp = synth.prefill_inputs(cfg, batch=1, seqlen=T)
    d = ops.SSDDims(nseq, T, cfg.nheads, cfg.headdim, cfg.ngroups, cfg.dstate, 4, 128, bf)
    cpool = torch.zeros(S, 3, cfg.channels, dtype=bf, device="cuda")
    spool = torch.zeros(S, cfg.nheads, cfg.headdim, cfg.dstate, device="cuda")
    spool.normal_(0.0, 0.1 ** 0.5)
    args = (torch.tensor(cu, device="cuda"), torch.tensor(slots, device="cuda"),
            to_dev(torch, inp["xbc"][0], bf), to_dev(torch, inp["z"][0], bf),
            to_dev(torch, inp["dt"][0], bf), to_dev(torch, prm["A"], torch.float32),
            to_dev(torch, prm["D"], torch.float32), to_dev(torch, prm["conv_w"], bf), None,
            to_dev(torch, prm["norm_w"], bf), cpool, spool)
    hs = torch.tensor(has, device="cuda")
    out = torch.empty(T, cfg.hp, dtype=bf, device="cuda")
    ws = ops.workspace(ops.ssd_mixer_varlen_workspace_bytes(d, S))

    def one(_i=0):
        ops.ssd_mixer_varlen(d, *args, eps=prm["eps"], has_state=hs, out=out, ws=ws)

    one()
    torch.cuda.synchronize()
    tm = Timer(torch)
    tm.start()
    for _ in range(reps):
        one()
    ms = tm.stop_ms() / reps
    kern = kernel_times(ops, one, reps) if kernel_events else {}
    status = ops.ssd_workspace_status(ws)
    # algorithmic bytes: every token's inputs and output, each sequence's
    # final states written, the decode steps' states read
    nb = token_bytes(cfg) * T + state_bytes(cfg) * (nseq + int(has.sum()))
    del cpool, spool, ws
    torch.cuda.empty_cache()
    return {"tokens_per_s": T / (ms * 1e-3), "us_per_call": ms * 1e3,
            "algorithmic_bytes": nb, "hbm_frac": nb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "kernels_us": {k: v * 1e3 for k, v in kern.items()}, "status": status,
            "config": f"one call: 16 prefills ({int(lens[:16].sum())} tokens, 64-1024 each, "
                      f"fresh) + 240 decode steps on a 512-slot pool, 256 heads x 64, 8 groups, "
                      f"state 128, bf16"}


BWD_CHUNK = 64  # chunk length of the backward kernels


def backward_flops(cfg):
    """Algorithmic fp32 MFMA FLOPs per launch of the backward's matrix
    kernels (causal products counted over their lower half): C B^T once per
    chunk and group, the y recompute (M X, C S_in^T), the state-gradient
    terms (Z) and the per-chunk gradients (dY X^T, dX's two terms, dC's and
    dB's two terms each)."""
    Q, P, N = BWD_CHUNK, cfg.headdim, cfg.dstate
    nc = -(-cfg.seqlen // Q)
    units = cfg.batch * cfg.nheads * nc
    tri = Q * Q / 2
    return {"chunk_cb": 2 * cfg.batch * cfg.ngroups * nc * tri * N,
            "bwd_y": 2 * units * (tri * P + Q * N * P),
            "bwd_chunk_z": 2 * units * Q * P * N,
            "bwd_chunk": 2 * units * (tri * (2 * P + 2 * N) + 3 * Q * P * N)}


def run_backward(torch, ops, synth, reps, kernel_events=True):
    """Backward pass of the large-model layer prefill (the headline layer:
    1 x 8192 tokens, 256 heads x 64, 8 groups, state 128, bf16 I/O): every
    gradient (xBC, z, dt, A, D, conv weight, norm weight) for a seeded
    upstream gradient, the forward recomputed inside the call."""
    bf = torch.bfloat16
    cfg = synth.CONFIGS["large_layer"]
    prm = synth.layer_params(cfg)
    inp = synth.prefill_inputs(cfg)
    seeds = synth.backward_seeds(cfg)
    d = ops.SSDDims(cfg.batch, cfg.seqlen, cfg.nheads, cfg.headdim, cfg.ngroups, cfg.dstate,
                    cfg.conv_width, cfg.chunk, bf)
    args = [to_dev(torch, inp["xbc"], bf), to_dev(torch, inp["z"], bf),
            to_dev(torch, inp["dt"], bf), to_dev(torch, prm["A"], torch.float32),
            to_dev(torch, prm["D"], torch.float32), to_dev(torch, prm["conv_w"], bf), None,
            to_dev(torch, seeds["norm_w"], bf), to_dev(torch, seeds["d_out"], bf)]
    ws = ops.workspace(ops.ssd_mixer_backward_workspace_bytes(d))
    grads = ops.ssd_mixer_backward(d, *args, eps=prm["eps"], ws=ws)

    def one(_i=0):
        ops.ssd_mixer_backward(d, *args, eps=prm["eps"], grads=grads, ws=ws)

    one()
    torch.cuda.synchronize()
    tm = Timer(torch)
    tm.start()
    for _ in range(reps):
        one()
    ms = tm.stop_ms() / reps
    kern = kernel_times(ops, one, reps, launches_per_step=20) if kernel_events else {}
    status = ops.ssd_workspace_status(ws)
    T = cfg.batch * cfg.seqlen
    # algorithmic bytes: xBC, z, dt and d_out read; d_xBC, d_z, d_dt written
    nb = 2 * T * (2 * cfg.channels + 2 * cfg.hp + 2 * cfg.nheads)
    fl = backward_flops(cfg)
    mats = {}
    for k, f in fl.items():
        if k in kern:
            tf = f / (kern[k] * 1e-3) / 1e12
            mats[k] = {"flops_per_launch": f, "us": kern[k] * 1e3, "tflops": tf,
                       "mfma_f32_frac": tf / MFMA_F32_PEAK_TFS}
    del grads, ws, args
    torch.cuda.empty_cache()
    return {"tokens_per_s": T / (ms * 1e-3), "ms_per_call": ms,
            "algorithmic_bytes": nb, "hbm_frac": nb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "roofline": ({"bound": "mfma", "kernel": "bwd_chunk", "dtype": "f32",
                          "achieved": mats["bwd_chunk"]["tflops"], "peak": MFMA_F32_PEAK_TFS,
                          "unit": "TFLOP/s", "frac": mats["bwd_chunk"]["mfma_f32_frac"]}
                         if "bwd_chunk" in mats else None),
            "matrix_kernels": mats,
            "kernels_us": {k: v * 1e3 for k, v in kern.items()}, "status": status,
            "config": "backward of the headline layer prefill: 1 x 8192 tokens, 256 heads x 64, "
                      "8 groups, state 128, conv width 4, bf16 I/O, no conv bias, zero initial "
                      "states; d_out ~ N(0,1), norm weight 1 + N(0,1)/4; gradients of xBC, z, dt "
                      "(bf16) and A, D, conv weight, norm weight (fp32); fp32 MFMA, 64-token "
                      "chunks, forward recomputed in the call"}


def ceilings(torch):
    """A streaming 2 GiB device copy and an MFMA-only loop on this GPU."""
    from mamba_ssd_selective_mixer_amd import build as hb
    lib = ctypes.CDLL(hb.CEIL_LIB)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.ceil_copy.argtypes = [vp, vp, i64, i32, vp]
    lib.ceil_mfma.argtypes = [vp, i32, i32, vp]
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    n = 2 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    dst = torch.empty_like(src)
    blocks = 256 * 8
    tm = Timer(torch)
    for _ in range(2):
        assert lib.ceil_copy(vp(src.data_ptr()), vp(dst.data_ptr()), n, blocks, st) == 0
    tm.start()
    reps = 5
    for _ in range(reps):
        assert lib.ceil_copy(vp(src.data_ptr()), vp(dst.data_ptr()), n, blocks, st) == 0
    copy_ms = tm.stop_ms() / reps
    del src, dst
    out = torch.empty(2048 * 256, dtype=torch.float32, device="cuda")
    iters = 2000
    assert lib.ceil_mfma(vp(out.data_ptr()), 2048, 50, st) == 0
    tm.start()
    assert lib.ceil_mfma(vp(out.data_ptr()), 2048, iters, st) == 0
    mfma_ms = tm.stop_ms()
    flops = 2048 * 4 * iters * 8 * 2 * 16 * 16 * 32
    torch.cuda.empty_cache()
    return {"copy_gbs": 2 * n / (copy_ms * 1e-3) / 1e9,
            "copy_desc": "2 GiB device-to-device copy, 16-byte non-temporal loads and stores, "
                         "2048 workgroups of 256 threads (GB/s counts bytes read + written)",
            "mfma_f16_tflops": flops / (mfma_ms * 1e-3) / 1e12,
            "mfma_desc": "fp16 16x16x32 MFMA only, 8 independent chains per wave, "
                         "2048 workgroups of 256 threads"}


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(synth, cfg, budget_s=12.0, one_thread_tokens=1024):
    """The fp64 oracle on the headline workload on the host cores: full
    steps (all 8192 tokens, all heads) repeated until about budget_s of wall
    time on all threads, then one thread on the first one_thread_tokens
    tokens of the same step."""
    from oracle import oracle
    prm = synth.layer_params(cfg)
    inp = synth.prefill_inputs(cfg)

    def one(x, z, dt):
        oracle.mixer_prefill(x, z, dt, prm["A"], prm["D"], prm["conv_w"], None, prm["norm_w"],
                             prm["eps"], cfg.nheads, cfg.headdim, cfg.ngroups, cfg.dstate)

    threads = oracle.num_threads()
    reps, sec = 0, 0.0
    while sec < budget_s and reps < 50:
        t = time.perf_counter()
        one(inp["xbc"], inp["z"], inp["dt"])
        sec += time.perf_counter() - t
        reps += 1
    tokens = cfg.batch * cfg.seqlen * reps
    n1 = one_thread_tokens
    oracle.set_num_threads(1)
    try:
        t = time.perf_counter()
        one(inp["xbc"][:, :n1], inp["z"][:, :n1], inp["dt"][:, :n1])
        sec1 = time.perf_counter() - t
    finally:
        oracle.set_num_threads(threads)
    return {"value": tokens / sec, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"{reps} full step(s) of {cfg.batch} x {cfg.seqlen} tokens of the "
                      f"large-model layer (fp64 sequential recurrence, explicit conv and gated "
                      f"norm), {sec:.1f} s wall on {threads} threads",
            "one_thread": {"value": cfg.batch * n1 / sec1, "unit": "tokens/s", "cores": 1,
                           "sample": f"the first {n1} tokens of the same step, {sec1:.1f} s"}}


def secondary(torch, ops, synth, args, which):
    wl = {}
    ke = not args.no_kernel_events
    if "tiny" in which:
        tiny_cfg = synth.CONFIGS["tiny_layer"]
        ms, kern, rc = prefill_workload(torch, ops, synth, tiny_cfg, max(10, args.steps), 3, 4, False,
                                        False, ke)
        wl["tiny_layer_prefill"] = dict(summarize_prefill(tiny_cfg, ms, kern, False, False), status=rc,
                                        config="4 x 2048 tokens, 32 heads x 64, 8 groups, state "
                                               "128, chunk 128, bf16, no states")
    if "chain" in which:
        chain_cfg = synth.CONFIGS["long_context"]
        ms, kern = run_chain(torch, ops, synth, chain_cfg, 3, ke)
        tokens = chain_cfg.seqlen * chain_cfg.pieces
        nb = prefill_bytes(chain_cfg, True, True) * chain_cfg.pieces
        wl["long_context_chain"] = {
            "tokens_per_s": tokens / (ms * 1e-3), "ms_per_chain": ms,
            "us_per_piece": ms * 1e3 / chain_cfg.pieces,
            "algorithmic_bytes_per_piece": nb // chain_cfg.pieces,
            "hbm_frac": nb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "kernels_us": {k: v * 1e3 for k, v in kern.items()},
            "config": "16 pieces of 1 x 8192 tokens, 32 heads x 64, 8 groups, state 128, "
                      "each resuming from the previous piece's conv and SSM state"}
    if "decode" in which:
        dec_cfg = synth.CONFIGS["decode_loop"]
        ms, kern = run_decode(torch, ops, synth, dec_cfg, 3, ke)
        dec_bytes = decode_bytes(dec_cfg) * dec_cfg.steps
        wl["decode"] = {"tokens_per_s": dec_cfg.batch * dec_cfg.steps / (ms * 1e-3),
                        "us_per_step": ms * 1e3 / dec_cfg.steps,
                        "algorithmic_bytes_per_step": decode_bytes(dec_cfg),
                        "hbm_gbs": dec_bytes / (ms * 1e-3) / 1e9,
                        "hbm_frac": dec_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                        "kernels_us": {k: v * 1e3 for k, v in kern.items()},
                        "config": "256 sequences x 64 steps, 256 heads x 64, 8 groups, "
                                  "state 128, states ~ N(0, 0.1) updated in place"}
    if "serving" in which:
        wl["serving_mixed_batch"] = run_serving(torch, ops, synth, 5, ke)
    if "backward" in which:
        wl["large_layer_backward"] = run_backward(torch, ops, synth, 3, ke)
    if "unpacked" in which:
        large_cfg = synth.CONFIGS["large_layer"]
        ms, kern, rc = prefill_workload(torch, ops, synth, large_cfg, max(10, args.steps), 3, 2, False,
                                        True, ke)
        wl["large_layer_prefill_unpacked"] = dict(
            summarize_prefill(large_cfg, ms, kern, False, True), status=rc,
            config="the headline layer and inputs with x | B | C, z and dt (already softplus-ed) "
                   "as separate tensors and A given")
    if "bias" in which:
        large_cfg = synth.CONFIGS["large_layer"]
        ms, kern, rc = prefill_workload(torch, ops, synth, large_cfg, max(10, args.steps), 3, 2, False,
                                        True, ke, packed=True, bias=True)
        wl["large_layer_prefill_conv_bias"] = dict(
            summarize_prefill(large_cfg, ms, kern, False, True), status=rc,
            config="the headline layer and packed rows with a conv bias ~ N(0, 0.25): the "
                   "fused kernels carry the state split S' + a bbar^T")
    if "general" in which:
        fp32_cfg = synth.CONFIGS["tiny_fp32"]
        ms, kern, rc = prefill_workload(torch, ops, synth, fp32_cfg, 50, 5, 1, False, False, ke)
        wl["tiny_fp32_layer"] = dict(summarize_prefill(fp32_cfg, ms, kern, False, False), status=rc,
                                     config="1 x 256 tokens, 4 heads x 16, 1 group, state 16, "
                                            "chunk 64, fp32 (general kernels)")
        cg = synth.replace(synth.CONFIGS["tiny_layer"], dstate=64)
        ms, kern, rc = prefill_workload(torch, ops, synth, cg, 10, 3, 2, False, False, ke)
        wl["general_bf16_prefill"] = dict(summarize_prefill(cg, ms, kern, False, False),
                                          status=rc,
                                          config="4 x 2048 tokens, 32 heads x 64, 8 groups, "
                                                 "state 64, chunk 128, bf16 (general kernels)")
    return wl


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the path is built and "
              "timed on a single MI355X.", file=sys.stderr)
        sys.exit(2)
    import torch
    from mamba_ssd_selective_mixer_amd import ops, synth

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        n = 512 << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 5}))
        return
    if args.only:
        print(json.dumps(secondary(torch, ops, synth, args, (args.only,))), flush=True)
        return
    cfg = synth.CONFIGS["large_layer"]
    ms, kern, rc = prefill_workload(torch, ops, synth, cfg, args.steps, args.warmup, args.sets,
                                    False, True, not args.no_kernel_events, packed=True,
                                    breakdown=not args.quick)
    if rc != 0:
        print(f"prefill reported status {rc}", file=sys.stderr)
        sys.exit(1)
    head = summarize_prefill(cfg, ms, kern, False, True)
    tokens = cfg.batch * cfg.seqlen
    nbytes = head["algorithmic_bytes"]
    if DOMINANT in kern:
        # the output kernel reads every input of the step (xBC, z, dt) and
        # writes its output: its algorithmic bytes per launch are the step's
        # token bytes (the final states are written by the other kernels)
        kb, k_ms = head["dominant_kernel_bytes"], kern[DOMINANT]
        traffic = {k: measured_traffic(k) for k in FUSED}
        roof = {"bound": "hbm", "kernel": DOMINANT, "achieved": kb / (k_ms * 1e-3) / 1e9,
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": kb / (k_ms * 1e-3) / 1e9 /
                HBM_PEAK_GBS, "traffic": traffic[DOMINANT],
                "algorithmic_bytes_per_launch": kb, "kernel_us": k_ms * 1e3,
                "traffic_per_launch": traffic,
                "step_traffic_over_algorithmic": (sum(traffic.values()) / nbytes
                                                  if all(traffic.values()) else None),
                "step_frac": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                "step_mfma_frac": head["mfma_frac"]}
    else:
        roof = {"bound": "hbm", "kernel": "whole prefill step",
                "achieved": nbytes / (ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, "traffic": None}
    rec = {
        "metric": "Mamba-2 mixer tokens/sec (prefill, decode) on 1 MI355X; % HBM/MFMA roofline",
        "value": tokens / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "large-model layer prefill: batch 1 x 8192 tokens, 256 heads x "
                               "64, 8 groups, state 128, conv width 4, chunk 256, bf16 I/O, "
                               "zero initial state, final conv and SSM states written; inputs "
                               "as the projection's packed rows [z | xBC | dt_raw] with "
                               "dt_bias = -2 and A_log ~ U(log 1, log 16)",
                   "global_batch": cfg.batch, "seq_len": cfg.seqlen, "parallelism": "none"},
        "roofline": roof,
        "headline": head,
    }
    if not args.quick:
        rec["workloads"] = secondary(torch, ops, synth, args, ("unpacked", "bias", "tiny",
                                                               "chain", "decode", "serving",
                                                               "general", "backward"))
        rec["ceilings"] = ceilings(torch)
    if not args.no_cpu:
        rec["cpu_baseline"] = cpu_baseline(synth, cfg)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
