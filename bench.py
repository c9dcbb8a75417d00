"""Benchmark of the Mamba-2 mixer core on one MI355X.

A step is one pass of the whole prefill hot path (conv + SiLU over xBC, the
chunked SSD scan, the gated RMSNorm) over one batch of synthetic input of
the tiny-model layer shape (4 x 2048 tokens, 32 heads x 64, 8 groups,
state 128, conv width 4, chunk 128, bf16 I/O), inputs already resident in
HBM. Four input/output buffer sets rotate across steps so no step reads
inputs the previous one left in the 256 MB Infinity Cache.

Also measured (reported under "workloads"): the large-model layer prefill
(1 x 8192 tokens, 256 heads), the long-context chained prefill (16 pieces
of 8192 tokens, each resuming from the previous piece's states) and the
decode loop (256 sequences x 64 single-token steps, 256 heads).

Prints one JSON line. Only one GPU is used: --gpus above 1 exits.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0      # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFS = 2500.0  # dense bf16 / fp16 MFMA, TFLOP/s

KERNEL_NAMES = ("conv1d_silu", "conv_state", "gated_rmsnorm", "decode_step", "chunk_state",
                "state_pass", "chunk_out", "fused_chunk_state", "fused_state_pass",
                "fused_chunk_out_norm")
DOMINANT = "fused_chunk_out_norm"
# HBM bytes per launch of a kernel from rocprofv3 FETCH_SIZE / WRITE_SIZE
# counters, with the hash of the kernel sources they were taken on.
TRAFFIC_FILES = {"fused_chunk_out_norm": "fused_chunk_out_norm.tiny_layer_prefill.traffic.txt"}
KERNEL_SOURCES = ("mamba_ssd_selective_mixer_amd/csrc/scan_fast.hip",
                  "mamba_ssd_selective_mixer_amd/csrc/common.hpp")


def kernel_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(kernel: str):
    """Counter-measured HBM bytes per launch, or None when no measurement
    exists or the kernel sources changed since it was taken."""
    name = TRAFFIC_FILES.get(kernel)
    path = os.path.join(ROOT, "profiles", name) if name else None
    if not path or not os.path.exists(path):
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


def copy_calibration(torch):
    """A plain device-to-device copy of 512 MiB, run 5 times, so HBM counters
    can be scaled by what they read for a known number of bytes."""
    n = 512 << 20
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 5}))


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--quick", action="store_true", help="headline workload only")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--sets", type=int, default=4, help="rotating input/output buffer sets")
    ap.add_argument("--no-kernel-events", action="store_true",
                    help="time the steps without the per-kernel HIP events")
    ap.add_argument("--only", choices=("large", "chain", "decode"),
                    help="time only one of the secondary workloads (for profiling)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 512 MiB device copy (for the HBM counter scale)")
    return ap.parse_args()


def prefill_bytes(cfg, L, with_states):
    """Algorithmic HBM bytes of one prefill call: xBC, z, dt read once, out
    written once, plus the requested state I/O."""
    e = 2 if cfg.dtype == "bf16" else 4
    tok = cfg.batch * L
    b = e * tok * (cfg.channels + 2 * cfg.hp + cfg.nheads)
    if with_states:
        ssm = cfg.batch * cfg.hp * cfg.dstate * 4
        conv = cfg.batch * (cfg.conv_width - 1) * cfg.channels * e
        b += 2 * (ssm + conv)
    return b


def prefill_flops(cfg, L):
    """Dense contractions of the chunked scan (causal half of the Q x Q
    products): C B^T per group, (C B^T o decay) X, C S_in^T and B^T X per head."""
    Q = cfg.chunk
    tok = cfg.batch * L
    per_tok_group = Q * cfg.dstate          # causal half of 2*Q*N
    per_tok_head = Q * cfg.headdim + 2 * cfg.headdim * cfg.dstate * 2
    return tok * (cfg.ngroups * per_tok_group + cfg.nheads * per_tok_head)


def decode_bytes(cfg):
    e = 2
    B = cfg.batch
    return (8 * B * cfg.hp * cfg.dstate + 2 * e * B * (cfg.conv_width - 1) * cfg.channels
            + e * B * (cfg.channels + 2 * cfg.hp + cfg.nheads))


class Timer:
    """HIP events on the stream the library launches on."""

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


def run_prefill(torch, ops, synth, cfg, steps, warmup, nsets, with_states, kernel_events=False):
    """Mean ms per prefill call over `steps` timed calls; with kernel_events,
    also {kernel: (launches, mean ms)} from the library's per-kernel HIP
    events recorded over the same timed calls."""
    bf = torch.bfloat16
    prm = synth.layer_params(cfg)
    d = ops.SSDDims(cfg.batch, cfg.seqlen, cfg.nheads, cfg.headdim, cfg.ngroups, cfg.dstate,
                    cfg.conv_width, cfg.chunk, bf)
    A, D = to_dev(torch, prm["A"], torch.float32), to_dev(torch, prm["D"], torch.float32)
    cw, nw = to_dev(torch, prm["conv_w"], bf), to_dev(torch, prm["norm_w"], bf)
    base = synth.prefill_inputs(cfg)
    sets = []
    for i in range(nsets):
        # distinct buffers per set; contents of set 0 are the seeded inputs
        s = {k: to_dev(torch, v, bf) for k, v in base.items()}
        s["out"] = torch.empty(cfg.batch, cfg.seqlen, cfg.hp, dtype=bf, device="cuda")
        if with_states:
            s["cs"] = torch.zeros(cfg.batch, cfg.conv_width - 1, cfg.channels, dtype=bf, device="cuda")
            s["ss"] = torch.zeros(cfg.batch, cfg.nheads, cfg.headdim, cfg.dstate, device="cuda")
        sets.append(s)
    ws = ops.workspace(ops.ssd_mixer_prefill_workspace_bytes(d))

    def step(i):
        s = sets[i % nsets]
        ops.ssd_mixer_prefill(d, s["xbc"], s["z"], s["dt"], A, D, cw, None, nw, prm["eps"],
                              s.get("cs"), s.get("cs"), s.get("ss"), s.get("ss"), s["out"], ws)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    tm = Timer(torch)
    tm.start()
    for i in range(steps):
        step(i)
    ms = tm.stop_ms() / steps
    torch.cuda.synchronize()
    kern = {}
    if kernel_events:
        # The same timed steps again, each kernel launch bracketed by a pair of
        # HIP events on its stream. The events add gaps between launches (not
        # to the kernels), so the step time above comes from the first pass.
        ops.profile_start(8 * steps)
        tm.start()
        for i in range(steps):
            step(i)
        kern["_step_ms"] = tm.stop_ms() / steps
        torch.cuda.synchronize()
        ops.profile_stop()
        for name in KERNEL_NAMES:
            n, t = ops.profile_read(name)
            if n:
                kern[name] = (n, t / n)
    return ms, kern


def run_chain(torch, ops, synth, cfg, reps, nsets_unused=None):
    """Long-context prefill: cfg.pieces pieces chained through conv/SSM state."""
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

    def chain():
        cs.zero_()
        ss.zero_()
        for p in pieces:
            ops.ssd_mixer_prefill(d, p["xbc"], p["z"], p["dt"], A, D, cw, None, nw, prm["eps"],
                                  cs, cs, ss, ss, out, ws)

    chain()
    torch.cuda.synchronize()
    tm = Timer(torch)
    tm.start()
    for _ in range(reps):
        chain()
    ms = tm.stop_ms()
    return ms / reps


def run_decode(torch, ops, synth, cfg, reps):
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

    def loop():
        for t in steps:
            ops.ssd_decode_step(d, t["xbc_t"], t["z_t"], t["dt_t"], A, D, cw, None, nw,
                                prm["eps"], cs, ss, y)

    loop()
    torch.cuda.synchronize()
    tm = Timer(torch)
    tm.start()
    for _ in range(reps):
        loop()
    ms = tm.stop_ms()
    return ms / reps  # per 64-step loop


def cpu_baseline(synth, cfg, budget_s=10.0):
    """The fp64 oracle on full steps of the headline workload on the host
    cores, repeated until about `budget_s` seconds of wall time are spent."""
    from oracle import oracle
    prm = synth.layer_params(cfg)
    inp = synth.prefill_inputs(cfg)
    reps, sec = 0, 0.0
    while sec < budget_s and reps < 100:
        t = time.perf_counter()
        oracle.mixer_prefill(inp["xbc"], inp["z"], inp["dt"], prm["A"], prm["D"], prm["conv_w"],
                             None, prm["norm_w"], prm["eps"], cfg.nheads, cfg.headdim,
                             cfg.ngroups, cfg.dstate)
        sec += time.perf_counter() - t
        reps += 1
    tokens = cfg.batch * cfg.seqlen * reps
    return {"value": tokens / sec, "unit": "tokens/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"{reps} full step(s) of {cfg.batch}x{cfg.seqlen} tokens (fp64 sequential "
                      f"recurrence + conv + gated norm), {sec:.1f} s wall"}


def secondary(torch, ops, synth, args, which):
    """The large-layer prefill, the long-context chain and the decode loop."""
    wl = {}
    if "large" in which:
        c2 = synth.CONFIGS["c2"]
        ms2, _ = run_prefill(torch, ops, synth, c2, max(3, args.steps // 5), 2, 2, True)
        b2 = prefill_bytes(c2, c2.seqlen, True)
        wl["large_prefill"] = {"tokens_per_s": c2.seqlen / (ms2 * 1e-3), "ms": ms2,
                               "hbm_frac": b2 / (ms2 * 1e-3) / 1e9 / HBM_PEAK_GBS,
                               "mfma_frac": prefill_flops(c2, c2.seqlen) / (ms2 * 1e-3) / 1e12
                               / MFMA_BF16_PEAK_TFS}
    if "chain" in which:
        c3 = synth.CONFIGS["c3"]
        ms3 = run_chain(torch, ops, synth, c3, 3)
        b3 = prefill_bytes(c3, c3.seqlen, True) * c3.pieces
        wl["long_context_chain"] = {"tokens_per_s": c3.seqlen * c3.pieces / (ms3 * 1e-3),
                                    "ms_per_chain": ms3,
                                    "hbm_frac": b3 / (ms3 * 1e-3) / 1e9 / HBM_PEAK_GBS}
    if "decode" in which:
        c4 = synth.CONFIGS["c4"]
        ms4 = run_decode(torch, ops, synth, c4, 3)
        b4 = decode_bytes(c4) * c4.steps
        wl["decode"] = {"tokens_per_s": c4.batch * c4.steps / (ms4 * 1e-3),
                        "us_per_step": ms4 * 1e3 / c4.steps,
                        "hbm_gbs": b4 / (ms4 * 1e-3) / 1e9,
                        "hbm_frac": b4 / (ms4 * 1e-3) / 1e9 / HBM_PEAK_GBS}
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
        copy_calibration(torch)
        return
    if args.only:
        print(json.dumps(secondary(torch, ops, synth, args, (args.only,))))
        return
    cfg = synth.CONFIGS["c1"]
    ms, kern = run_prefill(torch, ops, synth, cfg, args.steps, args.warmup, args.sets, False,
                           kernel_events=not args.no_kernel_events)
    tokens = cfg.batch * cfg.seqlen
    nbytes = prefill_bytes(cfg, cfg.seqlen, False)
    # the dominant kernel: chunk output + fused gated norm. It reads every
    # input of the step (xBC, z, dt) and writes the output, so its
    # algorithmic bytes per launch are the step's.
    if DOMINANT in kern:
        k_ms = kern[DOMINANT][1]
        roof = {"bound": "hbm", "kernel": DOMINANT, "achieved": nbytes / (k_ms * 1e-3) / 1e9,
                "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": nbytes / (k_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                "traffic": measured_traffic(DOMINANT), "algorithmic_bytes": nbytes,
                "kernel_us": k_ms * 1e3,
                "kernels_us": {k: v[1] * 1e3 for k, v in kern.items() if k != "_step_ms"},
                "events_pass_ms_per_step": kern["_step_ms"],
                "step_frac": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                "step_mfma_tflops": prefill_flops(cfg, cfg.seqlen) / (ms * 1e-3) / 1e12}
    else:
        roof = {"bound": "hbm", "kernel": "whole prefill step", "achieved":
                nbytes / (ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, "traffic": None,
                "algorithmic_bytes": nbytes}
    rec = {
        "metric": "Mamba-2 mixer tokens/sec (prefill, decode) on 1 MI355X; % HBM/MFMA roofline",
        "value": tokens / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "tiny-model layer prefill: batch 4 x 2048 tokens, 32 heads x 64, "
                               "8 groups, state 128, conv width 4, chunk 128",
                   "global_batch": cfg.batch, "seq_len": cfg.seqlen, "parallelism": "none"},
        "roofline": roof,
    }
    if not args.quick:
        rec["workloads"] = secondary(torch, ops, synth, args, ("large", "chain", "decode"))
    if not args.no_cpu:
        rec["cpu_baseline"] = cpu_baseline(synth, cfg)
    print(json.dumps(rec))


if __name__ == "__main__":
    main()
