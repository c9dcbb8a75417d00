"""Seeded synthetic inputs shaped like the pages' Mamba-2 layer sizes.

This module holds only random-number recipes and dtype rounding; none of the
mixer's arithmetic. It is the one piece shared by the HIP path's tests and
benchmark and by the fp64 oracle: both sides receive the same arrays.

Recipe (every draw from numpy ``Generator(PCG64(SeedSequence([1000 + cfg,
stream])))``; fp32, then round-to-nearest-even to the I/O dtype):
  x [B,L,H,P] ~ N(0,1); B, C [B,L,G,N] ~ N(0,1)/sqrt(N); z [B,L,H*P] ~ N(0,1);
  dt [B,L,H] = softplus(N(0,1) - 2) (computed in fp64);
  A [H] = -exp(U(log 1, log 16)) fp32; D [H] ~ N(0,1) fp32;
  conv w [Cch, W] ~ N(0, variance 1/4); no conv bias; norm w = 1; eps 1e-5.
The conv input per token is xBC = [x | B | C]. Stream 0 holds the layer
parameters; prefill tokens use stream 1 (long prefills split in pieces use
stream 1 + piece); decode step k uses stream 1 + k; initial states use
stream 100 with N(0, variance 0.1).

Layer shapes follow the NemotronH-0.3B-A0.3B card ("Configuration Changes":
mamba_num_heads 256 / 32, mamba_head_dim 64, n_groups 8) and the Modalities
PR #459 Nano-width run (64 Mamba-2 heads of dim 64).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np


@dataclasses.dataclass(frozen=True)
class Cfg:
    name: str
    index: int
    batch: int
    seqlen: int          # tokens per call (per piece for the chained prefill)
    nheads: int
    headdim: int
    ngroups: int
    dstate: int
    conv_width: int
    chunk: int
    dtype: str           # "f32" | "bf16"
    pieces: int = 1      # chained prefill pieces (each resumes from state)
    steps: int = 0       # decode steps (decode workload only)
    nonzero_init: bool = False

    @property
    def hp(self):
        return self.nheads * self.headdim

    @property
    def gn(self):
        return self.ngroups * self.dstate

    @property
    def channels(self):
        return self.hp + 2 * self.gn


CONFIGS = {
    # tiny fp32 layer: batch 1, 256 tokens, 4 heads x 16, 1 group, state 16
    "tiny_fp32": Cfg("tiny_fp32", 0, 1, 256, 4, 16, 1, 16, 4, 64, "f32"),
    # tiny-model layer (32 heads x 64, 8 groups, state 128), bf16 I/O
    "tiny_layer": Cfg("tiny_layer", 1, 4, 2048, 32, 64, 8, 128, 4, 128, "bf16"),
    # large-model layer prefill (256 heads x 64, 8 groups, state 128)
    "large_layer": Cfg("large_layer", 2, 1, 8192, 256, 64, 8, 128, 4, 256, "bf16"),
    # long context: 16 pieces of 8192 tokens, each resuming from state
    "long_context": Cfg("long_context", 3, 1, 8192, 32, 64, 8, 128, 4, 128, "bf16", pieces=16),
    # decode: 256 sequences x 64 single-token steps, states ~ N(0, 0.1)
    "decode_loop": Cfg("decode_loop", 4, 256, 1, 256, 64, 8, 128, 4, 0, "bf16", steps=64,
              nonzero_init=True),
}


def rng(cfg_index: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([1000 + cfg_index, stream])))


def round_bf16(a: np.ndarray) -> np.ndarray:
    """Round finite fp32 values to the nearest bf16 (ties to even); returns
    fp32. Works on the bit patterns in uint32 (no finite value carries out
    of 32 bits)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    r = u >> 16
    r &= 1
    r += 0x7FFF
    r += u
    r &= 0xFFFF0000
    return r.view(np.float32).reshape(a.shape)


def to_io(a: np.ndarray, dtype: str) -> np.ndarray:
    a = np.asarray(a, dtype=np.float32)
    return round_bf16(a) if dtype == "bf16" else np.ascontiguousarray(a)


def _softplus64(v: np.ndarray) -> np.ndarray:
    return np.logaddexp(0.0, v)


def layer_params(cfg: Cfg, slow_decay: bool = False, with_bias: bool = False,
                 dtype: str | None = None) -> dict:
    """A, D (fp32), conv weight [Cch, W] (+ optional bias), norm weight, eps.

    ``slow_decay`` draws A = -exp(U(log 0.005, log 0.05)) instead, so the
    state carries signal across many chunks and pieces."""
    dtype = dtype or cfg.dtype
    r = rng(cfg.index, 0)
    H, C, W = cfg.nheads, cfg.channels, cfg.conv_width
    if slow_decay:
        A = -np.exp(r.uniform(math.log(0.005), math.log(0.05), H))
    else:
        A = -np.exp(r.uniform(math.log(1.0), math.log(16.0), H))
    D = r.standard_normal(H)
    conv_w = r.standard_normal((C, W), dtype=np.float32) * np.float32(0.5)
    conv_b = r.standard_normal(C, dtype=np.float32) * np.float32(0.5) if with_bias else None
    return {
        "A": A.astype(np.float32),
        "D": D.astype(np.float32),
        "conv_w": to_io(conv_w, dtype),
        "conv_b": None if conv_b is None else to_io(conv_b, dtype),
        "norm_w": to_io(np.ones(cfg.hp, dtype=np.float32), dtype),
        "eps": 1e-5,
    }


def token_inputs(cfg: Cfg, batch: int, seqlen: int, stream: int,
                 dtype: str | None = None) -> dict:
    """xbc [B,L,Cch] = [x | B | C], z [B,L,H*P], dt [B,L,H] (I/O-rounded fp32)."""
    dtype = dtype or cfg.dtype
    r = rng(cfg.index, stream)
    Bn, L, H, P, G, N = batch, seqlen, cfg.nheads, cfg.headdim, cfg.ngroups, cfg.dstate
    sn = np.float32(1.0 / math.sqrt(N))
    x = r.standard_normal((Bn, L, H * P), dtype=np.float32)
    Bm = r.standard_normal((Bn, L, G * N), dtype=np.float32) * sn
    Cm = r.standard_normal((Bn, L, G * N), dtype=np.float32) * sn
    z = r.standard_normal((Bn, L, H * P), dtype=np.float32)
    dt = _softplus64(r.standard_normal((Bn, L, H)) - 2.0).astype(np.float32)
    xbc = np.concatenate([x, Bm, Cm], axis=-1)
    return {"xbc": to_io(xbc, dtype), "z": to_io(z, dtype), "dt": to_io(dt, dtype)}


def prefill_inputs(cfg: Cfg, piece: int = 0, batch: int | None = None,
                   seqlen: int | None = None, dtype: str | None = None) -> dict:
    return token_inputs(cfg, batch or cfg.batch, seqlen or cfg.seqlen, 1 + piece, dtype)


def decode_inputs(cfg: Cfg, step: int, batch: int | None = None,
                  dtype: str | None = None) -> dict:
    """One token per sequence: xbc_t [B,Cch], z_t [B,H*P], dt_t [B,H]."""
    t = token_inputs(cfg, batch or cfg.batch, 1, 1 + step, dtype)
    return {"xbc_t": t["xbc"][:, 0], "z_t": t["z"][:, 0], "dt_t": t["dt"][:, 0]}


def initial_states(cfg: Cfg, batch: int | None = None, dtype: str | None = None) -> dict:
    """conv state [B,W-1,Cch] (I/O dtype) and SSM state [B,H,P,N] (fp32),
    both ~ N(0, variance 0.1)."""
    dtype = dtype or cfg.dtype
    Bn = batch or cfg.batch
    r = rng(cfg.index, 100)
    sd = np.float32(math.sqrt(0.1))
    conv = r.standard_normal((Bn, cfg.conv_width - 1, cfg.channels), dtype=np.float32) * sd
    ssm = r.standard_normal((Bn, cfg.nheads, cfg.headdim, cfg.dstate), dtype=np.float32) * sd
    return {"conv_state": to_io(conv, dtype), "ssm_state": np.ascontiguousarray(ssm)}


# ---------------------------------------------------------------- backward
def backward_seeds(cfg: Cfg, batch: int | None = None, seqlen: int | None = None,
                   dtype: str | None = None) -> dict:
    """Upstream gradients for the backward pass and a non-trivial norm
    weight (stream 200): d_out [B,L,H*P] ~ N(0,1) (I/O dtype), d_ssm_state_out
    [B,H,P,N] ~ N(0, variance 0.1) fp32, norm_w [H*P] = 1 + N(0,1)/4 (I/O
    dtype)."""
    dtype = dtype or cfg.dtype
    Bn, L = batch or cfg.batch, seqlen or cfg.seqlen
    r = rng(cfg.index, 200)
    d_out = r.standard_normal((Bn, L, cfg.hp), dtype=np.float32)
    sd = np.float32(math.sqrt(0.1))
    d_s = r.standard_normal((Bn, cfg.nheads, cfg.headdim, cfg.dstate), dtype=np.float32) * sd
    nw = np.float32(1.0) + r.standard_normal(cfg.hp, dtype=np.float32) * np.float32(0.25)
    return {"d_out": to_io(d_out, dtype), "d_ssm_state_out": np.ascontiguousarray(d_s),
            "norm_w": to_io(nw, dtype)}


# ---------------------------------------------------------------- packed rows
# The same draws in the projection's raw form: the per-token row is
# [z | x | B | C | dt_raw] with dt_raw ~ N(0,1) (the normal that the recipe
# above shifts by -2 and passes through softplus), and the layer carries
# dt_bias = -2 and A_log ~ U(log 1, log 16) (the uniform whose exponential
# the recipe above negates). `pad` extra columns per row (filled with 30000,
# never read) make the row stride wider than the row.
PAD_VALUE = 30000.0


def packed_params(cfg: Cfg, slow_decay: bool = False, with_bias: bool = False,
                  dtype: str | None = None) -> dict:
    """A_log, dt_bias, D (fp32), conv weight (+ bias), norm weight, eps."""
    dtype = dtype or cfg.dtype
    r = rng(cfg.index, 0)
    H, C, W = cfg.nheads, cfg.channels, cfg.conv_width
    lo, hi = (math.log(0.005), math.log(0.05)) if slow_decay else (math.log(1.0), math.log(16.0))
    A_log = r.uniform(lo, hi, H)
    D = r.standard_normal(H)
    conv_w = r.standard_normal((C, W), dtype=np.float32) * np.float32(0.5)
    conv_b = r.standard_normal(C, dtype=np.float32) * np.float32(0.5) if with_bias else None
    return {
        "A_log": A_log.astype(np.float32),
        "dt_bias": np.full(H, -2.0, dtype=np.float32),
        "D": D.astype(np.float32),
        "conv_w": to_io(conv_w, dtype),
        "conv_b": None if conv_b is None else to_io(conv_b, dtype),
        "norm_w": to_io(np.ones(cfg.hp, dtype=np.float32), dtype),
        "eps": 1e-5,
    }


def packed_rows(cfg: Cfg, batch: int, seqlen: int, stream: int, pad: int = 0,
                dtype: str | None = None) -> np.ndarray:
    """[B, L, 2HP + 2GN + H + pad] rows [z | x | B | C | dt_raw | pad]."""
    dtype = dtype or cfg.dtype
    r = rng(cfg.index, stream)
    Bn, L, H, P, G, N = batch, seqlen, cfg.nheads, cfg.headdim, cfg.ngroups, cfg.dstate
    sn = np.float32(1.0 / math.sqrt(N))
    x = r.standard_normal((Bn, L, H * P), dtype=np.float32)
    Bm = r.standard_normal((Bn, L, G * N), dtype=np.float32) * sn
    Cm = r.standard_normal((Bn, L, G * N), dtype=np.float32) * sn
    z = r.standard_normal((Bn, L, H * P), dtype=np.float32)
    raw = r.standard_normal((Bn, L, H)).astype(np.float32)
    fill = np.full((Bn, L, pad), PAD_VALUE, dtype=np.float32)
    return to_io(np.concatenate([z, x, Bm, Cm, raw, fill], axis=-1), dtype)


def packed_prefill_inputs(cfg: Cfg, piece: int = 0, pad: int = 0, batch: int | None = None,
                          seqlen: int | None = None, dtype: str | None = None) -> np.ndarray:
    return packed_rows(cfg, batch or cfg.batch, seqlen or cfg.seqlen, 1 + piece, pad, dtype)


def packed_decode_inputs(cfg: Cfg, step: int, pad: int = 0, batch: int | None = None,
                         dtype: str | None = None) -> np.ndarray:
    """One token per sequence: [B, row]."""
    return packed_rows(cfg, batch or cfg.batch, 1, 1 + step, pad, dtype)[:, 0]


def split_channels(cfg: Cfg, xbc: np.ndarray):
    """Views x [.., H, P], B [.., G, N], C [.., G, N] of a [.., Cch] array."""
    HP, GN = cfg.hp, cfg.gn
    lead = xbc.shape[:-1]
    x = xbc[..., :HP].reshape(*lead, cfg.nheads, cfg.headdim)
    Bm = xbc[..., HP:HP + GN].reshape(*lead, cfg.ngroups, cfg.dstate)
    Cm = xbc[..., HP + GN:].reshape(*lead, cfg.ngroups, cfg.dstate)
    return x, Bm, Cm


def replace(cfg: Cfg, **kw) -> Cfg:
    return dataclasses.replace(cfg, **kw)
