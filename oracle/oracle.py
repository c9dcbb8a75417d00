"""fp64 CPU oracle for the Mamba-2 mixer core — TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the CPU-baseline leg of the
benchmark may import this module. It shares no code with the HIP path: the
primary oracle is the plain C file ``ssd_oracle.c`` next to this one
(sequential recurrence, explicit conv and gated norm, all fp64), loaded here
through ctypes; this module adds two independent NumPy fp64 formulations used
only to pin it:

* ``ssd_chunked`` — the chunk-parallel block decomposition of the scan (the
  "ssd_minimal_discrete / segsum" decomposition that the Modalities PR #459
  attribution commit names for its ``ssd.py``): intra-chunk quadratic form
  masked by the segment-sum decay, plus the state carried across chunks.
* ``ssd_unrolled`` — the recurrence unrolled into one explicit [L, L] matrix
  per (batch, head) (brute force, tiny inputs only).

Citations use the page title and section: "gllm PR #86" is "feat(model):
Nemotron-H hybrid (Mamba2 + attention + MoE) on the CPU"; "Modalities PR
#459" is "feat(model): add Nemotron-3 Nano hybrid Mamba-Transformer MoE
architecture"; "NemotronH-0.3B card" is the "NemotronH-0.3B-A0.3B" model card.

Parity status: the recurrence, the conv (up to tap orientation) and the
gated norm (up to gate/normalise order and grouping) are pinned by the tests
in ``tests/test_oracle_pins.py``. Three conventions the pages do not fix are
"parity unpinned" (tap orientation, head->group map, gate-then-normalise);
they are stated in the C file's header and in the design notes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ssd_oracle.c")
_LIB = os.path.join(_HERE, "libssd_oracle.so")

def build(force: bool = True, src: str = _SRC, out: str = _LIB) -> str:
    """Compile an oracle C source into a shared library (gcc, -O3, OpenMP)."""
    if force or not os.path.exists(out):
        cmd = ["gcc", "-O3", "-fopenmp", "-fPIC", "-shared", "-std=c11",
               "-o", out + ".tmp", src, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(out + ".tmp", out)
    return out


def _bind(path: str):
    lib = ctypes.CDLL(path)
    i64, dp = ctypes.c_int64, ctypes.c_void_p
    lib.oracle_conv1d_silu.argtypes = [i64] * 4 + [dp] * 6
    lib.oracle_ssm_scan.argtypes = [i64] * 6 + [dp] * 9
    lib.oracle_gated_rmsnorm.argtypes = [i64] * 3 + [dp] * 3 + [ctypes.c_double, dp]
    lib.oracle_mixer_prefill.argtypes = [i64] * 7 + [dp] * 8 + [ctypes.c_double] + [dp] * 6
    lib.oracle_decode_step.argtypes = [i64] * 6 + [dp] * 8 + [ctypes.c_double] + [dp] * 3
    lib.oracle_dt_a.argtypes = [i64] * 2 + [dp] * 5
    lib.oracle_mixer_prefill_packed.argtypes = [i64] * 8 + [dp] * 7 + [ctypes.c_double] + [dp] * 5
    lib.oracle_decode_step_packed.argtypes = [i64] * 7 + [dp] * 7 + [ctypes.c_double] + [dp] * 3
    lib.oracle_mixer_varlen.argtypes = ([i64] + [dp] * 3 + [i64] * 5 + [dp] * 8 + [ctypes.c_double]
                                        + [dp] * 3)
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
    return lib


def _f64(a):
    if a is None:
        return None
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


# ---------------------------------------------------------------- primary (C)

class Oracle:
    """The C oracle bound to one compiled library file (the default is
    ``libssd_oracle.so`` built from ``ssd_oracle.c``)."""

    def __init__(self, path: str | None = None):
        if path is None:
            path = _LIB if os.path.exists(_LIB) else build(force=True)
        self.path = path
        self._lib = _bind(path)

    def num_threads(self) -> int:
        return int(self._lib.oracle_num_threads())

    def set_num_threads(self, n: int) -> None:
        self._lib.oracle_set_num_threads(int(n))


    def conv1d_silu(self, xbc, w, bias=None, conv_in=None):
        """Depthwise causal conv + SiLU (gllm PR #86, "2. feat(model)": the
        CausalConv1D step over xBC). xbc [B,L,C], w [C,W] -> (out [B,L,C],
        conv_out [B,W-1,C])."""
        xbc, w, bias, conv_in = _f64(xbc), _f64(w), _f64(bias), _f64(conv_in)
        Bn, L, C = xbc.shape
        W = w.shape[1]
        out = np.empty((Bn, L, C))
        cs = np.empty((Bn, W - 1, C))
        self._lib.oracle_conv1d_silu(Bn, L, C, W, _p(xbc), _p(w), _p(bias), _p(conv_in),
                                   _p(out), _p(cs))
        return out, cs


    def ssm_scan(self, x, dt, A, Bm, Cm, D=None, s_in=None):
        """Sequential recurrence (gllm PR #86, "Validation": the plain sequential
        recurrence is the truth). x [B,L,H,P], dt [B,L,H], A [H], Bm/Cm
        [B,L,G,N], D [H] -> (y [B,L,H,P], s_out [B,H,P,N])."""
        x, dt, A, Bm, Cm, D, s_in = map(_f64, (x, dt, A, Bm, Cm, D, s_in))
        Bn, L, H, P = x.shape
        G, N = Bm.shape[2], Bm.shape[3]
        y = np.empty((Bn, L, H, P))
        s_out = np.empty((Bn, H, P, N))
        self._lib.oracle_ssm_scan(Bn, L, H, P, G, N, _p(x), _p(dt), _p(A), _p(Bm), _p(Cm),
                                _p(D), _p(s_in), _p(y), _p(s_out))
        return y, s_out


    def gated_rmsnorm(self, y, z, w, G, eps):
        """Grouped gated RMSNorm (Modalities PR #459 attribution commit: the
        GatedRMSNorm semantics), gate first. y, z [..., HP], w [HP]."""
        y, z, w = _f64(y), _f64(z), _f64(w)
        HP = y.shape[-1]
        rows = y.size // HP
        out = np.empty_like(y)
        self._lib.oracle_gated_rmsnorm(rows, HP, G, _p(y), _p(z), _p(w), float(eps), _p(out))
        return out


    def mixer_prefill(self, xbc, z, dt, A, D, conv_w, conv_b, norm_w, eps, H, P, G, N,
                      conv_in=None, s_in=None):
        """conv + SiLU -> split [x | B | C] -> recurrence -> gated norm.
        Returns dict(out, y, conv_out, s_out)."""
        xbc, z, dt, A, D, conv_w, conv_b, norm_w, conv_in, s_in = map(
            _f64, (xbc, z, dt, A, D, conv_w, conv_b, norm_w, conv_in, s_in))
        Bn, L, C = xbc.shape
        W = conv_w.shape[1]
        assert C == H * P + 2 * G * N
        out = np.empty((Bn, L, H * P))
        y = np.empty((Bn, L, H * P))
        cs = np.empty((Bn, W - 1, C))
        so = np.empty((Bn, H, P, N))
        self._lib.oracle_mixer_prefill(Bn, L, H, P, G, N, W, _p(xbc), _p(z), _p(dt), _p(A),
                                     _p(D), _p(conv_w), _p(conv_b), _p(norm_w), float(eps),
                                     _p(conv_in), _p(cs), _p(s_in), _p(so), _p(out), _p(y))
        return {"out": out, "y": y, "conv_out": cs, "s_out": so}


    def dt_a(self, dt_raw, dt_bias, A_log):
        """The step before the path: dt = softplus(dt_raw + dt_bias),
        A = -exp(A_log) (Modalities PR #459 attribution commit: A_log and
        dt_bias are the mixer's parameters). dt_raw [..., H] -> (dt, A)."""
        dt_raw, dt_bias, A_log = map(_f64, (dt_raw, dt_bias, A_log))
        H = dt_raw.shape[-1]
        dt = np.empty_like(dt_raw)
        A = np.empty(H)
        self._lib.oracle_dt_a(dt_raw.size // H, H, _p(dt_raw), _p(dt_bias), _p(A_log), _p(dt),
                              _p(A))
        return dt, A

    def mixer_prefill_packed(self, zxbcdt, dt_bias, A_log, D, conv_w, conv_b, norm_w, eps, H, P,
                             G, N, conv_in=None, s_in=None):
        """Prefill on packed projection rows [z | xBC | dt_raw] (gllm PR #86,
        "Supporting changes": in_proj emits [z | xBC | dt] in one row);
        zxbcdt [B, L, row] with row >= 2HP + 2GN + H. Returns dict(out,
        conv_out, s_out)."""
        zxbcdt, dt_bias, A_log, D, conv_w, conv_b, norm_w, conv_in, s_in = map(
            _f64, (zxbcdt, dt_bias, A_log, D, conv_w, conv_b, norm_w, conv_in, s_in))
        Bn, L, R = zxbcdt.shape
        W = conv_w.shape[1]
        C = H * P + 2 * G * N
        assert R >= H * P + C + H
        out = np.empty((Bn, L, H * P))
        cs = np.empty((Bn, W - 1, C))
        so = np.empty((Bn, H, P, N))
        self._lib.oracle_mixer_prefill_packed(Bn, L, H, P, G, N, W, R, _p(zxbcdt), _p(dt_bias),
                                              _p(A_log), _p(D), _p(conv_w), _p(conv_b),
                                              _p(norm_w), float(eps), _p(conv_in), _p(cs),
                                              _p(s_in), _p(so), _p(out))
        return {"out": out, "conv_out": cs, "s_out": so}

    def decode_step_packed(self, zxbcdt_t, dt_bias, A_log, D, conv_w, conv_b, norm_w, eps, H, P,
                           G, N, conv_state, ssm_state):
        """One token per sequence from packed rows [B, row]; returns
        (out [B,HP], conv_state', ssm_state') without touching the arguments."""
        zxbcdt_t, dt_bias, A_log, D, conv_w, conv_b, norm_w = map(
            _f64, (zxbcdt_t, dt_bias, A_log, D, conv_w, conv_b, norm_w))
        cs = np.array(conv_state, dtype=np.float64, copy=True, order="C")
        ss = np.array(ssm_state, dtype=np.float64, copy=True, order="C")
        Bn, R = zxbcdt_t.shape
        W = conv_w.shape[1]
        out = np.empty((Bn, H * P))
        self._lib.oracle_decode_step_packed(Bn, H, P, G, N, W, R, _p(zxbcdt_t), _p(dt_bias),
                                            _p(A_log), _p(D), _p(conv_w), _p(conv_b),
                                            _p(norm_w), float(eps), _p(cs), _p(ss), _p(out))
        return out, cs, ss

    def mixer_varlen(self, cu_seqlens, slots, has_state, xbc, z, dt, A, D, conv_w, conv_b,
                     norm_w, eps, H, P, G, N, conv_pool, ssm_pool):
        """Sequences packed back to back (tokens [cu[i], cu[i+1]) of xbc [T, C],
        z [T, HP], dt [T, H]), each resuming from its state slot (gllm PR #86,
        "Validation": two sequences in one batch on separate slots, one
        prefilling while the other decodes). Returns (out [T, HP], conv_pool',
        ssm_pool') without touching the arguments."""
        cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
        sl = np.ascontiguousarray(slots, dtype=np.int32)
        hs = None if has_state is None else np.ascontiguousarray(has_state, dtype=np.uint8)
        xbc, z, dt, A, D, conv_w, conv_b, norm_w = map(
            _f64, (xbc, z, dt, A, D, conv_w, conv_b, norm_w))
        cp = np.array(conv_pool, dtype=np.float64, copy=True, order="C")
        sp = np.array(ssm_pool, dtype=np.float64, copy=True, order="C")
        T = xbc.shape[0]
        W = conv_w.shape[1]
        out = np.zeros((T, H * P))
        self._lib.oracle_mixer_varlen(len(sl), _p(cu), _p(sl), _p(hs), H, P, G, N, W, _p(xbc),
                                      _p(z), _p(dt), _p(A), _p(D), _p(conv_w), _p(conv_b),
                                      _p(norm_w), float(eps), _p(cp), _p(sp), _p(out))
        return out, cp, sp

    def decode_step(self, xbc_t, z_t, dt_t, A, D, conv_w, conv_b, norm_w, eps, H, P, G, N,
                    conv_state, ssm_state):
        """One token per sequence; returns (out [B,HP], conv_state', ssm_state')
        without touching the arguments (gllm PR #86, "Validation": token-by-token
        decode resuming every Mamba layer from its slot)."""
        xbc_t, z_t, dt_t, A, D, conv_w, conv_b, norm_w = map(
            _f64, (xbc_t, z_t, dt_t, A, D, conv_w, conv_b, norm_w))
        cs = np.array(conv_state, dtype=np.float64, copy=True, order="C")
        ss = np.array(ssm_state, dtype=np.float64, copy=True, order="C")
        Bn = xbc_t.shape[0]
        W = conv_w.shape[1]
        out = np.empty((Bn, H * P))
        self._lib.oracle_decode_step(Bn, H, P, G, N, W, _p(xbc_t), _p(z_t), _p(dt_t), _p(A),
                                   _p(D), _p(conv_w), _p(conv_b), _p(norm_w), float(eps),
                                   _p(cs), _p(ss), _p(out))
        return out, cs, ss




_default: Oracle | None = None


def default() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def num_threads() -> int:
    return default().num_threads()


def set_num_threads(n: int) -> None:
    default().set_num_threads(n)


def conv1d_silu(*args, **kw):
    return default().conv1d_silu(*args, **kw)


def ssm_scan(*args, **kw):
    return default().ssm_scan(*args, **kw)


def gated_rmsnorm(*args, **kw):
    return default().gated_rmsnorm(*args, **kw)


def mixer_prefill(*args, **kw):
    return default().mixer_prefill(*args, **kw)


def decode_step(*args, **kw):
    return default().decode_step(*args, **kw)


def mixer_varlen(*args, **kw):
    return default().mixer_varlen(*args, **kw)


def dt_a(*args, **kw):
    return default().dt_a(*args, **kw)


def mixer_prefill_packed(*args, **kw):
    return default().mixer_prefill_packed(*args, **kw)


def decode_step_packed(*args, **kw):
    return default().decode_step_packed(*args, **kw)

def split_xbc(v, H, P, G, N):
    """Channel order of the conv output: x (H*P) | B (G*N) | C (G*N)
    (gllm PR #86, "Supporting changes": in_proj emits [z | xBC | dt];
    Modalities PR #459 attribution commit: packed [z, x, B, C, dt])."""
    Bn, L, _ = v.shape
    HP, GN = H * P, G * N
    x = v[..., :HP].reshape(Bn, L, H, P)
    Bm = v[..., HP:HP + GN].reshape(Bn, L, G, N)
    Cm = v[..., HP + GN:HP + 2 * GN].reshape(Bn, L, G, N)
    return x, Bm, Cm


# ------------------------------------------- independent NumPy formulations

def ssd_chunked(x, dt, A, Bm, Cm, D=None, s_in=None, Q=64):
    """Chunk-parallel block decomposition of the scan, fp64 (Modalities PR
    #459 attribution commit: ssd_minimal_discrete / segsum).

    Per chunk [t0, t1) and head h (group g = h // (H/G)):
      a_t = dt_t A_h;  Lam_t = sum_{r=t0..t} a_r       (inclusive segment sum)
      Y_diag[t] = sum_{s=t0..t} (C_t . B_s) exp(Lam_t - Lam_s) dt_s x_s
      Y_off[t]  = exp(Lam_t) (S_in C_t)
      S_out     = exp(Lam_{t1-1}) S_in + sum_s exp(Lam_{t1-1} - Lam_s) dt_s x_s (outer) B_s
    and y = Y_diag + Y_off + D x. Exact for every Q >= 1.
    """
    x, dt, A, Bm, Cm = map(_f64, (x, dt, A, Bm, Cm))
    Bn, L, H, P = x.shape
    G, N = Bm.shape[2], Bm.shape[3]
    hpg = H // G
    y = np.zeros((Bn, L, H, P))
    S_all = np.zeros((Bn, H, P, N)) if s_in is None else _f64(s_in).copy()
    for b in range(Bn):
        for h in range(H):
            g = h // hpg
            S = S_all[b, h].copy()
            for t0 in range(0, L, Q):
                t1 = min(L, t0 + Q)
                a = dt[b, t0:t1, h] * A[h]
                lam = np.cumsum(a)
                seg = lam[:, None] - lam[None, :]           # Lam_t - Lam_s
                causal = np.tril(np.ones((t1 - t0, t1 - t0), dtype=bool))
                decay = np.where(causal, np.exp(np.where(causal, seg, 0.0)), 0.0)
                CB = Cm[b, t0:t1, g] @ Bm[b, t0:t1, g].T     # [t, s]
                xdt = x[b, t0:t1, h] * dt[b, t0:t1, h][:, None]
                y_diag = (CB * decay) @ xdt
                y_off = np.exp(lam)[:, None] * (Cm[b, t0:t1, g] @ S.T)
                y[b, t0:t1, h] = y_diag + y_off
                w_end = np.exp(lam[-1] - lam) * dt[b, t0:t1, h]
                S = np.exp(lam[-1]) * S + (x[b, t0:t1, h] * w_end[:, None]).T @ Bm[b, t0:t1, g]
            S_all[b, h] = S
    if D is not None:
        y += _f64(D)[None, None, :, None] * x
    return y, S_all


def ssd_unrolled(x, dt, A, Bm, Cm, D=None, s_in=None):
    """Brute-force unrolled recurrence as one explicit [L, L] matrix per
    (batch, head):
      y_t = exp(sum_{r<=t} a_r) (S0 C_t)
            + sum_{s<=t} (C_t . B_s) exp(sum_{r=s+1..t} a_r) dt_s x_s + D x_t.
    Each decay is a direct sum over its own index range (no cumsum
    differences). O(L^3) per head: tiny inputs only."""
    x, dt, A, Bm, Cm = map(_f64, (x, dt, A, Bm, Cm))
    Bn, L, H, P = x.shape
    G, N = Bm.shape[2], Bm.shape[3]
    hpg = H // G
    y = np.zeros((Bn, L, H, P))
    for b in range(Bn):
        for h in range(H):
            g = h // hpg
            a = dt[b, :, h] * A[h]
            Mx = np.zeros((L, L))
            for t in range(L):
                for s in range(t + 1):
                    dec = np.exp(np.sum(a[s + 1:t + 1]))
                    Mx[t, s] = float(Cm[b, t, g] @ Bm[b, s, g]) * dec * dt[b, s, h]
            y[b, :, h] = Mx @ x[b, :, h]
            if s_in is not None:
                S0 = _f64(s_in)[b, h]
                for t in range(L):
                    y[b, t, h] += np.exp(np.sum(a[:t + 1])) * (S0 @ Cm[b, t, g])
    if D is not None:
        y += _f64(D)[None, None, :, None] * x
    return y
