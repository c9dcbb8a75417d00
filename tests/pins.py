"""Pins for the fp64 oracle: each checks it against something other than
itself — an independent formulation, a textbook or library routine, a closed
form, an invariant, or a value the pages print. Each returns an error figure
that must stay at or below ``LIMITS[name]``.

Used by ``test_oracle_pins.py`` (the oracle as built must pass every pin)
and ``test_oracle_mutations.py`` (a copy of the oracle with a planted mistake
must fail at least one pin).
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import scipy.signal
import scipy.special

from oracle import oracle as orc_mod

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _softplus(v):
    return np.logaddexp(0.0, v)


def rand_scan(seed, Bn=2, L=37, H=4, P=3, G=2, N=5, a_lo=0.05, a_hi=2.0,
              with_state=True, with_D=True):
    """Random fp64 scan inputs. Decay rates are moderate so the state carries
    signal across many tokens (index mistakes stay visible)."""
    r = np.random.default_rng(seed)
    x = r.standard_normal((Bn, L, H, P))
    dt = _softplus(r.standard_normal((Bn, L, H)) - 1.0)
    A = -np.exp(r.uniform(math.log(a_lo), math.log(a_hi), H))
    Bm = r.standard_normal((Bn, L, G, N)) / math.sqrt(N)
    Cm = r.standard_normal((Bn, L, G, N)) / math.sqrt(N)
    D = r.standard_normal(H) if with_D else None
    s0 = 0.3 * r.standard_normal((Bn, H, P, N)) if with_state else None
    return x, dt, A, Bm, Cm, D, s0


def rand_mixer(seed, Bn=2, L=29, H=4, P=4, G=2, N=3, W=4, bias=True):
    r = np.random.default_rng(seed)
    C = H * P + 2 * G * N
    return dict(
        xbc=r.standard_normal((Bn, L, C)),
        z=r.standard_normal((Bn, L, H * P)),
        dt=_softplus(r.standard_normal((Bn, L, H)) - 1.0),
        A=-np.exp(r.uniform(math.log(0.05), math.log(2.0), H)),
        D=r.standard_normal(H),
        conv_w=0.5 * r.standard_normal((C, W)),
        conv_b=0.5 * r.standard_normal(C) if bias else None,
        norm_w=1.0 + 0.2 * r.standard_normal(H * P),
        eps=1e-5, H=H, P=P, G=G, N=N,
        conv_in=0.3 * r.standard_normal((Bn, W - 1, C)),
        s_in=0.3 * r.standard_normal((Bn, H, P, N)),
    )


def _rel(a, b):
    a, b = np.asarray(a, float), np.asarray(b, float)
    return float(np.max(np.abs(a - b)) / (1.0 + np.max(np.abs(b))))


# ---------------------------------------------------------------------------
# P1: brute-force unrolled [L, L] matrix form of the recurrence.
def pin_unrolled(orc):
    errs = []
    for seed, kw in [(1, {}), (2, dict(L=48, H=2, G=1, P=2, N=4)),
                     (3, dict(with_state=False, L=20)), (4, dict(H=6, G=3, L=16))]:
        x, dt, A, Bm, Cm, D, s0 = rand_scan(seed, **kw)
        y, _ = orc.ssm_scan(x, dt, A, Bm, Cm, D, s0)
        errs.append(_rel(y, orc_mod.ssd_unrolled(x, dt, A, Bm, Cm, D, s0)))
    return max(errs)


# P2: the SSD identity — chunked block decomposition == recurrence for any Q.
def pin_chunked(orc):
    x, dt, A, Bm, Cm, D, s0 = rand_scan(5, L=70)
    y, s = orc.ssm_scan(x, dt, A, Bm, Cm, D, s0)
    errs = []
    for Q in (1, 2, 3, 5, 8, 16, 64, 70):
        yc, sc = orc_mod.ssd_chunked(x, dt, A, Bm, Cm, D, s0, Q=Q)
        errs += [_rel(y, yc), _rel(s, sc)]
        first = list(range(Q, 70, Q))  # first token of every later chunk
        if first:
            errs.append(_rel(y[:, first], yc[:, first]))
    return max(errs)


# P3: textbook IIR filter (scipy.signal.lfilter) for the scalar case with
# constant dt: h_t = a h_{t-1} + dt B_t x_t, y_t = C_t h_t + D x_t.
def pin_lfilter(orc):
    r = np.random.default_rng(6)
    L = 200
    x = r.standard_normal((1, L, 1, 1))
    Bm = r.standard_normal((1, L, 1, 1))
    Cm = r.standard_normal((1, L, 1, 1))
    errs = []
    for dtv, Av, Dv in [(0.3, -0.7, 0.4), (1.7, -0.05, -1.1), (0.01, -3.0, 0.0)]:
        dt = np.full((1, L, 1), dtv)
        y, s = orc.ssm_scan(x, dt, np.array([Av]), Bm, Cm, np.array([Dv]), None)
        u = Bm[0, :, 0, 0] * x[0, :, 0, 0]
        h = scipy.signal.lfilter([dtv], [1.0, -math.exp(dtv * Av)], u)
        ref = Cm[0, :, 0, 0] * h + Dv * x[0, :, 0, 0]
        errs += [_rel(y[0, :, 0, 0], ref), _rel(s[0, 0, 0, 0], h[-1])]
    return max(errs)


# P4: A = 0 turns the scan into a prefix sum (unnormalised linear attention).
def pin_prefix_sum(orc):
    x, dt, A, Bm, Cm, D, s0 = rand_scan(7, L=41)
    A = np.zeros_like(A)
    y, s = orc.ssm_scan(x, dt, A, Bm, Cm, D, s0)
    H, G = x.shape[2], Bm.shape[2]
    g_of_h = np.arange(H) // (H // G)
    Bh, Ch = Bm[:, :, g_of_h], Cm[:, :, g_of_h]          # [B,L,H,N]
    incr = np.einsum("blh,blhp,blhn->blhpn", dt, x, Bh)
    S = np.cumsum(incr, axis=1) + s0[:, None]
    ref = np.einsum("blhpn,blhn->blhp", S, Ch) + D[None, None, :, None] * x
    return max(_rel(y, ref), _rel(s, S[:, -1]))


# P5: memoryless limit — exp(dt A) underflows, y_t = dt_t (C_t . B_t) x_t + D x_t.
def pin_memoryless(orc):
    x, dt, A, Bm, Cm, D, s0 = rand_scan(8, L=23)
    dt = np.maximum(dt, 0.01)
    A = np.full_like(A, -1e4)
    y, s = orc.ssm_scan(x, dt, A, Bm, Cm, D, s0)
    H, G = x.shape[2], Bm.shape[2]
    g_of_h = np.arange(H) // (H // G)
    cb = np.einsum("blhn,blhn->blh", Cm[:, :, g_of_h], Bm[:, :, g_of_h])
    ref = (dt * cb)[..., None] * x + D[None, None, :, None] * x
    sref = dt[:, -1, :, None, None] * x[:, -1, :, :, None] * Bm[:, -1, g_of_h][:, :, None, :]
    return max(_rel(y, ref), _rel(s, sref))


# P6: the conv is a per-channel FIR cross-correlation (numpy.correlate), and
# matches torch's depthwise conv1d on CPU; the carried conv state is the last
# W-1 rows of [state ; input].
def pin_conv(orc):
    import torch
    errs = []
    r = np.random.default_rng(9)
    for (Bn, L, C, W) in [(2, 19, 7, 4), (1, 2, 5, 4), (3, 1, 4, 3), (1, 33, 6, 2)]:
        xbc = r.standard_normal((Bn, L, C))
        w = r.standard_normal((C, W))
        b = r.standard_normal(C)
        cin = r.standard_normal((Bn, W - 1, C))
        out, cout = orc.conv1d_silu(xbc, w, b, cin)
        ext = np.concatenate([cin, xbc], axis=1)
        u = np.empty((Bn, L, C))
        for bb in range(Bn):
            for c in range(C):
                u[bb, :, c] = np.correlate(ext[bb, :, c], w[c], mode="valid") + b[c]
        errs.append(_rel(out, u * scipy.special.expit(u)))
        ut = torch.nn.functional.conv1d(torch.from_numpy(ext).permute(0, 2, 1),
                                        torch.from_numpy(w)[:, None, :],
                                        torch.from_numpy(b), groups=C)
        ut = ut.permute(0, 2, 1).numpy()
        errs.append(_rel(out, ut * scipy.special.expit(ut)))
        errs.append(float(np.max(np.abs(cout - ext[:, L:L + W - 1]))))
        out0, _ = orc.conv1d_silu(xbc, w, None, None)     # null state = zeros
        ext0 = np.concatenate([np.zeros_like(cin), xbc], axis=1)
        u0 = np.stack([np.stack([np.correlate(ext0[bb, :, c], w[c], "valid") for c in range(C)], -1)
                       for bb in range(Bn)])
        errs.append(_rel(out0, u0 * scipy.special.expit(u0)))
    return max(errs)


# P7: gated RMSNorm closed forms. With unit weight each group's output RMS is
# sqrt(m / (m + eps)), m = mean(q^2); the whole result equals torch's
# rms_norm over each group of q = y * silu(z), times the weight.
def pin_norm(orc):
    import torch
    r = np.random.default_rng(10)
    errs = []
    for rows, HP, G in [(5, 64, 1), (7, 96, 4), (3, 16, 8)]:
        y = r.standard_normal((rows, HP))
        y[0] *= 1e-3                      # eps matters on this row
        z = r.standard_normal((rows, HP))
        w = r.standard_normal(HP)
        eps = 1e-5
        out1 = orc.gated_rmsnorm(y, z, np.ones(HP), G, eps)
        q = y * z * scipy.special.expit(z)
        S = HP // G
        m = (q.reshape(rows, G, S) ** 2).mean(-1)
        rms = np.sqrt((out1.reshape(rows, G, S) ** 2).mean(-1))
        errs.append(_rel(rms, np.sqrt(m / (m + eps))))
        out = orc.gated_rmsnorm(y, z, w, G, eps)
        ref = torch.nn.functional.rms_norm(torch.from_numpy(q.reshape(rows, G, S)), [S], eps=eps)
        ref = ref.reshape(rows, HP).numpy() * w
        errs.append(_rel(out, ref))
    return max(errs)


# P8: T decode steps == one T-token prefill from the same states.
def pin_decode_is_prefill(orc):
    k = rand_mixer(11, L=9)
    pre = orc.mixer_prefill(k["xbc"], k["z"], k["dt"], k["A"], k["D"], k["conv_w"], k["conv_b"],
                            k["norm_w"], k["eps"], k["H"], k["P"], k["G"], k["N"],
                            conv_in=k["conv_in"], s_in=k["s_in"])
    cs, ss = k["conv_in"].copy(), k["s_in"].copy()
    outs = []
    for t in range(k["xbc"].shape[1]):
        o, cs, ss = orc.decode_step(k["xbc"][:, t], k["z"][:, t], k["dt"][:, t], k["A"], k["D"],
                                    k["conv_w"], k["conv_b"], k["norm_w"], k["eps"],
                                    k["H"], k["P"], k["G"], k["N"], cs, ss)
        outs.append(o)
    return max(_rel(np.stack(outs, 1), pre["out"]), _rel(cs, pre["conv_out"]),
               _rel(ss, pre["s_out"]))


# P9: piecewise prefill == single shot, for uneven splits and for pieces
# shorter than W-1.
def pin_piecewise(orc):
    k = rand_mixer(12, L=31)
    args = lambda a, b: (k["xbc"][:, a:b], k["z"][:, a:b], k["dt"][:, a:b], k["A"], k["D"],
                         k["conv_w"], k["conv_b"], k["norm_w"], k["eps"],
                         k["H"], k["P"], k["G"], k["N"])
    full = orc.mixer_prefill(*args(0, 31), conv_in=k["conv_in"], s_in=k["s_in"])
    errs = []
    for cuts in ([13], [1, 2, 3], [2, 20, 21, 30], [5, 7, 8, 9, 17]):
        bounds = [0] + cuts + [31]
        cs, ss, outs = k["conv_in"], k["s_in"], []
        for a, b in zip(bounds[:-1], bounds[1:]):
            r = orc.mixer_prefill(*args(a, b), conv_in=cs, s_in=ss)
            cs, ss = r["conv_out"], r["s_out"]
            outs.append(r["out"])
        errs += [_rel(np.concatenate(outs, 1), full["out"]), _rel(cs, full["conv_out"]),
                 _rel(ss, full["s_out"])]
    return max(errs)


# P10: causality — perturbing token t leaves every earlier output bit-identical
# and changes the output at t.
def pin_causality(orc):
    k = rand_mixer(13, L=17)
    base = orc.mixer_prefill(k["xbc"], k["z"], k["dt"], k["A"], k["D"], k["conv_w"], k["conv_b"],
                             k["norm_w"], k["eps"], k["H"], k["P"], k["G"], k["N"],
                             conv_in=k["conv_in"], s_in=k["s_in"])["out"]
    bad = 0.0
    for t in (0, 5, 16):
        for which in ("xbc", "dt", "z"):
            kk = {**k, which: k[which].copy()}
            kk[which][:, t] += 0.5
            out = orc.mixer_prefill(kk["xbc"], kk["z"], kk["dt"], k["A"], k["D"], k["conv_w"],
                                    k["conv_b"], k["norm_w"], k["eps"], k["H"], k["P"], k["G"],
                                    k["N"], conv_in=k["conv_in"], s_in=k["s_in"])["out"]
            if not np.array_equal(out[:, :t], base[:, :t]):
                bad = 1.0
            if np.array_equal(out[:, t], base[:, t]):
                bad = 1.0
    return bad


# P11: the scan is linear in (x, S0) for fixed dt, A, B, C, D.
def pin_linearity(orc):
    x1, dt, A, Bm, Cm, D, s1 = rand_scan(14, L=25)
    x2, _, _, _, _, _, s2 = rand_scan(15, L=25)
    y1, f1 = orc.ssm_scan(x1, dt, A, Bm, Cm, D, s1)
    y2, f2 = orc.ssm_scan(x2, dt, A, Bm, Cm, D, s2)
    y3, f3 = orc.ssm_scan(2.0 * x1 - 3.0 * x2, dt, A, Bm, Cm, D, 2.0 * s1 - 3.0 * s2)
    return max(_rel(y3, 2 * y1 - 3 * y2), _rel(f3, 2 * f1 - 3 * f2))


# P12: the composite is conv+SiLU, then the [x | B | C] channel split the
# pages' packed projection layout gives, then the scan, then the gated norm.
def pin_composition(orc):
    k = rand_mixer(16, L=21)
    res = orc.mixer_prefill(k["xbc"], k["z"], k["dt"], k["A"], k["D"], k["conv_w"], k["conv_b"],
                            k["norm_w"], k["eps"], k["H"], k["P"], k["G"], k["N"],
                            conv_in=k["conv_in"], s_in=k["s_in"])
    v, _ = orc.conv1d_silu(k["xbc"], k["conv_w"], k["conv_b"], k["conv_in"])
    H, P, G, N = k["H"], k["P"], k["G"], k["N"]
    HP, GN = H * P, G * N
    Bn, L = v.shape[:2]
    x = v[..., :HP].reshape(Bn, L, H, P)
    Bm = v[..., HP:HP + GN].reshape(Bn, L, G, N)
    Cm = v[..., HP + GN:].reshape(Bn, L, G, N)
    y = orc_mod.ssd_unrolled(x, k["dt"], k["A"], Bm, Cm, k["D"], k["s_in"]).reshape(Bn, L, HP)
    q = y * k["z"] * scipy.special.expit(k["z"])
    S = HP // G
    qg = q.reshape(Bn, L, G, S)
    ref = (qg / np.sqrt((qg ** 2).mean(-1, keepdims=True) + k["eps"])).reshape(Bn, L, HP) * k["norm_w"]
    return max(_rel(res["y"], y), _rel(res["out"], ref))


# Worked example (tests/golden/scalar_worked_example.json): a two-token scalar
# recurrence whose values are derived by hand.
def pin_worked_example(orc):
    with open(os.path.join(GOLDEN, "scalar_worked_example.json")) as f:
        g = json.load(f)
    x = np.array(g["x"], float).reshape(1, -1, 1, 1)
    L = x.shape[1]
    y, s = orc.ssm_scan(x, np.full((1, L, 1), g["dt"]), np.array([g["A"]]),
                        np.array(g["B"], float).reshape(1, L, 1, 1),
                        np.array(g["C"], float).reshape(1, L, 1, 1),
                        np.array([g["D"]]), np.array(g["S0"], float).reshape(1, 1, 1, 1))
    ln2 = math.log(2.0)
    ref_y = [a * ln2 + b for a, b in g["y_as_a_ln2_plus_b"]]
    a, b = g["S_final_as_a_ln2_plus_b"]
    ref_s = a * ln2 + b
    return max(_rel(y.ravel(), ref_y), _rel(s.ravel(), [ref_s]))


# The step before the path: dt = softplus(dt_raw + dt_bias) against numpy's
# logaddexp and torch's softplus (fp64, across the range where exp overflows
# or underflows), A = -exp(A_log) on exact values, and the hand-worked values
# of tests/golden/dt_a_worked_example.json.
def pin_dt_a(orc):
    import torch
    errs = []
    v = np.concatenate([np.linspace(-40, 40, 161), [-700.0, -30.5, 30.5, 700.0, 745.0]])
    H = v.size
    dt, A = orc.dt_a(v[None, :] - 0.25, np.full(H, 0.25), np.log(np.arange(1, H + 1, dtype=float)))
    ref = np.logaddexp(0.0, v)
    errs.append(float(np.max(np.abs(dt[0] - ref) / np.maximum(ref, 1e-300))))
    ref_t = torch.nn.functional.softplus(torch.from_numpy(v), threshold=700.0).numpy()
    errs.append(float(np.max(np.abs(dt[0] - ref_t) / np.maximum(ref_t, 1e-300))))
    errs.append(_rel(A, -np.arange(1, H + 1, dtype=float)))
    with open(os.path.join(GOLDEN, "dt_a_worked_example.json")) as f:
        g = json.load(f)
    n = len(g["dt_raw"])
    dt, _ = orc.dt_a(np.array(g["dt_raw"])[None, :], np.array(g["dt_bias"]), np.zeros(n))
    errs.append(_rel(dt[0], [math.log(a / b) for a, b in g["dt_as_ln_of"]]))
    _, A = orc.dt_a(np.zeros((1, len(g["A_log"]))), np.zeros(len(g["A_log"])),
                    np.array(g["A_log"]))
    errs.append(_rel(A, g["A"]))
    return max(errs)


def rand_packed(seed, pad=5, **kw):
    """Random packed rows [z | xBC | dt_raw | pad] and the layer's dt_bias,
    A_log; the split below is written out here, independently of the
    oracle's."""
    k = rand_mixer(seed, **kw)
    r = np.random.default_rng(seed + 1000)
    Bn, L = k["xbc"].shape[:2]
    H = k["H"]
    raw = r.standard_normal((Bn, L, H))
    row = np.concatenate([k["z"], k["xbc"], raw, r.standard_normal((Bn, L, pad))], -1)
    k.update(row=row, raw=raw, dt_bias=r.uniform(-3.0, 1.0, H),
             A_log=r.uniform(math.log(0.05), math.log(2.0), H))
    k["dt"] = np.logaddexp(0.0, raw + k["dt_bias"])
    k["A"] = -np.exp(k["A_log"])
    return k


# The packed-row entry points equal the unpacked ones on z, xBC and dt taken
# from the row's three column ranges, with dt = logaddexp(0, raw + bias) and
# A = -exp(A_log) computed here (prefill in two pieces, and decode steps).
def pin_packed(orc):
    k = rand_packed(17, L=19)
    errs = []
    cs, ss = k["conv_in"], k["s_in"]
    full = orc.mixer_prefill(k["xbc"], k["z"], k["dt"], k["A"], k["D"], k["conv_w"], k["conv_b"],
                             k["norm_w"], k["eps"], k["H"], k["P"], k["G"], k["N"],
                             conv_in=cs, s_in=ss)
    outs = []
    for a, b in ((0, 7), (7, 19)):
        r = orc.mixer_prefill_packed(k["row"][:, a:b], k["dt_bias"], k["A_log"], k["D"],
                                     k["conv_w"], k["conv_b"], k["norm_w"], k["eps"], k["H"],
                                     k["P"], k["G"], k["N"], conv_in=cs, s_in=ss)
        cs, ss = r["conv_out"], r["s_out"]
        outs.append(r["out"])
    errs += [_rel(np.concatenate(outs, 1), full["out"]), _rel(cs, full["conv_out"]),
             _rel(ss, full["s_out"])]
    cs, ss, cs2, ss2 = k["conv_in"], k["s_in"], k["conv_in"], k["s_in"]
    for t in range(4):
        o1, cs, ss = orc.decode_step(k["xbc"][:, t], k["z"][:, t], k["dt"][:, t], k["A"], k["D"],
                                     k["conv_w"], k["conv_b"], k["norm_w"], k["eps"], k["H"],
                                     k["P"], k["G"], k["N"], cs, ss)
        o2, cs2, ss2 = orc.decode_step_packed(k["row"][:, t], k["dt_bias"], k["A_log"], k["D"],
                                              k["conv_w"], k["conv_b"], k["norm_w"], k["eps"],
                                              k["H"], k["P"], k["G"], k["N"], cs2, ss2)
        errs += [_rel(o2, o1), _rel(cs2, cs), _rel(ss2, ss)]
    return max(errs)


# Continuous batching over a state pool: ragged sequences packed back to back
# (lengths 5, 1, 13, 0, 2, 1: prefills, decode steps, an empty sequence),
# each on its own slot (out of order, unused slots in between, one fresh
# sequence starting from zeros), equal the per-sequence prefill and decode
# entries called one by one, with unused slots untouched.
def pin_varlen(orc):
    k = rand_mixer(18, Bn=1, L=22)
    r = np.random.default_rng(19)
    H, P, G, N, W = k["H"], k["P"], k["G"], k["N"], k["conv_w"].shape[1]
    C, HP = H * P + 2 * G * N, H * P
    lens = [5, 1, 13, 0, 2, 1]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    slots = np.array([4, 0, 7, 2, 5, 1], dtype=np.int32)
    has = np.array([1, 1, 0, 1, 1, 1], dtype=np.uint8)
    S = 8
    cpool = 0.3 * r.standard_normal((S, W - 1, C))
    spool = 0.3 * r.standard_normal((S, H, P, N))
    xbc, z, dt = k["xbc"][0], k["z"][0], k["dt"][0]
    out, cp, sp = orc.mixer_varlen(cu, slots, has, xbc, z, dt, k["A"], k["D"], k["conv_w"],
                                   k["conv_b"], k["norm_w"], k["eps"], H, P, G, N, cpool, spool)
    errs = []
    cp_ref, sp_ref = cpool.copy(), spool.copy()
    for i, L in enumerate(lens):
        if L == 0:
            continue
        a, s_ = cu[i], slots[i]
        cin = cpool[s_][None] if has[i] else np.zeros((1, W - 1, C))
        sin = spool[s_][None] if has[i] else np.zeros((1, H, P, N))
        if L == 1:
            o, cs, ss = orc.decode_step(xbc[a:a + 1], z[a:a + 1], dt[a:a + 1], k["A"], k["D"],
                                        k["conv_w"], k["conv_b"], k["norm_w"], k["eps"], H, P,
                                        G, N, cin, sin)
            errs.append(_rel(out[a], o[0]))
        else:
            res = orc.mixer_prefill(xbc[None, a:a + L], z[None, a:a + L], dt[None, a:a + L],
                                    k["A"], k["D"], k["conv_w"], k["conv_b"], k["norm_w"],
                                    k["eps"], H, P, G, N, conv_in=cin, s_in=sin)
            errs.append(_rel(out[a:a + L], res["out"][0]))
            cs, ss = res["conv_out"], res["s_out"]
        cp_ref[s_], sp_ref[s_] = cs[0], ss[0]
    errs += [_rel(cp, cp_ref), _rel(sp, sp_ref)]
    untouched = [3, 6]  # slots no sequence uses, and slot 2 (empty sequence)
    errs.append(float(np.max(np.abs(cp[untouched + [2]] - cpool[untouched + [2]]))))
    errs.append(float(np.max(np.abs(sp[untouched + [2]] - spool[untouched + [2]]))))
    return max(errs)


# Backward pass (oracle/backward.py: autograd of a plain torch fp64
# forward). Its forward equals the C oracle's; its gradients equal central
# finite differences of the C oracle's forward, element by element, for every
# input and parameter (the C oracle is a different implementation, so a
# mistake in either shows).
def pin_backward(orc, bwd=None):
    """bwd: the backward oracle module (a planted-mistake copy in the
    mutation tests); the real one by default."""
    if bwd is None:
        from oracle import backward as bwd
    errs = []
    for seed, kw in [(21, dict(L=11)), (22, dict(Bn=1, L=6, H=4, G=1, P=3, N=2, W=2))]:
        k = rand_mixer(seed, **kw)
        args = (k["xbc"], k["z"], k["dt"], k["A"], k["D"], k["conv_w"], k["conv_b"],
                k["norm_w"], k["eps"], k["H"], k["P"], k["G"], k["N"])
        o, s_ = bwd.mixer_forward(*args, conv_in=k["conv_in"], s_in=k["s_in"])
        r = orc.mixer_prefill(*args, conv_in=k["conv_in"], s_in=k["s_in"])
        errs += [_rel(o, r["out"]), _rel(s_, r["s_out"])]
    k = rand_mixer(23, Bn=1, L=7, H=2, P=2, G=1, N=3, W=3)
    rng = np.random.default_rng(24)
    d_out = rng.standard_normal((1, 7, 4))
    d_s = rng.standard_normal((1, 2, 2, 3))
    names = ["xbc", "z", "dt", "A", "D", "conv_w", "conv_b", "norm_w", "conv_in", "s_in"]
    g = bwd.mixer_backward(*(k[n] for n in names[:8]), k["eps"], k["H"], k["P"], k["G"], k["N"],
                           d_out, conv_in=k["conv_in"], s_in=k["s_in"], d_s_out=d_s)

    def loss(kk):
        r = orc.mixer_prefill(kk["xbc"], kk["z"], kk["dt"], kk["A"], kk["D"], kk["conv_w"],
                              kk["conv_b"], kk["norm_w"], kk["eps"], kk["H"], kk["P"], kk["G"],
                              kk["N"], conv_in=kk["conv_in"], s_in=kk["s_in"])
        return float((r["out"] * d_out).sum() + (r["s_out"] * d_s).sum())

    h = 1e-6
    for n in names:
        fd = np.zeros_like(k[n])
        for i in range(k[n].size):
            kp = {**k, n: k[n].copy()}
            km = {**k, n: k[n].copy()}
            kp[n].flat[i] += h
            km[n].flat[i] -= h
            fd.flat[i] = (loss(kp) - loss(km)) / (2 * h)
        errs.append(float(np.max(np.abs(fd - g[n])) / (1.0 + np.max(np.abs(fd)))))
    return max(errs)


PINS = {
    "unrolled": pin_unrolled,
    "chunked": pin_chunked,
    "lfilter": pin_lfilter,
    "prefix_sum": pin_prefix_sum,
    "memoryless": pin_memoryless,
    "conv": pin_conv,
    "norm": pin_norm,
    "decode_is_prefill": pin_decode_is_prefill,
    "piecewise": pin_piecewise,
    "causality": pin_causality,
    "linearity": pin_linearity,
    "composition": pin_composition,
    "worked_example": pin_worked_example,
    "dt_a": pin_dt_a,
    "packed": pin_packed,
    "varlen": pin_varlen,
    "backward": pin_backward,
}

LIMITS = {name: 1e-11 for name in PINS}
LIMITS["backward"] = 1e-7   # central differences with h = 1e-6 (truncation ~h^2, rounding ~1e-10)
LIMITS["causality"] = 0.0
