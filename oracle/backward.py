"""fp64 CPU oracle for the backward pass of the Mamba-2 mixer core — TEST
INFRASTRUCTURE ONLY (imported by the tests, the smoke check and the
benchmark's CPU leg; never by the product path).

The gradients are those of the plain forward: the same conv + SiLU, split,
sequential recurrence and gated norm as ``ssd_oracle.c``, written here as
plain torch fp64 CPU tensor operations (a loop over tokens for the
recurrence) and differentiated by torch's reverse-mode autograd. The
training use is the one "feat(model): add Nemotron-3 Nano hybrid ..." names
(Modalities PR #459, section "Testing": gradient flow through the mixer;
"Caveats": the native pure-PyTorch backend is activation-memory hungry).

Pinned (tests/pins.py): this forward equals the C oracle's forward, and its
gradients equal central finite differences of the C oracle's forward (an
evaluation of a different implementation), for every input and parameter.
"""
from __future__ import annotations

import numpy as np
import torch


def _t(a, req=False):
    if a is None:
        return None
    t = torch.tensor(np.asarray(a, dtype=np.float64), dtype=torch.float64)
    if req:
        t.requires_grad_(True)
    return t


def forward(xbc, z, dt, A, D, conv_w, conv_b, norm_w, eps, H, P, G, N, conv_in=None,
            s_in=None):
    """The mixer prefill (torch fp64 tensors): returns (out, s_out)."""
    Bn, L, C = xbc.shape
    W = conv_w.shape[1]
    HP, GN = H * P, G * N
    ext = torch.cat([conv_in if conv_in is not None else torch.zeros(Bn, W - 1, C,
                                                                       dtype=xbc.dtype),
                     xbc], dim=1)
    u = sum(conv_w[:, k] * ext[:, k:k + L] for k in range(W))
    if conv_b is not None:
        u = u + conv_b
    v = u * torch.sigmoid(u)
    x = v[..., :HP].reshape(Bn, L, H, P)
    Bm = v[..., HP:HP + GN].reshape(Bn, L, G, N)
    Cm = v[..., HP + GN:].reshape(Bn, L, G, N)
    hpg = H // G
    Bh = Bm.repeat_interleave(hpg, dim=2)   # head h reads group h // (H/G)
    Ch = Cm.repeat_interleave(hpg, dim=2)
    S = s_in if s_in is not None else torch.zeros(Bn, H, P, N, dtype=xbc.dtype)
    ys = []
    for t in range(L):
        a = torch.exp(dt[:, t] * A)                                  # [B, H]
        S = a[:, :, None, None] * S + (dt[:, t, :, None, None] * x[:, t, :, :, None]
                                       * Bh[:, t, :, None, :])
        ys.append((S * Ch[:, t, :, None, :]).sum(-1) + D[:, None] * x[:, t])
    y = torch.stack(ys, 1).reshape(Bn, L, HP)
    q = y * z * torch.sigmoid(z)
    Sg = HP // G
    qg = q.reshape(Bn, L, G, Sg)
    r = torch.rsqrt((qg * qg).mean(-1, keepdim=True) + eps)
    out = (qg * r).reshape(Bn, L, HP) * norm_w
    return out, S


def mixer_backward(xbc, z, dt, A, D, conv_w, conv_b, norm_w, eps, H, P, G, N, d_out,
                   conv_in=None, s_in=None, d_s_out=None):
    """Gradients of sum(out * d_out) (+ sum(s_out * d_s_out)) with respect to
    every input and parameter. Returns a dict of fp64 numpy arrays: xbc, z,
    dt, A, D, conv_w, conv_b (when given), norm_w, conv_in and s_in (when
    given)."""
    names = ["xbc", "z", "dt", "A", "D", "conv_w", "conv_b", "norm_w", "conv_in", "s_in"]
    vals = [xbc, z, dt, A, D, conv_w, conv_b, norm_w, conv_in, s_in]
    ts = {n: _t(v, req=True) for n, v in zip(names, vals)}
    out, s_out = forward(ts["xbc"], ts["z"], ts["dt"], ts["A"], ts["D"], ts["conv_w"],
                         ts["conv_b"], ts["norm_w"], float(eps), H, P, G, N, ts["conv_in"],
                         ts["s_in"])
    loss = (out * _t(d_out)).sum()
    if d_s_out is not None:
        loss = loss + (s_out * _t(d_s_out)).sum()
    live = [n for n in names if ts[n] is not None]
    grads = torch.autograd.grad(loss, [ts[n] for n in live])
    return {n: g.numpy() for n, g in zip(live, grads)}


def mixer_forward(xbc, z, dt, A, D, conv_w, conv_b, norm_w, eps, H, P, G, N, conv_in=None,
                  s_in=None):
    """The same forward on numpy inputs (for the pins): (out, s_out)."""
    with torch.no_grad():
        out, s = forward(_t(xbc), _t(z), _t(dt), _t(A), _t(D), _t(conv_w), _t(conv_b),
                         _t(norm_w), float(eps), H, P, G, N, _t(conv_in), _t(s_in))
    return out.numpy(), s.numpy()
