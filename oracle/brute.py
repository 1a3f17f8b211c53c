"""O3: brute-force unrolled form of the Mamba-2 scan -- TEST INFRASTRUCTURE ONLY.

Unrolling h_t = a_t h_{t-1} + dt_t B_t x_t^T from h_{-1} = h0 gives

    y_t = sum_{s<=t} (C_t . B_s) (prod_{r=s+1..t} a_r) dt_s x_s
          + (prod_{r=0..t} a_r) h0^T C_t + D x_t,     out_t = y_t * SiLU(z_t),

with a_r = exp(dt_r A) and dt_r = softplus(dt_raw_r + dt_bias). The decay
products are formed by explicit running multiplication (never as the exp of a
sum), so this form shares no step with the chunked form's log-decay
differences. O(L^2) work: tiny inputs only. Pure numpy, float64.
"""
from __future__ import annotations

import numpy as np


def _softplus(v):
    return np.logaddexp(0.0, v)


def _silu(v):
    return v / (1.0 + np.exp(-v))


def ssd_brute(x, Bm, Cm, dt_raw, dt_bias, A, D=None, z=None, h0=None, *, ngroups: int):
    x, Bm, Cm, dt_raw = (np.asarray(a, dtype=np.float64) for a in (x, Bm, Cm, dt_raw))
    dt_bias, A = np.asarray(dt_bias, np.float64), np.asarray(A, np.float64)
    Bsz, L, H = dt_raw.shape
    P = x.shape[2] // H
    N = Bm.shape[2] // ngroups
    hpg = H // ngroups
    y = np.zeros((Bsz, L, H * P))
    for b in range(Bsz):
        for h in range(H):
            g = h // hpg
            dt = _softplus(dt_raw[b, :, h] + dt_bias[h])
            a = np.exp(dt * A[h])
            X = x[b, :, h * P:(h + 1) * P]
            Bg = Bm[b, :, g * N:(g + 1) * N]
            Cg = Cm[b, :, g * N:(g + 1) * N]
            for t in range(L):
                acc = np.zeros(P)
                decay = 1.0           # prod_{r=s+1..t} a_r, built from s = t downwards
                for s in range(t, -1, -1):
                    acc += (Cg[t] @ Bg[s]) * decay * dt[s] * X[s]
                    decay *= a[s]
                if h0 is not None:
                    full = np.prod(a[:t + 1])
                    acc += full * (Cg[t] @ np.asarray(h0[b, h], np.float64))
                if D is not None:
                    acc += D[h] * X[t]
                if z is not None:
                    acc *= _silu(np.asarray(z[b, t, h * P:(h + 1) * P], np.float64))
                y[b, t, h * P:(h + 1) * P] = acc
    return y
