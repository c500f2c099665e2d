"""Float64 model of the chunkwise WY algorithm (test-only).

This is not the oracle. It is the chunked refactoring that the HIP kernels
implement, written in plain numpy so that the derivation itself can be
checked against the stepwise oracle before (and independently of) any GPU
code. Sources: the chunkwise WY algorithm with channel-wise decay absorbed
into asymmetric erase factors ([WIKI] "Key findings", [ABS]) and the
gate-aware backward ([ABS], [NEWS]); the algebra is written out below.

Per chunk of C tokens entered with state S0 (local index r = 0..C-1):

    g      = inclusive cumulative sum of log_alpha over the chunk     (C x Dk)
    Gam    = exp(g),  GamC = exp(g[C-1])
    Kh     = Gam * b * k          left erase factor (decayed b*k)
    Kt     = k / Gam              right erase factor (inverse-decayed k)
    A      = strict_lower(Kh Kt^T),   T = (I + A)^-1
    W      = T Kh,   Ut = T (w*v),   U = Ut - W S0       (WY factors; U = pseudo-values)
    Qh     = q * Gam,  P = lower_incl(Qh Kt^T)
    O      = Qh S0 + P U
    Kb     = k * exp(g[C-1] - g)
    S_exit = GamC * S0 + Kb^T U

Backward of one chunk, given dO and dS (gradient of the exit state):

    dU   = P^T dO + Kb dS
    dS0  = Qh^T dO + GamC * dS - W^T dU
    dP   = lower_incl(dO U^T);   dQh = dO S0^T + dP Kt;   dKb = U dS^T
    dW   = -dU S0^T;   dT = dW Kh^T + dU (w*v)^T;   d(w*v) = T^T dU
    dA   = strict_lower(-T^T dT T^T)
    dKh  = T^T dW + dA Kt;   dKt = dP^T Qh + dA^T Kh
    dq = dQh*Gam;  db = dKh*Gam*k;  dk = dKh*Gam*b + dKt/Gam + dKb*exp(g[C-1]-g)
    dw = d(w*v)*v;  dv = d(w*v)*w
    dlog_alpha[t] = sum_{s >= t in chunk} (q*dq + 2 b*db - k*dk)[s]
                    + GamC * rowsum(S0 * dS) + colsum_r(Kb * dKb)

The last line uses the invariance of the operator under a rescaling of the
key axis (q/l, l k, b/l^2, S*l): it makes the decay gradient a reverse
cumulative sum inside the chunk plus rowsum(S_exit * dS), and
rowsum(S_exit * dS) = GamC * rowsum(S0 * dS) + colsum_r(Kb * (U dS^T)).
"""

import numpy as np


def _chunk_fwd(S0, q, k, v, la, b, w):
    g = np.cumsum(la, axis=0)
    Gam = np.exp(g)
    gC = g[-1]
    Kh = Gam * b * k
    Kt = k / Gam
    C = q.shape[0]
    A = np.tril(Kh @ Kt.T, -1)
    T = np.linalg.inv(np.eye(C) + A)
    W = T @ Kh
    WV = w * v
    Ut = T @ WV
    U = Ut - W @ S0
    Qh = q * Gam
    P = np.tril(Qh @ Kt.T)
    O = Qh @ S0 + P @ U
    Kb = k * np.exp(gC - g)
    S1 = np.exp(gC)[:, None] * S0 + Kb.T @ U
    cache = dict(g=g, Gam=Gam, gC=gC, Kh=Kh, Kt=Kt, T=T, W=W, WV=WV, U=U, Qh=Qh, P=P, Kb=Kb)
    return O, S1, cache


def forward(q, k, v, la, b, w, S0, C):
    """One (batch, head) pair: q, k, b, la [T, Dk]; v, w [T, Dv]; S0 [Dk, Dv].

    Returns (o [T, Dv], S_T, list of chunk entry states).
    """
    Tn = q.shape[0]
    S = np.array(S0, dtype=np.float64)
    o = np.zeros((Tn, v.shape[1]))
    states = []
    for s in range(0, Tn, C):
        e = min(s + C, Tn)
        states.append(S.copy())
        o[s:e], S, _ = _chunk_fwd(S, q[s:e], k[s:e], v[s:e], la[s:e], b[s:e], w[s:e])
    return o, S, states


def backward(q, k, v, la, b, w, S0, dO, dS_final, C):
    """Chunked gradients for one (batch, head) pair; returns a dict like the oracle's."""
    Tn, Dk = q.shape
    Dv = v.shape[1]
    _, _, states = forward(q, k, v, la, b, w, S0, C)
    dS = np.zeros((Dk, Dv)) if dS_final is None else np.array(dS_final, dtype=np.float64)
    out = {n: np.zeros((Tn, Dk)) for n in ("dq", "dk", "db", "dlog_alpha")}
    out.update({n: np.zeros((Tn, Dv)) for n in ("dv", "dw")})
    for ci in reversed(range(len(states))):
        s = ci * C
        e = min(s + C, Tn)
        S0c = states[ci]
        qq, kk, vv, ll, bb, ww, dd = q[s:e], k[s:e], v[s:e], la[s:e], b[s:e], w[s:e], dO[s:e]
        _, _, c = _chunk_fwd(S0c, qq, kk, vv, ll, bb, ww)
        GamC = np.exp(c["gC"])
        dU = c["P"].T @ dd + c["Kb"] @ dS
        dS0 = c["Qh"].T @ dd + GamC[:, None] * dS - c["W"].T @ dU
        dP = np.tril(dd @ c["U"].T)
        dQh = dd @ S0c.T + dP @ c["Kt"]
        dKb = c["U"] @ dS.T
        dW = -dU @ S0c.T
        dT = dW @ c["Kh"].T + dU @ c["WV"].T
        dWV = c["T"].T @ dU
        dA = np.tril(-c["T"].T @ dT @ c["T"].T, -1)
        dKh = c["T"].T @ dW + dA @ c["Kt"]
        dKt = dP.T @ c["Qh"] + dA.T @ c["Kh"]
        Gam = c["Gam"]
        dq = dQh * Gam
        db = dKh * Gam * kk
        dk = dKh * Gam * bb + dKt / Gam + dKb * np.exp(c["gC"] - c["g"])
        x = qq * dq + 2.0 * bb * db - kk * dk
        exit_term = GamC * np.sum(S0c * dS, axis=1) + np.sum(c["Kb"] * dKb, axis=0)
        dla = np.cumsum(x[::-1], axis=0)[::-1] + exit_term
        out["dq"][s:e], out["dk"][s:e], out["db"][s:e], out["dlog_alpha"][s:e] = dq, dk, db, dla
        out["dw"][s:e], out["dv"][s:e] = dWV * vv, dWV * ww
        dS = dS0
    out["dS0"] = dS
    return out
