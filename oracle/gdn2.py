"""Stepwise float64 oracle: forward, one-token decode and reverse-mode backward.

Test infrastructure only (see the package docstring for who may import it and
for the source tags [README], [WIKI], [NEWS], [ABS]).

Layouts: q, k, b, log_alpha are [B, T, H, Dk]; v, w, dO, o are [B, T, H, Dv];
states are [B, H, Dk, Dv]. Every input is read as stored and widened to
float64 (bf16 and fp32 widen exactly); all arithmetic is float64.

Nothing here is blocked, chunked or reordered: the loop is over tokens, one
recurrence step at a time, vectorised only over the independent (batch, head)
pairs.
"""

import numpy as np


def _f64(x):
    """Widen an array-like (numpy, or a CPU torch tensor of any float dtype) to float64."""
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor: widen in torch so bf16 is read exactly
        import torch

        return x.detach().to(device="cpu", dtype=torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def _step(S, q_t, k_t, v_t, la_t, b_t, w_t):
    """One recurrence step for all (batch, head) pairs at once.

    The update as a fast-weight write ([ABS]): decay the state first (the
    [README] gate list has the erase gate act on the state after decay), read
    it through the erase key e_t = b_t * k_t (the erase gate scales the key-side
    factor of the rank-one erase, [README] update-rule paragraph), take that
    read away from the gated write w_t * v_t (the delta rule removes the
    current read before writing, [ABS]), write the difference along k_t, then
    read out with q_t.

    Expanding (I - k e^T) D S + k (w*v)^T gives exactly D S + k (w*v - (D S)^T e)^T,
    which is what is computed here.

    Shapes: S [n, Dk, Dv]; q_t, k_t, b_t, la_t [n, Dk]; v_t, w_t [n, Dv].
    Returns (S_tilde, u, S_new, o).
    """
    alpha = np.exp(la_t)                               # channel-wise decay on the key axis
    S_tilde = alpha[:, :, None] * S                    # Diag(alpha_t) S_{t-1}
    e = b_t * k_t                                      # erase key b_t * k_t
    read = np.einsum("ncj,nc->nj", S_tilde, e)         # (D S)^T (b * k)
    u = w_t * v_t - read                               # gated write minus gated read
    S_new = S_tilde + k_t[:, :, None] * u[:, None, :]  # rank-one write along k_t
    o = np.einsum("ncj,nc->nj", S_new, q_t)            # o_t = S_t^T q_t
    return S_tilde, u, S_new, o


def _flatten_inputs(q, k, v, log_alpha, b, w):
    q, k, v, la, b, w = (_f64(x) for x in (q, k, v, log_alpha, b, w))
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    for name, x, d in (("k", k, Dk), ("log_alpha", la, Dk), ("b", b, Dk), ("v", v, Dv), ("w", w, Dv)):
        if x.shape != (B, T, H, d):
            raise ValueError(f"{name} has shape {x.shape}, expected {(B, T, H, d)}")

    def bh(x):  # [B,T,H,D] -> [T, B*H, D]
        return np.ascontiguousarray(np.transpose(x, (1, 0, 2, 3)).reshape(T, B * H, x.shape[-1]))

    return (bh(q), bh(k), bh(v), bh(la), bh(b), bh(w)), (B, T, H, Dk, Dv)


def _state_in(S, B, H, Dk, Dv):
    if S is None:
        return np.zeros((B * H, Dk, Dv))
    S = _f64(S)
    if S.shape != (B, H, Dk, Dv):
        raise ValueError(f"state has shape {S.shape}, expected {(B, H, Dk, Dv)}")
    return S.reshape(B * H, Dk, Dv).copy()


def _unflatten(x, B, H):
    # [T, B*H, D] -> [B, T, H, D]
    T, _, D = x.shape
    return np.ascontiguousarray(np.transpose(x.reshape(T, B, H, D), (1, 0, 2, 3)))


def forward(q, k, v, log_alpha, b, w, S0=None):
    """Run the recurrence over all T tokens.

    Returns (o [B,T,H,Dv], S_T [B,H,Dk,Dv]), both float64. S0 = None means a
    zero initial state.
    """
    (q, k, v, la, b, w), (B, T, H, Dk, Dv) = _flatten_inputs(q, k, v, log_alpha, b, w)
    S = _state_in(S0, B, H, Dk, Dv)
    o = np.empty((T, B * H, Dv))
    for t in range(T):
        _, _, S, o[t] = _step(S, q[t], k[t], v[t], la[t], b[t], w[t])
    return _unflatten(o, B, H), S.reshape(B, H, Dk, Dv)


def decode_step(q, k, v, log_alpha, b, w, S):
    """Constant-memory decoding ([ABS], [NEWS]): one token per sequence.

    q, k, b, log_alpha are [B, H, Dk]; v, w are [B, H, Dv]; S is [B, H, Dk, Dv].
    Returns (o [B,H,Dv], S_new [B,H,Dk,Dv]) in float64; S is not modified.
    """
    q, k, v, la, b, w = (_f64(x) for x in (q, k, v, log_alpha, b, w))
    B, H, Dk = q.shape
    Dv = v.shape[-1]
    S = _state_in(S, B, H, Dk, Dv)
    r = lambda x: x.reshape(B * H, -1)  # noqa: E731
    _, _, S_new, o = _step(S, r(q), r(k), r(v), r(la), r(b), r(w))
    return o.reshape(B, H, Dv), S_new.reshape(B, H, Dk, Dv)


def backward(q, k, v, log_alpha, b, w, S0, dO, dS_final=None, checkpoint_every=64):
    """Reverse-mode gradients of L = <dO, o> + <dS_final, S_T>.

    Gradients are taken with respect to the tensors as passed (post-activation
    gates b, w and the log-decay log_alpha). The state path is recomputed from
    checkpoints stored every ``checkpoint_every`` steps, so memory holds
    T/checkpoint_every + checkpoint_every states per (batch, head) pair.

    Reverse of one step (forward: S~ = D S_prev, e = b*k, u = w*v - S~^T e,
    S = S~ + k u^T, o = S^T q), with G the gradient with respect to S_t:
        G    += q dO^T                       (from o = S^T q)
        dq    = S_t dO
        dk    = G u,  du = G^T k             (from S = S~ + k u^T)
        dw    = du * v,  dv = du * w         (from u = w*v - ...)
        G~    = G - e du^T,  de = -S~ du     (from the read S~^T e)
        db    = de * k,  dk += de * b        (from e = b*k)
        dlog_alpha = rowsum(G~ * S~)         (from S~ = exp(log_alpha) * S_prev)
        G     = D G~                         (gradient with respect to S_{t-1})
    and dS0 is G after the first token.

    Returns a dict of float64 arrays: dq, dk, db, dlog_alpha [B,T,H,Dk];
    dv, dw [B,T,H,Dv]; dS0 [B,H,Dk,Dv].
    """
    (q, k, v, la, b, w), (B, T, H, Dk, Dv) = _flatten_inputs(q, k, v, log_alpha, b, w)
    n = B * H
    dO_ = _f64(dO)
    if dO_.shape != (B, T, H, Dv):
        raise ValueError(f"dO has shape {dO_.shape}, expected {(B, T, H, Dv)}")
    dO_ = np.ascontiguousarray(np.transpose(dO_, (1, 0, 2, 3)).reshape(T, n, Dv))
    S = _state_in(S0, B, H, Dk, Dv)
    G = _state_in(dS_final, B, H, Dk, Dv)
    C = max(1, int(checkpoint_every))

    # forward pass keeping the state entering every segment of C tokens
    starts = list(range(0, T, C))
    checkpoints = []
    for s in starts:
        checkpoints.append(S.copy())
        for t in range(s, min(s + C, T)):
            _, _, S, _ = _step(S, q[t], k[t], v[t], la[t], b[t], w[t])

    dq = np.zeros((T, n, Dk))
    dk = np.zeros((T, n, Dk))
    db = np.zeros((T, n, Dk))
    dla = np.zeros((T, n, Dk))
    dv = np.zeros((T, n, Dv))
    dw = np.zeros((T, n, Dv))
    for seg in reversed(range(len(starts))):
        s0, s1 = starts[seg], min(starts[seg] + C, T)
        # recompute the segment, keeping each step's intermediates
        S = checkpoints[seg].copy()
        saved = []
        for t in range(s0, s1):
            S_tilde, u, S, _ = _step(S, q[t], k[t], v[t], la[t], b[t], w[t])
            saved.append((S_tilde, u, S))
        for t in reversed(range(s0, s1)):
            S_tilde, u, S_t = saved[t - s0]
            e = b[t] * k[t]
            G = G + q[t][:, :, None] * dO_[t][:, None, :]
            dq[t] = np.einsum("ncj,nj->nc", S_t, dO_[t])
            dk_t = np.einsum("ncj,nj->nc", G, u)
            du = np.einsum("ncj,nc->nj", G, k[t])
            dw[t] = du * v[t]
            dv[t] = du * w[t]
            G_tilde = G - e[:, :, None] * du[:, None, :]
            de = -np.einsum("ncj,nj->nc", S_tilde, du)
            db[t] = de * k[t]
            dk[t] = dk_t + de * b[t]
            dla[t] = np.einsum("ncj,ncj->nc", G_tilde, S_tilde)
            G = np.exp(la[t])[:, :, None] * G_tilde

    return {
        "dq": _unflatten(dq, B, H),
        "dk": _unflatten(dk, B, H),
        "db": _unflatten(db, B, H),
        "dlog_alpha": _unflatten(dla, B, H),
        "dv": _unflatten(dv, B, H),
        "dw": _unflatten(dw, B, H),
        "dS0": G.reshape(B, H, Dk, Dv),
    }
