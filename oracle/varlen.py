"""Float64 oracle of packed variable-length batches.

Test infrastructure only (see the package docstring for who may import it).

A packed batch is N independent sequences laid end to end along T of a
[1, T, H, D] layout: sequence n is tokens cu[n] .. cu[n+1]-1 and runs the
recurrence of ``oracle.gdn2`` from its own entry state S0[n]. The pages
train with 0.5M-token batches at sequence length 4K ([README] training-setup
list; [NEWS] training paragraph) and decode with a constant-size state per
sequence ([ABS]); they say nothing about how documents are cut into or
packed along those sequences, so the plainest reading is taken: no state
crosses a boundary. Written as that definition: a loop over the sequences,
each one through ``forward`` / ``backward`` / ``decode_step`` on its own slice.
"""

import numpy as np

from .gdn2 import _f64, backward, decode_step, forward


def _slices(cu, T):
    cu = [int(x) for x in np.asarray(cu).reshape(-1)]
    for n in range(len(cu) - 1):
        if not 0 <= cu[n] <= cu[n + 1] <= T:
            raise ValueError("cu_seqlens must be non-decreasing within [0, T]")
    return [(cu[n], cu[n + 1]) for n in range(len(cu) - 1)]


def forward_varlen(q, k, v, log_alpha, b, w, cu_seqlens, S0=None):
    """o [1,T,H,Dv] (zeros outside every sequence) and S_final [N,H,Dk,Dv]."""
    q, k, v, la, b, w = (_f64(x) for x in (q, k, v, log_alpha, b, w))
    _, T, H, Dk = q.shape
    Dv = v.shape[-1]
    sl = _slices(cu_seqlens, T)
    S0 = None if S0 is None else _f64(S0)
    o = np.zeros((1, T, H, Dv))
    S_final = np.zeros((len(sl), H, Dk, Dv))
    for n, (a, e) in enumerate(sl):
        s0 = None if S0 is None else S0[n:n + 1]
        if e == a:
            S_final[n] = 0.0 if s0 is None else s0[0]
            continue
        on, Sn = forward(q[:, a:e], k[:, a:e], v[:, a:e], la[:, a:e], b[:, a:e], w[:, a:e], s0)
        o[:, a:e] = on
        S_final[n] = Sn[0]
    return o, S_final


def backward_varlen(q, k, v, log_alpha, b, w, cu_seqlens, S0, dO, dS_final=None, checkpoint_every=64):
    """Gradients of L = <dO, o> + <dS_final, S_final> for a packed batch: per-token gradients
    [1,T,H,D] (zero outside every sequence) and dS0 [N,H,Dk,Dv]."""
    q, k, v, la, b, w, dO = (_f64(x) for x in (q, k, v, log_alpha, b, w, dO))
    _, T, H, Dk = q.shape
    Dv = v.shape[-1]
    sl = _slices(cu_seqlens, T)
    S0 = None if S0 is None else _f64(S0)
    dSf = None if dS_final is None else _f64(dS_final)
    out = {n: np.zeros((1, T, H, Dk)) for n in ("dq", "dk", "db", "dlog_alpha")}
    out.update({n: np.zeros((1, T, H, Dv)) for n in ("dv", "dw")})
    out["dS0"] = np.zeros((len(sl), H, Dk, Dv))
    for n, (a, e) in enumerate(sl):
        s0 = None if S0 is None else S0[n:n + 1]
        ds = None if dSf is None else dSf[n:n + 1]
        if e == a:
            out["dS0"][n] = 0.0 if ds is None else ds[0]
            continue
        g = backward(q[:, a:e], k[:, a:e], v[:, a:e], la[:, a:e], b[:, a:e], w[:, a:e], s0, dO[:, a:e], ds,
                     checkpoint_every)
        for name in ("dq", "dk", "db", "dlog_alpha", "dv", "dw"):
            out[name][:, a:e] = g[name]
        out["dS0"][n] = g["dS0"][0]
    return out


def decode_step_slots(q, k, v, log_alpha, b, w, S_pool, slots):
    """One decode step of B entries whose states are S_pool[slots[b]]; returns (o [B,H,Dv], new pool).
    An entry with a slot outside the pool gets o = 0 and changes nothing."""
    q, k, v, la, b, w = (_f64(x) for x in (q, k, v, log_alpha, b, w))
    pool = _f64(S_pool).copy()
    B, H, _ = q.shape
    o = np.zeros((B, H, v.shape[-1]))
    for i, s in enumerate(int(x) for x in np.asarray(slots).reshape(-1)):
        if not 0 <= s < pool.shape[0]:
            continue
        oi, Si = decode_step(q[i:i + 1], k[i:i + 1], v[i:i + 1], la[i:i + 1], b[i:i + 1], w[i:i + 1],
                             pool[s:s + 1])
        o[i] = oi[0]
        pool[s] = Si[0]
    return o, pool
