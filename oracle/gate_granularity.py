"""Float64 oracle of the gate-granularity variants: per-head scalar gates.

Test infrastructure only (see the package docstring for who may import it).

[README] (gate bullet list) and [ABS] present the erase gate b, the write gate
w and the decay alpha as channel-wise, and state that the model reduces to
KDA and to Gated DeltaNet when they collapse: one scalar beta per token and
head for both gates (KDA), and a scalar decay as well (Gated DeltaNet). A
gate given as one value per (token, head) ([B, T, H]) therefore means that
value on every channel; written here as that definition (a broadcast onto the
channels, then the recurrence of ``oracle.gdn2``). The gradient of such a
gate is the sum over the channels it was broadcast to.
"""

import numpy as np

from .front_end import gates_from_raw
from .gdn2 import _f64, backward, forward


def _expand(x, D, scalar):
    x = _f64(x)
    return np.repeat(x[..., None], D, axis=-1) if scalar else x


def forward_gates(q, k, v, log_alpha, b, w, S0=None, scalar_b=False, scalar_w=False, scalar_decay=False,
                  raw=False):
    """forward() with any of b, w, log_alpha given per (token, head); raw: pre-activation gates."""
    Dk, Dv = _f64(q).shape[-1], _f64(v).shape[-1]
    b, w, la = _expand(b, Dk, scalar_b), _expand(w, Dv, scalar_w), _expand(log_alpha, Dk, scalar_decay)
    if raw:
        b, w, la = gates_from_raw(b, w, la)
    return forward(q, k, v, la, b, w, S0)


def backward_gates(q, k, v, log_alpha, b, w, S0, dO, dS_final=None, scalar_b=False, scalar_w=False,
                   scalar_decay=False, raw=False, checkpoint_every=64):
    """backward() for forward_gates: a scalar gate's gradient is the channel sum of the broadcast one."""
    Dk, Dv = _f64(q).shape[-1], _f64(v).shape[-1]
    b_raw, w_raw, a_raw = _expand(b, Dk, scalar_b), _expand(w, Dv, scalar_w), _expand(log_alpha, Dk, scalar_decay)
    if raw:
        bb, ww, la = gates_from_raw(b_raw, w_raw, a_raw)
    else:
        bb, ww, la = b_raw, w_raw, a_raw
    g = backward(q, k, v, la, bb, ww, S0, dO, dS_final, checkpoint_every)
    if raw:
        g["db"] = g["db"] * bb * (1.0 - bb)
        g["dw"] = g["dw"] * ww * (1.0 - ww)
        g["dlog_alpha"] = -g["dlog_alpha"] * 0.5 * (1.0 + np.tanh(0.5 * a_raw))
    if scalar_b:
        g["db"] = g["db"].sum(axis=-1)
    if scalar_w:
        g["dw"] = g["dw"].sum(axis=-1)
    if scalar_decay:
        g["dlog_alpha"] = g["dlog_alpha"].sum(axis=-1)
    return g
