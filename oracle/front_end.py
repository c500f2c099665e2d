"""Float64 oracle of the fused gate front end (pre-activation gates).

Test infrastructure only (see the package docstring for who may import it).

The pages leave the gate parametrisation open: [README] describes an erase gate
b and a write gate w with values in [0, 1] (the gate bullet list) and a
channel-wise decay alpha in (0, 1), and says nothing about how they are
produced. The workloads draw them as b = sigmoid(x), w = sigmoid(y) and
log_alpha = -softplus(z), which is the reading taken here: the operator may be
handed the pre-activations x, y, z ("raw" gates) and applies

    b = sigmoid(b_raw),  w = sigmoid(w_raw),  log_alpha = -softplus(a_raw) = -log(1 + exp(a_raw)).

Gradients with respect to the raw inputs follow by the chain rule from the
gradients with respect to the activated gates:

    d b_raw = d b * b (1 - b),   d w_raw = d w * w (1 - w),   d a_raw = -d log_alpha * sigmoid(a_raw).

Everything else is the stepwise recurrence of ``oracle.gdn2``.
"""

import numpy as np

from .gdn2 import _f64, backward, decode_step, forward


def _sigmoid(x):
    # 1 / (1 + exp(-x)) written as (1 + tanh(x / 2)) / 2, which never overflows
    return 0.5 * (1.0 + np.tanh(0.5 * x))


def gates_from_raw(b_raw, w_raw, a_raw):
    """(b, w, log_alpha) from the pre-activations, float64."""
    b_raw, w_raw, a_raw = _f64(b_raw), _f64(w_raw), _f64(a_raw)
    return _sigmoid(b_raw), _sigmoid(w_raw), -np.logaddexp(0.0, a_raw)


def forward_raw(q, k, v, a_raw, b_raw, w_raw, S0=None):
    """forward() with pre-activation gates (argument order of forward: the decay input first)."""
    b, w, la = gates_from_raw(b_raw, w_raw, a_raw)
    return forward(q, k, v, la, b, w, S0)


def decode_step_raw(q, k, v, a_raw, b_raw, w_raw, S):
    """decode_step() with pre-activation gates."""
    b, w, la = gates_from_raw(b_raw, w_raw, a_raw)
    return decode_step(q, k, v, la, b, w, S)


def backward_raw(q, k, v, a_raw, b_raw, w_raw, S0, dO, dS_final=None, checkpoint_every=64):
    """backward() with pre-activation gates: db, dw and dlog_alpha are the gradients with respect to
    b_raw, w_raw and a_raw (the other gradients are unchanged)."""
    b, w, la = gates_from_raw(b_raw, w_raw, a_raw)
    g = backward(q, k, v, la, b, w, S0, dO, dS_final, checkpoint_every)
    g["db"] = g["db"] * b * (1.0 - b)
    g["dw"] = g["dw"] * w * (1.0 - w)
    g["dlog_alpha"] = -g["dlog_alpha"] * _sigmoid(_f64(a_raw))
    return g
