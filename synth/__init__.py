"""Seeded synthetic inputs for the Gated Delta Rule-2 operator.

Shared by the tests, the benchmark and the oracle checks. This module holds no
part of the operator's arithmetic: it only draws random tensors with the
workload's shapes and value distributions and rounds them to the storage
dtype. It imports neither the oracle nor the HIP package.

Recipe (numpy PCG64 ``default_rng(seed)``, float32 normal draws, drawn in the
order q, k, v, b, w, log_alpha, S0, dO):

* q, k ~ N(0, 1), each L2-normalised over the feature axis per (b, t, h), in fp32;
* v ~ N(0, 1);
* b, w = sigmoid(N(0, 1))                 (erase gate, write gate; post-activation);
* log_alpha = -softplus(N(-2, 1)) = -log1p(exp(x)), kept in fp32 (decay in (0, 1));
* S0 = s0_std * N(0, 1) in fp32 when requested, else zeros;
* dO ~ N(0, 1) when requested;
* q, k, v, b, w, dO are then rounded to the storage dtype (bf16 by
  round-to-nearest-even through torch's CPU cast, or kept fp32).

Layouts: q, k, b, log_alpha [B, T, H, Dk]; v, w, dO [B, T, H, Dv]; S0 [B, H, Dk, Dv].
"""

import numpy as np
import torch

# The five workloads, by name. Shapes follow the pages' layer (16 heads,
# d_k = d_v = 128, sequence length 4K) plus a tiny fp32 case, a long-sequence
# sweep and a decode batch.
WORKLOADS = {
    "tiny-fp32-fwd": dict(B=1, H=2, T=64, Dk=16, Dv=16, chunk=16, dtype="fp32", seed=0, s0_std=None, grad=False),
    "fwd-B8-H16-T4096-d128": dict(B=8, H=16, T=4096, Dk=128, Dv=128, chunk=64, dtype="bf16", seed=1,
                                  s0_std=None, grad=False),
    "fwd-long-B1-H16-d128": dict(B=1, H=16, T=(8192, 16384, 32768, 65536), Dk=128, Dv=128, chunk=64,
                                 dtype="bf16", seed=2, s0_std=0.02, grad=False),
    "decode-B256-H16-d128-128steps": dict(B=256, H=16, Dk=128, Dv=128, steps=128, dtype="bf16", seed=3,
                                          s0_std=0.02),
    "fwd+bwd-B8-H16-T4096-d128": dict(B=8, H=16, T=4096, Dk=128, Dv=128, chunk=64, dtype="bf16", seed=4,
                                      s0_std=None, grad=True),
}


_TORCH_DTYPES = {"fp32": torch.float32, "bf16": torch.bfloat16}


def torch_dtype(name):
    return _TORCH_DTYPES[name]


def _normal(rng, shape, mean=0.0):
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if mean:
        x += np.float32(mean)
    return x


def _l2n(x):
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True, dtype=np.float32))


def _sigmoid(x):
    return (np.float32(1.0) / (np.float32(1.0) + np.exp(-x))).astype(np.float32)


def _neg_softplus(x):
    return (-np.log1p(np.exp(x))).astype(np.float32)


def _cast(x, dtype):
    return torch.from_numpy(np.ascontiguousarray(x)).to(_TORCH_DTYPES[dtype])


def make_inputs(B, T, H, Dk, Dv, dtype="bf16", seed=0, s0_std=None, grad=False, raw_gates=False):
    """Draw one batch of sequence inputs. Returns a dict of CPU torch tensors.

    Keys: q, k, v, b, w (storage dtype), log_alpha (fp32), S0 (fp32 or None),
    dO (storage dtype, only when ``grad``). With ``raw_gates`` the same draws
    are returned before their activations: b, w are the normal draws (storage
    dtype) and log_alpha the N(-2, 1) draw (fp32).
    """
    rng = np.random.default_rng(seed)
    q = _l2n(_normal(rng, (B, T, H, Dk)))
    k = _l2n(_normal(rng, (B, T, H, Dk)))
    v = _normal(rng, (B, T, H, Dv))
    act = (lambda f, x: x) if raw_gates else (lambda f, x: f(x))  # noqa: E731
    b = act(_sigmoid, _normal(rng, (B, T, H, Dk)))
    w = act(_sigmoid, _normal(rng, (B, T, H, Dv)))
    la = act(_neg_softplus, _normal(rng, (B, T, H, Dk), mean=-2.0))
    out = dict(q=_cast(q, dtype), k=_cast(k, dtype), v=_cast(v, dtype), b=_cast(b, dtype),
               w=_cast(w, dtype), log_alpha=torch.from_numpy(la))
    out["S0"] = (torch.from_numpy(np.float32(s0_std) * _normal(rng, (B, H, Dk, Dv)))
                 if s0_std is not None else None)
    if grad:
        out["dO"] = _cast(_normal(rng, (B, T, H, Dv)), dtype)
    return out


def make_decode_inputs(B, H, Dk, Dv, steps, dtype="bf16", seed=3, s0_std=0.02, raw_gates=False):
    """Inputs for ``steps`` consecutive one-token decode steps.

    Each per-token input is one draw of shape [steps, B, H, D] (same
    distributions as ``make_inputs``, ``raw_gates`` as there); the state is
    [B, H, Dk, Dv] fp32.
    """
    rng = np.random.default_rng(seed)
    q = _l2n(_normal(rng, (steps, B, H, Dk)))
    k = _l2n(_normal(rng, (steps, B, H, Dk)))
    v = _normal(rng, (steps, B, H, Dv))
    act = (lambda f, x: x) if raw_gates else (lambda f, x: f(x))  # noqa: E731
    b = act(_sigmoid, _normal(rng, (steps, B, H, Dk)))
    w = act(_sigmoid, _normal(rng, (steps, B, H, Dv)))
    la = act(_neg_softplus, _normal(rng, (steps, B, H, Dk), mean=-2.0))
    S0 = np.float32(s0_std) * _normal(rng, (B, H, Dk, Dv))
    return dict(q=_cast(q, dtype), k=_cast(k, dtype), v=_cast(v, dtype), b=_cast(b, dtype),
                w=_cast(w, dtype), log_alpha=torch.from_numpy(la), S0=torch.from_numpy(S0))


def workload_inputs(name, T=None):
    """Inputs of one of the named workloads (the long-sequence sweep takes its sequence length T)."""
    c = WORKLOADS[name]
    if "steps" in c:
        return make_decode_inputs(c["B"], c["H"], c["Dk"], c["Dv"], c["steps"], c["dtype"], c["seed"],
                                  c["s0_std"])
    if isinstance(c["T"], tuple):
        if T is None:
            raise ValueError(f"{name} needs the sequence length T")
    else:
        T = c["T"]
    return make_inputs(c["B"], T, c["H"], c["Dk"], c["Dv"], c["dtype"], c["seed"], c["s0_std"], c["grad"])


def rel_err(x, ref):
    """max |x - ref| / rms(ref), over all elements (the parity metric)."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = np.sqrt(np.mean(ref * ref))
    if rms == 0.0:
        return float(np.max(np.abs(x - ref))) if x.size else 0.0
    return float(np.max(np.abs(x - ref)) / rms)
