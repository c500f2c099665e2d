"""Shared helpers for the parity tests: device transfer, oracle on sampled (batch, head) pairs."""

import numpy as np
import torch

import oracle

TOL_F32 = 1e-4    # fp32 inputs: max |x - ref| / rms(ref)
TOL_BF16 = 2e-2   # bf16 inputs, fp32 accumulation and state: outputs and states
TOL_GRAD = 5e-2   # bf16 inputs: every gradient


def tol_for(dtype):
    return TOL_F32 if dtype == torch.float32 else TOL_BF16


def rel_err(x, ref):
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = np.sqrt(np.mean(ref * ref))
    d = np.max(np.abs(x - ref)) if x.size else 0.0
    return float(d / rms) if rms > 0 else float(d)


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def to_dev(inp, device="cuda"):
    return {k: (v.to(device) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}


def take_pairs(x, pairs):
    """[B, T, H, D] -> [n, T, 1, D] float64 for the given (b, h) pairs."""
    a = f64(x) if isinstance(x, torch.Tensor) else np.asarray(x, np.float64)
    return np.stack([a[b, :, h] for b, h in pairs])[:, :, None, :]


def take_state_pairs(S, pairs):
    """[B, H, Dk, Dv] -> [n, 1, Dk, Dv] float64."""
    a = f64(S) if isinstance(S, torch.Tensor) else np.asarray(S, np.float64)
    return np.stack([a[b, h] for b, h in pairs])[:, None]


def oracle_fwd_pairs(inp, pairs):
    """Oracle forward on the sampled pairs; returns (o [n,T,Dv], S_T [n,Dk,Dv])."""
    args = [take_pairs(inp[n], pairs) for n in ("q", "k", "v", "log_alpha", "b", "w")]
    S0 = take_state_pairs(inp["S0"], pairs) if inp.get("S0") is not None else None
    o, S = oracle.forward(*args, S0)
    return o[:, :, 0], S[:, 0]


def gpu_pairs(x, pairs):
    """GPU output [B, T, H, D] -> [n, T, D] float64 for the pairs."""
    a = f64(x)
    return np.stack([a[b, :, h] for b, h in pairs])


def gpu_state_pairs(S, pairs):
    a = f64(S)
    return np.stack([a[b, h] for b, h in pairs])
