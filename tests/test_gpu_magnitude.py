"""GPU parity at input magnitudes far from one: the bf16 path's fp16 matrix-core operands.

bf16 inputs carry fp32's exponent range, while fp16 operands hold normal numbers only between 6.1e-5 and
65504. The forward is linear in (v, S0) jointly and the backward in (dO, dS_final) jointly (exact identity
F2 of the recurrence), so scaling them by a power of two must scale o, S_final or every gradient by the same
power and leave the error against the float64 oracle, relative to the output's RMS, unchanged. The
upstream gradients of a mean-reduced training loss are small (1e-6 .. 1e-8 per element), which is the case
the backward's power-of-two prescale of dO and dS_final exists for.
"""

import numpy as np
import pytest
import torch

import oracle
import synth
from delta_rule_recurrent_gdn_amd import (gdn2_bwd_chunked, gdn2_bwd_chunked_records, gdn2_bwd_varlen_records,
                                          gdn2_fwd_chunked, gdn2_fwd_chunked_train, gdn2_fwd_varlen_train)
from tests.helpers import TOL_BF16, TOL_F32, TOL_GRAD, f64, rel_err, to_dev

pytestmark = pytest.mark.gpu
GRADS = ("dq", "dk", "dv", "dlog_alpha", "db", "dw", "dS0")


def scaled(inp, names, f):
    out = dict(inp)
    for n in names:
        out[n] = (inp[n].to(torch.float32) * f).to(inp[n].dtype)  # a power of two: exact in bf16 and fp32
    return out


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("f", [2.0 ** 12, 2.0 ** -12])
def test_forward_value_scale(dtype, f):
    """v and S0 times 2^+-12 (d = 128, chunk 64, two-stage and single-pass and the training forward)."""
    C, T = 64, 3 * 64 + 5
    inp = scaled(synth.make_inputs(2, T, 2, 128, 128, dtype, seed=31, s0_std=0.3), ("v", "S0"), f)
    o_ref, S_ref = oracle.forward(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["b"], inp["w"], inp["S0"])
    d = to_dev(inp)
    x = (d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"])
    tol = TOL_F32 if dtype == "fp32" else TOL_BF16
    outs = {}
    for single in (False, True):
        o, S, _ = gdn2_fwd_chunked(*x, d["S0"], chunk=C, single_pass=single)
        outs["single" if single else "two-stage"] = (o, S)
    o, S, _ = gdn2_fwd_chunked_train(*x, d["S0"], chunk=C)
    outs["training"] = (o, S)
    torch.cuda.synchronize()
    for what, (o, S) in outs.items():
        e_o, e_s = rel_err(f64(o), o_ref), rel_err(f64(S), S_ref)
        print(f"{what} {dtype} x{f:g}: o {e_o:.2e} S {e_s:.2e}")
        assert e_o <= tol and e_s <= tol, (what, e_o, e_s)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("f", [2.0 ** 12, 2.0 ** -12, 1e-7, 1e-3])
def test_backward_upstream_scale(dtype, f):
    """dO and dS_final times f (2^+-12, 1e-7, 1e-3): all seven gradients, separate backward and training pair."""
    D, C = 128, 64
    T = 2 * C + 7
    base = synth.make_inputs(1, T, 3, D, D, dtype, seed=41, s0_std=0.3, grad=True)
    inp = dict(base)
    inp["dO"] = (base["dO"].to(torch.float32) * f).to(base["dO"].dtype)
    dS = torch.from_numpy((f * np.random.default_rng(42).standard_normal((1, 3, D, D))).astype(np.float32))
    ref = oracle.backward(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["b"], inp["w"], inp["S0"], inp["dO"],
                          dS)
    d = to_dev(inp)
    x = (d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"])
    tol = TOL_F32 if dtype == "fp32" else TOL_GRAD
    g1 = gdn2_bwd_chunked(*x, d["dO"], S0=d["S0"], dS_final=dS.cuda(), chunk=C)
    _, _, rec = gdn2_fwd_chunked_train(*x, d["S0"], chunk=C)
    g2 = gdn2_bwd_chunked_records(*x, d["dO"], rec, dS_final=dS.cuda(), chunk=C)
    torch.cuda.synchronize()
    for what, g in (("separate", g1), ("pair", g2)):
        for n in GRADS:
            e = rel_err(f64(g[n]), ref[n])
            print(f"{what} {dtype} x{f:g}: {n} {e:.2e}")
            assert np.isfinite(f64(g[n])).all() and e <= tol, (what, n, e)


def test_packed_backward_small_upstream():
    """A packed batch (lengths 100, 0, 61, 130) with dO and dS_final of order 1e-7, through the training pair."""
    lens = [100, 0, 61, 130]
    T, H, D, C = sum(lens), 2, 64, 32
    inp = synth.make_inputs(1, T, H, D, D, "bf16", seed=51, grad=True)
    inp["dO"] = (inp["dO"].to(torch.float32) * 1e-7).to(torch.bfloat16)
    rng = np.random.default_rng(52)
    S0 = torch.from_numpy((0.3 * rng.standard_normal((len(lens), H, D, D))).astype(np.float32))
    dS = torch.from_numpy((1e-7 * rng.standard_normal((len(lens), H, D, D))).astype(np.float32))
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int64)
    d = to_dev(inp)
    x = (d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"])
    _, _, rec = gdn2_fwd_varlen_train(*x, cu.cuda(), S0=S0.cuda(), chunk=C)
    g = gdn2_bwd_varlen_records(*x, d["dO"], cu.cuda(), rec, dS_final=dS.cuda(), chunk=C)
    torch.cuda.synchronize()
    ref = oracle.backward_varlen(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["b"], inp["w"], cu, S0,
                                 inp["dO"], dS)
    for n in GRADS:
        e = rel_err(f64(g[n]), ref[n])
        print(f"packed x1e-7: {n} {e:.2e}")
        assert np.isfinite(f64(g[n])).all() and e <= TOL_GRAD, (n, e)
