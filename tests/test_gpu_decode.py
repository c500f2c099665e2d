"""GPU parity of gdn2_decode_step against the float64 oracle (through the C ABI)."""

import numpy as np
import pytest
import torch

import oracle
import synth
from delta_rule_recurrent_gdn_amd import gdn2_decode_step, gdn2_fwd_chunked
from tests.helpers import TOL_BF16, TOL_F32, f64, rel_err, tol_for

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("Dk,Dv", [(16, 16), (16, 128), (128, 16), (32, 64), (64, 32), (128, 128)])
def test_decode_small(dtype, Dk, Dv):
    B, H, steps = 3, 5, 3
    inp = synth.make_decode_inputs(B, H, Dk, Dv, steps, dtype, seed=Dk + Dv, s0_std=0.3)
    S = inp["S0"].to(DEV).clone()
    S_ref = f64(inp["S0"])
    for t in range(steps):
        x = {n: inp[n][t].to(DEV).contiguous() for n in ("q", "k", "v", "log_alpha", "b", "w")}
        o = gdn2_decode_step(x["q"], x["k"], x["v"], x["log_alpha"], x["b"], x["w"], S)
        o_ref, S_ref = oracle.decode_step(*(inp[n][t] for n in ("q", "k", "v", "log_alpha", "b", "w")), S_ref)
        torch.cuda.synchronize()
        tol = tol_for(synth.torch_dtype(dtype))
        assert rel_err(f64(o), o_ref) <= tol
        assert rel_err(f64(S), S_ref) <= tol


def test_decode_B256_H16_128_steps_sampled():
    """B=256, H=16, d=128, fp32 state ~ 0.02 N(0,1), 128 consecutive steps; the oracle follows
    a sample of sequences through all steps (every head of each sampled sequence)."""
    c = synth.WORKLOADS["decode-B256-H16-d128-128steps"]
    inp = synth.workload_inputs("decode-B256-H16-d128-128steps")
    dev = {n: inp[n].to(DEV) for n in inp}
    S = dev["S0"].clone()
    seqs = [0, 77, 255]
    o_gpu = []
    for t in range(c["steps"]):
        o = gdn2_decode_step(dev["q"][t], dev["k"][t], dev["v"][t], dev["log_alpha"][t], dev["b"][t], dev["w"][t], S)
        o_gpu.append(o[seqs].cpu())
    torch.cuda.synchronize()
    S_ref = f64(inp["S0"][seqs])
    errs = []
    for t in range(c["steps"]):
        args = [inp[n][t][seqs] for n in ("q", "k", "v", "log_alpha", "b", "w")]
        o_ref, S_ref = oracle.decode_step(*args, S_ref)
        errs.append(rel_err(f64(o_gpu[t]), o_ref))
    es = rel_err(f64(S[seqs]), S_ref)
    print(f"decode B256 H16 max err o {max(errs):.3e} S {es:.3e}")
    assert max(errs) <= TOL_BF16 and es <= TOL_BF16


def test_decode_steps_equal_chunked_forward():
    """N decode steps on the GPU equal one chunked forward over those N tokens."""
    B, H, D, N = 4, 8, 128, 40
    inp = synth.make_inputs(B, N, H, D, D, "bf16", seed=21, s0_std=0.05)
    d = {k: v.to(DEV) for k, v in inp.items()}
    o_f, S_f, _ = gdn2_fwd_chunked(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], d["S0"], chunk=16)
    S = d["S0"].clone()
    outs = []
    for t in range(N):
        x = {n: d[n][:, t].contiguous() for n in ("q", "k", "v", "log_alpha", "b", "w")}
        outs.append(gdn2_decode_step(x["q"], x["k"], x["v"], x["log_alpha"], x["b"], x["w"], S))
    torch.cuda.synchronize()
    o_d = torch.stack(outs, dim=1)
    # decode is fp32 throughout; the bf16-input chunked path uses fp16 matrix-core
    # operands, so the two agree to that path's tolerance, not to fp32 rounding
    assert rel_err(f64(o_d), f64(o_f)) < TOL_BF16 and rel_err(f64(S), f64(S_f)) < TOL_BF16


def test_decode_fp32_exactness_at_full_head():
    inp = synth.make_decode_inputs(8, 16, 128, 128, 2, "fp32", seed=22, s0_std=0.02)
    S = inp["S0"].to(DEV).clone()
    S_ref = f64(inp["S0"])
    for t in range(2):
        x = {n: inp[n][t].to(DEV) for n in ("q", "k", "v", "log_alpha", "b", "w")}
        o = gdn2_decode_step(x["q"], x["k"], x["v"], x["log_alpha"], x["b"], x["w"], S)
        o_ref, S_ref = oracle.decode_step(*(inp[n][t] for n in ("q", "k", "v", "log_alpha", "b", "w")), S_ref)
    torch.cuda.synchronize()
    assert rel_err(f64(o), o_ref) <= TOL_F32 and rel_err(f64(S), S_ref) <= TOL_F32
    assert np.isfinite(f64(S)).all()
