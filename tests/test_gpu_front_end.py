"""GPU parity of the fused gate front end (GDN2_FLAG_RAW_GATES): b, w and log_alpha passed as
pre-activations, activated inside the kernels, gradients with respect to the pre-activations; against
the float64 oracle's front end (oracle.forward_raw / backward_raw / decode_step_raw), through the C ABI."""

import numpy as np
import pytest
import torch

import oracle
import synth
from delta_rule_recurrent_gdn_amd import gdn2_bwd_chunked, gdn2_decode_step, gdn2_fwd_chunked
from tests.helpers import TOL_BF16, TOL_F32, TOL_GRAD, f64, rel_err, to_dev

pytestmark = pytest.mark.gpu
GRADS = ("dq", "dk", "dv", "dlog_alpha", "db", "dw", "dS0")


def _ofwd(inp):
    return oracle.forward_raw(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["b"], inp["w"], inp.get("S0"))


@pytest.mark.parametrize("single", [False, True], ids=["two_stage", "single_pass"])
@pytest.mark.parametrize("B,H,T,Dk,Dv,C,dtype", [
    (1, 3, 2 * 32 + 5, 32, 64, 32, "fp32"),
    (2, 3, 3 * 64 + 9, 128, 128, 64, "bf16"),
    (1, 2, 2 * 16 + 3, 16, 16, 16, "bf16"),
])
def test_raw_gate_forward(B, H, T, Dk, Dv, C, dtype, single):
    inp = synth.make_inputs(B, T, H, Dk, Dv, dtype, seed=60 + Dk + C, s0_std=0.2, raw_gates=True)
    d = to_dev(inp)
    o, S, _ = gdn2_fwd_chunked(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], d["S0"], chunk=C,
                               single_pass=single, raw_gates=True)
    torch.cuda.synchronize()
    o_ref, S_ref = _ofwd(inp)
    tol = TOL_F32 if dtype == "fp32" else TOL_BF16
    assert rel_err(f64(o), o_ref) <= tol and rel_err(f64(S), S_ref) <= tol


def test_raw_gate_forward_two_level_chain():
    """Few heads, 40 chunks: the two-level chain with the activations applied in the chunk-parallel kernel."""
    inp = synth.make_inputs(1, 40 * 32 + 7, 2, 64, 64, "bf16", seed=61, s0_std=0.1, raw_gates=True)
    d = to_dev(inp)
    o, S, _ = gdn2_fwd_chunked(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], d["S0"], chunk=32,
                               raw_gates=True)
    torch.cuda.synchronize()
    o_ref, S_ref = _ofwd(inp)
    assert rel_err(f64(o), o_ref) <= TOL_BF16 and rel_err(f64(S), S_ref) <= TOL_BF16


def test_raw_gates_equal_activated_gates_fp32():
    """fp32 inputs: passing pre-activations equals passing the activations computed by torch in fp32.
    The only difference is the activations' own fp32 rounding: the kernels use the hardware exp2, log2 and
    reciprocal (about 1-2 ulp each), and a log-decay difference of an ulp or two passes through the
    in-chunk cumulative sum into every decay factor, so the bar is 5e-5 (the oracle bar is 1e-4)."""
    inp = synth.make_inputs(2, 150, 3, 64, 32, "fp32", seed=62, s0_std=0.2, raw_gates=True, grad=True)
    d = to_dev(inp)
    act = dict(d, b=torch.sigmoid(d["b"]), w=torch.sigmoid(d["w"]),
               log_alpha=-torch.nn.functional.softplus(d["log_alpha"]))
    o1, S1, c1 = gdn2_fwd_chunked(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], d["S0"], chunk=32,
                                  want_chunk_states=True, raw_gates=True)
    o2, S2, c2 = gdn2_fwd_chunked(act["q"], act["k"], act["v"], act["log_alpha"], act["b"], act["w"], act["S0"],
                                  chunk=32, want_chunk_states=True)
    g1 = gdn2_bwd_chunked(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], d["dO"], S0=d["S0"],
                          chunk_states=c1, chunk=32, raw_gates=True)
    g2 = gdn2_bwd_chunked(act["q"], act["k"], act["v"], act["log_alpha"], act["b"], act["w"], act["dO"],
                          S0=act["S0"], chunk_states=c2, chunk=32)
    torch.cuda.synchronize()
    bar = 5e-5
    assert rel_err(f64(o1), f64(o2)) < bar and rel_err(f64(S1), f64(S2)) < bar
    for n in ("dq", "dk", "dv", "dS0"):
        assert rel_err(f64(g1[n]), f64(g2[n])) < bar, n
    # the gate gradients differ by the activation derivatives
    b, w = act["b"], act["w"]
    assert rel_err(f64(g1["db"]), f64(g2["db"] * b * (1 - b))) < bar
    assert rel_err(f64(g1["dw"]), f64(g2["dw"] * w * (1 - w))) < bar
    assert rel_err(f64(g1["dlog_alpha"]), f64(-g2["dlog_alpha"] * torch.sigmoid(d["log_alpha"]))) < bar


@pytest.mark.parametrize("B,H,T,Dk,Dv,C,dtype", [
    (1, 3, 2 * 16 + 5, 16, 16, 16, "fp32"),
    (1, 3, 2 * 32 + 5, 32, 64, 32, "fp32"),
    (1, 2, 2 * 64 + 5, 128, 128, 64, "bf16"),
    (2, 1, 2 * 32 + 7, 64, 32, 32, "bf16"),
])
@pytest.mark.parametrize("use_states", [True, False], ids=["saved_states", "recomputed_states"])
def test_raw_gate_backward(B, H, T, Dk, Dv, C, dtype, use_states):
    inp = synth.make_inputs(B, T, H, Dk, Dv, dtype, seed=63 + Dk + C, s0_std=0.3, grad=True, raw_gates=True)
    dS = torch.from_numpy(np.random.default_rng(Dk).standard_normal((B, H, Dk, Dv)).astype(np.float32))
    d = to_dev(inp)
    states = None
    if use_states:
        _, _, states = gdn2_fwd_chunked(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], d["S0"], chunk=C,
                                        want_final_state=False, want_chunk_states=True, raw_gates=True)
    g = gdn2_bwd_chunked(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], d["dO"], S0=d["S0"],
                         dS_final=dS.cuda(), chunk_states=states, chunk=C, raw_gates=True)
    torch.cuda.synchronize()
    ref = oracle.backward_raw(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["b"], inp["w"], inp["S0"],
                              inp["dO"], dS)
    tol = TOL_F32 if dtype == "fp32" else TOL_GRAD
    errs = {n: rel_err(f64(g[n]), ref[n]) for n in GRADS}
    print("raw-gate backward", (B, H, T, Dk, Dv, C, dtype), {k: f"{v:.1e}" for k, v in errs.items()})
    for n, e in errs.items():
        assert e <= tol, (n, e)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_raw_gate_decode(dtype):
    dec = synth.make_decode_inputs(3, 4, 64, 128, 4, dtype, seed=64, s0_std=0.05, raw_gates=True)
    S = dec["S0"].cuda().clone()
    S_ref = dec["S0"]
    names = ("q", "k", "v", "log_alpha", "b", "w")
    tol = TOL_F32 if dtype == "fp32" else TOL_BF16
    for t in range(4):
        x = {n: dec[n][t].cuda() for n in names}
        o = gdn2_decode_step(x["q"], x["k"], x["v"], x["log_alpha"], x["b"], x["w"], S, raw_gates=True)
        torch.cuda.synchronize()
        o_ref, S_ref = oracle.decode_step_raw(*(dec[n][t] for n in names), S_ref)
        assert rel_err(f64(o), o_ref) <= tol
    assert rel_err(f64(S), S_ref) <= tol
