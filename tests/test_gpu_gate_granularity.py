"""GPU parity of the gate-granularity variants (GDN2_FLAG_SCALAR_B / _W / _DECAY): gates given as one value
per (token, head), broadcast inside the kernels; gradients summed over the channels. Against the float64
oracle's definitions (oracle.forward_gates / backward_gates), through the C ABI."""

import numpy as np
import pytest
import torch

import oracle
import synth
from delta_rule_recurrent_gdn_amd import (gdn2_bwd_chunked, gdn2_bwd_varlen, gdn2_decode_step, gdn2_fwd_chunked,
                                          gdn2_fwd_varlen)
from tests.helpers import TOL_BF16, TOL_F32, TOL_GRAD, f64, rel_err, to_dev

pytestmark = pytest.mark.gpu
GRADS = ("dq", "dk", "dv", "dlog_alpha", "db", "dw", "dS0")

# (scalar_b, scalar_w, scalar_decay): each gate alone, KDA (both gates) and Gated DeltaNet (all three)
COMBOS = [(True, False, False), (False, True, False), (False, False, True), (True, True, False), (True, True, True)]
IDS = ["b", "w", "decay", "kda", "gdn"]


def _scalar_inputs(B, T, H, Dk, Dv, dtype, seed, flags, grad=False, raw=False):
    """Full-size draws, with each scalar gate replaced by one seeded value per (token, head) in its range."""
    inp = synth.make_inputs(B, T, H, Dk, Dv, dtype, seed=seed, s0_std=0.2, grad=grad, raw_gates=raw)
    rng = np.random.default_rng(seed + 5)
    sb, sw, sd = flags
    tdt = synth.torch_dtype(dtype)
    gate = (lambda: rng.standard_normal((B, T, H))) if raw else (lambda: rng.uniform(0.05, 0.95, (B, T, H)))
    if sb:
        inp["b"] = torch.from_numpy(gate().astype(np.float32)).to(tdt)
    if sw:
        inp["w"] = torch.from_numpy(gate().astype(np.float32)).to(tdt)
    if sd:
        la = rng.standard_normal((B, T, H)) - 2.0 if raw else -np.log1p(np.exp(rng.standard_normal((B, T, H)) - 2))
        inp["log_alpha"] = torch.from_numpy(la.astype(np.float32))
    return inp


def _kw(flags, raw=False):
    return dict(scalar_b=flags[0], scalar_w=flags[1], scalar_decay=flags[2], raw_gates=raw)


def _okw(flags, raw=False):
    return dict(scalar_b=flags[0], scalar_w=flags[1], scalar_decay=flags[2], raw=raw)


@pytest.mark.parametrize("flags", COMBOS, ids=IDS)
@pytest.mark.parametrize("single", [False, True], ids=["two_stage", "single_pass"])
@pytest.mark.parametrize("B,H,T,Dk,Dv,C,dtype", [(1, 3, 2 * 32 + 5, 32, 64, 32, "fp32"),
                                                 (2, 2, 2 * 64 + 9, 128, 128, 64, "bf16")])
def test_scalar_gate_forward(flags, single, B, H, T, Dk, Dv, C, dtype):
    inp = _scalar_inputs(B, T, H, Dk, Dv, dtype, seed=90 + Dk, flags=flags)
    d = to_dev(inp)
    o, S, _ = gdn2_fwd_chunked(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], d["S0"], chunk=C,
                               single_pass=single, **_kw(flags))
    torch.cuda.synchronize()
    o_ref, S_ref = oracle.forward_gates(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["b"], inp["w"],
                                        inp["S0"], **_okw(flags))
    tol = TOL_F32 if dtype == "fp32" else TOL_BF16
    assert rel_err(f64(o), o_ref) <= tol and rel_err(f64(S), S_ref) <= tol


@pytest.mark.parametrize("flags", COMBOS, ids=IDS)
def test_scalar_gates_equal_broadcast_gates(flags):
    """The scalar path reads the same values as the per-channel path fed with the broadcast tensors: the
    forward results are identical, and the scalar gradients are the channel sums of the broadcast ones."""
    B, H, T, Dk, Dv, C = 2, 3, 150, 64, 32, 32
    inp = _scalar_inputs(B, T, H, Dk, Dv, "bf16", seed=95, flags=flags, grad=True)
    d = to_dev(inp)
    full = dict(d)
    if flags[0]:
        full["b"] = d["b"][..., None].expand(B, T, H, Dk).contiguous()
    if flags[1]:
        full["w"] = d["w"][..., None].expand(B, T, H, Dv).contiguous()
    if flags[2]:
        full["log_alpha"] = d["log_alpha"][..., None].expand(B, T, H, Dk).contiguous()
    o1, S1, c1 = gdn2_fwd_chunked(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], d["S0"], chunk=C,
                                  want_chunk_states=True, **_kw(flags))
    o2, S2, c2 = gdn2_fwd_chunked(full["q"], full["k"], full["v"], full["log_alpha"], full["b"], full["w"],
                                  full["S0"], chunk=C, want_chunk_states=True)
    g1 = gdn2_bwd_chunked(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], d["dO"], S0=d["S0"],
                          chunk_states=c1, chunk=C, **_kw(flags))
    g2 = gdn2_bwd_chunked(full["q"], full["k"], full["v"], full["log_alpha"], full["b"], full["w"], full["dO"],
                          S0=full["S0"], chunk_states=c2, chunk=C)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2) and torch.equal(c1, c2)
    for n in ("dq", "dk", "dv", "dS0"):
        assert torch.equal(g1[n], g2[n]), n
    for n, sc in (("db", flags[0]), ("dw", flags[1]), ("dlog_alpha", flags[2])):
        ref = g2[n].sum(-1) if sc else g2[n]
        assert rel_err(f64(g1[n]), f64(ref)) < 1e-5, n


@pytest.mark.parametrize("flags", COMBOS, ids=IDS)
@pytest.mark.parametrize("raw", [False, True], ids=["gates", "raw_gates"])
@pytest.mark.parametrize("B,H,T,Dk,Dv,C,dtype", [(1, 2, 2 * 16 + 5, 16, 32, 16, "fp32"),
                                                 (1, 2, 2 * 64 + 5, 128, 128, 64, "bf16")])
def test_scalar_gate_backward(flags, raw, B, H, T, Dk, Dv, C, dtype):
    inp = _scalar_inputs(B, T, H, Dk, Dv, dtype, seed=97 + Dk, flags=flags, grad=True, raw=raw)
    dS = torch.from_numpy(np.random.default_rng(Dk).standard_normal((B, H, Dk, Dv)).astype(np.float32))
    d = to_dev(inp)
    g = gdn2_bwd_chunked(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], d["dO"], S0=d["S0"],
                         dS_final=dS.cuda(), chunk=C, **_kw(flags, raw))
    torch.cuda.synchronize()
    ref = oracle.backward_gates(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["b"], inp["w"], inp["S0"],
                                inp["dO"], dS, **_okw(flags, raw))
    tol = TOL_F32 if dtype == "fp32" else TOL_GRAD
    errs = {n: rel_err(f64(g[n]), ref[n]) for n in GRADS}
    print("scalar-gate backward", flags, raw, dtype, {k: f"{v:.1e}" for k, v in errs.items()})
    for n, e in errs.items():
        assert tuple(g[n].shape) == ref[n].shape, n
        assert e <= tol, (n, e)


def test_scalar_gates_packed_batch():
    """Gated DeltaNet-style gates on a packed variable-length batch."""
    flags = (True, True, True)
    lengths, C = [37, 0, 80, 11], 32
    T, H, D = sum(lengths), 2, 32
    inp = _scalar_inputs(1, T, H, D, D, "fp32", seed=99, flags=flags, grad=True)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), dtype=torch.int64)
    S0 = torch.from_numpy((0.2 * np.random.default_rng(3).standard_normal((len(lengths), H, D, D))).astype(np.float32))
    d = to_dev(inp)
    o, Sf, _ = gdn2_fwd_varlen(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], cu.cuda(), S0.cuda(),
                               chunk=C, **_kw(flags))
    g = gdn2_bwd_varlen(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], d["dO"], cu.cuda(), S0=S0.cuda(),
                        chunk=C, **_kw(flags))
    torch.cuda.synchronize()
    ex = lambda x, n: x[..., None].expand(*x.shape, n).contiguous()  # noqa: E731
    b, w, la = ex(inp["b"], D), ex(inp["w"], D), ex(inp["log_alpha"], D)
    o_ref, S_ref = oracle.forward_varlen(inp["q"], inp["k"], inp["v"], la, b, w, cu, S0)
    assert rel_err(f64(o), o_ref) <= TOL_F32 and rel_err(f64(Sf), S_ref) <= TOL_F32
    ref = oracle.backward_varlen(inp["q"], inp["k"], inp["v"], la, b, w, cu, S0, inp["dO"])
    for n in ("db", "dw", "dlog_alpha"):
        ref[n] = ref[n].sum(-1)
    for n in GRADS:
        assert rel_err(f64(g[n]), ref[n]) <= TOL_F32, n


@pytest.mark.parametrize("flags", COMBOS, ids=IDS)
def test_scalar_gate_decode(flags):
    B, H, Dk, Dv = 3, 4, 64, 128
    dec = synth.make_decode_inputs(B, H, Dk, Dv, 2, "bf16", seed=101, s0_std=0.05)
    rng = np.random.default_rng(102)
    if flags[0]:
        dec["b"] = torch.from_numpy(rng.uniform(0.05, 0.95, (2, B, H)).astype(np.float32)).bfloat16()
    if flags[1]:
        dec["w"] = torch.from_numpy(rng.uniform(0.05, 0.95, (2, B, H)).astype(np.float32)).bfloat16()
    if flags[2]:
        dec["log_alpha"] = torch.from_numpy(-rng.uniform(0.01, 0.5, (2, B, H)).astype(np.float32))
    S = dec["S0"].cuda().clone()
    S_ref = dec["S0"]
    names = ("q", "k", "v", "log_alpha", "b", "w")
    for t in range(2):
        x = {n: dec[n][t].cuda() for n in names}
        o = gdn2_decode_step(x["q"], x["k"], x["v"], x["log_alpha"], x["b"], x["w"], S, **_kw(flags))
        torch.cuda.synchronize()
        ex = lambda y, n, sc: (y[..., None].expand(*y.shape, n) if sc else y)  # noqa: E731
        o_ref, S_ref = oracle.decode_step(dec["q"][t], dec["k"][t], dec["v"][t],
                                          ex(dec["log_alpha"][t], Dk, flags[2]), ex(dec["b"][t], Dk, flags[0]),
                                          ex(dec["w"][t], Dv, flags[1]), S_ref)
        assert rel_err(f64(o), o_ref) <= TOL_BF16
    assert rel_err(f64(S), S_ref) <= TOL_BF16
