"""GPU parity of gdn2_bwd_chunked against the float64 oracle's reverse mode (through the C ABI)."""

import numpy as np
import pytest
import torch

import oracle
import synth
from delta_rule_recurrent_gdn_amd import _lib, gdn2_bwd_chunked, gdn2_fwd_chunked
from tests.helpers import TOL_F32, TOL_GRAD, f64, rel_err, take_pairs, take_state_pairs

pytestmark = pytest.mark.gpu
DEV = "cuda"
GRADS = ("dq", "dk", "dv", "dlog_alpha", "db", "dw")


def _dev(inp):
    return {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}


def _gpu_bwd(inp, chunk, dS_final=None, use_states=True):
    d = _dev(inp)
    states = None
    if use_states:
        _, _, states = gdn2_fwd_chunked(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], d.get("S0"),
                                        chunk=chunk, want_final_state=False, want_chunk_states=True)
    g = gdn2_bwd_chunked(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], d["dO"], S0=d.get("S0"),
                         dS_final=None if dS_final is None else dS_final.to(DEV), chunk_states=states, chunk=chunk)
    torch.cuda.synchronize()
    return g


def _oracle_bwd(inp, dS_final=None):
    return oracle.backward(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["b"], inp["w"], inp.get("S0"),
                           inp["dO"], dS_final)


SWEEP = [(dk, dv, c) for (dk, dv) in ((16, 16), (32, 64), (64, 32), (128, 128), (16, 128), (128, 16))
         for c in (16, 32, 64)]


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("Dk,Dv,C", SWEEP)
def test_bwd_sweep_small(dtype, Dk, Dv, C):
    """All seven gradients; several tiles, a ragged tail, S0 and dS_final nonzero, odd B*H."""
    B, H = 1, 3
    T = 2 * C + 5
    inp = synth.make_inputs(B, T, H, Dk, Dv, dtype, seed=Dk * 5 + Dv + C, s0_std=0.3, grad=True)
    dS = torch.from_numpy(np.random.default_rng(Dk + C).standard_normal((B, H, Dk, Dv)).astype(np.float32))
    g = _gpu_bwd(inp, C, dS)
    ref = _oracle_bwd(inp, dS)
    tol = TOL_F32 if dtype == "fp32" else TOL_GRAD
    for name in GRADS + ("dS0",):
        e = rel_err(f64(g[name]), ref[name])
        assert e <= tol, (name, e)


def test_training_B8_H16_T4096_sampled_pairs():
    """B=8, H=16, T=4096, d=128, chunk 64, bf16, dO ~ N(0,1): every gradient of sampled (b, h) pairs."""
    inp = synth.workload_inputs("fwd+bwd-B8-H16-T4096-d128")
    g = _gpu_bwd(inp, 64)
    pairs = [(0, 0), (5, 11), (7, 15)]
    args = [take_pairs(inp[n], pairs) for n in ("q", "k", "v", "log_alpha", "b", "w")]
    ref = oracle.backward(*args, None, take_pairs(inp["dO"], pairs))
    errs = {}
    for name in GRADS:
        gp = np.stack([f64(g[name])[b, :, h] for b, h in pairs])[:, :, None, :]
        errs[name] = rel_err(gp, ref[name])
    gs = np.stack([f64(g["dS0"])[b, h] for b, h in pairs])[:, None]
    errs["dS0"] = rel_err(gs, ref["dS0"])
    print("B8 H16 T4096 gradient errors:", {k: f"{v:.2e}" for k, v in errs.items()})
    for name, e in errs.items():
        assert e <= TOL_GRAD, (name, e)
    for name in GRADS:
        assert torch.isfinite(g[name]).all()


def test_gradient_identities_at_full_size():
    """G1-G3 hold exactly for the true gradients; check them on the GPU gradients of a full-size head batch."""
    inp = synth.make_inputs(2, 2048, 16, 128, 128, "bf16", seed=41, s0_std=0.02, grad=True)
    d = _dev(inp)
    o, _, states = gdn2_fwd_chunked(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], d["S0"], chunk=64,
                                    want_chunk_states=True)
    g = gdn2_bwd_chunked(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], d["dO"], S0=d["S0"],
                         chunk_states=states, chunk=64)
    torch.cuda.synchronize()
    q, k, v, b, w = (f64(inp[n]) for n in ("q", "k", "v", "b", "w"))
    dO, oo = f64(inp["dO"]), f64(o)
    dq, dk, dv, db, dw, dla = (f64(g[n]) for n in ("dq", "dk", "dv", "db", "dw", "dlog_alpha"))
    # G1: q.dq = o.dO per token
    lhs, rhs = np.sum(q * dq, -1), np.sum(oo * dO, -1)
    assert np.max(np.abs(lhs - rhs)) / np.sqrt(np.mean(rhs ** 2)) < TOL_GRAD
    # G2: v dv = w dw
    assert np.max(np.abs(v * dv - w * dw)) / np.sqrt(np.mean((w * dw) ** 2)) < TOL_GRAD
    # G3: k.dk - 2 b.db - w.dw = 0 per token
    g3 = np.sum(k * dk, -1) - 2 * np.sum(b * db, -1) - np.sum(w * dw, -1)
    scale = np.sqrt(np.mean(np.sum(w * dw, -1) ** 2))
    assert np.max(np.abs(g3)) / scale < TOL_GRAD
    # G5: rowsum(S0 * dS0) = dlog_alpha at the first token
    S0 = f64(inp["S0"])
    g5 = np.sum(S0 * f64(g["dS0"]), -1)
    assert np.max(np.abs(g5 - dla[:, 0])) / np.sqrt(np.mean(dla[:, 0] ** 2)) < TOL_GRAD


def test_recompute_states_matches_saved_states_bitwise():
    inp = synth.make_inputs(2, 300, 4, 64, 64, "bf16", seed=42, s0_std=0.1, grad=True)
    g1 = _gpu_bwd(inp, 64, use_states=True)
    g2 = _gpu_bwd(inp, 64, use_states=False)
    for name in GRADS + ("dS0",):
        assert torch.equal(g1[name], g2[name]), name


def test_bwd_deterministic():
    inp = synth.make_inputs(4, 512, 16, 128, 128, "bf16", seed=43, grad=True)
    g1 = _gpu_bwd(inp, 64)
    g2 = _gpu_bwd(inp, 64)
    for name in GRADS + ("dS0",):
        assert torch.equal(g1[name], g2[name]), name


def test_bwd_empty_sequence():
    B, H, D = 2, 3, 32
    dS = torch.randn(B, H, D, D, device=DEV)
    z = torch.empty(B, 0, H, D, device=DEV)
    g = gdn2_bwd_chunked(z, z, z, z, z, z, z, dS_final=dS, chunk=32)
    torch.cuda.synchronize()
    assert torch.equal(g["dS0"], dS) and g["dq"].shape == (B, 0, H, D)


def test_bwd_gdn_special_case_matches_oracle():
    """Scalar gates and scalar decay (the Gated DeltaNet case) through the general kernels."""
    B, T, H, D = 1, 150, 2, 32
    inp = synth.make_inputs(B, T, H, D, D, "fp32", seed=45, s0_std=0.2, grad=True)
    rng = np.random.default_rng(7)
    beta = torch.from_numpy(rng.uniform(0.1, 0.9, (B, T, H, 1)).astype(np.float32))
    a = torch.from_numpy(np.log(rng.uniform(0.8, 0.99, (B, T, H, 1))).astype(np.float32))
    inp["b"] = beta.expand(B, T, H, D).contiguous()
    inp["w"] = beta.expand(B, T, H, D).contiguous()
    inp["log_alpha"] = a.expand(B, T, H, D).contiguous()
    g = _gpu_bwd(inp, 32)
    ref = _oracle_bwd(inp)
    for name in GRADS + ("dS0",):
        assert rel_err(f64(g[name]), ref[name]) <= TOL_F32, name


@pytest.mark.parametrize("B,H,T,Dk,Dv,C,dtype", [
    (1, 2, 33 * 16 + 5, 32, 32, 16, "fp32"),     # 34 chunks: 4 segments
    (1, 3, 40 * 64 + 7, 128, 128, 64, "bf16"),   # d = 128 heads: 5 segments
    (2, 1, 64 * 32, 16, 64, 32, "bf16"),         # Dk = 16 identity columns after 64 value columns
    (1, 1, 36 * 32, 64, 128, 32, "fp32"),
    (1, 4, 256 * 16 + 3, 32, 32, 16, "fp32"),   # 257 chunks: 29 segments of 9, a long composition
])
@pytest.mark.parametrize("use_states", [True, False], ids=["saved_states", "recomputed_states"])
def test_bwd_two_level_reverse_chain(B, H, T, Dk, Dv, C, dtype, use_states):
    """Few heads and at least 32 chunks: the reverse chain runs in segments (parallel segment maps of the
    exit-gradient, fp32 composition from dS_final backwards, re-run); every gradient against the oracle."""
    inp = synth.make_inputs(B, T, H, Dk, Dv, dtype, seed=120 + Dk + C, s0_std=0.3, grad=True)
    dS = torch.from_numpy(np.random.default_rng(Dk + 1).standard_normal((B, H, Dk, Dv)).astype(np.float32))
    g = _gpu_bwd(inp, C, dS, use_states=use_states)
    ref = _oracle_bwd(inp, dS)
    tol = TOL_F32 if dtype == "fp32" else TOL_GRAD
    errs = {n: rel_err(f64(g[n]), ref[n]) for n in GRADS + ("dS0",)}
    print("two-level bwd", (B, H, T, Dk, Dv, C, dtype), {k: f"{v:.1e}" for k, v in errs.items()})
    for n, e in errs.items():
        assert e <= tol, (n, e)
