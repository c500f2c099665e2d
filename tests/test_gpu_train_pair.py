"""GPU parity of the training pair (gdn2_fwd_chunked_train / gdn2_bwd_chunked_records): the forward's
chunk-parallel pass also writes the backward's per-chunk records, and the backward starts from them.

The fused pass forms every record value with the same operations, in the same order, as the separate
forward and backward record passes, so the pair's results equal gdn2_fwd_chunked (two-stage, saving chunk
states) followed by gdn2_bwd_chunked bit for bit. The equality is checked across the supported key widths,
chunk sizes, both input dtypes, ragged lengths, the two-level chains, pre-activation and scalar gates. One
shape is also checked against the float64 oracle, through the C ABI."""

import numpy as np
import pytest
import torch

import oracle
import synth
from delta_rule_recurrent_gdn_amd import (gdn2_bwd_chunked, gdn2_bwd_chunked_records, gdn2_fwd_chunked,
                                          gdn2_fwd_chunked_train)
from tests.helpers import TOL_GRAD, f64, rel_err, to_dev

pytestmark = pytest.mark.gpu
GRADS = ("dq", "dk", "dv", "dlog_alpha", "db", "dw", "dS0")


def _pair_equals_separate(inp, C, dS=None, **kw):
    d = to_dev(inp)
    x = (d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"])
    o1, S1, c1, rec = gdn2_fwd_chunked_train(*x, d["S0"], chunk=C, **kw)
    g1 = gdn2_bwd_chunked_records(*x, d["dO"], c1, rec, dS_final=dS, chunk=C, **kw)
    o2, S2, c2 = gdn2_fwd_chunked(*x, d["S0"], chunk=C, want_chunk_states=True, **kw)
    g2 = gdn2_bwd_chunked(*x, d["dO"], S0=d["S0"], dS_final=dS, chunk_states=c2, chunk=C, **kw)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2) and torch.equal(c1, c2)
    for n in GRADS:
        assert torch.equal(g1[n], g2[n]), n
    return o1, S1, g1


@pytest.mark.parametrize("B,H,T,Dk,Dv,C,dtype", [
    (1, 2, 3 * 16 + 5, 16, 16, 16, "fp32"),
    (1, 3, 2 * 32 + 7, 32, 64, 32, "fp32"),
    (2, 2, 2 * 32 + 1, 64, 32, 32, "bf16"),
    (2, 3, 3 * 64 + 9, 128, 128, 64, "bf16"),
    (1, 2, 4 * 64, 128, 64, 64, "bf16"),
    (1, 2, 5 * 16 + 3, 64, 128, 16, "bf16"),
])
def test_training_pair_equals_separate_calls(B, H, T, Dk, Dv, C, dtype):
    inp = synth.make_inputs(B, T, H, Dk, Dv, dtype, seed=110 + Dk + C, s0_std=0.2, grad=True)
    dS = torch.from_numpy(np.random.default_rng(Dk + 1).standard_normal((B, H, Dk, Dv)).astype(np.float32))
    _pair_equals_separate(inp, C, dS=dS.cuda())


def test_training_pair_two_level_chains():
    """Two heads, 40 chunks: both chains take the two-level form."""
    inp = synth.make_inputs(1, 40 * 32 + 7, 2, 64, 64, "bf16", seed=111, s0_std=0.1, grad=True)
    _pair_equals_separate(inp, 32)


@pytest.mark.parametrize("kw", [dict(raw_gates=True), dict(scalar_b=True, scalar_w=True, scalar_decay=True)],
                         ids=["raw_gates", "scalar_gates"])
def test_training_pair_gate_options(kw):
    B, H, T, D, C = 1, 2, 2 * 64 + 5, 128, 64
    inp = synth.make_inputs(B, T, H, D, D, "bf16", seed=112, s0_std=0.2, grad=True, raw_gates=kw.get("raw_gates",
                                                                                                    False))
    if kw.get("scalar_b"):
        rng = np.random.default_rng(113)
        for n in ("b", "w"):
            inp[n] = torch.from_numpy(rng.uniform(0.05, 0.95, (B, T, H)).astype(np.float32)).bfloat16()
        inp["log_alpha"] = torch.from_numpy(-np.log1p(np.exp(rng.standard_normal((B, T, H)) - 2)).astype(np.float32))
    _pair_equals_separate(inp, C, **kw)


def test_training_pair_against_oracle():
    B, H, T, D, C = 1, 2, 2 * 64 + 5, 128, 64
    inp = synth.make_inputs(B, T, H, D, D, "bf16", seed=114, s0_std=0.3, grad=True)
    dS = torch.from_numpy(np.random.default_rng(115).standard_normal((B, H, D, D)).astype(np.float32))
    o, S, g = _pair_equals_separate(inp, C, dS=dS.cuda())
    o_ref, S_ref = oracle.forward(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["b"], inp["w"], inp["S0"])
    assert rel_err(f64(o), o_ref) <= 2e-2 and rel_err(f64(S), S_ref) <= 2e-2
    ref = oracle.backward(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["b"], inp["w"], inp["S0"],
                          inp["dO"], dS)
    for n in GRADS:
        assert rel_err(f64(g[n]), ref[n]) <= TOL_GRAD, n
