"""Every workgroup of the full-size launch geometries against the float64 oracle.

The B = 8, H = 16, d = 128, chunk 64 launches (the training step's chain placement over 128 (batch, head)
pairs, the XCD-aware workgroup order, four-wave chains) run here at a reduced sequence length with a ragged
tail, and every (batch, head) pair is compared with the oracle: the two-stage and single-pass forwards, the
training pair and the separate backward, all seven gradients; so do B = 5, H = 13, whose chains fill only
part of the GPU. The decode batch (256 sequences x 16 heads) is compared on every sequence for a few steps.
"""

import numpy as np
import pytest
import torch

import oracle
import synth
from delta_rule_recurrent_gdn_amd import (gdn2_bwd_chunked, gdn2_bwd_chunked_records, gdn2_decode_step,
                                          gdn2_fwd_chunked, gdn2_fwd_chunked_train)
from tests.helpers import TOL_BF16, TOL_GRAD, f64, rel_err, to_dev

pytestmark = pytest.mark.gpu
GRADS = ("dq", "dk", "dv", "dlog_alpha", "db", "dw", "dS0")


@pytest.fixture(scope="module")
def geometry_case():
    T = 4 * 64 + 4  # four full chunks and a 4-token tail
    inp = synth.make_inputs(8, T, 16, 128, 128, "bf16", seed=4, grad=True)
    args = [inp[n] for n in ("q", "k", "v", "log_alpha", "b", "w")]
    o_ref, S_ref = oracle.forward(*args)
    g_ref = oracle.backward(*args, None, inp["dO"])
    return inp, o_ref, S_ref, g_ref


def _per_pair_worst(x, ref, state=False):
    """Largest per-(batch, head) error, and where."""
    worst, at = 0.0, None
    for b in range(ref.shape[0]):
        for h in range(ref.shape[1] if state else ref.shape[2]):
            e = rel_err(x[b, h], ref[b, h]) if state else rel_err(x[b, :, h], ref[b, :, h])
            if e > worst:
                worst, at = e, (b, h)
    return worst, at


@pytest.mark.parametrize("path", ["two-stage", "single-pass", "training"])
def test_forward_every_pair(geometry_case, path):
    inp, o_ref, S_ref, _ = geometry_case
    d = to_dev(inp)
    x = (d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"])
    if path == "training":
        o, S, _ = gdn2_fwd_chunked_train(*x, None, chunk=64)
    else:
        o, S, _ = gdn2_fwd_chunked(*x, None, chunk=64, single_pass=path == "single-pass")
    torch.cuda.synchronize()
    eo, at_o = _per_pair_worst(f64(o), o_ref)
    es, at_s = _per_pair_worst(f64(S), S_ref, state=True)
    print(f"{path}: worst pair o {eo:.2e} at {at_o}, S {es:.2e} at {at_s}")
    assert eo <= TOL_BF16 and es <= TOL_BF16


@pytest.mark.parametrize("path", ["training-pair", "separate"])
def test_backward_every_pair(geometry_case, path):
    inp, _, _, g_ref = geometry_case
    d = to_dev(inp)
    x = (d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"])
    if path == "training-pair":
        _, _, rec = gdn2_fwd_chunked_train(*x, None, chunk=64)
        g = gdn2_bwd_chunked_records(*x, d["dO"], rec, chunk=64)
    else:
        g = gdn2_bwd_chunked(*x, d["dO"], chunk=64)
    torch.cuda.synchronize()
    for n in GRADS:
        e, at = _per_pair_worst(f64(g[n]), g_ref[n], state=n == "dS0")
        print(f"{path}: {n} worst pair {e:.2e} at {at}")
        assert np.isfinite(f64(g[n])).all() and e <= TOL_GRAD, (n, e, at)


@pytest.mark.parametrize("path", ["training-pair", "separate"])
def test_partly_filled_chains_every_pair(path):
    """B = 5, H = 13 (65 (batch, head) pairs, 130 four-wave chain workgroups: fewer than the CUs, the last
    group of 8 ragged): every pair's o, S_final and gradients against the oracle."""
    T = 2 * 64 + 9
    inp = synth.make_inputs(5, T, 13, 128, 128, "bf16", seed=44, grad=True)
    args = [inp[n] for n in ("q", "k", "v", "log_alpha", "b", "w")]
    o_ref, S_ref = oracle.forward(*args)
    g_ref = oracle.backward(*args, None, inp["dO"])
    d = to_dev(inp)
    x = (d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"])
    if path == "training-pair":
        o, S, rec = gdn2_fwd_chunked_train(*x, None, chunk=64)
        g = gdn2_bwd_chunked_records(*x, d["dO"], rec, chunk=64)
    else:
        o, S, _ = gdn2_fwd_chunked(*x, None, chunk=64)
        g = gdn2_bwd_chunked(*x, d["dO"], chunk=64)
    torch.cuda.synchronize()
    eo, at_o = _per_pair_worst(f64(o), o_ref)
    es, at_s = _per_pair_worst(f64(S), S_ref, state=True)
    print(f"{path}: worst pair o {eo:.2e} at {at_o}, S {es:.2e} at {at_s}")
    assert eo <= TOL_BF16 and es <= TOL_BF16
    for n in GRADS:
        e, at = _per_pair_worst(f64(g[n]), g_ref[n], state=n == "dS0")
        assert np.isfinite(f64(g[n])).all() and e <= TOL_GRAD, (n, e, at)


def test_decode_every_sequence_4_steps():
    """B = 256, H = 16, d = 128 decode batch: all 256 sequences (every head) for 4 consecutive steps."""
    inp = synth.workload_inputs("decode-B256-H16-d128-128steps")
    dev = {n: inp[n].cuda() for n in inp}
    S = dev["S0"].clone()
    S_ref = f64(inp["S0"])
    for t in range(4):
        o = gdn2_decode_step(dev["q"][t], dev["k"][t], dev["v"][t], dev["log_alpha"][t], dev["b"][t], dev["w"][t],
                             S)
        torch.cuda.synchronize()
        o_ref, S_ref = oracle.decode_step(*[inp[n][t] for n in ("q", "k", "v", "log_alpha", "b", "w")], S_ref)
        eo = max(rel_err(f64(o[b]), o_ref[b]) for b in range(256))
        print(f"decode step {t}: worst sequence o {eo:.2e}")
        assert eo <= TOL_BF16
    es = max(rel_err(f64(S[b]), S_ref[b]) for b in range(256))
    assert es <= TOL_BF16
