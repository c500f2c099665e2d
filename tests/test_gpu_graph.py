"""HIP graph capture of the training step and of decode steps, replayed against eager runs.

No entry point allocates, synchronises or clears memory with a memset, so a training step (the training
pair) and a run of decode steps can be captured into a graph and replayed. Every replay must reproduce the
eager results bit for bit; between replays the outputs are overwritten and other eager work runs on the
same stream, so a replay that leaned on state left by the capture or by an earlier replay would show.
"""

import numpy as np
import pytest
import torch

import synth
from delta_rule_recurrent_gdn_amd import gdn2_bwd_chunked_records, gdn2_decode_step, gdn2_fwd_chunked_train
from tests.helpers import to_dev

pytestmark = pytest.mark.gpu
GRADS = ("dq", "dk", "dv", "dlog_alpha", "db", "dw", "dS0")


def _pair(x, S0, dO):
    o, S, rec = gdn2_fwd_chunked_train(*x, S0, chunk=64)
    g = gdn2_bwd_chunked_records(*x, dO, rec, chunk=64)
    return o, S, g


def test_training_pair_graph_replays():
    inp = synth.make_inputs(2, 3 * 64 + 11, 4, 64, 64, "bf16", seed=81, s0_std=0.3, grad=True)
    d = to_dev(inp)
    x = (d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"])
    o_e, S_e, g_e = _pair(x, d["S0"], d["dO"])
    torch.cuda.synchronize()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on a side stream before capture
        _pair(x, d["S0"], d["dO"])
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        o_g, S_g, g_g = _pair(x, d["S0"], d["dO"])
    torch.cuda.synchronize()

    for rep in range(3):
        o_g.fill_(float("nan"))
        S_g.fill_(float("nan"))
        for n in GRADS:
            g_g[n].fill_(float("nan"))
        _pair(x, d["S0"], d["dO"])  # eager work between replays
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o_g, o_e) and torch.equal(S_g, S_e), rep
        for n in GRADS:
            assert torch.equal(g_g[n], g_e[n]), (rep, n)


def test_decode_steps_graph_replays():
    steps = 4
    dec = synth.make_decode_inputs(8, 4, 64, 64, steps, "bf16", seed=82, s0_std=0.3)
    dd = {k: v.cuda() for k, v in dec.items()}
    xs = [[dd[n][t] for n in ("q", "k", "v", "log_alpha", "b", "w")] for t in range(steps)]

    S_e = dd["S0"].clone()
    o_e = [gdn2_decode_step(*xs[t], S_e).clone() for t in range(steps)]
    torch.cuda.synchronize()

    S = dd["S0"].clone()
    outs = [torch.empty_like(o_e[0]) for _ in range(steps)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for t in range(steps):
            gdn2_decode_step(*xs[t], S, o=outs[t])
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for t in range(steps):
            gdn2_decode_step(*xs[t], S, o=outs[t])
    torch.cuda.synchronize()

    for rep in range(3):
        S.copy_(dd["S0"])  # eager reset between replays
        for t in range(steps):
            outs[t].fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        for t in range(steps):
            assert torch.equal(outs[t], o_e[t]), (rep, t)
        assert torch.equal(S, S_e), rep
    assert np.isfinite(S.cpu().numpy()).all()
