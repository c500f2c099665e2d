"""GPU parity of packed variable-length batches (gdn2_fwd_varlen, gdn2_bwd_varlen) and of slot-indexed
decode (gdn2_decode_step_slots) against the float64 oracle's definitions, through the C ABI."""

import numpy as np
import pytest
import torch

import oracle
import synth
from delta_rule_recurrent_gdn_amd import (gdn2_bwd_varlen, gdn2_bwd_varlen_records, gdn2_decode_step_slots,
                                          gdn2_fwd_chunked, gdn2_fwd_varlen, gdn2_fwd_varlen_train,
                                          gdn2_varlen_max_chunks)
from tests.helpers import TOL_BF16, TOL_F32, TOL_GRAD, f64, rel_err, to_dev

pytestmark = pytest.mark.gpu
GRADS = ("dq", "dk", "dv", "dlog_alpha", "db", "dw", "dS0")


def _packed(lengths, H, Dk, Dv, dtype, seed, grad=False, raw_gates=False):
    T = int(sum(lengths))
    inp = synth.make_inputs(1, T, H, Dk, Dv, dtype, seed=seed, grad=grad, raw_gates=raw_gates)
    rng = np.random.default_rng(seed + 1)
    inp["S0"] = torch.from_numpy((0.3 * rng.standard_normal((len(lengths), H, Dk, Dv))).astype(np.float32))
    cu = torch.from_numpy(np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64))
    return inp, cu


def _chunk_map(lengths, C):
    """(sequence, local chunk, first token) of every global chunk, in order."""
    out, t = [], 0
    for n, L in enumerate(lengths):
        for c in range((L + C - 1) // C):
            out.append((n, c, t + c * C))
        t += L
    return out


# length mixes: empty, single-token, C-1, C, C+1 and long sequences, in different orders
MIXES = [
    ([37, 0, 1, 64, 65, 130], 64),
    ([16, 15, 17, 0, 48, 3], 16),
    ([200, 1, 31, 32, 33], 32),
]


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("Dk,Dv", [(32, 64), (128, 128), (16, 16)])
@pytest.mark.parametrize("mix", range(len(MIXES)))
def test_varlen_forward(dtype, Dk, Dv, mix):
    lengths, C = MIXES[mix]
    H = 2
    inp, cu = _packed(lengths, H, Dk, Dv, dtype, seed=70 + Dk + mix)
    d = to_dev(inp)
    o, Sf, cs = gdn2_fwd_varlen(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], cu.cuda(), d["S0"],
                                chunk=C, want_chunk_states=True)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle.forward_varlen(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["b"], inp["w"], cu,
                                         inp["S0"])
    tol = TOL_F32 if dtype == "fp32" else TOL_BF16
    eo, es = rel_err(f64(o), o_ref), rel_err(f64(Sf), S_ref)
    print(f"varlen fwd {lengths} C={C} Dk={Dk} Dv={Dv} {dtype}: err o {eo:.2e} S {es:.2e}")
    assert eo <= tol and es <= tol
    # chunk entry states [H, max_chunks, Dk, Dv]: the sequences' chunks in order
    assert cs.shape[1] == gdn2_varlen_max_chunks(len(lengths), int(sum(lengths)), C)
    cs64 = f64(cs)
    starts = np.concatenate([[0], np.cumsum(lengths)])
    for g, (n, c, t) in enumerate(_chunk_map(lengths, C)):
        if c == 0:
            ref = f64(inp["S0"])[n]
        else:
            a = int(starts[n])
            sl = {k_: v_[:, a:t] for k_, v_ in inp.items() if k_ != "S0"}
            _, ref = oracle.forward(sl["q"], sl["k"], sl["v"], sl["log_alpha"], sl["b"], sl["w"],
                                    inp["S0"][n:n + 1])
            ref = ref[0]
        assert rel_err(cs64[:, g], ref) <= tol, (g, n, c)


def test_varlen_equal_lengths_match_dense_bitwise():
    """Equal lengths that are multiples of the chunk: the packed call runs the same kernels on the same
    chunks as the dense call on [N, L, H, D], so the results are identical."""
    N, L, H, D, C = 3, 128, 4, 64, 64
    inp, cu = _packed([L] * N, H, D, D, "bf16", seed=75)
    d = to_dev(inp)
    o, Sf, _ = gdn2_fwd_varlen(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], cu.cuda(), d["S0"], chunk=C)
    dense = {k_: (v_.reshape(N, L, H, -1).contiguous() if k_ != "S0" else v_) for k_, v_ in d.items()}
    od, Sd, _ = gdn2_fwd_chunked(dense["q"], dense["k"], dense["v"], dense["log_alpha"], dense["b"], dense["w"],
                                 dense["S0"], chunk=C)
    torch.cuda.synchronize()
    assert torch.equal(o.reshape(N, L, H, D), od) and torch.equal(Sf, Sd)


@pytest.mark.parametrize("dtype,Dk,Dv,mix", [("fp32", 32, 64, 0), ("fp32", 16, 16, 1), ("bf16", 128, 128, 0),
                                             ("bf16", 64, 32, 2), ("fp32", 128, 128, 0)])
@pytest.mark.parametrize("use_states", [True, False], ids=["saved_states", "recomputed_states"])
def test_varlen_backward(dtype, Dk, Dv, mix, use_states):
    lengths, C = MIXES[mix]
    H = 2
    inp, cu = _packed(lengths, H, Dk, Dv, dtype, seed=80 + Dk + mix, grad=True)
    dS = torch.from_numpy(np.random.default_rng(Dk).standard_normal((len(lengths), H, Dk, Dv)).astype(np.float32))
    d = to_dev(inp)
    cs = None
    if use_states:
        _, _, cs = gdn2_fwd_varlen(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], cu.cuda(), d["S0"],
                                   chunk=C, want_final_state=False, want_chunk_states=True)
    g = gdn2_bwd_varlen(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], d["dO"], cu.cuda(), S0=d["S0"],
                        dS_final=dS.cuda(), chunk_states=cs, chunk=C)
    torch.cuda.synchronize()
    ref = oracle.backward_varlen(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["b"], inp["w"], cu, inp["S0"],
                                 inp["dO"], dS)
    tol = TOL_F32 if dtype == "fp32" else TOL_GRAD
    errs = {n: rel_err(f64(g[n]), ref[n]) for n in GRADS}
    print("varlen bwd", lengths, dtype, Dk, Dv, {k: f"{v:.1e}" for k, v in errs.items()})
    for n, e in errs.items():
        assert e <= tol, (n, e)


def test_varlen_raw_gates_backward():
    """Packed batch with the fused gate front end."""
    lengths, C = MIXES[1]
    inp, cu = _packed(lengths, 2, 32, 32, "fp32", seed=86, grad=True, raw_gates=True)
    d = to_dev(inp)
    g = gdn2_bwd_varlen(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], d["dO"], cu.cuda(), S0=d["S0"],
                        chunk=C, raw_gates=True)
    torch.cuda.synchronize()
    b, w, la = oracle.gates_from_raw(inp["b"], inp["w"], inp["log_alpha"])
    ref = oracle.backward_varlen(inp["q"], inp["k"], inp["v"], la, b, w, cu, inp["S0"], inp["dO"])
    ref["db"] = ref["db"] * b * (1 - b)
    ref["dw"] = ref["dw"] * w * (1 - w)
    ref["dlog_alpha"] = -ref["dlog_alpha"] * (1 - np.exp(la))  # sigmoid(a) = 1 - exp(-softplus(a))
    for n in GRADS:
        assert rel_err(f64(g[n]), ref[n]) <= TOL_F32, n


def test_varlen_offsets_are_clamped():
    """Offsets past T or decreasing are made non-decreasing within [0, T]: the call stays inside the tensors
    and equals the call on the clamped offsets."""
    H, D, C = 2, 32, 16
    inp, _ = _packed([40, 30], H, D, D, "fp32", seed=87)
    d = to_dev(inp)
    bad = torch.tensor([0, 50, 20, 999], dtype=torch.int64, device="cuda")     # -> 0, 50, 50, 70
    good = torch.tensor([0, 50, 50, 70], dtype=torch.int64, device="cuda")
    S0 = torch.zeros(3, H, D, D, device="cuda")
    o1, S1, _ = gdn2_fwd_varlen(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], bad, S0, chunk=C)
    o2, S2, _ = gdn2_fwd_varlen(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], good, S0, chunk=C)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_decode_slots(dtype):
    B, H, Dk, Dv, P = 5, 4, 64, 128, 8
    dec = synth.make_decode_inputs(B, H, Dk, Dv, 3, dtype, seed=88, s0_std=0.05)
    pool = torch.from_numpy((0.05 * np.random.default_rng(9).standard_normal((P, H, Dk, Dv))).astype(np.float32))
    slots = torch.tensor([6, 0, -1, 3, 9], dtype=torch.int32)  # -1 and 9: no state
    Sp = pool.cuda().clone()
    ref_pool = pool.numpy().astype(np.float64)
    names = ("q", "k", "v", "log_alpha", "b", "w")
    tol = TOL_F32 if dtype == "fp32" else TOL_BF16
    for t in range(3):
        x = {n: dec[n][t].cuda() for n in names}
        o = gdn2_decode_step_slots(x["q"], x["k"], x["v"], x["log_alpha"], x["b"], x["w"], Sp, slots.cuda())
        torch.cuda.synchronize()
        o_ref, ref_pool = oracle.decode_step_slots(*(dec[n][t] for n in names), ref_pool, slots.numpy())
        assert rel_err(f64(o), o_ref) <= tol
        assert torch.count_nonzero(o[2]) == 0 and torch.count_nonzero(o[4]) == 0
    assert rel_err(f64(Sp), ref_pool) <= tol
    for s in (1, 2, 4, 5, 7):  # untouched slots
        assert torch.equal(Sp[s].cpu(), pool[s])


@pytest.mark.parametrize("dtype,Dk,Dv", [("fp32", 32, 64), ("bf16", 128, 128), ("bf16", 16, 64)])
def test_varlen_two_level_chain(dtype, Dk, Dv):
    """Few sequence-heads and at least 32 chunks: the packed forward cuts the long sequences into segments
    (parallel segment maps, fp32 composition, re-run). Segments never cross a sequence boundary; empty and
    one-segment sequences pass through."""
    from delta_rule_recurrent_gdn_amd import _lib
    lengths, C, H = [1500, 37, 900, 3, 0, 600], 32, 2
    N, T = len(lengths), int(sum(lengths))
    lib = _lib.load()
    code = _lib.GDN2_F32 if dtype == "fp32" else _lib.GDN2_BF16
    mc = gdn2_varlen_max_chunks(N, T, C)
    per_chunk = lib.gdn2_workspace_bytes(_lib.GDN2_OP_FWD, 1, C, 1, Dk, Dv, C, code)
    ws = lib.gdn2_varlen_workspace_bytes(_lib.GDN2_OP_FWD, N, T, H, Dk, Dv, C, code)
    assert ws > H * mc * per_chunk + H * (Dk * Dk + 2 * Dk * Dv) * 4  # segment maps present
    inp, cu = _packed(lengths, H, Dk, Dv, dtype, seed=110 + Dk)
    d = to_dev(inp)
    o, Sf, cs = gdn2_fwd_varlen(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], cu.cuda(), d["S0"],
                                chunk=C, want_chunk_states=True)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle.forward_varlen(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["b"], inp["w"], cu,
                                         inp["S0"])
    tol = TOL_F32 if dtype == "fp32" else TOL_BF16
    eo, es = rel_err(f64(o), o_ref), rel_err(f64(Sf), S_ref)
    print(f"varlen two-level {dtype} Dk={Dk} Dv={Dv}: err o {eo:.2e} S {es:.2e}")
    assert eo <= tol and es <= tol
    cs64 = f64(cs)
    starts = np.concatenate([[0], np.cumsum(lengths)])
    cmap = _chunk_map(lengths, C)
    for g in (0, 7, 8, 9, 30, 46, 47, 48, len(cmap) - 1):  # around segment and sequence boundaries
        n, c, t = cmap[g]
        if c == 0:
            ref = f64(inp["S0"])[n]
        else:
            a = int(starts[n])
            sl = {k_: v_[:, a:t] for k_, v_ in inp.items() if k_ != "S0"}
            _, ref = oracle.forward(sl["q"], sl["k"], sl["v"], sl["log_alpha"], sl["b"], sl["w"],
                                    inp["S0"][n:n + 1])
            ref = ref[0]
        assert rel_err(cs64[:, g], ref) <= tol, (g, n, c)
    # the backward's state recompute takes the same path
    dO = torch.from_numpy(np.random.default_rng(5).standard_normal((1, T, H, Dv)).astype(np.float32))
    dO = dO.to(synth.torch_dtype(dtype)).cuda()
    g1 = gdn2_bwd_varlen(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], dO, cu.cuda(), S0=d["S0"],
                         chunk_states=cs, chunk=C)
    g2 = gdn2_bwd_varlen(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], dO, cu.cuda(), S0=d["S0"],
                         chunk=C)
    torch.cuda.synchronize()
    for n_ in GRADS:
        assert torch.equal(g1[n_], g2[n_]), n_
    # against the oracle (the reverse chain is segmented as well)
    dO_host = dO.cpu()
    ref = oracle.backward_varlen(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["b"], inp["w"], cu, inp["S0"],
                                 dO_host)
    gtol = TOL_F32 if dtype == "fp32" else TOL_GRAD
    for n_ in GRADS:
        assert rel_err(f64(g1[n_]), ref[n_]) <= gtol, n_


def test_varlen_past_32_chains_plain_walk():
    """The lengths of the two-level test with 8 heads (48 (sequence, head) chains, at least 32 chunks): no
    segments, the plain four-wave chains walk every sequence whole; forward, chunk states and the training
    pair's gradients against the oracle."""
    from delta_rule_recurrent_gdn_amd import _lib
    lengths, C, H, D = [1500, 37, 900, 3, 0, 600], 64, 8, 128
    N, T = len(lengths), int(sum(lengths))
    lib = _lib.load()
    mc = gdn2_varlen_max_chunks(N, T, C)
    per_chunk = lib.gdn2_workspace_bytes(_lib.GDN2_OP_FWD, 1, C, 1, D, D, C, _lib.GDN2_BF16)
    ws = lib.gdn2_varlen_workspace_bytes(_lib.GDN2_OP_FWD, N, T, H, D, D, C, _lib.GDN2_BF16)
    assert ws < H * mc * per_chunk + H * (D * D + 2 * D * D) * 4  # no segment maps
    inp, cu = _packed(lengths, H, D, D, "bf16", seed=150, grad=True)
    d = to_dev(inp)
    x = (d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"])
    o, S, rec = gdn2_fwd_varlen_train(*x, cu.cuda(), d["S0"], chunk=C)
    g = gdn2_bwd_varlen_records(*x, d["dO"], cu.cuda(), rec, chunk=C)
    torch.cuda.synchronize()
    args = [inp[n] for n in ("q", "k", "v", "log_alpha", "b", "w")]
    o_ref, S_ref = oracle.forward_varlen(*args, cu, inp["S0"])
    assert rel_err(f64(o), o_ref) <= TOL_BF16 and rel_err(f64(S), S_ref) <= TOL_BF16
    ref = oracle.backward_varlen(*args, cu, inp["S0"], inp["dO"])
    for n in GRADS:
        e = rel_err(f64(g[n]), ref[n])
        assert e <= TOL_GRAD, (n, e)


def test_varlen_many_sequences_four_wave_chains():
    """16 ragged sequences of 16 heads (256 (sequence, head) pairs of 128 value columns): the chains take
    their four-wave workgroups in the packed layout; outputs, states and every gradient against the
    oracle's per-sequence definition."""
    lengths = [37, 0, 1, 64, 65, 130, 16, 93, 7, 128, 3, 70, 64, 1, 90, 33]
    C, H, D = 64, 16, 128
    inp, cu = _packed(lengths, H, D, D, "bf16", seed=140, grad=True)
    dS = torch.from_numpy(np.random.default_rng(141).standard_normal((len(lengths), H, D, D)).astype(np.float32))
    d = to_dev(inp)
    x = (d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"])
    o, S, cs = gdn2_fwd_varlen(*x, cu.cuda(), d["S0"], chunk=C, want_chunk_states=True)
    g = gdn2_bwd_varlen(*x, d["dO"], cu.cuda(), S0=d["S0"], dS_final=dS.cuda(), chunk_states=cs, chunk=C)
    torch.cuda.synchronize()
    args = [inp[n] for n in ("q", "k", "v", "log_alpha", "b", "w")]
    o_ref, S_ref = oracle.forward_varlen(*args, cu, inp["S0"])
    assert rel_err(f64(o), o_ref) <= TOL_BF16 and rel_err(f64(S), S_ref) <= TOL_BF16
    ref = oracle.backward_varlen(*args, cu, inp["S0"], inp["dO"], dS)
    for n in GRADS:
        e = rel_err(f64(g[n]), ref[n])
        assert e <= TOL_GRAD, (n, e)
