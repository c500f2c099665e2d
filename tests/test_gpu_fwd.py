"""GPU parity of gdn2_fwd_chunked against the float64 oracle (through the C ABI)."""

import numpy as np
import pytest
import torch

import oracle
import synth
from delta_rule_recurrent_gdn_amd import _lib, gdn2_fwd_chunked
from tests.helpers import (f64, gpu_pairs, gpu_state_pairs, oracle_fwd_pairs, rel_err, to_dev, tol_for,
                           TOL_BF16, TOL_F32)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _run(inp, chunk, states=False, single=False):
    d = to_dev(inp)
    o, S, cs = gdn2_fwd_chunked(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], d.get("S0"), chunk=chunk,
                                want_chunk_states=states, single_pass=single)
    torch.cuda.synchronize()
    return o, S, cs


# both forward paths: the two-stage one (workspace) and the single-pass kernel
PATHS = pytest.mark.parametrize("single", [False, True], ids=["two_stage", "single_pass"])


@PATHS
def test_tiny_fp32_exact(single):
    """B=1, H=2, T=64, d=16, chunk 16, fp32, seed 0: every output against the stepwise oracle."""
    inp = synth.workload_inputs("tiny-fp32-fwd")
    o, S, _ = _run(inp, 16, single=single)
    o_ref, S_ref = oracle.forward(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["b"], inp["w"], None)
    print("tiny fp32 err o %.3e S %.3e" % (rel_err(f64(o), o_ref), rel_err(f64(S), S_ref)))
    assert rel_err(f64(o), o_ref) <= TOL_F32
    assert rel_err(f64(S), S_ref) <= TOL_F32


SWEEP = [(dk, dv, c) for (dk, dv) in ((16, 16), (32, 64), (64, 32), (128, 128), (128, 16), (16, 128))
         for c in (16, 32, 64)]


@PATHS
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("Dk,Dv,C", SWEEP)
def test_sweep_small(dtype, Dk, Dv, C, single):
    """Several tiles, a ragged tail, nonzero S0, chunk states, B*H not a multiple of 8."""
    B, H = 1, 3
    T = 2 * C + 5
    inp = synth.make_inputs(B, T, H, Dk, Dv, dtype, seed=Dk * 7 + Dv * 3 + C, s0_std=0.3)
    tdt = synth.torch_dtype(dtype)
    o, S, cs = _run(inp, C, states=True, single=single)
    o_ref, S_ref = oracle.forward(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["b"], inp["w"], inp["S0"])
    tol = tol_for(tdt)
    assert rel_err(f64(o), o_ref) <= tol, rel_err(f64(o), o_ref)
    assert rel_err(f64(S), S_ref) <= tol, rel_err(f64(S), S_ref)
    # chunk entry states: entry n is the state after n*C tokens
    cs = f64(cs)
    for n in range(cs.shape[2]):
        if n == 0:
            ref = f64(inp["S0"])
        else:
            sl = {k_: v_[:, :n * C] for k_, v_ in inp.items() if k_ not in ("S0",)}
            _, ref = oracle.forward(sl["q"], sl["k"], sl["v"], sl["log_alpha"], sl["b"], sl["w"], inp["S0"])
        assert rel_err(cs[:, :, n], ref) <= tol


@PATHS
def test_fwd_B8_H16_T4096_sampled_pairs(single):
    """B=8, H=16, T=4096, d=128, chunk 64, bf16: all outputs of sampled (b, h) pairs."""
    inp = synth.workload_inputs("fwd-B8-H16-T4096-d128")
    o, S, _ = _run(inp, 64, single=single)
    pairs = [(0, 0), (3, 7), (7, 15), (5, 2)]
    o_ref, S_ref = oracle_fwd_pairs(inp, pairs)
    eo, es = rel_err(gpu_pairs(o, pairs), o_ref), rel_err(gpu_state_pairs(S, pairs), S_ref)
    floor = rel_err(o_ref.astype(np.float32).astype(np.float64), o_ref)
    print(f"B8 H16 T4096 err o {eo:.3e} S {es:.3e} (fp32 output floor {floor:.1e})")
    assert eo <= TOL_BF16 and es <= TOL_BF16
    assert np.isfinite(f64(o)).all() and np.isfinite(f64(S)).all()


@pytest.mark.parametrize("T", [8192, 16384, 32768, 65536])
@PATHS
def test_long_sequence_B1_H16_sampled(T, single):
    """B=1, H=16, T up to 64K, d=128, chunk 64, bf16, S0 ~ 0.02 N(0,1)."""
    inp = synth.workload_inputs("fwd-long-B1-H16-d128", T=T)
    o, S, _ = _run(inp, 64, single=single)
    pairs = [(0, 0), (0, 9)] if T <= 8192 else [(0, 5)] if T == 65536 else [(0, 3), (0, 14)]
    o_ref, S_ref = oracle_fwd_pairs(inp, pairs)
    eo, es = rel_err(gpu_pairs(o, pairs), o_ref), rel_err(gpu_state_pairs(S, pairs), S_ref)
    print(f"long sequence T={T} err o {eo:.3e} S {es:.3e}")
    assert eo <= TOL_BF16 and es <= TOL_BF16


@PATHS
def test_bitwise_deterministic(single):
    inp = synth.make_inputs(4, 1000, 16, 128, 128, "bf16", seed=11, s0_std=0.02)
    o1, S1, _ = _run(inp, 64, single=single)
    o2, S2, _ = _run(inp, 64, single=single)
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


@PATHS
def test_split_sequence_composes_on_gpu(single):
    """fwd(x1 || x2) = fwd(x2; S0 = S_final(x1)) at full head size."""
    inp = synth.make_inputs(2, 640, 16, 128, 128, "bf16", seed=12, s0_std=0.02)
    o, S, _ = _run(inp, 64, single=single)
    a = {k_: (v_[:, :320].contiguous() if k_ != "S0" else v_) for k_, v_ in inp.items()}
    o1, S1, _ = _run(a, 64, single=single)
    b = {k_: (v_[:, 320:].contiguous() if k_ != "S0" else v_) for k_, v_ in inp.items()}
    b["S0"] = S1.cpu()
    o2, S2, _ = _run(b, 64, single=single)
    oc = torch.cat([o1, o2], dim=1)
    assert rel_err(f64(oc), f64(o)) < 1e-3 and rel_err(f64(S2), f64(S)) < 1e-3


@PATHS
def test_chunk_size_invariance(single):
    inp = synth.make_inputs(1, 300, 4, 64, 64, "bf16", seed=13, s0_std=0.1)
    ref, _ = oracle.forward(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["b"], inp["w"], inp["S0"])
    for C in (16, 32, 64):
        o, _, _ = _run(inp, C, single=single)
        assert rel_err(f64(o), ref) <= TOL_BF16


@PATHS
def test_reduces_to_kda_on_gpu(single):
    """b = w = beta * 1 on the GPU equals the oracle's KDA case (pinned separately on the CPU)."""
    inp = synth.make_inputs(2, 200, 3, 32, 32, "fp32", seed=14, s0_std=0.1)
    beta = torch.sigmoid(torch.randn(2, 200, 3, 1, generator=torch.Generator().manual_seed(3)))
    inp["b"] = beta.expand(2, 200, 3, 32).contiguous()
    inp["w"] = beta.expand(2, 200, 3, 32).contiguous()
    o, S, _ = _run(inp, 32, single=single)
    o_ref, S_ref = oracle.forward(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["b"], inp["w"], inp["S0"])
    assert rel_err(f64(o), o_ref) <= TOL_F32 and rel_err(f64(S), S_ref) <= TOL_F32


def test_empty_sequence_copies_state():
    B, H, D = 2, 3, 32
    S0 = torch.randn(B, H, D, D, device=DEV)
    z = torch.empty(B, 0, H, D, device=DEV)
    o, S, _ = gdn2_fwd_chunked(z, z, z, z, z, z, S0, chunk=32)
    torch.cuda.synchronize()
    assert o.shape == (B, 0, H, D) and torch.equal(S, S0)
    o, S, _ = gdn2_fwd_chunked(z, z, z, z, z, z, None, chunk=32)
    torch.cuda.synchronize()
    assert torch.count_nonzero(S) == 0


@PATHS
def test_single_token_and_odd_batch(single):
    for T in (1, 17):
        inp = synth.make_inputs(3, T, 5, 128, 64, "bf16", seed=15 + T, s0_std=0.2)
        o, S, _ = _run(inp, 64, single=single)
        o_ref, S_ref = oracle.forward(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["b"], inp["w"], inp["S0"])
        assert rel_err(f64(o), o_ref) <= TOL_BF16 and rel_err(f64(S), S_ref) <= TOL_BF16


@PATHS
def test_nan_propagates(single):
    inp = synth.make_inputs(1, 64, 2, 16, 16, "fp32", seed=16)
    inp["v"][0, 10, 1, 3] = float("nan")
    o, S, _ = _run(inp, 16, single=single)
    assert torch.isnan(o[0, 10:, 1]).any() and torch.isnan(S[0, 1]).any()
    assert not torch.isnan(o[0, :, 0]).any()


@pytest.mark.parametrize("Dk,Dv,C,dtype", [(128, 128, 64, "bf16"), (64, 32, 32, "fp32"), (16, 128, 16, "bf16")])
def test_two_stage_matches_single_pass(Dk, Dv, C, dtype):
    """The two paths perform the same products with the same operand roundings; only the fp32 accumulation
    order differs. With 16-bit operands that can move an operand's rounding by one fp16 ulp (2^-11 relative),
    which the state carries to later chunks, so the bar there is a few ulp; with fp32 operands it is 1e-5."""
    inp = synth.make_inputs(2, 3 * C + 7, 5, Dk, Dv, dtype, seed=17 + C, s0_std=0.1)
    a = _run(inp, C, states=True, single=False)
    b = _run(inp, C, states=True, single=True)
    bar = 1e-5 if dtype == "fp32" else 4e-3
    for x, y in zip(a, b):
        assert rel_err(f64(x), f64(y)) < bar


# Shapes where the two-stage forward takes the two-level (segmented) chain: few (batch, head) pairs and
# at least 32 chunks. The segment maps, their fp32 composition and the re-run from the composed entry
# states must reproduce the stepwise recurrence like the plain chain does.
SEGMENTED = [
    # B, H, T, Dk, Dv, C, dtype
    (1, 2, 33 * 16 + 5, 32, 32, 16, "fp32"),     # 34 chunks, ragged tail, 4 segments
    (1, 3, 40 * 64 + 7, 128, 128, 64, "bf16"),   # d = 128 heads, 5 segments
    (2, 1, 64 * 32, 16, 64, 32, "bf16"),         # Dk = 16: 16 identity columns after 64 value columns
    (1, 2, 48 * 32 + 31, 128, 32, 32, "bf16"),   # map pass of 160 columns: two column groups
    (1, 1, 36 * 32, 64, 128, 32, "fp32"),
    (1, 4, 256 * 16 + 3, 32, 32, 16, "fp32"),   # 257 chunks: 29 segments of 9, a long composition
]


@pytest.mark.parametrize("B,H,T,Dk,Dv,C,dtype", SEGMENTED)
def test_two_level_chain_matches_oracle(B, H, T, Dk, Dv, C, dtype):
    lib = _lib.load()
    code = _lib.GDN2_F32 if dtype == "fp32" else _lib.GDN2_BF16
    nc = (T + C - 1) // C
    plain = B * H * nc * (lib.gdn2_workspace_bytes(_lib.GDN2_OP_FWD, 1, C, 1, Dk, Dv, C, code))
    assert lib.gdn2_workspace_bytes(_lib.GDN2_OP_FWD, B, T, H, Dk, Dv, C, code) > plain  # segment buffers present
    inp = synth.make_inputs(B, T, H, Dk, Dv, dtype, seed=40 + Dk + Dv + C, s0_std=0.3)
    o, S, cs = _run(inp, C, states=True)
    o_ref, S_ref = oracle.forward(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["b"], inp["w"], inp["S0"])
    tol = tol_for(synth.torch_dtype(dtype))
    eo, es = rel_err(f64(o), o_ref), rel_err(f64(S), S_ref)
    print(f"two-level {B}x{H} T={T} Dk={Dk} Dv={Dv} C={C} {dtype}: err o {eo:.2e} S {es:.2e}")
    assert eo <= tol and es <= tol
    # chunk entry states at a few chunks across segment boundaries
    cs64 = f64(cs)
    for n in (1, nc // 3, nc // 2 + 1, nc - 1):
        sl = {k_: v_[:, :n * C] for k_, v_ in inp.items() if k_ != "S0"}
        _, ref = oracle.forward(sl["q"], sl["k"], sl["v"], sl["log_alpha"], sl["b"], sl["w"], inp["S0"])
        assert rel_err(cs64[:, :, n], ref) <= tol, n
    # and it agrees with the single-pass kernel (plain chunk order). With 16-bit operands the bar is wider
    # than for the plain two-stage chain (4e-3, accumulation order only): the two-level chain also rounds
    # the segment maps' own products (M's identity columns and N feed back as fp16 operands) before the
    # fp32 composition, so the paths carry separate roundings, each a few 1e-3 of RMS from the oracle.
    b = _run(inp, C, states=True, single=True)
    bar = 1e-5 if dtype == "fp32" else 1e-2
    for x, y in zip((o, S, cs), b):
        assert rel_err(f64(x), f64(y)) < bar


def test_two_level_chain_is_deterministic():
    inp = synth.make_inputs(1, 2000, 4, 128, 128, "bf16", seed=47, s0_std=0.05)
    o1, S1, c1 = _run(inp, 64, states=True)
    o2, S2, c2 = _run(inp, 64, states=True)
    assert torch.equal(o1, o2) and torch.equal(S1, S2) and torch.equal(c1, c2)
