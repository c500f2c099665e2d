"""gdn2_fwd_chunked_noalloc through the C ABI: identical to gdn2_fwd_chunked with a caller workspace.

The no-allocation entry point runs the same two-stage kernels with the workspace in the library's own device
array, so every output must match gdn2_fwd_chunked bit for bit. Two calls in a row, the second with a smaller
input (fewer chunks, smaller key width, fp32 inputs), check that the array's contents from the first call do
not leak into the second; a third call at the first call's sizes checks the reverse order.
"""

import ctypes

import numpy as np
import pytest
import torch

import oracle
import synth
from delta_rule_recurrent_gdn_amd import _lib
from tests.helpers import TOL_BF16, TOL_F32, f64, rel_err

pytestmark = pytest.mark.gpu

_DT = {"bf16": _lib.GDN2_BF16, "fp32": _lib.GDN2_F32}


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _run(lib, inp, dtype, chunk, noalloc):
    d = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    B, T, H, Dk = d["q"].shape
    Dv = d["v"].shape[-1]
    NC = (T + chunk - 1) // chunk
    o = torch.full((B, T, H, Dv), float("nan"), dtype=torch.float32, device="cuda")
    S = torch.full((B, H, Dk, Dv), float("nan"), dtype=torch.float32, device="cuda")
    cs = torch.full((B, H, NC, Dk, Dv), float("nan"), dtype=torch.float32, device="cuda")
    head = (_p(d["q"]), _p(d["k"]), _p(d["v"]), _p(d["log_alpha"]), _p(d["b"]), _p(d["w"]), _p(d["S0"]), _p(o),
            _p(S), _p(cs))
    sizes = (B, T, H, Dk, Dv, chunk, _DT[dtype])
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if noalloc:
        st = lib.gdn2_fwd_chunked_noalloc(*head, *sizes, stream)
    else:
        need = lib.gdn2_workspace_bytes(_lib.GDN2_OP_FWD, *sizes)
        assert 0 < need <= _lib.GDN2_NOALLOC_SCRATCH_BYTES
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        st = lib.gdn2_fwd_chunked(*head, _p(ws), need, *sizes, stream)
    _lib.check(st, "gdn2_fwd_chunked_noalloc" if noalloc else "gdn2_fwd_chunked")
    torch.cuda.synchronize()
    return o, S, cs


CASES = [  # (B, T, H, Dk, Dv, chunk, dtype, seed): the second and third are smaller than the first
    (2, 4 * 64 + 23, 3, 128, 128, 64, "bf16", 71),
    (1, 2 * 32 + 5, 2, 64, 32, 32, "fp32", 72),
    (1, 17, 1, 32, 64, 16, "bf16", 73),
]


def test_noalloc_matches_workspace_entry_point():
    lib = _lib.load()
    for case in CASES + CASES[:1]:
        B, T, H, Dk, Dv, chunk, dtype, seed = case
        print("case", case, flush=True)
        inp = synth.make_inputs(B, T, H, Dk, Dv, dtype, seed=seed, s0_std=0.3)
        ref = _run(lib, inp, dtype, chunk, noalloc=False)
        got = _run(lib, inp, dtype, chunk, noalloc=True)
        for name, x, y in zip(("o", "S_final", "chunk_states"), got, ref):
            assert torch.equal(x, y), (case, name, float((x - y).abs().max()))
        o_ref, S_ref = oracle.forward(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["b"], inp["w"], inp["S0"])
        tol = TOL_F32 if dtype == "fp32" else TOL_BF16
        assert rel_err(f64(got[0]), o_ref) <= tol and rel_err(f64(got[1]), S_ref) <= tol, case


def test_noalloc_rejects_sizes_beyond_the_array():
    lib = _lib.load()
    B, T, H, D, C = 8, 4096, 16, 128, 64
    need = lib.gdn2_workspace_bytes(_lib.GDN2_OP_FWD, B, T, H, D, D, C, _lib.GDN2_BF16)
    assert need > _lib.GDN2_NOALLOC_SCRATCH_BYTES
    x = torch.zeros(16, device="cuda")  # never read: the size check comes first
    st = lib.gdn2_fwd_chunked_noalloc(*([_p(x)] * 10), B, T, H, D, D, C, _lib.GDN2_BF16,
                                      ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == _lib.GDN2_ERR_WORKSPACE


def test_noalloc_python_binding():
    """The binding with caller-owned outputs: same bits as gdn2_fwd_chunked with its own workspace."""
    from delta_rule_recurrent_gdn_amd import gdn2_fwd_chunked, gdn2_fwd_chunked_noalloc

    inp = synth.make_inputs(1, 3 * 64 + 9, 2, 64, 64, "bf16", seed=74, s0_std=0.3)
    d = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    x = (d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"])
    o = torch.empty(1, 3 * 64 + 9, 2, 64, device="cuda")
    S = torch.empty(1, 2, 64, 64, device="cuda")
    gdn2_fwd_chunked_noalloc(*x, o, S0=d["S0"], S_final=S, chunk=64)
    o_ref, S_ref, _ = gdn2_fwd_chunked(*x, d["S0"], chunk=64)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(S, S_ref)
