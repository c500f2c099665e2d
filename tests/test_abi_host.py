"""Host-side checks of the C ABI: the library loads, exports every declared symbol,
and rejects bad arguments before launching anything (no GPU needed)."""

import ctypes
import os
import re

import pytest

from delta_rule_recurrent_gdn_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn2.h")


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char\*)\s+(gdn2_\w+)\s*\(", text, re.M)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert {"gdn2_fwd_chunked", "gdn2_decode_step", "gdn2_bwd_chunked", "gdn2_workspace_bytes",
            "gdn2_status_string", "gdn2_version"} <= set(names)
    lib = _lib.load()
    for n in names:
        assert hasattr(lib, n), n
        assert n in _lib.SIGNATURES, n


def test_status_strings_and_version():
    lib = _lib.load()
    for code in range(0, -8, -1):
        s = lib.gdn2_status_string(code).decode()
        assert s.startswith("GDN2_")
    assert lib.gdn2_status_string(-99).decode() == "unknown gdn2 status"
    assert lib.gdn2_version() >= 200


def test_ex_entry_points_check_flags():
    """The _ex entry points accept GDN2_FLAG_RAW_GATES and reject unknown flag bits before any launch."""
    lib = _lib.load()
    U = _lib.GDN2_ERR_UNSUPPORTED
    fwd = lambda flags, B=1: lib.gdn2_fwd_chunked_ex(A, A, A, A, A, A, None, A, None, None, None, 0, B, 64, 2, 16,  # noqa
                                                      16, 16, 0, flags, None)
    known = (_lib.GDN2_FLAG_RAW_GATES | _lib.GDN2_FLAG_SCALAR_B | _lib.GDN2_FLAG_SCALAR_W |
             _lib.GDN2_FLAG_SCALAR_DECAY)
    assert known == 15
    assert fwd(16) == U and fwd(1 << 31) == U
    assert fwd(known, B=0) == _lib.GDN2_OK and fwd(0, B=0) == _lib.GDN2_OK
    dec = lambda flags, B=4: lib.gdn2_decode_step_ex(A, A, A, A, A, A, A, A, B, 16, 128, 128, 1, flags, None)  # noqa
    assert dec(32) == U and dec(known, B=0) == _lib.GDN2_OK
    bwd = lambda flags, B=1: lib.gdn2_bwd_chunked_ex(A, A, A, A, A, A, None, A, None, None, A, A, A, A, A, A,  # noqa
                                                      None, A, 1 << 20, B, 64, 2, 16, 16, 16, 0, flags, None)
    assert bwd(64) == U and bwd(known, B=0) == _lib.GDN2_OK


def test_workspace_bytes():
    lib = _lib.load()
    B, T, H, D, C = 8, 4096, 16, 128, 64
    nc = T // C
    # backward: exit-state gradients and room for recomputed entry states (one [B,H,NC,D,D] fp32 array
    # each), then a records region that holds the forward records (for a state recompute: 57 units of
    # 1 KB per chunk plus T (w v), fp16 for 16-bit inputs) and later the backward ones (81 units per
    # chunk); for 16-bit inputs, at the end, the partial maxima of the upstream gradients: 8 floats per
    # (batch, head), 256-byte aligned
    rec = lambda n: B * H * n * max(81 * 1024, 57 * 1024 + C * D * 2)  # noqa: E731
    gsc = (B * H * 8 * 4 + 255) // 256 * 256
    assert lib.gdn2_workspace_bytes(_lib.GDN2_OP_BWD, B, T, H, D, D, C, 1) == 2 * nc * B * H * D * D * 4 + rec(nc) + gsc
    # fp32 inputs: no upstream-gradient scaling
    assert lib.gdn2_workspace_bytes(_lib.GDN2_OP_BWD, B, T, H, 64, 64, C, 0) > 0
    # two-stage forward: per chunk a record of 57 units of 1 KB (W, decayed q: 16 each; decayed k^T: 16;
    # causal term: 8; exp(g_last): 1) plus T (w v) in fp16 (fp32 for fp32 inputs)
    assert lib.gdn2_workspace_bytes(_lib.GDN2_OP_FWD, B, T, H, D, D, C, 1) == B * H * nc * (57 * 1024 + C * D * 2)
    # fp32: units of 16 contraction indices, so twice the units (113), and T (w v) the same size
    assert lib.gdn2_workspace_bytes(_lib.GDN2_OP_FWD, B, T, H, D, D, C, 0) == B * H * nc * (113 * 1024 + C * D * 4)
    assert lib.gdn2_workspace_bytes(_lib.GDN2_OP_DECODE, B, 1, H, D, D, C, 1) == 0
    assert lib.gdn2_workspace_bytes(_lib.GDN2_OP_BWD, B, T, H, 48, D, C, 1) == 0   # unsupported size
    # fp32 inputs at d_k = 128, chunk 64: the backward kernels run 32-token chunks (their LDS does not hold
    # 64), so the backward's sizes are those of chunk 32, and the forward workspace also holds the training
    # pair's chunk-32 forward
    for op in (_lib.GDN2_OP_BWD, _lib.GDN2_OP_BWD_RECORDS):
        assert lib.gdn2_workspace_bytes(op, B, T, H, D, D, C, 0) == lib.gdn2_workspace_bytes(op, B, T, H, D, D, 32, 0) > 0
    assert lib.gdn2_records_bytes(B, T, H, D, D, C, 0) == lib.gdn2_records_bytes(B, T, H, D, D, 32, 0) > 0
    assert lib.gdn2_workspace_bytes(_lib.GDN2_OP_FWD, B, T, H, D, D, C, 0) >= \
        lib.gdn2_workspace_bytes(_lib.GDN2_OP_FWD, B, T, H, D, D, 32, 0)
    n = 3
    assert lib.gdn2_varlen_workspace_bytes(_lib.GDN2_OP_BWD, n, T, H, D, D, C, 0) == \
        lib.gdn2_varlen_workspace_bytes(_lib.GDN2_OP_BWD, n, T, H, D, D, 32, 0) > 0
    assert lib.gdn2_varlen_records_bytes(n, T, H, D, D, C, 0) == lib.gdn2_varlen_records_bytes(n, T, H, D, D, 32, 0) > 0
    assert lib.gdn2_workspace_bytes(_lib.GDN2_OP_BWD, B, 100, H, D, D, 64, 1) == 2 * 2 * B * H * D * D * 4 + rec(2) + gsc


def test_workspace_bytes_two_level_forward():
    """Few heads and a long sequence: the forward workspace also holds the two-level chain's segment
    maps M [Dk x Dk], zero-entry exit states N and composed entry states [Dk x Dv] (fp32), 256-byte
    aligned after the records and T (w v). 16 heads x 512 chunks -> 8 segments of 64 chunks; from 1024 chunks
    (segments of 64 chunks or more when doubled) 16 segments."""
    lib = _lib.load()
    D, C = 128, 64
    for B, T, H, G in ((1, 32768, 16, 8), (1, 65536, 16, 16)):
        nc = T // C
        base = B * H * nc * (57 * 1024 + C * D * 2)
        seg = B * H * G * (D * D + 2 * D * D) * 4
        assert lib.gdn2_workspace_bytes(_lib.GDN2_OP_FWD, B, T, H, D, D, C, 1) == (base + 255) // 256 * 256 + seg
    # 128 heads fill the GPU with the plain chain: no segment buffers (the B=8 H=16 T=4096 training figure above)
    assert lib.gdn2_workspace_bytes(_lib.GDN2_OP_FWD, 8, 4096, 16, D, D, C, 1) == 8 * 16 * 64 * (57 * 1024 + C * D * 2)
    # fewer than 32 chunks: no segments
    assert lib.gdn2_workspace_bytes(_lib.GDN2_OP_FWD, 1, 31 * C, 2, D, D, C, 1) == 2 * 31 * (57 * 1024 + C * D * 2)


A = 4096  # a fake, 16-byte aligned address: never dereferenced because validation fails first


def fwd(**kw):
    args = dict(q=A, k=A, v=A, la=A, b=A, w=A, S0=None, o=A, Sf=None, cs=None, ws=None, ws_bytes=0, B=1, T=64,
                H=2, Dk=16, Dv=16, C=16, dt=0)
    args.update(kw)
    return _lib.load().gdn2_fwd_chunked(args["q"], args["k"], args["v"], args["la"], args["b"], args["w"],
                                        args["S0"], args["o"], args["Sf"], args["cs"], args["ws"], args["ws_bytes"],
                                        args["B"], args["T"], args["H"], args["Dk"], args["Dv"], args["C"],
                                        args["dt"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), _lib.GDN2_ERR_NULL),
    (dict(o=None), _lib.GDN2_ERR_NULL),
    (dict(k=A + 8), _lib.GDN2_ERR_ALIGN),
    (dict(Sf=A + 4), _lib.GDN2_ERR_ALIGN),
    (dict(dt=7), _lib.GDN2_ERR_DTYPE),
    (dict(Dk=48), _lib.GDN2_ERR_UNSUPPORTED),
    (dict(Dv=256), _lib.GDN2_ERR_UNSUPPORTED),
    (dict(C=128), _lib.GDN2_ERR_UNSUPPORTED),
    (dict(T=-1), _lib.GDN2_ERR_SHAPE),
    (dict(B=-2), _lib.GDN2_ERR_SHAPE),
    (dict(ws=A, ws_bytes=1), _lib.GDN2_ERR_WORKSPACE),              # two-stage path: workspace too small
    (dict(ws=A + 16, ws_bytes=1 << 30), _lib.GDN2_ERR_ALIGN),       # workspace must be 256-byte aligned
    (dict(B=0), _lib.GDN2_OK),                                       # nothing to do, nothing launched
    (dict(H=0), _lib.GDN2_OK),
])
def test_fwd_argument_errors(kw, status):
    assert fwd(**kw) == status


def test_decode_argument_errors():
    lib = _lib.load()
    call = lambda S=A, dt=1, Dk=128, Dv=128, B=4: lib.gdn2_decode_step(A, A, A, A, A, A, S, A, B, 16, Dk, Dv, dt,  # noqa
                                                                      None)
    assert call(S=None) == _lib.GDN2_ERR_NULL
    assert call(S=A + 2) == _lib.GDN2_ERR_ALIGN
    assert call(dt=5) == _lib.GDN2_ERR_DTYPE
    assert call(Dk=100) == _lib.GDN2_ERR_UNSUPPORTED
    assert call(B=0) == _lib.GDN2_OK


def test_error_raised_by_binding_names_the_status():
    e = _lib.GDN2Error(_lib.GDN2_ERR_WORKSPACE, "gdn2_bwd_chunked")
    assert "GDN2_ERR_WORKSPACE" in str(e) and e.status == _lib.GDN2_ERR_WORKSPACE


def test_signature_table_matches_header_arity():
    text = open(HEADER).read()
    for name, (_, args) in _lib.SIGNATURES.items():
        m = re.search(r"^\s*(?:int|size_t|const char\*)\s+" + name + r"\s*\(([^;]*)\);", text, re.S | re.M)
        assert m, name
        params = [p for p in m.group(1).split(",") if p.strip() and p.strip() != "void"]
        assert len(params) == len(args), name
    assert ctypes.sizeof(ctypes.c_size_t) == 8


def test_bwd_argument_errors():
    lib = _lib.load()

    def call(ws=A, ws_bytes=1 << 20, dO=A, dq=A, C=16, dt=0):
        return lib.gdn2_bwd_chunked(A, A, A, A, A, A, None, dO, None, None, dq, A, A, A, A, A, None, ws, ws_bytes,
                                    1, 64, 2, 16, 16, C, dt, None)

    need = lib.gdn2_workspace_bytes(_lib.GDN2_OP_BWD, 1, 64, 2, 16, 16, 16, 0)
    assert call(ws_bytes=need - 1) == _lib.GDN2_ERR_WORKSPACE
    assert call(ws=None) == _lib.GDN2_ERR_WORKSPACE
    assert call(ws=A + 16, ws_bytes=need) == _lib.GDN2_ERR_ALIGN      # workspace must be 256-byte aligned
    assert call(dO=None) == _lib.GDN2_ERR_NULL
    assert call(dq=A + 4) == _lib.GDN2_ERR_ALIGN
    assert call(C=48) == _lib.GDN2_ERR_UNSUPPORTED
    assert call(dt=3) == _lib.GDN2_ERR_DTYPE


def test_training_pair_sizes_and_argument_errors():
    """gdn2_records_bytes: per chunk the backward record (57 units of 1 KB for the reverse chain, then
    T: 8 and the decayed b*k: 16, at d = 128, chunk 64, bf16), then every chunk's entry state (fp16 for
    16-bit inputs); the backward from records needs only the exit-state gradients. Both calls check their
    buffers before launching."""
    lib = _lib.load()
    B, T, H, D, C = 8, 4096, 16, 128, 64
    nc = T // C
    rb = lib.gdn2_records_bytes(B, T, H, D, D, C, 1)
    assert rb == B * H * nc * 81 * 1024 + B * H * nc * D * D * 2
    assert lib.gdn2_workspace_bytes(_lib.GDN2_OP_BWD_RECORDS, B, T, H, D, D, C, 1) == B * H * nc * D * D * 4 + B * H * 32
    assert lib.gdn2_records_bytes(B, T, H, 48, D, C, 1) == 0 and lib.gdn2_records_bytes(B, 0, H, D, D, C, 1) == 0
    # fp32 inputs keep fp32 entry states
    rb32 = lib.gdn2_records_bytes(1, 64, 2, 16, 16, 16, 0)
    rb16 = lib.gdn2_records_bytes(1, 64, 2, 16, 16, 16, 1)
    assert rb32 > 0 and rb16 > 0
    rb = rb32
    fw = lib.gdn2_workspace_bytes(_lib.GDN2_OP_FWD, 1, 64, 2, 16, 16, 16, 0)
    bw = lib.gdn2_workspace_bytes(_lib.GDN2_OP_BWD_RECORDS, 1, 64, 2, 16, 16, 16, 0)
    assert fw > 0 and bw > 0

    def fwd(rec=A, rec_bytes=rb, ws=A, ws_bytes=fw, flags=0, B=1, T=64):
        return lib.gdn2_fwd_chunked_train(A, A, A, A, A, A, None, A, None, rec, rec_bytes, ws, ws_bytes, B, T, 2, 16,
                                          16, 16, 0, flags, None)

    def bwd(rec=A, rec_bytes=rb, ws=A, ws_bytes=bw, flags=0):
        return lib.gdn2_bwd_chunked_records(A, A, A, A, A, A, A, None, rec, rec_bytes, A, A, A, A, A, A, None, ws,
                                            ws_bytes, 1, 64, 2, 16, 16, 16, 0, flags, None)

    for call in (fwd, bwd):
        assert call(rec=None) == _lib.GDN2_ERR_NULL
        assert call(rec_bytes=rb - 1) == _lib.GDN2_ERR_WORKSPACE
        assert call(ws=None) == _lib.GDN2_ERR_WORKSPACE
        assert call(rec=A + 16) == _lib.GDN2_ERR_ALIGN       # records 256-byte aligned
        assert call(ws=A + 16) == _lib.GDN2_ERR_ALIGN
        assert call(flags=16) == _lib.GDN2_ERR_UNSUPPORTED
    assert fwd(ws_bytes=fw - 1) == _lib.GDN2_ERR_WORKSPACE
    assert bwd(ws_bytes=bw - 1) == _lib.GDN2_ERR_WORKSPACE
    assert fwd(B=0) == _lib.GDN2_OK
    # fp32 inputs at d = 128, chunk 64 are accepted (run as 32-token chunks) and checked against those sizes
    assert lib.gdn2_fwd_chunked_train(A, A, A, A, A, A, None, A, None, A, rb, A, fw, 1, 64, 2, 128, 128, 64, 0, 0,
                                      None) == _lib.GDN2_ERR_WORKSPACE


def test_packed_training_pair_sizes_and_argument_errors():
    """gdn2_varlen_records_bytes: backward records and entry states over [H][max_chunks]; the backward from
    records needs the packed-batch tables and the state gradients only."""
    lib = _lib.load()
    N, T, H, D, C = 7, 32768, 16, 128, 64
    mc = lib.gdn2_varlen_max_chunks(N, T, C)
    rb = lib.gdn2_varlen_records_bytes(N, T, H, D, D, C, 1)
    rec = (H * mc * 81 * 1024 + 255) // 256 * 256
    assert rb == rec + H * mc * D * D * 2
    bw = lib.gdn2_varlen_workspace_bytes(_lib.GDN2_OP_BWD_RECORDS, N, T, H, D, D, C, 1)
    assert 0 < bw < lib.gdn2_varlen_workspace_bytes(_lib.GDN2_OP_BWD, N, T, H, D, D, C, 1)
    assert lib.gdn2_varlen_records_bytes(N, T, H, 48, D, C, 1) == 0
    rb = lib.gdn2_varlen_records_bytes(3, 64, 2, 16, 16, 16, 0)
    fw = lib.gdn2_varlen_workspace_bytes(_lib.GDN2_OP_FWD, 3, 64, 2, 16, 16, 16, 0)
    bw = lib.gdn2_varlen_workspace_bytes(_lib.GDN2_OP_BWD_RECORDS, 3, 64, 2, 16, 16, 16, 0)

    def fwd(rec=A, rec_bytes=rb, ws=A, ws_bytes=fw, cu=A, N=3):
        return lib.gdn2_fwd_varlen_train(A, A, A, A, A, A, cu, N, None, A, None, rec, rec_bytes, ws, ws_bytes, 64, 2,
                                         16, 16, 16, 0, 0, None)

    def bwd(rec=A, rec_bytes=rb, ws=A, ws_bytes=bw, cu=A, N=3):
        return lib.gdn2_bwd_varlen_records(A, A, A, A, A, A, cu, N, A, None, rec, rec_bytes, A, A, A, A, A, A, None,
                                           ws, ws_bytes, 64, 2, 16, 16, 16, 0, 0, None)

    for call, need in ((fwd, fw), (bwd, bw)):
        assert call(rec=None) == _lib.GDN2_ERR_NULL
        assert call(cu=None) == _lib.GDN2_ERR_NULL
        assert call(cu=A + 4) == _lib.GDN2_ERR_ALIGN          # offsets 8-byte aligned
        assert call(rec_bytes=rb - 1) == _lib.GDN2_ERR_WORKSPACE
        assert call(ws_bytes=need - 1) == _lib.GDN2_ERR_WORKSPACE
        assert call(rec=A + 16) == _lib.GDN2_ERR_ALIGN
        assert call(N=0) == _lib.GDN2_OK


def test_noalloc_array_size_matches_header_and_refuses_oversize():
    """GDN2_NOALLOC_SCRATCH_BYTES agrees between the header and the binding, and sizes whose forward workspace
    exceeds it are refused on the host, before any device call (the pointers are never dereferenced)."""
    text = open(HEADER).read()
    m = re.search(r"#define\s+GDN2_NOALLOC_SCRATCH_BYTES\s+\((\d+)u\s*\*\s*(\d+)u\s*\*\s*(\d+)u\)", text)
    assert m, "the header defines the array size"
    size = int(m.group(1)) * int(m.group(2)) * int(m.group(3))
    assert size == _lib.GDN2_NOALLOC_SCRATCH_BYTES
    lib = _lib.load()
    B, T, H, D, C = 8, 4096, 16, 128, 64
    assert lib.gdn2_workspace_bytes(_lib.GDN2_OP_FWD, B, T, H, D, D, C, _lib.GDN2_BF16) > size
    fake = ctypes.c_void_p(1 << 20)  # 16-byte aligned, never dereferenced
    st = lib.gdn2_fwd_chunked_noalloc(*([fake] * 10), B, T, H, D, D, C, _lib.GDN2_BF16, None)
    assert st == _lib.GDN2_ERR_WORKSPACE
