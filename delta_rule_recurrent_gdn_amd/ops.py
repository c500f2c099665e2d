"""Thin torch binding of the GDN-2 C ABI (argument marshalling only).

Each function has the name of the C entry point it calls. torch supplies the
device memory and the current stream; every step of the computation runs in
the HIP kernels of libgdn2.so. Layouts and semantics are those of
include/gdn2.h:

    q, k, b, log_alpha : [B, T, H, Dk]     v, w, dO : [B, T, H, Dv]
    states             : [B, H, Dk, Dv] fp32
"""

import torch

from . import _lib

_DT = {torch.float32: _lib.GDN2_F32, torch.bfloat16: _lib.GDN2_BF16}


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(device):
    return torch.cuda.current_stream(device).cuda_stream


def _check_inputs(names, tensors, dtype, device):
    for n, t in zip(names, tensors):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{n} must be a torch.Tensor")
        if t.device != device:
            raise ValueError(f"{n} is on {t.device}, expected {device}")
        if not t.is_contiguous():
            raise ValueError(f"{n} must be contiguous")
        if t.dtype != dtype:
            raise TypeError(f"{n} has dtype {t.dtype}, expected {dtype}")


def _f32_state(t, name, device, shape):
    if t is None:
        return None
    if t.dtype != torch.float32 or t.device != device or not t.is_contiguous() or tuple(t.shape) != shape:
        raise ValueError(f"{name} must be a contiguous fp32 {shape} tensor on {device}")
    return t


def _flags(raw_gates, scalar_b, scalar_w, scalar_decay):
    return ((_lib.GDN2_FLAG_RAW_GATES if raw_gates else 0) | (_lib.GDN2_FLAG_SCALAR_B if scalar_b else 0) |
            (_lib.GDN2_FLAG_SCALAR_W if scalar_w else 0) | (_lib.GDN2_FLAG_SCALAR_DECAY if scalar_decay else 0))


def _gate_shapes(lead, Dk, Dv, scalar_b, scalar_w, scalar_decay):
    """Expected shapes of b, w, log_alpha: per channel, or one value per (token, head) when scalar."""
    return {"b": lead if scalar_b else lead + (Dk,), "w": lead if scalar_w else lead + (Dv,),
            "log_alpha": lead if scalar_decay else lead + (Dk,)}


def _dtype_code(dtype):
    if dtype not in _DT:
        raise TypeError(f"inputs must be float32 or bfloat16, got {dtype}")
    return _DT[dtype]


def gdn2_fwd_chunked(q, k, v, log_alpha, b, w, S0=None, chunk=64, want_final_state=True,
                     want_chunk_states=False, single_pass=False, workspace=None, raw_gates=False, scalar_b=False,
                     scalar_w=False, scalar_decay=False):
    """Chunked forward. Returns (o, S_final or None, chunk_states or None).

    By default the two-stage path runs (chunk-parallel factors into a workspace,
    then the sequential state chain); `workspace` may supply that scratch (a
    uint8 device tensor of at least gdn2_workspace_bytes(GDN2_OP_FWD, ...)
    bytes), else it is allocated here. single_pass=True runs the one-kernel
    path, which needs no workspace. raw_gates=True passes b, w, log_alpha as
    pre-activations (gdn2_fwd_chunked_ex with GDN2_FLAG_RAW_GATES); scalar_b / scalar_w /
    scalar_decay pass that gate as one value per (token, head), [B, T, H] (GDN2_FLAG_SCALAR_*)."""
    lib = _lib.load()
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    dev = q.device
    _check_inputs(("q", "k", "b"), (q, k, b), q.dtype, dev)
    _check_inputs(("v", "w"), (v, w), q.dtype, dev)
    _check_inputs(("log_alpha",), (log_alpha,), torch.float32, dev)
    gs = _gate_shapes((B, T, H), Dk, Dv, scalar_b, scalar_w, scalar_decay)
    for n, t, shp in (("k", k, (B, T, H, Dk)), ("v", v, (B, T, H, Dv)), ("b", b, gs["b"]), ("w", w, gs["w"]),
                      ("log_alpha", log_alpha, gs["log_alpha"])):
        if tuple(t.shape) != shp:
            raise ValueError(f"{n} has shape {tuple(t.shape)}, expected {shp}")
    S0 = _f32_state(S0, "S0", dev, (B, H, Dk, Dv))
    o = torch.empty((B, T, H, Dv), dtype=torch.float32, device=dev)
    S_final = torch.empty((B, H, Dk, Dv), dtype=torch.float32, device=dev) if want_final_state else None
    NC = (T + chunk - 1) // chunk
    states = (torch.empty((B, H, NC, Dk, Dv), dtype=torch.float32, device=dev) if want_chunk_states else None)
    need = 0 if single_pass else lib.gdn2_workspace_bytes(_lib.GDN2_OP_FWD, B, T, H, Dk, Dv, chunk,
                                                           _dtype_code(q.dtype))
    if need == 0:
        workspace = None
    elif workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(b), _ptr(w), _ptr(S0), _ptr(o), _ptr(S_final),
            _ptr(states), _ptr(workspace), ws_bytes, B, T, H, Dk, Dv, chunk, _dtype_code(q.dtype))
    flags = _flags(raw_gates, scalar_b, scalar_w, scalar_decay)
    if flags:
        st = lib.gdn2_fwd_chunked_ex(*args, flags, _stream(dev))
        _lib.check(st, "gdn2_fwd_chunked_ex")
    else:
        st = lib.gdn2_fwd_chunked(*args, _stream(dev))
        _lib.check(st, "gdn2_fwd_chunked")
    return o, S_final, states


def gdn2_fwd_chunked_noalloc(q, k, v, log_alpha, b, w, o, S0=None, S_final=None, chunk_states=None, chunk=64):
    """gdn2_fwd_chunked_noalloc: the two-stage forward with its workspace in the library's own device array
    (GDN2_NOALLOC_SCRATCH_BYTES per GPU), for callers that cannot allocate. Every output is the caller's:
    o [B, T, H, Dv] fp32, and S_final [B, H, Dk, Dv] / chunk_states [B, H, NC, Dk, Dv] fp32 when given. Sizes
    whose forward workspace exceeds the array raise (GDN2_ERR_WORKSPACE). Calls that overlap on one GPU race.
    Returns (o, S_final, chunk_states)."""
    lib = _lib.load()
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    dev = q.device
    _check_inputs(("q", "k", "b"), (q, k, b), q.dtype, dev)
    _check_inputs(("v", "w"), (v, w), q.dtype, dev)
    _check_inputs(("log_alpha",), (log_alpha,), torch.float32, dev)
    NC = (T + chunk - 1) // chunk
    for n, t, shp in (("k", k, (B, T, H, Dk)), ("b", b, (B, T, H, Dk)), ("log_alpha", log_alpha, (B, T, H, Dk)),
                      ("v", v, (B, T, H, Dv)), ("w", w, (B, T, H, Dv)), ("o", o, (B, T, H, Dv)),
                      ("S_final", S_final, (B, H, Dk, Dv)), ("chunk_states", chunk_states, (B, H, NC, Dk, Dv))):
        if t is not None and tuple(t.shape) != shp:
            raise ValueError(f"{n} has shape {tuple(t.shape)}, expected {shp}")
    for n, t in (("o", o), ("S_final", S_final), ("chunk_states", chunk_states)):
        if t is not None and (t.dtype != torch.float32 or t.device != dev or not t.is_contiguous()):
            raise ValueError(f"{n} must be a contiguous float32 tensor on {dev}")
    S0 = _f32_state(S0, "S0", dev, (B, H, Dk, Dv))
    st = lib.gdn2_fwd_chunked_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(b), _ptr(w), _ptr(S0),
                                      _ptr(o), _ptr(S_final), _ptr(chunk_states), B, T, H, Dk, Dv, chunk,
                                      _dtype_code(q.dtype), _stream(dev))
    _lib.check(st, "gdn2_fwd_chunked_noalloc")
    return o, S_final, chunk_states


def gdn2_decode_step(q, k, v, log_alpha, b, w, S, o=None, raw_gates=False, scalar_b=False, scalar_w=False,
                     scalar_decay=False):
    """One decode step; S ([B,H,Dk,Dv] fp32) is updated in place. Returns o [B,H,Dv] fp32.
    raw_gates=True passes b, w, log_alpha as pre-activations (gdn2_decode_step_ex)."""
    lib = _lib.load()
    B, H, Dk = q.shape
    Dv = v.shape[-1]
    dev = q.device
    _check_inputs(("q", "k", "b"), (q, k, b), q.dtype, dev)
    _check_inputs(("v", "w"), (v, w), q.dtype, dev)
    _check_inputs(("log_alpha",), (log_alpha,), torch.float32, dev)
    _f32_state(S, "S", dev, (B, H, Dk, Dv))
    if o is None:
        o = torch.empty((B, H, Dv), dtype=torch.float32, device=dev)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(b), _ptr(w), _ptr(S), _ptr(o), B, H, Dk, Dv,
            _dtype_code(q.dtype))
    flags = _flags(raw_gates, scalar_b, scalar_w, scalar_decay)
    if flags:
        st = lib.gdn2_decode_step_ex(*args, flags, _stream(dev))
        _lib.check(st, "gdn2_decode_step_ex")
    else:
        st = lib.gdn2_decode_step(*args, _stream(dev))
        _lib.check(st, "gdn2_decode_step")
    return o


def gdn2_workspace_bytes(op, B, T, H, Dk, Dv, chunk, dtype):
    return _lib.load().gdn2_workspace_bytes(op, B, T, H, Dk, Dv, chunk, _dtype_code(dtype))


def gdn2_bwd_chunked(q, k, v, log_alpha, b, w, dO, S0=None, dS_final=None, chunk_states=None, chunk=64,
                     want_dS0=True, workspace=None, raw_gates=False, scalar_b=False, scalar_w=False,
                     scalar_decay=False):
    """Chunked backward. Returns a dict with dq, dk, dv, dlog_alpha, db, dw (fp32) and dS0 (or None).
    raw_gates=True: b, w, log_alpha are pre-activations and db, dw, dlog_alpha the gradients with
    respect to them (gdn2_bwd_chunked_ex with GDN2_FLAG_RAW_GATES)."""
    lib = _lib.load()
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    dev = q.device
    _check_inputs(("q", "k", "b"), (q, k, b), q.dtype, dev)
    _check_inputs(("v", "w", "dO"), (v, w, dO), q.dtype, dev)
    _check_inputs(("log_alpha",), (log_alpha,), torch.float32, dev)
    S0 = _f32_state(S0, "S0", dev, (B, H, Dk, Dv))
    dS_final = _f32_state(dS_final, "dS_final", dev, (B, H, Dk, Dv))
    NC = (T + chunk - 1) // chunk
    chunk_states = _f32_state(chunk_states, "chunk_states", dev, (B, H, NC, Dk, Dv))
    kshape, vshape = (B, T, H, Dk), (B, T, H, Dv)
    gs = _gate_shapes((B, T, H), Dk, Dv, scalar_b, scalar_w, scalar_decay)
    g = {n: torch.empty(kshape, dtype=torch.float32, device=dev) for n in ("dq", "dk")}
    g["dv"] = torch.empty(vshape, dtype=torch.float32, device=dev)
    g.update({"d" + n: torch.empty(gs[n], dtype=torch.float32, device=dev) for n in ("b", "w", "log_alpha")})
    g["dS0"] = torch.empty((B, H, Dk, Dv), dtype=torch.float32, device=dev) if want_dS0 else None
    need = lib.gdn2_workspace_bytes(_lib.GDN2_OP_BWD, B, T, H, Dk, Dv, chunk, _dtype_code(q.dtype))
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(b), _ptr(w), _ptr(S0), _ptr(dO), _ptr(dS_final),
            _ptr(chunk_states), _ptr(g["dq"]), _ptr(g["dk"]), _ptr(g["dv"]), _ptr(g["dlog_alpha"]), _ptr(g["db"]),
            _ptr(g["dw"]), _ptr(g["dS0"]), _ptr(workspace), workspace.numel() * workspace.element_size(), B, T, H,
            Dk, Dv, chunk, _dtype_code(q.dtype))
    flags = _flags(raw_gates, scalar_b, scalar_w, scalar_decay)
    if flags:
        st = lib.gdn2_bwd_chunked_ex(*args, flags, _stream(dev))
        _lib.check(st, "gdn2_bwd_chunked_ex")
    else:
        st = lib.gdn2_bwd_chunked(*args, _stream(dev))
        _lib.check(st, "gdn2_bwd_chunked")
    return g


def gdn2_records_bytes(B, T, H, Dk, Dv, chunk, dtype):
    return _lib.load().gdn2_records_bytes(B, T, H, Dk, Dv, chunk, _dtype_code(dtype))


def _scratch(t, need, dev):
    """`t` if it is a device byte buffer of at least `need` bytes, else a new one."""
    if t is None or t.numel() * t.element_size() < need:
        t = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    return t


def _nbytes(t):
    return t.numel() * t.element_size()


def gdn2_fwd_chunked_train(q, k, v, log_alpha, b, w, S0=None, chunk=64, want_final_state=True, workspace=None,
                           records=None, raw_gates=False, scalar_b=False, scalar_w=False, scalar_decay=False):
    """Training forward (gdn2_fwd_chunked_train): the two-stage forward whose chunk-parallel pass also writes
    the backward's per-chunk records and whose chain stores every chunk's entry state with them. Returns
    (o, S_final or None, records); pass records to gdn2_bwd_chunked_records with the same inputs.
    `workspace` and `records` may supply the buffers (uint8 device tensors of at least
    gdn2_workspace_bytes(GDN2_OP_FWD, ...) and gdn2_records_bytes(...) bytes)."""
    lib = _lib.load()
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    dev = q.device
    _check_inputs(("q", "k", "b"), (q, k, b), q.dtype, dev)
    _check_inputs(("v", "w"), (v, w), q.dtype, dev)
    _check_inputs(("log_alpha",), (log_alpha,), torch.float32, dev)
    gs = _gate_shapes((B, T, H), Dk, Dv, scalar_b, scalar_w, scalar_decay)
    for n, t, shp in (("k", k, (B, T, H, Dk)), ("v", v, (B, T, H, Dv)), ("b", b, gs["b"]), ("w", w, gs["w"]),
                      ("log_alpha", log_alpha, gs["log_alpha"])):
        if tuple(t.shape) != shp:
            raise ValueError(f"{n} has shape {tuple(t.shape)}, expected {shp}")
    S0 = _f32_state(S0, "S0", dev, (B, H, Dk, Dv))
    o = torch.empty((B, T, H, Dv), dtype=torch.float32, device=dev)
    S_final = torch.empty((B, H, Dk, Dv), dtype=torch.float32, device=dev) if want_final_state else None
    dt = _dtype_code(q.dtype)
    workspace = _scratch(workspace, lib.gdn2_workspace_bytes(_lib.GDN2_OP_FWD, B, T, H, Dk, Dv, chunk, dt), dev)
    records = _scratch(records, lib.gdn2_records_bytes(B, T, H, Dk, Dv, chunk, dt), dev)
    st = lib.gdn2_fwd_chunked_train(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(b), _ptr(w), _ptr(S0), _ptr(o),
                                    _ptr(S_final), _ptr(records), _nbytes(records), _ptr(workspace),
                                    _nbytes(workspace), B, T, H, Dk, Dv, chunk, dt,
                                    _flags(raw_gates, scalar_b, scalar_w, scalar_decay), _stream(dev))
    _lib.check(st, "gdn2_fwd_chunked_train")
    return o, S_final, records


def gdn2_bwd_chunked_records(q, k, v, log_alpha, b, w, dO, records, dS_final=None, chunk=64, want_dS0=True,
                             workspace=None, raw_gates=False, scalar_b=False, scalar_w=False, scalar_decay=False):
    """Backward from the training forward's records (gdn2_bwd_chunked_records): the reverse chain and the
    per-chunk gradients, without the backward's own record pass. Returns the dict of gdn2_bwd_chunked."""
    lib = _lib.load()
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    dev = q.device
    _check_inputs(("q", "k", "b"), (q, k, b), q.dtype, dev)
    _check_inputs(("v", "w", "dO"), (v, w, dO), q.dtype, dev)
    _check_inputs(("log_alpha",), (log_alpha,), torch.float32, dev)
    dS_final = _f32_state(dS_final, "dS_final", dev, (B, H, Dk, Dv))
    if records is None or records.device != dev or records.dtype != torch.uint8:
        raise ValueError("records must be the uint8 device tensor returned by gdn2_fwd_chunked_train")
    gs = _gate_shapes((B, T, H), Dk, Dv, scalar_b, scalar_w, scalar_decay)
    g = {n: torch.empty((B, T, H, Dk), dtype=torch.float32, device=dev) for n in ("dq", "dk")}
    g["dv"] = torch.empty((B, T, H, Dv), dtype=torch.float32, device=dev)
    g.update({"d" + n: torch.empty(gs[n], dtype=torch.float32, device=dev) for n in ("b", "w", "log_alpha")})
    g["dS0"] = torch.empty((B, H, Dk, Dv), dtype=torch.float32, device=dev) if want_dS0 else None
    dt = _dtype_code(q.dtype)
    workspace = _scratch(workspace, lib.gdn2_workspace_bytes(_lib.GDN2_OP_BWD_RECORDS, B, T, H, Dk, Dv, chunk, dt),
                         dev)
    st = lib.gdn2_bwd_chunked_records(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(b), _ptr(w), _ptr(dO),
                                      _ptr(dS_final), _ptr(records), _nbytes(records), _ptr(g["dq"]), _ptr(g["dk"]),
                                      _ptr(g["dv"]), _ptr(g["dlog_alpha"]), _ptr(g["db"]), _ptr(g["dw"]),
                                      _ptr(g["dS0"]), _ptr(workspace), _nbytes(workspace), B, T, H, Dk, Dv, chunk,
                                      dt, _flags(raw_gates, scalar_b, scalar_w, scalar_decay), _stream(dev))
    _lib.check(st, "gdn2_bwd_chunked_records")
    return g


def gdn2_varlen_max_chunks(N, T, chunk):
    return _lib.load().gdn2_varlen_max_chunks(N, T, chunk)


def gdn2_fwd_varlen(q, k, v, log_alpha, b, w, cu_seqlens, S0=None, chunk=64, want_final_state=True,
                    want_chunk_states=False, workspace=None, raw_gates=False, scalar_b=False, scalar_w=False,
                    scalar_decay=False):
    """Packed variable-length forward: q, k, b, log_alpha [1,T,H,Dk], v, w [1,T,H,Dv]; cu_seqlens int64 [N+1]
    on the device. Returns (o [1,T,H,Dv], S_final [N,H,Dk,Dv] or None, chunk_states
    [H, max_chunks, Dk, Dv] or None)."""
    lib = _lib.load()
    _, T, H, Dk = q.shape
    Dv = v.shape[-1]
    dev = q.device
    _check_inputs(("q", "k", "b"), (q, k, b), q.dtype, dev)
    _check_inputs(("v", "w"), (v, w), q.dtype, dev)
    _check_inputs(("log_alpha",), (log_alpha,), torch.float32, dev)
    _check_inputs(("cu_seqlens",), (cu_seqlens,), torch.int64, dev)
    N = cu_seqlens.numel() - 1
    S0 = _f32_state(S0, "S0", dev, (N, H, Dk, Dv))
    o = torch.zeros((1, T, H, Dv), dtype=torch.float32, device=dev)
    S_final = torch.empty((N, H, Dk, Dv), dtype=torch.float32, device=dev) if want_final_state else None
    mc = lib.gdn2_varlen_max_chunks(N, T, chunk)
    states = torch.empty((H, mc, Dk, Dv), dtype=torch.float32, device=dev) if want_chunk_states else None
    need = lib.gdn2_varlen_workspace_bytes(_lib.GDN2_OP_FWD, N, T, H, Dk, Dv, chunk, _dtype_code(q.dtype))
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    st = lib.gdn2_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(b), _ptr(w), _ptr(cu_seqlens), N,
                             _ptr(S0), _ptr(o), _ptr(S_final), _ptr(states), _ptr(workspace),
                             workspace.numel() * workspace.element_size(), T, H, Dk, Dv, chunk, _dtype_code(q.dtype),
                             _flags(raw_gates, scalar_b, scalar_w, scalar_decay), _stream(dev))
    _lib.check(st, "gdn2_fwd_varlen")
    return o, S_final, states


def gdn2_bwd_varlen(q, k, v, log_alpha, b, w, dO, cu_seqlens, S0=None, dS_final=None, chunk_states=None, chunk=64,
                    want_dS0=True, workspace=None, raw_gates=False, scalar_b=False, scalar_w=False,
                    scalar_decay=False):
    """Packed variable-length backward. Returns a dict with dq, dk, dv, dlog_alpha, db, dw ([1,T,H,D] fp32,
    zero outside every sequence) and dS0 ([N,H,Dk,Dv] or None)."""
    lib = _lib.load()
    _, T, H, Dk = q.shape
    Dv = v.shape[-1]
    dev = q.device
    _check_inputs(("q", "k", "b"), (q, k, b), q.dtype, dev)
    _check_inputs(("v", "w", "dO"), (v, w, dO), q.dtype, dev)
    _check_inputs(("log_alpha",), (log_alpha,), torch.float32, dev)
    _check_inputs(("cu_seqlens",), (cu_seqlens,), torch.int64, dev)
    N = cu_seqlens.numel() - 1
    S0 = _f32_state(S0, "S0", dev, (N, H, Dk, Dv))
    dS_final = _f32_state(dS_final, "dS_final", dev, (N, H, Dk, Dv))
    mc = lib.gdn2_varlen_max_chunks(N, T, chunk)
    chunk_states = _f32_state(chunk_states, "chunk_states", dev, (H, mc, Dk, Dv))
    kshape, vshape = (1, T, H, Dk), (1, T, H, Dv)
    gs = _gate_shapes((1, T, H), Dk, Dv, scalar_b, scalar_w, scalar_decay)
    g = {n: torch.zeros(kshape, dtype=torch.float32, device=dev) for n in ("dq", "dk")}
    g["dv"] = torch.zeros(vshape, dtype=torch.float32, device=dev)
    g.update({"d" + n: torch.zeros(gs[n], dtype=torch.float32, device=dev) for n in ("b", "w", "log_alpha")})
    g["dS0"] = torch.empty((N, H, Dk, Dv), dtype=torch.float32, device=dev) if want_dS0 else None
    need = lib.gdn2_varlen_workspace_bytes(_lib.GDN2_OP_BWD, N, T, H, Dk, Dv, chunk, _dtype_code(q.dtype))
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    st = lib.gdn2_bwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(b), _ptr(w), _ptr(cu_seqlens), N,
                             _ptr(S0), _ptr(dO), _ptr(dS_final), _ptr(chunk_states), _ptr(g["dq"]), _ptr(g["dk"]),
                             _ptr(g["dv"]), _ptr(g["dlog_alpha"]), _ptr(g["db"]), _ptr(g["dw"]), _ptr(g["dS0"]),
                             _ptr(workspace), workspace.numel() * workspace.element_size(), T, H, Dk, Dv, chunk,
                             _dtype_code(q.dtype), _flags(raw_gates, scalar_b, scalar_w, scalar_decay), _stream(dev))
    _lib.check(st, "gdn2_bwd_varlen")
    return g


def gdn2_varlen_records_bytes(N, T, H, Dk, Dv, chunk, dtype):
    return _lib.load().gdn2_varlen_records_bytes(N, T, H, Dk, Dv, chunk, _dtype_code(dtype))


def gdn2_fwd_varlen_train(q, k, v, log_alpha, b, w, cu_seqlens, S0=None, chunk=64, want_final_state=True,
                          workspace=None, records=None, raw_gates=False, scalar_b=False, scalar_w=False,
                          scalar_decay=False):
    """Packed-batch training forward (gdn2_fwd_varlen_train). Returns (o [1,T,H,Dv], S_final [N,H,Dk,Dv] or
    None, records); pass records to gdn2_bwd_varlen_records with the same inputs and cu_seqlens."""
    lib = _lib.load()
    _, T, H, Dk = q.shape
    Dv = v.shape[-1]
    dev = q.device
    _check_inputs(("q", "k", "b"), (q, k, b), q.dtype, dev)
    _check_inputs(("v", "w"), (v, w), q.dtype, dev)
    _check_inputs(("log_alpha",), (log_alpha,), torch.float32, dev)
    _check_inputs(("cu_seqlens",), (cu_seqlens,), torch.int64, dev)
    N = cu_seqlens.numel() - 1
    S0 = _f32_state(S0, "S0", dev, (N, H, Dk, Dv))
    o = torch.zeros((1, T, H, Dv), dtype=torch.float32, device=dev)
    S_final = torch.empty((N, H, Dk, Dv), dtype=torch.float32, device=dev) if want_final_state else None
    dt = _dtype_code(q.dtype)
    workspace = _scratch(workspace, lib.gdn2_varlen_workspace_bytes(_lib.GDN2_OP_FWD, N, T, H, Dk, Dv, chunk, dt),
                         dev)
    records = _scratch(records, lib.gdn2_varlen_records_bytes(N, T, H, Dk, Dv, chunk, dt), dev)
    st = lib.gdn2_fwd_varlen_train(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(b), _ptr(w), _ptr(cu_seqlens),
                                   N, _ptr(S0), _ptr(o), _ptr(S_final), _ptr(records), _nbytes(records),
                                   _ptr(workspace), _nbytes(workspace), T, H, Dk, Dv, chunk, dt,
                                   _flags(raw_gates, scalar_b, scalar_w, scalar_decay), _stream(dev))
    _lib.check(st, "gdn2_fwd_varlen_train")
    return o, S_final, records


def gdn2_bwd_varlen_records(q, k, v, log_alpha, b, w, dO, cu_seqlens, records, dS_final=None, chunk=64,
                            want_dS0=True, workspace=None, raw_gates=False, scalar_b=False, scalar_w=False,
                            scalar_decay=False):
    """Packed-batch backward from the training forward's records (gdn2_bwd_varlen_records). Returns the dict
    of gdn2_bwd_varlen."""
    lib = _lib.load()
    _, T, H, Dk = q.shape
    Dv = v.shape[-1]
    dev = q.device
    _check_inputs(("q", "k", "b"), (q, k, b), q.dtype, dev)
    _check_inputs(("v", "w", "dO"), (v, w, dO), q.dtype, dev)
    _check_inputs(("log_alpha",), (log_alpha,), torch.float32, dev)
    _check_inputs(("cu_seqlens",), (cu_seqlens,), torch.int64, dev)
    N = cu_seqlens.numel() - 1
    dS_final = _f32_state(dS_final, "dS_final", dev, (N, H, Dk, Dv))
    if records is None or records.device != dev or records.dtype != torch.uint8:
        raise ValueError("records must be the uint8 device tensor returned by gdn2_fwd_varlen_train")
    gs = _gate_shapes((1, T, H), Dk, Dv, scalar_b, scalar_w, scalar_decay)
    g = {n: torch.zeros((1, T, H, Dk), dtype=torch.float32, device=dev) for n in ("dq", "dk")}
    g["dv"] = torch.zeros((1, T, H, Dv), dtype=torch.float32, device=dev)
    g.update({"d" + n: torch.zeros(gs[n], dtype=torch.float32, device=dev) for n in ("b", "w", "log_alpha")})
    g["dS0"] = torch.empty((N, H, Dk, Dv), dtype=torch.float32, device=dev) if want_dS0 else None
    dt = _dtype_code(q.dtype)
    workspace = _scratch(workspace,
                         lib.gdn2_varlen_workspace_bytes(_lib.GDN2_OP_BWD_RECORDS, N, T, H, Dk, Dv, chunk, dt), dev)
    st = lib.gdn2_bwd_varlen_records(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(b), _ptr(w), _ptr(cu_seqlens),
                                     N, _ptr(dO), _ptr(dS_final), _ptr(records), _nbytes(records), _ptr(g["dq"]),
                                     _ptr(g["dk"]), _ptr(g["dv"]), _ptr(g["dlog_alpha"]), _ptr(g["db"]),
                                     _ptr(g["dw"]), _ptr(g["dS0"]), _ptr(workspace), _nbytes(workspace), T, H, Dk,
                                     Dv, chunk, dt, _flags(raw_gates, scalar_b, scalar_w, scalar_decay),
                                     _stream(dev))
    _lib.check(st, "gdn2_bwd_varlen_records")
    return g


def gdn2_decode_step_slots(q, k, v, log_alpha, b, w, S_pool, slots, o=None, raw_gates=False):
    """One decode step for B entries whose states are S_pool[slots[b]] ([num_slots,H,Dk,Dv] fp32, in place);
    slots int32 [B] on the device (an entry outside the pool gets o = 0). Returns o [B,H,Dv] fp32."""
    lib = _lib.load()
    B, H, Dk = q.shape
    Dv = v.shape[-1]
    dev = q.device
    _check_inputs(("q", "k", "b"), (q, k, b), q.dtype, dev)
    _check_inputs(("v", "w"), (v, w), q.dtype, dev)
    _check_inputs(("log_alpha",), (log_alpha,), torch.float32, dev)
    _check_inputs(("slots",), (slots,), torch.int32, dev)
    _f32_state(S_pool, "S_pool", dev, (S_pool.shape[0], H, Dk, Dv))
    if o is None:
        o = torch.empty((B, H, Dv), dtype=torch.float32, device=dev)
    st = lib.gdn2_decode_step_slots(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(b), _ptr(w), _ptr(S_pool),
                                    _ptr(slots), S_pool.shape[0], _ptr(o), B, H, Dk, Dv, _dtype_code(q.dtype),
                                    _lib.GDN2_FLAG_RAW_GATES if raw_gates else 0, _stream(dev))
    _lib.check(st, "gdn2_decode_step_slots")
    return o
