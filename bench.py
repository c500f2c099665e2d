"""Benchmark of the GDN-2 operator on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-decode] [--no-curve] [--no-front-end]
                    [--no-varlen] [--no-gate-granularity] [--no-prefill] [--no-flush] [--decode-only]

A step is one training pass of the operator over one batch of synthetic input
with the pages' layer shape: the chunked forward that also saves the chunk
entry states, then the gate-aware chunked backward (B=8, H=16, T=4096,
d_k=d_v=128, chunk 64, bf16 q/k/v/b/w/dO, fp32 log_alpha). W untimed steps,
then K timed steps between two synchronisations; before every step a 512 MiB
scratch buffer is read (outside the step's events) so that no step starts
with its inputs in L2 or the Infinity Cache. The forward alone on the same
shape (prefill: no chunk states, the configuration's own seeded inputs) is
reported under "prefill". The one-token decode step
(B=256 sequences, H=16, d=128, fp32 state, 128 consecutive steps) is timed
separately and reported under "decode", and the long-sequence forward (B=1,
H=16, d=128, T = 8K..64K: few heads, so the two-level chain) under
"fwd_long_sequence_curve", and the same training step with pre-activation
gates (fused gate front end against torch elementwise passes) under
"front_end", the same tokens as a packed batch of variable-length
sequences under "varlen", and the step with per-head scalar gates (KDA and
Gated DeltaNet specialisations) under "gate_granularity". Inputs are resident in HBM before any timed region.

Prints one JSON line: value = whole-job tokens/s of the forward+backward step,
plus "roofline" for the dominant kernel (HIP events on the launch stream),
"mfma_frac" (FLOP model / bf16 dense peak), "decode" and "cpu_baseline" (the
float64 oracle on a bounded sample, on this host's cores).
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# MI355X published peaks
PEAK_HBM_GBS = 8000.0        # HBM3E, GB/s
PEAK_BF16_TFLOPS = 2500.0    # dense bf16/fp16 matrix cores, TFLOP/s
FLUSH_BYTES = 512 << 20      # read between timed steps: twice the 256 MB Infinity Cache


def evict_caches(buf):
    """Read `buf` (FLUSH_BYTES) on the current stream: every L2 and Infinity Cache line is then one of its
    clean lines, so the next kernel's data comes from HBM and no dirty flush data is written back meanwhile."""
    buf.sum()


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"

# FLOP and byte models per token-head at chunk C, d_k = d_v = d (algorithmic,
# dense-counted; redundant recompute is not counted).
def fwd_flops(C, d):
    return 2 * (C * (3 * d + 2 * d) + 3 * d * d) + C * C / 3


def bwd_flops(C, d):
    return 2 * (C * (9 * d + 5 * d) + 7 * d * d) + 13 * C * C / 3


def fwd_bytes(C, d, e_in=2, save_states=True):
    # q, k, v, b, w read once (e_in bytes), log_alpha fp32 read, o fp32 written,
    # chunk entry states fp32 written once per chunk
    return 5 * d * e_in + 4 * d + 4 * d + (4 * d * d / C if save_states else 0)


def bwd_bytes(C, d, e_in=2):
    # reads q, k, v, b, w, dO (e_in), log_alpha (fp32), chunk states (fp32 per chunk);
    # writes dq, dk, db, dlog_alpha, dv, dw (fp32)
    return 6 * d * e_in + 4 * d + 4 * d * d / C + 6 * d * 4


def decode_bytes(B, H, d, e_in=2):
    # state read + written once (fp32), q, k, v, b, w (e_in), log_alpha fp32, o fp32
    return B * H * (2 * 4 * d * d + 5 * d * e_in + 4 * d + 4 * d)


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "gdn2_fwd_bwd_B8H16T4096_hbm_traffic.md")


def kernel_sources_sha256():
    """sha256 over the HIP sources (name and bytes of every .hip / .h file, sorted by name)."""
    import hashlib

    d = os.path.join(ROOT, "delta_rule_recurrent_gdn_amd", "csrc")
    h = hashlib.sha256()
    for n in sorted(os.listdir(d)):
        if n.endswith((".hip", ".h")):
            with open(os.path.join(d, n), "rb") as f:
                h.update(n.encode() + b"\0" + f.read())
    return h.hexdigest()


def measured_traffic(key):
    """HBM bytes per launch from the committed FETCH_SIZE / WRITE_SIZE counter summary (scaled by the
    copy calibration there), or None when the kernel sources have changed since the counters were taken."""
    try:
        with open(TRAFFIC_PROFILE) as f:
            kv = dict(line.split(": ", 1) for line in f.read().splitlines() if ": " in line and " " not in
                      line.split(": ", 1)[0])
    except OSError:
        return None
    if kv.get("sources_sha256", "").strip() != kernel_sources_sha256() or key not in kv:
        return None
    return int(kv[key].strip())


def _segments_from_workspace(lib, _lib, T, D, C, H=16):
    """Segments of the two-level forward chain at B=1 (1 = the plain chain), read off the workspace size:
    past the 256-byte aligned records and T (w v), each segment of each head holds M [D x D] and N, S_in
    [D x D] in fp32."""
    nc = (T + C - 1) // C
    base = H * nc * (lib.gdn2_workspace_bytes(_lib.GDN2_OP_FWD, 1, C, 1, D, D, C, _lib.GDN2_BF16))
    extra = lib.gdn2_workspace_bytes(_lib.GDN2_OP_FWD, 1, T, H, D, D, C, _lib.GDN2_BF16) - (base + 255) // 256 * 256
    return max(1, extra // (H * 3 * D * D * 4)) if extra > 0 else 1


def _oracle_worker(args):
    """One (batch row, head) slice of the workload through the float64 oracle (fwd + bwd)."""
    from threadpoolctl import threadpool_limits

    import oracle

    q, k, v, la, b, w, dO = args
    with threadpool_limits(limits=1):
        oracle.forward(q, k, v, la, b, w, None)
        oracle.backward(q, k, v, la, b, w, None, dO)
    return q.shape[1]


def cpu_baseline(inp, heads):
    """Time the oracle (fwd + bwd) on batch row 0, `heads` heads, full T, over a process pool."""
    import multiprocessing as mp

    import torch

    cores = min(len(os.sched_getaffinity(0)), 16, heads)
    f = lambda t: t[0:1, :, :heads].to(torch.float64).numpy()  # noqa: E731
    full = [f(inp[n]) for n in ("q", "k", "v", "log_alpha", "b", "w", "dO")]
    jobs = [tuple(x[:, :, h:h + 1].copy() for x in full) for h in range(heads)]
    ctx = mp.get_context("fork")
    t = time.perf_counter()
    with ctx.Pool(cores) as pool:
        pool.map(_oracle_worker, jobs, chunksize=1)
    dt = time.perf_counter() - t
    T = full[0].shape[1]
    H = inp["q"].shape[2]
    # tokens of the workload carry H heads each: the sample covers heads/H of T tokens
    tokens = T * heads / H
    return {"value": tokens / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle", "cpu": cpu_model(),
            "sample": f"batch row 0, {heads} of {H} heads, T={T}: float64 stepwise forward + reverse-mode "
                      f"backward, one process per head ({dt:.1f} s wall)"}


def _oracle_fwd_worker(args):
    from threadpoolctl import threadpool_limits

    import oracle

    with threadpool_limits(limits=1):
        oracle.forward(*args, None)
    return args[0].shape[1]


def cpu_baseline_prefill(inp, heads):
    """Time the oracle forward on batch row 0, `heads` heads, full T, over a process pool."""
    import multiprocessing as mp

    import torch

    cores = min(len(os.sched_getaffinity(0)), 16, heads)
    f = lambda t: t[0:1, :, :heads].to(torch.float64).numpy()  # noqa: E731
    full = [f(inp[n]) for n in ("q", "k", "v", "log_alpha", "b", "w")]
    jobs = [tuple(x[:, :, h:h + 1].copy() for x in full) for h in range(heads)]
    t = time.perf_counter()
    with mp.get_context("fork").Pool(cores) as pool:
        pool.map(_oracle_fwd_worker, jobs, chunksize=1)
    dt = time.perf_counter() - t
    T, H = full[0].shape[1], inp["q"].shape[2]
    return {"value": T * heads / H / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle", "cpu": cpu_model(),
            "sample": f"batch row 0, {heads} of {H} heads, T={T}: float64 stepwise forward, one process per head "
                      f"({dt:.1f} s wall)"}


def cpu_baseline_decode(dec, steps):
    """Time the oracle's decode step over every (sequence, head) of the decode batch for `steps` steps
    (numpy vectorised over the pairs, one process, BLAS threads as the host sets them)."""
    import oracle

    S = dec["S0"]
    t = time.perf_counter()
    for i in range(steps):
        _, S = oracle.decode_step(*(dec[n][i] for n in ("q", "k", "v", "log_alpha", "b", "w")), S)
    dt = time.perf_counter() - t
    B = dec["q"].shape[1]
    return {"value": B * steps / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle", "cpu": cpu_model(),
            "sample": f"{steps} of the 128 decode steps, all {B} sequences x {dec['q'].shape[2]} heads: float64 "
                      f"oracle decode step vectorised over the pairs in one process ({dt:.1f} s wall)"}


def run_decode(lib, _lib, dev, stream):
    """The one-token decode (B=256 sequences, H=16, d=128, fp32 state, bf16 token inputs) over its 128
    consecutive steps: microseconds per step against the HBM roofline (the state exceeds the Infinity Cache,
    so no flush is needed between steps)."""
    import torch

    import synth

    P = lambda t: None if t is None else t.data_ptr()  # noqa: E731
    sh = stream.cuda_stream
    c3 = synth.WORKLOADS["decode-B256-H16-d128-128steps"]
    dec = synth.workload_inputs("decode-B256-H16-d128-128steps")
    dd = {k: v.to(dev) for k, v in dec.items()}
    S = dd["S0"].clone()
    od = torch.empty(c3["B"], c3["H"], c3["Dv"], device=dev)
    steps = c3["steps"]
    xs = [[dd[n][t] for n in ("q", "k", "v", "log_alpha", "b", "w")] for t in range(steps)]

    def dstep(t):
        x = xs[t]
        st = lib.gdn2_decode_step(P(x[0]), P(x[1]), P(x[2]), P(x[3]), P(x[4]), P(x[5]), P(S), P(od),
                                  c3["B"], c3["H"], c3["Dk"], c3["Dv"], _lib.GDN2_BF16, sh)
        _lib.check(st, "gdn2_decode_step")

    for t in range(8):
        dstep(t)
    S.copy_(dd["S0"])
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for t in range(steps):
        dstep(t)
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / steps
    # the same steps with FLUSH_BYTES read before each (outside its events): no state line can come
    # from the Infinity Cache, so this time is the HBM-served one
    flush = torch.ones(FLUSH_BYTES // 4, device=dev)
    S.copy_(dd["S0"])
    nfl = 32
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(nfl)]
    for t in range(nfl):
        evict_caches(flush)
        ev[t][0].record(stream)
        dstep(t)
        ev[t][1].record(stream)
    torch.cuda.synchronize()
    us_fl = sum(a.elapsed_time(b) for a, b in ev) * 1e3 / nfl
    byt = decode_bytes(c3["B"], c3["H"], c3["Dk"])
    gbs = byt / (us / 1e6) / 1e9
    return {"workload": "one-token decode, B=256 H=16 d=128, fp32 state 256x16x128x128, "
                        "bf16 token inputs, 128 consecutive steps",
            "us_per_step": round(us, 2), "tokens_per_s": round(c3["B"] / (us / 1e6), 1),
            "achieved_GBs": round(gbs, 1), "hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
            "algorithmic_bytes_per_step": int(byt),
            "flushed_us_per_step": round(us_fl, 2),
            "flushed_hbm_frac": round(byt / (us_fl / 1e6) / 1e9 / PEAK_HBM_GBS, 4),
            "flushed_note": f"{nfl} steps, each after {FLUSH_BYTES >> 20} MiB read (Infinity Cache evicted)"}


def run_curve(lib, _lib, dev, sh, timed, Ts):
    """The long-sequence forward (B=1, H=16, d=128, chunk 64, bf16, S0 ~ 0.02 N(0,1), no chunk states) at
    each T in Ts, timed by timed(fn) (ms). Few heads and long sequences: the two-level chain."""
    import torch

    import synth

    P = lambda t: None if t is None else t.data_ptr()  # noqa: E731
    D, C = 128, 64
    # the long-sequence sweep: B=1, H=16, d=128, chunk 64, bf16, S0 ~ 0.02 N(0,1); forward (no chunk
    # states) at each T.
    # Few heads and long sequences: the two-stage forward takes the two-level chain here.
    curve = {}
    for Tc in Ts:
        ci = synth.workload_inputs("fwd-long-B1-H16-d128", T=Tc)
        cd = {k: v.to(dev) for k, v in ci.items()}
        oc = torch.empty(1, Tc, 16, D, device=dev)
        Sf = torch.empty(1, 16, D, D, device=dev)
        nwc = lib.gdn2_workspace_bytes(_lib.GDN2_OP_FWD, 1, Tc, 16, D, D, C, _lib.GDN2_BF16)
        wc = torch.empty(max(nwc, 1), dtype=torch.uint8, device=dev)

        def cf():
            st = lib.gdn2_fwd_chunked(P(cd["q"]), P(cd["k"]), P(cd["v"]), P(cd["log_alpha"]), P(cd["b"]),
                                      P(cd["w"]), P(cd["S0"]), P(oc), P(Sf), None, P(wc), nwc, 1, Tc, 16, D,
                                      D, C, _lib.GDN2_BF16, sh)
            _lib.check(st, "gdn2_fwd_chunked")

        ms = timed(cf)
        byt = fwd_bytes(C, D, save_states=False) * Tc * 16
        gbs = byt / (ms / 1e3) / 1e9
        curve[str(Tc)] = {"ms": round(ms, 3), "tokens_per_s": round(Tc / (ms / 1e3), 1),
                          "achieved_GBs": round(gbs, 1), "hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
                          "segments": _segments_from_workspace(lib, _lib, Tc, D, C)}
        del cd, ci
    return curve


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle baseline")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-front-end", action="store_true", help="skip the fused gate front end comparison")
    ap.add_argument("--no-varlen", action="store_true", help="skip the packed variable-length step")
    ap.add_argument("--no-gate-granularity", action="store_true", help="skip the scalar-gate (KDA / GDN) steps")
    ap.add_argument("--no-curve", action="store_true", help="skip the long-sequence forward curve (T = 8K..64K)")
    ap.add_argument("--no-prefill", action="store_true", help="skip the forward-only (prefill) row")
    ap.add_argument("--no-flush", action="store_true", help="no cache flush between timed training steps")
    ap.add_argument("--decode-only", action="store_true",
                    help="only the decode section (for hardware-counter runs of the decode kernel)")
    ap.add_argument("--curve-only", type=int, default=0, metavar="T",
                    help="only the long-sequence forward at this T, 3 runs (for hardware-counter runs)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy three times (the reference kernel for "
                         "scaling the FETCH_SIZE / WRITE_SIZE counters to bytes)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the operator runs on a single MI355X; "
              "multi-GPU runs are not part of this benchmark", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_calibration:
        n = 1 << 28  # fp32 elements: 1 GiB read + 1 GiB written per copy
        src = torch.ones(n, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": 4 * n, "copy_calibration_bytes_written": 4 * n,
                          "copies": 3}), flush=True)
        return

    import synth
    from delta_rule_recurrent_gdn_amd import _lib

    if args.curve_only:
        dev = torch.device("cuda:0")
        lib = _lib.load()
        stream = torch.cuda.current_stream(dev)

        def three(fn):
            fn()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(3):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / 3

        print(json.dumps({"fwd_long_sequence_curve": run_curve(lib, _lib, dev, stream.cuda_stream, three,
                                                               [args.curve_only])}), flush=True)
        return

    if args.decode_only:
        dev = torch.device("cuda:0")
        lib = _lib.load()
        print(json.dumps({"decode": run_decode(lib, _lib, dev, torch.cuda.current_stream(dev))}), flush=True)
        return

    cfg = synth.WORKLOADS["fwd+bwd-B8-H16-T4096-d128"]
    B, T, H, D, C = cfg["B"], cfg["T"], cfg["H"], cfg["Dk"], cfg["chunk"]
    inp = synth.workload_inputs("fwd+bwd-B8-H16-T4096-d128")
    pre = None if args.no_prefill else synth.workload_inputs("fwd-B8-H16-T4096-d128")
    # the oracle baselines run first, in forked worker processes, before this
    # process touches the GPU
    cpu = None if args.no_cpu else cpu_baseline(inp, heads=16)
    cpu_pre = None if (args.no_cpu or pre is None) else cpu_baseline_prefill(pre, heads=16)
    cpu_long = None
    if not args.no_cpu and not args.no_curve:
        cpu_long = cpu_baseline_prefill(synth.workload_inputs("fwd-long-B1-H16-d128", T=8192), heads=16)
    cpu_dec = None
    if not args.no_cpu and not args.no_decode:
        cpu_dec = cpu_baseline_decode(synth.workload_inputs("decode-B256-H16-d128-128steps"), steps=4)

    dev = torch.device("cuda:0")
    d = {k: (v.to(dev) if v is not None else None) for k, v in inp.items()}
    lib = _lib.load()
    stream = torch.cuda.current_stream(dev)
    flush = None if args.no_flush else torch.ones(FLUSH_BYTES // 4, device=dev)

    # preallocated outputs and workspace: the timed region only launches kernels
    NC = (T + C - 1) // C
    o = torch.empty(B, T, H, D, device=dev)
    states = torch.empty(B, H, NC, D, D, device=dev)
    grads = {n: torch.empty(B, T, H, D, device=dev) for n in ("dq", "dk", "dv", "dlog_alpha", "db", "dw")}
    dS0 = torch.empty(B, H, D, D, device=dev)
    need = lib.gdn2_workspace_bytes(_lib.GDN2_OP_BWD, B, T, H, D, D, C, _lib.GDN2_BF16)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    need_f = lib.gdn2_workspace_bytes(_lib.GDN2_OP_FWD, B, T, H, D, D, C, _lib.GDN2_BF16)
    ws_f = torch.empty(max(need_f, 1), dtype=torch.uint8, device=dev)
    # the training pair: the forward's record pass also writes the backward's records, and its chain the
    # chunk entry states (fp16) beside them
    need_r = lib.gdn2_records_bytes(B, T, H, D, D, C, _lib.GDN2_BF16)
    recs = torch.empty(need_r, dtype=torch.uint8, device=dev)
    need_br = lib.gdn2_workspace_bytes(_lib.GDN2_OP_BWD_RECORDS, B, T, H, D, D, C, _lib.GDN2_BF16)
    ws_br = torch.empty(need_br, dtype=torch.uint8, device=dev)
    P = lambda t: None if t is None else t.data_ptr()  # noqa: E731
    sh = stream.cuda_stream
    launch = {"sh": sh}  # the stream the step's calls launch on (a capture stream while a graph is captured)

    def fwd(flags=0, x=d):
        st = lib.gdn2_fwd_chunked_train(P(x["q"]), P(x["k"]), P(x["v"]), P(x["log_alpha"]), P(x["b"]), P(x["w"]),
                                        None, P(o), None, P(recs), need_r, P(ws_f), need_f, B, T, H, D, D, C,
                                        _lib.GDN2_BF16, flags, launch["sh"])
        _lib.check(st, "gdn2_fwd_chunked_train")

    def bwd(flags=0, x=d, gb=None, gw=None, gla=None):
        st = lib.gdn2_bwd_chunked_records(P(x["q"]), P(x["k"]), P(x["v"]), P(x["log_alpha"]), P(x["b"]), P(x["w"]),
                                          P(x["dO"]), None, P(recs), need_r, P(grads["dq"]),
                                          P(grads["dk"]), P(grads["dv"]), P(grads["dlog_alpha"] if gla is None else gla),
                                          P(grads["db"] if gb is None else gb), P(grads["dw"] if gw is None else gw),
                                          P(dS0), P(ws_br), need_br,
                                          B, T, H, D, D, C, _lib.GDN2_BF16, flags, launch["sh"])
        _lib.check(st, "gdn2_bwd_chunked_records")

    # the separate entry points (each call with its own record pass), for comparison
    def fwd_sep(single_pass=False):
        wsp, wsn = (None, 0) if single_pass else (P(ws_f), need_f)
        st = lib.gdn2_fwd_chunked(P(d["q"]), P(d["k"]), P(d["v"]), P(d["log_alpha"]), P(d["b"]), P(d["w"]), None,
                                  P(o), None, P(states), wsp, wsn, B, T, H, D, D, C, _lib.GDN2_BF16, sh)
        _lib.check(st, "gdn2_fwd_chunked")

    def bwd_sep():
        st = lib.gdn2_bwd_chunked(P(d["q"]), P(d["k"]), P(d["v"]), P(d["log_alpha"]), P(d["b"]), P(d["w"]), None,
                                  P(d["dO"]), None, P(states), P(grads["dq"]), P(grads["dk"]), P(grads["dv"]),
                                  P(grads["dlog_alpha"]), P(grads["db"]), P(grads["dw"]), P(dS0), P(ws), need,
                                  B, T, H, D, D, C, _lib.GDN2_BF16, sh)
        _lib.check(st, "gdn2_bwd_chunked")

    def timed_pair(f, b, n, warm, fl=None):
        """Average ms of f, of b and of the whole step over n steps (HIP events on the launch stream).
        With fl, the buffer fl is read before every step (evict_caches), outside the step's events."""
        for _ in range(warm):
            f()
            b()
        torch.cuda.synchronize()
        if fl is None:
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * n + 1)]
            ev[0].record(stream)
            for i in range(n):
                f()
                ev[2 * i + 1].record(stream)
                b()
                ev[2 * i + 2].record(stream)
            torch.cuda.synchronize()
            tf = sum(ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(n)) / n
            tb = sum(ev[2 * i + 1].elapsed_time(ev[2 * i + 2]) for i in range(n)) / n
            return tf, tb, ev[0].elapsed_time(ev[-1]) / n
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n)]
        for i in range(n):
            evict_caches(fl)
            ev[i][0].record(stream)
            f()
            ev[i][1].record(stream)
            b()
            ev[i][2].record(stream)
        torch.cuda.synchronize()
        tf = sum(e[0].elapsed_time(e[1]) for e in ev) / n
        tb = sum(e[1].elapsed_time(e[2]) for e in ev) / n
        return tf, tb, tf + tb

    def timed_flushed(fn, n=10, warm=3):
        """Average ms of fn over n calls, the flush buffer read before each (outside the events)."""
        for _ in range(warm):
            fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for i in range(n):
            if flush is not None:
                evict_caches(flush)
            ev[i][0].record(stream)
            fn()
            ev[i][1].record(stream)
        torch.cuda.synchronize()
        return sum(a.elapsed_time(b) for a, b in ev) / n

    t_wall = time.perf_counter()
    t_fwd, t_bwd, ms_step = timed_pair(fwd, bwd, args.steps, args.warmup, flush)
    wall = time.perf_counter() - t_wall
    _, _, ms_step_nf = timed_pair(fwd, bwd, min(args.steps, 10), 1) if flush is not None else (0, 0, ms_step)
    s_fwd, s_bwd, s_step = timed_pair(fwd_sep, bwd_sep, min(args.steps, 10), 1, flush)
    # the single-pass forward (no workspace), timed on its own for comparison
    t_fwd_single = timed_flushed(lambda: fwd_sep(single_pass=True), n=min(args.steps, 10))
    # the same training step captured once in a HIP graph and replayed (no allocation, synchronisation or
    # memset inside it): the launch overhead of its kernels removed
    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        launch["sh"] = torch.cuda.current_stream().cuda_stream
        fwd()
        bwd()
    launch["sh"] = sh
    torch.cuda.synchronize()
    ms_graph = timed_flushed(graph.replay, n=min(args.steps, 10))
    ms_graph_nf = timed_pair(graph.replay, lambda: None, min(args.steps, 10), 2)[2]
    del graph
    tokens = B * T
    value = tokens / (ms_step / 1e3)

    th = B * T * H
    F_f, F_b = fwd_flops(C, D) * th, bwd_flops(C, D) * th
    by_f, by_b = fwd_bytes(C, D) * th, bwd_bytes(C, D) * th
    # dominant launch: the entry-point call with the larger share of the step
    # (each call is its kernels back to back on one stream)
    if t_fwd >= t_bwd:
        tkey = "train_fwd_launch_traffic_bytes"
        dom, t_dom, by_dom, f_dom = ("gdn2_fwd_chunked_train launch (gdn2_prep_kernel forward and backward records "
                                     "+ gdn2_chain_fwd_kernel, chunk states saved)", t_fwd, by_f, F_f)
    else:
        tkey = "bwd_records_launch_traffic_bytes"
        dom, t_dom, by_dom, f_dom = ("gdn2_bwd_chunked_records launch (gdn2_chain_bwd_kernel + "
                                     "gdn2_bwd_grad_kernel; its records come from the training forward)", t_bwd,
                                     by_b, F_b)
    achieved = by_dom / (t_dom / 1e3) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": measured_traffic(tkey), "kernel": dom,
                "algorithmic_bytes_per_launch": int(by_dom), "avg_launch_ms": round(t_dom, 4)}
    mfma = (F_f + F_b) / (ms_step / 1e3) / (PEAK_BF16_TFLOPS * 1e12)

    out = {
        "metric": "GDN-2 fwd+bwd tokens/s (H=16,d=128,T=4K) + % MFMA peak; decode % HBM peak",
        "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (seeded normal / sigmoid / -softplus draws, workload "
                                 "fwd+bwd-B8-H16-T4096-d128, seed 4)",
        "config": {"workload": "GDN-2 training step: gdn2_fwd_chunked_train (chunkwise forward saving the "
                               "backward records and fp16 chunk entry states) + gdn2_bwd_chunked_records "
                               "(gate-aware backward), "
                               "B=8 H=16 T=4096 d_k=d_v=128 chunk=64, bf16 q/k/v/b/w/dO, fp32 log_alpha, "
                               "fp32 outputs and gradients",
                   "global_batch": B, "seq_len": T, "heads": H, "d_k": D, "d_v": D, "chunk": C,
                   "parallelism": "single GPU"},
        "fwd_ms": round(t_fwd, 4), "bwd_ms": round(t_bwd, 4), "fwd_single_pass_ms": round(t_fwd_single, 4),
        "cache_flush": None if flush is None else f"{FLUSH_BYTES >> 20} MiB read before every timed step",
        "ms_per_step_back_to_back": round(ms_step_nf, 4),
        "graph_ms_per_step": round(ms_graph, 4), "graph_ms_per_step_back_to_back": round(ms_graph_nf, 4),
        "separate_calls": {"fwd_ms": round(s_fwd, 4), "bwd_ms": round(s_bwd, 4), "ms_per_step": round(s_step, 4),
                           "note": "gdn2_fwd_chunked + gdn2_bwd_chunked, each with its own record pass"},
        "mfma_frac": round(mfma, 4),
        # at this path's arithmetic intensity, HBM caps the matrix-core fraction (by the FLOP model) at this
        # value even at full HBM bandwidth
        "mfma_frac_ceiling_at_hbm_peak": round((F_f + F_b) / ((by_f + by_b) / (PEAK_HBM_GBS * 1e9))
                                               / (PEAK_BF16_TFLOPS * 1e12), 4),
        "hbm_frac_step": round((by_f + by_b) / (ms_step / 1e3) / 1e9 / PEAK_HBM_GBS, 4),
        "roofline": roofline,
        "wall_s_timed": round(wall, 3),
    }

    if pre is not None:
        # prefill: the forward alone on the per-layer training shape (B=8 H=16 T=4096 d=128 chunk 64,
        # bf16, S0 = 0, seed 1), returning o only (no chunk states, no final state)
        pdv = {k: (v.to(dev) if v is not None else None) for k, v in pre.items()}
        po = torch.empty(B, T, H, D, device=dev)

        def prefill_call(single_pass=False):
            wsp, wsn = (None, 0) if single_pass else (P(ws_f), need_f)
            st = lib.gdn2_fwd_chunked(P(pdv["q"]), P(pdv["k"]), P(pdv["v"]), P(pdv["log_alpha"]), P(pdv["b"]),
                                      P(pdv["w"]), None, P(po), None, None, wsp, wsn, B, T, H, D, D, C,
                                      _lib.GDN2_BF16, sh)
            _lib.check(st, "gdn2_fwd_chunked")

        tp = timed_flushed(prefill_call, n=min(args.steps, 10))
        tp1 = timed_flushed(lambda: prefill_call(True), n=min(args.steps, 10))
        Fp, Bp = F_f, fwd_bytes(C, D, save_states=False) * th
        pr = {"workload": "forward only (prefill) of the per-layer training shape: gdn2_fwd_chunked two-stage "
                          "path, B=8 H=16 T=4096 d_k=d_v=128 chunk 64, bf16 q/k/v/b/w, fp32 log_alpha, fp32 o, "
                          "no chunk states, seeded inputs of that workload (seed 1)",
              "ms": round(tp, 4), "tokens_per_s": round(B * T / (tp / 1e3), 1),
              "mfma_frac": round(Fp / (tp / 1e3) / (PEAK_BF16_TFLOPS * 1e12), 4),
              "hbm_frac": round(Bp / (tp / 1e3) / 1e9 / PEAK_HBM_GBS, 4),
              "roofline_frac": round(max(Fp / (PEAK_BF16_TFLOPS * 1e12), Bp / (PEAK_HBM_GBS * 1e9)) / (tp / 1e3), 4),
              "mfma_frac_ceiling_at_hbm_peak": round(Fp / (Bp / (PEAK_HBM_GBS * 1e9)) / (PEAK_BF16_TFLOPS * 1e12), 4),
              "algorithmic_flops": int(Fp), "algorithmic_bytes": int(Bp),
              "single_pass_ms": round(tp1, 4),
              "single_pass_tokens_per_s": round(B * T / (tp1 / 1e3), 1)}
        if cpu_pre is not None:
            pr["cpu_baseline"] = cpu_pre
        out["prefill"] = pr
        del pdv, po

    if not args.no_front_end:
        # the fused gate front end: the same training step with the gates passed as pre-activations
        # (b, w = sigmoid(.), log_alpha = -softplus(.) inside the kernels; gradients with respect to the
        # pre-activations), against the same step with the activations and their chain rule done as torch
        # elementwise passes around the plain entry points
        raw = synth.make_inputs(B, T, H, D, D, "bf16", seed=4, grad=True, raw_gates=True)
        rd = {k: (v.to(dev) if v is not None else None) for k, v in raw.items()}
        del raw
        FLAG = _lib.GDN2_FLAG_RAW_GATES

        def raw_step():
            fwd(FLAG, rd)
            bwd(FLAG, rd)

        def unfused_step():
            bb = torch.sigmoid(rd["b"])
            ww = torch.sigmoid(rd["w"])
            la = -torch.nn.functional.softplus(rd["log_alpha"])
            act = dict(rd, b=bb, w=ww, log_alpha=la)
            fwd(0, act)
            bwd(0, act)
            grads["db"].mul_(bb * (1 - bb))
            grads["dw"].mul_(ww * (1 - ww))
            grads["dlog_alpha"].mul_(-torch.sigmoid(rd["log_alpha"]))

        fe = {}
        for name, fn in (("fused_ms_per_step", raw_step), ("unfused_ms_per_step", unfused_step)):
            fe[name] = round(timed_flushed(fn), 4)
        fe["fused_tokens_per_s"] = round(tokens / (fe["fused_ms_per_step"] / 1e3), 1)
        fe["workload"] = ("the B=8 H=16 T=4096 training step (training pair) with pre-activation gates b, w "
                          "(bf16) and a (fp32); unfused = torch sigmoid / softplus passes before and chain-rule "
                          "passes after the same entry points without the flag")
        out["front_end"] = fe
        del rd

    if not args.no_gate_granularity:
        # gate granularity: the same training step with per-head scalar gates ([B, T, H] tensors,
        # broadcast inside the kernels): KDA (one beta for both gates) and Gated DeltaNet (also a scalar decay)
        rng_g = torch.Generator(device="cpu").manual_seed(6)
        beta = torch.sigmoid(torch.randn(B, T, H, generator=rng_g)).to(torch.bfloat16).to(dev)
        adec = (-torch.nn.functional.softplus(torch.randn(B, T, H, generator=rng_g) - 2.0)).to(dev)
        gsc = {n: torch.empty(B, T, H, device=dev) for n in ("db", "dw", "dlog_alpha")}

        def scalar_step(flags, la):
            x = dict(d, log_alpha=la, b=beta, w=beta)
            fwd(flags, x)
            bwd(flags, x, gb=gsc["db"], gw=gsc["dw"], gla=gsc["dlog_alpha"] if la is adec else None)

        gg = {}
        SB, SW, SD = _lib.GDN2_FLAG_SCALAR_B, _lib.GDN2_FLAG_SCALAR_W, _lib.GDN2_FLAG_SCALAR_DECAY
        for name, flags, la in (("kda_ms_per_step", SB | SW, d["log_alpha"]),
                                ("gated_deltanet_ms_per_step", SB | SW | SD, adec)):
            gg[name] = round(timed_flushed(lambda: scalar_step(flags, la)), 4)
        gg["channel_wise_ms_per_step"] = round(ms_step, 4)
        gg["workload"] = ("the B=8 H=16 T=4096 training step (training pair) with per-head scalar gates: KDA = "
                          "one beta [B,T,H] for both gates, Gated DeltaNet = also a scalar decay [B,T,H]; "
                          "channel-wise = the main step")
        out["gate_granularity"] = gg
        del beta, adec, gsc

    if not args.no_varlen:
        # packed variable-length batches: the same 8 x 4096 = 32768 tokens of H = 16 heads (d = 128,
        # chunk 64, bf16) cut into documents of seeded lengths (uniform 256 .. 8192, the last one takes the
        # remainder), packed along T; one training step = gdn2_fwd_varlen (saving chunk states) +
        # gdn2_bwd_varlen
        import numpy as np

        rng = np.random.default_rng(5)
        lens = []
        while sum(lens) < B * T:
            lens.append(int(min(rng.integers(256, 8193), B * T - sum(lens))))
        N = len(lens)
        cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int64, device=dev)
        pk = {n: d[n].reshape(1, B * T, H, -1) for n in ("q", "k", "v", "log_alpha", "b", "w", "dO")}
        mcx = lib.gdn2_varlen_max_chunks(N, B * T, C)
        vstates = torch.empty(H, mcx, D, D, device=dev)
        vws_f = torch.empty(lib.gdn2_varlen_workspace_bytes(_lib.GDN2_OP_FWD, N, B * T, H, D, D, C, _lib.GDN2_BF16),
                            dtype=torch.uint8, device=dev)
        vws_b = torch.empty(lib.gdn2_varlen_workspace_bytes(_lib.GDN2_OP_BWD, N, B * T, H, D, D, C, _lib.GDN2_BF16),
                            dtype=torch.uint8, device=dev)
        vo = torch.empty(1, B * T, H, D, device=dev)
        vrec = torch.empty(lib.gdn2_varlen_records_bytes(N, B * T, H, D, D, C, _lib.GDN2_BF16), dtype=torch.uint8,
                           device=dev)
        vws_r = torch.empty(lib.gdn2_varlen_workspace_bytes(_lib.GDN2_OP_BWD_RECORDS, N, B * T, H, D, D, C,
                                                            _lib.GDN2_BF16), dtype=torch.uint8, device=dev)

        def varlen_pair_step():
            st = lib.gdn2_fwd_varlen_train(P(pk["q"]), P(pk["k"]), P(pk["v"]), P(pk["log_alpha"]), P(pk["b"]),
                                           P(pk["w"]), P(cu), N, None, P(vo), None, P(vrec), vrec.numel(), P(vws_f),
                                           vws_f.numel(), B * T, H, D, D, C, _lib.GDN2_BF16, 0, sh)
            _lib.check(st, "gdn2_fwd_varlen_train")
            st = lib.gdn2_bwd_varlen_records(P(pk["q"]), P(pk["k"]), P(pk["v"]), P(pk["log_alpha"]), P(pk["b"]),
                                             P(pk["w"]), P(cu), N, P(pk["dO"]), None, P(vrec), vrec.numel(),
                                             P(grads["dq"]), P(grads["dk"]), P(grads["dv"]), P(grads["dlog_alpha"]),
                                             P(grads["db"]), P(grads["dw"]), None, P(vws_r), vws_r.numel(), B * T, H,
                                             D, D, C, _lib.GDN2_BF16, 0, sh)
            _lib.check(st, "gdn2_bwd_varlen_records")

        def varlen_step():
            st = lib.gdn2_fwd_varlen(P(pk["q"]), P(pk["k"]), P(pk["v"]), P(pk["log_alpha"]), P(pk["b"]),
                                     P(pk["w"]), P(cu), N, None, P(vo), None, P(vstates), P(vws_f), vws_f.numel(),
                                     B * T, H, D, D, C, _lib.GDN2_BF16, 0, sh)
            _lib.check(st, "gdn2_fwd_varlen")
            st = lib.gdn2_bwd_varlen(P(pk["q"]), P(pk["k"]), P(pk["v"]), P(pk["log_alpha"]), P(pk["b"]),
                                     P(pk["w"]), P(cu), N, None, P(pk["dO"]), None, P(vstates), P(grads["dq"]),
                                     P(grads["dk"]), P(grads["dv"]), P(grads["dlog_alpha"]), P(grads["db"]),
                                     P(grads["dw"]), None, P(vws_b), vws_b.numel(), B * T, H, D, D, C,
                                     _lib.GDN2_BF16, 0, sh)
            _lib.check(st, "gdn2_bwd_varlen")

        vt = {}
        for name, fn in (("pair", varlen_pair_step), ("separate", varlen_step)):
            vt[name] = timed_flushed(fn)
        vms = vt["pair"]
        out["varlen"] = {"workload": f"packed batch of {N} sequences (lengths uniform 256..8192, seed 5) totalling "
                                     f"{B * T} tokens, H=16 d=128 chunk 64 bf16: training step "
                                     f"(gdn2_fwd_varlen_train + gdn2_bwd_varlen_records)",
                         "sequences": N, "ms_per_step": round(vms, 4), "tokens_per_s": round(B * T / (vms / 1e3), 1),
                         "separate_calls_ms_per_step": round(vt["separate"], 4)}
        del vstates, vws_f, vws_b, vo, vrec, vws_r

    if not args.no_decode:
        out["decode"] = run_decode(lib, _lib, dev, stream)
        if cpu_dec is not None:
            out["decode"]["cpu_baseline"] = cpu_dec

    if not args.no_curve:
        curve = run_curve(lib, _lib, dev, sh, lambda fn: timed_flushed(fn, n=10, warm=2),
                          synth.WORKLOADS["fwd-long-B1-H16-d128"]["T"])
        out["fwd_long_sequence_curve"] = curve
        if cpu_long is not None:
            out["fwd_long_sequence_cpu_baseline"] = cpu_long

    if cpu is not None:
        out["cpu_baseline"] = cpu

    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
