"""Benchmark of the hot path on one MI355X; prints ONE JSON line.

A step is one pass of the whole path on synthetic inputs already resident in
HBM:
  * attn_fwd on the headline workload -- one head, Nq = Nk = 4096, D = 64,
    float32 in and out (the size "Flash attention, f32" benchmarks), and
  * flash-decoding -- attn_decode_split + attn_decode_combine on batch 8,
    32 heads, one query row, KV length 32768, D = 128, float16.
``value`` is the forward's TFLOP/s (4*Nq*Nk*D flops per call); the decode's
KV GB/s rides along in ``decode``.  Both carry a roofline fraction; the
kernels' own durations come from HIP events recorded on the stream the
kernels are launched on, around each part of every timed step.

Before the timed steps the multi-head f16/bf16 workload (B4 H12 M=N=2048
D64, no LSE) and the causal f16 workload (Z1 H2 N1024, scale 0.5, with LSE,
causal and not) are timed as the FlashAttention-2 README times its table
(warm-up, then the median of 7 samples of 50 back-to-back calls, HIP events)
and reported under ``extra`` (not part of ``value``), as are the generalised
prefill shapes (D = 128 in f16, bf16 and f32, a ragged N = 2000, Nq != Nk) and
the backward (attn_bwd) on the multi-head shape in f16 and bf16, causal f16,
f16 and f32 at D = 128, and on the single-head f32 shape.

The fp64 CPU oracle is timed on the host cores first (``cpu_baseline``): the
whole headline workload, all 4096 rows, repeated for about three seconds.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_F32 = 157.3          # TFLOP/s, MI355X dense f32 matrix (= f32 vector)
PEAK_F16 = 2516.6         # TFLOP/s, MI355X dense f16/bf16 matrix
PEAK_HBM = 8000.0         # GB/s
PAGES_F32_TFLOPS = 5.5    # "Flash attention, f32": same workload, RTX 2080 SUPER (context)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def cpu_baseline(cfg, seconds=3.0):
    """The fp64 oracle on the whole workload, repeated until about ``seconds``
    of wall time have passed (at least once); mean TFLOP/s."""
    import oracle
    from exact_attention_fa2_amd import inputs
    q, k, v = inputs.qkv((cfg.B, cfg.H, cfg.Nq, cfg.D), (cfg.B, cfg.H, cfg.Nk, cfg.D), cfg.seed,
                         cfg.dtype)
    q, k, v = (inputs.to_f64(x, cfg.dtype) for x in (q, k, v))
    cores = len(os.sched_getaffinity(0))
    runs = 0
    t0 = time.perf_counter()
    while True:
        oracle.attn(q, k, v, cfg.scale, cfg.causal, nthreads=cores)
        runs += 1
        dt = time.perf_counter() - t0
        if dt >= seconds:
            break
    return {"value": cfg.flops * runs / dt / 1e12, "unit": "TFLOP/s", "cores": cores,
            "kind": "oracle",
            "sample": "%s: all %d rows, fp64, %d runs in %.2f s wall" % (
                cfg.name, cfg.B * cfg.H * cfg.Nq, runs, dt)}


def measured_traffic():
    """HBM bytes per launch measured with rocprofv3 FETCH_SIZE / WRITE_SIZE
    (profiles/traffic.json, written from a profile of this bench), each scaled
    by the counter's reading for a plain device copy of known size.  None when
    absent or when it was taken on a different version of a kernel."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return {}
    out = {}
    for name, rec in data.get("kernels", {}).items():
        if rec.get("source_sha") == kernel_source_sha(rec.get("source", "")):
            out[name] = rec.get("bytes_per_launch")
    return out


def kernel_source_sha(rel):
    import hashlib
    try:
        with open(os.path.join(ROOT, rel), "rb") as f:
            return hashlib.sha256(f.read()).hexdigest()[:16]
    except OSError:
        return None


def upload(a, dt):
    import numpy as np
    import torch
    if dt == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def prefill_inputs(cfg):
    from exact_attention_fa2_amd import inputs
    q, k, v = inputs.qkv((cfg.B, cfg.H, cfg.Nq, cfg.D), (cfg.B, cfg.H, cfg.Nk, cfg.D), cfg.seed,
                         cfg.dtype)
    return [upload(x, cfg.dtype) for x in (q, k, v)]


def decode_inputs(cfg):
    from exact_attention_fa2_amd import inputs
    out = []
    for tid, shape in ((0, (cfg.B, cfg.H, cfg.D)), (1, (cfg.B, cfg.H, cfg.N, cfg.D)),
                       (2, (cfg.B, cfg.H, cfg.N, cfg.D))):
        a = inputs.normal(shape, cfg.seed, tid, cfg.dtype)
        out.append(upload(a, cfg.dtype))
        del a
    return out


def f32_peak(dtype):
    """float32 workloads are rated against the float32 matrix-core peak."""
    return {"peak_tflops": PEAK_F32} if dtype == "f32" else {}


GRAPH_CALLS = 20


def capture(fn, n):
    """A HIP graph of n back-to-back calls of fn (torch.cuda.graph; one
    warm-up call on a side stream first, as torch recommends)."""
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(n):
            fn()
    torch.cuda.synchronize()
    return graph


def extra_cases():
    """The workloads reported under ``extra``, one at a time, as (name, call,
    flops, info, calls per timing sample); each case's inputs are made when it
    is reached and dropped after.

    Forward: the multi-head f16/bf16 shape (no LSE), the causal f16 workload
    (with LSE, causal and not; also replayed from a HIP graph of 20 calls,
    "us" then per call), and the generalised prefill shapes (D = 128,
    a ragged N = 2000, Nq != Nk; D = 128 also in f32).  Backward: attn_bwd
    alone on the multi-head N = 2048 shape (f16, bf16, causal f16, and f16 and
    f32 at D = 128) and on the single-head f32 N = 4096 shape (O and the LSE
    from one untimed attn_fwd), 10*Nq*Nk*D flops per head (five products),
    halved when causal.  f32 cases are rated against the f32 peak."""
    import dataclasses

    import torch

    from exact_attention_fa2_amd import fa2, inputs, workloads
    ws = torch.empty(64 << 20, dtype=torch.uint8, device="cuda")
    fwd = [workloads.multihead(2048, "f16"), workloads.multihead(2048, "bf16"),
           workloads.causal_lse(True), workloads.causal_lse(False)]
    fwd += [workloads.Prefill("B4 H12 M=N=2048 D128 %s" % dt, 4, 12, 2048, 2048, 128, dt,
                              1 / math.sqrt(128), False, 0) for dt in ("f16", "bf16", "f32")]
    fwd += [workloads.Prefill("B4 H12 M=N=2000 D64 f16 (ragged)", 4, 12, 2000, 2000, 64, "f16",
                              0.125, False, 0),
            workloads.Prefill("B4 H12 M=1024 N=4096 D64 f16", 4, 12, 1024, 4096, 64, "f16",
                              0.125, False, 0)]
    for cfg in fwd:
        q, k, v = prefill_inputs(cfg)
        o = torch.empty_like(q)
        with_lse = cfg.name.startswith("Z1")  # the causal workload's check includes the LSE
        lse = torch.empty((cfg.B, cfg.H, cfg.Nq), dtype=torch.float32, device="cuda")
        need = fa2.workspace_size(cfg.B, cfg.H, cfg.Nq, cfg.Nk, cfg.D, cfg.causal,
                                  fa2.dtype_code(q))
        assert need <= ws.numel()
        call = lambda: fa2.attn_fwd(q, k, v, scale=cfg.scale, causal=cfg.causal,  # noqa: E731
                                    out=o, return_lse=with_lse, lse=lse, workspace=ws)
        yield cfg.name, call, cfg.flops, dict({"lse": with_lse}, **f32_peak(cfg.dtype)), 50
        if with_lse:
            # the same calls replayed from a HIP graph, as a serving loop would
            # run this small, launch-bound shape (no host work per call)
            graph = capture(call, GRAPH_CALLS)
            yield (cfg.name + " (HIP graph of %d calls)" % GRAPH_CALLS, graph.replay,
                   GRAPH_CALLS * cfg.flops, {"lse": True, "calls_per_replay": GRAPH_CALLS}, 5)
            del graph
        del q, k, v, o, lse, call
    del ws
    bwd = [dataclasses.replace(workloads.multihead(2048, dt), causal=causal)
           for dt, causal in (("f16", False), ("bf16", False), ("f16", True))]
    bwd += [workloads.Prefill("B4 H12 M=N=2048 D128 %s" % dt, 4, 12, 2048, 2048, 128, dt,
                              1 / math.sqrt(128), False, 0) for dt in ("f16", "f32")]
    bwd.append(workloads.HEADLINE_F32)
    for cfg in bwd:
        dt, causal = cfg.dtype, cfg.causal
        q, k, v = prefill_inputs(cfg)
        g = upload(inputs.normal((cfg.B, cfg.H, cfg.Nq, cfg.D), cfg.seed, 3, dt), dt)
        o, lse = fa2.attn_fwd(q, k, v, scale=cfg.scale, causal=causal, return_lse=True)
        dq_, dk_, dv_ = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        delta = torch.empty((cfg.B, cfg.H, cfg.Nq), dtype=torch.float32, device="cuda")
        yield ("bwd %s%s" % (cfg.name, " causal" if causal else ""),
               lambda: fa2.attn_bwd(q, k, v, o, g, lse, scale=cfg.scale, causal=causal, dq=dq_,
                                    dk=dk_, dv=dv_, delta=delta),
               2.5 * cfg.flops, f32_peak(dt), 20)
        del q, k, v, g, o, lse, dq_, dk_, dv_, delta


def time_loop(fn, iters, warmup):
    """Mean kernel time (ms) of fn() over iters calls, events on the current stream."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(iters):
        fn()
    e.record()
    e.synchronize()
    return s.elapsed_time(e) / iters


def time_median(fn, warm_ms=500.0, samples=7, calls=50):
    """The FlashAttention-2 README's protocol: warm up with at least 25 calls
    and about ``warm_ms`` of GPU work, then the median of ``samples`` samples
    of ``calls`` back-to-back calls, each bracketed by HIP events (ms per call)."""
    one = time_loop(fn, 25, 25)
    time_loop(fn, max(25, int(warm_ms / max(one, 1e-3))), 0)
    ts = sorted(time_loop(fn, calls, 0) for _ in range(samples))
    return ts[len(ts) // 2]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=25)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--decode-dtype", default="f16", choices=["f16", "bf16"])
    ap.add_argument("--profile-extra", default=None, metavar="PATTERN",
                    help="only run the extra workloads whose name contains PATTERN, "
                         "--profile-calls times each (for counter profiles), and exit")
    ap.add_argument("--profile-calls", type=int, default=5)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy 5 times (to scale the FETCH_SIZE "
                         "and WRITE_SIZE counters of a profile) and exit")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the path has no multi-GPU form "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration:
        import torch
        torch.cuda.set_device(0)
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": 1 << 30, "calls": 5}))
        return

    from exact_attention_fa2_amd import fa2, workloads
    pre = workloads.HEADLINE_F32
    dec = workloads.decode(args.decode_dtype)

    base = None
    if not args.no_cpu_baseline:
        log("cpu baseline: oracle on %s" % pre.name)
        base = cpu_baseline(pre)
        log("cpu baseline: %.4f TFLOP/s on %d cores" % (base["value"], base["cores"]))

    import torch
    torch.cuda.set_device(0)
    props = torch.cuda.get_device_properties(0)
    log("device: %s, %d CUs" % (props.name, props.multi_processor_count))

    if args.profile_extra is not None:
        # Counter runs: the matching extra workloads only, one call and then
        # --profile-calls back-to-back calls each, no timing protocol.
        for name, call, _, _, _ in extra_cases():
            if args.profile_extra in name:
                call()
                torch.cuda.synchronize()
                for _ in range(args.profile_calls):
                    call()
                torch.cuda.synchronize()
                log("profiled %s" % name)
        return

    extra = {}
    if not args.no_extra:
        for name, call, flops, info, calls in extra_cases():
            ms = time_median(call, calls=calls)
            tf = flops / (ms * 1e-3) / 1e12
            peak = info.get("peak_tflops", PEAK_F16)
            ms /= info.get("calls_per_replay", 1)  # reported per call
            extra[name] = dict({"us": round(ms * 1e3, 2), "tflops": round(tf, 2),
                                "frac_of_mfma_peak": round(tf / peak, 4)}, **info)
            log("%s: %.2f us, %.1f TFLOP/s (%.1f%% of MFMA peak)" % (name, ms * 1e3, tf,
                                                                     100 * tf / peak))
        torch.cuda.empty_cache()

    pq, pk, pv = prefill_inputs(pre)
    po = torch.empty_like(pq)
    need = fa2.workspace_size(pre.B, pre.H, pre.Nq, pre.Nk, pre.D, pre.causal, fa2.FA2_F32)
    pws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
    log("decode inputs: generating %s" % dec.name)
    dq, dk, dv = decode_inputs(dec)
    ns = fa2.default_splits(dec.B, dec.H, dec.N, dec.D)
    op = torch.empty((dec.B, dec.H, ns, dec.D), dtype=torch.float32, device="cuda")
    mp = torch.empty((dec.B, dec.H, ns), dtype=torch.float32, device="cuda")
    lp = torch.empty((dec.B, dec.H, ns), dtype=torch.float32, device="cuda")
    do = torch.empty((dec.B, dec.H, dec.D), dtype=dq.dtype, device="cuda")

    def prefill():
        fa2.attn_fwd(pq, pk, pv, scale=pre.scale, out=po, workspace=pws)

    def split():
        fa2.attn_decode_split(dq, dk, dv, dec.scale, ns, op, mp, lp)

    def combine():
        fa2.attn_decode_combine(op, mp, lp, dq.dtype, out=do)

    for _ in range(args.warmup):
        prefill()
        split()
        combine()
    torch.cuda.synchronize()

    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(K)]
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record()
    for i in range(K):
        ev[i][0].record()
        prefill()
        ev[i][1].record()
        split()
        ev[i][2].record()
        combine()
        ev[i][3].record()
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t_start.elapsed_time(t_end)
    pre_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / K
    split_ms = sum(e[1].elapsed_time(e[2]) for e in ev) / K
    comb_ms = sum(e[2].elapsed_time(e[3]) for e in ev) / K
    dec_ms = split_ms + comb_ms

    tflops = pre.flops / (pre_ms * 1e-3) / 1e12
    dec_gbs = dec.kv_bytes / (dec_ms * 1e-3) / 1e9
    split_gbs = dec.kv_bytes / (split_ms * 1e-3) / 1e9
    log("prefill %.2f us (%.2f TFLOP/s)  decode split %.2f us + combine %.2f us (%.1f GB/s)" % (
        pre_ms * 1e3, tflops, split_ms * 1e3, comb_ms * 1e3, dec_gbs))

    traffic = measured_traffic()
    line = {
        "metric": "attention fwd TFLOP/s (N=4096,D=64) + decode KV GB/s; % of roofline",
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(total_ms / K, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": round(tflops / PAGES_F32_TFLOPS, 3),
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "prefill: %s, scale 1/8, non-causal; decode: %s, n_splits %d" % (
                pre.name, dec.name, ns),
            "prefill": {"B": pre.B, "H": pre.H, "Nq": pre.Nq, "Nk": pre.Nk, "D": pre.D,
                        "dtype": pre.dtype, "causal": pre.causal},
            "decode": {"B": dec.B, "H": dec.H, "N": dec.N, "D": dec.D, "dtype": dec.dtype,
                       "n_splits": ns},
        },
        "roofline": {"bound": "mfma", "achieved": round(tflops, 3), "peak": PEAK_F32,
                     "unit": "TFLOP/s", "frac": round(tflops / PEAK_F32, 4),
                     "traffic": traffic.get("fwd_f32"), "kernel": "fwd_f32_rows_kernel<64, false>",
                     "us": round(pre_ms * 1e3, 3)},
        "decode": {"value": round(dec_gbs, 1), "unit": "GB/s", "us": round(dec_ms * 1e3, 2),
                   "split_us": round(split_ms * 1e3, 2), "combine_us": round(comb_ms * 1e3, 2),
                   "bytes": dec.kv_bytes},
        "roofline_decode": {"bound": "hbm", "achieved": round(split_gbs, 1), "peak": PEAK_HBM,
                            "unit": "GB/s", "frac": round(split_gbs / PEAK_HBM, 4),
                            "traffic": traffic.get("decode_split"), "kernel": "decode_split",
                            "us": round(split_ms * 1e3, 2)},
        "extra": extra,
        "cpu_baseline": base,
        "wall_s_timed": round(wall, 3),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
