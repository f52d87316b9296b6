"""Benchmark of the hot path on one MI355X; prints ONE JSON line.

A step is one pass of the whole path on synthetic inputs already resident in
HBM:
  * attn_fwd on the headline workload -- one head, Nq = Nk = 4096, D = 64,
    float32 in and out (the size "Flash attention, f32" benchmarks), and
  * flash-decoding -- attn_decode_split + attn_decode_combine on batch 8,
    32 heads, one query row, KV length 32768, D = 128, float16.
``value`` is the forward's TFLOP/s (4*Nq*Nk*D flops over its mean time per
step); the decode's KV GB/s rides along in ``decode``.  Both carry a roofline
fraction; the kernels' own durations come from HIP events on the stream the
kernels are launched on: each kernel of every timed step records a pair of
events from its own dispatch (fa2.time_next_launch, hipExtLaunchKernel), so
the interval is that kernel alone, and ``ms_per_step`` comes from events
around all the timed steps.

Order of a run (so that no idle gap precedes any timing):
  1. CPU leg: the fp64 oracle is timed on the headline workload on the host
     cores (``cpu_baseline``) and, in the same leg, computes the reference
     outputs of every named workload that the accuracy figures compare with.
  2. Every input, host and device, is generated and uploaded (the 4 GiB
     decode caches too), and each named workload runs once for its accuracy
     figures (max abs, mean abs, RMSE, relative L2 against the oracle).
  3. The extra workloads are timed as the FlashAttention-2 README times its
     table: each warmed with at least 25 calls and about 500 ms of its own GPU
     work, then 7 samples of back-to-back calls between HIP events, the
     workloads interleaved in a seeded random order in every sample round;
     the median sample is reported.
  4. The step: ``--warmup`` steps, then more steps until at least
     ``--prewarm-ms`` of the step's own GPU work has run (``prewarm_ms`` and
     ``prewarm_steps`` in the line), then exactly ``--steps`` timed steps
     bracketed by synchronisation.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import dataclasses
import json
import math
import os
import random
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_F32 = 157.3          # TFLOP/s, MI355X dense f32 matrix (= f32 vector)
PEAK_F16 = 2516.6         # TFLOP/s, MI355X dense f16/bf16 matrix
PEAK_HBM = 8000.0         # GB/s
PAGES_F32_TFLOPS = 5.5    # "Flash attention, f32": same workload, RTX 2080 SUPER, f16 operands (context)
EXTRA_SEED = 2024         # order of the interleaved extra samples


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ---------------------------------------------------------------- accuracy

def accuracy(got, want):
    """The FlashAttention-2 README's accuracy figures of ``got`` against the
    fp64 reference: max abs, mean abs, RMSE and relative L2."""
    import numpy as np
    err = np.abs(np.asarray(got, dtype=np.float64) - want)
    return {"max_abs": float(err.max()), "mean_abs": float(err.mean()),
            "rmse": float(np.sqrt(np.mean(err ** 2))),
            "rel_l2": float(np.linalg.norm(err) / max(float(np.linalg.norm(want)), 1e-300))}


def download_f64(t):
    import torch
    return t.detach().to(torch.float32).cpu().numpy().astype("float64")


# ------------------------------------------------------------------- inputs

def upload(a, dt):
    import numpy as np
    import torch
    if dt == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host_prefill(cfg):
    from exact_attention_fa2_amd import inputs
    return inputs.qkv((cfg.B, cfg.H, cfg.Nq, cfg.D), (cfg.B, cfg.H, cfg.Nk, cfg.D), cfg.seed,
                      cfg.dtype)


def host_decode(cfg):
    from exact_attention_fa2_amd import inputs
    return (inputs.normal((cfg.B, cfg.H, cfg.D), cfg.seed, 0, cfg.dtype),
            inputs.normal((cfg.B, cfg.H, cfg.N, cfg.D), cfg.seed, 1, cfg.dtype),
            inputs.normal((cfg.B, cfg.H, cfg.N, cfg.D), cfg.seed, 2, cfg.dtype))


# ------------------------------------------------------------------ CPU leg

def cpu_leg(headline, named_prefill, named_decode, host, seconds=3.0):
    """The oracle on the host cores: timed on the whole headline workload
    (repeated for about ``seconds``), and run once on every named workload to
    give the reference outputs of the accuracy figures.  Returns
    (cpu_baseline entry, {name: reference O})."""
    import numpy as np

    import oracle
    from exact_attention_fa2_amd import inputs
    cores = len(os.sched_getaffinity(0))
    refs = {}
    q, k, v = (inputs.to_f64(x, headline.dtype) for x in host[headline.name])
    runs = 0
    t0 = time.perf_counter()
    while True:
        ro, _ = oracle.attn(q, k, v, headline.scale, headline.causal, nthreads=cores)
        runs += 1
        dt = time.perf_counter() - t0
        if dt >= seconds:
            break
    refs[headline.name] = ro
    base = {"value": headline.flops * runs / dt / 1e12, "unit": "TFLOP/s", "cores": cores,
            "kind": "oracle",
            "sample": "%s: all %d rows, fp64, %d runs in %.2f s wall" % (
                headline.name, headline.B * headline.H * headline.Nq, runs, dt)}
    log("cpu baseline: %.4f TFLOP/s on %d cores" % (base["value"], cores))
    t1 = time.perf_counter()
    for cfg in named_prefill:
        if cfg.name in refs:
            continue
        q, k, v = (inputs.to_f64(x, cfg.dtype) for x in host[cfg.name])
        refs[cfg.name] = oracle.attn(q, k, v, cfg.scale, cfg.causal, nthreads=cores)[0]
    for cfg in named_decode:
        # the unsplit definition, one (b,h) per task on a pool of host threads
        # (each promotes its own slice, so host memory stays bounded)
        qd, kd, vd = host[cfg.name]
        ref = np.empty((cfg.B, cfg.H, cfg.D))

        def one(bh, cfg=cfg, qd=qd, kd=kd, vd=vd, ref=ref):
            b, h = divmod(bh, cfg.H)
            sl = (slice(b, b + 1), slice(h, h + 1))
            ro, _ = oracle.attn(inputs.to_f64(qd[sl], cfg.dtype)[:, :, None],
                                inputs.to_f64(kd[sl], cfg.dtype), inputs.to_f64(vd[sl], cfg.dtype),
                                cfg.scale, False, nthreads=1)
            ref[b, h] = ro[0, 0, 0]
        with cf.ThreadPoolExecutor(max_workers=min(16, cores)) as ex:
            list(ex.map(one, range(cfg.B * cfg.H)))
        refs[cfg.name] = ref
    log("cpu leg: reference outputs of %d named workloads in %.1f s" % (
        len(refs), time.perf_counter() - t1))
    return base, refs


# -------------------------------------------------------------------- cases

@dataclasses.dataclass
class Case:
    name: str
    call: object            # one call (or one graph replay)
    work: float             # flops (or bytes for decode) per call
    unit: str               # "TFLOP/s" or "GB/s"
    peak: float             # the kernel's peak in ``unit``
    ceiling: float          # the roofline ceiling at this workload's intensity
    calls: int = 50         # calls per timing sample
    per_replay: int = 1     # calls inside one graph replay
    info: dict = dataclasses.field(default_factory=dict)


def min_bytes(cfg):
    """Q, K, V read once and O written once."""
    esz = 4 if cfg.dtype == "f32" else 2
    return esz * cfg.B * cfg.H * (2 * cfg.Nq + 2 * cfg.Nk) * cfg.D


def fwd_ceiling(cfg):
    """Roofline ceiling: the dtype's matrix peak, or HBM bandwidth times the
    intensity (flops per minimum byte) when that is lower."""
    peak = PEAK_F32 if cfg.dtype == "f32" else PEAK_F16
    return min(peak, PEAK_HBM * 1e9 * cfg.flops / min_bytes(cfg) / 1e12)


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


def fwd_extra_cfgs():
    from exact_attention_fa2_amd import workloads
    cfgs = [workloads.multihead(n, dt) for n in (512, 1024, 2048) for dt in ("f16", "bf16")]
    cfgs += [workloads.causal_lse(True), workloads.causal_lse(False)]
    cfgs += [workloads.Prefill("B4 H12 M=N=2048 D128 %s" % dt, 4, 12, 2048, 2048, 128, dt,
                               1 / math.sqrt(128), False, 0) for dt in ("f16", "bf16", "f32")]
    cfgs += [workloads.Prefill("B4 H12 M=N=2000 D64 f16 (ragged)", 4, 12, 2000, 2000, 64, "f16",
                               0.125, False, 0),
             workloads.Prefill("B4 H12 M=1024 N=4096 D64 f16", 4, 12, 1024, 4096, 64, "f16",
                               0.125, False, 0)]
    # the headline's f32 kernel on more rows and longer keys
    cfgs += [workloads.Prefill("B4 H12 M=N=2048 D64 f32", 4, 12, 2048, 2048, 64, "f32",
                               0.125, False, 0),
             workloads.Prefill("single-head f32 Nq=Nk=8192 D64", 1, 1, 8192, 8192, 64, "f32",
                               0.125, False, 0)]
    return cfgs


def bwd_extra_cfgs():
    from exact_attention_fa2_amd import workloads
    cfgs = [dataclasses.replace(workloads.multihead(2048, dt), causal=causal)
            for dt, causal in (("f16", False), ("bf16", False), ("f16", True))]
    cfgs += [workloads.Prefill("B4 H12 M=N=2048 D128 %s" % dt, 4, 12, 2048, 2048, 128, dt,
                               1 / math.sqrt(128), False, 0) for dt in ("f16", "f32")]
    cfgs.append(workloads.HEADLINE_F32)
    return cfgs


def build_extras(host, refs, acc, pattern=None):
    """Device inputs and calls of every extra workload (only those whose name
    contains ``pattern`` when it is given); each named workload runs once
    first and its output is compared with the oracle's (``acc``)."""
    import torch

    from exact_attention_fa2_amd import fa2, inputs, workloads
    cases = []
    ws = torch.empty(64 << 20, dtype=torch.uint8, device="cuda")
    want = lambda name: pattern is None or pattern in name  # noqa: E731
    for cfg in fwd_extra_cfgs():
        if not want(cfg.name):
            continue
        q, k, v = (upload(x, cfg.dtype) for x in host.get(cfg.name) or host_prefill(cfg))
        o = torch.empty_like(q)
        with_lse = cfg.name.startswith("Z1")  # the causal workload's check includes the LSE
        lse = torch.empty((cfg.B, cfg.H, cfg.Nq), dtype=torch.float32, device="cuda")
        assert fa2.workspace_size(cfg.B, cfg.H, cfg.Nq, cfg.Nk, cfg.D, cfg.causal,
                                  fa2.dtype_code(q)) <= ws.numel()

        def call(q=q, k=k, v=v, o=o, lse=lse, cfg=cfg, with_lse=with_lse):
            fa2.attn_fwd(q, k, v, scale=cfg.scale, causal=cfg.causal, out=o,
                         return_lse=with_lse, lse=lse, workspace=ws)
        info = {"lse": with_lse, "dtype": cfg.dtype}
        if cfg.name in refs:
            call()
            torch.cuda.synchronize()
            acc[cfg.name] = accuracy(download_f64(o), refs[cfg.name])
            info["accuracy"] = acc[cfg.name]
        peak = PEAK_F32 if cfg.dtype == "f32" else PEAK_F16
        cases.append(Case(cfg.name, call, cfg.flops, "TFLOP/s", peak, fwd_ceiling(cfg), info=info))
        if with_lse:
            # the same calls replayed from a HIP graph, as a serving loop would
            # run this small, launch-bound shape (no host work per call)
            graph = capture(call, GRAPH_CALLS)
            cases.append(Case(cfg.name + " (HIP graph of %d calls)" % GRAPH_CALLS, graph.replay,
                              cfg.flops, "TFLOP/s", peak, fwd_ceiling(cfg), calls=5,
                              per_replay=GRAPH_CALLS, info={"lse": True, "dtype": cfg.dtype,
                                                            "graph": graph}))
    dec = workloads.decode("bf16")
    if want(dec.name + " (split + combine)"):
        cases.append(decode_case(dec, host, refs, acc))
    for cfg in bwd_extra_cfgs():
        name = "bwd %s%s" % (cfg.name, " causal" if cfg.causal else "")
        if want(name):
            cases.append(bwd_case(name, cfg, host))
    return cases


def decode_case(dec, host, refs, acc):
    import torch

    from exact_attention_fa2_amd import fa2
    qd, kd, vd = (upload(x, dec.dtype) for x in host.get(dec.name) or host_decode(dec))
    ns = fa2.default_splits(dec.B, dec.H, dec.N, dec.D)
    parts = [torch.empty(s, dtype=torch.float32, device="cuda")
             for s in ((dec.B, dec.H, ns, dec.D), (dec.B, dec.H, ns), (dec.B, dec.H, ns))]
    od = torch.empty((dec.B, dec.H, dec.D), dtype=qd.dtype, device="cuda")

    def dcall():
        fa2.attn_decode_split(qd, kd, vd, dec.scale, ns, *parts)
        fa2.attn_decode_combine(*parts, qd.dtype, out=od)
    dcall()
    torch.cuda.synchronize()
    acc[dec.name] = accuracy(download_f64(od), refs[dec.name]) if dec.name in refs else None
    return Case(dec.name + " (split + combine)", dcall, dec.kv_bytes, "GB/s", PEAK_HBM,
                PEAK_HBM, calls=20, info={"dtype": dec.dtype, "n_splits": ns,
                                          "accuracy": acc[dec.name]})


def bwd_case(name, cfg, host):
    import torch

    from exact_attention_fa2_amd import fa2, inputs
    dt, causal = cfg.dtype, cfg.causal
    q, k, v = (upload(x, dt) for x in host.get(cfg.name) or host_prefill(cfg))
    g = upload(inputs.normal((cfg.B, cfg.H, cfg.Nq, cfg.D), cfg.seed, 3, dt), dt)
    o, lse = fa2.attn_fwd(q, k, v, scale=cfg.scale, causal=causal, return_lse=True)
    dq_, dk_, dv_ = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    delta = torch.empty((cfg.B, cfg.H, cfg.Nq), dtype=torch.float32, device="cuda")

    def bcall():
        fa2.attn_bwd(q, k, v, o, g, lse, scale=cfg.scale, causal=causal, dq=dq_, dk=dk_,
                     dv=dv_, delta=delta)
    peak = PEAK_F32 if dt == "f32" else PEAK_F16
    return Case(name, bcall, 2.5 * cfg.flops, "TFLOP/s", peak, peak, calls=20, info={"dtype": dt})


def time_loop(fn, iters, warmup=0):
    """Mean time (ms) of fn() over iters calls, events on the current stream."""
    import torch
    for _ in range(warmup):
        fn()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(iters):
        fn()
    e.record()
    e.synchronize()
    return s.elapsed_time(e) / iters


def time_extras(cases, warm_ms=500.0, samples=7, seed=EXTRA_SEED):
    """Warm each case (at least 25 calls and about ``warm_ms`` of its GPU
    work), then ``samples`` rounds; every round times each case once
    (``calls`` back-to-back calls) in a fresh seeded random order.  Median
    sample per case, in ms per call."""
    one = {}
    for c in cases:
        t = time_loop(c.call, 25, 0)
        time_loop(c.call, max(1, int(warm_ms / max(t, 1e-3))), 0)
        one[c.name] = t
    rng = random.Random(seed)
    got = {c.name: [] for c in cases}
    for _ in range(samples):
        order = list(cases)
        rng.shuffle(order)
        for c in order:
            got[c.name].append(time_loop(c.call, c.calls) / c.per_replay)
    return {n: sorted(ts)[len(ts) // 2] for n, ts in got.items()}


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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=25)
    ap.add_argument("--prewarm-ms", type=float, default=500.0,
                    help="after --warmup steps, run more untimed steps until at least this "
                         "much of the step's own GPU work has run")
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the CPU leg (oracle timing and the accuracy figures)")
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--decode-dtype", default="f16", choices=["f16", "bf16"])
    ap.add_argument("--profile-extra", default=None, metavar="PATTERN",
                    help="only run the extra workloads whose name contains PATTERN, "
                         "--profile-calls times each (for counter profiles), and exit")
    ap.add_argument("--profile-calls", type=int, default=5)
    ap.add_argument("--extra-only", default=None, metavar="PATTERN",
                    help="only time the extra workloads whose name contains PATTERN (same "
                         "protocol), print them as one JSON line, and exit")
    ap.add_argument("--library", default=None, metavar="PATH",
                    help="use this build of the library instead of libfa2.so (for example "
                         "exact_attention_fa2_amd/libfa2_polyexp.so)")
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

    import torch  # noqa: F401  (before any library load: one HIP runtime in the process)

    from exact_attention_fa2_amd import fa2 as _fa2, workloads
    if args.library:
        _fa2._lib = _fa2.load(os.path.abspath(args.library))
    if args.extra_only is not None:
        import torch
        torch.cuda.set_device(0)
        cases = build_extras({}, {}, {}, args.extra_only)
        med = time_extras(cases)
        out = {}
        for c in cases:
            ms = med[c.name]
            rate = c.work / (ms * 1e-3) / (1e12 if c.unit == "TFLOP/s" else 1e9)
            out[c.name] = {"us": round(ms * 1e3, 2), "rate": round(rate, 2), "unit": c.unit,
                           "frac_of_peak": round(rate / c.peak, 4)}
            log("%s: %.2f us, %.1f %s (%.1f%% of peak)" % (c.name, ms * 1e3, rate, c.unit,
                                                           100 * rate / c.peak))
        print(json.dumps({"library": os.path.basename(args.library or _fa2.LIB_PATH),
                          "extra": out}), flush=True)
        return
    pre = workloads.HEADLINE_F32
    dec = workloads.decode(args.decode_dtype)
    want_extra = not args.no_extra and args.profile_extra is None

    # 1-2. host inputs of everything, then the CPU leg on them
    t0 = time.perf_counter()
    host = {pre.name: host_prefill(pre), dec.name: host_decode(dec)}
    named_prefill = [pre]
    named_decode = [dec]
    if want_extra:
        for cfg in fwd_extra_cfgs():
            host[cfg.name] = host_prefill(cfg)
            if cfg.name.startswith(("B4 H12 M=N=512 D64", "B4 H12 M=N=1024 D64",
                                    "B4 H12 M=N=2048 D64", "Z1")):
                named_prefill.append(cfg)
        bdec = workloads.decode("bf16")
        if bdec.name not in host:
            host[bdec.name] = host_decode(bdec)
        named_decode.append(bdec)
    log("host inputs: %.1f s" % (time.perf_counter() - t0))
    base, refs = None, {}
    if not args.no_cpu_baseline and args.profile_extra is None:
        base, refs = cpu_leg(pre, named_prefill, named_decode, host)

    import torch

    from exact_attention_fa2_amd import fa2
    torch.cuda.set_device(0)
    props = torch.cuda.get_device_properties(0)
    log("device: %s, %d CUs" % (props.name, props.multi_processor_count))

    if args.profile_extra is not None:
        # Counter runs: the matching extra workloads only, one call and then
        # --profile-calls back-to-back calls each, no timing protocol.
        for c in build_extras(host, {}, {}, args.profile_extra):
            if args.profile_extra in c.name:
                c.call()
                torch.cuda.synchronize()
                for _ in range(args.profile_calls):
                    c.call()
                torch.cuda.synchronize()
                log("profiled %s" % c.name)
        return

    # device inputs of the step
    pq, pk, pv = (upload(x, pre.dtype) for x in host[pre.name])
    po = torch.empty_like(pq)
    need = fa2.workspace_size(pre.B, pre.H, pre.Nq, pre.Nk, pre.D, pre.causal, fa2.FA2_F32)
    pws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
    dq, dk, dv = (upload(x, dec.dtype) for x in host[dec.name])
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

    acc = {}
    prefill()
    split()
    combine()
    torch.cuda.synchronize()
    if refs:
        acc[pre.name] = accuracy(download_f64(po), refs[pre.name])
        acc[dec.name] = accuracy(download_f64(do), refs[dec.name])

    # 3. extras
    extra = {}
    if want_extra:
        cases = build_extras(host, refs, acc)
        del host
        med = time_extras(cases)
        for c in cases:
            ms = med[c.name]
            rate = c.work / (ms * 1e-3) / (1e12 if c.unit == "TFLOP/s" else 1e9)
            e = {"us": round(ms * 1e3, 2), "tflops" if c.unit == "TFLOP/s" else "gbs": round(rate, 2),
                 "unit": c.unit, "frac_of_peak": round(rate / c.peak, 4), "peak": c.peak,
                 "ceiling": round(c.ceiling, 1), "frac_of_ceiling": round(rate / c.ceiling, 4)}
            e.update({k: v for k, v in c.info.items() if k != "graph"})
            extra[c.name] = e
            log("%s: %.2f us, %.1f %s (%.1f%% of peak)" % (c.name, ms * 1e3, rate, c.unit,
                                                           100 * rate / c.peak))
        del cases
    else:
        del host

    # 4. the step: warm-up steps, then at least --prewarm-ms of them, then K timed
    for _ in range(args.warmup):
        prefill()
        split()
        combine()
    torch.cuda.synchronize()
    pw_steps, pw_ms = 0, 0.0
    while pw_ms < args.prewarm_ms:
        n = 10
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(n):
            prefill()
            split()
            combine()
        e.record()
        e.synchronize()
        pw_ms += s.elapsed_time(e)
        pw_steps += n

    # Each kernel of a timed step records a pair of events from its own
    # dispatch (fa2.time_next_launch), so its interval is the kernel alone;
    # the step's own events bracket all K steps.
    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(K)]
    for row in ev:
        for e in row:
            e.record()  # created before the timed region
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record()
    for i in range(K):
        fa2.time_next_launch(ev[i][0], ev[i][1])
        prefill()
        fa2.time_next_launch(ev[i][2], ev[i][3])
        split()
        fa2.time_next_launch(ev[i][4], ev[i][5])
        combine()
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t_start.elapsed_time(t_end)
    pre_t = sorted(e[0].elapsed_time(e[1]) for e in ev)
    split_t = [e[2].elapsed_time(e[3]) for e in ev]
    comb_t = [e[4].elapsed_time(e[5]) for e in ev]
    dec_t = sorted(a + b for a, b in zip(split_t, comb_t))
    pre_ms = sum(pre_t) / K
    split_ms = sum(split_t) / K
    comb_ms = sum(comb_t) / K
    dec_ms = split_ms + comb_ms

    tflops = pre.flops / (pre_ms * 1e-3) / 1e12
    dec_gbs = dec.kv_bytes / (dec_ms * 1e-3) / 1e9
    log("prefill %.2f us (%.2f TFLOP/s; median %.2f us)  decode split %.2f us + combine %.2f us "
        "(%.1f GB/s)" % (pre_ms * 1e3, tflops, pre_t[K // 2] * 1e3, split_ms * 1e3, comb_ms * 1e3,
                         dec_gbs))

    traffic = measured_traffic()
    line = {
        "metric": "attention fwd TFLOP/s (N=4096,D=64) + decode KV GB/s; % of roofline",
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "prewarm_ms": round(pw_ms, 1),
        "prewarm_steps": pw_steps,
        "ms_per_step": round(total_ms / K, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "context_pages_tflops": PAGES_F32_TFLOPS,
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
                     "traffic": traffic.get("fwd_f32"), "kernel": "fwd_f32_rows_kernel<64, false, 2, 2>",
                     "us": round(pre_ms * 1e3, 3), "us_median": round(pre_t[K // 2] * 1e3, 3),
                     "flops_per_launch": pre.flops},
        "accuracy": acc.get(pre.name),
        "decode": {"value": round(dec_gbs, 1), "unit": "GB/s", "us": round(dec_ms * 1e3, 2),
                   "us_median": round(dec_t[K // 2] * 1e3, 2),
                   "split_us": round(split_ms * 1e3, 2), "combine_us": round(comb_ms * 1e3, 2),
                   "bytes": dec.kv_bytes, "accuracy": acc.get(dec.name)},
        "roofline_decode": {"bound": "hbm", "achieved": round(dec_gbs, 1), "peak": PEAK_HBM,
                            "unit": "GB/s", "frac": round(dec_gbs / PEAK_HBM, 4),
                            "traffic": traffic.get("decode_split"),
                            "kernel": "decode_split + decode_combine",
                            "us": round(dec_ms * 1e3, 2)},
        "extra": extra,
        "cpu_baseline": base,
        "speedup_vs_cpu_baseline": round(tflops / base["value"], 1) if base else None,
        "wall_s_timed": round(wall, 3),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
