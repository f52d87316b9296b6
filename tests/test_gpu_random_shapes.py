"""Parity on a fixed list of pseudo-random shapes, forward, backward and
flash-decoding, against the fp64 oracle through the C ABI.

The named workloads and the hand-picked ragged cases test what was designed
for; this list (drawn once from a seeded generator, so every run checks the
same cases) mixes batch, heads, lengths from 1 to 2000 (700 backward), head
dimension, dtype, scale and the causal flag in combinations nobody chose,
which reach the schedules (key split or not, 128 or 256 rows per workgroup,
one round of workgroups or several) and their ragged edges in other ways.
Bounds are those of the other parity tests: gpu_util.edge_tol on O, 1e-4 on
the LSE, and the backward's u-relative bounds.
"""
import math

import numpy as np
import pytest

from exact_attention_fa2_amd import fa2, workloads
from test_gpu_bwd import check as check_bwd
from test_gpu_bwd import run as run_bwd
from test_gpu_fwd import check_full

pytestmark = pytest.mark.gpu


def _length(g, hi):
    """Half log-uniform on [1, hi] (short and ragged), half uniform on
    [128, hi] (several tiles and blocks)."""
    if g.integers(2):
        return int(g.integers(128, hi + 1))
    return int(min(hi, max(1, round(math.exp(g.uniform(0.0, math.log(hi)))))))


def _forward_cases(n=96, seed=2024):
    g = np.random.default_rng(seed)
    out = []
    for i in range(n):
        dt = ("f32", "f16", "bf16")[i % 3]
        D = int(g.choice([64, 128]))
        causal = bool(g.integers(2))
        B, H = int(g.integers(1, 4)), int(g.integers(1, 5))
        Nq = _length(g, 2000)
        Nk = Nq if causal else _length(g, 2000)
        # scale 0.5 makes the softmax peaky; it is the fused-attention
        # tutorial's setting at D = 64 only (at D = 128 the f16 bound would not
        # hold for the largest outputs), so larger D takes 1/sqrt(D)
        scale = float(g.choice([D ** -0.5, 0.07] + ([0.5] if D == 64 else [])))
        out.append((B, H, Nq, Nk, D, dt, scale, causal, 1000 + i))
    return out


def _backward_cases(n=32, seed=77):
    g = np.random.default_rng(seed)
    out = []
    for i in range(n):
        dt = ("f16", "bf16", "f32")[i % 3]
        D = int(g.choice([64, 128]))
        causal = bool(g.integers(2))
        B, H = int(g.integers(1, 3)), int(g.integers(1, 4))
        Nq = _length(g, 700)
        Nk = Nq if causal else _length(g, 700)
        out.append((B, H, Nq, Nk, D, dt, D ** -0.5, causal, 2000 + i))
    return out


def _large_forward_cases(n=30, seed=7):
    """Many heads and long rows: several rounds of workgroups, 256-row tiles,
    the XCD remap.  Checked on sampled rows."""
    g = np.random.default_rng(seed)
    out = []
    for i in range(n):
        dt = ("f32", "f16", "bf16")[i % 3]
        D = int(g.choice([64, 128]))
        causal = bool(g.integers(2))
        B, H = int(g.integers(1, 9)), int(g.integers(1, 33))
        Nq = int(g.integers(128, 4097))
        Nk = Nq if causal else int(g.integers(128, 4097))
        out.append((B, H, Nq, Nk, D, dt, float(g.choice([D ** -0.5, 0.07])), causal, 5000 + i))
    return out


def _large_backward_cases(n=12, seed=11):
    """Up to 64 heads and 2048 rows; checked on a few sampled heads."""
    g = np.random.default_rng(seed)
    out = []
    for i in range(n):
        dt = ("f16", "bf16", "f32")[i % 3]
        D = int(g.choice([64, 128]))
        causal = bool(g.integers(2))
        B, H = int(g.integers(1, 5)), int(g.integers(1, 17))
        Nq = int(g.integers(64, 2049))
        Nk = Nq if causal else int(g.integers(64, 2049))
        out.append((B, H, Nq, Nk, D, dt, D ** -0.5, causal, 7000 + i))
    return out


def _decode_cases(n=48, seed=777):
    """Flash-decoding: lengths log-uniform on [1, 70000], split counts from 1
    to 64 (more splits than 64-key blocks included), unusual scales."""
    g = np.random.default_rng(seed)
    out = []
    for i in range(n):
        dt = ("f16", "bf16", "f32")[i % 3]
        D = int(g.choice([64, 128]))
        B, H = int(g.integers(1, 5)), int(g.integers(1, 9))
        N = int(min(70000, max(1, round(math.exp(g.uniform(0, math.log(70000)))))))
        ns = int(g.choice([1, 2, 3, 5, 8, 13, 16, 32, 64]))
        scale = float(g.choice([D ** -0.5, D ** -0.5, 0.0, -0.1, 0.5]))
        out.append((B, H, N, D, dt, ns, scale, 300 + i))
    return out


FWD = _forward_cases()
BWD = _backward_cases()
FWD_LARGE = _large_forward_cases()
BWD_LARGE = _large_backward_cases()
DEC = _decode_cases()


def _id(c):
    B, H, Nq, Nk, D, dt, scale, causal, _ = c
    return "B%dH%d_%dx%d_D%d_%s_s%.3g%s" % (B, H, Nq, Nk, D, dt, scale, "_c" if causal else "")


@pytest.mark.parametrize("case", FWD, ids=_id)
def test_forward(case):
    B, H, Nq, Nk, D, dt, scale, causal, seed = case
    check_full(workloads.Prefill("random " + _id(case), B, H, Nq, Nk, D, dt, scale, causal, seed),
               edge=True)


@pytest.mark.parametrize("case", BWD, ids=_id)
def test_backward(case):
    B, H, Nq, Nk, D, dt, scale, causal, seed = case
    got, ref, g64 = run_bwd(B, H, Nq, Nk, dt, scale, causal, seed, D=D)
    check_bwd("random " + _id(case), dt, got, ref, g64)


@pytest.mark.parametrize("case", FWD_LARGE, ids=_id)
def test_forward_large(case):
    B, H, Nq, Nk, D, dt, scale, causal, seed = case
    total = B * H * Nq
    g = np.random.default_rng(seed)
    rows = np.unique(np.concatenate([g.choice(total, min(total, 384), replace=False),
                                     np.arange(64), total - 1 - np.arange(64)]))
    check_full(workloads.Prefill("random " + _id(case), B, H, Nq, Nk, D, dt, scale, causal, seed),
               rows, edge=True)


@pytest.mark.parametrize("case", BWD_LARGE, ids=_id)
def test_backward_large(case):
    B, H, Nq, Nk, D, dt, scale, causal, seed = case
    g = np.random.default_rng(seed)
    heads = sorted(set(g.choice(B * H, min(B * H, 3), replace=False).tolist()) | {0, B * H - 1})
    got, ref, g64 = run_bwd(B, H, Nq, Nk, dt, scale, causal, seed, heads=heads, D=D)
    check_bwd("random " + _id(case), dt, got, ref, g64)


@pytest.mark.parametrize("dt,D", [("f32", 64), ("f16", 64), ("bf16", 64), ("f32", 128),
                                  ("f16", 128), ("bf16", 128)])
@pytest.mark.parametrize("scale", [0.0, -0.125, 2.0])
@pytest.mark.parametrize("causal", [False, True])
def test_forward_unusual_scales(scale, causal, dt, D):
    """scale 0 (every score 0: the mean of the live values), a negative scale
    (attention to the least similar keys) and a large one (one key per row
    dominates)."""
    check_full(workloads.Prefill("scale %g" % scale, 2, 3, 200, 200, D, dt, scale, causal, 31),
               edge=True)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("dt", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("scale", [0.0, -0.125])
def test_backward_unusual_scales(scale, dt, D):
    got, ref, g64 = run_bwd(1, 2, 150, 150, dt, scale, True, 32, D=D)
    check_bwd("scale %g" % scale, dt, got, ref, g64)


@pytest.mark.parametrize("scale", [0.0, -0.125, 2.0])
@pytest.mark.parametrize("causal", [False, True])
def test_forward_unusual_scales_without_workspace(scale, causal):
    """The same for the float32 16-row kernel (no workspace, no key split)."""
    import torch
    from gpu_util import LSE_TOL, TOL, assert_close, download_f64, seeded, upload
    import oracle
    from exact_attention_fa2_amd import inputs
    q, k, v = seeded(1, 2, 300, 300, 64, "f32", 33)
    o, lse = fa2.attn_fwd(upload(q, "f32"), upload(k, "f32"), upload(v, "f32"), scale=scale,
                          causal=causal, return_lse=True, use_workspace=False)
    torch.cuda.synchronize()
    ro, rl = oracle.attn(*(inputs.to_f64(x, "f32") for x in (q, k, v)), scale, causal)
    assert_close("f32 no workspace scale %g O" % scale, download_f64(o), ro, TOL["f32"])
    assert_close("f32 no workspace scale %g LSE" % scale, download_f64(lse), rl, LSE_TOL)


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("scale", [0.0, -0.09, 1.5])
def test_decode_unusual_scales(scale, dt):
    """Flash-decoding with the same scales.  A large scale makes the softmax
    peaky and |O| passes 2, where half a bf16 spacing (2^-7) exceeds the plain
    4e-3 bar: bf16 takes the output-rounding bound of gpu_util.edge_tol."""
    import oracle
    from exact_attention_fa2_amd import inputs
    from gpu_util import assert_close, edge_tol
    from test_gpu_decode import run as run_decode
    (q, k, v, _), o, *_ = run_decode(2, 3, 777, 128, dt, 5, seed=34, scale=scale)
    q64, k64, v64 = (inputs.to_f64(x, dt) for x in (q, k, v))
    ref = oracle.attn(q64[:, :, None], k64, v64, scale)[0][:, :, 0]
    assert_close("decode scale %g %s" % (scale, dt), o, ref, edge_tol(dt, ref, o))


@pytest.mark.parametrize("case", DEC, ids=lambda c: "B%dH%d_N%d_D%d_%s_ns%d_s%.3g" % c[:7])
def test_decode(case):
    """The combined output against the oracle's attention of the one row, and
    the partials against the oracle's split."""
    import oracle
    from exact_attention_fa2_amd import inputs
    from gpu_util import TOL, assert_close, edge_tol
    from test_gpu_decode import check_partials
    from test_gpu_decode import run as run_decode
    B, H, N, D, dt, ns, scale, seed = case
    name = "random decode B%d H%d N%d D%d %s splits %d scale %g" % (B, H, N, D, dt, ns, scale)
    (q, k, v, sc), o, op, mp, lp = run_decode(B, H, N, D, dt, ns, seed=seed, scale=scale)
    q64, k64, v64 = (inputs.to_f64(x, dt) for x in (q, k, v))
    ro = oracle.attn(q64[:, :, None], k64, v64, sc)[0][:, :, 0]
    assert_close(name, o, ro, edge_tol(dt, ro, o))
    rop, rmp, rlp = oracle.decode_split(q64, k64, v64, sc, ns)
    check_partials(name + " partials", op, mp, lp, rop, rmp, rlp, TOL[dt])
