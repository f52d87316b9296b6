"""GPU parity of attn_bwd against the fp64 oracle, through the C ABI.

The path under test is the one a caller runs: attn_fwd (O and LSE on the
GPU) then attn_bwd.  The oracle sees only Q, K, V and dO and forms O, P and
D itself in float64.

Bounds, with u the unit roundoff of the I/O dtype (2^-11 for f16, 2^-8 for
bf16).  P and dS are rounded to the dtype before their products and the
gradients are rounded on output; everything else is float32 with errors far
below u.  Each rounding is a relative error of at most u on one term, so
  * over a whole gradient tensor the error behaves like a sum of independent
    rounding errors: relative L2 error at most 2u;
  * elementwise, the error of one entry is at most about u times the sum of
    the absolute values of its terms, which for these N(0,1) inputs stays
    below 4u times the largest entry of that tensor (the check used);
  * D = rowsum(dO o O) uses the forward's rounded O, so it may differ from
    the oracle's exact D by at most sum_d |dO_id| times the forward's bound
    on O (4e-3);
  * where a gradient is exactly zero (one key: dS = dP - D cancels) the
    float32 difference of two 64-term dot products is left: an absolute
    floor of 1e-5 covers it, and the relative L2 check is skipped for
    tensors whose largest entry is below 1e-3;
  * the relative L2 bound rests on many independent errors averaging out,
    so it applies only where each entry sums at least 16 terms (dQ: keys,
    dK and dV: queries).  With two keys, dQ_1 = scale dS_10 (k_0 - k_1) and
    dS_10 carries the error of D, which is formed from the rounded O: when
    the entry nearly cancels, its relative error is not bounded by u and only
    the max-abs bound holds.
"""
import numpy as np
import pytest

import oracle
from exact_attention_fa2_amd import fa2, inputs
from gpu_util import TOL, download_f64, report, torch_dtype, upload

pytestmark = pytest.mark.gpu

# float32 rounds nothing to a narrower type: its gradients carry only float32
# sums of a few thousand terms, whose errors stay far below 2^-16 of the
# largest entry (the bounds below are then loose, not tight).
U = {"f16": 2.0 ** -11, "bf16": 2.0 ** -8, "f32": 2.0 ** -16}
FLOOR = 1e-5


def run(B, H, Nq, Nk, dt, scale, causal, seed, heads=None, D=64):
    import torch
    q, k, v = inputs.qkv((B, H, Nq, D), (B, H, Nk, D), seed, dt)
    g = inputs.normal((B, H, Nq, D), seed, 3, dt)
    tq, tk, tv, tg = (upload(x, dt) for x in (q, k, v, g))
    if Nq > 0:
        o, lse = fa2.attn_fwd(tq, tk, tv, scale=scale, causal=causal, return_lse=True)
    else:
        o, lse = torch.empty_like(tq), torch.empty((B, H, 0), dtype=torch.float32, device="cuda")
    dq, dk, dv, delta = fa2.attn_bwd(tq, tk, tv, o, tg, lse, scale=scale, causal=causal)
    torch.cuda.synchronize()
    got = [download_f64(t).reshape(B * H, -1, D) for t in (dq, dk, dv)]
    got.append(download_f64(delta).reshape(B * H, -1))
    q64, k64, v64, g64 = (inputs.to_f64(x, dt) for x in (q, k, v, g))
    ref = oracle.attn_bwd(q64, k64, v64, g64, scale, causal, heads=heads)
    if heads is not None:
        got = [x[heads] for x in got]
        g64 = g64.reshape(B * H, Nq, D)[heads]
    return got, ref, g64.reshape(len(got[0]), Nq, D)


def check(name, dt, got, ref, g64):
    u = U[dt]
    nq, nk = ref[0].shape[1], ref[1].shape[1]
    for label, x, r, terms in zip(("dQ", "dK", "dV"), got[:3], ref[:3], (nk, nq, nq)):
        if r.size == 0:
            continue
        e, msg = report("%s %s" % (name, label), x, r)
        assert np.all(np.isfinite(x)), msg
        scale_ = float(np.abs(r).max())
        assert e <= 4 * u * scale_ + FLOOR, msg + " > 4u max|ref| = %.3e" % (4 * u * scale_)
        if scale_ >= 1e-3 and terms >= 16:
            rel = float(np.linalg.norm(x - r) / np.linalg.norm(r))
            assert rel <= 2 * u, msg + " rel L2 %.3e > 2u" % rel
    if ref[3].size:
        bound = TOL[dt] * np.abs(g64).sum(axis=-1)
        e, msg = report("%s D" % name, got[3], ref[3])
        assert np.all(np.abs(got[3] - ref[3]) <= bound + 1e-6), msg


SMALL = [  # B, H, Nq, Nk, causal, scale
    (1, 2, 256, 256, False, 0.125),
    (1, 2, 256, 256, True, 0.125),
    (1, 1, 300, 200, False, 0.125),
    (1, 2, 333, 333, True, 0.125),
    (2, 1, 100, 1000, False, 0.125),
    (1, 1, 1000, 70, False, 0.125),
    (1, 1, 65, 65, True, 0.125),
    (1, 1, 129, 129, True, 0.125),
    (1, 1, 1, 1, False, 0.125),
    (1, 1, 1, 1, True, 0.125),
    (1, 1, 2, 31, False, 0.125),
    (1, 2, 1024, 1024, True, 0.5),   # the fused-attention tutorial's shape and scale
    (1, 2, 1024, 1024, False, 0.5),
]


@pytest.mark.parametrize("dt", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("B,H,Nq,Nk,causal,scale", SMALL)
def test_bwd_parity(B, H, Nq, Nk, causal, scale, dt):
    name = "bwd B%d H%d Nq%d Nk%d %s %s s%.3g" % (B, H, Nq, Nk, dt, "causal" if causal else "full",
                                                   scale)
    print(name, flush=True)
    got, ref, g64 = run(B, H, Nq, Nk, dt, scale, causal, seed=5)
    check(name, dt, got, ref, g64)


@pytest.mark.parametrize("dt,causal", [("f16", False), ("bf16", False), ("f16", True),
                                       ("bf16", True), ("f32", False), ("f32", True)])
def test_bwd_bench_shape_heads(dt, causal):
    """B4 H12 N2048 (the multi-head benchmark shape), three whole heads
    (first, middle, last) against the oracle."""
    heads = [0, 23, 47]
    name = "bwd B4 H12 N2048 %s %s heads %s" % (dt, "causal" if causal else "full", heads)
    print(name, flush=True)
    got, ref, g64 = run(4, 12, 2048, 2048, dt, 0.125, causal, seed=0, heads=heads)
    check(name, dt, got, ref, g64)


SMALL_D128 = [  # B, H, Nq, Nk, causal
    (1, 2, 256, 256, False), (1, 2, 256, 256, True), (1, 1, 300, 200, False),
    (1, 2, 333, 333, True), (2, 1, 100, 1000, False), (1, 1, 1000, 70, False),
    (1, 1, 1, 1, False), (1, 1, 1, 1, True), (1, 1, 65, 65, True), (1, 2, 1024, 1024, True),
]


@pytest.mark.parametrize("dt", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("B,H,Nq,Nk,causal", SMALL_D128)
def test_bwd_parity_d128(B, H, Nq, Nk, causal, dt):
    """Head dimension 128: two waves share each slice of queries in the dK/dV
    pass and split its output columns; same bounds as D = 64."""
    scale = 1.0 / 128 ** 0.5
    name = "bwd D128 B%d H%d Nq%d Nk%d %s %s" % (B, H, Nq, Nk, dt, "causal" if causal else "full")
    print(name, flush=True)
    got, ref, g64 = run(B, H, Nq, Nk, dt, scale, causal, seed=8, D=128)
    check(name, dt, got, ref, g64)


@pytest.mark.parametrize("dt,causal", [("f16", False), ("bf16", False), ("f16", True),
                                       ("f32", False), ("f32", True)])
def test_bwd_d128_bench_shape_heads(dt, causal):
    heads = [0, 23, 47]
    name = "bwd B4 H12 N2048 D128 %s %s heads %s" % (dt, "causal" if causal else "full", heads)
    print(name, flush=True)
    got, ref, g64 = run(4, 12, 2048, 2048, dt, 1.0 / 128 ** 0.5, causal, seed=0, heads=heads, D=128)
    check(name, dt, got, ref, g64)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("dt", ["f16", "bf16", "f32"])
def test_bwd_no_queries(dt, D):
    """Nq = 0: no query attends any key, so dK = dV = 0 exactly."""
    import torch
    tdt = torch_dtype(dt)
    k = torch.randn(2, 3, 100, D, device="cuda").to(tdt)
    v = torch.randn(2, 3, 100, D, device="cuda").to(tdt)
    q = torch.empty(2, 3, 0, D, device="cuda", dtype=tdt)
    lse = torch.empty(2, 3, 0, device="cuda")
    dk = torch.full_like(k, 7.0)
    dv = torch.full_like(v, 7.0)
    fa2.attn_bwd(q, k, v, q, q, lse, dk=dk, dv=dv)
    torch.cuda.synchronize()
    assert torch.count_nonzero(dk).item() == 0 and torch.count_nonzero(dv).item() == 0


@pytest.mark.parametrize("dt", ["f16", "bf16", "f32"])
def test_bwd_rejects(dt):
    """D other than 64 and 128 is refused before anything is enqueued."""
    import torch
    lse = torch.zeros(1, 1, 8, device="cuda")
    for D in (32, 96):
        h = torch.zeros(1, 1, 8, D, device="cuda", dtype=torch_dtype(dt))
        with pytest.raises(fa2.FA2Error) as e:
            fa2.attn_bwd(h, h, h, h, h, lse)
        assert e.value.status == 3


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("dt", ["f16", "bf16", "f32"])
def test_bwd_deterministic(dt, D):
    """No atomics: two runs give the same bits."""
    import torch
    q, k, v = inputs.qkv((2, 3, 300, D), (2, 3, 300, D), 6, dt)
    g = inputs.normal((2, 3, 300, D), 6, 3, dt)
    tq, tk, tv, tg = (upload(x, dt) for x in (q, k, v, g))
    o, lse = fa2.attn_fwd(tq, tk, tv, scale=0.125, causal=True, return_lse=True)
    a = fa2.attn_bwd(tq, tk, tv, o, tg, lse, scale=0.125, causal=True)
    b = fa2.attn_bwd(tq, tk, tv, o, tg, lse, scale=0.125, causal=True)
    torch.cuda.synchronize()
    assert all(torch.equal(x, y) for x, y in zip(a, b))


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("dt", ["f16", "bf16", "f32"])
def test_bwd_offsets_past_2_31_elements(dt, D):
    """B*H = 8192 heads of N = 4096 at D = 64 (4096 heads at D = 128): each
    [B,H,N,D] tensor holds 2^31 elements, so the last heads sit past any
    32-bit element offset.
    Q = K = 0 makes every P exactly 2^-12; with dO and V in {-1, +1} the
    gradients are exact: dQ = dK = 0 and dV_j = 2^-12 sum_q dO_q for every key
    j (a sum of 4096 terms of +-1, exact in float32).  Checked in full for the
    first, a middle and the last heads, and dQ = dK = 0 everywhere."""
    import torch
    tdt = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}[dt]
    B, H, N = 128 * 64 // D, 64, 4096
    gen = torch.Generator(device="cuda").manual_seed(7)
    shape = (B, H, N, D)
    q = torch.zeros(shape, device="cuda", dtype=tdt)
    k = torch.zeros(shape, device="cuda", dtype=tdt)
    v = (torch.randint(0, 2, shape, device="cuda", generator=gen, dtype=torch.int8) * 2 - 1).to(tdt)
    g = (torch.randint(0, 2, shape, device="cuda", generator=gen, dtype=torch.int8) * 2 - 1).to(tdt)
    o, lse = fa2.attn_fwd(q, k, v, scale=0.125, return_lse=True)
    dq, dk, dv, _ = fa2.attn_bwd(q, k, v, o, g, lse, scale=0.125)
    torch.cuda.synchronize()
    assert torch.count_nonzero(dq).item() == 0
    assert torch.count_nonzero(dk).item() == 0
    gf = g.view(B * H, N, D)
    dvf = dv.view(B * H, N, D)
    for head in (0, B * H // 2 + 3, B * H - 1):
        # the exact value, rounded to the output dtype as the kernel rounds its exact f32 sum
        want = (gf[head].double().sum(dim=0) / N).to(tdt).double()
        got = dvf[head].double()
        assert torch.equal(got, want.expand_as(got)), head
