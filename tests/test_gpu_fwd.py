"""GPU parity of attn_fwd against the fp64 oracle, through the C ABI.

Tolerances (max abs on O): 1e-4 for f32 I/O, 4e-3 for f16/bf16 I/O; LSE
1e-4.  Inputs are the seeded N(0,1) workloads of workloads.py plus ragged and
degenerate cases.
"""
import numpy as np
import pytest

import oracle
from exact_attention_fa2_amd import fa2, inputs, workloads
from gpu_util import (LSE_TOL, TOL, assert_close, download_f64, edge_tol, seeded, torch_dtype,
                      upload)

pytestmark = pytest.mark.gpu


def run_fwd(q, k, v, dt, scale, causal, lse=True):
    """Run attn_fwd; with ``lse`` also run it without the LSE output (the
    kernels then skip the float32 row sum) and require the same O bit for
    bit."""
    tq, tk, tv = upload(q, dt), upload(k, dt), upload(v, dt)
    out = fa2.attn_fwd(tq, tk, tv, scale=scale, causal=causal, return_lse=lse)
    import torch
    torch.cuda.synchronize()
    if lse:
        o_only = fa2.attn_fwd(tq, tk, tv, scale=scale, causal=causal)
        torch.cuda.synchronize()
        assert torch.equal(o_only, out[0]), "O differs between the runs with and without LSE"
        return download_f64(out[0]), download_f64(out[1])
    return download_f64(out), None


def check_full(cfg, rows=None, edge=False):
    """Compare with the oracle.  ``edge`` selects the bound for cases outside
    the named workloads (see gpu_util.edge_tol); named workloads use the plain
    bar."""
    q, k, v = seeded(cfg.B, cfg.H, cfg.Nq, cfg.Nk, cfg.D, cfg.dtype, cfg.seed)
    o, lse = run_fwd(q, k, v, cfg.dtype, cfg.scale, cfg.causal)
    q64, k64, v64 = (inputs.to_f64(x, cfg.dtype) for x in (q, k, v))
    if rows is None:
        ro, rl = oracle.attn(q64, k64, v64, cfg.scale, cfg.causal)
        wabs = oracle.attn(q64, k64, np.abs(v64), cfg.scale, cfg.causal)[0] if edge else None
        tol = edge_tol(cfg.dtype, ro, o, wabs) if edge else TOL[cfg.dtype]
        assert_close(cfg.name + " O", o, ro, tol)
        assert_close(cfg.name + " LSE", lse, rl, LSE_TOL)
    else:
        ro, rl = oracle.attn_rows(q64, k64, v64, cfg.scale, cfg.causal, rows)
        got = o.reshape(-1, cfg.D)[rows]
        tol = TOL[cfg.dtype]
        if edge:
            wabs = oracle.attn_rows(q64, k64, np.abs(v64), cfg.scale, cfg.causal, rows)[0]
            tol = edge_tol(cfg.dtype, ro, got, wabs)
        assert_close(cfg.name + " O (sampled rows)", got, ro, tol)
        assert_close(cfg.name + " LSE (sampled rows)", lse.reshape(-1)[rows], rl, LSE_TOL)


def test_tiny_f32():
    check_full(workloads.TINY_F32)


def test_headline_f32_4096():
    check_full(workloads.HEADLINE_F32)


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("n", [512, 1024])
def test_multihead_full(n, dt):
    check_full(workloads.multihead(n, dt))


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_multihead_2048_full(dt):
    """The multi-head workload at its primary length, every one of the
    4*12*2048 rows (O and LSE) against the oracle, at the plain bar."""
    check_full(workloads.multihead(2048, dt))


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_causal_one_round_snake_order(dt):
    """B4 H12 N2048 causal: the 768 tiles fit one round of workgroup slots, so
    the kernel deals them to the compute units in a snake by length; every
    row of heads 0, 23 and 47 plus 1024 random rows against the oracle (bf16
    takes the format bound: early causal rows average few keys)."""
    cfg = workloads.Prefill("B4 H12 N2048 causal %s" % dt, 4, 12, 2048, 2048, 64, dt, 0.125, True,
                            16)
    g = np.random.default_rng(4)
    total = cfg.B * cfg.H * cfg.Nq
    rows = np.unique(np.concatenate([np.arange(2048), 23 * 2048 + np.arange(2048),
                                     total - 2048 + np.arange(2048), g.choice(total, 1024, replace=False)]))
    check_full(cfg, rows, edge=(dt == "bf16"))


@pytest.mark.parametrize("dt,causal", [("f16", False), ("f16", True), ("bf16", False)])
def test_many_heads_64_rows_per_wave(dt, causal):
    """B4 H64 N2048: 256-row query tiles fill every compute unit with two
    workgroups in whole rounds, so the f16/bf16 kernel runs 64 query rows per
    wave.  Sampled rows against the oracle (the early causal rows of bf16
    would need the format bound of the edge tests, so bf16 runs non-causal)."""
    cfg = workloads.Prefill("B4 H64 N2048 %s" % dt, 4, 64, 2048, 2048, 64, dt, 0.125, causal, 14)
    g = np.random.default_rng(2)
    total = cfg.B * cfg.H * cfg.Nq
    rows = np.unique(np.concatenate([np.arange(256), total - 1 - np.arange(256),
                                     g.choice(total, 768, replace=False)]))
    check_full(cfg, rows)


@pytest.mark.parametrize("causal", [True, False])
def test_causal_lse_f16(causal):
    check_full(workloads.causal_lse(causal))


@pytest.mark.parametrize("causal", [True, False])
def test_causal_lse_shape_in_bf16(causal):
    """The causal workload's shape in bf16 (not a named workload): early causal
    rows average few keys, so |O| reaches ~3 and the bf16 format bound applies."""
    c = workloads.causal_lse(causal)
    cfg = workloads.Prefill(c.name + " bf16", c.B, c.H, c.Nq, c.Nk, c.D, "bf16", c.scale,
                            c.causal, c.seed)
    check_full(cfg, edge=True)


RAGGED = [  # (B, H, Nq, Nk, causal)
    (1, 1, 1, 1, False), (1, 1, 1, 1, True), (2, 3, 77, 131, False), (1, 2, 200, 200, True),
    (3, 1, 129, 65, False), (1, 1, 17, 1000, False), (2, 2, 300, 300, True),
    (1, 4, 129, 129, True), (1, 1, 64, 1, False),
]


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("shape", RAGGED, ids=lambda s: "x".join(map(str, s)))
def test_ragged_and_degenerate(shape, dt):
    B, H, Nq, Nk, causal = shape
    cfg = workloads.Prefill("ragged", B, H, Nq, Nk, 64, dt, 0.125, causal, 3)
    check_full(cfg, edge=True)


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
def test_tile_grid_not_multiple_of_eight(dt):
    # 3 heads x 3 query tiles: the XCD remap is skipped when the tile count is not a multiple of 8
    cfg = workloads.Prefill("odd grid", 1, 3, 384, 256, 64, dt, 0.125, False, 4)
    check_full(cfg, edge=True)
    cfg = workloads.Prefill("odd grid causal", 1, 3, 384, 384, 64, dt, 0.125, True, 4)
    check_full(cfg, edge=True)


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
def test_identity_values_rows_sum_to_one(dt):
    """V = I with Nk = D = 64: O is the probability matrix; rows sum to 1."""
    q, k, _ = seeded(1, 2, 100, 64, 64, dt, 7)
    eye = np.broadcast_to(np.eye(64, dtype=np.float32), (1, 2, 64, 64)).copy()
    v = inputs.f32_to_bf16_bits(eye) if dt == "bf16" else eye.astype(
        inputs.storage_numpy_dtype(dt))
    o, _ = run_fwd(q, k, v, dt, 0.3, False)
    # P is rounded to the storage dtype before the PV product (relative 2^-11
    # for f16, 2^-9 for bf16) and each output once more, so a row sum can
    # drift by twice that relative step; f32 keeps full precision.
    sums = o.sum(axis=-1)
    bound = {"f32": 1e-5, "f16": 2e-3, "bf16": 8e-3}[dt]
    assert np.max(np.abs(sums - 1.0)) <= bound, np.max(np.abs(sums - 1.0))
    ro, _ = oracle.attn(inputs.to_f64(q, dt), inputs.to_f64(k, dt), inputs.to_f64(v, dt), 0.3)
    assert_close("V=I " + dt, o, ro, edge_tol(dt, ro, o))


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
def test_zero_keys_give_mean_of_values(dt, causal):
    q, _, v = seeded(1, 1, 256, 256, 64, dt, 8)
    k = np.zeros_like(q)
    o, lse = run_fwd(q, k, v, dt, 0.125, causal)
    v64 = inputs.to_f64(v, dt)[0, 0]
    if causal:
        want = np.cumsum(v64, axis=0) / np.arange(1, 257)[:, None]
        want_lse = np.log(np.arange(1, 257))
    else:
        want = np.broadcast_to(v64.mean(axis=0), (256, 64))
        want_lse = np.full(256, np.log(256))
    assert_close("K=0 " + dt, o[0, 0], want, edge_tol(dt, want, o[0, 0]))
    assert_close("K=0 LSE " + dt, lse[0, 0], want_lse, LSE_TOL)
    if causal:  # row 0 sees key 0 alone: exactly V_0
        assert np.array_equal(o[0, 0, 0], v64[0])


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
def test_large_score_shift_is_safe(dt):
    """Scores far past exp's f32 overflow (about 88) must not overflow: the
    kernels subtract the running max.  K' = K + u shifts every score of row i
    by the same scale*q_i.u, and GPU(K') is compared with oracle(K')."""
    q, k, v = seeded(1, 2, 130, 190, 64, dt, 9)
    k64 = inputs.to_f64(k, dt)
    k64[..., :4] += 64.0
    k32 = k64.astype(np.float32)
    k2 = inputs.f32_to_bf16_bits(k32) if dt == "bf16" else k32.astype(inputs.storage_numpy_dtype(dt))
    o, lse = run_fwd(q, k2, v, dt, 0.5, False)
    ro, rl = oracle.attn(inputs.to_f64(q, dt), inputs.to_f64(k2, dt), inputs.to_f64(v, dt), 0.5)
    wabs = oracle.attn(inputs.to_f64(q, dt), inputs.to_f64(k2, dt), np.abs(inputs.to_f64(v, dt)),
                       0.5)[0]
    assert np.max(np.abs(rl)) > 100
    assert np.all(np.isfinite(o))
    # float32 keeps the plain 1e-4 bar even with scores near 100 (measured
    # 3.7e-5); half-precision inputs keep their own bound.
    tol = TOL["f32"] if dt == "f32" else edge_tol(dt, ro, o, wabs)
    assert_close("shift O " + dt, o, ro, tol)
    assert_close("shift LSE " + dt, lse, rl, LSE_TOL)


@pytest.mark.parametrize("order", ["rising", "falling"])
@pytest.mark.parametrize("dt,shape", [("f32", (1, 1, 1024, 1024)), ("f32", (4, 16, 256, 256)),
                                      ("f16", (1, 2, 1024, 1024)), ("bf16", (2, 4, 1024, 1024))],
                         ids=lambda v: "x".join(map(str, v)) if isinstance(v, tuple) else str(v))
def test_running_max_moves_often(order, dt, shape):
    """Scores that grow (or shrink) steadily along the keys: with Q[..., 0] = 4
    and K[j, 0] += 0.05 j, scale 0.5 adds 0.1 j to every score of key j (up to
    about 100), so while a wave walks its keys the running max passes its
    previous value by far more than the kernels' rescale threshold again and
    again ("rising"), or is set by the first keys and never moves
    ("falling").  Every schedule runs (f32: with and without a workspace, and
    the shared-K/V kernel at 4x16 heads of 256 rows)."""
    import torch
    B, H, Nq, Nk = shape
    q, k, v = seeded(B, H, Nq, Nk, 64, dt, 14)
    q64, k64 = inputs.to_f64(q, dt), inputs.to_f64(k, dt)
    ramp = 0.05 * np.arange(Nk)
    q64[..., 0] = 4.0
    k64[..., 0] += ramp if order == "rising" else ramp[::-1]
    def store(x):
        x32 = x.astype(np.float32)
        return inputs.f32_to_bf16_bits(x32) if dt == "bf16" else x32.astype(inputs.storage_numpy_dtype(dt))
    q, k = store(q64), store(k64)
    q64, k64, v64 = (inputs.to_f64(x, dt) for x in (q, k, v))
    tq, tk, tv = upload(q, dt), upload(k, dt), upload(v, dt)
    for causal in (False, True):
        ro, rl = oracle.attn(q64, k64, v64, 0.5, causal)
        wabs = oracle.attn(q64, k64, np.abs(v64), 0.5, causal)[0]
        for use_ws in ((True, False) if dt == "f32" else (True,)):
            o, lse = fa2.attn_fwd(tq, tk, tv, scale=0.5, causal=causal, return_lse=True,
                                  use_workspace=use_ws)
            torch.cuda.synchronize()
            o = download_f64(o)
            tag = "%s %s causal=%d ws=%d" % (order, dt, causal, use_ws)
            assert_close(tag + " O", o, ro, TOL["f32"] if dt == "f32" else edge_tol(dt, ro, o, wabs))
            assert_close(tag + " LSE", download_f64(lse), rl, LSE_TOL)


@pytest.mark.parametrize("scale", [0.0, -0.125, 2.0])
def test_f32_unusual_scales(scale):
    """Scale 0, a negative scale and a large one on the float32 kernels:
    B4 H16 N256 runs 32-row tiles unmasked and the shared-K/V kernel (256
    groups of 64 rows, one per compute unit) causal; one head of 4096 rows
    runs 32-row tiles with the keys split in two and merged in the kernel."""
    import torch
    for (B, H, N), causals in (((4, 16, 256), (False, True)), ((1, 1, 4096), (False,))):
        q, k, v = seeded(B, H, N, N, 64, "f32", 15)
        q64, k64, v64 = (inputs.to_f64(x, "f32") for x in (q, k, v))
        tq, tk, tv = upload(q, "f32"), upload(k, "f32"), upload(v, "f32")
        for causal in causals:
            o, lse = fa2.attn_fwd(tq, tk, tv, scale=scale, causal=causal, return_lse=True)
            torch.cuda.synchronize()
            ro, rl = oracle.attn(q64, k64, v64, scale, causal)
            tag = "f32 B%d H%d N%d scale %g causal=%d" % (B, H, N, scale, causal)
            assert_close(tag + " O", download_f64(o), ro, TOL["f32"])
            assert_close(tag + " LSE", download_f64(lse), rl, LSE_TOL)


def test_f32_split_tile_large_score_shift():
    """The float32 key split merged in the kernel with scores near 100 (far
    past exp's overflow): K' = K + u shifts every score of a row by the same
    amount, so both chunks of a tile carry large maxima."""
    import torch
    q, k, v = seeded(1, 1, 4096, 4096, 64, "f32", 10)
    k = k.copy()
    k[..., :4] += 64.0
    assert fa2.workspace_size(1, 1, 4096, 4096, 64, False, fa2.FA2_F32) > 0
    q64, k64, v64 = (inputs.to_f64(x, "f32") for x in (q, k, v))
    tq, tk, tv = upload(q, "f32"), upload(k, "f32"), upload(v, "f32")
    o, lse = fa2.attn_fwd(tq, tk, tv, scale=0.5, return_lse=True)
    torch.cuda.synchronize()
    ro, rl = oracle.attn(q64, k64, v64, 0.5, False)
    assert np.max(np.abs(rl)) > 100
    assert_close("f32 split shift O", download_f64(o), ro, TOL["f32"])
    assert_close("f32 split shift LSE", download_f64(lse), rl, LSE_TOL)


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
def test_deterministic(dt):
    import torch
    q, k, v = seeded(2, 4, 300, 300, 64, dt, 10)
    tq, tk, tv = upload(q, dt), upload(k, dt), upload(v, dt)
    a = fa2.attn_fwd(tq, tk, tv, scale=0.125, causal=True, return_lse=True)
    b = fa2.attn_fwd(tq, tk, tv, scale=0.125, causal=True, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


F32_SHAPES = [(1, 1, 4096, 4096), (1, 2, 1024, 1024), (1, 1, 200, 200), (2, 3, 77, 131),
              (8, 48, 256, 256), (2, 12, 1024, 1024), (3, 7, 832, 832)]


@pytest.mark.parametrize("shape,causal",
                         [(sh, c) for sh in F32_SHAPES for c in (False, True)
                          if not (c and sh[2] != sh[3])],  # causal needs Nq == Nk
                         ids=lambda v: "x".join(map(str, v)) if isinstance(v, tuple) else str(v))
def test_f32_schedules(shape, causal):
    """The three float32 schedules, each against the oracle: keys split across
    workgroups with a workspace and the combine, the same call without a
    workspace (16-row workgroups), and many 64-row groups (shared K/V, no
    split -- the last three shapes: 16 query tiles per head in two rounds of
    workgroups, then 13 tiles for each of 21 heads, b*h not a multiple of 8)."""
    import torch
    B, H, Nq, Nk = shape
    q, k, v = seeded(B, H, Nq, Nk, 64, "f32", 12)
    ro, rl = oracle.attn(*(inputs.to_f64(x, "f32") for x in (q, k, v)), 0.125, causal)
    tq, tk, tv = upload(q, "f32"), upload(k, "f32"), upload(v, "f32")
    need = fa2.workspace_size(B, H, Nq, Nk, 64, causal, fa2.FA2_F32)
    for use_ws in (True, False):
        o, lse = fa2.attn_fwd(tq, tk, tv, scale=0.125, causal=causal, return_lse=True,
                              use_workspace=use_ws)
        torch.cuda.synchronize()
        tag = "ws=%d need=%d" % (use_ws, need)
        assert_close("f32 schedule %s O" % tag, download_f64(o), ro, TOL["f32"])
        assert_close("f32 schedule %s LSE" % tag, download_f64(lse), rl, LSE_TOL)


# Unmasked float32 D = 64 shapes whose 32-row tiles, split in two, cover the
# device run 32-row workgroups, or 16-row ones where those should finish
# first; where the key split should finish first (split = True, on 256
# compute units) each tile's keys go to two workgroups whose states are
# merged by the second to finish.
ROWS32_SHAPES = [(1, 1, 4090, 4096, True),   # ragged last tile
                 (1, 1, 4096, 4000, True),   # ragged keys
                 (1, 2, 2040, 3333, True),
                 (1, 4, 1000, 4000, True),
                 (1, 1, 4096, 16, False),    # one or two key steps: 32-row tiles, no split
                 (1, 1, 4096, 17, False),
                 (1, 1, 4096, 1, False),
                 (1, 2, 4096, 4096, False),  # 256 tiles of 32 rows
                 (2, 12, 1024, 1024, False),
                 (3, 1, 3000, 2000, False)]  # 282 tiles of 32 rows: the split would save under 3%


@pytest.mark.parametrize("shape", ROWS32_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_f32_rows32(shape):
    """The 32-row float32 kernel, O and LSE against the oracle.  With the key
    split, the workspace starts out as random bytes (the handshake words'
    earlier contents must not matter), every call must leave those words at 0,
    the same call twice must give the same bits, and a call on other values
    with the same workspace must match the oracle again (no state carried
    over).  Without a workspace the shape runs the 16-row kernel."""
    import torch
    B, H, Nq, Nk, split = shape
    need = fa2.workspace_size(B, H, Nq, Nk, 64, False, fa2.FA2_F32)
    assert (need > 0) == split, "the shape takes another schedule (need=%d)" % need
    tiles = B * H * ((Nq + 31) // 32)
    ws = torch.randint(0, 256, (max(need, 1),), dtype=torch.uint8, device="cuda")
    first = None
    for seed in (16, 16, 17):
        q, k, v = seeded(B, H, Nq, Nk, 64, "f32", seed)
        ro, rl = oracle.attn(*(inputs.to_f64(x, "f32") for x in (q, k, v)), 0.125, False)
        tq, tk, tv = upload(q, "f32"), upload(k, "f32"), upload(v, "f32")
        o, lse = fa2.attn_fwd(tq, tk, tv, scale=0.125, return_lse=True, workspace=ws)
        torch.cuda.synchronize()
        tag = "rows32 seed %d split=%d" % (seed, split)
        assert_close(tag + " O", download_f64(o), ro, TOL["f32"])
        assert_close(tag + " LSE", download_f64(lse), rl, LSE_TOL)
        if split:
            words = ws[:8 * tiles].cpu().numpy()
            assert not words.any(), "handshake words left set after the call"
        if first is None:
            first = (o.clone(), lse.clone())
        elif seed == 16:
            assert torch.equal(o, first[0]) and torch.equal(lse, first[1]), "not deterministic"
    o = fa2.attn_fwd(tq, tk, tv, scale=0.125, workspace=ws)  # no LSE asked for
    torch.cuda.synchronize()
    assert_close("rows32 without LSE O", download_f64(o), ro, TOL["f32"])
    o, lse = fa2.attn_fwd(tq, tk, tv, scale=0.125, return_lse=True, use_workspace=False)
    torch.cuda.synchronize()
    assert_close("rows32 shape without workspace O", download_f64(o), ro, TOL["f32"])
    assert_close("rows32 shape without workspace LSE", download_f64(lse), rl, LSE_TOL)


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("shape", [(1, 2, 1024, 1024, True), (1, 2, 1024, 1024, False),
                                   (1, 1, 700, 700, True), (2, 3, 300, 300, False),
                                   (1, 1, 64, 4096, False), (1, 3, 129, 2000, False),
                                   (1, 2, 2048, 8192, False), (1, 1, 33, 33, True),
                                   (2, 2, 1, 1, False), (1, 4, 4096, 4096, True),
                                   (1, 2, 4096, 4096, False), (1, 2, 8192, 8192, False)],
                         ids=lambda s: "x".join(map(str, s)))
def test_mfma_few_tile_schedules(shape, dt):
    """f16/bf16 with few query tiles, O and LSE against the oracle, with and
    without a workspace.  At most one 128-row tile per eight compute units and
    keys up to 2048: one launch of 32-row workgroups whose waves split the
    keys (no workspace asked for).  Longer keys (with few tiles, or with the
    tiles filling at most a quarter of the workgroup slots): the keys are split
    across workgroups into partials that the combine kernel merges when a
    workspace is given, and the plain kernel runs without one."""
    import torch
    B, H, Nq, Nk, causal = shape
    q, k, v = seeded(B, H, Nq, Nk, 64, dt, 13)
    q64, k64, v64 = (inputs.to_f64(x, dt) for x in (q, k, v))
    ro, rl = oracle.attn(q64, k64, v64, 0.125, causal)
    wabs = oracle.attn(q64, k64, np.abs(v64), 0.125, causal)[0]
    tq, tk, tv = upload(q, dt), upload(k, dt), upload(v, dt)
    code = fa2.FA2_F16 if dt == "f16" else fa2.FA2_BF16
    need = fa2.workspace_size(B, H, Nq, Nk, 64, causal, code)
    assert (need > 0) == (Nk > 2048), "the shape takes the other schedule"
    for use_ws in (True, False):
        o, lse = fa2.attn_fwd(tq, tk, tv, scale=0.125, causal=causal, return_lse=True,
                              use_workspace=use_ws)
        torch.cuda.synchronize()
        got = download_f64(o)
        tag = "%s ws=%d need=%d" % (dt, use_ws, need)
        assert_close("few-tile schedule %s O" % tag, got, ro, edge_tol(dt, ro, got, wabs))
        assert_close("few-tile schedule %s LSE" % tag, download_f64(lse), rl, LSE_TOL)


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_long_keys_split_at_half_the_slots(dt):
    """200 query tiles of 128 rows (more than a quarter, at most half of the
    768 workgroup slots of 256 compute units) over 8192 keys: the keys are
    split across workgroups when a workspace is given (not with 2048 keys).
    Three heads (first, middle, last) against the oracle, with and without a
    workspace."""
    import torch
    B, H, Nq, Nk = 1, 25, 1024, 8192
    code = fa2.FA2_F16 if dt == "f16" else fa2.FA2_BF16
    need = fa2.workspace_size(B, H, Nq, Nk, 64, False, code)
    assert need > 0 and fa2.workspace_size(B, H, Nq, 2048, 64, False, code) == 0
    q, k, v = seeded(B, H, Nq, Nk, 64, dt, 16)
    tq, tk, tv = upload(q, dt), upload(k, dt), upload(v, dt)
    heads = [0, 12, 24]
    q64, k64, v64 = (inputs.to_f64(x, dt)[:, heads] for x in (q, k, v))
    ro, rl = oracle.attn(q64, k64, v64, 0.125, False)
    wabs = oracle.attn(q64, k64, np.abs(v64), 0.125, False)[0]
    for use_ws in (True, False):
        o, lse = fa2.attn_fwd(tq, tk, tv, scale=0.125, return_lse=True, use_workspace=use_ws)
        torch.cuda.synchronize()
        got = download_f64(o)[:, heads]
        tag = "%s ws=%d" % (dt, use_ws)
        assert_close("half-slot split %s O" % tag, got, ro, edge_tol(dt, ro, got, wabs))
        assert_close("half-slot split %s LSE" % tag, download_f64(lse)[:, heads], rl, LSE_TOL)


# f16/bf16 shapes that run 16-row waves on 16x16x32 MFMAs (64-row tiles, keys
# not split): at D = 64 the 128-row tiles fill at most half of the wave slots
# (three per CU) and the shape is causal or its 64-row tiles fill at least three
# quarters of the slots (256 CUs).  (B, H, Nq, Nk, causal, scale)
Q16_SHAPES = [(4, 12, 1024, 1024, 64, False, 0.125),  # the B4 H12 N1024 workload's shape
              (4, 12, 1024, 1024, 64, True, 0.125),
              (2, 12, 1024, 1024, 64, True, 0.5),      # 384 tiles: half of the slots, causal
              (8, 12, 512, 512, 64, True, 0.125),
              (4, 12, 1000, 1000, 64, False, 0.125),   # ragged rows and keys
              (3, 16, 1000, 1000, 64, True, 0.5),      # ragged, causal, peaky softmax
              (4, 12, 1024, 700, 64, False, 0.125),    # Nq != Nk, ragged keys
              # D = 128, causal, at most 1.5 128-row tiles per CU
              (2, 12, 1024, 1024, 128, True, 0.125),   # 192 tiles
              (4, 12, 512, 512, 128, True, 0.5),
              (1, 16, 2048, 2048, 128, True, 0.088),   # 256 tiles
              (4, 12, 1024, 1024, 128, True, 0.125),   # 384 tiles: 1.5 per CU
              (2, 7, 1000, 1000, 128, True, 0.125)]    # ragged: 112 tiles, 16 key blocks


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("shape", Q16_SHAPES, ids=lambda s: "x".join(map(str, s[:6])))
def test_mfma16_row_waves(shape, dt):
    """Every row against the oracle, with and without LSE (the same O bit for
    bit), and the same bits on a second call."""
    import torch
    B, H, Nq, Nk, D, causal, scale = shape
    code = fa2.FA2_F16 if dt == "f16" else fa2.FA2_BF16
    assert fa2.workspace_size(B, H, Nq, Nk, D, causal, code) == 0, "the shape splits its keys"
    q, k, v = seeded(B, H, Nq, Nk, D, dt, 17)
    o, lse = run_fwd(q, k, v, dt, scale, causal)
    q64, k64, v64 = (inputs.to_f64(x, dt) for x in (q, k, v))
    ro, rl = oracle.attn(q64, k64, v64, scale, causal)
    wabs = oracle.attn(q64, k64, np.abs(v64), scale, causal)[0]
    tag = "16-row waves %s %s" % (dt, "x".join(map(str, shape)))
    assert_close(tag + " O", o, ro, edge_tol(dt, ro, o, wabs))
    assert_close(tag + " LSE", lse, rl, LSE_TOL)
    o2, lse2 = run_fwd(q, k, v, dt, scale, causal)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2), "not deterministic"


# f16/bf16 shapes whose keys are split in exactly two chunks, the pair's
# states merged in the kernel: (B, H, Nq, Nk, D, causal, flat heads checked
# against the oracle, None for all)
PAIR_SHAPES = [(1, 8, 1024, 2500, 64, False, None),  # 64 tiles over 40 key blocks, ragged keys
               (1, 8, 2500, 2500, 64, True, None),   # causal: the early tiles' second chunk
                                                     # holds no visible key for most rows
               (1, 2, 1000, 300, 128, False, None),  # few tiles at D = 128, five key blocks
               (1, 2, 300, 300, 128, True, None),
               (4, 12, 1024, 4096, 64, False, [0, 23, 47]),  # B4 H12 1024 x 4096: three heads
               (1, 8, 1024, 1024, 64, True, None),   # 64 tiles: an eighth of the slots, 16 blocks
               (2, 12, 2048, 2048, 64, True, [0, 11, 23])]  # causal, half of the slots


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("shape", PAIR_SHAPES, ids=lambda s: "x".join(map(str, s[:6])))
def test_mfma_two_chunk_pair_merge(shape, dt):
    """The two workgroups of a tile meet through a handshake word; the second
    to finish merges both states.  The workspace starts out as random bytes
    (the words' earlier contents must not matter), every call must leave the
    words at 0, the same call twice must give the same bits (the merge runs
    in chunk order whichever workgroup does it), a call on other values with
    the same workspace must match the oracle again, and the call without LSE
    must give the same O.  Without a workspace the shape runs unsplit."""
    import torch
    B, H, Nq, Nk, D, causal, heads = shape
    code = fa2.FA2_F16 if dt == "f16" else fa2.FA2_BF16
    tiles = B * H * ((Nq + 127) // 128)
    need = fa2.workspace_size(B, H, Nq, Nk, D, causal, code)
    assert need == (tiles * 8 + 255) // 256 * 256 + tiles * 2 * 128 * (D + 3) * 4, \
        "the shape takes another schedule (need=%d)" % need
    ws = torch.randint(0, 256, (need,), dtype=torch.uint8, device="cuda")
    scale = 1 / np.sqrt(D)
    pick = (lambda x: x) if heads is None else \
        (lambda x: x.reshape((B * H, 1) + x.shape[2:])[heads])
    first = None
    for seed in (41, 41, 42):
        q, k, v = seeded(B, H, Nq, Nk, D, dt, seed)
        q64, k64, v64 = (pick(inputs.to_f64(x, dt)) for x in (q, k, v))
        ro, rl = oracle.attn(q64, k64, v64, scale, causal)
        wabs = oracle.attn(q64, k64, np.abs(v64), scale, causal)[0]
        tq, tk, tv = upload(q, dt), upload(k, dt), upload(v, dt)
        o, lse = fa2.attn_fwd(tq, tk, tv, scale=scale, causal=causal, return_lse=True, workspace=ws)
        torch.cuda.synchronize()
        tag = "pair %s seed %d" % (dt, seed)
        got = pick(download_f64(o))
        assert_close(tag + " O", got, ro, edge_tol(dt, ro, got, wabs))
        assert_close(tag + " LSE", pick(download_f64(lse)), rl, LSE_TOL)
        assert not ws[:8 * tiles].cpu().numpy().any(), "handshake words left set after the call"
        if first is None:
            first = (o.clone(), lse.clone())
        elif seed == 41:
            assert torch.equal(o, first[0]) and torch.equal(lse, first[1]), "not deterministic"
    o_only = fa2.attn_fwd(tq, tk, tv, scale=scale, causal=causal, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(o_only, o), "O differs between the runs with and without LSE"
    o, lse = fa2.attn_fwd(tq, tk, tv, scale=scale, causal=causal, return_lse=True,
                          use_workspace=False)
    torch.cuda.synchronize()
    got = pick(download_f64(o))
    assert_close("pair shape without workspace O", got, ro, edge_tol(dt, ro, got, wabs))
    assert_close("pair shape without workspace LSE", pick(download_f64(lse)), rl, LSE_TOL)


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("shape", [(1, 2, 1024, 1024, True), (1, 1, 700, 700, False),
                                   (1, 3, 129, 2000, True), (2, 1, 300, 300, True)],
                         ids=lambda s: "x".join(map(str, s)))
def test_mfma_few_tile_d128(shape, dt):
    """Few query tiles at D = 128 (these keep the key split across workgroups,
    with a workspace from the binding)."""
    B, H, Nq, Nk, causal = shape
    if causal and Nq != Nk:
        Nk = Nq
    check_full(workloads.Prefill("few tiles D128", B, H, Nq, Nk, 128, dt, 1 / np.sqrt(128), causal,
                                 15), edge=True)


def test_lse_optional_and_stream_order():
    import torch
    q, k, v = seeded(1, 2, 256, 256, 64, "f16", 11)
    tq, tk, tv = upload(q, "f16"), upload(k, "f16"), upload(v, "f16")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        o1 = fa2.attn_fwd(tq, tk, tv, scale=0.125)
    s.synchronize()
    o2, _ = fa2.attn_fwd(tq, tk, tv, scale=0.125, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    assert o1.dtype == torch_dtype("f16")
