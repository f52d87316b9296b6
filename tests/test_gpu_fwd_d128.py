"""GPU parity of attn_fwd with head dimension 128 (f16, bf16 and f32) against
the fp64 oracle, through the C ABI.

Same bars as D = 64: 4e-3 max abs on O for the multi-head N(0,1) shapes, the
format bound of gpu_util.edge_tol for ragged and few-key cases, 1e-4 on the
LSE.  Scale 1/sqrt(128) throughout.
"""
import math

import numpy as np
import pytest

import oracle
from exact_attention_fa2_amd import fa2, inputs, workloads
from gpu_util import LSE_TOL, assert_close, download_f64, edge_tol, seeded, upload
from test_gpu_fwd import check_full, run_fwd

pytestmark = pytest.mark.gpu

D = 128
SCALE = 1.0 / math.sqrt(D)


@pytest.mark.parametrize("dt", ["f16", "bf16", "f32"])
def test_multihead_1024_full(dt):
    check_full(workloads.Prefill("B4 H12 N1024 D128 %s" % dt, 4, 12, 1024, 1024, D, dt, SCALE,
                                 False, 21))


@pytest.mark.parametrize("dt,causal", [("f16", False), ("f16", True), ("bf16", False)])
def test_multihead_2048_sampled(dt, causal):
    cfg = workloads.Prefill("B4 H12 N2048 D128 %s" % dt, 4, 12, 2048, 2048, D, dt, SCALE, causal,
                            22)
    g = np.random.default_rng(3)
    total = cfg.B * cfg.H * cfg.Nq
    rows = np.unique(np.concatenate([np.arange(300, 700), total - 1 - np.arange(256),
                                     g.choice(total, 768, replace=False)]))
    check_full(cfg, rows)


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_causal_one_round_snake_order(dt):
    """B2 H12 N2048 causal D128: 384 tiles within one round of slots (two per
    compute unit at D = 128), dealt to the compute units in a snake."""
    cfg = workloads.Prefill("B2 H12 N2048 D128 causal %s" % dt, 2, 12, 2048, 2048, D, dt, SCALE,
                            True, 26)
    g = np.random.default_rng(5)
    total = cfg.B * cfg.H * cfg.Nq
    rows = np.unique(np.concatenate([np.arange(2048), total - 2048 + np.arange(2048),
                                     g.choice(total, 1024, replace=False)]))
    check_full(cfg, rows, edge=(dt == "bf16"))


RAGGED = [  # (B, H, Nq, Nk, causal)
    (1, 1, 1, 1, False), (1, 1, 1, 1, True), (2, 3, 77, 131, False), (1, 2, 200, 200, True),
    (3, 1, 129, 65, False), (1, 1, 17, 1000, False), (2, 2, 300, 300, True), (1, 1, 64, 1, False),
]


@pytest.mark.parametrize("dt", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("shape", RAGGED, ids=lambda s: "x".join(map(str, s)))
def test_ragged_and_degenerate(shape, dt):
    B, H, Nq, Nk, causal = shape
    check_full(workloads.Prefill("ragged D128", B, H, Nq, Nk, D, dt, SCALE, causal, 23), edge=True)


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("shape", [(1, 2, 4096, 4096, True), (1, 2, 4096, 4096, False),
                                   (1, 3, 2048, 6000, False)],
                         ids=lambda s: "x".join(map(str, s)))
def test_split_schedules(shape, dt):
    """Long keys with few query tiles: keys split across workgroups with a
    workspace (partials of D + 3 floats per row) and merged by the combine, or
    run whole without one; both against the oracle.  (Fewer tiles still run
    the 32-row kernel whose waves split the keys: test_gpu_fwd.py.)"""
    import torch
    B, H, Nq, Nk, causal = shape
    q, k, v = seeded(B, H, Nq, Nk, D, dt, 24)
    q64, k64, v64 = (inputs.to_f64(x, dt) for x in (q, k, v))
    ro, rl = oracle.attn(q64, k64, v64, SCALE, causal)
    wabs = oracle.attn(q64, k64, np.abs(v64), SCALE, causal)[0]
    tq, tk, tv = upload(q, dt), upload(k, dt), upload(v, dt)
    code = fa2.FA2_F16 if dt == "f16" else fa2.FA2_BF16
    assert fa2.workspace_size(B, H, Nq, Nk, D, causal, code) > 0
    for use_ws in (True, False):
        o, lse = fa2.attn_fwd(tq, tk, tv, scale=SCALE, causal=causal, return_lse=True,
                              use_workspace=use_ws)
        torch.cuda.synchronize()
        got = download_f64(o)
        tag = "D128 %s ws=%d" % (dt, use_ws)
        assert_close("split %s O" % tag, got, ro, edge_tol(dt, ro, got, wabs))
        assert_close("split %s LSE" % tag, download_f64(lse), rl, LSE_TOL)


@pytest.mark.parametrize("dt", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("causal", [False, True])
def test_zero_keys_give_mean_of_values(dt, causal):
    """K = 0: every score is 0, so O is the mean of the live V rows (the
    running mean when causal) and LSE = ln(number of live keys)."""
    q, _, v = seeded(1, 1, 256, 256, D, dt, 25)
    k = np.zeros_like(q)
    o, lse = run_fwd(q, k, v, dt, SCALE, causal)
    v64 = inputs.to_f64(v, dt)[0, 0]
    if causal:
        want = np.cumsum(v64, axis=0) / np.arange(1, 257)[:, None]
        want_lse = np.log(np.arange(1, 257))
    else:
        want = np.broadcast_to(v64.mean(axis=0), (256, D))
        want_lse = np.full(256, np.log(256))
    assert_close("D128 K=0 " + dt, o[0, 0], want, edge_tol(dt, want, o[0, 0]))
    assert_close("D128 K=0 LSE " + dt, lse[0, 0], want_lse, LSE_TOL)
    if causal:
        assert np.array_equal(o[0, 0, 0], v64[0])
