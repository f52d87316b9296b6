"""The f16/bf16 forward built with the polynomial exp2 of the FlashAttention-4
section ("Flash Attention", section FlashAttention 4) for 2 of every 8
exponential pairs (exact_attention_fa2_amd/libfa2_polyexp.so, a measurement
build made by the same build step) against the fp64 oracle, through the C ABI,
at the bars of the product build: the named multi-head and causal workloads in
full, and the key-split, ragged, head-dimension-128 and large-score cases."""
import numpy as np
import pytest

import oracle
from exact_attention_fa2_amd import fa2, inputs, workloads
from gpu_util import LSE_TOL, TOL, assert_close, download_f64, edge_tol, seeded, upload
from test_gpu_fwd import check_full

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def polyexp_build(monkeypatch):
    monkeypatch.setattr(fa2, "_lib", fa2.load(fa2.POLYEXP_LIB_PATH))
    yield


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_multihead_2048_full(dt):
    check_full(workloads.multihead(2048, dt))


@pytest.mark.parametrize("causal", [True, False])
def test_causal_lse_f16(causal):
    check_full(workloads.causal_lse(causal))


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("shape", [(2, 3, 77, 131, False), (1, 2, 200, 200, True),
                                   (1, 1, 64, 4096, False), (1, 4, 129, 129, True)],
                         ids=lambda s: "x".join(map(str, s)))
def test_ragged_and_split(shape, dt):
    B, H, Nq, Nk, causal = shape
    check_full(workloads.Prefill("poly ragged", B, H, Nq, Nk, 64, dt, 0.125, causal, 3), edge=True)


def test_d128():
    check_full(workloads.Prefill("poly D128", 2, 3, 300, 300, 128, "f16", 1 / np.sqrt(128), False,
                                 5))


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_large_scores(dt):
    """Scores far from zero: exponents well past the polynomial's reduced
    range on both sides (and masked keys at -inf)."""
    import torch
    q, k, v = seeded(1, 2, 190, 190, 64, dt, 9)
    k64 = inputs.to_f64(k, dt)
    k64[..., :4] += 64.0
    k32 = k64.astype(np.float32)
    k2 = inputs.f32_to_bf16_bits(k32) if dt == "bf16" else k32.astype(inputs.storage_numpy_dtype(dt))
    tq, tk, tv = upload(q, dt), upload(k2, dt), upload(v, dt)
    o, lse = fa2.attn_fwd(tq, tk, tv, scale=0.5, causal=True, return_lse=True)
    torch.cuda.synchronize()
    q64, kk, v64 = inputs.to_f64(q, dt), inputs.to_f64(k2, dt), inputs.to_f64(v, dt)
    ro, rl = oracle.attn(q64, kk, v64, 0.5, True)
    wabs = oracle.attn(q64, kk, np.abs(v64), 0.5, True)[0]
    got = download_f64(o)
    assert np.all(np.isfinite(got))
    assert_close("poly shift O " + dt, got, ro, edge_tol(dt, ro, got, wabs))
    assert_close("poly shift LSE " + dt, download_f64(lse), rl, LSE_TOL)
