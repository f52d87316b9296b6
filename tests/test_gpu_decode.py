"""GPU parity of attn_decode_split / attn_decode_combine against the fp64
oracle, through the C ABI.

The final O is compared with the UNSPLIT oracle (tolerance 4e-3 for f16/bf16,
1e-4 for f32); the partials are compared with the oracle's own partials:
m_s within 1e-4*max(1,|m_s|), l_s within 1e-4 relative, O_s/l_s within the
I/O tolerance.
"""
import numpy as np
import pytest

import oracle
from exact_attention_fa2_amd import fa2, inputs, workloads
from gpu_util import TOL, assert_close, download_f64, upload

pytestmark = pytest.mark.gpu


def check_partials(name, op, mp, lp, rop, rmp, rlp, tol):
    fin = np.isfinite(rmp)
    assert np.array_equal(np.isfinite(mp), fin), name + ": empty splits differ"
    assert np.all(lp[~fin] == 0) and np.all(op[~fin] == 0)
    assert np.all(np.abs(mp[fin] - rmp[fin]) <= 1e-4 * np.maximum(1.0, np.abs(rmp[fin]))), name
    assert np.all(np.abs(lp[fin] - rlp[fin]) <= 1e-4 * rlp[fin]), name
    assert_close(name + " O_s/l_s", op[fin] / lp[fin][..., None], rop[fin] / rlp[fin][..., None],
                 tol)


def run(B, H, N, D, dt, n_splits, seed=0, scale=None):
    import torch
    q = inputs.normal((B, H, D), seed, 0, dt)
    k = inputs.normal((B, H, N, D), seed, 1, dt)
    v = inputs.normal((B, H, N, D), seed, 2, dt)
    scale = scale if scale is not None else 1.0 / np.sqrt(D)
    tq, tk, tv = upload(q, dt), upload(k, dt), upload(v, dt)
    op, mp, lp = fa2.attn_decode_split(tq, tk, tv, scale, n_splits)
    o = fa2.attn_decode_combine(op, mp, lp, dtype=tq.dtype)
    torch.cuda.synchronize()
    return (q, k, v, scale), download_f64(o), download_f64(op), download_f64(mp), download_f64(lp)


@pytest.mark.parametrize("dt", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("N", [1, 37, 1000, 4099])
def test_small_decode_all_split_counts(N, D, dt):
    B, H = 2, 3
    for ns in sorted({1, 2, 3, 7, 16, 64, 128}):
        (q, k, v, scale), o, op, mp, lp = run(B, H, N, D, dt, ns, seed=N + D)
        q64, k64, v64 = (inputs.to_f64(x, dt) for x in (q, k, v))
        ro, _ = oracle.attn(q64[:, :, None], k64, v64, scale)
        assert_close("decode N%d D%d %s splits %d" % (N, D, dt, ns), o, ro[:, :, 0], TOL[dt])
        rop, rmp, rlp = oracle.decode_split(q64, k64, v64, scale, ns)
        check_partials("partials N%d ns%d" % (N, ns), op, mp, lp, rop, rmp, rlp, TOL[dt])


def test_default_split_count_runs():
    import torch
    q = upload(inputs.normal((2, 2, 128), 1, 0, "f16"), "f16")
    k = upload(inputs.normal((2, 2, 5000, 128), 1, 1, "f16"), "f16")
    v = upload(inputs.normal((2, 2, 5000, 128), 1, 2, "f16"), "f16")
    ns = fa2.default_splits(2, 2, 5000, 128)
    assert ns >= 1
    o = fa2.attn_decode(q, k, v)
    torch.cuda.synchronize()
    ro, _ = oracle.attn(inputs.to_f64(q.cpu().numpy(), "f16")[:, :, None],
                        inputs.to_f64(k.cpu().numpy(), "f16"), inputs.to_f64(v.cpu().numpy(), "f16"),
                        1 / np.sqrt(128))
    assert_close("default splits", download_f64(o), ro[:, :, 0], TOL["f16"])


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_full_size_decode_all_heads(dt):
    """The full workload (batch 8, 32 heads, KV 32768, D 128) at the split
    count the bench uses: the final O of all 256 (b,h) pairs against the
    unsplit oracle and every partial against the oracle's partials, one (b,h)
    per task on a pool of host threads (each promotes only its own slice)."""
    import concurrent.futures as cf

    import torch
    cfg = workloads.decode(dt)
    B, H, N, D = cfg.B, cfg.H, cfg.N, cfg.D
    q = inputs.normal((B, H, D), cfg.seed, 0, dt)
    k = inputs.normal((B, H, N, D), cfg.seed, 1, dt)
    v = inputs.normal((B, H, N, D), cfg.seed, 2, dt)
    ns = fa2.default_splits(B, H, N, D)
    tq, tk, tv = upload(q, dt), upload(k, dt), upload(v, dt)
    op, mp, lp = fa2.attn_decode_split(tq, tk, tv, cfg.scale, ns)
    o = fa2.attn_decode_combine(op, mp, lp, dtype=tq.dtype)
    torch.cuda.synchronize()
    o = download_f64(o)
    op, mp, lp = download_f64(op), download_f64(mp), download_f64(lp)
    del tk, tv
    torch.cuda.empty_cache()
    assert np.all(np.isfinite(o))
    ro = np.empty_like(o)
    rop, rmp, rlp = np.empty_like(op), np.empty_like(mp), np.empty_like(lp)

    def one(bh):
        b, h = divmod(bh, H)
        sl = (slice(b, b + 1), slice(h, h + 1))
        q64, k64, v64 = (inputs.to_f64(x[sl], dt) for x in (q, k, v))
        ro[b, h] = oracle.attn(q64[:, :, None], k64, v64, cfg.scale, nthreads=1)[0][0, 0, 0]
        a, m_, l_ = oracle.decode_split(q64, k64, v64, cfg.scale, ns)
        rop[b, h], rmp[b, h], rlp[b, h] = a[0, 0], m_[0, 0], l_[0, 0]

    with cf.ThreadPoolExecutor(max_workers=16) as ex:
        list(ex.map(one, range(B * H)))
    assert_close("full decode %s, all %d heads" % (dt, B * H), o, ro, TOL[dt])
    check_partials("full partials %s" % dt, op, mp, lp, rop, rmp, rlp, TOL[dt])


def test_decode_deterministic():
    import torch
    q = upload(inputs.normal((4, 4, 128), 3, 0, "bf16"), "bf16")
    k = upload(inputs.normal((4, 4, 3000, 128), 3, 1, "bf16"), "bf16")
    v = upload(inputs.normal((4, 4, 3000, 128), 3, 2, "bf16"), "bf16")
    a = fa2.attn_decode(q, k, v, n_splits=7)
    b = fa2.attn_decode(q, k, v, n_splits=7)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
