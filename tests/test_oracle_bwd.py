"""Pins of the backward oracle (oracle.attn_bwd) that do not use its own
formulas: central finite differences of the forward definition (itself pinned
in test_oracle.py), closed forms, and torch's CPU float64 autograd.  A planted
mistake anywhere in the backward must fail one of them."""
import numpy as np
import pytest

import oracle


def rnd(shape, seed, scale=1.0):
    return scale * np.random.default_rng(seed).standard_normal(shape)


def loss(q, k, v, w, scale, causal, lib=None):
    """L = sum(W o O): its gradient w.r.t. q, k, v is the backward with dO = W."""
    o, _ = oracle.attn(q, k, v, scale, causal, lib=lib)
    return float(np.sum(w * o))


def finite_diff(q, k, v, w, scale, causal, h=1e-6, lib=None):
    grads = []
    for x in (q, k, v):
        g = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            i = it.multi_index
            old = x[i]
            x[i] = old + h
            fp = loss(q, k, v, w, scale, causal, lib)
            x[i] = old - h
            fm = loss(q, k, v, w, scale, causal, lib)
            x[i] = old
            g[i] = (fp - fm) / (2 * h)
        grads.append(g)
    return grads


CASES = [  # (B, H, Nq, Nk, D, causal, scale)
    (1, 2, 5, 6, 3, False, 0.7),
    (1, 1, 6, 6, 4, True, 0.9),
    (2, 1, 3, 7, 2, False, 1.3),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c[:5])) + ("c" if c[5] else ""))
def test_finite_differences(case):
    B, H, Nq, Nk, D, causal, scale = case
    q, k, v = rnd((B, H, Nq, D), 1), rnd((B, H, Nk, D), 2), rnd((B, H, Nk, D), 3)
    w = rnd((B, H, Nq, D), 4)
    dq, dk, dv, delta = oracle.attn_bwd(q, k, v, w, scale, causal)
    fq, fk, fv = finite_diff(q, k, v, w, scale, causal)
    n = B * H
    np.testing.assert_allclose(dq, fq.reshape(n, Nq, D), rtol=0, atol=2e-8)
    np.testing.assert_allclose(dk, fk.reshape(n, Nk, D), rtol=0, atol=2e-8)
    np.testing.assert_allclose(dv, fv.reshape(n, Nk, D), rtol=0, atol=2e-8)
    o, _ = oracle.attn(q, k, v, scale, causal)
    np.testing.assert_allclose(delta, np.sum(w * o, axis=-1).reshape(n, Nq), rtol=0, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_constant_values_give_zero_q_and_k_gradients(causal):
    """Every V row equal: O does not depend on Q or K at all."""
    q, k, w = rnd((1, 2, 7, 4), 5), rnd((1, 2, 7, 4), 6), rnd((1, 2, 7, 4), 7)
    v = np.broadcast_to(rnd((4,), 8), (1, 2, 7, 4)).copy()
    dq, dk, dv, _ = oracle.attn_bwd(q, k, v, w, 0.6, causal)
    assert np.max(np.abs(dq)) < 1e-13 and np.max(np.abs(dk)) < 1e-13
    # dV still collects P^T dO; its rows sum (over keys) to the column sums of dO
    np.testing.assert_allclose(dv.sum(axis=1), w.reshape(2, 7, 4).sum(axis=1), rtol=0, atol=1e-12)


def test_zero_keys_give_mean_of_upstream():
    """K = 0: every weight is 1/Nk, so dV_j = mean_i dO_i for every key j."""
    q, v, w = rnd((1, 1, 5, 3), 9), rnd((1, 1, 8, 3), 10), rnd((1, 1, 5, 3), 11)
    k = np.zeros((1, 1, 8, 3))
    _, _, dv, _ = oracle.attn_bwd(q, k, v, w, 0.5, False)
    np.testing.assert_allclose(dv[0], np.broadcast_to(w[0, 0].sum(axis=0) / 8, (8, 3)), rtol=0,
                               atol=1e-14)


def test_selected_heads_match_all_heads():
    q, k, v, w = rnd((2, 3, 4, 3), 12), rnd((2, 3, 5, 3), 13), rnd((2, 3, 5, 3), 14), rnd((2, 3, 4, 3), 15)
    full = oracle.attn_bwd(q, k, v, w, 0.4, False)
    part = oracle.attn_bwd(q, k, v, w, 0.4, False, heads=[4, 1])
    for a, b in zip(full, part):
        np.testing.assert_array_equal(a[[4, 1]], b)


@pytest.mark.parametrize("causal", [False, True])
def test_torch_cpu_float64_autograd(causal):
    torch = pytest.importorskip("torch")
    B, H, N, D = 2, 2, 33, 8
    q, k, v, w = rnd((B, H, N, D), 16), rnd((B, H, N, D), 17), rnd((B, H, N, D), 18), rnd((B, H, N, D), 19)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    s = torch.matmul(tq, tk.transpose(-1, -2).contiguous()) * 0.3
    if causal:
        s = s.masked_fill(torch.ones(N, N, dtype=torch.bool).triu(1), float("-inf"))
    o = torch.matmul(torch.softmax(s, dim=-1), tv)
    o.backward(torch.tensor(w))
    dq, dk, dv, _ = oracle.attn_bwd(q, k, v, w, 0.3, causal)
    for got, want in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        np.testing.assert_allclose(got, want.numpy().reshape(got.shape), rtol=0, atol=1e-12)


# planted mistakes in the backward; each must make one of the pins above fail
BWD_MUTANTS = [
    ("delta dropped", "P[(size_t)i * Nk + j] *= dp - dlt[i];", "P[(size_t)i * Nk + j] *= dp;"),
    ("dQ scale dropped", "dqh[(size_t)i * D + d] = scale * acc;", "dqh[(size_t)i * D + d] = acc;"),
    ("dK from Q of the wrong row", "for (int i = 0; i < Nq; ++i) acc += P[(size_t)i * Nk + j] * qh[(size_t)i * D + d];",
     "for (int i = 0; i < Nq; ++i) acc += P[(size_t)i * Nk + j] * qh[(size_t)(Nq - 1 - i) * D + d];"),
    ("dV from V instead of dO", "for (int i = 0; i < Nq; ++i) acc += P[(size_t)i * Nk + j] * gh[(size_t)i * D + d];",
     "for (int i = 0; i < Nq; ++i) acc += P[(size_t)i * Nk + j] * vh[(size_t)(i % Nk) * D + d];"),
    ("dP from K instead of V", "for (int d = 0; d < D; ++d) dp += gh[(size_t)i * D + d] * vh[(size_t)j * D + d];",
     "for (int d = 0; d < D; ++d) dp += gh[(size_t)i * D + d] * kh[(size_t)j * D + d];"),
    ("causal ignored in P", "const int nlive = causal ? i + 1 : Nk;\n                double *pr",
     "const int nlive = Nk;\n                double *pr"),
    ("softmax not normalised", "for (int j = 0; j < nlive; ++j) pr[j] /= z;", ""),
]


def _bwd_pins_pass(lib):
    try:
        for case in CASES[:2]:
            B, H, Nq, Nk, D, causal, scale = case
            q, k, v = rnd((B, H, Nq, D), 1), rnd((B, H, Nk, D), 2), rnd((B, H, Nk, D), 3)
            w = rnd((B, H, Nq, D), 4)
            dq, dk, dv, _ = oracle.attn_bwd(q, k, v, w, scale, causal, lib=lib)
            fq, fk, fv = finite_diff(q, k, v, w, scale, causal)  # the clean forward
            n = B * H
            for got, want in ((dq, fq.reshape(n, Nq, D)), (dk, fk.reshape(n, Nk, D)),
                              (dv, fv.reshape(n, Nk, D))):
                if not np.allclose(got, want, rtol=0, atol=2e-8):
                    return False
    except ValueError:
        return False
    return True


def test_backward_pins_catch_planted_mistakes(tmp_path):
    src = oracle.source_text()
    clean = oracle.compile_variant(src, str(tmp_path / "clean.so"))
    assert _bwd_pins_pass(clean.lib)
    for idx, (name, old, new) in enumerate(BWD_MUTANTS):
        assert src.count(old) == 1, name
        mut = oracle.compile_variant(src.replace(old, new), str(tmp_path / ("b%d.so" % idx)))
        assert not _bwd_pins_pass(mut.lib), "pins missed the planted mistake: " + name
