"""Pins for the fp64 oracle, independent of the oracle itself (CPU only).

Each pin comes from the pages or from mathematics, not from re-typing the
oracle's formula: a brute force without max subtraction, closed forms, exact
special cases, invariants the pages state (streaming equals batch for any
tile size, the (m, l) monoid, split-then-combine equals unsplit), hand-derived
golden cases and a library routine (torch CPU float64).  The mutation test at
the end plants plausible mistakes in copies of oracle.c and checks that these
pins catch every one of them.
"""
import math
import os

import numpy as np
import pytest

import oracle
from oracle import brute, recurrence
from exact_attention_fa2_amd import inputs


def rnd(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def as_lists(a):
    return [list(map(float, r)) for r in a]


# ---------------------------------------------------------------- golden cases

def test_golden_attention(golden):
    for case in golden["attention"]:
        q = np.array(case["q"])[None, None]
        k = np.array(case["k"])[None, None]
        v = np.array(case["v"])[None, None]
        o, lse = oracle.attn(q, k, v, case["scale"], case["causal"])
        np.testing.assert_allclose(o[0, 0], np.array(case["o"]), rtol=0, atol=1e-14,
                                   err_msg=case["name"])
        np.testing.assert_allclose(lse[0, 0], np.array(case["lse"]), rtol=0, atol=1e-14,
                                   err_msg=case["name"])


def test_golden_decode(golden):
    for case in golden["decode"]:
        q = np.array(case["q"])[None, None]
        k = np.array(case["k"])[None, None]
        v = np.array(case["v"])[None, None]
        for ns, want in case["splits"].items():
            op, mp, lp = oracle.decode_split(q, k, v, case["scale"], int(ns))
            wm = np.array([float(x) for x in want["m"]])
            np.testing.assert_array_equal(np.isinf(mp[0, 0]), np.isinf(wm))
            fin = np.isfinite(wm)
            np.testing.assert_allclose(mp[0, 0][fin], wm[fin], atol=1e-14, rtol=0)
            np.testing.assert_allclose(lp[0, 0], want["l"], atol=1e-14, rtol=0)
            np.testing.assert_allclose(op[0, 0], want["o"], atol=1e-14, rtol=0)
            o = oracle.decode_combine(op, mp, lp)
            np.testing.assert_allclose(o[0, 0], case["o"], atol=1e-14, rtol=0)


# ------------------------------------------------------------ brute force pin

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("seed", range(6))
def test_brute_force(seed, causal):
    g = np.random.default_rng(100 + seed)
    nq = int(g.integers(1, 9))
    nk = nq if causal else int(g.integers(1, 9))
    d = int(g.integers(1, 5))
    q, k, v = rnd((nq, d), seed), rnd((nk, d), seed + 50), rnd((nk, d), seed + 99)
    scale = float(g.uniform(0.2, 1.5))
    bo, bl = brute.attention(as_lists(q), as_lists(k), as_lists(v), scale, causal)
    o, lse = oracle.attn(q[None, None], k[None, None], v[None, None], scale, causal)
    np.testing.assert_allclose(o[0, 0], np.array(bo), rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(lse[0, 0], np.array(bl), rtol=1e-13, atol=1e-13)


def test_brute_force_multihead_layout():
    """Row ids walk (b, h, i) in that order; heads never mix."""
    B, H, nq, nk, d = 2, 3, 4, 5, 3
    q, k, v = rnd((B, H, nq, d), 1), rnd((B, H, nk, d), 2), rnd((B, H, nk, d), 3)
    o, lse = oracle.attn(q, k, v, 0.7, False)
    for b in range(B):
        for h in range(H):
            bo, bl = brute.attention(as_lists(q[b, h]), as_lists(k[b, h]), as_lists(v[b, h]), 0.7)
            np.testing.assert_allclose(o[b, h], bo, rtol=1e-13, atol=1e-13)
            np.testing.assert_allclose(lse[b, h], bl, rtol=1e-13, atol=1e-13)
    rows = np.array([0, 7, 23, B * H * nq - 1])
    so, sl = oracle.attn_rows(q, k, v, 0.7, False, rows)
    np.testing.assert_array_equal(so, o.reshape(-1, d)[rows])
    np.testing.assert_array_equal(sl, lse.reshape(-1)[rows])


# --------------------------------------------------------------- closed forms

@pytest.mark.parametrize("causal", [False, True])
def test_identity_values_rows_sum_to_one(causal):
    """V = I with Nk = D: O is the probability matrix itself, so each row is a
    distribution ("softmax rows sum to 1")."""
    n = 24
    q, k = rnd((n, n), 5), rnd((n, n), 6)
    o, _ = oracle.attn(q[None, None], k[None, None], np.eye(n)[None, None], 0.4, causal)
    o = o[0, 0]
    np.testing.assert_allclose(o.sum(axis=1), 1.0, rtol=0, atol=1e-14)
    assert (o >= 0).all()
    if causal:
        assert np.all(np.triu(o, 1) == 0.0)
    bo, _ = brute.attention(as_lists(q), as_lists(k), as_lists(np.eye(n)), 0.4, causal)
    np.testing.assert_allclose(o, bo, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_zero_keys_give_mean_of_values(causal):
    """K = 0 makes every score 0: uniform weights, O = mean of the live V rows,
    LSE = ln(number of live keys)."""
    n, d = 37, 8
    q, v = rnd((n, d), 7), rnd((n, d), 8)
    o, lse = oracle.attn(q[None, None], np.zeros((1, 1, n, d)), v[None, None], 0.9, causal)
    if causal:
        want = np.cumsum(v, axis=0) / np.arange(1, n + 1)[:, None]
        want_lse = np.log(np.arange(1, n + 1))
    else:
        want = np.broadcast_to(v.mean(axis=0), (n, d))
        want_lse = np.full(n, math.log(n))
    np.testing.assert_allclose(o[0, 0], want, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse[0, 0], want_lse, rtol=0, atol=1e-13)


def test_single_key_and_causal_row_zero():
    """One live key has weight 1: O = V_0 and LSE = s_00."""
    d = 16
    q, k, v = rnd((5, d), 9), rnd((1, d), 10), rnd((1, d), 11)
    o, lse = oracle.attn(q[None, None], k[None, None], v[None, None], 0.3, False)
    np.testing.assert_allclose(o[0, 0], np.broadcast_to(v[0], (5, d)), atol=1e-15, rtol=0)
    np.testing.assert_allclose(lse[0, 0], 0.3 * (q @ k[0]), atol=1e-14, rtol=0)
    q, k, v = rnd((9, d), 12), rnd((9, d), 13), rnd((9, d), 14)
    o, lse = oracle.attn(q[None, None], k[None, None], v[None, None], 0.3, True)
    np.testing.assert_allclose(o[0, 0, 0], v[0], atol=1e-15, rtol=0)
    assert abs(lse[0, 0, 0] - 0.3 * float(q[0] @ k[0])) < 1e-14


# ----------------------------------------------------------------- invariants

@pytest.mark.parametrize("shift", [512.0, 2048.0, 8192.0])
def test_shift_invariance_far_past_overflow(shift):
    """Adding one vector u to every key shifts row i's scores by scale*q_i.u.
    O must not move and LSE moves by exactly that amount.  Shifts put raw
    scores in the hundreds to thousands, far past exp's overflow (about 88 in
    f32, 709 in f64), so this also pins the max subtraction.  Keys are f16
    values so K + u is exact in fp64."""
    d, n = 64, 50
    q = inputs.to_f64(inputs.normal((1, 1, 7, d), 3, 0, "f16"), "f16")
    k = inputs.to_f64(inputs.normal((1, 1, n, d), 3, 1, "f16"), "f16")
    v = inputs.to_f64(inputs.normal((1, 1, n, d), 3, 2, "f16"), "f16")
    u = np.zeros(d)
    u[:4] = shift
    scale = 1.0 / 8.0
    o0, l0 = oracle.attn(q, k, v, scale)
    o1, l1 = oracle.attn(q, k + u, v, scale)
    assert np.max(np.abs(scale * (q[0, 0] @ (k[0, 0] + u).T))) > 100
    np.testing.assert_allclose(o1, o0, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l1[0, 0] - l0[0, 0], scale * (q[0, 0] @ u), rtol=1e-12, atol=1e-9)


def test_key_permutation_invariance():
    n, d = 41, 12
    q, k, v = rnd((1, 2, 6, d), 20), rnd((1, 2, n, d), 21), rnd((1, 2, n, d), 22)
    perm = np.random.default_rng(3).permutation(n)
    o0, l0 = oracle.attn(q, k, v, 0.5)
    o1, l1 = oracle.attn(q, k[:, :, perm], v[:, :, perm], 0.5)
    np.testing.assert_allclose(o1, o0, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l1, l0, rtol=0, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_convex_hull_and_lse_bounds(causal):
    """O_i is a convex combination of the live value rows; LSE lies between the
    row max and the row max + ln(#live) ("Flash Attention": 1 <= l <= j)."""
    n, d = 33, 10
    q, k, v = rnd((n, d), 30, 2.0), rnd((n, d), 31), rnd((n, d), 32)
    o, lse = oracle.attn(q[None, None], k[None, None], v[None, None], 0.6, causal)
    s = 0.6 * q @ k.T
    for i in range(n):
        live = slice(0, i + 1) if causal else slice(0, n)
        assert np.all(o[0, 0, i] >= v[live].min(axis=0) - 1e-13)
        assert np.all(o[0, 0, i] <= v[live].max(axis=0) + 1e-13)
        mx = s[i, live].max()
        cnt = (i + 1) if causal else n
        assert mx - 1e-13 <= lse[0, 0, i] <= mx + math.log(cnt) + 1e-13


@pytest.mark.parametrize("causal", [False, True])
def test_tiled_recurrence_equals_batched(causal):
    """"Flash Attention", Deriving the online softmax: the m/l/O recurrence
    reaches the batched softmax exactly, for any tile sizes."""
    n, d = 45, 16
    q, k, v = rnd((n, d), 40), rnd((n, d), 41), rnd((n, d), 42)
    o_ref, l_ref = oracle.attn(q[None, None], k[None, None], v[None, None], 0.35, causal)
    for br in (1, 3, 16, n):
        for bc in (1, 2, 3, 5, 8, n):
            o, lse = recurrence.tiled_forward(q, k, v, 0.35, causal, br, bc)
            np.testing.assert_allclose(o, o_ref[0, 0], rtol=0, atol=1e-12)
            np.testing.assert_allclose(lse, l_ref[0, 0], rtol=0, atol=1e-12)


def test_monoid_merge_any_grouping():
    """"Flash Attention": (m, l) is a commutative monoid with identity
    (-inf, 0); with O carried alongside, any partition of the keys merged in
    any order and grouping gives the full row."""
    g = np.random.default_rng(7)
    n, d = 60, 6
    q, k, v = rnd((1, d), 50), rnd((n, d), 51), rnd((n, d), 52)
    o_ref, l_ref = oracle.attn(q[None, None], k[None, None], v[None, None], 0.8)
    s = 0.8 * (k @ q[0])
    for _ in range(20):
        cuts = np.sort(g.choice(np.arange(1, n), size=int(g.integers(1, 12)), replace=False))
        groups = np.split(np.arange(n), cuts)
        parts = [recurrence.partial_state(s[ix], v[ix]) for ix in groups]
        parts.append((-np.inf, 0.0, np.zeros(d)))  # the identity
        g.shuffle(parts)
        while len(parts) > 1:
            i = int(g.integers(0, len(parts) - 1))
            parts[i:i + 2] = [recurrence.merge(parts[i], parts[i + 1])]
        m, l, acc = parts[0]
        np.testing.assert_allclose(acc / l, o_ref[0, 0, 0], rtol=0, atol=1e-13)
        assert abs(m + math.log(l) - l_ref[0, 0, 0]) < 1e-13


@pytest.mark.parametrize("n", [1, 2, 7, 64, 129])
def test_split_then_combine_equals_unsplit(n):
    """"Flash decoding": the combine of the split partials is the unsplit
    attention for every split count, including counts that leave empty
    splits (n_splits = N + 3)."""
    B, H, d = 2, 3, 8
    q, k, v = rnd((B, H, d), 60), rnd((B, H, n, d), 61), rnd((B, H, n, d), 62)
    o_ref, _ = oracle.attn(q[:, :, None], k, v, 0.5)
    for ns in sorted({1, 2, 3, 7, n, n + 3}):
        op, mp, lp = oracle.decode_split(q, k, v, 0.5, ns)
        S = -(-n // ns)
        empty = np.arange(ns) * S >= n
        assert np.all(np.isneginf(mp[..., empty])) and np.all(lp[..., empty] == 0)
        assert np.all(op[..., empty, :] == 0)
        assert np.all(lp[..., ~empty] >= 1.0)
        o = oracle.decode_combine(op, mp, lp)
        np.testing.assert_allclose(o, o_ref[:, :, 0], rtol=0, atol=1e-13)


def test_split_partials_match_brute_force():
    """Each split's (m, l, O) from its definition, by brute force."""
    n, d, ns = 11, 3, 4
    q, k, v = rnd((1, 1, d), 70), rnd((1, 1, n, d), 71), rnd((1, 1, n, d), 72)
    op, mp, lp = oracle.decode_split(q, k, v, 0.9, ns)
    S = -(-n // ns)
    for s in range(ns):
        ix = range(s * S, min(n, s * S + S))
        sc = [0.9 * math.fsum(q[0, 0, t] * k[0, 0, j, t] for t in range(d)) for j in ix]
        m = max(sc)
        w = [math.exp(x - m) for x in sc]
        assert abs(mp[0, 0, s] - m) < 1e-14
        assert abs(lp[0, 0, s] - math.fsum(w)) < 1e-14
        for t in range(d):
            want = math.fsum(wi * v[0, 0, j, t] for wi, j in zip(w, ix))
            assert abs(op[0, 0, s, t] - want) < 1e-13


# ------------------------------------------------------- library cross-check

@pytest.mark.parametrize("causal", [False, True])
def test_torch_cpu_float64_cross_check(causal):
    torch = pytest.importorskip("torch")
    B, H, n, d = 2, 3, 40, 16
    nk = n if causal else 37
    q, k, v = rnd((B, H, n, d), 80), rnd((B, H, nk, d), 81), rnd((B, H, nk, d), 82)
    o, _ = oracle.attn(q, k, v, 0.25, causal)
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    s = torch.matmul(tq, tk.transpose(-1, -2).contiguous()) * 0.25
    if causal:
        mask = torch.ones(n, nk, dtype=torch.bool).tril()
        s = s.masked_fill(~mask, float("-inf"))
    want = torch.matmul(torch.softmax(s, dim=-1), tv).numpy()
    np.testing.assert_allclose(o, want, rtol=0, atol=1e-13)
    lse = torch.logsumexp(s, dim=-1).numpy()
    _, got_lse = oracle.attn(q, k, v, 0.25, causal)
    np.testing.assert_allclose(got_lse, lse, rtol=0, atol=1e-13)


# --------------------------------------------------------- mutation coverage

MUTANTS = [
    ("dropped scale", "s[j] = scale * acc;", "s[j] = acc;"),
    ("transposed K index", "acc += qrow[d] * kh[(size_t)j * D + d];",
     "acc += qrow[d] * kh[(size_t)d * D + j];"),
    ("wrong max sign", "s[j] = exp(s[j] - mx);", "s[j] = exp(s[j] + mx);"),
    ("missing normalisation", "for (int d = 0; d < D; ++d) orow[d] /= z;", ""),
    ("LSE without max", "if (lse) *lse = mx + log(z);", "if (lse) *lse = log(z);"),
    ("causal off by one", "const int nlive = causal ? i + 1 : Nk;\n            one_row(",
     "const int nlive = causal ? i : Nk;\n            one_row("),
    ("causal ignored", "const int nlive = causal ? i + 1 : Nk;\n            one_row(",
     "const int nlive = Nk;\n            one_row("),
    ("V row index", "const double *vr = vh + (size_t)j * D;",
     "const double *vr = vh + (size_t)(Nk - 1 - j) * D;"),
    ("split size floor", "const long long S = ((long long)N + n_splits - 1) / n_splits;",
     "const long long S = (long long)N / n_splits + (N % n_splits > 1);"),
    ("split scale dropped", "s[j - n0] = scale * acc;", "s[j - n0] = acc;"),
    ("combine weight sign", "if (mp[sp] != -INFINITY) lg += exp(mp[sp] - mg) * lp[sp];",
     "if (mp[sp] != -INFINITY) lg += exp(mg - mp[sp]) * lp[sp];"),
    ("combine unweighted O",
     "a += exp(mp[sp] - mg) * o_part[((size_t)bh * n_splits + sp) * D + d];",
     "a += o_part[((size_t)bh * n_splits + sp) * D + d];"),
]


def _pins_pass(lib, golden):
    """A compact run of the pins above against one oracle build."""
    try:
        for case in golden["attention"]:
            q = np.array(case["q"])[None, None]
            k = np.array(case["k"])[None, None]
            v = np.array(case["v"])[None, None]
            o, lse = oracle.attn(q, k, v, case["scale"], case["causal"], lib=lib)
            if not (np.allclose(o[0, 0], case["o"], atol=1e-12) and
                    np.allclose(lse[0, 0], case["lse"], atol=1e-12)):
                return False
        for causal in (False, True):
            for seed in range(3):
                nq, nk, d = 6, 6 if causal else 5, 3
                q, k, v = rnd((nq, d), seed), rnd((nk, d), seed + 9), rnd((nk, d), seed + 19)
                bo, bl = brute.attention(as_lists(q), as_lists(k), as_lists(v), 0.7, causal)
                o, lse = oracle.attn(q[None, None], k[None, None], v[None, None], 0.7, causal,
                                     lib=lib)
                if not (np.allclose(o[0, 0], bo, atol=1e-12) and np.allclose(lse[0, 0], bl,
                                                                             atol=1e-12)):
                    return False
        for case in golden["decode"]:
            q = np.array(case["q"])[None, None]
            k = np.array(case["k"])[None, None]
            v = np.array(case["v"])[None, None]
            for ns, want in case["splits"].items():
                op, mp, lp = oracle.decode_split(q, k, v, case["scale"], int(ns), lib=lib)
                wm = np.array([float(x) for x in want["m"]])
                if not (np.array_equal(np.isinf(mp[0, 0]), np.isinf(wm)) and
                        np.allclose(lp[0, 0], want["l"], atol=1e-12) and
                        np.allclose(op[0, 0], want["o"], atol=1e-12)):
                    return False
                o = oracle.decode_combine(op, mp, lp, lib=lib)
                if not np.allclose(o[0, 0], case["o"], atol=1e-12):
                    return False
        n = 29
        q, k, v = rnd((1, 1, 4), 90), rnd((1, 1, n, 4), 91), rnd((1, 1, n, 4), 92)
        o_ref, _ = oracle.attn(q[:, :, None], k, v, 0.5, lib=lib)
        for ns in (3, 7):
            op, mp, lp = oracle.decode_split(q, k, v, 0.5, ns, lib=lib)
            if not np.allclose(oracle.decode_combine(op, mp, lp, lib=lib), o_ref[:, :, 0],
                               atol=1e-12):
                return False
    except ValueError:
        return False
    return True


def test_pins_catch_planted_mistakes(tmp_path, golden):
    src = oracle.source_text()
    clean = oracle.compile_variant(src, str(tmp_path / "clean.so"))
    assert _pins_pass(clean.lib, golden)
    for name, old, new in MUTANTS:
        assert src.count(old) == 1, name
        mut = oracle.compile_variant(src.replace(old, new),
                                     str(tmp_path / ("m%d.so" % MUTANTS.index((name, old, new)))))
        assert not _pins_pass(mut.lib, golden), "pins missed the planted mistake: " + name
