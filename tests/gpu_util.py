"""Helpers for the GPU parity tests: upload seeded inputs, compare with the oracle."""
import numpy as np

from exact_attention_fa2_amd import inputs

TOL = {"f32": 1e-4, "f16": 4e-3, "bf16": 4e-3}   # max abs error on O
LSE_TOL = 1e-4                                     # max abs error on the f32 LSE


def torch_dtype(dt):
    import torch
    return {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dt]


def upload(a, dt):
    import torch
    if dt == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a))
    return t.cuda()


def download_f64(t):
    import torch
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def report(name, got, want):
    """Max abs error and where it is, plus the pages' secondary metrics."""
    err = np.abs(got - want)
    i = np.unravel_index(int(np.argmax(err)), err.shape)
    rmse = float(np.sqrt(np.mean(err ** 2)))
    rel = float(np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-300))
    msg = "%s: max abs %.3e at %s (got %.6g want %.6g), mean abs %.3e, rmse %.3e, rel L2 %.3e" % (
        name, err[i], i, got[i], want[i], float(err.mean()), rmse, rel)
    print(msg, flush=True)
    return float(err[i]), msg


def assert_close(name, got, want, tol):
    """Max abs error within ``tol`` (a scalar, or an array broadcast against
    the outputs)."""
    e, msg = report(name, got, want)
    over = np.abs(got - want) - tol
    assert np.all(over <= 0), msg + " > tol (worst excess %.3e)" % float(np.max(over))


def bf16_half_ulp(x):
    """Half the spacing of bfloat16 numbers at |x| (8 significant bits)."""
    a = np.maximum(np.abs(np.asarray(x, dtype=np.float64)), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(a)) - 8)


def edge_tol(dt, ref, got=None):
    """Bound for cases outside the named N(0,1) workloads.

    f32 and f16 keep the plain bar.  A bf16 output cannot be closer to an
    exact value than half a bf16 spacing, which is 3.9e-3 on [1,2) and 7.8e-3
    on [2,4) -- at or above the 4e-3 bar -- so for bf16 the bar is 4e-3 of
    arithmetic error on top of that unavoidable rounding of the result.  The
    spacing is taken at the larger of |ref| and |got|, since a result that
    rounds across a power of two takes the spacing of the upper binade."""
    if dt != "bf16":
        return TOL[dt]
    mag = np.abs(ref) if got is None else np.maximum(np.abs(ref), np.abs(got))
    return TOL[dt] + bf16_half_ulp(mag)


def seeded(B, H, Nq, Nk, D, dt, seed):
    q, k, v = inputs.qkv((B, H, Nq, D), (B, H, Nk, D), seed, dt)
    return q, k, v
