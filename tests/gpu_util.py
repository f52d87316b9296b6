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
    if not np.all(over <= 0):
        j = np.unravel_index(int(np.argmax(over)), over.shape)
        tj = float(np.broadcast_to(tol, over.shape)[j])
        raise AssertionError(msg + " > tol: worst excess %.3e at %s (got %.6g want %.6g tol %.3e)"
                             % (float(over[j]), j, got[j], want[j], tj))


def bf16_half_ulp(x):
    """Half the spacing of bfloat16 numbers at |x| (8 significant bits)."""
    a = np.maximum(np.abs(np.asarray(x, dtype=np.float64)), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(a)) - 8)


def edge_tol(dt, ref, got=None, wabs=None):
    """Bound for cases outside the named N(0,1) workloads.

    f32 and f16 keep the plain bar.  bf16 carries two unavoidable roundings
    that the named workloads (flat softmax, |O| < 1) never expose:
      * the output itself: it cannot be closer to the exact value than half a
        bf16 spacing, 3.9e-3 on [1,2) and 7.8e-3 on [2,4), taken at the larger
        of |ref| and |got| (a result may round across a power of two);
      * the weights: P is rounded to bf16 (relative 2^-9) before the P V
        product, and normalising by the sum of the rounded weights moves each
        normalised weight by at most about 2^-8 of itself, so O moves by at
        most 2^-8 * sum_j w_j |V_j| -- ``wabs``, the attention of |V| with the
        same weights, computed by the oracle.  When two large V rows of
        opposite sign nearly cancel, this exceeds 4e-3 while |O| is small.
    """
    if dt != "bf16":
        return TOL[dt]
    mag = np.abs(ref) if got is None else np.maximum(np.abs(ref), np.abs(got))
    tol = TOL[dt] + bf16_half_ulp(mag)
    if wabs is not None:
        tol = tol + 2.0 ** -8 * wabs
    return tol


def seeded(B, H, Nq, Nk, D, dt, seed):
    q, k, v = inputs.qkv((B, H, Nq, D), (B, H, Nk, D), seed, dt)
    return q, k, v
