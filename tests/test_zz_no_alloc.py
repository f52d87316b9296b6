"""attn_fwd_noalloc (the forward that allocates nothing) against attn_fwd_ws,
through the C ABI.

Two calls in a row on one device share the library's scratch array; the
second, smaller one must not see anything of the first.  Each output is
compared with attn_fwd_ws given a torch workspace on the same inputs (the same
kernels run, so the outputs are equal bit for bit) and with the fp64 oracle at
the bars of the parity tests.  A shape whose workspace would exceed the array
is refused with FA2_ERR_UNSUPPORTED before anything is enqueued.
"""
import numpy as np
import pytest

import oracle
from exact_attention_fa2_amd import fa2, inputs
from gpu_util import LSE_TOL, assert_close, download_f64, edge_tol, upload

pytestmark = pytest.mark.gpu

CODES = {"f32": fa2.FA2_F32, "f16": fa2.FA2_F16, "bf16": fa2.FA2_BF16}


def one_pair(B, H, Nq, Nk, D, dt, causal, seed):
    """attn_fwd_noalloc and attn_fwd_ws on the same inputs; both against the
    oracle, and against each other bit for bit."""
    import torch
    need = fa2.workspace_size(B, H, Nq, Nk, D, causal, CODES[dt])
    assert 0 < need <= fa2.NOALLOC_SCRATCH_BYTES, "the shape must use the scratch array"
    q, k, v = inputs.qkv((B, H, Nq, D), (B, H, Nk, D), seed, dt)
    tq, tk, tv = upload(q, dt), upload(k, dt), upload(v, dt)
    scale = 1.0 / np.sqrt(D)
    o = torch.empty_like(tq)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device="cuda")
    # fill the outputs so that nothing left over can pass for a result
    o.fill_(float("nan"))
    lse.fill_(float("nan"))
    fa2.attn_fwd_noalloc(tq, tk, tv, o, scale=scale, causal=causal, lse=lse)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    o_ws, lse_ws = fa2.attn_fwd(tq, tk, tv, scale=scale, causal=causal, return_lse=True,
                                workspace=ws)
    torch.cuda.synchronize()
    tag = "B%d H%d Nq%d Nk%d D%d %s causal=%d" % (B, H, Nq, Nk, D, dt, causal)
    assert torch.equal(o, o_ws), tag + ": O differs from attn_fwd_ws"
    assert torch.equal(lse, lse_ws), tag + ": LSE differs from attn_fwd_ws"
    q64, k64, v64 = (inputs.to_f64(x, dt) for x in (q, k, v))
    ro, rl = oracle.attn(q64, k64, v64, scale, causal)
    got = download_f64(o)
    wabs = oracle.attn(q64, k64, np.abs(v64), scale, causal)[0]
    assert_close("noalloc " + tag + " O", got, ro, edge_tol(dt, ro, got, wabs))
    assert_close("noalloc " + tag + " LSE", download_f64(lse), rl, LSE_TOL)


@pytest.mark.parametrize("dt", ["f16", "bf16", "f32"])
def test_two_calls_in_a_row_second_smaller(dt):
    # a large split-path shape, then a smaller one on the same scratch array
    if dt == "f32":
        one_pair(1, 3, 1024, 1024, 64, dt, False, 31)
        one_pair(1, 1, 300, 700, 64, dt, False, 32)
    else:
        one_pair(1, 4, 4096, 4096, 64, dt, False, 31)
        one_pair(1, 2, 4096, 4096, 64, dt, True, 32)


def test_f32_tile_split_on_the_scratch_array():
    """The float32 split whose two workgroups per tile meet through handshake
    words: on the scratch array those words first hold whatever an earlier
    call left there (here the partials of a split-and-combine shape), and each
    call must leave them ready for the next one."""
    one_pair(1, 2, 1024, 1024, 64, "f32", False, 35)   # keys split, merged by the combine
    one_pair(1, 1, 4096, 4096, 64, "f32", False, 36)   # 32-row tiles, keys in two chunks
    one_pair(1, 1, 4096, 4096, 64, "f32", False, 37)


def test_f16_pair_merge_on_the_scratch_array():
    """The f16/bf16 split in two chunks, whose workgroups meet through
    handshake words: first a split-and-combine shape leaves its partials in
    the scratch array, then two pair shapes, the second smaller."""
    one_pair(1, 4, 4096, 4096, 64, "f16", False, 38)   # four chunks, the combine kernel
    one_pair(1, 8, 1024, 2500, 64, "f16", False, 39)   # two chunks, merged in the kernel
    one_pair(1, 2, 300, 300, 128, "bf16", True, 40)


def test_d128_split_and_no_split_shapes():
    import torch
    one_pair(1, 2, 4096, 4096, 128, "f16", False, 33)
    # a shape that needs no workspace runs as attn_fwd does
    q, k, v = inputs.qkv((4, 12, 512, 64), (4, 12, 512, 64), 34, "f16")
    tq, tk, tv = upload(q, "f16"), upload(k, "f16"), upload(v, "f16")
    assert fa2.workspace_size(4, 12, 512, 512, 64, False, fa2.FA2_F16) == 0
    o = torch.empty_like(tq)
    fa2.attn_fwd_noalloc(tq, tk, tv, o, scale=0.125)
    o_ref = fa2.attn_fwd(tq, tk, tv, scale=0.125)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref)


def test_workspace_beyond_the_array_is_refused():
    import torch
    B, H, Nq, Nk, D = 1, 4, 4096, 4096, 128
    need = fa2.workspace_size(B, H, Nq, Nk, D, False, fa2.FA2_F16)
    assert need > fa2.NOALLOC_SCRATCH_BYTES
    t = torch.zeros(B, H, Nq, D, device="cuda", dtype=torch.float16)
    kv = torch.zeros(B, H, Nk, D, device="cuda", dtype=torch.float16)
    with pytest.raises(fa2.FA2Error, match="unsupported configuration"):
        fa2.attn_fwd_noalloc(t, kv, kv, torch.empty_like(t))
    # the ABI status, directly
    L = fa2.lib()
    import ctypes
    st = L.attn_fwd_noalloc(ctypes.c_void_p(t.data_ptr()), ctypes.c_void_p(kv.data_ptr()),
                            ctypes.c_void_p(kv.data_ptr()), ctypes.c_void_p(t.data_ptr()), None,
                            B, H, Nq, Nk, D, 0.1, 0, fa2.FA2_F16, None)
    assert st == 3
