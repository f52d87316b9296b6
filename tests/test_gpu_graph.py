"""The library's launches under HIP graph capture (torch.cuda.graph), the way a
serving loop replays a fixed-shape step: the library enqueues kernels only
(no allocation, memset or synchronisation of its own), so a captured call
replays correctly.

Each case captures one call on static buffers and replays it three times.
Before every replay the inputs are refilled in place with new values and the
outputs are overwritten with NaN (eager work between the replays, then a
synchronisation); after it, every output must equal, bit for bit, an eager
call on the same inputs (all kernels are deterministic)."""
import pytest

from exact_attention_fa2_amd import fa2

pytestmark = pytest.mark.gpu


def _fill(tensors, seed):
    import torch
    g = torch.Generator(device="cuda").manual_seed(seed)
    for t in tensors:
        t.copy_(torch.randn(t.shape, device="cuda", generator=g).to(t.dtype))


def _check_replays(name, refill, call):
    import torch
    torch.cuda.synchronize()
    # warm-up on a side stream, as torch recommends before a capture
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()
    torch.cuda.current_stream().wait_stream(s)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        outs = call()
    for rep in range(3):
        print("%s replay %d" % (name, rep), flush=True)
        refill(100 + rep)
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        want = call()
        torch.cuda.synchronize()
        for i, (got, ref) in enumerate(zip(outs, want)):
            assert torch.equal(got, ref), "%s replay %d output %d" % (name, rep, i)


@pytest.mark.parametrize("dt,D,causal,N,H", [("f16", 64, True, 1024, 2), ("bf16", 128, False, 700, 2),
                                             ("f32", 64, False, 4096, 1), ("f32", 128, True, 512, 2),
                                             ("bf16", 64, True, 4096, 2), ("f16", 64, True, 1024, 8)])
def test_forward_graph(dt, D, causal, N, H):
    """attn_fwd with the LSE; the f16 causal case with two heads (16 query
    tiles of 128 rows) runs the 32-row keys-across-waves kernel, the bf16
    N4096 case the key split across workgroups with its workspace and combine
    kernel, and the f16 case with eight heads (64 tiles) the split in two
    merged in the kernel, whose handshake tag is drawn once, at capture, and
    replayed."""
    import torch
    from gpu_util import torch_dtype
    B = 1
    q, k, v = (torch.empty(B, H, N, D, device="cuda", dtype=torch_dtype(dt)) for _ in range(3))
    _fill((q, k, v), 1)
    ws = torch.empty(max(1, fa2.workspace_size(B, H, N, N, D, causal, fa2.dtype_code(q))),
                     dtype=torch.uint8, device="cuda")
    call = lambda: fa2.attn_fwd(q, k, v, scale=D ** -0.5, causal=causal, return_lse=True,  # noqa: E731
                                workspace=ws)
    _check_replays("fwd %s D%d N%d" % (dt, D, N), lambda seed: _fill((q, k, v), seed), call)


@pytest.mark.parametrize("dt", ["f16", "bf16", "f32"])
def test_decode_graph(dt):
    """flash-decoding: split then combine, both in the graph."""
    import torch
    from gpu_util import torch_dtype
    B, H, N, D = 2, 4, 8192, 128
    q = torch.empty(B, H, D, device="cuda", dtype=torch_dtype(dt))
    k, v = (torch.empty(B, H, N, D, device="cuda", dtype=torch_dtype(dt)) for _ in range(2))
    _fill((q, k, v), 2)
    call = lambda: (fa2.attn_decode(q, k, v, n_splits=16),)  # noqa: E731
    _check_replays("decode %s" % dt, lambda seed: _fill((q, k, v), seed), call)


@pytest.mark.parametrize("dt,D", [("f16", 64), ("bf16", 128), ("f32", 64), ("f32", 128)])
def test_backward_graph(dt, D):
    """attn_bwd alone is captured; between replays the inputs are refilled and
    O and the LSE recomputed eagerly into the same buffers."""
    import torch
    from gpu_util import torch_dtype
    B, H, N = 1, 2, 333
    tdt = torch_dtype(dt)
    q, k, v, g = (torch.empty(B, H, N, D, device="cuda", dtype=tdt) for _ in range(4))
    _fill((q, k, v, g), 3)
    o, lse = fa2.attn_fwd(q, k, v, scale=D ** -0.5, causal=True, return_lse=True)

    def refill(seed):
        _fill((q, k, v, g), seed)
        fa2.attn_fwd(q, k, v, scale=D ** -0.5, causal=True, out=o, return_lse=True, lse=lse)

    call = lambda: fa2.attn_bwd(q, k, v, o, g, lse, scale=D ** -0.5, causal=True)  # noqa: E731
    _check_replays("bwd %s D%d" % (dt, D), refill, call)
