"""Caller-supplied outputs and workspaces are checked by the Python binding
before the library is called: a buffer of the wrong shape, dtype or device
is refused (the library sees raw pointers and would overrun a short one).
Nothing is launched by these calls."""
import pytest

from exact_attention_fa2_amd import fa2

pytestmark = pytest.mark.gpu


def test_forward_outputs():
    import torch
    q = torch.zeros(1, 2, 8, 64, device="cuda", dtype=torch.float16)
    with pytest.raises(ValueError, match="out must have shape"):
        fa2.attn_fwd(q, q, q, out=torch.empty(1, 2, 7, 64, device="cuda", dtype=torch.float16))
    with pytest.raises(TypeError, match="out must be torch.float16"):
        fa2.attn_fwd(q, q, q, out=torch.empty_like(q, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="out must be on"):
        fa2.attn_fwd(q, q, q, out=torch.empty(1, 2, 8, 64, dtype=torch.float16))
    with pytest.raises(TypeError, match="lse must be torch.float32"):
        fa2.attn_fwd(q, q, q, return_lse=True, lse=torch.empty(1, 2, 8, device="cuda",
                                                                dtype=torch.float16))
    with pytest.raises(ValueError, match="lse must have shape"):
        fa2.attn_fwd(q, q, q, return_lse=True, lse=torch.empty(1, 2, 4, device="cuda"))
    with pytest.raises(ValueError, match="k must be on"):
        fa2.attn_fwd(q, q.cpu(), q)


def test_forward_workspace_on_the_host_is_refused():
    import torch
    q = torch.zeros(1, 1, 64, 64, device="cuda", dtype=torch.float16)
    k = torch.zeros(1, 1, 8192, 64, device="cuda", dtype=torch.float16)
    assert fa2.workspace_size(1, 1, 64, 8192, 64, False, fa2.FA2_F16) > 0
    with pytest.raises(ValueError, match="workspace must be on"):
        fa2.attn_fwd(q, k, k, workspace=torch.empty(1 << 24, dtype=torch.uint8))


def test_backward_outputs():
    import torch
    q = torch.zeros(1, 2, 8, 64, device="cuda", dtype=torch.float16)
    lse = torch.zeros(1, 2, 8, device="cuda")
    with pytest.raises(ValueError, match="dq must have shape"):
        fa2.attn_bwd(q, q, q, q, q, lse, dq=torch.empty(1, 2, 4, 64, device="cuda",
                                                        dtype=torch.float16))
    with pytest.raises(TypeError, match="dv must be torch.float16"):
        fa2.attn_bwd(q, q, q, q, q, lse, dv=torch.empty_like(q, dtype=torch.float32))
    with pytest.raises(ValueError, match="delta must have shape"):
        fa2.attn_bwd(q, q, q, q, q, lse, delta=torch.empty(1, 2, 9, device="cuda"))


def test_decode_outputs():
    import torch
    q = torch.zeros(2, 4, 128, device="cuda", dtype=torch.float16)
    k = torch.zeros(2, 4, 100, 128, device="cuda", dtype=torch.float16)
    with pytest.raises(ValueError, match="o_part must have shape"):
        fa2.attn_decode_split(q, k, k, 0.1, 4,
                              o_part=torch.empty(2, 4, 3, 128, device="cuda"))
    with pytest.raises(TypeError, match="l_part must be torch.float32"):
        fa2.attn_decode_split(q, k, k, 0.1, 4,
                              l_part=torch.empty(2, 4, 4, device="cuda", dtype=torch.float16))
    o_part = torch.zeros(2, 4, 4, 128, device="cuda")
    m = torch.zeros(2, 4, 4, device="cuda")
    with pytest.raises(ValueError, match="out must have shape"):
        fa2.attn_decode_combine(o_part, m, m, torch.float16,
                                out=torch.empty(2, 4, 64, device="cuda", dtype=torch.float16))
