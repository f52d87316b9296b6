"""The Python binding's checks, which run before the library is called: every
tensor must have the exact shape and dtype, be contiguous, and live on the GPU
(the library sees raw pointers and cannot tell a short buffer).  Inputs are
checked with CPU tensors here; caller-supplied outputs need GPU tensors and
are checked in test_gpu_binding.py."""
import pytest
import torch

from exact_attention_fa2_amd import fa2


def t(*shape, dtype=torch.float16):
    return torch.zeros(*shape, dtype=dtype)


def test_forward_inputs_on_the_host_are_refused():
    q = t(1, 2, 8, 64)
    with pytest.raises(ValueError, match="on a GPU"):
        fa2.attn_fwd(q, q, q)


def test_forward_shape_dtype_and_layout():
    q = t(1, 2, 8, 64)
    with pytest.raises(ValueError, match="k must have shape"):
        fa2.attn_fwd(q, t(1, 3, 8, 64), q)
    with pytest.raises(ValueError, match="v must have shape"):
        fa2.attn_fwd(q, t(1, 2, 9, 64), t(1, 2, 8, 64))
    with pytest.raises(TypeError, match="v must be torch.float16"):
        fa2.attn_fwd(q, q, t(1, 2, 8, 64, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="k must be contiguous"):
        fa2.attn_fwd(q, t(1, 2, 64, 8).transpose(2, 3), q)
    with pytest.raises(ValueError, match="q must have 4 dimensions"):
        fa2.attn_fwd(t(2, 8, 64), q, q)


def test_backward_inputs():
    q = t(1, 2, 8, 64)
    lse = t(1, 2, 8, dtype=torch.float32)
    with pytest.raises(TypeError, match="lse must be torch.float32"):
        fa2.attn_bwd(q, q, q, q, q, t(1, 2, 8))
    with pytest.raises(ValueError, match="lse must have shape"):
        fa2.attn_bwd(q, q, q, q, q, t(1, 2, 9, dtype=torch.float32))
    with pytest.raises(ValueError, match="dout must have shape"):
        fa2.attn_bwd(q, q, q, q, t(1, 2, 7, 64), lse)
    with pytest.raises(ValueError, match="on a GPU"):
        fa2.attn_bwd(q, q, q, q, q, lse)


def test_decode_inputs():
    q, k = t(2, 4, 128), t(2, 4, 100, 128)
    with pytest.raises(ValueError, match="k must have shape"):
        fa2.attn_decode_split(q, t(2, 4, 100, 64), k, 0.1, 4)
    with pytest.raises(ValueError, match="n_splits must be at least 1"):
        fa2.attn_decode_split(q, k, k, 0.1, 0)
    with pytest.raises(ValueError, match="on a GPU"):
        fa2.attn_decode_split(q, k, k, 0.1, 4)
    o_part = t(2, 4, 3, 128, dtype=torch.float32)
    with pytest.raises(ValueError, match="m_part must have shape"):
        fa2.attn_decode_combine(o_part, t(2, 4, 4, dtype=torch.float32),
                                t(2, 4, 3, dtype=torch.float32), torch.float16)
    with pytest.raises(TypeError, match="o_part must be torch.float32"):
        fa2.attn_decode_combine(t(2, 4, 3, 128), t(2, 4, 3, dtype=torch.float32),
                                t(2, 4, 3, dtype=torch.float32), torch.float16)
