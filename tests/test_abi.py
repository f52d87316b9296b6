"""The C ABI without a GPU: the library loads, exports exactly what
include/fa2.h declares, and rejects bad arguments with a status code before
anything is enqueued.  No compute call is made here."""
import ctypes
import os
import re
import subprocess

import pytest

from exact_attention_fa2_amd import fa2

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa2.h")

pytestmark = pytest.mark.skipif(not os.path.exists(fa2.LIB_PATH),
                                reason="libfa2.so not built (run __graft_entry__.build())")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M))


def test_exports_match_header():
    declared = header_functions()
    assert declared == set(fa2.EXPORTS)
    out = subprocess.check_output(["nm", "-D", "--defined-only", fa2.LIB_PATH], text=True)
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    assert declared <= exported, declared - exported
    # nothing else of ours leaks out of the library
    ours = {s for s in exported if "fa2" in s or s.startswith("attn")}
    assert ours == declared


def test_status_strings():
    L = fa2.lib()
    for code, text in fa2.STATUS.items():
        assert L.fa2_status_string(code).decode() == text
    assert L.fa2_status_string(99).decode() == "unknown status"


def _fwd(q=1, k=1, v=1, o=1, lse=None, B=1, H=1, Nq=4, Nk=4, D=64, scale=0.125, causal=0,
         dt=fa2.FA2_F16):
    p = lambda x: None if x is None else ctypes.c_void_p(x * 4096)  # noqa: E731
    return fa2.lib().attn_fwd(p(q), p(k), p(v), p(o), p(lse), B, H, Nq, Nk, D, scale, causal, dt,
                              None)


def test_fwd_error_paths():
    assert _fwd(Nk=0) == 2
    assert _fwd(B=-1) == 2
    assert _fwd(D=0) == 2
    assert _fwd(D=96) == 3
    assert _fwd(D=32) == 3
    assert _fwd(dt=7) == 3
    assert _fwd(causal=1, Nq=4, Nk=8) == 3
    assert _fwd(causal=2) == 3
    assert _fwd(scale=float("nan")) == 3
    assert _fwd(scale=float("inf")) == 3
    assert _fwd(q=None) == 1
    assert _fwd(v=None) == 1
    L = fa2.lib()
    mis = ctypes.c_void_p(4096 + 8)
    ok = ctypes.c_void_p(4096)
    assert L.attn_fwd(mis, ok, ok, ok, None, 1, 1, 4, 4, 64, 0.1, 0, 1, None) == 4
    assert L.attn_fwd(ok, ok, ok, ok, ctypes.c_void_p(4098), 1, 1, 4, 4, 64, 0.1, 0, 1, None) == 4
    # a slice of 2 GiB or more is refused up front
    assert _fwd(Nk=1 << 24, D=64) == 3
    # B*H is limited to 65535 (the grids' second dimension)
    assert _fwd(B=256, H=256) == 3
    assert _fwd(B=1, H=65536) == 3
    assert fa2.lib().attn_fwd_ws(*([ctypes.c_void_p(4096)] * 4), None, 2, 32768, 4, 4, 64, 0.1, 0, 1,
                                 None, 0, None) == 3


def test_fwd_empty_outputs_enqueue_nothing():
    # zero rows: valid and a no-op, even with NULL pointers
    assert fa2.lib().attn_fwd(None, None, None, None, None, 0, 1, 4, 4, 64, 0.1, 0, 1, None) == 0
    assert fa2.lib().attn_fwd(None, None, None, None, None, 1, 1, 0, 4, 64, 0.1, 0, 1, None) == 0


def test_decode_error_paths():
    L = fa2.lib()
    ok = ctypes.c_void_p(4096)
    args = lambda **kw: dict(dict(B=1, H=1, N=64, D=128, ns=4, dt=1), **kw)  # noqa: E731

    def split(q=ok, **kw):
        a = args(**kw)
        return L.attn_decode_split(q, ok, ok, ok, ok, ok, a["B"], a["H"], a["N"], a["D"], 0.1,
                                   a["ns"], a["dt"], None)

    assert split(N=0) == 2
    assert split(ns=0) == 2
    assert split(D=96) == 3
    assert split(dt=5) == 3
    assert L.attn_decode_split(ok, ok, ok, ok, ok, ok, 1, 1, 64, 128, float("nan"), 4, 1, None) == 3
    assert split(q=None) == 1
    assert split(q=ctypes.c_void_p(4100)) == 4
    assert split(B=0) == 0
    assert split(B=256, H=256) == 3
    assert L.attn_decode_combine(ok, ok, ok, ok, 1, 1, 128, 0, 1, None) == 2
    assert L.attn_decode_combine(ok, ok, ok, None, 1, 1, 128, 4, 1, None) == 1
    assert L.attn_decode_combine(ok, ok, ok, ok, 1, 1, 80, 4, 1, None) == 3
    assert L.attn_decode_combine(ok, ok, ok, ok, 0, 1, 128, 4, 1, None) == 0
    # o_part is read 16 bytes at a time; m_part and l_part need only 4
    assert L.attn_decode_combine(ctypes.c_void_p(4100), ok, ok, ok, 1, 1, 128, 4, 1, None) == 4


def test_default_splits_host_logic():
    L = fa2.lib()
    for B, H, N in ((8, 32, 32768), (1, 1, 100), (1, 1, 1 << 20), (64, 64, 4096)):
        s = L.attn_decode_default_splits(B, H, N, 128)
        assert 1 <= s <= max(1, (N + 255) // 256)
    assert L.attn_decode_default_splits(0, 1, 10, 128) == 1


def test_python_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(fa2, "_lib", None)
    monkeypatch.setattr(fa2, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="not built"):
        fa2.lib()


def test_workspace_size_plan():
    """attn_fwd_workspace_size without a GPU (256 compute units assumed)."""
    f16, bf16, f32 = fa2.FA2_F16, fa2.FA2_BF16, fa2.FA2_F32
    # very few query tiles and keys up to 2048 at D = 64: one launch of 32-row
    # workgroups whose waves split the keys, no workspace
    assert fa2.workspace_size(1, 2, 1024, 1024, 64, 1, f16) == 0
    assert fa2.workspace_size(1, 3, 129, 2000, 64, 0, bf16) == 0
    # ... longer keys, or D = 128: the key split across workgroups
    assert fa2.workspace_size(1, 1, 64, 4096, 64, 0, f16) > 0
    assert fa2.workspace_size(1, 2, 1024, 1024, 128, 1, bf16) % (2 * 1024 * 131 * 4) == 0
    assert fa2.workspace_size(1, 2, 1024, 1024, 128, 1, bf16) > 0
    # long keys with the tiles filling at most a quarter of the workgroup
    # slots: the keys are split, partials need (D + 3) floats per row and chunk
    need = fa2.workspace_size(1, 4, 4096, 4096, 64, 1, f16)
    assert need > 0 and need % (4 * 4096 * 67 * 4) == 0
    assert fa2.workspace_size(1, 4, 4096, 4096, 64, 0, bf16) == need
    # enough query tiles to fill the device: no split
    assert fa2.workspace_size(4, 12, 2048, 2048, 64, 0, f16) == 0
    # a split in exactly two chunks is merged in the kernel: a 64-bit
    # handshake word per 128-row tile (padded to 256 bytes), then per tile
    # two states of 128 x (D + 3) floats.  B4 H12 with 1024 queries (384
    # tiles, half the 768 slots) over 4096 keys; 64 tiles over 2500 keys (40
    # blocks: two chunks of at least 16); D = 128 with 16 tiles over 300 keys
    # (five blocks: two chunks of at least two)
    pair = lambda tiles, d: (tiles * 8 + 255) // 256 * 256 + tiles * 2 * 128 * (d + 3) * 4  # noqa: E731
    assert fa2.workspace_size(4, 12, 1024, 4096, 64, 0, f16) == pair(384, 64)
    assert fa2.workspace_size(4, 12, 1024, 4096, 64, 0, bf16) == pair(384, 64)
    assert fa2.workspace_size(1, 8, 1024, 2500, 64, 0, f16) == pair(64, 64)
    assert fa2.workspace_size(1, 8, 2500, 2500, 64, 1, f16) == pair(160, 64)
    assert fa2.workspace_size(1, 2, 1000, 300, 128, 0, bf16) == pair(16, 128)
    assert fa2.workspace_size(1, 2, 300, 300, 128, 1, f16) == pair(6, 128)
    # ... also at shorter keys where the tiles fill at most an eighth of the
    # slots (16 blocks or more), and at D = 64 at most half of them (32 blocks
    # or more) when causal or when the halves lower the most tiles per CU
    assert fa2.workspace_size(1, 8, 1024, 1024, 64, 0, f16) == pair(64, 64)
    assert fa2.workspace_size(1, 8, 1024, 1024, 128, 1, bf16) == pair(64, 128)
    assert fa2.workspace_size(2, 12, 2048, 2048, 64, 1, f16) == pair(384, 64)
    assert fa2.workspace_size(2, 12, 2048, 2048, 64, 0, f16) == pair(384, 64)
    assert fa2.workspace_size(2, 8, 2048, 2048, 64, 1, f16) == pair(256, 64)
    assert fa2.workspace_size(2, 8, 2048, 2048, 64, 0, f16) == 0     # 256 tiles: one per CU either way
    assert fa2.workspace_size(1, 12, 2048, 2048, 128, 0, f16) == 0   # D = 128 at half the slots
    assert fa2.workspace_size(4, 12, 1024, 1024, 64, 0, f16) == 0    # 16 blocks at half the slots
    # D = 128 splits the same way, with D + 3 floats per row and chunk
    need128 = fa2.workspace_size(1, 2, 4096, 4096, 128, 1, f16)
    assert need128 > 0 and need128 % (2 * 4096 * 131 * 4) == 0
    # float32 at D = 128 always runs whole (16-row workgroups); unsupported
    # requests ask for nothing
    assert fa2.workspace_size(1, 2, 1024, 1024, 128, 0, f32) == 0
    assert fa2.workspace_size(1, 2, 1024, 1024, 96, 0, f16) == 0
    assert fa2.workspace_size(1, 2, 1024, 512, 64, 1, f16) == 0
    assert fa2.workspace_size(0, 2, 1024, 1024, 64, 0, f16) == 0
    # float32 at D = 64, unmasked, where 32-row tiles split in two cover the
    # device: the key split with the in-kernel merge needs a 64-bit handshake
    # word per 32-row tile (padded to 256 bytes) and two partial states of
    # 32 x 64 + 2 x 32 floats per tile.  One head of 4096 rows: 128 tiles.
    part = lambda tiles: (tiles * 8 + 255) // 256 * 256 + tiles * 2 * (32 * 64 + 64) * 4  # noqa: E731
    assert fa2.workspace_size(1, 1, 4096, 4096, 64, 0, f32) == part(128)
    assert fa2.workspace_size(1, 1, 4090, 4096, 64, 0, f32) == part(128)
    assert fa2.workspace_size(1, 4, 1000, 4000, 64, 0, f32) == part(128)
    # ... no split where it would save under 3% (short keys, or tile counts
    # that fill whole rounds), causal shapes (the 16-row kernel), and many
    # heads (32-row tiles without a split)
    assert fa2.workspace_size(1, 1, 4096, 16, 64, 0, f32) == 0
    assert fa2.workspace_size(1, 2, 4096, 4096, 64, 0, f32) == 0
    assert fa2.workspace_size(3, 1, 3000, 2000, 64, 0, f32) == 0
    assert fa2.workspace_size(1, 1, 4096, 4096, 64, 1, f32) == 0
    assert fa2.workspace_size(8, 48, 256, 256, 64, 0, f32) == 0
    # fewer rows: the shared kernel's key split and the combine, D + 2 floats
    # per row and chunk
    need32 = fa2.workspace_size(1, 2, 1024, 1024, 64, 0, f32)
    assert need32 > 0 and need32 % (2 * 1024 * 66 * 4) == 0


def _bwd(q=1, k=1, v=1, o=1, g=1, lse=1, dq=1, dk=1, dv=1, delta=1, B=1, H=1, Nq=4, Nk=4, D=64,
         causal=0, dt=fa2.FA2_F16):
    p = lambda x: None if x is None else ctypes.c_void_p(x * 4096)  # noqa: E731
    return fa2.lib().attn_bwd(p(q), p(k), p(v), p(o), p(g), p(lse), p(dq), p(dk), p(dv), p(delta),
                              B, H, Nq, Nk, D, 0.125, causal, dt, None)


def test_bwd_error_paths():
    assert _bwd(Nk=0) == 2
    assert _bwd(Nq=-1) == 2
    assert _bwd(D=0) == 2
    assert _bwd(D=96) == 3
    assert _bwd(D=32, dt=fa2.FA2_F32) == 3
    assert _bwd(dt=9) == 3
    assert _bwd(causal=1, Nq=4, Nk=8) == 3
    assert _bwd(causal=3) == 3
    ok = ctypes.c_void_p(4096)
    assert fa2.lib().attn_bwd(*([ok] * 10), 1, 1, 4, 4, 64, float("-inf"), 0, 1, None) == 3
    for name in ("q", "k", "v", "o", "g", "lse", "dq", "dk", "dv", "delta"):
        assert _bwd(**{name: None}) == 1, name
    # with no queries only k, v, dk and dv are needed
    assert _bwd(q=None, o=None, g=None, lse=None, dq=None, delta=None, Nq=0, dk=None) == 1
    ok, mis = ctypes.c_void_p(4096), ctypes.c_void_p(4096 + 4)
    L = fa2.lib()
    for pos in range(10):
        ptrs = [ok] * 10
        ptrs[pos] = mis
        assert L.attn_bwd(*ptrs, 1, 1, 4, 4, 64, 0.1, 0, 1, None) == 4, pos
    assert _bwd(Nk=1 << 24) == 3
    assert _bwd(B=300, H=300) == 3
    assert _bwd(B=256, H=256) == 3
    # the grid limit: B*H*ceil(max(Nq,Nk)/128) must stay below 2^24 at D = 64
    assert _bwd(B=1, H=65535, Nq=1 << 16, Nk=4) == 3
    # B*H == 0: a valid no-op, even with NULL pointers
    assert fa2.lib().attn_bwd(*([None] * 10), 0, 4, 4, 4, 64, 0.1, 0, 1, None) == 0


def test_bench_refuses_more_than_one_gpu():
    """The path has no multi-GPU form: bench.py --gpus N with N > 1 exits with
    a message before touching a GPU."""
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)
