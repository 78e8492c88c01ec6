"""The C ABI on the host: the library loads, exports every declared symbol,
and rejects bad arguments before touching the GPU (no compute call here)."""
import ctypes
import os
import re

import pytest

from spatial_sparse_attention_ssa_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _lib():
    if not os.path.exists(B.LIB_PATH):
        pytest.fail("libssa.so is not built (run __graft_entry__.build())")
    return B.lib()


def test_header_declares_exactly_the_exported_list():
    with open(os.path.join(ROOT, "include", "ssa.h")) as f:
        text = f.read()
    declared = set(re.findall(r"\b(ssa_[a-z_]+)\s*\(", text))
    assert declared == set(B.EXPORTED)


def test_every_declared_symbol_is_exported():
    L = _lib()
    for name in B.EXPORTED:
        assert hasattr(L, name), name


def test_version_and_status_strings():
    L = _lib()
    assert L.ssa_version() == 100
    for s in range(5):
        assert L.ssa_status_string(s)
    assert L.ssa_status_string(SSA_OK := 0) == b"ok"


def _fake_blocks(n=1000, batch=1, nb=-1):
    fake = 0x100000  # never dereferenced: validation fails first
    st = B.SsaBlocks(perm=fake, blk_off=fake, win_off=fake, win_blk_off=fake, seq_blk_off=fake,
                     seq_win_off=fake, counts=fake, n_tokens=n, batch=batch, nb=nb, nw=-1)
    return st


def _build(L, n=100, batch=1, geo=(64, 4, 8), ws=None, ws_bytes=0, out=True, coords=0x100000,
           cu=0x100000):
    g = B.SsaGeometry(*geo)
    st = _fake_blocks(n, batch)
    return L.ssa_build_blocks(ctypes.c_void_p(coords), ctypes.c_void_p(cu), n, batch, ctypes.byref(g),
                              ctypes.byref(st) if out else None, 1, ws, ws_bytes, None)


@pytest.mark.parametrize("geo", [(63, 4, 8), (64, 3, 8), (64, 8, 4), (2048, 4, 8), (64, 4, 128),
                                 (64, 4, 8, 2), (64, 4, 8, 8), (64, 4, 8, -4), (64, 8, 8, 4)])
def test_build_rejects_bad_geometry(geo):
    L = _lib()
    assert _build(L, geo=geo) == B.SSA_ERR_INVALID_ARGUMENT
    assert L.ssa_last_error()


def test_build_rejects_bad_sizes_and_pointers():
    L = _lib()
    assert _build(L, n=-1) == B.SSA_ERR_INVALID_ARGUMENT
    assert _build(L, batch=0) == B.SSA_ERR_INVALID_ARGUMENT
    assert _build(L, out=False) == B.SSA_ERR_INVALID_ARGUMENT
    assert _build(L, coords=0) == B.SSA_ERR_INVALID_ARGUMENT
    assert _build(L, cu=0) == B.SSA_ERR_INVALID_ARGUMENT


def test_build_key_wider_than_32_bits_is_unsupported():
    L = _lib()
    # R=1024, m_cmp=1: 30 bits of position; 8 sequences add 3 bits
    assert _build(L, batch=8, geo=(1024, 1, 8)) == B.SSA_ERR_UNSUPPORTED
    assert b"33 bits" in L.ssa_last_error()


def test_build_workspace_checks():
    L = _lib()
    g = B.SsaGeometry(64, 4, 8)
    need = L.ssa_build_blocks_workspace(100000, 1, ctypes.byref(g))
    assert need >= 3 * 4 * 100000
    assert _build(L, n=100000) == B.SSA_ERR_WORKSPACE
    assert _build(L, n=100000, ws=ctypes.c_void_p(0x100000), ws_bytes=need - 1) == B.SSA_ERR_WORKSPACE


def _attn(**kw):
    a = dict(h_q=16, h_kv=16, head_dim=64, topk=16, scale=0.0, dtype=B.SSA_BF16)
    a.update(kw)
    return B.SsaAttn(**a)


def _fwd(L, attn, blocks=True, ws=None, ws_bytes=0, ptr=0x100000):
    st = _fake_blocks()
    p = ctypes.c_void_p(ptr)
    return L.ssa_forward(ctypes.byref(st) if blocks else None, ctypes.byref(attn), p, p, p, p, p,
                         None, None, None, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=48), B.SSA_ERR_UNSUPPORTED),
    (dict(head_dim=128), B.SSA_ERR_UNSUPPORTED),
    (dict(topk=0), B.SSA_ERR_INVALID_ARGUMENT),
    (dict(topk=33), B.SSA_ERR_UNSUPPORTED),
    (dict(h_q=16, h_kv=3), B.SSA_ERR_INVALID_ARGUMENT),
    (dict(h_q=0), B.SSA_ERR_INVALID_ARGUMENT),
    (dict(h_q=64, h_kv=1), B.SSA_ERR_UNSUPPORTED),
    (dict(dtype=7), B.SSA_ERR_INVALID_ARGUMENT),
    (dict(scale=float("inf")), B.SSA_ERR_INVALID_ARGUMENT),
    (dict(routing=5), B.SSA_ERR_INVALID_ARGUMENT),
    (dict(routing=1, dtype=B.SSA_F32), B.SSA_ERR_UNSUPPORTED),
    (dict(routing=1, h_q=32, h_kv=1), B.SSA_ERR_UNSUPPORTED),   # 32 query heads per group: off the MFMA layouts
    (dict(routing=1), B.SSA_ERR_INVALID_ARGUMENT),     # the blocks carry no coordinates
])
def test_forward_rejects_bad_layout(kw, status):
    L = _lib()
    assert _fwd(L, _attn(**kw)) == status
    assert L.ssa_last_error()


def test_forward_rejects_null_inputs_and_small_workspace():
    L = _lib()
    assert _fwd(L, _attn(), blocks=False) == B.SSA_ERR_INVALID_ARGUMENT
    assert _fwd(L, _attn(), ptr=0) == B.SSA_ERR_INVALID_ARGUMENT
    assert _fwd(L, _attn()) == B.SSA_ERR_WORKSPACE
    st = _fake_blocks(n=1000, nb=50)
    need = L.ssa_forward_workspace(ctypes.byref(st), ctypes.byref(_attn()))
    # pooled keys and values for 50 blocks x 16 heads x 64 dims (bf16) + top-k ids
    assert need >= 2 * 50 * 16 * 64 * 2 + 1000 * 16 * 16 * 4
    st2 = _fake_blocks(n=1000, nb=-1)
    assert L.ssa_forward_workspace(ctypes.byref(st2), ctypes.byref(_attn())) > need


def test_binding_raises_without_gpu_tensors():
    import torch
    import spatial_sparse_attention_ssa_amd as ssa
    with pytest.raises(ValueError):
        ssa.build_blocks(torch.zeros((4, 3), dtype=torch.int32), torch.tensor([0, 4], dtype=torch.int32),
                         8, 2, 4)


def _bwd(L, attn, blocks=True, ptr=0x1000, lse=True, ws=None, ws_bytes=0, timed=False):
    st = _fake_blocks()
    p = ctypes.c_void_p(ptr)
    args = (ctypes.byref(st) if blocks else None, ctypes.byref(attn), p, p, p, p, p, p,
            p if lse else None, p, p, p, None, ws, ws_bytes, None)
    if timed:
        return L.ssa_backward_timed(*args, None, None)
    return L.ssa_backward(*args)


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=48), B.SSA_ERR_UNSUPPORTED),
    (dict(topk=0), B.SSA_ERR_INVALID_ARGUMENT),
    (dict(h_q=16, h_kv=3), B.SSA_ERR_INVALID_ARGUMENT),
    (dict(dtype=7), B.SSA_ERR_INVALID_ARGUMENT),
])
def test_backward_rejects_bad_layout(kw, status):
    L = _lib()
    assert _bwd(L, _attn(**kw)) == status
    assert L.ssa_last_error()


def test_backward_rejects_null_inputs_and_small_workspace():
    L = _lib()
    assert _bwd(L, _attn(), blocks=False) == B.SSA_ERR_INVALID_ARGUMENT
    assert _bwd(L, _attn(), ptr=0) == B.SSA_ERR_INVALID_ARGUMENT
    assert _bwd(L, _attn(), lse=False) == B.SSA_ERR_INVALID_ARGUMENT
    assert _bwd(L, _attn()) == B.SSA_ERR_WORKSPACE
    assert _bwd(L, _attn(), timed=True) == B.SSA_ERR_INVALID_ARGUMENT   # no stage_ms
    st = _fake_blocks(n=1000, nb=50)
    a = _attn()
    need = L.ssa_backward_workspace(ctypes.byref(st), ctypes.byref(a))
    # float32 dq accumulator plus the sorted-order dk / dv accumulators at least
    assert need >= 4 * 1000 * 16 * 64 * 3
    assert L.ssa_backward_stage_name(ctypes.byref(a), 0) == b"pool_kernel"
    assert L.ssa_backward_stage_name(ctypes.byref(a), 99) == b""


def test_forward_train_needs_its_outputs():
    L = _lib()
    st = _fake_blocks()
    p = ctypes.c_void_p(0x1000)
    a = _attn()
    assert L.ssa_forward_train(ctypes.byref(st), ctypes.byref(a), p, p, p, p, p, None, p, p, 1 << 40,
                               None) == B.SSA_ERR_INVALID_ARGUMENT
    assert L.ssa_forward_train(ctypes.byref(st), ctypes.byref(a), p, p, p, p, p, p, None, p, 1 << 40,
                               None) == B.SSA_ERR_INVALID_ARGUMENT


def test_forward_rejects_bad_out_buffers():
    # the kernels write N * Hq * D elements of q's dtype, 16 bytes at a time:
    # anything else passed as `out` is refused before the library is called
    import torch

    import spatial_sparse_attention_ssa_amd as ssa
    q = torch.zeros(10, 4, 64, dtype=torch.bfloat16)
    bad = {
        "dtype": torch.zeros(10, 4, 64, dtype=torch.float32),
        "shape": torch.zeros(9, 4, 64, dtype=torch.bfloat16),
        "contiguous": torch.zeros(10, 64, 4, dtype=torch.bfloat16).transpose(1, 2),
        "aligned": torch.zeros(10 * 4 * 64 + 1, dtype=torch.bfloat16)[1:].view(10, 4, 64),
        "GPU": torch.zeros(10, 4, 64, dtype=torch.bfloat16),   # a host tensor
    }
    for what, out in bad.items():
        with pytest.raises(ValueError, match=what):
            ssa._check_out(out, q)


def test_noalloc_forward_rejects_inputs_beyond_its_scratch():
    # 60000 tokens x 16 heads x 64 dims: the float32 branch accumulator alone
    # is 245 MB, beyond the 64 MiB array; rejected before anything runs
    L = _lib()
    st = _fake_blocks(n=60000)
    a = B.SsaAttn(h_q=16, h_kv=16, head_dim=64, topk=16, scale=0.0, dtype=B.SSA_BF16, routing=0)
    assert L.ssa_forward_workspace(ctypes.byref(st), ctypes.byref(a)) > B.SSA_NOALLOC_SCRATCH_BYTES
    fake = ctypes.c_void_p(0x100000)
    assert L.ssa_forward_noalloc(ctypes.byref(st), ctypes.byref(a), fake, fake, fake, fake, fake, None, None, None,
                                 None) == B.SSA_ERR_WORKSPACE
    assert b"64" in L.ssa_last_error() or b"scratch" in L.ssa_last_error()
