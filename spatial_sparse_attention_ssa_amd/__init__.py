"""Spatial Sparse Attention (SSA) for MI355X (gfx950).

Python face of libssa.so (include/ssa.h).  Torch provides device memory and
the current HIP stream; every step of the block build and of the forward pass
runs in the library's HIP kernels.

    blocks = build_blocks(coords, cu_seqlens, grid_res=1024, m_cmp=4, m_win=8)
    out = forward(blocks, q, k, v, gates, topk=16)

    saved = forward_train(blocks, q, k, v, gates, topk=16)      # out + saved state
    grads = backward(blocks, q, k, v, gates, saved, dout)       # dq, dk, dv, dgates

Method: Direct3D-S2 (hyper.ai summary of arXiv 2505.17412, "Method"):
mean-pooled compressed attention, top-k spatial block selection and
non-overlapping window attention over 3D-blocked sparse voxel tokens, summed
with per-token gates; grouped query heads share the selection (LSRM article,
"Stage 1").
"""
from __future__ import annotations

import ctypes
import dataclasses

import torch

from . import _binding as B

__all__ = ["Blocks", "build_blocks", "forward", "forward_workspace_bytes", "forward_train", "backward",
           "backward_workspace_bytes", "SsaError", "library_path", "version"]

SsaError = B.SsaError


def library_path() -> str:
    return B.LIB_PATH


def version() -> int:
    return int(B.lib().ssa_version())


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


@dataclasses.dataclass
class Blocks:
    """Result of the block build; tensors live on the GPU."""
    perm: torch.Tensor
    blk_off: torch.Tensor
    win_off: torch.Tensor
    win_blk_off: torch.Tensor
    seq_blk_off: torch.Tensor
    seq_win_off: torch.Tensor
    counts: torch.Tensor
    struct: B.SsaBlocks
    coords: torch.Tensor | None = None   # kept alive: geometric routing reads it

    @property
    def n_tokens(self) -> int:
        return int(self.struct.n_tokens)

    @property
    def nb(self) -> int:
        return int(self.struct.nb)

    @property
    def nw(self) -> int:
        return int(self.struct.nw)

    def trimmed(self) -> dict:
        """Host copies of the segment arrays cut to their used lengths (syncs)."""
        c = self.counts.cpu().tolist()
        nb, nw = c[B.SSA_COUNT_NB], c[B.SSA_COUNT_NW]
        return dict(perm=self.perm.cpu(), blk_off=self.blk_off[:nb + 1].cpu(),
                    win_off=self.win_off[:nw + 1].cpu(), win_blk_off=self.win_blk_off[:nw + 1].cpu(),
                    seq_blk_off=self.seq_blk_off.cpu(), seq_win_off=self.seq_win_off.cpu(),
                    counts=c)


def build_blocks(coords: torch.Tensor, cu_seqlens: torch.Tensor, grid_res: int, m_cmp: int,
                 m_win: int, sync: bool = True, workspace: torch.Tensor | None = None,
                 win_shift: int = 0) -> Blocks:
    """Sort tokens by 3D block key and build the block / window segments.

    coords: int32 [N, 3] on the GPU; cu_seqlens: int32 [B + 1] on the GPU.
    ``win_shift`` (a multiple of m_cmp below m_win) moves the window origin
    to -win_shift on every axis (shifted windows).
    """
    if coords.dtype != torch.int32 or cu_seqlens.dtype != torch.int32:
        raise TypeError("coords and cu_seqlens must be int32")
    if not (coords.is_cuda and cu_seqlens.is_cuda):
        raise ValueError("coords and cu_seqlens must be GPU tensors")
    coords = coords.contiguous()
    cu_seqlens = cu_seqlens.contiguous()
    L = B.lib()
    n = int(coords.shape[0])
    batch = int(cu_seqlens.shape[0]) - 1
    dev = coords.device
    geo = B.SsaGeometry(grid_res, m_cmp, m_win, win_shift)
    i32 = dict(dtype=torch.int32, device=dev)
    perm = torch.empty(max(n, 1), **i32)
    blk_off = torch.empty(n + 1, **i32)
    win_off = torch.empty(n + 1, **i32)
    win_blk_off = torch.empty(n + 1, **i32)
    seq_blk_off = torch.empty(max(batch, 0) + 1, **i32)
    seq_win_off = torch.empty(max(batch, 0) + 1, **i32)
    counts = torch.empty(B.SSA_COUNTS, **i32)
    st = B.SsaBlocks(perm=perm.data_ptr(), blk_off=blk_off.data_ptr(), win_off=win_off.data_ptr(),
                     win_blk_off=win_blk_off.data_ptr(), seq_blk_off=seq_blk_off.data_ptr(),
                     seq_win_off=seq_win_off.data_ptr(), counts=counts.data_ptr())
    ws_bytes = int(L.ssa_build_blocks_workspace(n, batch, ctypes.byref(geo)))
    if workspace is None or workspace.numel() < ws_bytes:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    B.check(L.ssa_build_blocks(_ptr(coords), _ptr(cu_seqlens), n, batch, ctypes.byref(geo),
                               ctypes.byref(st), 1 if sync else 0, _ptr(workspace), ws_bytes,
                               _stream(dev)))
    return Blocks(perm[:n], blk_off, win_off, win_blk_off, seq_blk_off, seq_win_off, counts, st, coords)


_DTYPES = {torch.bfloat16: B.SSA_BF16, torch.float32: B.SSA_F32}


_ROUTING = {"score": B.SSA_ROUTE_SCORE, "geometric": B.SSA_ROUTE_GEOMETRIC}


def _attn(q, k, topk, scale, routing="score"):
    if q.dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {q.dtype}")
    if routing not in _ROUTING:
        raise ValueError(f"routing must be one of {sorted(_ROUTING)}")
    return B.SsaAttn(h_q=int(q.shape[1]), h_kv=int(k.shape[1]), head_dim=int(q.shape[2]),
                     topk=int(topk), scale=float(scale) if scale else 0.0, dtype=_DTYPES[q.dtype],
                     routing=_ROUTING[routing])


def forward_workspace_bytes(blocks: Blocks, q, k, topk: int, scale=None, routing: str = "score") -> int:
    a = _attn(q, k, topk, scale, routing)
    return int(B.lib().ssa_forward_workspace(ctypes.byref(blocks.struct), ctypes.byref(a)))


def forward(blocks: Blocks, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, gates: torch.Tensor,
            topk: int, scale: float | None = None, return_pooled: bool = False,
            return_topk: bool = False, out: torch.Tensor | None = None,
            workspace: torch.Tensor | None = None, stage_times: dict | None = None,
            routing: str = "score"):
    """SSA forward.  q [N, Hq, D], k/v [N, Hkv, D], gates [N, Hq, 3], all one dtype.

    Returns ``out`` [N, Hq, D]; with ``return_pooled`` / ``return_topk`` also
    the pooled keys/values [nb, Hkv, D] and the selected block ids
    [N, Hkv, topk] in a dict.  Passing a dict as ``stage_times`` runs the
    timed variant (blocks until done) and fills it with {kernel name: ms}.
    ``routing="geometric"`` selects the blocks nearest to each query voxel
    instead of the best-scored ones.
    """
    for name, t in (("q", q), ("k", k), ("v", v), ("gates", gates)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if t.dtype != q.dtype:
            raise TypeError(f"{name} dtype {t.dtype} differs from q dtype {q.dtype}")
    n = blocks.n_tokens
    if q.shape[0] != n or k.shape[0] != n or v.shape[0] != n or gates.shape[0] != n:
        raise ValueError("token count of q/k/v/gates differs from the blocks")
    if k.shape != v.shape or gates.shape != (n, q.shape[1], 3) or k.shape[2] != q.shape[2]:
        raise ValueError("shape mismatch among q, k, v, gates")
    q, k, v, gates = (t.contiguous() for t in (q, k, v, gates))
    L = B.lib()
    a = _attn(q, k, topk, scale, routing)
    dev = q.device
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_out(out, q)
    kc = vc = tk = None
    if return_pooled:
        if blocks.nb < 0:
            raise ValueError("return_pooled needs blocks built with sync=True")
        kc = torch.empty((max(blocks.nb, 1), k.shape[1], k.shape[2]), dtype=k.dtype, device=dev)
        vc = torch.empty_like(kc)
    if return_topk:
        tk = torch.empty((max(n, 1), k.shape[1], topk), dtype=torch.int32, device=dev)
    ws_bytes = int(L.ssa_forward_workspace(ctypes.byref(blocks.struct), ctypes.byref(a)))
    if workspace is None or workspace.numel() < ws_bytes:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    args = (ctypes.byref(blocks.struct), ctypes.byref(a), _ptr(q), _ptr(k), _ptr(v), _ptr(gates),
            _ptr(out), _ptr(kc), _ptr(vc), _ptr(tk), _ptr(workspace), ws_bytes, _stream(dev))
    if stage_times is None:
        B.check(L.ssa_forward(*args))
    else:
        ms = (ctypes.c_float * B.SSA_STAGES)()
        ns = ctypes.c_int32(0)
        B.check(L.ssa_forward_timed(*args, ms, ctypes.byref(ns)))
        for i in range(ns.value):
            stage_times[L.ssa_stage_name(ctypes.byref(a), i).decode()] = float(ms[i])
    if not (return_pooled or return_topk):
        return out
    res = dict(out=out)
    if return_pooled:
        res["k_cmp"], res["v_cmp"] = kc[:blocks.nb], vc[:blocks.nb]
    if return_topk:
        res["topk"] = tk[:n]
    return res


def _check_out(out, q):
    """A caller's output buffer must be exactly what the kernels write: a
    contiguous GPU tensor shaped and typed like q, 16-byte aligned, on q's
    device (the kernels write N * Hq * D elements 16 bytes at a time)."""
    if not isinstance(out, torch.Tensor):
        raise ValueError("out must be a tensor")
    if out.dtype != q.dtype:
        raise ValueError(f"out dtype {out.dtype} differs from q dtype {q.dtype}")
    if tuple(out.shape) != tuple(q.shape):
        raise ValueError(f"out shape {tuple(out.shape)} differs from q shape {tuple(q.shape)}")
    if not out.is_contiguous():
        raise ValueError("out must be contiguous")
    if out.data_ptr() % 16:
        raise ValueError("out must be 16-byte aligned")
    if not out.is_cuda or out.device != q.device:
        raise ValueError("out must be a GPU tensor on q's device")


def _check_inputs(blocks, q, k, v, gates):
    for name, t in (("q", q), ("k", k), ("v", v), ("gates", gates)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if t.dtype != q.dtype:
            raise TypeError(f"{name} dtype {t.dtype} differs from q dtype {q.dtype}")
    n = blocks.n_tokens
    if q.shape[0] != n or k.shape[0] != n or v.shape[0] != n or gates.shape[0] != n:
        raise ValueError("token count of q/k/v/gates differs from the blocks")
    if k.shape != v.shape or gates.shape != (n, q.shape[1], 3) or k.shape[2] != q.shape[2]:
        raise ValueError("shape mismatch among q, k, v, gates")
    return tuple(t.contiguous() for t in (q, k, v, gates))


def forward_train(blocks: Blocks, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                  gates: torch.Tensor, topk: int, scale: float | None = None,
                  workspace: torch.Tensor | None = None, routing: str = "score") -> dict:
    """SSA forward that also keeps what ``backward`` needs.

    Returns a dict: ``out`` [N, Hq, D], ``topk`` [N, Hkv, topk] int32 and
    ``lse`` [3, N, Hq] float32 (natural-log softmax denominators of the
    compressed, selected and window branches), plus ``topk_k`` and ``scale``.
    """
    q, k, v, gates = _check_inputs(blocks, q, k, v, gates)
    L = B.lib()
    a = _attn(q, k, topk, scale, routing)
    dev = q.device
    n, hq, d = q.shape
    out = torch.empty_like(q)
    tk = torch.empty((max(n, 1), k.shape[1], topk), dtype=torch.int32, device=dev)
    lse = torch.empty((3, max(n, 1), hq), dtype=torch.float32, device=dev)
    ws_bytes = int(L.ssa_forward_workspace(ctypes.byref(blocks.struct), ctypes.byref(a)))
    if workspace is None or workspace.numel() < ws_bytes:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    B.check(L.ssa_forward_train(ctypes.byref(blocks.struct), ctypes.byref(a), _ptr(q), _ptr(k), _ptr(v),
                                _ptr(gates), _ptr(out), _ptr(tk), _ptr(lse), _ptr(workspace), ws_bytes,
                                _stream(dev)))
    return dict(out=out, topk=tk, lse=lse, topk_k=int(topk), scale=scale)


def backward_workspace_bytes(blocks: Blocks, q, k, topk: int, scale=None) -> int:
    a = _attn(q, k, topk, scale)
    return int(B.lib().ssa_backward_workspace(ctypes.byref(blocks.struct), ctypes.byref(a)))


def backward(blocks: Blocks, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, gates: torch.Tensor,
             saved: dict, dout: torch.Tensor, want_dgates: bool = True,
             workspace: torch.Tensor | None = None, stage_times: dict | None = None) -> dict:
    """Gradients of sum(dout * out) for the forward that produced ``saved``.

    Returns a dict with ``dq`` [N, Hq, D], ``dk`` / ``dv`` [N, Hkv, D] and,
    with ``want_dgates``, ``dgates`` [N, Hq, 3], all in the input dtype.
    """
    q, k, v, gates = _check_inputs(blocks, q, k, v, gates)
    if dout.shape != q.shape or dout.dtype != q.dtype or not dout.is_cuda:
        raise ValueError("dout must be a GPU tensor shaped and typed like q")
    dout = dout.contiguous()
    L = B.lib()
    a = _attn(q, k, saved["topk_k"], saved["scale"])
    dev = q.device
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    dg = torch.empty_like(gates) if want_dgates else None
    ws_bytes = int(L.ssa_backward_workspace(ctypes.byref(blocks.struct), ctypes.byref(a)))
    if workspace is None or workspace.numel() < ws_bytes:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    args = (ctypes.byref(blocks.struct), ctypes.byref(a), _ptr(q), _ptr(k), _ptr(v), _ptr(gates), _ptr(dout),
            _ptr(saved["topk"]), _ptr(saved["lse"]), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg), _ptr(workspace),
            ws_bytes, _stream(dev))
    if stage_times is None:
        B.check(L.ssa_backward(*args))
    else:
        ms = (ctypes.c_float * B.SSA_STAGES)()
        ns = ctypes.c_int32(0)
        B.check(L.ssa_backward_timed(*args, ms, ctypes.byref(ns)))
        for i in range(ns.value):
            stage_times[L.ssa_backward_stage_name(ctypes.byref(a), i).decode()] = float(ms[i])
    res = dict(dq=dq, dk=dk, dv=dv)
    if want_dgates:
        res["dgates"] = dg
    return res
