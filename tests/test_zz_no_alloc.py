"""The allocation-free forward (ssa_forward_noalloc) against ssa_forward,
through the C ABI: two calls in a row on one GPU, the second on a smaller
input (the scratch array keeps the first call's bytes), each output equal bit
for bit to ssa_forward's and within the oracle's bar."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import spatial_sparse_attention_ssa_amd as ssa
from spatial_sparse_attention_ssa_amd import _binding as B
from tests import _parity as P
from workloads import make_custom

pytestmark = pytest.mark.gpu


def _noalloc_forward(blocks, q, k, v, gates, topk):
    L = B.lib()
    a = ssa._attn(q, k, topk, None)
    out = torch.empty_like(q)
    tk = torch.empty((q.shape[0], k.shape[1], topk), dtype=torch.int32, device=q.device)
    ptr = lambda t: ctypes.c_void_p(t.data_ptr())
    stream = ctypes.c_void_p(torch.cuda.current_stream(q.device).cuda_stream)
    B.check(L.ssa_forward_noalloc(ctypes.byref(blocks.struct), ctypes.byref(a), ptr(q), ptr(k), ptr(v), ptr(gates),
                                  ptr(out), None, None, ptr(tk), stream))
    return out, tk


@pytest.mark.parametrize("order", ["large_then_small"])
@pytest.mark.parametrize("h_q,h_kv,head_dim", [(4, 4, 64), (8, 2, 32)])
def test_noalloc_forward_matches_forward(order, h_q, h_kv, head_dim):
    # the first input has a sequence of more than 512 blocks (the compressed
    # kernels' probe paths); the second is smaller
    cases = [dict(seqs=[14000, 700], grid_res=128, n_prims=4, seed=71),
             dict(seqs=[1500, 0, 900], grid_res=64, n_prims=3, seed=72)]
    for c in cases:
        wl = make_custom(c["seqs"], grid_res=c["grid_res"], n_prims=c["n_prims"], topk=16, h_q=h_q, h_kv=h_kv,
                         head_dim=head_dim, dtype="bf16", seed=c["seed"])
        print(f"noalloc case: {c['seqs']} tokens, {h_q}/{h_kv} heads, D = {head_dim}", flush=True)
        gb = P.gpu_build(wl)
        dt = torch.bfloat16
        q, k, v, g = (P.to_dev(x, dt) for x in (wl.q, wl.k, wl.v, wl.gates))
        assert ssa.forward_workspace_bytes(gb, q, k, wl.topk) <= B.SSA_NOALLOC_SCRATCH_BYTES
        ref = ssa.forward(gb, q, k, v, g, wl.topk, return_topk=True)
        out, tk = _noalloc_forward(gb, q, k, v, g, wl.topk)
        torch.cuda.synchronize()
        assert torch.equal(out, ref["out"]), "output differs from ssa_forward"
        assert torch.equal(tk, ref["topk"]), "selection differs from ssa_forward"
        oref = oracle.forward(wl, blocks=P.oracle_blocks(wl))
        D = wl.head_dim
        P.check_outputs(P.host(out).reshape(-1, D), oref["out_exact"].reshape(-1, D), dtype="bf16")
        same = (np.sort(tk.cpu().numpy(), -1) == np.sort(oref["topk"], -1)).all(-1).mean()
        assert same >= P.TOPK_AGREE, f"top-k agreement {same:.5f}"
