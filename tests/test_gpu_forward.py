"""GPU SSA forward vs the float64 oracle on the same seeded inputs.

Small workloads (several query tiles, ragged tails, empty sequences) are
compared element by element over every token and head.  The named workloads
are run in full on the GPU and compared on sampled (token, head) rows that the
oracle evaluates one by one; each branch is isolated with one-hot gates
(Direct3D-S2 page, "Method", second paragraph; LSRM article, "Stage 1" for the
grouped heads).
"""
import numpy as np
import pytest
import torch

import oracle
from tests import _parity as P
from workloads import make_custom, make_workload
from workloads.tensors import bf16_bits_from_f32, bf16_bits_to_f32

pytestmark = pytest.mark.gpu


def _full_compare(wl, branches=True):
    ob = P.oracle_blocks(wl)
    gb = P.gpu_build(wl)
    P.check_build(gb, ob)
    res = P.gpu_forward(wl, gb, return_topk=True, return_pooled=True)
    N, H, Hkv = wl.n_tokens, wl.h_q, wl.h_kv
    rows = [(t, h) for t in range(N) for h in range(H)]
    ref = oracle.forward_rows(wl, ob, rows, with_branches=branches, with_scores=True)
    got = P.host(res["out"]).reshape(N * H, -1)
    mx, mean = P.check_outputs(got, ref["out"], dtype=wl.dtype)
    G = H // Hkv
    gsel = res["topk"].cpu().numpy()[[t for t, _ in rows], [h // G for _, h in rows]]
    agree, gap = P.check_topk(gsel, ref["topk"], ref["scores"], ref["first_block"])
    kb = oracle.pool_blocks(wl.k, ob, wl.dtype)
    vb = oracle.pool_blocks(wl.v, ob, wl.dtype)
    _check_pooled(P.host(res["k_cmp"]), kb, wl.dtype)
    _check_pooled(P.host(res["v_cmp"]), vb, wl.dtype)
    if branches:
        for i, name in enumerate(("o_cmp", "o_sel", "o_win")):
            o = P.host(P.gpu_forward(wl, gb, gates=P.one_hot_gates(wl, i))).reshape(N * H, -1)
            P.check_branch(o, ref[name], name)
    print(f"N={N} H={H}/{Hkv}: max|err| {mx:.2e} mean|err| {mean:.2e} topk agree {agree:.5f} gap {gap:.1e}")


def _check_pooled(got, ref, dtype):
    if dtype == "f32":
        np.testing.assert_allclose(got, ref, rtol=1e-6, atol=1e-7)
        return
    # bfloat16: at most one unit in the last place, almost always identical
    ulp = np.abs(ref) * 2.0 ** -7 + 2.0 ** -133
    diff = np.abs(got - ref)
    assert (diff <= ulp).all(), f"pooled value off by more than 1 ulp: {diff.max():.3e}"
    assert (diff == 0).mean() >= 0.9999, f"only {(diff == 0).mean():.6f} bit-identical"


@pytest.mark.parametrize("case", [
    dict(seqs=[1500, 0, 900], h_q=4, h_kv=4, head_dim=64, topk=16, dtype="bf16"),
    dict(seqs=[2100], h_q=8, h_kv=2, head_dim=32, topk=8, dtype="bf16"),
    dict(seqs=[700, 1300], h_q=2, h_kv=2, head_dim=32, topk=4, dtype="f32"),
    dict(seqs=[333, 64, 1], h_q=2, h_kv=1, head_dim=64, topk=32, dtype="bf16"),
    # one query head per key/value head with k above 16 (the compressed
    # kernel's 32-entry list variant)
    dict(seqs=[2000, 0, 1100], h_q=4, h_kv=4, head_dim=64, topk=32, dtype="bf16"),
    dict(seqs=[1600], h_q=2, h_kv=2, head_dim=64, topk=20, dtype="bf16"),
    # one query head per key/value head at head_dim 32 (the generic kernel), k above 16
    dict(seqs=[800, 450], h_q=4, h_kv=4, head_dim=32, topk=20, dtype="bf16"),
    # grouped heads, 16 query heads per key/value head (the MFMA group path)
    dict(seqs=[900, 0, 701], h_q=16, h_kv=1, head_dim=32, topk=8, dtype="bf16"),
    dict(seqs=[1203], h_q=32, h_kv=2, head_dim=64, topk=16, dtype="bf16"),
    dict(seqs=[517, 35], h_q=32, h_kv=2, head_dim=32, topk=32, dtype="bf16"),
])
def test_small_full(case):
    wl = make_custom(case["seqs"], grid_res=64, n_prims=3, topk=case["topk"], h_q=case["h_q"],
                     h_kv=case["h_kv"], head_dim=case["head_dim"], dtype=case["dtype"], seed=21)
    _full_compare(wl)


@pytest.mark.parametrize("case", [
    dict(seqs=[1500, 0, 700], h_q=4, h_kv=4, head_dim=64, topk=16),
    dict(seqs=[900, 400], h_q=16, h_kv=1, head_dim=32, topk=8),
])
def test_shifted_windows_full(case):
    # window origin at -m_win / 2 on every axis (shifted windows)
    wl = make_custom(case["seqs"], grid_res=64, n_prims=3, topk=case["topk"], h_q=case["h_q"],
                     h_kv=case["h_kv"], head_dim=case["head_dim"], dtype="bf16", seed=41, win_shift=4)
    _full_compare(wl)


def test_shifted_windows_headline_sampled():
    wl = make_workload(3)
    wl.win_shift = wl.m_win // 2
    _sampled_check(wl, P.sample_rows(wl, 200, seed=33), tag="workload 3, shifted windows")


@pytest.mark.parametrize("case", [
    dict(seqs=[1500, 0, 700], h_q=4, h_kv=4, head_dim=64, topk=16),
    dict(seqs=[900, 400], h_q=16, h_kv=1, head_dim=32, topk=8),
    dict(seqs=[600], h_q=32, h_kv=2, head_dim=64, topk=32),
])
def test_geometric_routing_full(case):
    # the k blocks nearest to each query voxel (exact integer distances): the
    # lists must equal the oracle's, order included
    wl = make_custom(case["seqs"], grid_res=64, n_prims=3, topk=case["topk"], h_q=case["h_q"],
                     h_kv=case["h_kv"], head_dim=case["head_dim"], dtype="bf16", seed=43, routing="geometric")
    ob = P.oracle_blocks(wl)
    gb = P.gpu_build(wl)
    res = P.gpu_forward(wl, gb, return_topk=True, routing="geometric")
    N, H = wl.n_tokens, wl.h_q
    rows = [(t, h) for t in range(N) for h in range(H)]
    ref = oracle.forward_rows(wl, ob, rows, with_branches=True)
    G = H // wl.h_kv
    gsel = res["topk"].cpu().numpy()[[t for t, _ in rows], [h // G for _, h in rows]]
    assert np.array_equal(gsel, ref["topk"])
    P.check_outputs(P.host(res["out"]).reshape(N * H, -1), ref["out"], dtype=wl.dtype)
    o = P.host(P.gpu_forward(wl, gb, gates=P.one_hot_gates(wl, 1), routing="geometric")).reshape(N * H, -1)
    P.check_branch(o, ref["o_sel"], "o_sel")


def test_geometric_routing_headline_sampled():
    wl = make_workload(3)
    wl.routing = "geometric"
    ob = P.oracle_blocks(wl)
    gb = P.gpu_build(wl)
    res = P.gpu_forward(wl, gb, return_topk=True, routing="geometric")
    rows = P.sample_rows(wl, 64, seed=34)
    ref = oracle.forward_rows(wl, ob, rows)
    gsel = res["topk"].cpu().numpy()[[t for t, _ in rows], [h for _, h in rows]]
    assert np.array_equal(gsel, ref["topk"])
    tt = torch.tensor([t for t, _ in rows], device=P.DEV)
    hh = torch.tensor([h for _, h in rows], device=P.DEV)
    P.check_outputs(P.host(res["out"][tt, hh]), ref["out"], dtype=wl.dtype)


def test_tiny_fp32_workload_full():
    _full_compare(make_workload(1))


def _sampled_check(wl, rows, branches=True, min_agree=0.99, tag=""):
    ob = P.oracle_blocks(wl)
    gb = P.gpu_build(wl)
    P.check_build(gb, ob)
    res = P.gpu_forward(wl, gb, return_topk=True)
    kbar = oracle.pool_blocks(wl.k, ob, wl.dtype)
    vbar = oracle.pool_blocks(wl.v, ob, wl.dtype)
    ref = oracle.forward_rows(wl, ob, rows, kbar=kbar, vbar=vbar, with_branches=branches,
                              with_scores=True)
    tt = torch.tensor([t for t, _ in rows], device=P.DEV)
    hh = torch.tensor([h for _, h in rows], device=P.DEV)
    got = P.host(res["out"][tt, hh])
    mx, mean = P.check_outputs(got, ref["out"], dtype=wl.dtype)
    G = wl.h_q // wl.h_kv
    gsel = res["topk"][tt, hh // G].cpu().numpy()
    agree, gap = P.check_topk(gsel, ref["topk"], ref["scores"], ref["first_block"], min_agree=min_agree)
    if branches:
        for i, name in enumerate(("o_cmp", "o_sel", "o_win")):
            o = P.gpu_forward(wl, gb, gates=P.one_hot_gates(wl, i))
            P.check_branch(P.host(o[tt, hh]), ref[name], name)
    print(f"{tag}: max|err| {mx:.2e} mean|err| {mean:.2e} topk agree {agree:.4f} gap {gap:.1e}")
    return ob, gb, res


def _sampled_compare(cfg, n_rows, branches=True):
    wl = make_workload(cfg)
    print(f"workload {cfg}: N={wl.n_tokens}", flush=True)
    _sampled_check(wl, P.sample_rows(wl, n_rows, seed=cfg), branches, tag=f"workload {cfg}")


def test_workload2_sampled():
    _sampled_compare(2, 1500)


def test_headline_workload3_sampled():
    _sampled_compare(3, 400)


def test_gqa_workload4_sampled():
    _sampled_compare(4, 96)


def test_varlen_workload5_sampled():
    _sampled_compare(5, 256, branches=False)


@pytest.mark.parametrize("h_q,h_kv,head_dim,topk", [(4, 2, 64, 16), (16, 1, 32, 16), (32, 2, 64, 16),
                                                   (4, 4, 64, 16), (4, 4, 64, 32)])
def test_zero_queries_pick_first_blocks(h_q, h_kv, head_dim, topk):
    # every score ties, so the lowest block ids of the sequence are chosen
    # (on the one-head-per-group kernel every query overflows its candidate
    # list and goes to the exact fallback)
    wl = make_custom([1200, 500], grid_res=64, n_prims=3, topk=topk, h_q=h_q, h_kv=h_kv,
                     head_dim=head_dim, dtype="bf16", seed=31)
    wl.q[:] = 0
    ob = oracle.build_blocks(wl.coords, wl.cu_seqlens, wl.grid_res, wl.m_cmp, wl.m_win)
    gb = P.gpu_build(wl)
    res = P.gpu_forward(wl, gb, return_topk=True)
    sel = res["topk"].cpu().numpy()
    for b in range(wl.batch):
        j0, j1 = ob.seq_blk_off[b], ob.seq_blk_off[b + 1]
        toks = ob.perm[ob.blk_off[j0]:ob.blk_off[j1]]
        expect = np.arange(j0, min(j0 + topk, j1))
        assert (sel[toks][:, :, :len(expect)] == expect).all()


@pytest.mark.parametrize("head_dim", [32, 64])
def test_gqa_top_blocks_in_one_lane(head_dim):
    # Scattered voxels give about one token per block (over a thousand blocks
    # in one sequence).  Keys of the blocks whose id is 5 mod 32 are pushed
    # along one direction that every query shares, so the top k all come from
    # the same column of 32-block key tiles: the grouped top-k kernel keeps
    # only 8 blocks per column and token, and the exact fallback must decide.
    rng = np.random.default_rng(7)
    lin = rng.choice(64 ** 3, size=1500, replace=False)
    coords = np.stack(np.unravel_index(lin, (64,) * 3), -1)
    wl = make_custom(None, coords=coords, grid_res=64, topk=16, h_q=16, h_kv=1,
                     head_dim=head_dim, dtype="bf16", seed=7)
    ob = oracle.build_blocks(wl.coords, wl.cu_seqlens, wl.grid_res, wl.m_cmp, wl.m_win)
    nb = int(ob.seq_blk_off[1])
    assert nb > 32 * 9
    u = rng.standard_normal(head_dim).astype(np.float32)
    u /= np.linalg.norm(u)
    fav = np.flatnonzero(np.arange(nb) % 32 == 5)
    toks = np.concatenate([ob.perm[ob.blk_off[j]:ob.blk_off[j + 1]] for j in fav])
    k = wl.k.copy()
    k[toks, 0] += 4.0 * u
    q = 3.0 * u + 0.3 * wl.q
    wl.k = bf16_bits_to_f32(bf16_bits_from_f32(k))
    wl.q = bf16_bits_to_f32(bf16_bits_from_f32(q))
    rows = P.sample_rows(wl, 320, seed=7)
    _, _, res = _sampled_check(wl, rows, min_agree=P.TOPK_AGREE, tag=f"one-lane top-k D={head_dim}")
    sel = res["topk"].cpu().numpy()
    assert np.isin(sel[:, 0, :], fav).mean() > 0.99


def dense_cube(n, side, seed):
    """n distinct voxels drawn uniformly from a side^3 grid"""
    rng = np.random.default_rng(seed)
    lin = rng.choice(side ** 3, size=n, replace=False)
    return np.stack(np.unravel_index(lin, (side,) * 3), -1)


@pytest.mark.parametrize("h_q,h_kv,head_dim", [(4, 4, 64), (16, 1, 32)])
def test_large_windows_full(h_q, h_kv, head_dim):
    # 2900 of the 4096 voxels of a 16^3 grid: eight windows of about 360
    # tokens, each staged by the window kernel in several chunks
    wl = make_custom(None, coords=dense_cube(2900, 16, 11), grid_res=16, m_cmp=4, m_win=8, topk=8, h_q=h_q,
                     h_kv=h_kv, head_dim=head_dim, dtype="bf16", seed=13)
    assert np.diff(P.oracle_blocks(wl).win_off).min() > 256
    _full_compare(wl)


def test_many_sequences_full():
    # 1100 sequences of 1 to 5 tokens (every per-sequence tile prefix and
    # search over a long batch)
    from tests.test_gpu_backward import many_sequences
    lengths = np.random.default_rng(1100).choice([1, 2, 3, 5], size=1100)
    _full_compare(many_sequences(lengths, seed=41))


def test_dense_reduction():
    # one window over the grid, voxel blocks, top-k covering every block:
    # every branch is dense attention and out = (G0 + G1 + G2) * dense
    rng = np.random.default_rng(3)
    lin = rng.choice(16 ** 3, size=30, replace=False)
    coords = np.stack(np.unravel_index(lin, (16,) * 3), -1)
    wl = make_custom(None, coords=coords, grid_res=16, m_cmp=1, m_win=16, topk=32, h_q=2, h_kv=2,
                     head_dim=32, dtype="f32", seed=3)
    _full_compare(wl)


def test_run_to_run_bit_identical():
    wl = make_workload(2)
    gb = P.gpu_build(wl)
    a = P.gpu_forward(wl, gb, return_topk=True)
    b = P.gpu_forward(wl, gb, return_topk=True)
    assert torch.equal(a["out"], b["out"]) and torch.equal(a["topk"], b["topk"])
