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
from oracle import parallel as oracle_pool
from tests import _parity as P
import spatial_sparse_attention_ssa_amd as ssa
from workloads import make_custom, make_workload
from workloads.tensors import bf16_bits_from_f32, bf16_bits_to_f32

pytestmark = pytest.mark.gpu


def _oracle_rows(wl, ob, rows, **kw):
    """oracle.forward_rows, over worker processes when there are many rows"""
    if len(rows) > 20000:
        return oracle_pool.forward_rows(wl, ob, rows, **kw)
    return oracle.forward_rows(wl, ob, rows, **kw)


def _full_compare(wl, branches=True, tag="full"):
    ob = P.oracle_blocks(wl)
    gb = P.gpu_build(wl)
    P.check_build(gb, ob)
    res = P.gpu_forward(wl, gb, return_topk=True, return_pooled=True)
    N, H, Hkv = wl.n_tokens, wl.h_q, wl.h_kv
    rows = [(t, h) for t in range(N) for h in range(H)]
    kb = oracle.pool_blocks(wl.k, ob, wl.dtype)
    vb = oracle.pool_blocks(wl.v, ob, wl.dtype)
    ref = _oracle_rows(wl, ob, rows, kbar=kb, vbar=vb, with_branches=branches, with_scores=True)
    got = P.host(res["out"]).reshape(N * H, -1)
    mx, mean = P.check_outputs(got, ref["out_exact"], dtype=wl.dtype)
    G = H // Hkv
    gsel = res["topk"].cpu().numpy()[[t for t, _ in rows], [h // G for _, h in rows]]
    agree, gap = P.check_topk(gsel, ref["topk"], ref["scores"], ref["first_block"])
    _check_pooled(P.host(res["k_cmp"]), kb, wl.dtype)
    _check_pooled(P.host(res["v_cmp"]), vb, wl.dtype)
    rels = {}
    if branches:
        for i, name in enumerate(("o_cmp", "o_sel", "o_win")):
            o = P.host(P.gpu_forward(wl, gb, gates=P.one_hot_gates(wl, i))).reshape(N * H, -1)
            rels[name] = P.check_branch(o, ref[name], name)
    P.record("forward_full", tag=tag, n_tokens=N, h_q=H, h_kv=Hkv, head_dim=wl.head_dim, topk=wl.topk,
             dtype=wl.dtype, rows=len(rows), topk_agree=agree, worst_gap=gap, max_err=mx, mean_err=mean,
             branch_rel=rels)
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
    # groups of 2, 4 and 8 query heads (the grouped MFMA kernels with the
    # rest of the top-k kernel's 16 heads empty)
    dict(seqs=[333, 64, 1], h_q=2, h_kv=1, head_dim=64, topk=32, dtype="bf16"),
    dict(seqs=[1700, 0, 600], h_q=16, h_kv=2, head_dim=64, topk=16, dtype="bf16"),
    dict(seqs=[900, 1200], h_q=12, h_kv=4, head_dim=32, topk=8, dtype="bf16"),
    # one query head per key/value head with k above 16 (the compressed
    # kernel's 32-entry list variant)
    dict(seqs=[2000, 0, 1100], h_q=4, h_kv=4, head_dim=64, topk=32, dtype="bf16"),
    dict(seqs=[1600], h_q=2, h_kv=2, head_dim=64, topk=20, dtype="bf16"),
    # one query head per key/value head at head_dim 32 (the compressed MFMA
    # kernel's D = 32 variant), k at most 16 and above 16
    dict(seqs=[1500, 0, 900], h_q=4, h_kv=4, head_dim=32, topk=16, dtype="bf16"),
    dict(seqs=[800, 450], h_q=4, h_kv=4, head_dim=32, topk=20, dtype="bf16"),
    dict(seqs=[333, 64, 1], h_q=2, h_kv=2, head_dim=32, topk=4, dtype="bf16"),
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
    dict(seqs=[1000, 500], h_q=4, h_kv=4, head_dim=32, topk=16),
    dict(seqs=[1200], h_q=8, h_kv=2, head_dim=64, topk=8),
])
def test_shifted_windows_full(case):
    # window origin at -m_win / 2 on every axis (shifted windows)
    wl = make_custom(case["seqs"], grid_res=64, n_prims=3, topk=case["topk"], h_q=case["h_q"],
                     h_kv=case["h_kv"], head_dim=case["head_dim"], dtype="bf16", seed=41, win_shift=4)
    _full_compare(wl)


def test_shifted_windows_headline_sampled():
    wl = make_workload(3)
    wl.win_shift = wl.m_win // 2
    _sampled_check(wl, P.sample_rows(wl, 10000, seed=33), tag="workload 3, shifted windows")


@pytest.mark.parametrize("case", [
    dict(seqs=[1500, 0, 700], h_q=4, h_kv=4, head_dim=64, topk=16),
    dict(seqs=[900, 400], h_q=16, h_kv=1, head_dim=32, topk=8),
    dict(seqs=[600], h_q=32, h_kv=2, head_dim=64, topk=32),
    dict(seqs=[1100, 300], h_q=4, h_kv=4, head_dim=32, topk=16),
    dict(seqs=[800], h_q=8, h_kv=2, head_dim=32, topk=8),
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
    P.check_outputs(P.host(res["out"]).reshape(N * H, -1), ref["out_exact"], dtype=wl.dtype)
    o = P.host(P.gpu_forward(wl, gb, gates=P.one_hot_gates(wl, 1), routing="geometric")).reshape(N * H, -1)
    P.check_branch(o, ref["o_sel"], "o_sel")


def test_geometric_routing_headline_sampled():
    wl = make_workload(3)
    wl.routing = "geometric"
    ob = P.oracle_blocks(wl)
    gb = P.gpu_build(wl)
    res = P.gpu_forward(wl, gb, return_topk=True, routing="geometric")
    rows = P.sample_rows(wl, 10000, seed=34)
    ref = oracle_pool.forward_rows(wl, ob, rows, with_branches=True)
    gsel = res["topk"].cpu().numpy()[[t for t, _ in rows], [h for _, h in rows]]
    assert np.array_equal(gsel, ref["topk"])
    tt = torch.tensor([t for t, _ in rows], device=P.DEV)
    hh = torch.tensor([h for _, h in rows], device=P.DEV)
    mx, mean = P.check_outputs(P.host(res["out"][tt, hh]), ref["out_exact"], dtype=wl.dtype)
    o = P.gpu_forward(wl, gb, gates=P.one_hot_gates(wl, 1), routing="geometric")
    rel = P.check_branch(P.host(o[tt, hh]), ref["o_sel"], "o_sel")
    P.record("forward_sampled", tag="workload 3, geometric routing", rows=len(rows), topk_agree=1.0,
             worst_gap=0.0, max_err=mx, mean_err=mean, branch_rel={"o_sel": rel})


def test_tiny_fp32_workload_full():
    _full_compare(make_workload(1))


def _sampled_check(wl, rows, branches=True, tag=""):
    ob = P.oracle_blocks(wl)
    gb = P.gpu_build(wl)
    P.check_build(gb, ob)
    res = P.gpu_forward(wl, gb, return_topk=True)
    ref = oracle_pool.forward_rows(wl, ob, rows, with_branches=branches, with_scores=True)
    tt = torch.tensor([t for t, _ in rows], device=P.DEV)
    hh = torch.tensor([h for _, h in rows], device=P.DEV)
    got = P.host(res["out"][tt, hh])
    mx, mean = P.check_outputs(got, ref["out_exact"], dtype=wl.dtype)
    G = wl.h_q // wl.h_kv
    gsel = res["topk"][tt, hh // G].cpu().numpy()
    agree, gap = P.check_topk(gsel, ref["topk"], ref["scores"], ref["first_block"])
    rels = {}
    if branches:
        for i, name in enumerate(("o_cmp", "o_sel", "o_win")):
            o = P.gpu_forward(wl, gb, gates=P.one_hot_gates(wl, i))
            rels[name] = P.check_branch(P.host(o[tt, hh]), ref[name], name)
    P.record("forward_sampled", tag=tag, n_tokens=wl.n_tokens, h_q=wl.h_q, h_kv=wl.h_kv, rows=len(rows),
             topk_agree=agree, worst_gap=gap, max_err=mx, mean_err=mean, branch_rel=rels)
    print(f"{tag}: {len(rows)} rows, max|err| {mx:.2e} mean|err| {mean:.2e} topk agree {agree:.5f} gap {gap:.1e}")
    return ob, gb, res


def _sampled_compare(cfg, n_rows, branches=True):
    wl = make_workload(cfg)
    print(f"workload {cfg}: N={wl.n_tokens}", flush=True)
    _sampled_check(wl, P.sample_rows(wl, n_rows, seed=cfg), branches, tag=f"workload {cfg}")


def test_workload2_full():
    # every (token, head) row of the 16384-token workload
    _full_compare(make_workload(2), tag="workload 2")


def test_headline_workload3_sampled():
    _sampled_compare(3, 10000)


def test_gqa_workload4_sampled():
    # each row costs the oracle 16 heads' compressed attention (the group score)
    _sampled_compare(4, 4000)


def test_varlen_workload5_sampled():
    _sampled_compare(5, 10000)


@pytest.mark.parametrize("h_q,h_kv,head_dim,topk", [(4, 2, 64, 16), (16, 1, 32, 16), (32, 2, 64, 16),
                                                   (4, 4, 64, 16), (4, 4, 64, 32), (4, 4, 32, 16)])
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
    # the same column of 32-block key tiles (the same lane of the grouped
    # top-k kernel's MFMA tiles) and stand far above every other block.
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
    _, _, res = _sampled_check(wl, rows, tag=f"one-lane top-k D={head_dim}")
    sel = res["topk"].cpu().numpy()
    assert np.isin(sel[:, 0, :], fav).mean() > 0.99


@pytest.mark.parametrize("head_dim,q_scale", [(64, 1.0), (64, 4.0), (32, 1.0), (32, 6.0)])
def test_probe_bound_paths_full(head_dim, q_scale):
    # a sequence with more than 512 blocks takes the compressed kernel's
    # first pass over its 512 largest-norm pooled keys; scaled queries break
    # the magnitude guard (|q| max |Kbar| scale log2 e <= 60), so the same
    # sequence takes the pass over all of its key tiles
    wl = make_custom([14000, 700], grid_res=128, n_prims=4, topk=16, h_q=4, h_kv=4, head_dim=head_dim,
                     dtype="bf16", seed=51)
    assert np.diff(P.oracle_blocks(wl).seq_blk_off).max() > 512
    if q_scale != 1.0:
        wl.q = bf16_bits_to_f32(bf16_bits_from_f32(wl.q * np.float32(q_scale)))
    _full_compare(wl, tag=f"probe paths D={head_dim}, q x {q_scale:g}")


@pytest.mark.parametrize("h_q,h_kv,head_dim,topk", [(32, 2, 64, 16), (16, 1, 32, 8)])
@pytest.mark.parametrize("q_scale", [1.0, 8.0])
def test_gqa_shift_paths_full(h_q, h_kv, head_dim, topk, q_scale):
    # the grouped compressed kernel shifts each query's softmax by the bound
    # |q| max_j |Kbar_j| scale log2 e when that is at most 60 for every query
    # of the workgroup, and otherwise keeps a running maximum; queries scaled
    # by 8 put the bound above 60 for most queries
    wl = make_custom([3000, 900], grid_res=64, n_prims=3, topk=topk, h_q=h_q, h_kv=h_kv, head_dim=head_dim,
                     dtype="bf16", seed=61)
    if q_scale != 1.0:
        wl.q = bf16_bits_to_f32(bf16_bits_from_f32(wl.q * np.float32(q_scale)))
    ob = P.oracle_blocks(wl)
    kbar = oracle.pool_blocks(wl.k, ob, wl.dtype)
    kmax = np.zeros((wl.batch, wl.h_kv))
    for b in range(wl.batch):
        j0, j1 = ob.seq_blk_off[b], ob.seq_blk_off[b + 1]
        kmax[b] = np.linalg.norm(kbar[j0:j1].astype(np.float64), axis=-1).max(0)
    seq = np.searchsorted(wl.cu_seqlens, np.arange(wl.n_tokens), side="right") - 1
    bound = (np.linalg.norm(wl.q.astype(np.float64), axis=-1) *
             kmax[seq][:, np.arange(wl.h_q) // (wl.h_q // wl.h_kv)]) / np.sqrt(wl.head_dim) * np.log2(np.e)
    if q_scale == 1.0:
        assert bound.max() < 30
    else:
        assert (bound > 60).mean() > 0.5
    _full_compare(wl, tag=f"grouped shift paths D={head_dim}, q x {q_scale:g}")


def test_constant_keys_pick_first_blocks():
    # every pooled key equal: all norms fall in one histogram bin (the probe
    # takes the sequence's first 512 blocks) and all logits tie, so each
    # query selects the sequence's lowest block ids
    wl = make_custom([14000, 300], grid_res=128, n_prims=4, topk=16, h_q=4, h_kv=4, head_dim=64, dtype="bf16",
                     seed=52)
    wl.k[:] = wl.k[0:1, 0:1, :]
    ob = P.oracle_blocks(wl)
    assert np.diff(ob.seq_blk_off).max() > 512
    gb = P.gpu_build(wl)
    sel = P.gpu_forward(wl, gb, return_topk=True)["topk"].cpu().numpy()
    for b in range(wl.batch):
        j0, j1 = ob.seq_blk_off[b], ob.seq_blk_off[b + 1]
        toks = ob.perm[ob.blk_off[j0]:ob.blk_off[j1]]
        expect = np.arange(j0, min(j0 + wl.topk, j1))
        assert (sel[toks][:, :, :len(expect)] == expect).all()


@pytest.mark.parametrize("head_dim", [32, 64])
def test_gqa_constant_keys_pick_first_blocks(head_dim):
    # grouped heads with every pooled key equal: all of a token's block scores
    # tie, so the grouped top-k kernel admits every block and cuts its lists
    # to the top k again and again (ties: lower block first); the long
    # sequence takes the probe-set warm-up, the short one its own tiles
    wl = make_custom([14000, 300], grid_res=128, n_prims=4, topk=16, h_q=16, h_kv=1, head_dim=head_dim,
                     dtype="bf16", seed=53)
    wl.k[:] = wl.k[0:1, 0:1, :]
    ob = P.oracle_blocks(wl)
    nbs = np.diff(ob.seq_blk_off)
    assert nbs[0] > 512 >= nbs[1]
    gb = P.gpu_build(wl)
    sel = P.gpu_forward(wl, gb, return_topk=True)["topk"].cpu().numpy()
    for b in range(wl.batch):
        j0, j1 = ob.seq_blk_off[b], ob.seq_blk_off[b + 1]
        toks = ob.perm[ob.blk_off[j0]:ob.blk_off[j1]]
        expect = np.arange(j0, min(j0 + wl.topk, j1))
        assert (sel[toks][:, :, :len(expect)] == expect).all()


@pytest.mark.parametrize("h_q,h_kv", [(16, 1), (8, 2)])
def test_gqa_probe_warmup_full(h_q, h_kv):
    # grouped heads on a sequence of more than 512 blocks (its lower bound on
    # each token's k-th score comes from the probe set) beside a short one
    # (bounded from its own blocks); compared in full with the oracle
    wl = make_custom([14000, 700], grid_res=128, n_prims=4, topk=16, h_q=h_q, h_kv=h_kv, head_dim=32, dtype="bf16",
                     seed=54)
    nbs = np.diff(P.oracle_blocks(wl).seq_blk_off)
    assert nbs[0] > 512 >= nbs[1]
    _full_compare(wl, tag=f"grouped probe warm-up {h_q}/{h_kv}")


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


@pytest.mark.parametrize("h_q,h_kv,head_dim,dtype", [(2, 2, 32, "f32"), (4, 4, 64, "bf16"), (16, 1, 32, "bf16"),
                                                   (32, 2, 64, "bf16"), (2, 2, 32, "bf16"), (8, 2, 32, "bf16")])
def test_dense_reduction(h_q, h_kv, head_dim, dtype):
    # one window over the grid, voxel blocks, top-k covering every block:
    # every branch is dense attention and out = (G0 + G1 + G2) * dense (the
    # bfloat16 layouts run the MFMA kernels)
    rng = np.random.default_rng(3)
    lin = rng.choice(16 ** 3, size=30, replace=False)
    coords = np.stack(np.unravel_index(lin, (16,) * 3), -1)
    wl = make_custom(None, coords=coords, grid_res=16, m_cmp=1, m_win=16, topk=32, h_q=h_q, h_kv=h_kv,
                     head_dim=head_dim, dtype=dtype, seed=3)
    _full_compare(wl, tag=f"dense reduction {h_q}/{h_kv} D={head_dim} {dtype}")
    # and directly against dense softmax attention in float64
    gb = P.gpu_build(wl)
    got = P.host(P.gpu_forward(wl, gb))
    G = h_q // h_kv
    q = wl.q.astype(np.float64)
    k = np.repeat(wl.k.astype(np.float64), G, axis=1)
    v = np.repeat(wl.v.astype(np.float64), G, axis=1)
    s = np.einsum("thd,uhd->htu", q, k) / np.sqrt(head_dim)
    p = np.exp(s - s.max(-1, keepdims=True))
    p /= p.sum(-1, keepdims=True)
    dense = np.einsum("htu,uhd->thd", p, v)
    expect = wl.gates.astype(np.float64).sum(-1)[..., None] * dense
    P.check_outputs(got.reshape(-1, head_dim), expect.reshape(-1, head_dim), dtype=dtype)


def test_run_to_run_bit_identical():
    wl = make_workload(2)
    gb = P.gpu_build(wl)
    a = P.gpu_forward(wl, gb, return_topk=True)
    b = P.gpu_forward(wl, gb, return_topk=True)
    assert torch.equal(a["out"], b["out"]) and torch.equal(a["topk"], b["topk"])


@pytest.mark.parametrize("h_q,h_kv,head_dim", [(4, 4, 64), (16, 1, 32), (2, 2, 32)])
def test_empty_token_set_forward_and_backward(h_q, h_kv, head_dim):
    # no tokens in any of the batch's sequences: every call succeeds and
    # returns empty tensors (the forward and backward launch nothing)
    wl = make_custom(None, coords=np.zeros((0, 3), np.int64), cu_seqlens=[0, 0, 0], grid_res=64, topk=8, h_q=h_q,
                     h_kv=h_kv, head_dim=head_dim, dtype="bf16", seed=1)
    assert wl.n_tokens == 0
    gb = P.gpu_build(wl)
    res = P.gpu_forward(wl, gb, return_topk=True)
    assert tuple(res["out"].shape) == (0, h_q, head_dim) and res["topk"].shape[0] == 0
    dt = torch.bfloat16
    q, k, v, g = (P.to_dev(a, dt) for a in (wl.q, wl.k, wl.v, wl.gates))
    saved = ssa.forward_train(gb, q, k, v, g, wl.topk)
    grads = ssa.backward(gb, q, k, v, g, saved, torch.zeros_like(q))
    torch.cuda.synchronize()
    assert tuple(grads["dq"].shape) == (0, h_q, head_dim) and tuple(grads["dk"].shape) == (0, h_kv, head_dim)
