"""Pins of the oracle's float stages: pooling, the three attention branches,
top-k selection and the gated sum.

Pinned against: the hand-worked fixture tests/golden/forward_gqa_d4.json;
torch's bfloat16 conversion; exact rational block means; torch's
scaled_dot_product_attention in float64 where a branch reduces to dense
attention (m_cmp = 1, k >= blocks, one window covering the grid); closed forms
(constant V, Q = 0, one token per window); brute-force top-k; and the
equivariance of the whole map under a reordering of the input tokens
(Direct3D-S2 page, "Method"; LSRM article, "Stage 1" for the grouped heads).
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from tests import _golden
from workloads import make_custom


def _dense(q, k, v):
    """Library dense attention, float64: q [Lq, D], k/v [Lk, D]."""
    t = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float64))[None, None]
    return torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v))[0, 0].numpy()


def _wl_from_golden(g):
    wl = make_custom(None, coords=np.array(g["coords"]), cu_seqlens=g["cu_seqlens"],
                     grid_res=g["grid_res"], m_cmp=g["m_cmp"], m_win=g["m_win"], topk=g["topk"],
                     h_q=g["h_q"], h_kv=g["h_kv"], head_dim=g["head_dim"], dtype=g["dtype"])
    wl.q = _golden.arr(g["q"]).astype(np.float32)
    wl.k = _golden.arr(g["k"]).astype(np.float32)
    wl.v = _golden.arr(g["v"]).astype(np.float32)
    wl.gates = np.broadcast_to(np.array(g["gates"], np.float32), wl.q.shape[:2] + (3,)).copy()
    return wl


# ---------------------------------------------------------------- rounding

def test_bf16_round_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000),
                        [0.0, -0.0, 1.0, 1.00390625, 1.01171875, 2.0 ** -130, -(2.0 ** -127) * 3]])
    x32 = x.astype(np.float32)
    ref = torch.from_numpy(x32).to(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.bf16_round(x32.astype(np.float64))
    assert np.array_equal(got, ref)


# ---------------------------------------------------------------- hand-worked

def test_golden_gqa_forward():
    g = _golden.load("forward_gqa_d4.json")
    wl = _wl_from_golden(g)
    res = oracle.forward(wl, with_branches=True)
    b = res["blocks"]
    assert b.perm.tolist() == g["perm"]
    np.testing.assert_allclose(res["kbar"], _golden.arr(g["kbar"]), rtol=1e-6, atol=1e-7)
    np.testing.assert_allclose(res["vbar"], _golden.arr(g["vbar"]), rtol=0, atol=0)
    assert res["topk"].tolist() == g["selected"]
    np.testing.assert_allclose(res["out"], _golden.arr(g["out"]), rtol=1e-6, atol=1e-6)


# ---------------------------------------------------------------- pooling

def test_pool_is_exact_block_mean():
    wl = make_custom([400], grid_res=32, m_cmp=4, m_win=8, h_q=2, h_kv=2, head_dim=8, seed=3)
    b = oracle.build_blocks(wl.coords, wl.cu_seqlens, wl.grid_res, wl.m_cmp, wl.m_win)
    kbar = oracle.pool_blocks(wl.k, b, "bf16")
    for j in range(0, b.nb, 3):
        toks = b.perm[b.blk_off[j]:b.blk_off[j + 1]]
        for h in range(2):
            for d in range(8):
                exact = sum(Fraction(float(wl.k[t, h, d])) for t in toks) / len(toks)
                ref = torch.tensor(float(exact), dtype=torch.float64).to(torch.float32)
                # the exact mean is within 2^-24 relative of its float32 image, far
                # below bf16 spacing: compare against torch's bf16 rounding of it
                ref = float(ref.to(torch.bfloat16).to(torch.float64))
                assert kbar[j, h, d] == ref or abs(kbar[j, h, d] - ref) <= 2.0 ** -8 * abs(ref)


def test_pool_constant_blocks():
    wl = make_custom([300], grid_res=32, m_cmp=4, m_win=8, h_q=1, h_kv=1, head_dim=4, seed=4)
    b = oracle.build_blocks(wl.coords, wl.cu_seqlens, wl.grid_res, wl.m_cmp, wl.m_win)
    blk_of_tok = np.empty(wl.n_tokens, np.int64)
    for j in range(b.nb):
        blk_of_tok[b.perm[b.blk_off[j]:b.blk_off[j + 1]]] = j
    const = (np.arange(b.nb) * 0.25 - 3.0)[:, None, None] * np.array([1, -2, 0.5, 4])
    k = const[blk_of_tok].astype(np.float32)
    assert np.array_equal(oracle.pool_blocks(k, b, "bf16"), oracle.bf16_round(const))


# ---------------------------------------------------------------- reductions to dense attention

def _single_window_dense_workload(seed, n=150, R=16, hq=2, hkv=2, d=8, dtype="f32"):
    rng = np.random.default_rng(seed)
    lin = rng.choice(R ** 3, size=n, replace=False)       # unique voxels
    coords = np.stack(np.unravel_index(lin, (R,) * 3), -1)
    return make_custom(None, coords=coords, grid_res=R, m_cmp=1, m_win=R, topk=n,
                       h_q=hq, h_kv=hkv, head_dim=d, dtype=dtype, seed=seed)


@pytest.mark.parametrize("seed", [0, 1])
def test_every_branch_reduces_to_dense(seed):
    wl = _single_window_dense_workload(seed)
    res = oracle.forward(wl, with_branches=True)
    for h in range(wl.h_q):
        g = h // (wl.h_q // wl.h_kv)
        ref = _dense(wl.q[:, h], wl.k[:, g], wl.v[:, g])
        for name in ("o_cmp", "o_sel", "o_win"):
            np.testing.assert_allclose(res[name][:, h], ref, rtol=1e-10, atol=1e-12)
        gs = wl.gates[:, h].astype(np.float64).sum(-1, keepdims=True)
        np.testing.assert_allclose(res["out"][:, h], oracle.round_to(gs * ref, "f32"), rtol=1e-6, atol=1e-6)


def test_compressed_branch_dense_when_blocks_are_voxels():
    wl = make_custom([500], grid_res=32, m_cmp=1, m_win=8, topk=3, h_q=2, h_kv=1, head_dim=16,
                     dtype="f32", seed=7)
    res = oracle.forward(wl, with_branches=True)
    b = res["blocks"]
    for h in range(2):
        ref = _dense(wl.q[:, h], wl.k[b.perm, 0], wl.v[b.perm, 0])
        np.testing.assert_allclose(res["o_cmp"][:, h], ref, rtol=1e-10, atol=1e-12)


def test_window_branch_dense_per_window():
    wl = make_custom([500], grid_res=32, m_cmp=4, m_win=8, topk=2, h_q=2, h_kv=2, head_dim=8,
                     dtype="f32", seed=8)
    res = oracle.forward(wl, with_branches=True)
    b = res["blocks"]
    for w in range(b.nw):
        toks = b.perm[b.win_off[w]:b.win_off[w + 1]]
        for h in range(2):
            ref = _dense(wl.q[toks, h], wl.k[toks, h], wl.v[toks, h])
            np.testing.assert_allclose(res["o_win"][toks, h], ref, rtol=1e-10, atol=1e-12)


def test_shifted_window_branch_is_dense_per_shifted_cell():
    # windows start at -4 on every axis: group the tokens by ((c + 4) // 8)
    # independently and compare with dense attention inside each group
    wl = make_custom([500], grid_res=32, m_cmp=4, m_win=8, topk=2, h_q=2, h_kv=1, head_dim=8,
                     dtype="f32", seed=12, win_shift=4)
    res = oracle.forward(wl, with_branches=True)
    cells = {}
    for t, c in enumerate(wl.coords):
        cells.setdefault(tuple((int(x) + 4) // 8 for x in c), []).append(t)
    assert len(cells) == res["blocks"].nw
    for toks in cells.values():
        toks = np.array(toks)
        for h in range(2):
            ref = _dense(wl.q[toks, h], wl.k[toks, 0], wl.v[toks, 0])
            np.testing.assert_allclose(res["o_win"][toks, h], ref, rtol=1e-10, atol=1e-12)


# ---------------------------------------------------------------- closed forms

def test_constant_values_give_constant_output():
    wl = make_custom([300, 120], grid_res=32, topk=3, h_q=4, h_kv=2, head_dim=8, dtype="f32", seed=9)
    c = np.array([0.5, -1.0, 2.0, 0.0, 3.0, -0.25, 1.5, 7.0], np.float32)
    wl.v[:] = c
    res = oracle.forward(wl, with_branches=True)
    for name in ("o_cmp", "o_sel", "o_win"):
        np.testing.assert_allclose(res[name], np.broadcast_to(c, res[name].shape), rtol=1e-12, atol=1e-12)


def test_zero_queries_select_first_blocks_and_average():
    wl = make_custom([400, 0, 250], grid_res=32, topk=5, h_q=2, h_kv=2, head_dim=8, dtype="bf16", seed=10)
    wl.q[:] = 0
    res = oracle.forward(wl, with_branches=True)
    b = res["blocks"]
    for s in range(wl.batch):
        j0, j1 = b.seq_blk_off[s], b.seq_blk_off[s + 1]
        toks = b.perm[b.blk_off[j0]:b.blk_off[j1]] if j1 > j0 else []
        if not len(toks):
            continue
        expect_sel = list(range(j0, min(j0 + 5, j1)))
        pos0, pos1 = b.blk_off[j0], b.blk_off[min(j0 + 5, j1)]
        first_k_toks = b.perm[pos0:pos1]
        for h in range(2):
            assert all(res["topk"][t, h, :len(expect_sel)].tolist() == expect_sel for t in toks)
            np.testing.assert_allclose(res["o_cmp"][toks, h], np.broadcast_to(res["vbar"][j0:j1, h].mean(0), (len(toks), 8)), atol=1e-12)
            np.testing.assert_allclose(res["o_sel"][toks, h], np.broadcast_to(wl.v[first_k_toks, h].astype(np.float64).mean(0), (len(toks), 8)), atol=1e-12)


def test_one_token_per_window_returns_own_value():
    R, mw = 32, 4
    cells = np.stack(np.meshgrid(*[np.arange(0, R, mw)] * 3, indexing="ij"), -1).reshape(-1, 3)
    rng = np.random.default_rng(11)
    coords = cells + rng.integers(0, mw, size=cells.shape)
    wl = make_custom(None, coords=coords, grid_res=R, m_cmp=2, m_win=mw, topk=2, h_q=2, h_kv=2,
                     head_dim=8, dtype="f32", seed=11)
    res = oracle.forward(wl, with_branches=True)
    np.testing.assert_allclose(res["o_win"], wl.v.astype(np.float64), rtol=0, atol=0)


def test_gates_are_linear_and_one_hot_isolates_branches():
    wl = make_custom([300], grid_res=32, topk=3, h_q=2, h_kv=2, head_dim=8, dtype="f32", seed=12)
    base = oracle.forward(wl, with_branches=True)
    for i, name in enumerate(("o_cmp", "o_sel", "o_win")):
        w2 = make_custom([300], grid_res=32, topk=3, h_q=2, h_kv=2, head_dim=8, dtype="f32", seed=12)
        w2.gates[:] = 0
        w2.gates[..., i] = 1
        res = oracle.forward(w2)
        np.testing.assert_allclose(res["out"], oracle.round_to(base[name], "f32"), rtol=0, atol=0)


# ---------------------------------------------------------------- top-k

@pytest.mark.parametrize("seed", range(6))
def test_topk_brute_force(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 40))
    s = rng.integers(0, 6, size=n).astype(np.float64) / 7.0  # many exact ties
    for k in (1, 3, 8, 50):
        ref = sorted(range(n), key=lambda j: (-s[j], j))[:k]
        assert oracle.topk_blocks(s, k).tolist() == ref


def test_gqa_equal_heads_rank_like_one_head():
    wl = make_custom([400], grid_res=32, topk=4, h_q=4, h_kv=1, head_dim=8, dtype="f32", seed=13)
    wl.q[:] = wl.q[:, :1]
    res = oracle.forward(wl)
    b = res["blocks"]
    kbar = res["kbar"]
    for t in range(0, wl.n_tokens, 13):
        logits = kbar[:, 0] @ wl.q[t, 0].astype(np.float64)
        ref = sorted(range(b.nb), key=lambda j: (-logits[j], j))[:4]
        assert res["topk"][t, 0].tolist() == ref


# ---------------------------------------------------------------- structure

def test_input_order_equivariance():
    wl = make_custom([350, 200], grid_res=32, topk=4, h_q=2, h_kv=1, head_dim=8, dtype="bf16", seed=14)
    res = oracle.forward(wl)
    rng = np.random.default_rng(1)
    cu = wl.cu_seqlens
    p = np.concatenate([cu[b] + rng.permutation(cu[b + 1] - cu[b]) for b in range(wl.batch)])
    w2 = make_custom([350, 200], grid_res=32, topk=4, h_q=2, h_kv=1, head_dim=8, dtype="bf16", seed=14)
    for name in ("coords", "q", "k", "v", "gates"):
        setattr(w2, name, getattr(wl, name)[p].copy())
    res2 = oracle.forward(w2)
    np.testing.assert_array_equal(res2["kbar"], res["kbar"])
    np.testing.assert_array_equal(res2["topk"], res["topk"][p])
    np.testing.assert_allclose(res2["out"], res["out"][p], rtol=0, atol=1e-12)


def test_sequences_do_not_interact():
    one = make_custom([300], grid_res=32, topk=4, h_q=2, h_kv=2, head_dim=8, dtype="bf16", seed=15)
    two = make_custom([300], grid_res=32, topk=4, h_q=2, h_kv=2, head_dim=8, dtype="bf16", seed=15)
    for name in ("coords", "q", "k", "v", "gates"):
        setattr(two, name, np.concatenate([getattr(one, name)] * 2))
    two.cu_seqlens = np.array([0, 300, 600], np.int32)
    r1 = oracle.forward(one)
    r2 = oracle.forward(two)
    np.testing.assert_array_equal(r2["out"][:300], r1["out"])
    np.testing.assert_array_equal(r2["out"][300:], r1["out"])
    nb = r1["blocks"].nb
    np.testing.assert_array_equal(r2["topk"][300:], r1["topk"] + nb)


# ---------------------------------------------------------------- geometric routing

@pytest.mark.parametrize("seed", [0, 1, 2])
def test_geometric_routing_brute_force(seed):
    # every block's distance from scipy's pairwise distances, ranked with the
    # block id as the tie break
    from scipy.spatial.distance import cdist
    rng = np.random.default_rng(seed)
    coords = rng.integers(0, 24, size=(300, 3)).astype(np.int32)
    b = oracle.build_blocks(coords, [0, 300], 32, 4, 8)
    dist = cdist(coords.astype(np.float64), coords.astype(np.float64), "sqeuclidean")
    blk_of = np.empty(300, np.int64)
    for j in range(b.nb):
        blk_of[b.perm[b.blk_off[j]:b.blk_off[j + 1]]] = j
    for t in rng.integers(0, 300, size=40):
        per_block = np.full(b.nb, np.inf)
        np.minimum.at(per_block, blk_of, dist[t])
        expect = sorted(range(b.nb), key=lambda j: (per_block[j], j))[:7]
        got = oracle.geometric_topk(coords, b, int(t), 0, b.nb, 7)
        assert got.tolist() == expect
        assert got[0] == blk_of[t]          # the query's own block is nearest (distance 0)


def test_geometric_routing_is_translation_invariant():
    rng = np.random.default_rng(4)
    coords = rng.integers(0, 16, size=(200, 3)).astype(np.int32)
    a = oracle.build_blocks(coords, [0, 200], 32, 4, 8)
    moved = coords + np.array([8, 16, 8], np.int32)
    c = oracle.build_blocks(moved, [0, 200], 32, 4, 8)
    for t in range(0, 200, 7):
        assert np.array_equal(oracle.geometric_topk(coords, a, t, 0, a.nb, 5),
                              oracle.geometric_topk(moved, c, t, 0, c.nb, 5))


def test_geometric_routing_forward_uses_the_nearest_blocks():
    wl = make_custom([400, 150], grid_res=32, topk=3, h_q=2, h_kv=1, head_dim=8, dtype="f32", seed=5,
                     routing="geometric")
    res = oracle.forward(wl, with_branches=True)
    b = res["blocks"]
    for t in (0, 77, 399, 549):
        seq = 0 if t < 400 else 1
        j0, j1 = int(b.seq_blk_off[seq]), int(b.seq_blk_off[seq + 1])
        chosen = oracle.geometric_topk(wl.coords, b, t, j0, j1, 3) + j0
        assert res["topk"][t, 0].tolist() == chosen.tolist()
        toks = np.concatenate([b.perm[b.blk_off[j]:b.blk_off[j + 1]] for j in chosen])
        for h in range(2):
            np.testing.assert_allclose(res["o_sel"][t, h], _dense(wl.q[t:t + 1, h], wl.k[toks, 0], wl.v[toks, 0])[0],
                                       rtol=1e-10, atol=1e-12)
