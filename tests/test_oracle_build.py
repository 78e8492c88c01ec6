"""Pins of the oracle's integer stage (block keys, stable sort, segments).

Pinned against: the hand-worked fixture tests/golden/build_two_seq_dup.json,
an independent brute force (group tokens in a dict by (sequence, window cell,
block cell), order groups lexicographically), and invariants of the partition
(Direct3D-S2 page, "Method": blocking by 3D coordinate, non-overlapping
windows).
"""
import numpy as np
import pytest

import oracle
from tests import _golden


def _random_tokens(rng, n, R, n_seq, dup_frac=0.1):
    coords = rng.integers(0, R, size=(n, 3))
    ndup = int(n * dup_frac)
    if ndup and n > 1:
        src = rng.integers(0, n, size=ndup)
        dst = rng.integers(0, n, size=ndup)
        coords[dst] = coords[src]
    cuts = np.sort(rng.integers(0, n + 1, size=n_seq - 1))
    cu = np.concatenate([[0], cuts, [n]]).astype(np.int32)
    return coords.astype(np.int32), cu


def _brute_force(coords, cu, R, m_cmp, m_win, shift=0):
    """Group by (seq, window cell, block cell) with plain Python; order groups
    by (seq, window cell in x,y,z order, block cell in x,y,z order).  With
    ``shift`` the window cells start at -shift on every axis."""
    groups = {}
    for b in range(len(cu) - 1):
        for t in range(cu[b], cu[b + 1]):
            c = tuple(int(x) for x in coords[t])
            wcell = tuple((x + shift) // m_win for x in c)
            bcell = tuple(x // m_cmp for x in c)
            groups.setdefault((b, wcell, bcell), []).append(t)
    keys = sorted(groups)
    perm = [t for k in keys for t in groups[k]]
    blk_sizes = [len(groups[k]) for k in keys]
    win_of_blk = [(k[0], k[1]) for k in keys]
    return perm, blk_sizes, win_of_blk, [k[0] for k in keys]


def test_golden_two_sequences_with_empty_and_duplicates():
    g = _golden.load("build_two_seq_dup.json")
    key, valid = oracle.block_keys(g["coords"], g["cu_seqlens"], g["grid_res"], g["m_cmp"], g["m_win"])
    assert key.tolist() == g["keys"] and valid.all()
    b = oracle.build_blocks(g["coords"], g["cu_seqlens"], g["grid_res"], g["m_cmp"], g["m_win"])
    for name in ("perm", "blk_off", "win_off", "win_blk_off", "seq_blk_off", "seq_win_off"):
        assert getattr(b, name).tolist() == g[name], name


@pytest.mark.parametrize("seed", range(12))
def test_brute_force_partition(seed):
    rng = np.random.default_rng(seed)
    R = int(rng.choice([8, 16, 32]))
    m_cmp = int(rng.choice([1, 2, 4]))
    m_win = m_cmp * int(rng.choice([1, 2, 4]))
    if m_win > R:
        m_win = R
    n = int(rng.integers(1, 300))
    coords, cu = _random_tokens(rng, n, R, int(rng.integers(1, 5)))
    b = oracle.build_blocks(coords, cu, R, m_cmp, m_win)
    perm, sizes, win_of_blk, seq_of_blk = _brute_force(coords, cu, R, m_cmp, m_win)
    assert b.perm.tolist() == perm
    assert np.diff(b.blk_off).tolist() == sizes
    # windows: consecutive blocks sharing (seq, window cell)
    wstarts = [0] + [j for j in range(1, len(sizes)) if win_of_blk[j] != win_of_blk[j - 1]]
    assert b.win_blk_off.tolist() == wstarts + [len(sizes)]
    assert b.win_off.tolist() == [int(np.sum(sizes[:j])) for j in wstarts] + [n]
    B = len(cu) - 1
    assert b.seq_blk_off.tolist() == [sum(1 for s in seq_of_blk if s < q) for q in range(B + 1)]


@pytest.mark.parametrize("seed", range(8))
def test_brute_force_partition_with_shifted_windows(seed):
    rng = np.random.default_rng(100 + seed)
    R = int(rng.choice([8, 16, 32]))
    m_cmp = int(rng.choice([1, 2, 4]))
    m_win = min(m_cmp * int(rng.choice([2, 4])), R)
    shift = m_cmp * int(rng.integers(1, m_win // m_cmp)) if m_win > m_cmp else 0
    n = int(rng.integers(1, 300))
    coords, cu = _random_tokens(rng, n, R, int(rng.integers(1, 5)))
    b = oracle.build_blocks(coords, cu, R, m_cmp, m_win, shift)
    perm, sizes, win_of_blk, seq_of_blk = _brute_force(coords, cu, R, m_cmp, m_win, shift)
    assert b.perm.tolist() == perm
    assert np.diff(b.blk_off).tolist() == sizes
    wstarts = [0] + [j for j in range(1, len(sizes)) if win_of_blk[j] != win_of_blk[j - 1]]
    assert b.win_blk_off.tolist() == wstarts + [len(sizes)]


def test_shifted_windows_equal_translated_tokens():
    # windows shifted by s on a grid R are the unshifted windows of the tokens
    # moved by +s on a grid large enough to hold them; blocks do not move
    rng = np.random.default_rng(9)
    coords, cu = _random_tokens(rng, 400, 32, 3)
    a = oracle.build_blocks(coords, cu, 32, 4, 8, 4)
    t = oracle.build_blocks(coords + 4, cu, 64, 4, 8, 0)
    for name in ("perm", "blk_off", "win_off", "win_blk_off", "seq_blk_off", "seq_win_off"):
        assert np.array_equal(getattr(a, name), getattr(t, name)), name
    z = oracle.build_blocks(coords, cu, 32, 4, 8, 0)
    as_sets = lambda bl: sorted(tuple(sorted(bl.perm[bl.blk_off[j]:bl.blk_off[j + 1]])) for j in range(bl.nb))
    assert as_sets(a) == as_sets(z)


def test_bad_shift_is_rejected():
    coords, cu = np.zeros((2, 3), np.int32), [0, 2]
    for shift in (2, 8, -4):
        with pytest.raises(ValueError):
            oracle.build_blocks(coords, cu, 16, 4, 8, shift)


def test_invariants_on_surface_band():
    from workloads import make_workload
    wl = make_workload(2, with_tensors=False)
    b = oracle.build_blocks(wl.coords, wl.cu_seqlens, wl.grid_res, wl.m_cmp, wl.m_win)
    n = wl.n_tokens
    assert sorted(b.perm.tolist()) == list(range(n))                  # a permutation
    assert (np.diff(b.blk_off) > 0).all() and b.blk_off[-1] == n       # non-empty blocks
    assert (np.diff(b.win_off) > 0).all() and b.win_off[-1] == n
    ks = b.key_sorted
    assert (np.diff(ks[b.blk_off[:-1]]) > 0).all()                    # keys strictly increase across blocks
    for j in range(b.nb):                                              # stability inside each block
        seg = b.perm[b.blk_off[j]:b.blk_off[j + 1]]
        assert (np.diff(seg) > 0).all()
        assert (ks[b.blk_off[j]:b.blk_off[j + 1]] == ks[b.blk_off[j]]).all()
    # each window is a run of whole blocks
    assert set(b.win_off.tolist()) <= set(b.blk_off.tolist())
    assert (b.blk_off[b.win_blk_off] == b.win_off).all()
    # every token of a block lies in one m_cmp cell
    c = wl.coords[b.perm] // wl.m_cmp
    for j in range(0, b.nb, 37):
        seg = c[b.blk_off[j]:b.blk_off[j + 1]]
        assert (seg == seg[0]).all()


def test_translation_by_window_multiples_keeps_partition():
    rng = np.random.default_rng(5)
    coords, cu = _random_tokens(rng, 200, 16, 2)
    coords = coords % 8
    b0 = oracle.build_blocks(coords, cu, 32, 2, 8)
    b1 = oracle.build_blocks(coords + np.array([8, 16, 8]), cu, 32, 2, 8)
    for name in ("perm", "blk_off", "win_off", "win_blk_off", "seq_blk_off", "seq_win_off"):
        assert getattr(b0, name).tolist() == getattr(b1, name).tolist()


def test_out_of_range_is_counted():
    coords = np.array([[0, 0, 0], [8, 0, 0], [-1, 2, 2]], np.int32)
    b = oracle.build_blocks(coords, [0, 3], 8, 2, 4)
    assert b.n_invalid == 2


def test_empty_input():
    b = oracle.build_blocks(np.zeros((0, 3), np.int32), [0, 0], 8, 2, 4)
    assert b.nb == 0 and b.nw == 0
    assert b.blk_off.tolist() == [0] and b.seq_blk_off.tolist() == [0, 0]
