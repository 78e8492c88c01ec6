"""GPU block build vs the oracle: bit-exact sort order and segments.

Direct3D-S2 page, "Method": tokens are blocked by 3D coordinate into m_cmp^3
blocks and non-overlapping m_win^3 windows.  Covers every named workload's
geometry plus adversarial inputs (one block, one token per block, duplicates,
empty sequences, no tokens, coordinates out of range).
"""
import types
import zlib

import numpy as np
import pytest
import torch

import oracle
from tests import _parity as P
from workloads import make_custom, make_workload

pytestmark = pytest.mark.gpu


def _oracle_blocks(wl):
    return P.oracle_blocks(wl)


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_named_workload_build_bit_exact(cfg):
    wl = make_workload(cfg, with_tensors=False)
    print(f"build parity: workload {cfg} N={wl.n_tokens} B={wl.batch}", flush=True)
    gb = P.gpu_build(wl)
    P.check_build(gb, _oracle_blocks(wl))


def _custom(coords, cu, R=64, m_cmp=4, m_win=8, win_shift=0):
    return make_custom(None, coords=np.asarray(coords), cu_seqlens=cu, grid_res=R, m_cmp=m_cmp,
                       m_win=m_win, h_q=1, h_kv=1, head_dim=32, win_shift=win_shift)


@pytest.mark.parametrize("case", ["one_block", "voxel_blocks", "duplicates", "empty_seqs",
                                  "many_seqs", "single_token", "one_window"])
def test_adversarial_build(case):
    rng = np.random.default_rng(zlib.crc32(case.encode()))
    if case == "one_block":
        coords = rng.integers(0, 4, size=(5000, 3))
        wl = _custom(coords, [0, 5000])
    elif case == "voxel_blocks":
        lin = rng.choice(64 ** 3, size=20000, replace=False)
        wl = _custom(np.stack(np.unravel_index(lin, (64,) * 3), -1), [0, 20000], m_cmp=1, m_win=2)
    elif case == "duplicates":
        base = rng.integers(0, 64, size=(300, 3))
        wl = _custom(base[rng.integers(0, 300, size=9000)], [0, 9000])
    elif case == "empty_seqs":
        coords = rng.integers(0, 64, size=(7000, 3))
        wl = _custom(coords, [0, 0, 3000, 3000, 3000, 7000, 7000])
    elif case == "many_seqs":
        coords = rng.integers(0, 32, size=(12000, 3))
        cuts = np.sort(rng.integers(0, 12000, size=99))
        wl = _custom(coords, np.concatenate([[0], cuts, [12000]]), R=32, m_cmp=2, m_win=4)
    elif case == "single_token":
        wl = _custom([[5, 6, 7]], [0, 1])
    else:
        coords = rng.integers(0, 16, size=(4097, 3))
        wl = _custom(coords, [0, 4097], R=16, m_cmp=4, m_win=16)
    gb = P.gpu_build(wl)
    P.check_build(gb, _oracle_blocks(wl))


@pytest.mark.parametrize("R,m_cmp,m_win,shift", [(64, 4, 8, 4), (32, 2, 8, 2), (32, 2, 8, 6), (1024, 4, 8, 4)])
def test_shifted_window_build_bit_exact(R, m_cmp, m_win, shift):
    rng = np.random.default_rng(R + shift)
    n = 20000
    coords = rng.integers(0, R, size=(n, 3))
    cuts = np.sort(rng.integers(0, n, size=3))
    wl = _custom(coords, np.concatenate([[0], cuts, [n]]), R=R, m_cmp=m_cmp, m_win=m_win, win_shift=shift)
    gb = P.gpu_build(wl)
    P.check_build(gb, _oracle_blocks(wl))


def test_shifted_window_build_of_the_headline_geometry():
    wl = make_workload(3, with_tensors=False)
    wl.win_shift = wl.m_win // 2
    gb = P.gpu_build(wl)
    P.check_build(gb, _oracle_blocks(wl))


def test_empty_token_set():
    wl = _custom(np.zeros((0, 3), np.int64), [0, 0, 0])
    gb = P.gpu_build(wl)
    h = gb.trimmed()
    assert h["counts"][0] == 0 and h["counts"][1] == 0
    assert h["seq_blk_off"].tolist() == [0, 0, 0]


def test_async_build_matches_synced():
    wl = make_workload(2, with_tensors=False)
    g1 = P.gpu_build(wl, sync=True)
    g2 = P.gpu_build(wl, sync=False)
    assert g2.nb == -1
    torch.cuda.synchronize()
    a, b = g1.trimmed(), g2.trimmed()
    for name in ("perm", "blk_off", "win_off", "win_blk_off", "seq_blk_off", "seq_win_off"):
        assert torch.equal(a[name], b[name])


def test_out_of_range_coordinates_are_rejected_when_synced():
    import spatial_sparse_attention_ssa_amd as ssa
    coords = np.array([[0, 0, 0], [64, 1, 1], [3, -2, 5]], np.int32)
    wl = _custom(coords, [0, 3])
    with pytest.raises(ssa.SsaError) as e:
        P.gpu_build(wl)
    assert e.value.status == 1
    gb = P.gpu_build(wl, sync=False)
    torch.cuda.synchronize()
    assert gb.counts.cpu().tolist()[2] == 2


@pytest.mark.parametrize("lg", [20, 22])
def test_large_random_build_bit_exact(lg):
    """2^20 and 2^22 uniformly random voxels of a 1024^3 grid (duplicates
    included) in three sequences: the multi-workgroup histogram scan and the
    LDS-staged scatter at the sizes where they take over, nearly one token
    per block."""
    n = 1 << lg
    rng = np.random.default_rng(lg)
    coords = rng.integers(0, 1024, size=(n, 3))
    cu = np.array([0, n // 3, n // 3 + 17, n], dtype=np.int32)
    # the build needs only the geometry (no tensors at this size)
    wl = types.SimpleNamespace(coords=coords.astype(np.int32), cu_seqlens=cu, grid_res=1024, m_cmp=4, m_win=8,
                               win_shift=0)
    print(f"large random build: N={n}", flush=True)
    gb = P.gpu_build(wl)
    P.check_build(gb, _oracle_blocks(wl))
