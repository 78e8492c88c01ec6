"""Helpers shared by the GPU parity tests: move seeded workloads to the GPU,
run the library through its C ABI, and compare with the CPU oracle.

Tolerances (the stated parity bar for this path):
  * block build: bit-exact;
  * top-k: the selected set equals the oracle's for >= 99.9 % of (token, KV
    group) pairs, and every mismatch has a score gap ln S(b_k) - ln S(a)
    below 1e-3, where b_k is the oracle's k-th block and a the lowest-scored
    block only the GPU chose;
  * output: max |dO| <= 2e-2 and mean |dO| <= 2e-3 against the float64
    oracle's unrounded output.  The library rounds its float32 result once to
    the output dtype, which alone moves a bfloat16 value by up to half a unit
    in its last place: 2^-6 for 4 <= |O| < 8, 2^-5 from 8 up.  So the bar per
    entry is max(2e-2, ulp/2 + 4e-3), the 4e-3 covering the float32
    accumulation; it is 2e-2 everywhere below |O| = 8;
  * each branch alone (one-hot gates): ||do_x||_2 / ||o_x||_2 <= 1e-2.

With SSA_PARITY_LOG set to a file path, every check appends one JSON line
with what it measured (agreement, worst gap, errors), so the figures of a run
are kept.
"""
from __future__ import annotations

import json
import os

import numpy as np
import torch

import oracle
import spatial_sparse_attention_ssa_amd as ssa

DEV = torch.device("cuda:0")
MAX_ABS, MEAN_ABS, BRANCH_REL = 2e-2, 2e-3, 1e-2
ACC_ABS = 4e-3
TOPK_AGREE, TOPK_GAP = 0.999, 1e-3


def torch_dtype(wl):
    return torch.bfloat16 if wl.dtype == "bf16" else torch.float32


def to_dev(a, dtype):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV).to(dtype)


def gpu_build(wl, sync=True):
    return ssa.build_blocks(to_dev(wl.coords, torch.int32), to_dev(wl.cu_seqlens, torch.int32),
                            wl.grid_res, wl.m_cmp, wl.m_win, sync=sync, win_shift=wl.win_shift)


def oracle_blocks(wl):
    return oracle.build_blocks(wl.coords, wl.cu_seqlens, wl.grid_res, wl.m_cmp, wl.m_win, wl.win_shift)


def gpu_forward(wl, blocks, gates=None, **kw):
    dt = torch_dtype(wl)
    g = wl.gates if gates is None else gates
    kw.setdefault("routing", wl.routing)
    return ssa.forward(blocks, to_dev(wl.q, dt), to_dev(wl.k, dt), to_dev(wl.v, dt), to_dev(g, dt),
                       wl.topk, **kw)


def host(t):
    return t.float().cpu().numpy().astype(np.float64) if t.is_floating_point() else t.cpu().numpy()


def check_build(gblocks, ob):
    h = gblocks.trimmed()
    assert h["counts"][0] == ob.nb and h["counts"][1] == ob.nw
    assert np.array_equal(h["perm"].numpy(), ob.perm)
    for name in ("blk_off", "win_off", "win_blk_off", "seq_blk_off", "seq_win_off"):
        assert np.array_equal(h[name].numpy(), getattr(ob, name)), name
    if ob.nb:
        assert h["counts"][3] == int(np.diff(ob.blk_off).max())
        assert h["counts"][4] == int(np.diff(ob.win_off).max())


def bf16_ulp(x):
    """Unit in the last place of bfloat16 values of magnitude |x| (8
    significant bits)."""
    e = np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** -126)))
    return 2.0 ** (e - 7)


def check_outputs(got, ref_exact, what="out", dtype="bf16"):
    """got: the library's output (rounded to its dtype); ref_exact: the
    oracle's unrounded float64 output."""
    err = np.abs(got - ref_exact)
    if dtype == "bf16":
        tol = np.maximum(MAX_ABS, 0.5 * bf16_ulp(np.maximum(np.abs(got), np.abs(ref_exact))) + ACC_ABS)
    else:
        tol = MAX_ABS
    bad = err > tol
    assert not bad.any(), f"{what}: |err| {err[bad].max():.3e} above the bar at {int(bad.sum())} entries"
    assert err.mean() <= MEAN_ABS, f"{what}: mean |err| {err.mean():.3e}"
    return float(err.max()), float(err.mean())


def check_branch(got, ref, what):
    rel = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)
    assert rel <= BRANCH_REL, f"{what}: relative L2 error {rel:.3e}"
    return float(rel)


def record(kind, **fields):
    """Append one JSON line of measured parity figures to $SSA_PARITY_LOG."""
    path = os.environ.get("SSA_PARITY_LOG")
    if not path:
        return
    with open(path, "a") as fh:
        fh.write(json.dumps(dict(kind=kind, **fields)) + "\n")


def topk_agreement(gpu_sel, ref_sel, scores, firsts):
    """gpu_sel/ref_sel: [R, k] global block ids (-1 padded); scores: per-row
    oracle scores over the row's sequence blocks; firsts: first block id."""
    n_rows = len(ref_sel)
    mismatches, worst_gap = 0, 0.0
    for r in range(n_rows):
        g = [int(x) for x in gpu_sel[r] if x >= 0]
        o = [int(x) for x in ref_sel[r] if x >= 0]
        assert len(g) == len(o), f"row {r}: {len(g)} selected on GPU vs {len(o)} in the oracle"
        assert len(set(g)) == len(g), f"row {r}: duplicate selection {g}"
        if set(g) == set(o):
            continue
        mismatches += 1
        s = scores[r]
        j0 = firsts[r]
        assert all(0 <= x - j0 < len(s) for x in g), f"row {r}: selection outside its sequence"
        only_gpu = [x for x in g if x not in o]
        a = min(only_gpu, key=lambda x: s[x - j0])
        gap = np.log(max(s[o[-1] - j0], 1e-300)) - np.log(max(s[a - j0], 1e-300))
        worst_gap = max(worst_gap, gap)
    agree = 1.0 - mismatches / max(n_rows, 1)
    return agree, float(worst_gap)


def check_topk(gpu_sel, ref_sel, scores, firsts, min_agree=TOPK_AGREE):
    agree, gap = topk_agreement(gpu_sel, ref_sel, scores, firsts)
    assert agree >= min_agree, f"top-k agreement {agree:.5f}"
    assert gap < TOPK_GAP, f"top-k mismatch with score gap {gap:.3e}"
    return agree, gap


def sample_rows(wl, n_rows, seed=0):
    rng = np.random.default_rng(seed)
    t = rng.integers(0, wl.n_tokens, size=n_rows)
    h = rng.integers(0, wl.h_q, size=n_rows)
    t[:2] = [0, wl.n_tokens - 1]
    return list(zip(t.tolist(), h.tolist()))


def one_hot_gates(wl, branch):
    g = np.zeros_like(wl.gates)
    g[..., branch] = 1.0
    return g
