"""GPU SSA backward vs the float64 oracle on the same seeded inputs.

The forward runs in its training form (it also saves each branch's
log-sum-exp), then the backward gives dq, dk, dv and dgates for a seeded
output gradient.  Small workloads and the whole 16384-token workload are
compared element by element against oracle.backward.  On the varlen workload
every gradient of its shortest sequence is compared element by element (the
oracle runs that sequence alone: sequences never interact), and dq / dgates
on sampled rows of all sequences; the grouped-head workload is compared on
sampled rows for dq and dgates.  On both, the key / value gradients are also
checked through two closed forms that hold at any size (Direct3D-S2 page,
"Method": the softmax of every branch is unchanged when all keys of a
sequence move together, and every branch output moves with a common shift of
the values).

Bar: relative L2 error of each gradient tensor <= 1e-2 for bfloat16 (1e-4
for float32 storage), and max |error| <= 5 % of the tensor's largest
reference value.  The gradients are computed with the selection fixed, so
each case first checks that the GPU selected the same blocks as the oracle.
"""
import copy

import numpy as np
import pytest
import torch

import oracle
import spatial_sparse_attention_ssa_amd as ssa
from oracle import parallel as oracle_pool
from tests import _parity as P
from workloads import make_custom, make_workload

pytestmark = pytest.mark.gpu

REL = {"bf16": 1e-2, "f32": 1e-4}
MAX_FRAC = 5e-2


def _dout(wl, seed):
    rng = np.random.default_rng(seed)
    d = rng.standard_normal(wl.q.shape).astype(np.float32)
    if wl.dtype == "bf16":
        d = torch.from_numpy(d).to(torch.bfloat16).float().numpy()
    return d


def _gpu_grads(wl, gb, dout, gates=None):
    dt = P.torch_dtype(wl)
    q, k, v = P.to_dev(wl.q, dt), P.to_dev(wl.k, dt), P.to_dev(wl.v, dt)
    g = P.to_dev(wl.gates if gates is None else gates, dt)
    saved = ssa.forward_train(gb, q, k, v, g, wl.topk, routing=wl.routing)
    grads = ssa.backward(gb, q, k, v, g, saved, P.to_dev(dout, dt))
    return saved, grads


def _compare(name, got, ref, dtype):
    rel = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)
    mx = np.abs(got - ref).max() / max(np.abs(ref).max(), 1e-30)
    assert rel <= REL[dtype], f"{name}: relative L2 error {rel:.3e}"
    assert mx <= MAX_FRAC, f"{name}: max error {mx:.3e} of the largest value"
    return rel


def _full_compare(wl, seed, one_hot=False):
    ob = P.oracle_blocks(wl)
    gb = P.gpu_build(wl)
    dout = _dout(wl, seed)
    ref_fwd = oracle.forward(wl, blocks=ob)
    gate_sets = [None] + ([P.one_hot_gates(wl, i) for i in range(3)] if one_hot else [])
    for gates in gate_sets:
        saved, grads = _gpu_grads(wl, gb, dout, gates)
        sel = np.sort(saved["topk"].cpu().numpy(), axis=-1)
        assert np.array_equal(sel, np.sort(ref_fwd["topk"], axis=-1)), "selection differs from the oracle's"
        w2 = wl
        if gates is not None:
            w2 = copy.copy(wl)
            w2.gates = gates
        ref = oracle.backward(w2, dout, blocks=ob)
        tag = "gates" if gates is None else f"one-hot {int(np.argmax(gates[0, 0]))}"
        rels = {nm: _compare(f"{nm} ({tag})", P.host(grads[nm]), ref[nm], wl.dtype)
                for nm in ("dq", "dk", "dv", "dgates")}
        print(tag, {k2: f"{v2:.2e}" for k2, v2 in rels.items()})


@pytest.mark.parametrize("case", [
    dict(seqs=[700, 0, 433], h_q=4, h_kv=4, head_dim=64, topk=8, dtype="bf16"),
    dict(seqs=[600, 257], h_q=16, h_kv=1, head_dim=32, topk=8, dtype="bf16"),
    dict(seqs=[500, 300], h_q=4, h_kv=2, head_dim=32, topk=4, dtype="bf16"),
    dict(seqs=[400], h_q=2, h_kv=2, head_dim=32, topk=4, dtype="f32"),
    dict(seqs=[350, 90], h_q=32, h_kv=2, head_dim=64, topk=16, dtype="bf16"),
    dict(seqs=[900, 0, 300], h_q=4, h_kv=4, head_dim=64, topk=24, dtype="bf16"),
    dict(seqs=[800, 450], h_q=4, h_kv=4, head_dim=32, topk=20, dtype="bf16"),
    dict(seqs=[700, 0, 433], h_q=4, h_kv=4, head_dim=32, topk=8, dtype="bf16"),
    dict(seqs=[600, 257], h_q=8, h_kv=1, head_dim=64, topk=8, dtype="bf16"),
])
def test_small_backward_full(case):
    wl = make_custom(case["seqs"], grid_res=64, n_prims=3, topk=case["topk"], h_q=case["h_q"],
                     h_kv=case["h_kv"], head_dim=case["head_dim"], dtype=case["dtype"], seed=23)
    _full_compare(wl, seed=5, one_hot=case["h_q"] == 4 and case["h_kv"] == 4)


def test_shifted_windows_backward_full():
    wl = make_custom([800, 333], grid_res=64, n_prims=3, topk=8, h_q=4, h_kv=4, head_dim=64,
                     dtype="bf16", seed=29, win_shift=4)
    _full_compare(wl, seed=6)


def test_large_windows_backward_full():
    # 2900 of the 4096 voxels of a 16^3 grid: eight windows of about 360 tokens
    from tests.test_gpu_forward import dense_cube
    wl = make_custom(None, coords=dense_cube(2900, 16, 11), grid_res=16, m_cmp=4, m_win=8, topk=8, h_q=4, h_kv=4,
                     head_dim=64, dtype="bf16", seed=13)
    _full_compare(wl, seed=8)


def many_sequences(lengths, seed):
    """A varlen batch of the given sequence lengths, each sequence a set of
    distinct random voxels of a 64^3 grid."""
    rng = np.random.default_rng(seed)
    lens = np.asarray(lengths, dtype=np.int64)
    lin = rng.choice(64 ** 3, size=int(lens.sum()), replace=False)
    coords = np.stack(np.unravel_index(lin, (64,) * 3), -1)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    return make_custom(None, coords=coords, cu_seqlens=cu, grid_res=64, m_cmp=4, m_win=8, topk=4, h_q=4, h_kv=4,
                       head_dim=64, dtype="bf16", seed=seed)


@pytest.mark.parametrize("n_seq", [40, 1100])
def test_many_sequences_backward_full(n_seq):
    # 40 sequences with repeated lengths (ties in the longest-first chunk
    # order of the pooled-row gradients), and 1100, past the 1024 sequences
    # that are put in cost order
    rng = np.random.default_rng(n_seq)
    lengths = rng.choice([7, 7, 13, 30, 30, 64], size=n_seq) if n_seq < 1024 else rng.choice([1, 2, 3, 5], size=n_seq)
    _full_compare(many_sequences(lengths, seed=41), seed=9)


def test_geometric_routing_backward_full():
    wl = make_custom([700, 300], grid_res=64, n_prims=3, topk=8, h_q=4, h_kv=4, head_dim=64,
                     dtype="bf16", seed=31, routing="geometric")
    _full_compare(wl, seed=7)


def test_zero_output_gradient():
    wl = make_custom([600, 200], grid_res=64, n_prims=3, topk=8, h_q=4, h_kv=4, head_dim=64,
                     dtype="bf16", seed=3)
    gb = P.gpu_build(wl)
    _, grads = _gpu_grads(wl, gb, np.zeros(wl.q.shape, np.float32))
    for nm in ("dq", "dk", "dv", "dgates"):
        assert not grads[nm].float().abs().max().item(), nm


def test_backward_run_to_run_bit_identical():
    wl = make_workload(2)
    gb = P.gpu_build(wl)
    dout = _dout(wl, 2)
    _, a = _gpu_grads(wl, gb, dout)
    _, b = _gpu_grads(wl, gb, dout)
    for nm in ("dq", "dk", "dv", "dgates"):
        assert torch.equal(a[nm], b[nm]), nm


def _sequence_sums(wl, grads, dout):
    """sum_t dK[t, g] = 0 and sum_t dV[t, g] = sum_{t, h in g} (G0 + G1 + G2) dO,
    per sequence and group, relative to the size of the summands."""
    dk, dv = P.host(grads["dk"]), P.host(grads["dv"])
    G = wl.h_q // wl.h_kv
    gw = wl.gates.astype(np.float64).sum(-1)[..., None] * dout
    worst = 0.0
    for b in range(wl.batch):
        sl = slice(wl.cu_seqlens[b], wl.cu_seqlens[b + 1])
        if sl.stop == sl.start:
            continue
        for g in range(wl.h_kv):
            ek = np.abs(dk[sl, g].sum(0)) / np.linalg.norm(dk[sl, g], axis=0)
            expect = gw[sl, g * G:(g + 1) * G].sum((0, 1))
            ev = np.abs(dv[sl, g].sum(0) - expect) / np.linalg.norm(dv[sl, g], axis=0)
            worst = max(worst, ek.max(), ev.max())
    return worst


def _selection_agreement(saved_topk, ref_topk, G, rows=None):
    """share of (token, group) selections equal as sets; ref_topk is
    [N, Hkv, k] (or [len(rows), k] with rows)"""
    sel = np.sort(saved_topk.cpu().numpy(), axis=-1)
    if rows is None:
        return float((sel == np.sort(ref_topk, axis=-1)).all(-1).mean())
    got = sel[[t for t, _ in rows], [h // G for _, h in rows]]
    return float((got == np.sort(ref_topk, axis=-1)).all(-1).mean())


def test_workload2_backward_full():
    # every gradient entry of the 16384-token workload (multi-tile MFMA paths,
    # real inverted top-k lists), the oracle over worker processes
    wl = make_workload(2)
    ob = P.oracle_blocks(wl)
    gb = P.gpu_build(wl)
    dout = _dout(wl, 2)
    saved, grads = _gpu_grads(wl, gb, dout)
    torch.cuda.synchronize()
    fwd = oracle_pool.forward_rows(wl, ob, [(t, g) for t in range(wl.n_tokens) for g in range(wl.h_kv)])
    agree = _selection_agreement(saved["topk"], fwd["topk"].reshape(wl.n_tokens, wl.h_kv, -1), 1)
    assert agree >= P.TOPK_AGREE, f"selection agrees on only {agree:.5f} of (token, group) pairs"
    ref = oracle_pool.backward_full(wl, dout, ob)
    rels = {nm: _compare(nm, P.host(grads[nm]), ref[nm], wl.dtype) for nm in ("dq", "dk", "dv", "dgates")}
    P.record("backward_full", tag="workload 2", n_tokens=wl.n_tokens, selection_agree=agree, rel_l2=rels)
    print("workload 2:", agree, {k2: f"{v2:.2e}" for k2, v2 in rels.items()})


def _subsequence(wl, b, dout):
    """Sequence b of a varlen workload as a workload of its own (and its slice
    of the output gradient)."""
    s, e = int(wl.cu_seqlens[b]), int(wl.cu_seqlens[b + 1])
    sub = copy.copy(wl)
    sub.coords = wl.coords[s:e]
    sub.cu_seqlens = np.array([0, e - s], dtype=np.int32)
    sub.q, sub.k, sub.v, sub.gates = wl.q[s:e], wl.k[s:e], wl.v[s:e], wl.gates[s:e]
    return sub, dout[s:e], slice(s, e)


@pytest.mark.parametrize("cfg,n_rows", [(5, 2000), (4, 1000)])
def test_large_workload_backward(cfg, n_rows):
    wl = make_workload(cfg)
    print(f"workload {cfg}: N={wl.n_tokens}", flush=True)
    ob = P.oracle_blocks(wl)
    gb = P.gpu_build(wl)
    dout = _dout(wl, cfg)
    saved, grads = _gpu_grads(wl, gb, dout)
    torch.cuda.synchronize()
    rows = P.sample_rows(wl, n_rows, seed=cfg)
    G = wl.h_q // wl.h_kv
    fwd = oracle_pool.forward_rows(wl, ob, rows)
    same = np.sort(saved["topk"].cpu().numpy(), axis=-1)[[t for t, _ in rows], [h // G for _, h in rows]] \
        == np.sort(fwd["topk"], axis=-1)
    same = same.all(-1)
    agree = float(same.mean())
    assert agree >= P.TOPK_AGREE, f"selection agrees on only {agree:.5f} of the rows"
    ref = oracle_pool.backward_rows(wl, dout, ob, rows)
    rr = np.flatnonzero(same)
    tt = [rows[r][0] for r in rr]
    hh = [rows[r][1] for r in rr]
    rels = {nm: _compare(nm, P.host(grads[nm])[tt, hh], ref[nm][rr], wl.dtype) for nm in ("dq", "dgates")}
    worst = _sequence_sums(wl, grads, dout)
    print(f"workload {cfg}: selection agree {agree:.5f}, sequence-sum residual {worst:.2e}")
    assert worst <= 2e-2, f"sequence sums of dk / dv off by {worst:.3e}"
    if cfg == 5:
        # every gradient of the shortest sequence, element by element
        b = int(np.argmin(np.diff(wl.cu_seqlens)))
        sub, sub_dout, sl = _subsequence(wl, b, dout)
        sob = P.oracle_blocks(sub)
        sfwd = oracle_pool.forward_rows(sub, sob, [(t, g) for t in range(sub.n_tokens) for g in range(sub.h_kv)])
        # the batch numbers blocks globally, the sequence alone from 0
        j0 = int(ob.seq_blk_off[b])
        sel_b = saved["topk"][sl]
        sel_b = torch.where(sel_b >= 0, sel_b - j0, sel_b)
        sagree = _selection_agreement(sel_b, sfwd["topk"].reshape(sub.n_tokens, sub.h_kv, -1), 1)
        assert sagree >= P.TOPK_AGREE, f"sequence {b}: selection agrees on only {sagree:.5f}"
        sref = oracle_pool.backward_full(sub, sub_dout, sob)
        for nm in ("dq", "dk", "dv", "dgates"):
            rels[f"seq{b}_{nm}"] = _compare(f"sequence {b} {nm}", P.host(grads[nm][sl]), sref[nm], wl.dtype)
        print(f"workload 5, sequence {b} ({sub.n_tokens} tokens): selection agree {sagree:.5f}")
    P.record("backward_sampled", tag=f"workload {cfg}", rows=len(rows), selection_agree=agree,
             sequence_sum_residual=worst, rel_l2=rels)
