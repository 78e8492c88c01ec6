"""Pins of the oracle's backward pass (gradients of the SSA output with
respect to Q, K, V and the gates, the top-k choice held fixed).

Pinned against: central finite differences of the oracle's own forward
(float64, no rounding), one input at a time; torch autograd of float64 dense
attention where every branch reduces to it (m_cmp = 1, k >= blocks, one window
covering the grid); and two closed forms that hold at any size: the softmax is
unchanged when every key of a sequence moves by the same vector, so the key
gradients of a sequence sum to zero, and every branch output moves by c when
every value of a sequence moves by c, so the value gradients of a sequence sum
to the gate-weighted output gradients (Direct3D-S2 page, "Method": the three
branches and their gated sum).
"""
import numpy as np
import pytest
import torch

import oracle
from workloads import make_custom


def _tiny(seed, seqs=(40, 0, 25), h_q=4, h_kv=2, d=8, topk=3):
    wl = make_custom(list(seqs), grid_res=16, n_prims=2, m_cmp=2, m_win=4, topk=topk, h_q=h_q,
                     h_kv=h_kv, head_dim=d, dtype="f32", seed=seed)
    wl.dtype = "f64"   # exact: no rounding of the pooled rows or the output
    return wl


def _loss_and_topk(wl, dout, blocks):
    res = oracle.forward(wl, blocks=blocks)
    return float((res["out_exact"] * dout).sum()), res["topk"]


@pytest.mark.parametrize("seed,h_q,h_kv", [(3, 4, 2), (4, 2, 2), (5, 4, 1)])
def test_gradients_match_finite_differences(seed, h_q, h_kv):
    wl = _tiny(seed, h_q=h_q, h_kv=h_kv)
    rng = np.random.default_rng(seed)
    dout = rng.standard_normal(wl.q.shape)
    blocks = oracle.build_blocks(wl.coords, wl.cu_seqlens, wl.grid_res, wl.m_cmp, wl.m_win)
    grads = oracle.backward(wl, dout, blocks=blocks)
    _, topk0 = _loss_and_topk(wl, dout, blocks)
    eps = 1e-5
    for name, gname in (("q", "dq"), ("k", "dk"), ("v", "dv"), ("gates", "dgates")):
        x0 = getattr(wl, name).astype(np.float64)
        delta = rng.standard_normal(x0.shape)
        lp, lm = [], []
        for sgn, acc in ((1.0, lp), (-1.0, lm)):
            setattr(wl, name, x0 + sgn * eps * delta)
            loss, topk = _loss_and_topk(wl, dout, blocks)
            assert np.array_equal(topk, topk0), "the perturbation changed the selection"
            acc.append(loss)
        setattr(wl, name, x0)
        fd = (lp[0] - lm[0]) / (2 * eps)
        an = float((grads[gname] * delta).sum())
        assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), f"{name}: finite difference {fd} vs {an}"


def _dense_grads(q, k, v, gsum, dout):
    """torch autograd of sum_h gsum[:, h] * softmax attention, float64."""
    t = lambda a: torch.tensor(np.asarray(a, dtype=np.float64), requires_grad=True)
    q_, k_, v_ = t(q), t(k), t(v)
    H, G = q.shape[1], q.shape[1] // k.shape[1]
    outs = []
    for h in range(H):
        o = torch.nn.functional.scaled_dot_product_attention(q_[None, None, :, h], k_[None, None, :, h // G],
                                                            v_[None, None, :, h // G])[0, 0]
        outs.append(o)
    o = torch.stack(outs, 1)
    (o * torch.from_numpy(gsum)[..., None] * torch.from_numpy(dout)).sum().backward()
    return q_.grad.numpy(), k_.grad.numpy(), v_.grad.numpy(), o.detach().numpy()


@pytest.mark.parametrize("seed,h_q,h_kv", [(0, 2, 2), (1, 4, 2)])
def test_every_branch_reduces_to_dense_attention_gradients(seed, h_q, h_kv):
    rng = np.random.default_rng(seed)
    R, n = 16, 120
    lin = rng.choice(R ** 3, size=n, replace=False)       # one token per voxel block
    coords = np.stack(np.unravel_index(lin, (R,) * 3), -1)
    wl = make_custom(None, coords=coords, grid_res=R, m_cmp=1, m_win=R, topk=n, h_q=h_q, h_kv=h_kv,
                     head_dim=8, dtype="f32", seed=seed)
    wl.dtype = "f64"
    dout = rng.standard_normal(wl.q.shape)
    got = oracle.backward(wl, dout)
    gsum = wl.gates.astype(np.float64).sum(-1)
    dq, dk, dv, o = _dense_grads(wl.q, wl.k, wl.v, gsum, dout)
    np.testing.assert_allclose(got["dq"], dq, rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(got["dk"], dk, rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(got["dv"], dv, rtol=1e-9, atol=1e-11)
    ref_dg = np.repeat(((dout * o).sum(-1))[..., None], 3, axis=-1)
    np.testing.assert_allclose(got["dgates"], ref_dg, rtol=1e-9, atol=1e-11)


def test_sequence_sums_of_key_and_value_gradients():
    wl = make_custom([300, 7, 180], grid_res=32, n_prims=2, topk=4, h_q=4, h_kv=2, head_dim=8,
                     dtype="bf16", seed=11)
    rng = np.random.default_rng(11)
    dout = rng.standard_normal(wl.q.shape)
    got = oracle.backward(wl, dout)
    G = wl.h_q // wl.h_kv
    gw = wl.gates.astype(np.float64).sum(-1)[..., None] * dout    # [N, H, D]
    for b in range(wl.batch):
        sl = slice(wl.cu_seqlens[b], wl.cu_seqlens[b + 1])
        for g in range(wl.h_kv):
            np.testing.assert_allclose(got["dk"][sl, g].sum(0), 0.0, atol=1e-10)
            expect = gw[sl, g * G:(g + 1) * G].sum((0, 1))
            np.testing.assert_allclose(got["dv"][sl, g].sum(0), expect, rtol=1e-10, atol=1e-10)


def test_row_subset_gives_the_same_rows():
    wl = _tiny(9)
    dout = np.random.default_rng(9).standard_normal(wl.q.shape)
    full = oracle.backward(wl, dout)
    rows = [(0, 1), (17, 3), (wl.n_tokens - 1, 0)]
    part = oracle.backward(wl, dout, rows=rows)
    for r, (t, h) in enumerate(rows):
        np.testing.assert_array_equal(part["dq"][r], full["dq"][t, h])
        np.testing.assert_array_equal(part["dgates"][r], full["dgates"][t, h])


def test_zero_output_gradient_gives_zero_gradients():
    wl = _tiny(2)
    got = oracle.backward(wl, np.zeros(wl.q.shape))
    for name in ("dq", "dk", "dv", "dgates"):
        assert not got[name].any()
