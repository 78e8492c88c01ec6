"""Direct pins of the oracle's per-row primitives, each against something
other than itself: softmax attention against torch's float64
scaled_dot_product_attention (with its scale argument) and against a shift of
every logit; its gradient against torch autograd of the same library call and
against the identities sum_j ds_j = 0 and sum_j dv_j = do; the pooled-row
gradient's share against the mean's derivative checked by finite differences
of oracle.pool_blocks (Direct3D-S2 page, "Method": compression by mean
pooling, softmax attention in every branch).
"""
import numpy as np
import pytest
import torch

import oracle
from workloads import make_custom


def _lib_attention(q, k, v, scale):
    t = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float64))
    return torch.nn.functional.scaled_dot_product_attention(t(q)[None, None, None], t(k)[None, None],
                                                            t(v)[None, None], scale=scale)[0, 0, 0].numpy()


@pytest.mark.parametrize("n,d,scale", [(1, 4, 0.5), (7, 16, 0.25), (40, 64, 0.125), (300, 32, 1.7)])
def test_softmax_attention_matches_library(n, d, scale):
    rng = np.random.default_rng(n * 100 + d)
    q, k, v = rng.standard_normal(d), rng.standard_normal((n, d)), rng.standard_normal((n, d))
    o, p = oracle.softmax_attention(q, k, v, scale)
    np.testing.assert_allclose(o, _lib_attention(q, k, v, scale), rtol=1e-12, atol=1e-12)
    assert abs(p.sum() - 1.0) < 1e-12 and (p >= 0).all()


def test_softmax_attention_is_shift_invariant_and_handles_large_logits():
    rng = np.random.default_rng(5)
    q, k, v = rng.standard_normal(8), rng.standard_normal((12, 8)), rng.standard_normal((12, 8))
    # adding the same vector c to every key moves every logit by q . c
    o1, p1 = oracle.softmax_attention(q, k, v, 0.3)
    o2, p2 = oracle.softmax_attention(q, k + 50.0 * q, v, 0.3)
    np.testing.assert_allclose(p1, p2, rtol=1e-10, atol=1e-14)
    np.testing.assert_allclose(o1, o2, rtol=1e-10, atol=1e-12)
    # logits of 1e4 would overflow without the subtracted maximum
    o3, p3 = oracle.softmax_attention(q * 1e3, k, v, 10.0)
    assert np.isfinite(o3).all() and abs(p3.sum() - 1.0) < 1e-12


@pytest.mark.parametrize("n,d,scale", [(1, 4, 0.5), (9, 16, 0.25), (33, 64, 0.125)])
def test_softmax_attention_grad_matches_autograd(n, d, scale):
    rng = np.random.default_rng(7 * n + d)
    q, k, v, do = (rng.standard_normal(d), rng.standard_normal((n, d)), rng.standard_normal((n, d)),
                   rng.standard_normal(d))
    dq, dk, dv, o = oracle.softmax_attention_grad(q, k, v, do, scale)
    tq, tk, tv = (torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (q, k, v))
    to = torch.nn.functional.scaled_dot_product_attention(tq[None, None, None], tk[None, None], tv[None, None],
                                                          scale=scale)[0, 0, 0]
    (to * torch.from_numpy(do)).sum().backward()
    np.testing.assert_allclose(o, to.detach().numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=1e-10, atol=1e-12)
    # identities: the logit gradients sum to zero (so sum_j dk_j = 0) and the
    # value gradients sum to do (the probabilities sum to one)
    np.testing.assert_allclose(dk.sum(0), 0.0, atol=1e-12)
    np.testing.assert_allclose(dv.sum(0), do, rtol=1e-12, atol=1e-12)


def test_pooled_to_tokens_is_the_derivative_of_the_mean():
    # L = sum_j <G_j, mean of block j's rows>: dL/dx_t = G_j / n_j for the
    # block j holding token t; compared with central differences of
    # oracle.pool_blocks (float64, no rounding) on a few tokens
    wl = make_custom([90, 0, 40], grid_res=16, n_prims=2, topk=4, h_q=2, h_kv=2, head_dim=4, dtype="f32", seed=3)
    ob = oracle.build_blocks(wl.coords, wl.cu_seqlens, wl.grid_res, wl.m_cmp, wl.m_win)
    rng = np.random.default_rng(3)
    x = rng.standard_normal(wl.k.shape)
    gk = rng.standard_normal((ob.nb,) + wl.k.shape[1:])
    gv = rng.standard_normal((ob.nb,) + wl.k.shape[1:])
    dk, dv = oracle.pooled_to_tokens(ob, np.zeros_like(x), np.zeros_like(x), gk, gv)
    loss = lambda a: float((oracle.pool_blocks(a, ob, "f64") * gk).sum())
    eps = 1e-6
    for t in rng.choice(wl.n_tokens, size=12, replace=False):
        for h in range(x.shape[1]):
            for c in range(x.shape[2]):
                xp, xm = x.copy(), x.copy()
                xp[t, h, c] += eps
                xm[t, h, c] -= eps
                num = (loss(xp) - loss(xm)) / (2 * eps)
                assert abs(num - dk[t, h, c]) < 1e-7, (t, h, c, num, dk[t, h, c])
    # the value side takes the same shares: every block's token gradients sum
    # to its pooled row's gradient
    for j in range(ob.nb):
        toks = ob.perm[ob.blk_off[j]:ob.blk_off[j + 1]]
        np.testing.assert_allclose(dv[toks].sum(0), gv[j], rtol=1e-12, atol=1e-12)
