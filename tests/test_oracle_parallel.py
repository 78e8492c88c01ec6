"""The oracle's process-pool driver returns what the serial oracle returns:
the same per-row results, and the same key / value gradient sums up to float64
summation order."""
import numpy as np

import oracle
from oracle import parallel
from workloads import make_custom


def _wl():
    return make_custom([500, 0, 220], grid_res=32, topk=4, h_q=4, h_kv=2, head_dim=32, dtype="bf16", seed=3)


def test_parallel_forward_rows_equal_serial():
    wl = _wl()
    ob = oracle.build_blocks(wl.coords, wl.cu_seqlens, wl.grid_res, wl.m_cmp, wl.m_win)
    rows = [(t, h) for t in range(0, wl.n_tokens, 3) for h in range(wl.h_q)]
    a = oracle.forward_rows(wl, ob, rows, with_branches=True, with_scores=True)
    b = parallel.forward_rows(wl, ob, rows, with_branches=True, with_scores=True, workers=3)
    for name in a:
        if isinstance(a[name], list):
            assert all(np.array_equal(x, y) for x, y in zip(a[name], b[name])), name
        else:
            assert np.array_equal(a[name], b[name]), name


def test_parallel_backward_equals_serial():
    wl = _wl()
    ob = oracle.build_blocks(wl.coords, wl.cu_seqlens, wl.grid_res, wl.m_cmp, wl.m_win)
    dout = np.random.default_rng(1).standard_normal(wl.q.shape)
    ref = oracle.backward(wl, dout, blocks=ob)
    got = parallel.backward_full(wl, dout, ob, workers=3)
    for name in ("dq", "dgates"):
        assert np.array_equal(ref[name], got[name]), name
    for name in ("dk", "dv", "dkbar", "dvbar"):
        np.testing.assert_allclose(got[name], ref[name], rtol=0, atol=1e-12 * np.abs(ref[name]).max())
    rows = [(t, h) for t in range(0, wl.n_tokens, 5) for h in range(wl.h_q)]
    part = parallel.backward_rows(wl, dout, ob, rows, workers=2)
    t = [r[0] for r in rows]
    h = [r[1] for r in rows]
    assert np.array_equal(part["dq"], ref["dq"][t, h]) and np.array_equal(part["dgates"], ref["dgates"][t, h])
