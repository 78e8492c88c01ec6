"""Run the oracle's per-row functions over worker processes (test
infrastructure only, like the rest of ``oracle/``).

This module holds no arithmetic of the method.  It writes a workload's arrays
and the oracle's block partition once to a temporary directory (under
/dev/shm when it exists), starts ``workers`` fresh Python processes (the
"spawn" start method: the children load numpy and the oracle only and open no
GPU device), and has each worker memory-map the arrays and call
``forward_rows`` or ``backward_rows`` on its share of the rows.  The parent
concatenates the per-row results in row order and adds the summed key / value
gradients in a fixed task order, so the result does not depend on which worker
finished first.

Workers use one BLAS thread each.  The worker count defaults to the CPUs this
process may run on, capped at 16.
"""
from __future__ import annotations

import multiprocessing as mp
import os
import shutil
import tempfile
import time
import types

import numpy as np

from . import ssa_oracle as O

MAX_WORKERS = 16
_ARRAYS = ("coords", "cu_seqlens", "q", "k", "v", "gates")
_BLOCK_ARRAYS = ("perm", "key_sorted", "blk_off", "win_off", "win_blk_off", "seq_blk_off", "seq_win_off")
_SCALARS = ("name", "grid_res", "m_cmp", "m_win", "topk", "h_q", "h_kv", "head_dim", "dtype", "win_shift",
            "routing")

_state = {}


def default_workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(MAX_WORKERS, n))


def _init(root, scalars, n_invalid, r3):
    from threadpoolctl import threadpool_limits
    _state["limits"] = threadpool_limits(limits=1)
    ld = lambda name: np.load(os.path.join(root, name + ".npy"), mmap_mode="r")
    wl = types.SimpleNamespace(**scalars, **{a: ld(a) for a in _ARRAYS})
    wl.n_tokens = int(wl.coords.shape[0])
    wl.batch = int(wl.cu_seqlens.shape[0] - 1)
    blocks = O.Blocks(**{a: np.asarray(ld("blk_" + a)) for a in _BLOCK_ARRAYS}, n_invalid=n_invalid, r3=r3)
    _state.update(wl=wl, blocks=blocks, kbar=np.asarray(ld("kbar")), vbar=np.asarray(ld("vbar")))
    if os.path.exists(os.path.join(root, "dout.npy")):
        _state["dout"] = ld("dout")


def _ready(_):
    return os.getpid()


def _forward_task(args):
    rows, with_branches, with_scores = args
    return O.forward_rows(_state["wl"], _state["blocks"], rows, kbar=_state["kbar"], vbar=_state["vbar"],
                          with_branches=with_branches, with_scores=with_scores)


def _backward_task(args):
    rows, groups = args
    res = O.backward_rows(_state["wl"], _state["dout"], _state["blocks"], rows, kbar=_state["kbar"],
                          vbar=_state["vbar"])
    if groups is None:       # per-row results only
        return dict(dq=res["dq"], dgates=res["dgates"])
    for name in ("dk", "dv", "dkbar", "dvbar"):   # only these KV groups were touched
        res[name] = np.ascontiguousarray(res[name][:, groups])
    return res


class _Pool:
    def __init__(self, wl, blocks, kbar, vbar, dout=None, workers=None):
        self.workers = workers or default_workers()
        need = sum(np.asarray(getattr(wl, a)).nbytes for a in _ARRAYS) + kbar.nbytes + vbar.nbytes
        need += 0 if dout is None else np.asarray(dout).nbytes
        need += sum(getattr(blocks, a).nbytes for a in _BLOCK_ARRAYS)
        base = None   # the default temporary directory, unless /dev/shm has room
        if os.path.isdir("/dev/shm") and shutil.disk_usage("/dev/shm").free > 2 * need:
            base = "/dev/shm"
        self.root = tempfile.mkdtemp(prefix="ssa_oracle_", dir=base)
        try:
            for a in _ARRAYS:
                np.save(os.path.join(self.root, a + ".npy"), np.ascontiguousarray(getattr(wl, a)))
            for a in _BLOCK_ARRAYS:
                np.save(os.path.join(self.root, "blk_" + a + ".npy"), getattr(blocks, a))
            np.save(os.path.join(self.root, "kbar.npy"), kbar)
            np.save(os.path.join(self.root, "vbar.npy"), vbar)
            if dout is not None:
                np.save(os.path.join(self.root, "dout.npy"), np.ascontiguousarray(dout))
            scalars = {a: getattr(wl, a, None) for a in _SCALARS}
            scalars["win_shift"] = scalars["win_shift"] or 0
            scalars["routing"] = scalars["routing"] or "score"
            ctx = mp.get_context("spawn")
            self.pool = ctx.Pool(self.workers, initializer=_init,
                                 initargs=(self.root, scalars, blocks.n_invalid, blocks.r3))
        except BaseException:
            shutil.rmtree(self.root, ignore_errors=True)
            raise

    def close(self):
        try:
            self.pool.terminate()
            self.pool.join()
        finally:
            shutil.rmtree(self.root, ignore_errors=True)


def _chunks(rows, n):
    step = max(1, -(-len(rows) // n))
    return [rows[i:i + step] for i in range(0, len(rows), step)]


def forward_rows(wl, blocks, rows, kbar=None, vbar=None, with_branches=False, with_scores=False,
                 workers=None, timing=None):
    """``oracle.forward_rows`` over worker processes; same result layout.
    A dict passed as ``timing`` receives the set-up time (arrays written,
    workers started) and the time of the rows themselves, in seconds."""
    if kbar is None:
        kbar = O.pool_blocks(wl.k, blocks, wl.dtype)
    if vbar is None:
        vbar = O.pool_blocks(wl.v, blocks, wl.dtype)
    t0 = time.perf_counter()
    p = _Pool(wl, blocks, kbar, vbar, workers=workers)
    try:
        p.pool.map(_ready, range(p.workers))
        t1 = time.perf_counter()
        parts = p.pool.map(_forward_task, [(c, with_branches, with_scores)
                                           for c in _chunks(list(rows), 4 * p.workers)])
        t2 = time.perf_counter()
    finally:
        p.close()
    if timing is not None:
        timing.update(setup_s=t1 - t0, rows_s=t2 - t1, workers=p.workers)
    res = {}
    for name in parts[0]:
        if isinstance(parts[0][name], list):
            res[name] = [x for part in parts for x in part[name]]
        else:
            res[name] = np.concatenate([part[name] for part in parts], axis=0)
    return res


def backward_rows(wl, dout, blocks, rows, workers=None, timing=None):
    """dq [len(rows), D] and dgates [len(rows), 3] of the given (token, head)
    rows (``oracle.backward(..., rows=rows)``) over worker processes;
    ``timing`` as in ``forward_rows``."""
    kbar = O.pool_blocks(wl.k, blocks, wl.dtype)
    vbar = O.pool_blocks(wl.v, blocks, wl.dtype)
    t0 = time.perf_counter()
    p = _Pool(wl, blocks, kbar, vbar, dout=dout, workers=workers)
    try:
        p.pool.map(_ready, range(p.workers))
        t1 = time.perf_counter()
        parts = p.pool.map(_backward_task, [(c, None) for c in _chunks(list(rows), 4 * p.workers)])
        t2 = time.perf_counter()
    finally:
        p.close()
    if timing is not None:
        timing.update(setup_s=t1 - t0, rows_s=t2 - t1, workers=p.workers)
    return {name: np.concatenate([part[name] for part in parts], axis=0) for name in ("dq", "dgates")}


def backward_full(wl, dout, blocks, workers=None):
    """``oracle.backward`` (every row) over worker processes: one task per
    (KV group, share of its rows); the per-row results are put back in row
    order and the key / value gradient sums added in task order."""
    kbar = O.pool_blocks(wl.k, blocks, wl.dtype)
    vbar = O.pool_blocks(wl.v, blocks, wl.dtype)
    N, H, Hkv, D = wl.n_tokens, wl.h_q, wl.h_kv, wl.head_dim
    G = H // Hkv
    p = _Pool(wl, blocks, kbar, vbar, dout=dout, workers=workers)
    try:
        per_group = max(1, -(-4 * p.workers // Hkv))
        tasks = []
        for g in range(Hkv):
            rows = [(t, h) for h in range(g * G, (g + 1) * G) for t in range(N)]
            tasks += [(c, [g]) for c in _chunks(rows, per_group)]
        parts = p.pool.map(_backward_task, tasks)
    finally:
        p.close()
    dq = np.zeros((N, H, D))
    dgates = np.zeros((N, H, 3))
    dk = np.zeros((N, Hkv, D))
    dv = np.zeros((N, Hkv, D))
    dkbar = np.zeros((blocks.nb, Hkv, D))
    dvbar = np.zeros((blocks.nb, Hkv, D))
    for (rows, (g,)), part in zip(tasks, parts):
        t = np.array([r[0] for r in rows], dtype=np.int64)
        h = np.array([r[1] for r in rows], dtype=np.int64)
        dq[t, h] = part["dq"]
        dgates[t, h] = part["dgates"]
        dk[:, g] += part["dk"][:, 0]
        dv[:, g] += part["dv"][:, 0]
        dkbar[:, g] += part["dkbar"][:, 0]
        dvbar[:, g] += part["dvbar"][:, 0]
    dk, dv = O.pooled_to_tokens(blocks, dk, dv, dkbar, dvbar)
    return dict(dq=dq, dk=dk, dv=dv, dgates=dgates, dkbar=dkbar, dvbar=dvbar)
