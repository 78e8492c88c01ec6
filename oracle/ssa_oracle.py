"""Float64 numpy oracle of the SSA forward and backward passes (test
infrastructure only).

Page references: "Direct3D-S2 page" is the hyper.ai summary of arXiv
2505.17412; "LSRM page" is the article on LSRM (Meta Reality Labs / NVIDIA).

Readings taken where the pages are silent (each listed in the design notes):

* Blocks and windows are aligned to the grid origin and do not overlap; a block
  is the set of tokens of one sequence inside one m_cmp^3 cell, a window the
  set inside one m_win^3 cell (Direct3D-S2 page, "Method": blocks follow 3D
  coordinates; windows are non-overlapping).
* Compression is the plain mean over the block's occupied tokens; the learned
  sparse convolution before it is not part of this path.  The mean is rounded
  once to the input dtype (the compressed keys/values are tokens of that
  dtype).
* Block numbering: ascending hierarchical key (sequence, window in C order,
  sub-block in C order inside the window).  Ties in the top-k go to the lower
  block number.
* Selection score of block j for query t and KV group g: the softmax
  probability of j in the compressed branch, summed over the query heads of g.
  k_eff = min(k, blocks in the sequence).  No block is forced, no causality.
* Softmax scale 1/sqrt(D) in every branch.  Gates are used as given, in the
  order (compressed, selected, window).
* Geometric routing (the optional 3D-aware selection): the distance from a
  query voxel to a block is the smallest squared distance between the query's
  voxel centre and the centres of the block's voxels; the k nearest blocks of
  the sequence are selected, ties to the lower block id.  The compressed
  branch is still computed; only the selection changes.
* Backward: the top-k choice is held fixed (it is piecewise constant in Q and
  K, so it has no gradient), and the one rounding of the pooled blocks to the
  input dtype is differentiated as the identity; a pooled row's gradient is
  shared equally by the block's tokens (the derivative of a mean).
"""

from __future__ import annotations

import dataclasses
import math

import numpy as np


# ----------------------------------------------------------------------------
# dtype rounding (the only rounding the method applies: the pooled blocks, and
# the final output, are values of the input dtype)
# ----------------------------------------------------------------------------

def bf16_round(x) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 value, ties to even.

    bfloat16 keeps 8 significant bits and float32's exponent range; below the
    normal range its spacing is the fixed subnormal step 2^-133.
    """
    x = np.asarray(x, dtype=np.float64)
    mant, expo = np.frexp(x)                      # x = mant * 2^expo, 0.5 <= |mant| < 1
    expo = np.maximum(expo, -125)                 # spacing of bf16 below 2^-126 is 2^-133
    step_exp = expo - 8                           # 8 significant bits
    return np.ldexp(np.rint(np.ldexp(x, -step_exp)), step_exp)


def round_to(x, dtype: str) -> np.ndarray:
    """Round to the dtype's values ("f64": no rounding, for exact derivative checks)."""
    if dtype == "f64":
        return np.asarray(x, dtype=np.float64)
    if dtype == "bf16":
        return bf16_round(x)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)
    raise ValueError(dtype)


# ----------------------------------------------------------------------------
# Integer stage: block keys, stable sort, segments
# ----------------------------------------------------------------------------

def _log2_exact(v: int) -> int:
    if v <= 0 or v & (v - 1):
        raise ValueError(f"{v} is not a power of two")
    return v.bit_length() - 1


def block_keys(coords, cu_seqlens, grid_res: int, m_cmp: int, m_win: int, shift: int = 0):
    """Hierarchical block key of every token (input order), plus validity.

    key = ((seq * Rw^3 + lin(w)) * r^3 + lin(s)) with w = floor(c / m_win),
    s = floor(c / m_cmp) mod r, Rw = R / m_win, r = m_win / m_cmp and
    lin(x, y, z) = (x * n + y) * n + z.  Sorting by this key groups tokens by
    sequence, then window, then block (Direct3D-S2 page, "Method": blocking by
    3D coordinate; non-overlapping windows).

    ``shift`` (a multiple of m_cmp below m_win) moves the window origin by
    -shift on every axis, as in shifted-window attention (Direct3D-S2 page,
    "Method", the sparse VAE's shifted windows): the coordinates are taken as
    c + shift on a grid with one more window per axis.  Blocks stay the same
    cells, since shift is a whole number of blocks.
    """
    coords = np.asarray(coords, dtype=np.int64).reshape(-1, 3)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    n = coords.shape[0]
    if m_win % m_cmp:
        raise ValueError("m_win must be a multiple of m_cmp")
    if shift % m_cmp or not 0 <= shift < m_win:
        raise ValueError("shift must be a multiple of m_cmp in [0, m_win)")
    Rw = grid_res // m_win + (1 if shift else 0)
    r = m_win // m_cmp
    seq = np.zeros(n, dtype=np.int64)
    for b in range(len(cu) - 1):
        seq[cu[b]:cu[b + 1]] = b
    valid = np.all((coords >= 0) & (coords < grid_res), axis=1)
    w = (coords + shift) // m_win
    s = ((coords + shift) // m_cmp) % r
    lin_w = (w[:, 0] * Rw + w[:, 1]) * Rw + w[:, 2]
    lin_s = (s[:, 0] * r + s[:, 1]) * r + s[:, 2]
    key = (seq * Rw ** 3 + lin_w) * r ** 3 + lin_s
    return key, valid


@dataclasses.dataclass
class Blocks:
    perm: np.ndarray         # sorted position -> input token index
    key_sorted: np.ndarray   # block key at each sorted position
    blk_off: np.ndarray      # [nb + 1] first sorted position of each block
    win_off: np.ndarray      # [nw + 1] first sorted position of each window
    win_blk_off: np.ndarray  # [nw + 1] first block id of each window
    seq_blk_off: np.ndarray  # [B + 1] first block id of each sequence
    seq_win_off: np.ndarray  # [B + 1] first window id of each sequence
    n_invalid: int
    r3: int                  # sub-blocks per window (r^3)

    @property
    def nb(self) -> int:
        return len(self.blk_off) - 1

    @property
    def nw(self) -> int:
        return len(self.win_off) - 1


def build_blocks(coords, cu_seqlens, grid_res: int, m_cmp: int, m_win: int, shift: int = 0) -> Blocks:
    """Stable sort of tokens by block key and the CSR segments over it."""
    key, valid = block_keys(coords, cu_seqlens, grid_res, m_cmp, m_win, shift)
    n = len(key)
    r3 = (m_win // m_cmp) ** 3
    perm = np.argsort(key, kind="stable")
    ks = key[perm]
    wk = ks // r3
    new_blk = np.ones(n, dtype=bool)
    new_win = np.ones(n, dtype=bool)
    if n:
        new_blk[1:] = ks[1:] != ks[:-1]
        new_win[1:] = wk[1:] != wk[:-1]
    blk_start = np.nonzero(new_blk)[0]
    win_start = np.nonzero(new_win)[0]
    blk_off = np.append(blk_start, n)
    win_off = np.append(win_start, n)
    blk_id_of_pos = np.cumsum(new_blk) - 1
    win_blk_off = np.append(blk_id_of_pos[win_start], len(blk_start))
    # sequence of each block / window (the key's top part)
    Rw3 = (grid_res // m_win + (1 if shift else 0)) ** 3
    seq_of_blk = ks[blk_start] // (Rw3 * r3)
    seq_of_win = ks[win_start] // (Rw3 * r3)
    B = len(cu_seqlens) - 1
    seq_blk_off = np.searchsorted(seq_of_blk, np.arange(B + 1), side="left")
    seq_win_off = np.searchsorted(seq_of_win, np.arange(B + 1), side="left")
    return Blocks(perm=perm, key_sorted=ks, blk_off=blk_off, win_off=win_off,
                  win_blk_off=win_blk_off, seq_blk_off=seq_blk_off,
                  seq_win_off=seq_win_off, n_invalid=int((~valid).sum()), r3=r3)


# ----------------------------------------------------------------------------
# Compression: mean pooling of keys/values per block
# ----------------------------------------------------------------------------

def pool_blocks(x, blocks: Blocks, dtype: str) -> np.ndarray:
    """Mean of x over each block's tokens, rounded once to ``dtype``.

    x: [N, H, D] in input order.  Returns [nb, H, D] float64 holding values of
    ``dtype`` (Direct3D-S2 page, "Method": mean pooling gives block-level
    compressed keys and values; LSRM page, "Stage 2": AvgPool inside a block).
    """
    x = np.asarray(x)
    out = np.zeros((blocks.nb,) + x.shape[1:], dtype=np.float64)
    for j in range(blocks.nb):
        toks = blocks.perm[blocks.blk_off[j]:blocks.blk_off[j + 1]]
        out[j] = np.asarray(x[toks], dtype=np.float64).sum(axis=0) / len(toks)
    return round_to(out, dtype)


# ----------------------------------------------------------------------------
# Attention pieces
# ----------------------------------------------------------------------------

def softmax_attention(q, k, v, scale: float):
    """Softmax attention of one query q [D] over keys k [n, D], values v [n, D].

    Returns (o [D], p [n]).  The maximum is subtracted before exponentiation.
    """
    s = scale * (k @ q)
    s = s - s.max()
    e = np.exp(s)
    p = e / e.sum()
    return p @ v, p


def geometric_topk(coords, blocks: Blocks, t: int, j0: int, j1: int, k: int):
    """The k blocks of [j0, j1) nearest to token t, nearest first.

    LSRM article, "3D-aware block routing": a voxel token stands at its
    voxel's centre, and a query selects the blocks whose points lie closest to
    it in Euclidean distance (the shortest distance from the query to the
    block's point set).  Distances between voxel centres are compared as exact
    integer squared distances; ties go to the lower block id.
    """
    c = np.asarray(coords[t], dtype=np.int64)
    first, last = int(blocks.blk_off[j0]), int(blocks.blk_off[j1])
    if j1 <= j0:
        return np.zeros(0, dtype=np.int64)
    toks = blocks.perm[first:last]
    diff = np.asarray(coords[toks], dtype=np.int64) - c
    d_tok = (diff * diff).sum(axis=1)                     # squared distance of every voxel
    # the block's distance is the smallest over its voxels (blocks are
    # contiguous runs of the sorted order)
    d = np.minimum.reduceat(d_tok, np.asarray(blocks.blk_off[j0:j1], dtype=np.int64) - first)
    order = np.lexsort((np.arange(j1 - j0), d))
    return order[:min(k, j1 - j0)]


def topk_blocks(score, k: int):
    """Indices of the k largest scores, largest first; ties to the lower index."""
    score = np.asarray(score, dtype=np.float64)
    k_eff = min(k, len(score))
    order = np.lexsort((np.arange(len(score)), -score))  # primary: -score, secondary: index
    return order[:k_eff]


# ----------------------------------------------------------------------------
# Full forward
# ----------------------------------------------------------------------------

def _token_rows(blocks: Blocks, t_sorted: int):
    """(sequence, window) of the token at sorted position ``t_sorted``."""
    w = int(np.searchsorted(blocks.win_off, t_sorted, side="right") - 1)
    b = int(np.searchsorted(blocks.seq_win_off, w, side="right") - 1)
    return b, w


def forward_rows(wl, blocks: Blocks, rows, kbar=None, vbar=None, with_branches=False,
                 with_scores=False):
    """SSA output for selected (input token index, query head) pairs.

    ``wl`` carries q/k/v/gates (float arrays), head counts, topk and dtype.
    Returns a dict with ``out`` [len(rows), D] (rounded to the dtype), the
    per-branch outputs (float64), and ``topk`` [len(rows), k] (-1 padded) for
    the KV group of each row.  ``with_scores`` adds, per row, the selection
    score of every block of the row's sequence (float64, sequence-local order)
    and the sequence's first block id.
    """
    H, Hkv, D, K = wl.h_q, wl.h_kv, wl.head_dim, wl.topk
    G = H // Hkv
    scale = 1.0 / math.sqrt(D)
    if kbar is None:
        kbar = pool_blocks(wl.k, blocks, wl.dtype)
    if vbar is None:
        vbar = pool_blocks(wl.v, blocks, wl.dtype)
    pos_of_tok = np.empty(len(blocks.perm), dtype=np.int64)
    pos_of_tok[blocks.perm] = np.arange(len(blocks.perm))

    def f64(a):
        return np.asarray(a, dtype=np.float64)

    out = np.zeros((len(rows), D))
    o_c = np.zeros((len(rows), D))
    o_s = np.zeros((len(rows), D))
    o_w = np.zeros((len(rows), D))
    sel = -np.ones((len(rows), K), dtype=np.int64)
    scores, firsts = [], []
    for n_row, (t, h) in enumerate(rows):
        i = int(pos_of_tok[t])
        b, w = _token_rows(blocks, i)
        g = h // G
        j0, j1 = int(blocks.seq_blk_off[b]), int(blocks.seq_blk_off[b + 1])
        # (a) compressed attention over the sequence's blocks, for every head of
        # the group (the selection score sums their probabilities)
        score = np.zeros(j1 - j0)
        for hh in range(g * G, (g + 1) * G):
            o_hh, p_hh = softmax_attention(f64(wl.q[t, hh]), kbar[j0:j1, g], vbar[j0:j1, g], scale)
            score += p_hh
            if hh == h:
                o_cmp = o_hh
        # (b) top-k blocks (by score, or by distance with geometric routing);
        # attention over all their tokens
        if getattr(wl, "routing", "score") == "geometric":
            chosen = geometric_topk(wl.coords, blocks, t, j0, j1, K)
        else:
            chosen = topk_blocks(score, K)
        if with_scores:
            scores.append(score)
            firsts.append(j0)
        sel[n_row, :len(chosen)] = chosen + j0
        pos = np.concatenate([np.arange(blocks.blk_off[j0 + c], blocks.blk_off[j0 + c + 1])
                              for c in chosen])
        toks = blocks.perm[pos]
        o_sel, _ = softmax_attention(f64(wl.q[t, h]), f64(wl.k[toks, g]), f64(wl.v[toks, g]), scale)
        # (c) attention inside the token's window
        toks = blocks.perm[blocks.win_off[w]:blocks.win_off[w + 1]]
        o_win, _ = softmax_attention(f64(wl.q[t, h]), f64(wl.k[toks, g]), f64(wl.v[toks, g]), scale)
        gt = f64(wl.gates[t, h])
        o_c[n_row], o_s[n_row], o_w[n_row] = o_cmp, o_sel, o_win
        out[n_row] = gt[0] * o_cmp + gt[1] * o_sel + gt[2] * o_win
    res = dict(out=round_to(out, wl.dtype), out_exact=out, topk=sel)
    if with_branches:
        res.update(o_cmp=o_c, o_sel=o_s, o_win=o_w)
    if with_scores:
        res.update(scores=scores, first_block=firsts)
    return res


def forward(wl, blocks: Blocks | None = None, with_branches=False):
    """Full SSA forward for every token and head (small inputs only).

    Returns dict: out [N, H, D] (dtype-rounded, float64), topk [N, Hkv, k]
    (block ids, -1 padded; identical for all heads of a group), kbar, vbar,
    and optionally the per-branch outputs.
    """
    if blocks is None:
        blocks = build_blocks(wl.coords, wl.cu_seqlens, wl.grid_res, wl.m_cmp, wl.m_win,
                              getattr(wl, "win_shift", 0))
    kbar = pool_blocks(wl.k, blocks, wl.dtype)
    vbar = pool_blocks(wl.v, blocks, wl.dtype)
    N, H, Hkv = wl.n_tokens, wl.h_q, wl.h_kv
    G = H // Hkv
    rows = [(t, h) for t in range(N) for h in range(H)]
    res = forward_rows(wl, blocks, rows, kbar=kbar, vbar=vbar, with_branches=with_branches)
    D = wl.head_dim
    full = dict(out=res["out"].reshape(N, H, D), out_exact=res["out_exact"].reshape(N, H, D),
                kbar=kbar, vbar=vbar, blocks=blocks)
    full["topk"] = res["topk"].reshape(N, H, -1)[:, ::G, :]
    if with_branches:
        for name in ("o_cmp", "o_sel", "o_win"):
            full[name] = res[name].reshape(N, H, D)
    return full


# ----------------------------------------------------------------------------
# Backward pass
# ----------------------------------------------------------------------------

def softmax_attention_grad(q, k, v, do, scale: float):
    """Gradients of o = softmax(scale * k q) v for one query, given do = dL/do.

    With p the probabilities: dp_j = do . v_j is the gradient of p_j, the
    softmax turns it into the logit gradient ds_j = p_j (dp_j - sum_i p_i dp_i),
    and the logits scale * q . k_j give dq = scale * sum_j ds_j k_j and
    dk_j = scale * ds_j q; dv_j = p_j do.  Returns (dq [D], dk [n, D],
    dv [n, D], o [D]).
    """
    o, p = softmax_attention(q, k, v, scale)
    dp = v @ do
    ds = p * (dp - p @ dp)
    return scale * (ds @ k), scale * np.outer(ds, q), np.outer(p, do), o


def backward_rows(wl, dout, blocks: Blocks, rows, kbar=None, vbar=None):
    """Backward contributions of the given (input token index, query head) rows.

    O[t, h] = G0 o_cmp + G1 o_sel + G2 o_win (Direct3D-S2 page, "Method"), so
    branch x sees the output gradient G_x * dout[t, h] and the gate gets
    dout[t, h] . o_x.  Every row's own dq [len(rows), D] and dgates
    [len(rows), 3] depend on that row alone.  The key / value gradients are
    sums over rows: each row adds its selected- and window-branch terms to the
    token gradients dk, dv [N, Hkv, D] and its compressed-branch terms to the
    pooled-row gradients dkbar, dvbar [nb, Hkv, D].  The sum over all rows,
    passed to ``pooled_to_tokens``, is the gradient.  The top-k choice is held
    fixed.
    """
    H, Hkv, D, K = wl.h_q, wl.h_kv, wl.head_dim, wl.topk
    G = H // Hkv
    N = wl.n_tokens
    scale = 1.0 / math.sqrt(D)
    if kbar is None:
        kbar = pool_blocks(wl.k, blocks, wl.dtype)
    if vbar is None:
        vbar = pool_blocks(wl.v, blocks, wl.dtype)
    pos_of_tok = np.empty(len(blocks.perm), dtype=np.int64)
    pos_of_tok[blocks.perm] = np.arange(len(blocks.perm))

    def f64(a):
        return np.asarray(a, dtype=np.float64)

    dq = np.zeros((len(rows), D))
    dgates = np.zeros((len(rows), 3))
    dk = np.zeros((N, Hkv, D))
    dv = np.zeros((N, Hkv, D))
    dkbar = np.zeros((blocks.nb, Hkv, D))
    dvbar = np.zeros((blocks.nb, Hkv, D))
    for n_row, (t, h) in enumerate(rows):
        i = int(pos_of_tok[t])
        b, w = _token_rows(blocks, i)
        g = h // G
        j0, j1 = int(blocks.seq_blk_off[b]), int(blocks.seq_blk_off[b + 1])
        # the selection, as in the forward
        if getattr(wl, "routing", "score") == "geometric":
            chosen = geometric_topk(wl.coords, blocks, t, j0, j1, K)
        else:
            score = np.zeros(j1 - j0)
            for hh in range(g * G, (g + 1) * G):
                score += softmax_attention(f64(wl.q[t, hh]), kbar[j0:j1, g], vbar[j0:j1, g], scale)[1]
            chosen = topk_blocks(score, K)
        sel = blocks.perm[np.concatenate([np.arange(blocks.blk_off[j0 + c], blocks.blk_off[j0 + c + 1])
                                          for c in chosen])]
        win = blocks.perm[blocks.win_off[w]:blocks.win_off[w + 1]]
        q, do, gt = f64(wl.q[t, h]), f64(dout[t, h]), f64(wl.gates[t, h])
        # (a) compressed branch: gradients of the pooled rows
        dq_c, dkb, dvb, o_c = softmax_attention_grad(q, kbar[j0:j1, g], vbar[j0:j1, g], gt[0] * do, scale)
        # (b) selected tokens and (c) window tokens (each a set of distinct tokens)
        dq_s, dks, dvs, o_s = softmax_attention_grad(q, f64(wl.k[sel, g]), f64(wl.v[sel, g]), gt[1] * do, scale)
        dq_w, dkw, dvw, o_w = softmax_attention_grad(q, f64(wl.k[win, g]), f64(wl.v[win, g]), gt[2] * do, scale)
        dkbar[j0:j1, g] += dkb
        dvbar[j0:j1, g] += dvb
        dk[sel, g] += dks
        dv[sel, g] += dvs
        dk[win, g] += dkw
        dv[win, g] += dvw
        dq[n_row] = dq_c + dq_s + dq_w
        dgates[n_row] = (do @ o_c, do @ o_s, do @ o_w)
    return dict(dq=dq, dgates=dgates, dk=dk, dv=dv, dkbar=dkbar, dvbar=dvbar)


def pooled_to_tokens(blocks: Blocks, dk, dv, dkbar, dvbar):
    """Token gradients from the summed row contributions: the pooling is a
    mean, so each token of block j gets 1 / n_j of the pooled row's gradient
    (added to dk, dv in place, which are returned)."""
    for j in range(blocks.nb):
        toks = blocks.perm[blocks.blk_off[j]:blocks.blk_off[j + 1]]
        dk[toks] += dkbar[j] / len(toks)
        dv[toks] += dvbar[j] / len(toks)
    return dk, dv


def backward(wl, dout, blocks: Blocks | None = None, rows=None):
    """Gradients of L = sum(dout * O), O the SSA output before its rounding.

    The compressed branch's key / value gradients land on the pooled rows and
    are then shared by each block's tokens, divided by the token count (the
    pooling is a mean).  The top-k choice is held fixed.

    Without ``rows``: float64 dq [N, H, D], dk / dv [N, Hkv, D], dgates
    [N, H, 3] and dkbar / dvbar [nb, Hkv, D].  With ``rows`` (a list of
    (token, head)): only dq [len(rows), D] and dgates [len(rows), 3] of those
    rows, which depend on nothing else.
    """
    if blocks is None:
        blocks = build_blocks(wl.coords, wl.cu_seqlens, wl.grid_res, wl.m_cmp, wl.m_win,
                              getattr(wl, "win_shift", 0))
    if rows is not None:
        part = backward_rows(wl, dout, blocks, rows)
        return dict(dq=part["dq"], dgates=part["dgates"])
    N, H, D = wl.n_tokens, wl.h_q, wl.head_dim
    part = backward_rows(wl, dout, blocks, [(t, h) for t in range(N) for h in range(H)])
    dk, dv = pooled_to_tokens(blocks, part["dk"], part["dv"], part["dkbar"], part["dvbar"])
    return dict(dq=part["dq"].reshape(N, H, D), dk=dk, dv=dv, dgates=part["dgates"].reshape(N, H, 3),
                dkbar=part["dkbar"], dvbar=part["dvbar"])
