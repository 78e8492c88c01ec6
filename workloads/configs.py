"""The five named workloads and a builder for smaller custom ones.

Seeds for named workload ``c`` (1-based): geometry ``1000c+1``, tensors
``1000c+2``, input-order permutation ``1000c+3``.  The varlen workload draws its
per-sequence token counts from seed 5001 and the shape of sequence ``b`` from
seed ``5100+b``.

Workload shapes follow the tokens and attention layouts the pages describe:
Direct3D-S2's 1024^3 sparse latent with about 128k tokens (hyper.ai summary of
arXiv 2505.17412, "Experiments") and LSRM's grouped-query layout of 32 query
heads over 2 key/value heads with hidden size 1024 (LSRM article, "Stage 1").
"""

from __future__ import annotations

import dataclasses
import functools
import math

import numpy as np

from .geometry import ellipsoid_band, primitive_union_band
from .tensors import bf16_bits_from_f32, bf16_bits_to_f32, draw_normal, sigmoid_f32


@dataclasses.dataclass
class Workload:
    name: str
    grid_res: int
    m_cmp: int
    m_win: int
    topk: int
    h_q: int
    h_kv: int
    head_dim: int
    dtype: str                 # "bf16" or "f32"
    coords: np.ndarray         # int32 [N, 3], in input (permuted) order
    cu_seqlens: np.ndarray     # int32 [B + 1]
    q: np.ndarray | None = None      # float32 [N, Hq, D]  (bf16-exact values when dtype == "bf16")
    k: np.ndarray | None = None      # float32 [N, Hkv, D]
    v: np.ndarray | None = None      # float32 [N, Hkv, D]
    gates: np.ndarray | None = None  # float32 [N, Hq, 3]  order: compressed, selected, window
    win_shift: int = 0               # window origin at -win_shift per axis (0: unshifted)
    routing: str = "score"           # block selection: "score" or "geometric"

    @property
    def n_tokens(self) -> int:
        return int(self.coords.shape[0])

    @property
    def batch(self) -> int:
        return int(self.cu_seqlens.shape[0] - 1)


# Named workloads (index 1..5).  Each entry: geometry recipe + attention layout.
CONFIGS = {
    1: dict(name="tiny-f32-ellipsoid-32", kind="ellipsoid", grid_res=32, n_tokens=None,
            n_prims=1, h_q=2, h_kv=2, head_dim=32, dtype="f32", gates="uniform",
            m_cmp=4, m_win=8, topk=4),
    2: dict(name="bf16-256-6prims-16384", kind="union", grid_res=256, n_tokens=16384,
            n_prims=6, h_q=16, h_kv=16, head_dim=64, dtype="bf16", gates="sigmoid",
            m_cmp=4, m_win=8, topk=16),
    3: dict(name="bf16-1024-12prims-131072", kind="union", grid_res=1024, n_tokens=131072,
            n_prims=12, h_q=16, h_kv=16, head_dim=64, dtype="bf16", gates="sigmoid",
            m_cmp=4, m_win=8, topk=16),
    4: dict(name="bf16-gqa-1024-16prims-262144", kind="union", grid_res=1024, n_tokens=262144,
            n_prims=16, h_q=32, h_kv=2, head_dim=32, dtype="bf16", gates="sigmoid",
            m_cmp=4, m_win=8, topk=16),
    5: dict(name="bf16-varlen-8x[16k,150k]", kind="varlen", grid_res=1024, n_tokens=None,
            n_prims=12, h_q=16, h_kv=16, head_dim=64, dtype="bf16", gates="sigmoid",
            m_cmp=4, m_win=8, topk=16),
}


def _varlen_counts() -> list[int]:
    rng = np.random.default_rng(5001)
    lo, hi = math.log(16384), math.log(150000)
    return [int(round(math.exp(x))) for x in rng.uniform(lo, hi, size=8)]


@functools.lru_cache(maxsize=8)
def _geometry(cfg_id: int):
    cfg = CONFIGS[cfg_id]
    R = cfg["grid_res"]
    if cfg["kind"] == "ellipsoid":
        seqs = [ellipsoid_band(R, np.random.default_rng(1000 * cfg_id + 1))]
    elif cfg["kind"] == "union":
        rng = np.random.default_rng(1000 * cfg_id + 1)
        seqs = [primitive_union_band(cfg["n_tokens"], cfg["n_prims"], R, rng, rng)]
    else:
        seqs = []
        for b, n in enumerate(_varlen_counts()):
            rng = np.random.default_rng(5100 + b)
            seqs.append(primitive_union_band(n, cfg["n_prims"], R, rng, rng))
    perm_rng = np.random.default_rng(1000 * cfg_id + 3)
    return _pack(seqs, perm_rng)


def _pack(seqs, perm_rng):
    """Concatenate per-sequence voxel sets, each in its own seeded random order."""
    parts, cu = [], [0]
    for c in seqs:
        parts.append(c[perm_rng.permutation(len(c))])
        cu.append(cu[-1] + len(c))
    coords = np.concatenate(parts, axis=0) if parts else np.zeros((0, 3), np.int32)
    return np.ascontiguousarray(coords, dtype=np.int32), np.asarray(cu, dtype=np.int32)


def _draw_tensors(n, h_q, h_kv, d, dtype, gates_kind, seed):
    rng = np.random.default_rng(seed)
    q = draw_normal(rng, (n, h_q, d))
    k = draw_normal(rng, (n, h_kv, d))
    v = draw_normal(rng, (n, h_kv, d))
    if gates_kind == "uniform":
        g = rng.uniform(0.0, 1.0, size=(n, h_q, 3)).astype(np.float32)
    else:
        g = sigmoid_f32(draw_normal(rng, (n, h_q, 3)))
    if dtype == "bf16":
        q, k, v, g = (bf16_bits_to_f32(bf16_bits_from_f32(x)) for x in (q, k, v, g))
    return q, k, v, g


def make_workload(cfg_id: int, with_tensors: bool = True) -> Workload:
    """Build named workload ``cfg_id`` (1..5) from its seeds."""
    cfg = CONFIGS[cfg_id]
    coords, cu = _geometry(cfg_id)
    wl = Workload(name=cfg["name"], grid_res=cfg["grid_res"], m_cmp=cfg["m_cmp"],
                  m_win=cfg["m_win"], topk=cfg["topk"], h_q=cfg["h_q"], h_kv=cfg["h_kv"],
                  head_dim=cfg["head_dim"], dtype=cfg["dtype"], coords=coords.copy(),
                  cu_seqlens=cu.copy())
    if with_tensors:
        wl.q, wl.k, wl.v, wl.gates = _draw_tensors(
            len(coords), cfg["h_q"], cfg["h_kv"], cfg["head_dim"], cfg["dtype"],
            cfg["gates"], 1000 * cfg_id + 2)
    return wl


def make_custom(seq_tokens, *, grid_res=64, n_prims=3, m_cmp=4, m_win=8, topk=4,
                h_q=2, h_kv=2, head_dim=32, dtype="bf16", seed=0, gates="sigmoid",
                coords=None, cu_seqlens=None, win_shift=0, routing="score") -> Workload:
    """A small workload: one surface-band shape per entry of ``seq_tokens``.

    ``coords``/``cu_seqlens`` may be given directly instead (adversarial
    geometry in tests); tensors are then drawn for that token count.
    """
    if coords is None:
        seqs = []
        for b, n in enumerate(seq_tokens):
            if n == 0:
                seqs.append(np.zeros((0, 3), np.int32))
                continue
            rng = np.random.default_rng(seed * 1000 + 17 * b + 1)
            seqs.append(primitive_union_band(n, n_prims, grid_res, rng, rng))
        coords, cu_seqlens = _pack(seqs, np.random.default_rng(seed * 1000 + 3))
    else:
        coords = np.ascontiguousarray(coords, dtype=np.int32)
        if cu_seqlens is None:
            cu_seqlens = np.asarray([0, len(coords)], dtype=np.int32)
        cu_seqlens = np.asarray(cu_seqlens, dtype=np.int32)
    wl = Workload(name="custom", grid_res=grid_res, m_cmp=m_cmp, m_win=m_win, topk=topk,
                  h_q=h_q, h_kv=h_kv, head_dim=head_dim, dtype=dtype, coords=coords,
                  cu_seqlens=cu_seqlens, win_shift=win_shift, routing=routing)
    wl.q, wl.k, wl.v, wl.gates = _draw_tensors(len(coords), h_q, h_kv, head_dim, dtype,
                                               gates, seed * 1000 + 2)
    return wl
