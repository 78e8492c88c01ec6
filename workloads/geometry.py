"""Seeded sparse surface-band voxel sets.

A token is an occupied voxel of a narrow band around a surface: the voxel with
integer corner ``c`` is kept when the signed distance at its centre ``c + 0.5``
lies within one cell of zero.  This mirrors the near-surface sparse SDF voxels
that Direct3D-S2's SS-VAE and SS-DiT operate on (hyper.ai summary of
arXiv 2505.17412, "Method" and "Dataset": sparse SDF voxels; "Method": sparse
voxels become variable-length tokens).

Two shape families:

* ``ellipsoid_band``: one randomly rotated ellipsoid on a small grid.  The
  distance is the common first-order estimate for an ellipsoid,
  ``k0 * (k0 - 1) / k1`` with ``k0 = |p / a|`` and ``k1 = |p / a^2|``.
* ``primitive_union_band``: the union (pointwise minimum of exact SDFs) of
  spheres and axis-aligned boxes, scaled by bisection so the band holds at
  least the requested token count, then trimmed to exactly that count by a
  seeded uniform subsample.
"""

from __future__ import annotations

import numpy as np

BAND = 1.0  # keep voxels whose centre is within one cell of the surface


def _sphere_sdf(p: np.ndarray, centre: np.ndarray, radius: float) -> np.ndarray:
    return np.sqrt(((p - centre) ** 2).sum(axis=-1)) - radius


def _box_sdf(p: np.ndarray, centre: np.ndarray, half: np.ndarray) -> np.ndarray:
    q = np.abs(p - centre) - half
    outside = np.sqrt((np.maximum(q, 0.0) ** 2).sum(axis=-1))
    inside = np.minimum(q.max(axis=-1), 0.0)
    return outside + inside


def ellipsoid_band(grid_res: int, rng: np.random.Generator) -> np.ndarray:
    """Band voxels of one random rotated ellipsoid; returns int32 [n, 3]."""
    centre = grid_res / 2.0 + rng.uniform(-1.0, 1.0, size=3)
    axes = rng.uniform(7.0, 12.0, size=3) * (grid_res / 32.0)
    qmat, rmat = np.linalg.qr(rng.standard_normal((3, 3)))
    qmat = qmat * np.sign(np.diag(rmat))  # a proper random orthogonal matrix
    g = np.arange(grid_res, dtype=np.float64)
    x, y, z = np.meshgrid(g, g, g, indexing="ij")
    p = np.stack([x, y, z], axis=-1).reshape(-1, 3) + 0.5 - centre
    local = p @ qmat  # coordinates in the ellipsoid frame
    k0 = np.sqrt(((local / axes) ** 2).sum(axis=-1))
    k1 = np.sqrt(((local / axes**2) ** 2).sum(axis=-1))
    with np.errstate(divide="ignore", invalid="ignore"):
        d = np.where(k1 > 0, k0 * (k0 - 1.0) / k1, -axes.min())
    keep = np.abs(d) <= BAND
    idx = np.nonzero(keep)[0]
    coords = np.stack(np.unravel_index(idx, (grid_res,) * 3), axis=-1)
    return coords.astype(np.int32)


def make_primitives(n_prims: int, grid_res: int, rng: np.random.Generator):
    """Random spheres / axis-aligned boxes: (kind, centre, unit size)."""
    prims = []
    for _ in range(n_prims):
        kind = "sphere" if rng.uniform() < 0.5 else "box"
        centre = rng.uniform(0.3 * grid_res, 0.7 * grid_res, size=3)
        if kind == "sphere":
            unit = np.full(3, rng.uniform(0.5, 1.0))
        else:
            unit = rng.uniform(0.5, 1.0, size=3)
        prims.append((kind, centre, unit))
    return prims


def _union_band(prims, scale: float, grid_res: int) -> np.ndarray:
    """Linear voxel indices of the band of the union at the given scale."""
    cand = []
    for kind, centre, unit in prims:
        ext = unit * scale
        lo = np.maximum(np.floor(centre - ext - BAND - 1.0), 0).astype(np.int64)
        hi = np.minimum(np.ceil(centre + ext + BAND + 1.0), grid_res - 1).astype(np.int64)
        if np.any(hi < lo):
            continue
        axes = [np.arange(lo[a], hi[a] + 1) for a in range(3)]
        x, y, z = np.meshgrid(*axes, indexing="ij")
        c = np.stack([x.ravel(), y.ravel(), z.ravel()], axis=-1)
        p = c + 0.5
        d = _sphere_sdf(p, centre, ext[0]) if kind == "sphere" else _box_sdf(p, centre, ext)
        c = c[np.abs(d) <= BAND]  # a band voxel of the union is in the band of its nearest primitive
        cand.append((c[:, 0] * grid_res + c[:, 1]) * grid_res + c[:, 2])
    if not cand:
        return np.zeros(0, dtype=np.int64)
    lin = np.unique(np.concatenate(cand))
    c = np.stack(np.unravel_index(lin, (grid_res,) * 3), axis=-1).astype(np.float64)
    p = c + 0.5
    d = np.full(len(lin), np.inf)
    for kind, centre, unit in prims:
        ext = unit * scale
        di = _sphere_sdf(p, centre, ext[0]) if kind == "sphere" else _box_sdf(p, centre, ext)
        d = np.minimum(d, di)
    return lin[np.abs(d) <= BAND]


def primitive_union_band(n_tokens: int, n_prims: int, grid_res: int,
                         geo_rng: np.random.Generator,
                         trim_rng: np.random.Generator) -> np.ndarray:
    """Exactly ``n_tokens`` band voxels of a random union; int32 [n, 3].

    The scale is bisected until the band holds at least ``n_tokens`` voxels
    with at most 0.2 % excess (or the bracket collapses); the excess is dropped
    by a seeded uniform subsample.  Output rows are in linear-index order; the
    caller applies its own random input order.
    """
    prims = make_primitives(n_prims, grid_res, geo_rng)
    # Bracket the scale from the band volume: about 2 * BAND cells per unit of
    # surface area.  Widen until the bracket holds the target count.
    area = 0.0
    for kind, _, unit in prims:
        if kind == "sphere":
            area += 4.0 * np.pi * unit[0] ** 2
        else:
            area += 8.0 * (unit[0] * unit[1] + unit[1] * unit[2] + unit[0] * unit[2])
    s0 = np.sqrt(n_tokens / (2.0 * BAND * area))
    lo, hi = 0.5 * s0, 2.0 * s0
    while hi < 0.25 * grid_res and len(_union_band(prims, hi, grid_res)) < n_tokens:
        lo, hi = hi, 2.0 * hi
    best = None
    for _ in range(60):
        mid = 0.5 * (lo + hi)
        lin = _union_band(prims, mid, grid_res)
        if len(lin) >= n_tokens:
            best = lin
            hi = mid
            if len(lin) <= n_tokens * 1.002:
                break
        else:
            lo = mid
        if hi - lo < 1e-6:
            break
    if best is None:
        raise ValueError(f"cannot place {n_tokens} band voxels on a {grid_res}^3 grid")
    keep = np.sort(trim_rng.choice(len(best), size=n_tokens, replace=False))
    lin = best[keep]
    coords = np.stack(np.unravel_index(lin, (grid_res,) * 3), axis=-1)
    return coords.astype(np.int32)
