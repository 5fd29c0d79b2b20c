"""Seeded synthetic scenes and cameras.

This module only draws inputs: it holds none of the rasteriser's arithmetic, and both the
HIP path and the float64 oracle consume what it returns.  Every array is drawn with
NumPy's PCG64 generator (``default_rng(seed)``) in float64, in the order written below,
then rounded to float32.

Workload recipes (the pages measure on real captured scenes, which are not available;
these synthetic scenes stand in for them):

* ``tiny``: 1,000 Gaussians, SH degree 0, colours uniform in [0, 1]; means uniform in
  x, y in [-1, 1], z in [2, 4]; scales exp(U[-4, -2]); rotations normalised N(0, 1)
  quaternions (w, x, y, z); opacity sigmoid(N(0, 1)); one 64x64 camera at the origin
  looking along +z with fx = fy = 64, cx = cy = 32, near plane 0.2.
* ``spheres``: Gaussians on the surfaces of 5 random spheres plus 10% uniform clutter,
  SH degree 3 (DC uniform in [-1, 1], higher orders N(0, 0.1)), scales exp(U[-5, -3]),
  or anisotropic (one axis exp(U[-6, -5]), two axes exp(U[-4, -3])).  Cameras sit on a
  radius-4 orbit in the x-z plane and look at the origin.

The colour of a degree-0 Gaussian is 0.5 + Y00 * k0 with Y00 = 1 / (2 sqrt(pi)); the
``tiny`` recipe stores the DC coefficient k0 = (rgb - 0.5) * 2 sqrt(pi) so that the
rendered colour is the drawn rgb.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

TILE = 16


@dataclass
class Camera:
    """Pinhole camera, OpenCV frame (x right, y down, z forward).

    ``R`` (3x3, row major) and ``t`` map world to camera: x_cam = R x_world + t.
    Pixel (i, j) has its centre at (i + 0.5, j + 0.5).
    """

    R: np.ndarray  # (3, 3) float32
    t: np.ndarray  # (3,) float32
    fx: float
    fy: float
    cx: float
    cy: float
    width: int
    height: int
    near: float = 0.2

    @property
    def tiles_x(self) -> int:
        return (self.width + TILE - 1) // TILE

    @property
    def tiles_y(self) -> int:
        return (self.height + TILE - 1) // TILE

    @property
    def num_tiles(self) -> int:
        return self.tiles_x * self.tiles_y


@dataclass
class Scene:
    """Per-Gaussian parameters, float32, one row per Gaussian.

    means (N, 3); scales (N, 3) linear; quats (N, 4) as (w, x, y, z), not necessarily
    unit length; opacities (N,) in (0, 1); sh (N, K, 3) with K = (degree + 1)^2.
    """

    means: np.ndarray
    scales: np.ndarray
    quats: np.ndarray
    opacities: np.ndarray
    sh: np.ndarray
    sh_degree: int

    @property
    def n(self) -> int:
        return int(self.means.shape[0])


def _f32(x) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64).astype(np.float32))


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-x))


def look_at(eye, target, fx, fy, cx, cy, width, height, near=0.2, down=(0.0, 1.0, 0.0)) -> Camera:
    """Camera at ``eye`` looking at ``target``; the image's y axis follows ``down``.

    Rows of R are right = normalise(down x f), down' = f x right and f, with f the unit
    vector from eye to target; t = -R eye.
    """
    eye = np.asarray(eye, dtype=np.float64)
    f = np.asarray(target, dtype=np.float64) - eye
    f /= np.linalg.norm(f)
    right = np.cross(np.asarray(down, dtype=np.float64), f)
    right /= np.linalg.norm(right)
    d2 = np.cross(f, right)
    R = np.stack([right, d2, f])
    t = -R @ eye
    return Camera(_f32(R), _f32(t), float(np.float32(fx)), float(np.float32(fy)),
                  float(np.float32(cx)), float(np.float32(cy)), int(width), int(height),
                  float(np.float32(near)))


def orbit_camera(theta: float, width: int, height: int, f: float = 1000.0, radius: float = 4.0) -> Camera:
    """Radius-``radius`` orbit in the x-z plane: eye = r (sin theta, 0, -cos theta)."""
    eye = radius * np.array([math.sin(theta), 0.0, -math.cos(theta)])
    return look_at(eye, (0.0, 0.0, 0.0), f, f, width / 2.0, height / 2.0, width, height)


def _random_quats(rng, n):
    q = rng.normal(size=(n, 4))
    return q / np.linalg.norm(q, axis=1, keepdims=True)


def tiny_scene(seed: int = 1, n: int = 1000):
    """The 1k-Gaussian SH0 scene and its 64x64 camera."""
    rng = np.random.default_rng(seed)
    xy = rng.uniform(-1.0, 1.0, size=(n, 2))
    z = rng.uniform(2.0, 4.0, size=n)
    means = np.concatenate([xy, z[:, None]], axis=1)
    scales = np.exp(rng.uniform(-4.0, -2.0, size=(n, 3)))
    quats = _random_quats(rng, n)
    opac = _sigmoid(rng.normal(size=n))
    rgb = rng.uniform(0.0, 1.0, size=(n, 3))
    k0 = (rgb - 0.5) * (2.0 * math.sqrt(math.pi))
    scene = Scene(_f32(means), _f32(scales), _f32(quats), _f32(opac), _f32(k0[:, None, :]), 0)
    cam = Camera(np.eye(3, dtype=np.float32), np.zeros(3, dtype=np.float32), 64.0, 64.0, 32.0, 32.0,
                 64, 64, float(np.float32(0.2)))
    return scene, cam


def sphere_scene(seed: int, n: int, anisotropic: bool, chunk: int = 1 << 20) -> Scene:
    """Gaussians on 5 random spheres (90%) plus uniform clutter in [-2, 2]^3 (10%), SH3.

    Sphere centres are uniform in [-1, 1]^3 and radii uniform in [0.3, 1]; a surface
    point is c + r v/|v| with v ~ N(0, I).  Ids are shuffled so that spatial neighbours
    are not id neighbours.
    """
    rng = np.random.default_rng(seed)
    centres = rng.uniform(-1.0, 1.0, size=(5, 3))
    radii = rng.uniform(0.3, 1.0, size=5)
    n_sphere = (9 * n) // 10
    per = [n_sphere // 5 + (1 if s < n_sphere % 5 else 0) for s in range(5)]
    parts = []
    for s in range(5):
        v = rng.normal(size=(per[s], 3))
        v /= np.linalg.norm(v, axis=1, keepdims=True)
        parts.append(centres[s] + radii[s] * v)
    parts.append(rng.uniform(-2.0, 2.0, size=(n - n_sphere, 3)))
    means = np.concatenate(parts, axis=0)
    means = means[rng.permutation(n)]
    if anisotropic:
        thin = rng.uniform(-6.0, -5.0, size=(n, 1))
        wide = rng.uniform(-4.0, -3.0, size=(n, 2))
        scales = np.exp(np.concatenate([thin, wide], axis=1))
    else:
        scales = np.exp(rng.uniform(-5.0, -3.0, size=(n, 3)))
    quats = _random_quats(rng, n)
    opac = _sigmoid(rng.normal(size=n))
    sh = np.empty((n, 16, 3), dtype=np.float32)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        sh[s:e, 0, :] = rng.uniform(-1.0, 1.0, size=(e - s, 3)).astype(np.float32)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        sh[s:e, 1:, :] = rng.normal(0.0, 0.1, size=(e - s, 15, 3)).astype(np.float32)
    return Scene(_f32(means), _f32(scales), _f32(quats), _f32(opac), sh, 3)


def target_image(seed: int, width: int, height: int) -> np.ndarray:
    """A [3][H][W] float32 target, uniform in [0, 1]."""
    rng = np.random.default_rng(seed)
    return _f32(rng.uniform(0.0, 1.0, size=(3, height, width)))


# Named workloads.  Seeds: the workload's number, except that the backward workload
# reuses the 1M scene (seed 3) and draws its target from seed 5.
WORKLOADS = {
    "tiny_1k_sh0_64": dict(n=1000, res=(64, 64)),
    "spheres_100k_sh3_800": dict(n=100_000, res=(800, 800)),
    "aniso_1m_sh3_1080p_8cam": dict(n=1_000_000, res=(1920, 1080)),
    "aniso_10m_sh3_1080p": dict(n=10_000_000, res=(1920, 1080)),
    "aniso_1m_sh3_720p_bwd": dict(n=1_000_000, res=(1280, 720)),
}


def workload(name: str, n: int | None = None):
    """Return (scene, [cameras], extra) for a named workload.

    ``n`` overrides the Gaussian count (same recipe, for scaled-down parity runs).
    ``extra`` holds the backward workload's target image.
    """
    extra = {}
    if name == "tiny_1k_sh0_64":
        scene, cam = tiny_scene(1, n or 1000)
        return scene, [cam], extra
    if name == "spheres_100k_sh3_800":
        scene = sphere_scene(2, n or 100_000, anisotropic=False)
        return scene, [orbit_camera(0.0, 800, 800)], extra
    if name == "aniso_1m_sh3_1080p_8cam":
        scene = sphere_scene(3, n or 1_000_000, anisotropic=True)
        cams = [orbit_camera(2 * math.pi * k / 8, 1920, 1080) for k in range(8)]
        return scene, cams, extra
    if name == "aniso_10m_sh3_1080p":
        scene = sphere_scene(4, n or 10_000_000, anisotropic=True)
        return scene, [orbit_camera(0.0, 1920, 1080)], extra
    if name == "aniso_1m_sh3_720p_bwd":
        scene = sphere_scene(3, n or 1_000_000, anisotropic=True)
        extra["target"] = target_image(5, 1280, 720)
        return scene, [orbit_camera(0.0, 1280, 720)], extra
    raise KeyError(name)
