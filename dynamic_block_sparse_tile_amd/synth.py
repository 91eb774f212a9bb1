"""Seeded synthetic multi-view token generator.

This module only draws inputs.  It holds none of the attention method's
arithmetic or definitions (no pooling, scoring, selection, subsampling or
softmax), so both the HIP path and the fp64 CPU oracle consume what it
produces without sharing code.

The token shapes follow a VGGT-style global-attention layer: S frames, each
with ``specials`` leading camera/register tokens followed by a ``gh x gw``
patch grid, padded to a multiple of the tile size.  Cross-view structure is
planted the way the EPFL "(Full) Attention is More Than You Need" project
frames it (patches of different views that image the same 3D point are the
ones worth attending to): corresponding patches share a latent vector, and
every head adds its own noise.

Arrays are float32 holding values exactly representable in the workload's
dtype (bf16 rounding here is round-to-nearest-even), so a device tensor built
from them carries bit-identical values to what the oracle reads after
upcasting to float64.

Draw order (fixed, so a seed names one input): per-frame 2-D shifts,
frame-unique positions, the patch latent bank (shared bank first, then the
frame-unique latents), special-token latents, then per head the Q/K noise,
then V (heads x rows x d).
"""
from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Optional, Tuple

import numpy as np

__all__ = ["Workload", "WORKLOADS", "Inputs", "make_inputs", "round_bf16", "with_frames"]


@dataclass(frozen=True)
class Workload:
    """One synthetic global-attention workload (all sizes explicit)."""
    name: str
    frames: int                 # S
    tokens: int                 # valid tokens per frame (specials + patches)
    stride: int                 # padded rows per frame, a multiple of ``tile``
    specials: int               # leading camera/register tokens per frame
    heads: int
    head_dim: int = 64
    tile: int = 64
    dtype: str = "bf16"         # "f32" or "bf16"
    structure: str = "shift2d"  # "cyclic1d" (bank index shifts) or "shift2d"
    bank: int = 0               # cyclic1d: latent bank size
    grid: Tuple[int, int] = (37, 37)
    cyclic_step: int = 3        # cyclic1d: frame s, patch p uses bank[(p + step*s) % bank]
    max_shift: int = 4          # shift2d: per-frame (dy, dx) uniform in [-max_shift, max_shift]^2
    unique_patches: int = 0     # shift2d: patches per frame given frame-unique latents
    noise: float = 0.5
    k: Optional[int] = None     # fixed top-k, or None: calibrate to target_sparsity
    target_sparsity: Optional[float] = None
    anchor: int = 0
    landmarks: bool = False
    kv_window: int = 1          # 2: keys/values subsampled 2x2 on the patch grid

    @property
    def rows(self) -> int:
        return self.frames * self.stride

    @property
    def patches(self) -> int:
        return self.tokens - self.specials

    @property
    def layout(self) -> Tuple[int, int, int, int]:
        """(frames, tokens, stride, specials) of the query (and unsubsampled key) sequence."""
        return (self.frames, self.tokens, self.stride, self.specials)


def _vggt(name, frames, **kw):
    return Workload(name=name, frames=frames, tokens=1374, stride=1408, specials=5,
                    heads=16, **kw)


WORKLOADS = {
    # 2 frames x 256 tokens (16x16 grid), 2 heads, fp32, top-4 of 8 tiles, frame 0 anchor
    "tiny_s2": Workload(name="tiny_s2", frames=2, tokens=256, stride=256, specials=0,
                        heads=2, dtype="f32", structure="cyclic1d", bank=256,
                        grid=(16, 16), k=4),
    # VGGT layer at 8 views: 1 camera + 4 register + 37x37 patches; keep 10% (k=18) + anchor
    "vggt_s8": _vggt("vggt_s8", 8, structure="cyclic1d", bank=1369, k=18),
    # 32 views, 2-D shifted correspondences, 90% tile sparsity
    "vggt_s32": _vggt("vggt_s32", 32, target_sparsity=0.90),
    # 128 views, 20% frame-unique patches (274 of 1369), 94% mean sparsity
    "vggt_s128": _vggt("vggt_s128", 128, unique_patches=274, target_sparsity=0.94),
    # same shape at 90% sparsity (the speedup-over-dense comparison point)
    "vggt_s128_90": _vggt("vggt_s128_90", 128, unique_patches=274, target_sparsity=0.90),
    # 256 views, 96% sparsity plus landmark summaries of unselected tiles
    "vggt_s256_lm": _vggt("vggt_s256_lm", 256, unique_patches=274, target_sparsity=0.96,
                          landmarks=True),
    # as above with keys/values subsampled 2x2 on the patch grid; all queries kept
    "vggt_s256_lm_sub2": _vggt("vggt_s256_lm_sub2", 256, unique_patches=274,
                               target_sparsity=0.96, landmarks=True, kv_window=2),
}


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round finite float32 values to the nearest bfloat16 (ties to even), kept as float32.

    Matches ``torch.Tensor.to(torch.bfloat16)`` on finite inputs.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).reshape(x.shape)


@dataclass
class Inputs:
    """Seeded inputs for one workload.  Arrays are float32 [heads, frames*stride, d]."""
    workload: Workload
    seed: int
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    shifts: Optional[np.ndarray] = None

    @property
    def layout(self) -> Tuple[int, int, int, int]:
        return self.workload.layout


def _patch_latent_index(w: Workload, rng: np.random.Generator):
    """Latent-bank index of every patch of every frame, and the bank size."""
    S, n_p = w.frames, w.patches
    p = np.arange(n_p)
    if w.structure == "cyclic1d":
        idx = (p[None, :] + w.cyclic_step * np.arange(S)[:, None]) % w.bank
        return idx, w.bank, None
    gh, gw = w.grid
    assert gh * gw == n_p, "patch grid must cover the patch tokens"
    shifts = rng.integers(-w.max_shift, w.max_shift + 1, size=(S, 2))
    shifts[0] = 0                                  # the anchor view is the reference
    y, x = p // gw, p % gw
    ys = (y[None, :] + shifts[:, :1]) % gh
    xs = (x[None, :] + shifts[:, 1:]) % gw
    idx = ys * gw + xs
    bank = gh * gw
    if w.unique_patches:
        uniq = np.stack([rng.choice(n_p, size=w.unique_patches, replace=False)
                         for _ in range(S)])
        # each frame-unique patch points at its own fresh latent after the shared bank
        fresh = bank + np.arange(S * w.unique_patches).reshape(S, w.unique_patches)
        np.put_along_axis(idx, uniq, fresh, axis=1)
        bank += S * w.unique_patches
    return idx, bank, shifts


def make_inputs(w: Workload, seed: int = 0, pad_value: float = 0.0) -> Inputs:
    """Draw Q (= K) and V for workload ``w`` from ``numpy.random.default_rng(seed)``.

    Q and K are the same array (one noise draw serves both); V is N(0,1) on
    valid rows.  Pad rows (in-frame position >= tokens) hold ``pad_value``
    (use NaN to check that pad rows are masked by index, never read as data).
    """
    rng = np.random.default_rng(seed)
    S, P, d, H = w.frames, w.stride, w.head_dim, w.heads
    idx, bank, shifts = _patch_latent_index(w, rng)
    Z = rng.standard_normal((bank, d), dtype=np.float32)
    Zs = rng.standard_normal((max(w.specials, 1), d), dtype=np.float32)

    latent = np.zeros((S, P, d), dtype=np.float32)
    latent[:, : w.specials] = Zs[None, : w.specials]
    latent[:, w.specials: w.tokens] = Z[idx]
    latent = latent.reshape(S * P, d)

    valid = (np.arange(S * P) % P) < w.tokens
    qk = np.empty((H, S * P, d), dtype=np.float32)
    for h in range(H):
        qk[h] = latent + np.float32(w.noise) * rng.standard_normal((S * P, d), dtype=np.float32)
    v = rng.standard_normal((H, S * P, d), dtype=np.float32)
    if w.dtype == "bf16":
        qk = round_bf16(qk)
        v = round_bf16(v)
    qk[:, ~valid] = pad_value
    v[:, ~valid] = pad_value
    return Inputs(workload=w, seed=seed, q=qk, k=qk, v=v, shifts=shifts)


def with_frames(w: Workload, frames: int, **kw) -> Workload:
    """A copy of ``w`` with a different frame count (for small parity cases)."""
    return replace(w, frames=frames, name=f"{w.name}_f{frames}", **kw)
