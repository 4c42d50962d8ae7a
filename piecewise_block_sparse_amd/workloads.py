"""Seeded synthetic inputs shaped like the DiT attention workloads of the pages.

This module holds input generation only -- no step of the attention method.
Both the GPU path (through the tests and the benchmark) and the fp64 oracle
receive exactly the arrays made here, so neither side generates its own data.

Every tensor is drawn per (workload id, head) from
``numpy.random.Generator(PCG64(SeedSequence([workload_id, head])))`` in float32
and, for bf16 workloads, rounded to bfloat16 with round-to-nearest-even; the
returned float32 arrays then hold bf16-exact values, so an upcast to float64
on the oracle side and a cast to bfloat16 on the device side see the same
numbers.

Workloads (shapes from the PISA summary's video and image DiT experiments and
from the block-sparse notes' multimodal mask; generators are readings of the
one-line descriptions and are stated in full below):

1 tiny       b1 h1  L1024  d64  fp32  B64  k4    lambda 0.1
2 image      b1 h24 L4096  d128 bf16  B64  k10   lambda 0.1
3 video-S    b1 h12 L32768 d128 bf16  B64  k64   lambda 0.1   (16x32x64 latent grid)
4 video-L    b1 h40 L32768 d128 bf16  B128 k32   lambda 0.1   (16x32x64 latent grid)
5 multimodal b1 h24 L4608  d128 bf16  B64  fixed text/image block mask
"""

from __future__ import annotations

import dataclasses
from concurrent.futures import ThreadPoolExecutor

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    wid: int
    name: str
    batch: int
    heads: int
    seq_len: int
    head_dim: int
    block: int
    k: int              # exact blocks per query block (0 = fixed mask, see idx_fixed_mask)
    lam: float
    dtype: str          # "fp32" or "bf16"
    text_tokens: int = 0

    @property
    def nb(self) -> int:
        return self.seq_len // self.block

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.head_dim))


WORKLOADS = {
    1: Workload(1, "tiny-fp32", 1, 1, 1024, 64, 64, 4, 0.1, "fp32"),
    2: Workload(2, "image-dit", 1, 24, 4096, 128, 64, 10, 0.1, "bf16"),
    3: Workload(3, "video-dit-S", 1, 12, 32768, 128, 64, 64, 0.1, "bf16"),
    4: Workload(4, "video-dit-L", 1, 40, 32768, 128, 128, 32, 0.1, "bf16"),
    5: Workload(5, "multimodal-dit", 1, 24, 4608, 128, 64, 0, 0.1, "bf16", text_tokens=512),
}

# latent grid of the video workloads: T x H x W tokens, flattened frame-major
VIDEO_GRID = (16, 32, 64)
VIDEO_COARSE = (4, 8, 16)
VIDEO_FIELD_AMPLITUDE = 0.5


def round_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> nearest bfloat16 (ties to even), returned as float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    r = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    out = ((u + r) & np.uint32(0xFFFF0000)).astype(np.uint32)
    return out.view(np.float32)


def _rng(wid: int, head: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([wid, head])))


def _trilinear_x4(coarse: np.ndarray, out_shape) -> np.ndarray:
    """[C, t, y, x] -> [C, *out_shape] trilinear resampling with half-pixel
    centres (sample u of an axis of size n_out maps to (u + 0.5) n_in / n_out - 0.5,
    clamped to the grid)."""
    res = coarse.astype(np.float64)
    for axis, n_out in zip((1, 2, 3), out_shape):
        n_in = res.shape[axis]
        pos = (np.arange(n_out) + 0.5) * n_in / n_out - 0.5
        pos = np.clip(pos, 0.0, n_in - 1)
        lo = np.floor(pos).astype(np.int64)
        hi = np.minimum(lo + 1, n_in - 1)
        w = (pos - lo).reshape([-1 if a == axis else 1 for a in range(4)])
        res = np.take(res, lo, axis=axis) * (1 - w) + np.take(res, hi, axis=axis) * w
    return res


def _head_tensors(w: Workload, head: int):
    """(Q, K, V) for one head, each [L, d] float32."""
    L, d, B = w.seq_len, w.head_dim, w.block
    g = _rng(w.wid, head)
    if w.wid == 1:
        # Q, V ~ N(0,1); K ~ N(0,1) plus a per-block offset N(0, 0.5^2)^d shared
        # by the block's tokens, so block centroids differ.
        Q = g.standard_normal((L, d), dtype=np.float32)
        K = g.standard_normal((L, d), dtype=np.float32)
        off = (0.5 * g.standard_normal((L // B, d))).astype(np.float32)
        K = K + np.repeat(off, B, axis=0)
        V = g.standard_normal((L, d), dtype=np.float32)
    elif w.wid == 2:
        # Q, K ~ N(0,1) with independent per-block mean offsets N(0, 0.5^2)^d;
        # 4 random KV blocks get their keys shifted along the head's mean-query
        # direction u by gamma = 2 * sqrt(d) / ||mean query||, i.e. about
        # +2 nats of logit for the average query, so high-score blocks exist.
        nb = L // B
        Q = g.standard_normal((L, d), dtype=np.float32)
        Q = Q + np.repeat((0.5 * g.standard_normal((nb, d))).astype(np.float32), B, axis=0)
        K = g.standard_normal((L, d), dtype=np.float32)
        K = K + np.repeat((0.5 * g.standard_normal((nb, d))).astype(np.float32), B, axis=0)
        qmean = Q.astype(np.float64).mean(axis=0)
        nrm = float(np.linalg.norm(qmean))
        u = qmean / nrm
        gamma = 2.0 * np.sqrt(d) / nrm
        for j in g.choice(nb, size=4, replace=False):
            K[j * B:(j + 1) * B] += (gamma * u).astype(np.float32)
        V = g.standard_normal((L, d), dtype=np.float32)
    elif w.wid in (3, 4):
        # Shared smooth field F per head: a coarse N(0,1) grid of 4x8x16 per
        # channel, resampled x4 to the 16x32x64 latent grid, normalised to unit
        # std per channel, times 0.5.  Q = F + N(0,1), K = F + N(0,1) with
        # independent noise, so spatial neighbours score higher.  V ~ N(0,1).
        coarse = g.standard_normal((d,) + VIDEO_COARSE)
        F = _trilinear_x4(coarse, VIDEO_GRID).reshape(d, -1)
        F = F / F.std(axis=1, keepdims=True) * VIDEO_FIELD_AMPLITUDE
        F = np.ascontiguousarray(F.T, dtype=np.float32)          # [L, d], frame-major
        Q = F + g.standard_normal((L, d), dtype=np.float32)
        K = F + g.standard_normal((L, d), dtype=np.float32)
        V = g.standard_normal((L, d), dtype=np.float32)
    elif w.wid == 5:
        # text tokens first, then image tokens; per-modality mean vectors
        # N(0, 0.5^2)^d for Q-text, Q-image, K-text, K-image added to N(0,1).
        T = w.text_tokens
        mu = (0.5 * g.standard_normal((4, d))).astype(np.float32)
        Q = g.standard_normal((L, d), dtype=np.float32)
        K = g.standard_normal((L, d), dtype=np.float32)
        Q[:T] += mu[0]
        Q[T:] += mu[1]
        K[:T] += mu[2]
        K[T:] += mu[3]
        V = g.standard_normal((L, d), dtype=np.float32)
    else:
        raise ValueError(f"unknown workload {w.wid}")
    if w.dtype == "bf16":
        Q, K, V = round_bf16(Q), round_bf16(K), round_bf16(V)
    return Q, K, V


def make_inputs(w: Workload, heads=None, threads: int = 8):
    """Q, K, V as float32 [b, len(heads), L, d] (bf16-exact for bf16 workloads).

    ``heads`` selects a subset of head ids (default: all); each head's draw is
    independent of the others, so a subset equals the same slice of the full set.
    """
    heads = list(range(w.heads)) if heads is None else list(heads)
    if w.batch != 1:
        raise ValueError("the workloads here have batch 1")
    with ThreadPoolExecutor(max_workers=max(1, min(threads, len(heads)))) as ex:
        per_head = list(ex.map(lambda hh: _head_tensors(w, hh), heads))
    Q = np.stack([t[0] for t in per_head])[None]
    K = np.stack([t[1] for t in per_head])[None]
    V = np.stack([t[2] for t in per_head])[None]
    return Q, K, V


def block_mask_multimodal(num_text_blocks: int, num_image_blocks: int,
                          window: int, global_stride: int) -> np.ndarray:
    """Binary block mask of the block-sparse notes, section 4.2 (1 = compute).

    text<->text, text->image and image->text are fully connected; image->image
    keeps |i - j| <= window, else columns j with j % global_stride == 0
    (indices counted within the image blocks).
    """
    T, I = num_text_blocks, num_image_blocks
    n = T + I
    mask = np.zeros((n, n), dtype=np.int8)
    mask[:T, :] = 1
    mask[:, :T] = 1
    for i in range(I):
        for j in range(I):
            if abs(i - j) <= window or j % global_stride == 0:
                mask[T + i, T + j] = 1
    return mask


def mask_to_idx(mask: np.ndarray, kmax: int | None = None) -> np.ndarray:
    """Row-wise ascending block-id lists of a binary mask, padded with -1."""
    rows = [np.nonzero(r)[0] for r in mask]
    kmax = max(len(r) for r in rows) if kmax is None else kmax
    idx = np.full((mask.shape[0], kmax), -1, dtype=np.int32)
    for i, r in enumerate(rows):
        idx[i, :len(r)] = r
    return idx


def idx_fixed_mask(w: Workload) -> np.ndarray:
    """idx [b, h, nqb, kmax] of the multimodal workload: 8 text blocks and 64
    image blocks, image window +-2 blocks, 2 global image blocks (stride 32, so
    image blocks 0 and 32), same mask for every head."""
    if w.wid != 5:
        raise ValueError("fixed mask belongs to the multimodal workload")
    T = w.text_tokens // w.block
    I = (w.seq_len - w.text_tokens) // w.block
    mask = block_mask_multimodal(T, I, window=2, global_stride=I // 2)
    idx = mask_to_idx(mask, kmax=T + I)
    return np.broadcast_to(idx, (w.batch, w.heads) + idx.shape).copy()
