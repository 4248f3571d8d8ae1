"""Seeded synthetic inputs for content-routed block sparse attention.

This module only draws tensors.  It holds none of the method's arithmetic
(no block means, no routing scores, no selection, no softmax), so both the
GPU path and the CPU oracle can consume exactly the same bytes.

Every tensor is bf16, stored as raw ``uint16`` bit patterns, laid out
``[B, H, N, D]`` with D fastest.  Floats are drawn in float32 from numpy's
PCG64 (one child ``SeedSequence`` per tensor) and rounded once to bf16 with
round-to-nearest-even.

Workloads (sizes follow the problem statement of the pages: Q/K/V
``[B,H,N,D]`` with grouped-query heads, a key block size, top-k, a local
causal window and a causal flag):

* ``tiny_causal_n1024``    B1 Hq2 Hkv1 N1024 D64, block 64, top-k 4, window 128,
  causal; Q, K, V ~ N(0,1).
* ``qwen05b_n32k``         B1 Hq14 Hkv2 N32768 D64, block 64, top-k 16, window 512,
  causal; Q, K = 0.5*N(0,1) + 2*U_g[topic(t)], 64 topics; V ~ N(0,1).
* ``qwen05b_n128k_needles`` the same at N=131072 plus 32 planted needle keys.
* ``image_zorder_128x128`` B4 H16 (no GQA) N16384 D64, block 16, top-k 8, no window,
  non-causal; a smooth Gaussian random field (correlation length 8 px) per
  image, projected to Q/K/V by fixed random matrices, tokens in Z-order.
* ``qwen05b_n1m_needles``  as the 32K layer at N=1048576 with 256 topics and
  128 needles.

The head counts (14 query / 2 KV heads, D=64) are the Qwen2.5-0.5B attention
shape used by the SSA page (jonsmirl/ssa, "Sparse reads plus bounded tail
state": 336 gains over 24 layers and 49,920 summary scalars imply 14 query
heads, 2 KV heads and D=64).  The Z-order is the quadtree token permutation
the LLSA page recommends for images ("Preprocessing for Non-Sequential
Data"), with the row bit above the column bit at every level.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "Inputs", "Needle", "generate",
    "to_bf16_bits", "bf16_bits_to_f32", "zorder_permutation",
]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    q_heads: int
    kv_heads: int
    seq_len: int
    head_dim: int
    block: int
    top_k: int
    window: int
    causal: int
    dist: str            # "normal" | "topics" | "grf"
    topics: int = 0
    needles: int = 0
    seed: int = 0
    image_side: int = 0  # grf only: the image is image_side x image_side pixels

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS: Dict[str, Workload] = {
    w.name: w for w in [
        Workload("tiny_causal_n1024", 1, 2, 1, 1024, 64, 64, 4, 128, 1,
                 "normal", seed=0),
        Workload("qwen05b_n32k", 1, 14, 2, 32768, 64, 64, 16, 512, 1,
                 "topics", topics=64, seed=1),
        Workload("qwen05b_n128k_needles", 1, 14, 2, 131072, 64, 64, 16, 512, 1,
                 "topics", topics=64, needles=32, seed=2),
        Workload("image_zorder_128x128", 4, 16, 16, 16384, 64, 16, 8, 0, 0,
                 "grf", seed=3, image_side=128),
        Workload("qwen05b_n1m_needles", 1, 14, 2, 1048576, 64, 64, 16, 512, 1,
                 "topics", topics=256, needles=128, seed=4),
    ]
}


@dataclasses.dataclass(frozen=True)
class Needle:
    b: int   # batch
    g: int   # KV head whose key was overwritten
    h: int   # query head whose query was copied
    t: int   # query position
    p: int   # key position that now holds 4 * q


@dataclasses.dataclass
class Inputs:
    workload: Workload
    q: np.ndarray          # uint16 bf16 bits [B, Hq, N, D]
    k: np.ndarray          # uint16 bf16 bits [B, Hkv, N, D]
    v: np.ndarray          # uint16 bf16 bits [B, Hkv, N, D]
    needles: List[Needle]


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit pattern, round to nearest, ties to even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit pattern -> float32 (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32)
            << np.uint32(16)).view(np.float32)


def zorder_permutation(side: int) -> np.ndarray:
    """perm[s] = raster index (row*side + col) of the pixel at sequence slot s.

    Slot s is the Morton code of the pixel: bits of row and column
    interleaved, the row bit above the column bit at each level, so each
    aligned run of 4**j slots is a 2**j x 2**j square of the image.
    """
    assert side > 0 and side & (side - 1) == 0
    r, c = np.meshgrid(np.arange(side, dtype=np.int64),
                       np.arange(side, dtype=np.int64), indexing="ij")
    code = np.zeros_like(r)
    for i in range(int(side).bit_length() - 1):
        code |= ((r >> i) & 1) << (2 * i + 1)
        code |= ((c >> i) & 1) << (2 * i)
    perm = np.empty(side * side, dtype=np.int64)
    perm[code.ravel()] = np.arange(side * side, dtype=np.int64)
    return perm


def _rngs(seed: int, n: int) -> List[np.random.Generator]:
    return [np.random.Generator(np.random.PCG64(s))
            for s in np.random.SeedSequence(seed).spawn(n)]


def _unit_rows(rng: np.random.Generator, n: int, d: int) -> np.ndarray:
    u = rng.standard_normal((n, d))
    return (u / np.linalg.norm(u, axis=1, keepdims=True)).astype(np.float32)


def _gen_normal(w: Workload, rngs):
    B, Hq, Hkv, N, D = w.batch, w.q_heads, w.kv_heads, w.seq_len, w.head_dim
    q = to_bf16_bits(rngs[0].standard_normal((B, Hq, N, D), dtype=np.float32))
    k = to_bf16_bits(rngs[1].standard_normal((B, Hkv, N, D), dtype=np.float32))
    v = to_bf16_bits(rngs[2].standard_normal((B, Hkv, N, D), dtype=np.float32))
    return q, k, v


def _gen_topics(w: Workload, rngs):
    """Q, K = 0.5*N(0,1) + 2*U_g[topic(t)]: one i.i.d. uniform topic per token,
    shared by every head; each KV group g has its own unit topic directions,
    used by its keys and by the query heads of that group."""
    B, Hq, Hkv, N, D = w.batch, w.q_heads, w.kv_heads, w.seq_len, w.head_dim
    rep = Hq // Hkv
    q = np.empty((B, Hq, N, D), dtype=np.uint16)
    k = np.empty((B, Hkv, N, D), dtype=np.uint16)
    v = np.empty((B, Hkv, N, D), dtype=np.uint16)
    r_topic, r_dir, r_k, r_q, r_v = rngs[0], rngs[1], rngs[2], rngs[3], rngs[4]
    for b in range(B):
        topic = r_topic.integers(0, w.topics, size=N)
        for g in range(Hkv):
            U = _unit_rows(r_dir, w.topics, D)
            sig = 2.0 * U[topic]                                  # [N, D]
            k[b, g] = to_bf16_bits(0.5 * r_k.standard_normal((N, D), dtype=np.float32) + sig)
            for h in range(g * rep, (g + 1) * rep):
                q[b, h] = to_bf16_bits(0.5 * r_q.standard_normal((N, D), dtype=np.float32) + sig)
            v[b, g] = to_bf16_bits(r_v.standard_normal((N, D), dtype=np.float32))
            del sig
    return q, k, v


def _plant_needles(w: Workload, q: np.ndarray, k: np.ndarray, rng) -> List[Needle]:
    """Overwrite key p of KV head g with 4 * (query t of head h in g).

    The needle key lies at least window + block positions before its query,
    so its block is complete and lies before the local window of that query.
    Needle blocks are distinct.
    """
    B, Hq, Hkv, N = w.batch, w.q_heads, w.kv_heads, w.seq_len
    rep = Hq // Hkv
    bs, W = w.block, w.window
    lo_t = W + 2 * bs
    used = set()
    out: List[Needle] = []
    while len(out) < w.needles:
        b = int(rng.integers(0, B))
        g = int(rng.integers(0, Hkv))
        h = g * rep + int(rng.integers(0, rep))
        t = int(rng.integers(lo_t, N))
        p = int(rng.integers(0, t - W - bs + 1))
        blk = (b, g, p // bs)
        if blk in used:
            continue
        used.add(blk)
        qf = bf16_bits_to_f32(q[b, h, t])
        k[b, g, p] = to_bf16_bits(4.0 * qf)   # exact: scaling by 4 keeps bf16
        out.append(Needle(b, g, h, t, p))
    return out


def _gaussian_kernel_fft(side: int, corr_len: float) -> np.ndarray:
    """rfft2 of a periodic Gaussian smoothing kernel, scaled so that smoothing
    unit white noise gives unit variance and covariance exp(-r^2/(2 l^2))."""
    sigma = corr_len / np.sqrt(2.0)
    d = np.minimum(np.arange(side), side - np.arange(side)).astype(np.float64)
    g = np.exp(-(d[:, None] ** 2 + d[None, :] ** 2) / (2.0 * sigma ** 2))
    g /= np.sqrt((g ** 2).sum())
    return np.fft.rfft2(g)


def _gen_grf(w: Workload, rngs):
    """Per image: H*D channels of periodic smooth Gaussian noise with
    correlation length 8 px, projected by three fixed N(0, 1/C) matrices to
    Q, K, V, tokens placed in Z-order, reshaped to [H, N, D]."""
    B, H, N, D = w.batch, w.q_heads, w.seq_len, w.head_dim
    side = w.image_side
    assert side * side == N and w.kv_heads == H
    C = H * D
    r_field, r_w = rngs[0], rngs[1]
    Wq, Wk, Wv = (r_w.standard_normal((C, C), dtype=np.float32) / np.float32(np.sqrt(C))
                  for _ in range(3))
    G = _gaussian_kernel_fft(side, 8.0)
    perm = zorder_permutation(side)
    outs = [np.empty((B, H, N, D), dtype=np.uint16) for _ in range(3)]
    for b in range(B):
        x = np.empty((N, C), dtype=np.float32)
        for c0 in range(0, C, 128):
            white = r_field.standard_normal((128, side, side), dtype=np.float32)
            sm = np.fft.irfft2(np.fft.rfft2(white) * G, s=(side, side))
            x[:, c0:c0 + 128] = sm.reshape(128, N).T
        x = x[perm]                                   # raster -> Z-order
        for o, Wm in zip(outs, (Wq, Wk, Wv)):
            y = (x @ Wm).reshape(N, H, D).transpose(1, 0, 2)
            o[b] = to_bf16_bits(y)
    return outs[0], outs[1], outs[2]


def generate(w: Workload, seed: Optional[int] = None) -> Inputs:
    """Draw the workload's Q, K, V (bf16 bits) and needles, deterministically."""
    seed = w.seed if seed is None else seed
    rngs = _rngs(seed, 8)
    if w.dist == "normal":
        q, k, v = _gen_normal(w, rngs)
    elif w.dist == "topics":
        q, k, v = _gen_topics(w, rngs)
    elif w.dist == "grf":
        q, k, v = _gen_grf(w, rngs)
    else:
        raise ValueError(f"unknown distribution {w.dist!r}")
    needles: List[Needle] = []
    if w.needles:
        needles = _plant_needles(w, q, k, rngs[7])
    return Inputs(w, q, k, v, needles)
