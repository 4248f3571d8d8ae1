"""ctypes wrapper of the CPU oracle (``lsa_oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
CPU-baseline leg of the benchmark, never by the product path.  It shares no
code with the GPU library.  All arrays are host numpy arrays; bf16 tensors
are passed as their raw ``uint16`` bit patterns.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "lsa_oracle.c")
_LIB = os.path.join(_HERE, "liblsa_oracle.so")

_i64 = ctypes.c_int64
_p = ctypes.c_void_p


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (fp64, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call([
            "gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off",
            "-fno-fast-math", "-fPIC", "-shared", "-Wall", "-Wextra",
            "-Wno-unused-parameter", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        path = os.environ.get("LSA_ORACLE_LIB")   # a deliberately broken build, for mutation tests
        if not path:
            path = _LIB
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build(force=True)
        L = ctypes.CDLL(path)
        L.orc_num_threads.restype = ctypes.c_int
        L.orc_block_means.argtypes = [_p, _i64, _i64, _i64, _i64, _p]
        L.orc_route_causal.argtypes = [_p, _p] + [_i64] * 8 + [_p, _i64, _p, _p]
        L.orc_route_image.argtypes = [_p, _p] + [_i64] * 6 + [_p, _i64, _p, _p]
        L.orc_route_scores.argtypes = [_p, _p, _p] + [_i64] * 8 + [_p, _i64, _p]
        L.orc_route_consensus.argtypes = [_p, _p, _p] + [_i64] * 9 + [_p, _i64, _p, _p, _p]
        L.orc_route_cumulant.argtypes = [_p, _p, _p] + [_i64] * 8 + [ctypes.c_double, _p, _i64,
                                                                     _p, _p, _p]
        L.orc_route_tree.argtypes = [_p, _p, _p] + [_i64] * 11 + [_p, _i64, _p, _p, _p, _p, _p]
        L.orc_attend.argtypes = [_p, _p, _p] + [_i64] * 9 + [ctypes.c_double, _p, _i64, _p, _p]
        L.orc_forward.argtypes = [_p, _p, _p] + [_i64] * 9 + [ctypes.c_double, _p, _i64, _p, _p]
        for f in ("orc_block_means", "orc_route_causal", "orc_route_image",
                  "orc_route_scores", "orc_route_consensus", "orc_route_cumulant",
                  "orc_route_tree", "orc_attend", "orc_forward"):
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


def num_threads() -> int:
    return int(lib().orc_num_threads())


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"oracle {what} failed with code {rc}")


def _rows(rows):
    if rows is None:
        return None, 0
    r = _c(rows, np.int64).ravel()
    return r, r.size


def block_means(x: np.ndarray, block: int) -> np.ndarray:
    """x: uint16 bf16 bits [..., N, D] -> fp32 [..., N/block, D]."""
    x = _c(x, np.uint16)
    *lead, N, D = x.shape
    BH = int(np.prod(lead)) if lead else 1
    out = np.empty((*lead, N // block, D), dtype=np.float32)
    _check(lib().orc_block_means(_ptr(x), BH, N, D, block, _ptr(out)), "block_means")
    return out


def route_causal(q, kbar, block, top_k, window, rows=None, with_gap=False):
    """Causal routing.  q: bf16 bits [B,Hq,N,D]; kbar: fp32 [B,Hkv,N/block,D].
    Returns idx [n_rows, top_k] (or [B,Hq,N,top_k] when rows is None) and,
    with with_gap, the k-th / (k+1)-th score gap per row."""
    q = _c(q, np.uint16)
    kbar = _c(kbar, np.float32)
    B, Hq, N, D = q.shape
    Hkv = kbar.shape[1]
    r, n = _rows(rows)
    total = n if r is not None else B * Hq * N
    idx = np.empty((total, top_k), dtype=np.int32)
    gap = np.empty(total, dtype=np.float64) if with_gap else None
    _check(lib().orc_route_causal(_ptr(q), _ptr(kbar), B, Hq, Hkv, N, D, block,
                                  top_k, window, _ptr(r), n, _ptr(idx), _ptr(gap)),
           "route_causal")
    if r is None:
        idx = idx.reshape(B, Hq, N, top_k)
        if gap is not None:
            gap = gap.reshape(B, Hq, N)
    return (idx, gap) if with_gap else idx


def route_image(qbar, kbar, top_k, rows=None, with_gap=False):
    """Image-mode routing.  qbar: fp32 [B,Hq,nb,D]; kbar: fp32 [B,Hkv,nb,D].
    Returns idx [n_rows, top_k] (or [B,Hq,nb,top_k])."""
    qbar = _c(qbar, np.float32)
    kbar = _c(kbar, np.float32)
    B, Hq, nb, D = qbar.shape
    Hkv = kbar.shape[1]
    r, n = _rows(rows)
    total = n if r is not None else B * Hq * nb
    idx = np.empty((total, top_k), dtype=np.int32)
    gap = np.empty(total, dtype=np.float64) if with_gap else None
    _check(lib().orc_route_image(_ptr(qbar), _ptr(kbar), B, Hq, Hkv, nb, D, top_k,
                                 _ptr(r), n, _ptr(idx), _ptr(gap)), "route_image")
    if r is None:
        idx = idx.reshape(B, Hq, nb, top_k)
        if gap is not None:
            gap = gap.reshape(B, Hq, nb)
    return (idx, gap) if with_gap else idx


def route_scores(kbar, rows, *, q=None, qbar=None, block, window=0, causal=1, seq_len=None):
    """Every block's routing score (fp64) for the given rows, -inf where the
    block is not a candidate.  Returns [n_rows, nb]."""
    kbar = _c(kbar, np.float32)
    B, Hkv, nb, D = kbar.shape
    r, n = _rows(rows)
    if causal:
        q = _c(q, np.uint16)
        Hq, N = q.shape[1], q.shape[2]
    else:
        qbar = _c(qbar, np.float32)
        Hq, N = qbar.shape[1], nb * block
    out = np.empty((n, nb), dtype=np.float64)
    _check(lib().orc_route_scores(_ptr(q), _ptr(qbar), _ptr(kbar), B, Hq, Hkv, N, D,
                                  block, window, int(causal), _ptr(r), n, _ptr(out)),
           "route_scores")
    return out


def route_cumulant(q, k, kbar, block, top_k, window, beta, rows=None, with_gap=False,
                   with_scores=False):
    """Causal routing by the second-cumulant score <q, mu_c> + (beta/2)
    q^T Sigma_c q.  q bf16 bits [B,Hq,N,D], k bf16 bits [B,Hkv,N,D], kbar the
    fp32 block means.  Returns idx [n_rows, top_k] (or [B,Hq,N,top_k] when
    rows is None), then the gap per row and every block's score [n_rows, nb]
    when asked for."""
    q, k = _c(q, np.uint16), _c(k, np.uint16)
    kbar = _c(kbar, np.float32)
    B, Hq, N, D = q.shape
    Hkv, nb = k.shape[1], kbar.shape[2]
    r, n = _rows(rows)
    total = n if r is not None else B * Hq * N
    idx = np.empty((total, top_k), dtype=np.int32)
    gap = np.empty(total, dtype=np.float64) if with_gap else None
    sc = np.empty((total, nb), dtype=np.float64) if with_scores else None
    _check(lib().orc_route_cumulant(_ptr(q), _ptr(k), _ptr(kbar), B, Hq, Hkv, N, D, block, top_k,
                                    window, float(beta), _ptr(r), n, _ptr(idx), _ptr(gap),
                                    _ptr(sc)), "route_cumulant")
    if r is None:
        idx = idx.reshape(B, Hq, N, top_k)
        if gap is not None:
            gap = gap.reshape(B, Hq, N)
    res = (idx,) + ((gap,) if with_gap else ()) + ((sc,) if with_scores else ())
    return res if len(res) > 1 else idx


def route_tree(kbar, block, top_k, beam, *, q=None, qbar=None, window=0, causal=1, fanout=16,
               rows=None, details=False):
    """Two-level routing: nodes of `fanout` blocks summarised by the mean of
    their block means, the best `beam` complete candidate nodes kept, then
    top-k over the kept nodes' blocks plus the incomplete tail.  Causal: q
    bf16 bits [B,Hq,N,D]; image mode: qbar fp32 [B,Hq,nb,D].  Returns idx
    [n_rows, top_k] (or [B,Hq,P,top_k] when rows is None); with details,
    also a dict of per-row gap1 (node level), gap2 (block level), node
    scores [n_rows, nb // fanout] and the kept nodes [n_rows, beam]."""
    kbar = _c(kbar, np.float32)
    B, Hkv, nb, D = kbar.shape
    if causal:
        q = _c(q, np.uint16)
        Hq, N = q.shape[1], q.shape[2]
        per = N
    else:
        qbar = _c(qbar, np.float32)
        Hq, N = qbar.shape[1], nb * block
        per = nb
    r, n = _rows(rows)
    total = n if r is not None else B * Hq * per
    idx = np.empty((total, top_k), dtype=np.int32)
    nn = nb // fanout
    g1 = np.empty(total, np.float64) if details else None
    g2 = np.empty(total, np.float64) if details else None
    ns = np.empty((total, max(nn, 1)), np.float64) if details else None
    bo = np.empty((total, beam), np.int32) if details else None
    _check(lib().orc_route_tree(_ptr(q), _ptr(qbar), _ptr(kbar), B, Hq, Hkv, N, D, block, top_k,
                                window, int(causal), fanout, beam, _ptr(r), n, _ptr(idx),
                                _ptr(g1), _ptr(g2), _ptr(ns), _ptr(bo)), "route_tree")
    if r is None:
        idx = idx.reshape(B, Hq, per, top_k)
    if details:
        return idx, {"gap1": g1, "gap2": g2, "node_scores": ns[:, :nn], "beam": bo}
    return idx


def route_consensus(kbar, block, top_k, *, q=None, qbar=None, window=0, causal=1, rows=None,
                    with_gap=False, with_scores=False):
    """Consensus routing, one route per KV group, scored by the sum of the
    group's query heads' routing scores.  Causal: q bf16 bits [B,Hq,N,D],
    rows (b*Hkv + g)*N + t.  Image mode: qbar fp32 [B,Hq,nb,D], rows
    (b*Hkv + g)*nb + i.  Returns idx [n_rows, top_k] (or [B,Hkv,P,top_k]
    when rows is None), then the gap per row and every block's score
    [n_rows, nb] when asked for."""
    kbar = _c(kbar, np.float32)
    B, Hkv, nb, D = kbar.shape
    if causal:
        q = _c(q, np.uint16)
        Hq, N = q.shape[1], q.shape[2]
        per = N
    else:
        qbar = _c(qbar, np.float32)
        Hq, N = qbar.shape[1], nb * block
        per = nb
    r, n = _rows(rows)
    total = n if r is not None else B * Hkv * per
    idx = np.empty((total, top_k), dtype=np.int32)
    gap = np.empty(total, dtype=np.float64) if with_gap else None
    sc = np.empty((total, nb), dtype=np.float64) if with_scores else None
    _check(lib().orc_route_consensus(_ptr(q), _ptr(qbar), _ptr(kbar), B, Hq, Hkv, N, D, block,
                                     top_k, window, int(causal), _ptr(r), n, _ptr(idx),
                                     _ptr(gap), _ptr(sc)), "route_consensus")
    if r is None:
        idx = idx.reshape(B, Hkv, per, top_k)
        if gap is not None:
            gap = gap.reshape(B, Hkv, per)
    res = (idx,) + ((gap,) if with_gap else ()) + ((sc,) if with_scores else ())
    return res if len(res) > 1 else idx


def consensus_rows(rows, q_heads, kv_heads, per):
    """The group row (b*Hkv + g)*per + p that serves query row
    (b*Hq + h)*per + p."""
    rows = np.asarray(rows, dtype=np.int64)
    bh, p = rows // per, rows % per
    b, h = bh // q_heads, bh % q_heads
    return (b * kv_heads + h // (q_heads // kv_heads)) * per + p


def forward_consensus(q, k, v, block, top_k, window, causal, scale=0.0, rows=None):
    """Steps 1-4 with consensus routing: block means, one route per KV group
    (image mode: per KV group and query block), the group's route shared by
    its query heads, attention.  Returns (out, sel) shaped as forward's."""
    q, k, v = (_c(a, np.uint16) for a in (q, k, v))
    B, Hq, N, D = q.shape
    Hkv = k.shape[1]
    kbar = block_means(k, block)
    qrows = np.arange(B * Hq * N, dtype=np.int64) if rows is None else _c(rows, np.int64).ravel()
    if causal:
        grows = consensus_rows(qrows, Hq, Hkv, N)
        uniq, inv = np.unique(grows, return_inverse=True)
        gidx = route_consensus(kbar, block, top_k, q=q, window=window, causal=1, rows=uniq)
    else:
        nb = N // block
        qb = (qrows // N) * nb + (qrows % N) // block
        grows = consensus_rows(qb, Hq, Hkv, nb)
        uniq, inv = np.unique(grows, return_inverse=True)
        gidx = route_consensus(kbar, block, top_k, qbar=block_means(q, block), causal=0, rows=uniq)
    sel = np.ascontiguousarray(gidx[inv.ravel()])
    out = attend(q, k, v, sel, block, top_k, window, causal, scale, rows=qrows)
    if rows is None:
        return out.reshape(B, Hq, N, D), sel.reshape(B, Hq, N, top_k)
    return out, sel


def attend(q, k, v, sel, block, top_k, window, causal, scale=0.0, rows=None):
    """Exact softmax over routed blocks (+ causal window).  sel: [n_rows, top_k]
    aligned with rows (image mode: the row's query-block selection).
    Returns fp32 [n_rows, D] (or [B,Hq,N,D] when rows is None)."""
    q, k, v = (_c(a, np.uint16) for a in (q, k, v))
    sel = _c(sel, np.int32)
    B, Hq, N, D = q.shape
    Hkv = k.shape[1]
    r, n = _rows(rows)
    total = n if r is not None else B * Hq * N
    assert sel.size == total * top_k, (sel.shape, total, top_k)
    out = np.empty((total, D), dtype=np.float32)
    _check(lib().orc_attend(_ptr(q), _ptr(k), _ptr(v), B, Hq, Hkv, N, D, block, top_k,
                            window, int(causal), float(scale), _ptr(r), n, _ptr(sel),
                            _ptr(out)), "attend")
    return out.reshape(B, Hq, N, D) if r is None else out


def forward(q, k, v, block, top_k, window, causal, scale=0.0, rows=None):
    """Steps 1-4 end to end.  Returns (out [n_rows, D], sel [n_rows, top_k])
    (full [B,Hq,N,...] shapes when rows is None)."""
    q, k, v = (_c(a, np.uint16) for a in (q, k, v))
    B, Hq, N, D = q.shape
    Hkv = k.shape[1]
    r, n = _rows(rows)
    total = n if r is not None else B * Hq * N
    out = np.empty((total, D), dtype=np.float32)
    sel = np.empty((total, top_k), dtype=np.int32)
    _check(lib().orc_forward(_ptr(q), _ptr(k), _ptr(v), B, Hq, Hkv, N, D, block, top_k,
                             window, int(causal), float(scale), _ptr(r), n, _ptr(sel),
                             _ptr(out)), "forward")
    if r is None:
        return out.reshape(B, Hq, N, D), sel.reshape(B, Hq, N, top_k)
    return out, sel
