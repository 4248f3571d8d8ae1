"""Thin Python binding of liblsa.so (the C ABI in include/lsa.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI.  PyTorch provides device memory and the current
HIP stream.  Importing this module fails loudly when liblsa.so has not been
built; there is no fallback path.

Tensors are torch tensors on the GPU, contiguous, laid out [B, H, N, D];
bf16 inputs may be torch.bfloat16 or torch.uint16/int16 bit patterns.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "liblsa.so")
if not os.path.exists(_LIB_PATH):
    raise ImportError(
        f"{_LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'` "
        "or `python content_routed_block_amd/build.py`")

_lib = ctypes.CDLL(_LIB_PATH)

OP_SUMMARIZE, OP_ROUTE, OP_ATTEND, OP_FORWARD, OP_DECODE = 0, 1, 2, 3, 4
STATUS = {0: "LSA_OK", 1: "LSA_ERR_NULL", 2: "LSA_ERR_SHAPE", 3: "LSA_ERR_UNSUPPORTED",
          4: "LSA_ERR_ALIGN", 5: "LSA_ERR_WORKSPACE", 6: "LSA_ERR_DEVICE", 7: "LSA_ERR_SCRATCH"}
STATIC_SCRATCH_BYTES = 16 << 20   # LSA_STATIC_SCRATCH_BYTES


class LsaParams(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("q_heads", ctypes.c_int32),
                ("kv_heads", ctypes.c_int32), ("seq_len", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("block", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("window", ctypes.c_int32),
                ("causal", ctypes.c_int32), ("scale", ctypes.c_float),
                ("consensus", ctypes.c_int32), ("beta", ctypes.c_float),
                ("beam", ctypes.c_int32), ("chunk", ctypes.c_int32)]


_P = ctypes.POINTER(LsaParams)
_v = ctypes.c_void_p
_lib.lsa_workspace_bytes.argtypes = [_P, ctypes.c_int32]
_lib.lsa_workspace_bytes.restype = ctypes.c_size_t
_lib.lsa_block_summarize.argtypes = [_P, _v, ctypes.c_int32, _v, _v]
_lib.lsa_route_topk.argtypes = [_P, _v, _v, _v, _v, ctypes.c_size_t, _v]
_lib.lsa_route_cumulant.argtypes = [_P, _v, _v, _v, _v]
_lib.lsa_route_cumulant.restype = ctypes.c_int
_lib.lsa_sparse_attend.argtypes = [_P, _v, _v, _v, _v, _v, _v, ctypes.c_size_t, _v]
_lib.lsa_forward.argtypes = [_P, _v, _v, _v, _v, _v, _v, ctypes.c_size_t, _v]
for _f in ("lsa_block_summarize", "lsa_route_topk", "lsa_sparse_attend", "lsa_forward"):
    getattr(_lib, _f).restype = ctypes.c_int
_lib.lsa_decode.argtypes = [_P, ctypes.c_int32, _v, _v, _v, _v, _v, _v, _v, ctypes.c_size_t, _v]
_lib.lsa_decode.restype = ctypes.c_int
_lib.lsa_decode_noalloc.argtypes = [_P, ctypes.c_int32, _v, _v, _v, _v, _v, _v, _v]
_lib.lsa_decode_noalloc.restype = ctypes.c_int
_lib.lsa_forward_profiled.argtypes = [_P, _v, _v, _v, _v, _v, _v, ctypes.c_size_t, _v, _v]
_lib.lsa_forward_profiled.restype = ctypes.c_int
_lib.lsa_status_str.argtypes = [ctypes.c_int]
_lib.lsa_status_str.restype = ctypes.c_char_p

SIZE_MAX = (1 << 64) - 1
PROFILE_EVENTS = 9
PROFILE_STAGES = ["key summary", "routing", "routing fallback", "V transpose + bucket count",
                  "bucket scan",
                  "bucket scatter", "routed-block partials", "window + merge"]

# HIP event calls resolve through liblsa's own dependency (the process's single
# libamdhip64, already loaded by torch).
_lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
_lib.hipEventCreate.restype = ctypes.c_int
_lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
_lib.hipEventDestroy.restype = ctypes.c_int
_lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                     ctypes.c_void_p]
_lib.hipEventElapsedTime.restype = ctypes.c_int


class LsaError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: {STATUS.get(code, code)} ({_lib.lsa_status_str(code).decode()})")
        self.code = code


def library():
    return _lib


def params(batch, q_heads, kv_heads, seq_len, head_dim=64, block=64, top_k=16, window=512,
           causal=1, scale=0.0, consensus=0, beta=0.0, beam=0, chunk=0) -> LsaParams:
    return LsaParams(batch, q_heads, kv_heads, seq_len, head_dim, block, top_k, window, causal,
                     float(scale), consensus, float(beta), beam, chunk)


def idx_shape(p: LsaParams):
    """Shape of the routing output: [B, heads, rows, top_k] with heads = Hq
    (Hkv with consensus routing) and rows = N (N / block in image mode)."""
    heads = p.kv_heads if p.consensus else p.q_heads
    return (p.batch, heads, p.seq_len if p.causal else p.seq_len // p.block, p.top_k)


def workspace_bytes(p: LsaParams, op: int) -> int:
    n = _lib.lsa_workspace_bytes(ctypes.byref(p), op)
    if n == SIZE_MAX:
        raise LsaError(2, "lsa_workspace_bytes")
    return n


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _bits(t: torch.Tensor, shape, name) -> torch.Tensor:
    if t.dtype not in (torch.bfloat16, torch.uint16, torch.int16):
        raise TypeError(f"{name}: expected bf16 data, got {t.dtype}")
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous GPU tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


def _tensor(t: torch.Tensor, dtype, shape, name) -> torch.Tensor:
    if t.dtype != dtype or not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous GPU {dtype} tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


def _check(code: int, what: str):
    if code != 0:
        raise LsaError(code, what)


def _on(stream):
    """The torch stream a call runs on: `stream`, or the current stream.

    Every buffer a call allocates for itself (workspace, and out / idx when
    the caller passes none) is allocated while that stream is current, so
    torch's caching allocator ties it to the stream the kernels run on: once
    freed it is handed out again only to work ordered after those kernels."""
    return torch.cuda.current_stream() if stream is None else stream


def _workspace(p, op, workspace, device):
    need = workspace_bytes(p, op)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return workspace, nbytes


def block_summarize(p: LsaParams, x: torch.Tensor, heads: Optional[int] = None,
                    out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    heads = p.kv_heads if heads is None else heads
    x = _bits(x, (p.batch, heads, p.seq_len, p.head_dim), "x")
    nb = p.seq_len // p.block
    s = _on(stream)
    if out is None:
        with torch.cuda.stream(s):
            out = torch.empty((p.batch, heads, nb, p.head_dim), dtype=torch.float32,
                              device=x.device)
    _check(_lib.lsa_block_summarize(ctypes.byref(p), _ptr(x), heads, _ptr(out), _stream(s)),
           "lsa_block_summarize")
    return out


def route_topk(p: LsaParams, q: torch.Tensor, kbar: torch.Tensor,
               idx: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
               stream=None) -> torch.Tensor:
    q = _bits(q, (p.batch, p.q_heads, p.seq_len, p.head_dim), "q")
    _tensor(kbar, torch.float32, (p.batch, p.kv_heads, p.seq_len // p.block, p.head_dim), "kbar")
    s = _on(stream)
    with torch.cuda.stream(s):
        if idx is None:
            idx = torch.empty(idx_shape(p), dtype=torch.int32, device=q.device)
        workspace, nbytes = _workspace(p, OP_ROUTE, workspace, q.device)
    _tensor(idx, torch.int32, idx_shape(p), "idx")
    _check(_lib.lsa_route_topk(ctypes.byref(p), _ptr(q), _ptr(kbar), _ptr(idx), _ptr(workspace),
                               nbytes, _stream(s)), "lsa_route_topk")
    return idx


def route_cumulant(p: LsaParams, q: torch.Tensor, k: torch.Tensor,
                   idx: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Routing by the second-cumulant score with weight p.beta (see
    lsa_route_cumulant)."""
    q = _bits(q, (p.batch, p.q_heads, p.seq_len, p.head_dim), "q")
    k = _bits(k, (p.batch, p.kv_heads, p.seq_len, p.head_dim), "k")
    s = _on(stream)
    if idx is None:
        with torch.cuda.stream(s):
            idx = torch.empty(idx_shape(p), dtype=torch.int32, device=q.device)
    _tensor(idx, torch.int32, idx_shape(p), "idx")
    _check(_lib.lsa_route_cumulant(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(idx), _stream(s)),
           "lsa_route_cumulant")
    return idx


def sparse_attend(p: LsaParams, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                  idx: torch.Tensor, out: Optional[torch.Tensor] = None,
                  workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    q = _bits(q, (p.batch, p.q_heads, p.seq_len, p.head_dim), "q")
    k = _bits(k, (p.batch, p.kv_heads, p.seq_len, p.head_dim), "k")
    v = _bits(v, (p.batch, p.kv_heads, p.seq_len, p.head_dim), "v")
    _tensor(idx, torch.int32, idx_shape(p), "idx")
    s = _on(stream)
    with torch.cuda.stream(s):
        if out is None:
            out = torch.empty((p.batch, p.q_heads, p.seq_len, p.head_dim), dtype=torch.float32,
                              device=q.device)
        workspace, nbytes = _workspace(p, OP_ATTEND, workspace, q.device)
    _tensor(out, torch.float32, (p.batch, p.q_heads, p.seq_len, p.head_dim), "out")
    _check(_lib.lsa_sparse_attend(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(idx), _ptr(out),
                                  _ptr(workspace), nbytes, _stream(s)), "lsa_sparse_attend")
    return out


def forward(p: LsaParams, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
            out: Optional[torch.Tensor] = None, idx: Optional[torch.Tensor] = None,
            want_idx: bool = True, workspace: Optional[torch.Tensor] = None,
            stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    q = _bits(q, (p.batch, p.q_heads, p.seq_len, p.head_dim), "q")
    k = _bits(k, (p.batch, p.kv_heads, p.seq_len, p.head_dim), "k")
    v = _bits(v, (p.batch, p.kv_heads, p.seq_len, p.head_dim), "v")
    s = _on(stream)
    with torch.cuda.stream(s):
        if out is None:
            out = torch.empty((p.batch, p.q_heads, p.seq_len, p.head_dim), dtype=torch.float32,
                              device=q.device)
        if idx is None and want_idx:
            idx = torch.empty(idx_shape(p), dtype=torch.int32, device=q.device)
        workspace, nbytes = _workspace(p, OP_FORWARD, workspace, q.device)
    _tensor(out, torch.float32, (p.batch, p.q_heads, p.seq_len, p.head_dim), "out")
    if idx is not None:
        _tensor(idx, torch.int32, idx_shape(p), "idx")
    _check(_lib.lsa_forward(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(idx),
                            _ptr(workspace), nbytes, _stream(s)), "lsa_forward")
    return out, idx


def _cache_params(p: LsaParams, cache_len: int) -> LsaParams:
    """p with seq_len = cache_len (the geometry decode workspaces are sized by)."""
    pc = LsaParams(*[getattr(p, f) for f, _ in LsaParams._fields_])
    pc.seq_len = cache_len
    return pc


def decode(p: LsaParams, cache_len: int, q: torch.Tensor, k_cache: torch.Tensor,
           v_cache: torch.Tensor, kbar_cache: torch.Tensor, out: Optional[torch.Tensor] = None,
           idx: Optional[torch.Tensor] = None, want_idx: bool = True,
           workspace: Optional[torch.Tensor] = None,
           stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """One decode step for the query at position p.seq_len - 1 (see lsa_decode).

    q [B, Hq, 64] bf16; k_cache, v_cache [B, Hkv, cache_len, 64] bf16;
    kbar_cache [B, Hkv, cache_len // block, 64] fp32 (updated in place when
    p.seq_len is a multiple of the block size)."""
    q = _bits(q, (p.batch, p.q_heads, p.head_dim), "q")
    k_cache = _bits(k_cache, (p.batch, p.kv_heads, cache_len, p.head_dim), "k_cache")
    v_cache = _bits(v_cache, (p.batch, p.kv_heads, cache_len, p.head_dim), "v_cache")
    if kbar_cache.dtype != torch.float32 or not kbar_cache.is_contiguous() or \
            tuple(kbar_cache.shape) != (p.batch, p.kv_heads, cache_len // p.block, p.head_dim):
        raise ValueError("kbar_cache: expected a contiguous fp32 tensor "
                         f"[{p.batch}, {p.kv_heads}, {cache_len // p.block}, {p.head_dim}]")
    s = _on(stream)
    with torch.cuda.stream(s):
        if out is None:
            out = torch.empty((p.batch, p.q_heads, p.head_dim), dtype=torch.float32,
                              device=q.device)
        if idx is None and want_idx:
            idx = torch.empty((p.batch, p.q_heads, p.top_k), dtype=torch.int32, device=q.device)
        if workspace is None:
            workspace = torch.empty(workspace_bytes(_cache_params(p, cache_len), OP_DECODE),
                                    dtype=torch.uint8, device=q.device)
    nbytes = workspace.numel() * workspace.element_size()
    _check(_lib.lsa_decode(ctypes.byref(p), cache_len, _ptr(q), _ptr(k_cache), _ptr(v_cache),
                           _ptr(kbar_cache), _ptr(out), _ptr(idx), _ptr(workspace), nbytes,
                           _stream(s)), "lsa_decode")
    return out, idx


def decode_noalloc(p: LsaParams, cache_len: int, q: torch.Tensor, k_cache: torch.Tensor,
                   v_cache: torch.Tensor, kbar_cache: torch.Tensor, out: torch.Tensor,
                   idx: Optional[torch.Tensor] = None, stream=None) -> None:
    """lsa_decode_noalloc: one decode step with the library's static scratch
    array instead of a workspace.  Allocates nothing: out (and idx, if wanted)
    must be preallocated.  Calls that overlap on one GPU race."""
    q = _bits(q, (p.batch, p.q_heads, p.head_dim), "q")
    k_cache = _bits(k_cache, (p.batch, p.kv_heads, cache_len, p.head_dim), "k_cache")
    v_cache = _bits(v_cache, (p.batch, p.kv_heads, cache_len, p.head_dim), "v_cache")
    _tensor(kbar_cache, torch.float32, (p.batch, p.kv_heads, cache_len // p.block, p.head_dim),
            "kbar_cache")
    _tensor(out, torch.float32, (p.batch, p.q_heads, p.head_dim), "out")
    if idx is not None:
        _tensor(idx, torch.int32, (p.batch, p.q_heads, p.top_k), "idx")
    _check(_lib.lsa_decode_noalloc(ctypes.byref(p), cache_len, _ptr(q), _ptr(k_cache),
                                   _ptr(v_cache), _ptr(kbar_cache), _ptr(out), _ptr(idx),
                                   _stream(_on(stream))), "lsa_decode_noalloc")


class StageEvents:
    """PROFILE_EVENTS HIP events for one lsa_forward_profiled call."""

    def __init__(self):
        self.handles = []
        for _ in range(PROFILE_EVENTS):
            h = ctypes.c_void_p()
            if _lib.hipEventCreate(ctypes.byref(h)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.handles.append(h)
        self.array = (ctypes.c_void_p * PROFILE_EVENTS)(*[h.value for h in self.handles])

    def stage_ms(self):
        """Durations (ms) of the PROFILE_EVENTS-1 stages; call after a sync."""
        out = []
        for i in range(1, PROFILE_EVENTS):
            ms = ctypes.c_float()
            if _lib.hipEventElapsedTime(ctypes.byref(ms), self.handles[i - 1], self.handles[i]) != 0:
                raise RuntimeError("hipEventElapsedTime failed")
            out.append(ms.value)
        return out

    def close(self):
        for h in self.handles:
            _lib.hipEventDestroy(h)
        self.handles = []


def forward_profiled(p: LsaParams, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                     events: StageEvents, out: torch.Tensor, idx: Optional[torch.Tensor],
                     workspace: torch.Tensor, stream=None) -> None:
    """lsa_forward recording the stage events (buffers must be preallocated)."""
    nbytes = workspace.numel() * workspace.element_size()
    _check(_lib.lsa_forward_profiled(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(out),
                                     _ptr(idx), _ptr(workspace), nbytes, _stream(stream),
                                     events.array), "lsa_forward_profiled")

