"""The C ABI library without a GPU: it loads, exports every function that
include/*.h declares, and its host-side validation returns the documented
status codes before anything is launched."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in sorted(os.listdir(os.path.join(ROOT, "include")))
           if h.endswith(".h")]
LIB = os.path.join(ROOT, "content_routed_block_amd", "liblsa.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="liblsa.so not built")


def declared_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(lsa_[a-z_]+)\s*\(", text))
    return sorted(names)


@pytest.fixture(scope="module")
def lsa():
    from content_routed_block_amd import lsa as m
    return m


def test_exports_every_declared_symbol():
    lib = ctypes.CDLL(LIB)
    names = declared_functions()
    assert set(names) >= {"lsa_block_summarize", "lsa_route_topk", "lsa_sparse_attend",
                          "lsa_forward", "lsa_workspace_bytes", "lsa_status_str"}
    for n in names:
        assert hasattr(lib, n), n


def test_struct_layout_matches_header(lsa):
    assert ctypes.sizeof(lsa.LsaParams) == 56
    assert lsa.LsaParams.beam.offset == 48
    assert lsa.LsaParams.chunk.offset == 52
    assert lsa.LsaParams.consensus.offset == 40
    assert lsa.LsaParams.beta.offset == 44


def good(lsa, **kw):
    base = dict(batch=1, q_heads=14, kv_heads=2, seq_len=131072, head_dim=64, block=64,
                top_k=16, window=512, causal=1)
    base.update(kw)
    return lsa.params(**base)


@pytest.mark.parametrize("kw,code", [
    (dict(q_heads=13), 2), (dict(seq_len=1000), 2), (dict(window=100), 2), (dict(window=32), 2),
    (dict(causal=0, window=512, block=16), 2), (dict(causal=2), 2), (dict(batch=0), 2),
    (dict(consensus=2), 2), (dict(consensus=-1), 2), (dict(beta=float("nan")), 2),
    (dict(beta=float("inf")), 2), (dict(beta=0.5, consensus=1), 3),
    (dict(beta=0.5, causal=0, window=0, block=16), 3), (dict(beam=-1), 2), (dict(beam=16), 3),
    (dict(beam=4, consensus=1), 3), (dict(beam=4, beta=0.5), 3),
    (dict(beam=4, causal=0, window=0, block=16, consensus=1), 3),
    (dict(chunk=-64), 2), (dict(chunk=32), 2), (dict(chunk=96), 2),
    (dict(head_dim=128), 3), (dict(top_k=33), 3), (dict(block=48, window=96, seq_len=960), 3),
    (dict(causal=0, window=0, block=64), 3), (dict(seq_len=1 << 24, block=16, window=512), 3),
])
def test_invalid_parameters(lsa, kw, code):
    p = good(lsa, **kw)
    assert lsa.library().lsa_workspace_bytes(ctypes.byref(p), lsa.OP_FORWARD) == lsa.SIZE_MAX
    dummy = ctypes.c_void_p(256)
    rc = lsa.library().lsa_forward(ctypes.byref(p), dummy, dummy, dummy, dummy, None, dummy,
                                   1 << 40, None)
    assert rc == code


def test_null_alignment_and_workspace_checks(lsa):
    L = lsa.library()
    p = good(lsa)
    a = ctypes.c_void_p(4096)
    assert L.lsa_forward(None, a, a, a, a, None, a, 1 << 40, None) == 1
    assert L.lsa_forward(ctypes.byref(p), None, a, a, a, None, a, 1 << 40, None) == 1
    assert L.lsa_forward(ctypes.byref(p), ctypes.c_void_p(4098), a, a, a, None, a, 1 << 40, None) == 4
    assert L.lsa_forward(ctypes.byref(p), a, a, a, a, None, ctypes.c_void_p(4096 + 16), 1 << 40, None) == 4
    need = lsa.workspace_bytes(p, lsa.OP_FORWARD)
    assert L.lsa_forward(ctypes.byref(p), a, a, a, a, None, a, need - 1, None) == 5
    assert L.lsa_route_topk(ctypes.byref(p), a, a, a, a, lsa.workspace_bytes(p, lsa.OP_ROUTE) - 1,
                            None) == 5
    assert L.lsa_sparse_attend(ctypes.byref(p), a, a, a, None, a, a, 1 << 40, None) == 1
    assert L.lsa_block_summarize(ctypes.byref(p), a, 0, a, None) == 2
    for code in range(7):
        assert L.lsa_status_str(code)


def test_workspace_sizes_are_plausible(lsa):
    p = good(lsa)
    pairs = 14 * 131072 * 16
    vt = 2 * 131072 * 64 * 2                      # V^T copy of both KV heads
    att = lsa.workspace_bytes(p, lsa.OP_ATTEND)
    # per routed pair of the layer: pair id and position; per pair of one
    # chunk (here the whole layer): the bf16 partial row and its log-mass
    want = pairs * (8 + 64 * 2 + 4) + vt
    assert want <= att < want + (1 << 20)
    # chunks of 4096 positions: the partial rows of one chunk only, and
    # buckets per (chunk, KV head, key block)
    chunked = lsa.workspace_bytes(good(lsa, chunk=4096), lsa.OP_ATTEND)
    want_c = pairs * 8 + 14 * 4096 * 16 * (64 * 2 + 4) + vt + 32 * 2 * 2048 * 16
    assert want_c <= chunked < want_c + (1 << 20)
    # past 32 GiB of partial rows the layer is chunked by itself
    big = good(lsa, batch=4, seq_len=1 << 20)
    assert lsa.workspace_bytes(big, lsa.OP_ATTEND) < 4 * 14 * (1 << 20) * 16 * 8 + (33 << 30)
    assert lsa.workspace_bytes(p, lsa.OP_SUMMARIZE) == 0
    img = lsa.params(4, 16, 16, 16384, 64, 16, 8, 0, 0)
    assert lsa.workspace_bytes(img, lsa.OP_ATTEND) == 0  # image mode reads V rows directly
    assert lsa.workspace_bytes(img, lsa.OP_ROUTE) >= 4 * 16 * 1024 * 64 * 4


def test_wide_top_k_is_accepted(lsa):
    """top_k 17..32 is part of the boundary: its pair ids take a stride of 32
    slots (so the attention workspace holds 32 partial rows per query row and
    the 32-bit pair-id limit binds at half the rows), and decode keeps 32-key
    chunk sets."""
    pairs = 14 * 131072
    vt = 2 * 131072 * 64 * 2
    for k in (17, 24, 32):
        p = good(lsa, top_k=k)
        att = lsa.workspace_bytes(p, lsa.OP_ATTEND)
        want = pairs * k * 8 + pairs * 32 * 64 * 2 + pairs * k * 4 + vt
        # plus the bucket tables: four words per (bucket chunk, KV head, key
        # block), up to 16 bucket chunks of 8192 positions at k = 32
        assert want <= att < want + (2 << 20)
        assert lsa.idx_shape(p) == (1, 14, 131072, k)
        assert lsa.workspace_bytes(p, lsa.OP_FORWARD) < lsa.SIZE_MAX
        d16 = lsa.workspace_bytes(good(lsa), lsa.OP_DECODE)
        assert lsa.workspace_bytes(p, lsa.OP_DECODE) > d16
    # B*Hq*N*2^ceil(log2 top_k) + 64 < 2^32: 128 x 14 x 131072 rows fit 16
    # slots each but not 32
    assert lsa.workspace_bytes(good(lsa, batch=128), lsa.OP_FORWARD) < lsa.SIZE_MAX
    big = good(lsa, batch=128, top_k=17)
    assert lsa.library().lsa_workspace_bytes(ctypes.byref(big), lsa.OP_FORWARD) == lsa.SIZE_MAX


def test_consensus_workspace_and_decode(lsa):
    """Consensus routing adds the group-summed queries (fp32, one row per KV
    group and position) to the routing workspace and is not offered by the
    decode call."""
    p, pc = good(lsa), good(lsa, consensus=1)
    extra = lsa.workspace_bytes(pc, lsa.OP_ROUTE) - lsa.workspace_bytes(p, lsa.OP_ROUTE)
    assert 2 * 131072 * 64 * 4 - 14 * 131072 * 4 <= extra <= 2 * 131072 * 64 * 4 + 4096
    assert lsa.workspace_bytes(pc, lsa.OP_ATTEND) == lsa.workspace_bytes(p, lsa.OP_ATTEND)
    assert lsa.library().lsa_workspace_bytes(ctypes.byref(pc), lsa.OP_DECODE) == lsa.SIZE_MAX
    assert lsa.idx_shape(pc) == (1, 2, 131072, 16)
    img = lsa.params(4, 16, 4, 16384, 64, 16, 8, 0, 0, consensus=1)
    assert lsa.idx_shape(img) == (4, 4, 1024, 8)
    a = ctypes.c_void_p(4096)
    assert lsa.library().lsa_decode(ctypes.byref(pc), 131072, a, a, a, a, a, None, a, 1 << 40,
                                    None) == 3


def test_cumulant_routing_checks(lsa):
    L = lsa.library()
    a = ctypes.c_void_p(4096)
    p = good(lsa, beta=0.125)
    assert L.lsa_route_topk(ctypes.byref(p), a, a, a, a, 1 << 40, None) == 3
    assert L.lsa_route_cumulant(ctypes.byref(p), None, a, a, None) == 1
    assert L.lsa_route_cumulant(ctypes.byref(p), a, ctypes.c_void_p(4100), a, None) == 4
    assert L.lsa_route_cumulant(ctypes.byref(good(lsa, beta=0.5, consensus=1)), a, a, a, None) == 3
    assert L.lsa_workspace_bytes(ctypes.byref(p), lsa.OP_DECODE) == lsa.SIZE_MAX


def test_tree_routing_workspace(lsa):
    """Two-level routing adds, per row, beam + 1 slots, pair ids, positions
    and 64-byte score rows to the routing workspace; decode refuses it."""
    p, pt = good(lsa), good(lsa, beam=8)
    rows = 14 * 131072
    extra = lsa.workspace_bytes(pt, lsa.OP_ROUTE)
    assert rows * 9 * (4 + 4 + 4 + 64) <= extra <= rows * 9 * (4 + 4 + 4 + 64) + (64 << 20)
    assert lsa.workspace_bytes(pt, lsa.OP_ATTEND) == lsa.workspace_bytes(p, lsa.OP_ATTEND)
    assert lsa.library().lsa_workspace_bytes(ctypes.byref(pt), lsa.OP_DECODE) == lsa.SIZE_MAX


def test_decode_argument_checks(lsa):
    """lsa_decode validates the step position against the cache and the
    cache geometry before anything is launched."""
    L = lsa.library()
    a = ctypes.c_void_p(4096)
    big = 1 << 40
    ok = good(lsa, seq_len=1000)                       # T = 1000 (need not be a block multiple)
    assert L.lsa_decode(ctypes.byref(good(lsa, seq_len=0)), 131072, a, a, a, a, a, None, a, big,
                        None) == 2                    # T < 1
    assert L.lsa_decode(ctypes.byref(good(lsa, seq_len=131136)), 131072, a, a, a, a, a, None, a,
                        big, None) == 2               # T > cache_len
    assert L.lsa_decode(ctypes.byref(ok), 131072 + 1, a, a, a, a, a, None, a, big, None) == 2
    assert L.lsa_decode(ctypes.byref(good(lsa, seq_len=1000, causal=0, window=0, block=16)),
                        131072, a, a, a, a, a, None, a, big, None) == 2
    assert L.lsa_decode(ctypes.byref(ok), 131072, None, a, a, a, a, None, a, big, None) == 1
    assert L.lsa_decode(ctypes.byref(ok), 131072, ctypes.c_void_p(4100), a, a, a, a, None, a, big,
                        None) == 4
    pc = good(lsa, seq_len=131072)
    need = L.lsa_workspace_bytes(ctypes.byref(pc), lsa.OP_DECODE)
    assert L.lsa_decode(ctypes.byref(ok), 131072, a, a, a, a, a, None, a, need - 1, None) == 5


def test_bench_refuses_more_than_one_gpu():
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr


def test_noalloc_decode_argument_checks(lsa):
    """lsa_decode_noalloc validates like lsa_decode and refuses, before
    anything runs, a geometry whose scratch exceeds the static array."""
    L = lsa.library()
    a = ctypes.c_void_p(256)
    ok = good(lsa, seq_len=4096)
    assert L.lsa_decode_noalloc(None, 4096, a, a, a, a, a, None, None) == 1
    assert L.lsa_decode_noalloc(ctypes.byref(ok), 4096, None, a, a, a, a, None, None) == 1
    assert L.lsa_decode_noalloc(ctypes.byref(ok), 4096, ctypes.c_void_p(264), a, a, a, a, None,
                                None) == 4
    assert L.lsa_decode_noalloc(ctypes.byref(ok), 2048, a, a, a, a, a, None, None) == 2  # T > cache
    big = lsa.params(1, 64, 8, 1 << 20, 64, 64, 16, 1 << 19, 1)   # a 512K-token window
    assert L.lsa_workspace_bytes(ctypes.byref(big), lsa.OP_DECODE) > lsa.STATIC_SCRATCH_BYTES
    assert L.lsa_decode_noalloc(ctypes.byref(big), 1 << 20, a, a, a, a, a, None, None) == 7
    assert L.lsa_status_str(7).decode().startswith("needs more scratch")


def test_image_tree_routing_workspace(lsa):
    """Image-mode two-level routing is accepted: its rows are query blocks,
    so its slot lists and pair tables scale with B * Hq * N / 16."""
    L = lsa.library()
    flat = lsa.params(4, 16, 16, 16384, 64, 16, 8, 0, 0)
    tree = lsa.params(4, 16, 16, 16384, 64, 16, 8, 0, 0, beam=8)
    wf = L.lsa_workspace_bytes(ctypes.byref(flat), lsa.OP_ROUTE)
    wt = L.lsa_workspace_bytes(ctypes.byref(tree), lsa.OP_ROUTE)
    assert wf != lsa.SIZE_MAX and wt != lsa.SIZE_MAX
    qblocks = 4 * 16 * 1024
    # slots, pair ids, positions (9 words each) and 9 score rows of 64 bytes per query block
    assert wt >= qblocks * 9 * (4 + 4 + 4 + 64)
    assert wt < qblocks * 9 * (4 + 4 + 4 + 64) + 3 * wf + (64 << 20)
