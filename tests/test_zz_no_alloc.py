"""lsa_decode_noalloc (the decode step whose scratch lives in the library's
static device array) against lsa_decode (the same step with a caller
workspace), through the C ABI: two calls in a row, the second on a smaller
geometry, so the second runs on what the first left in the shared array.
The two entry points launch the same kernels, so outputs, selections and
the block-mean cache update must agree bit for bit."""
import sys

import numpy as np
import pytest
import torch

from content_routed_block_amd.workloads import Workload, generate
from tests.parity import dev, params_of

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lsa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from content_routed_block_amd import lsa as m
    return m


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


# (workload of the cache, T: tokens filled); each call is smaller than the
# one before (the second takes 32-key chunk sets, top_k above 16), and the
# last is smaller in every dimension and ends mid-block
CASES = [
    (Workload("noalloc_big", 2, 8, 2, 16384, 64, 64, 16, 512, 1, "topics", topics=16, seed=81),
     16384),
    (Workload("noalloc_wide", 1, 8, 2, 8192, 64, 64, 32, 256, 1, "topics", topics=16, seed=83),
     8000),
    (Workload("noalloc_small", 1, 4, 1, 4096, 64, 32, 8, 256, 1, "normal", seed=82), 3001),
]


def step(lsa, w, inp, T, noalloc):
    p = params_of(lsa, w, seq_len=T)
    pc = params_of(lsa, w)
    k, v = dev(inp.k), dev(inp.v)
    kbar = lsa.block_summarize(pc, k)
    # the block that token T-1 completes is left stale, so the call must write it
    kbar[:, :, T // w.block - 1:, :] = -7.0
    q = dev(inp.q)[:, :, T - 1, :].contiguous()
    out = torch.full((w.batch, w.q_heads, 64), float("nan"), dtype=torch.float32, device="cuda")
    idx = torch.full((w.batch, w.q_heads, w.top_k), -5, dtype=torch.int32, device="cuda")
    if noalloc:
        lsa.decode_noalloc(p, w.seq_len, q, k, v, kbar, out, idx)
    else:
        lsa.decode(p, w.seq_len, q, k, v, kbar, out=out, idx=idx)
    torch.cuda.synchronize()
    return out.cpu(), idx.cpu(), kbar.cpu()


def test_noalloc_decode_equals_workspace_decode(lsa):
    for w, T in CASES:
        p = params_of(lsa, w)
        assert lsa.workspace_bytes(p, lsa.OP_DECODE) <= lsa.STATIC_SCRATCH_BYTES
    inputs = [generate(w) for w, _ in CASES]
    for (w, T), inp in zip(CASES, inputs):
        say("noalloc decode", w.name, "T", T)
        o_ref, i_ref, kb_ref = step(lsa, w, inp, T, noalloc=False)
        o, i, kb = step(lsa, w, inp, T, noalloc=True)
        assert torch.equal(i, i_ref)
        assert torch.equal(o.view(torch.int32), o_ref.view(torch.int32))
        assert torch.equal(kb.view(torch.int32), kb_ref.view(torch.int32))
        assert torch.isfinite(o).all()
        say("  ok: selections and outputs bit-identical")
