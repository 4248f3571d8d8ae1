"""The C ABI's conventions on the GPU: lsa_forward without idx_out (the
routes then live in the workspace) equals the call that returns them, for
every routing variant; lsa_forward's routes equal lsa_route_topk's on the
same inputs; a call on a side stream equals one on the default
stream bit for bit; a workspace of exactly lsa_workspace_bytes works and,
when the routes must live in it, one byte less is refused before anything
runs."""
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


def causal_w(seed=61):
    return Workload("api_causal", 1, 4, 2, 2048 + 64, 64, 64, 8, 192, 1, "topics", topics=16,
                    seed=seed)


def image_w(seed=62):
    return Workload("api_image", 2, 2, 2, 1024, 64, 16, 6, 0, 0, "normal", seed=seed)


VARIANTS = [
    (causal_w, {}),
    (causal_w, {"consensus": 1}),
    (causal_w, {"beta": 0.25}),
    (causal_w, {"beam": 3}),
    (image_w, {}),
    (image_w, {"consensus": 1}),
]


@pytest.mark.parametrize("make,over", VARIANTS,
                         ids=["flat", "consensus", "cumulant", "tree", "image", "image-consensus"])
def test_forward_without_idx_out_equals_with(lsa, make, over):
    w = make()
    inp = generate(w)
    q, k, v = dev(inp.q), dev(inp.k), dev(inp.v)
    p = params_of(lsa, w, **over)
    o1, i1 = lsa.forward(p, q, k, v)
    o2, i2 = lsa.forward(p, q, k, v, want_idx=False)
    torch.cuda.synchronize()
    assert i2 is None
    assert torch.equal(o1, o2)


# lsa_forward writes the router's hi/lo split and chunk norm maxima from the
# key-summary kernel; lsa_route_topk, handed K-bar, prepares them separately.
# Both use the same arithmetic, so the routes must agree bit for bit:
# block sizes 16 to 128, block counts that leave a partial 32-block chunk,
# rows long enough for the lean second pass, and image mode.
PREP_CASES = [
    Workload("prep_bs16", 1, 3, 1, 16 * 150, 64, 16, 8, 64, 1, "topics", topics=8, seed=71),
    Workload("prep_bs32", 2, 2, 2, 32 * 77, 64, 32, 5, 96, 1, "normal", seed=72),
    Workload("prep_bs64", 1, 4, 2, 64 * 70, 64, 64, 16, 192, 1, "topics", topics=16, seed=73),
    Workload("prep_bs128", 1, 2, 1, 128 * 41, 64, 128, 4, 256, 1, "normal", seed=74),
    Workload("prep_long", 1, 2, 1, 16 * 4200, 64, 16, 16, 64, 1, "topics", topics=16, seed=75),
    Workload("prep_image", 2, 2, 2, 16 * 80, 64, 16, 6, 0, 0, "normal", seed=76),
]


@pytest.mark.parametrize("w", PREP_CASES, ids=lambda w: w.name)
def test_forward_routes_equal_route_topk_routes(lsa, w):
    inp = generate(w)
    q, k, v = dev(inp.q), dev(inp.k), dev(inp.v)
    p = params_of(lsa, w)
    _, i_fwd = lsa.forward(p, q, k, v)
    i_rt = lsa.route_topk(p, q, lsa.block_summarize(p, k))
    torch.cuda.synchronize()
    assert torch.equal(i_fwd, i_rt)


def test_forward_on_a_side_stream_equals_default_stream(lsa):
    w = causal_w()
    inp = generate(w)
    q, k, v = dev(inp.q), dev(inp.k), dev(inp.v)
    p = params_of(lsa, w)
    o1, i1 = lsa.forward(p, q, k, v)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        o2, i2 = lsa.forward(p, q, k, v, stream=side)
    side.synchronize()
    assert torch.equal(i1, i2) and torch.equal(o1, o2)


def test_side_stream_call_from_the_default_stream_keeps_its_buffers(lsa):
    """forward(stream=side) called while the default stream is current: the
    buffers the binding allocates for the call (workspace, out, idx) belong to
    the side stream, so allocations and writes on the default stream made
    before the side stream finishes cannot reuse them mid-flight."""
    w = causal_w(seed=67)
    inp = generate(w)
    q, k, v = dev(inp.q), dev(inp.k), dev(inp.v)
    p = params_of(lsa, w)
    ref_o, ref_i = lsa.forward(p, q, k, v)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    need = lsa.workspace_bytes(p, lsa.OP_FORWARD)
    results = []
    for _ in range(3):
        results.append(lsa.forward(p, q, k, v, stream=side))   # default stream stays current
        # the call's own workspace is freed on return; allocations of the same
        # size on the default stream, written at once, must not land on it
        junk = [torch.empty(need, dtype=torch.uint8, device="cuda") for _ in range(2)]
        for j in junk:
            j.fill_(0xA5)
        del junk
    side.synchronize()
    torch.cuda.synchronize()
    for o, i in results:
        assert torch.equal(o, ref_o) and torch.equal(i, ref_i)


def test_workspace_exact_size_and_one_byte_short(lsa):
    w = causal_w()
    inp = generate(w)
    q, k, v = dev(inp.q), dev(inp.k), dev(inp.v)
    p = params_of(lsa, w)
    need = lsa.workspace_bytes(p, lsa.OP_FORWARD)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    o1, _ = lsa.forward(p, q, k, v, workspace=ws)
    o0, _ = lsa.forward(p, q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(o0, o1)
    # without idx_out the routes live in the workspace, so all of it is needed
    o2, _ = lsa.forward(p, q, k, v, want_idx=False, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(o0, o2)
    short = torch.empty(need - 1, dtype=torch.uint8, device="cuda")
    with pytest.raises(Exception, match="LSA_ERR_WORKSPACE"):
        lsa.forward(p, q, k, v, want_idx=False, workspace=short)


def test_concurrent_calls_on_two_streams(lsa):
    """Two layers in flight at once on two streams, each with its own
    workspace and outputs, give what each gives alone."""
    wa, wb = causal_w(seed=63), causal_w(seed=64)
    ia, ib = generate(wa), generate(wb)
    qa, ka, va = dev(ia.q), dev(ia.k), dev(ia.v)
    qb, kb, vb = dev(ib.q), dev(ib.k), dev(ib.v)
    pa, pb = params_of(lsa, wa), params_of(lsa, wb)
    ref_a, ref_ia = lsa.forward(pa, qa, ka, va)
    ref_b, ref_ib = lsa.forward(pb, qb, kb, vb)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    outs = []
    for _ in range(3):
        with torch.cuda.stream(s1):
            oa, xa = lsa.forward(pa, qa, ka, va, stream=s1)
        with torch.cuda.stream(s2):
            ob, xb = lsa.forward(pb, qb, kb, vb, stream=s2)
        outs.append((oa, xa, ob, xb))
    s1.synchronize()
    s2.synchronize()
    for oa, xa, ob, xb in outs:
        assert torch.equal(oa, ref_a) and torch.equal(xa, ref_ia)
        assert torch.equal(ob, ref_b) and torch.equal(xb, ref_ib)


def test_forward_replays_from_a_graph(lsa):
    """lsa_forward captured in a HIP graph (preallocated outputs and
    workspace) replays to the eager result, also after the inputs change in
    place, with eager work and synchronisations between replays."""
    w = causal_w(seed=65)
    i1, i2 = generate(w), generate(causal_w(seed=66))
    q, k, v = dev(i1.q), dev(i1.k), dev(i1.v)
    p = params_of(lsa, w)
    out = torch.empty((w.batch, w.q_heads, w.seq_len, 64), dtype=torch.float32, device="cuda")
    idx = torch.empty(lsa.idx_shape(p), dtype=torch.int32, device="cuda")
    ws = torch.empty(lsa.workspace_bytes(p, lsa.OP_FORWARD), dtype=torch.uint8, device="cuda")
    ref1, rid1 = lsa.forward(p, q, k, v)
    ref2, rid2 = lsa.forward(p, dev(i2.q), dev(i2.k), dev(i2.v))
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up outside the capture
        lsa.forward(p, q, k, v, out=out, idx=idx, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        lsa.forward(p, q, k, v, out=out, idx=idx, workspace=ws)
    torch.cuda.synchronize()
    for rep in range(4):
        src = i1 if rep % 2 == 0 else i2
        q.copy_(dev(src.q))
        k.copy_(dev(src.k))
        v.copy_(dev(src.v))
        lsa.forward(p, dev(i2.q), dev(i2.k), dev(i2.v))   # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        want_o, want_i = (ref1, rid1) if rep % 2 == 0 else (ref2, rid2)
        assert torch.equal(out, want_o), rep
        assert torch.equal(idx, want_i), rep
