"""Parity of consensus routing (one route per KV group, scored by the sum of
the group's query heads' routing scores) through the C ABI with the CPU
oracle: routing bit-exact on rows with a clear gap and valid on near ties,
outputs of every query head through its group's route within the prefill
tolerances, and the reduction to per-head routing when each group has one
head."""
import sys

import numpy as np
import pytest
import torch

import oracle
from content_routed_block_amd.workloads import WORKLOADS, Workload, bf16_bits_to_f32, generate
from tests.parity import (check_needles, check_output, check_routing, causal_candidates, dev,
                          params_of)

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


def custom(B, Hq, Hkv, N, bs, k, W, causal=1, dist="normal", seed=41, topics=16):
    return Workload(f"cons_b{B}_h{Hq}x{Hkv}_n{N}_bs{bs}_k{k}_w{W}_{dist}", B, Hq, Hkv, N, 64, bs, k,
                    W, causal, dist, topics=topics if dist == "topics" else 0, seed=seed)


CASES = [
    WORKLOADS["tiny_causal_n1024"],
    custom(2, 4, 2, 2048 + 3 * 64, 64, 16, 128, dist="topics"),
    custom(1, 7, 1, 3072, 64, 16, 512, dist="topics", seed=5),
    custom(1, 3, 1, 1536, 16, 8, 32),
    custom(1, 6, 2, 2048, 128, 3, 256),
    custom(1, 4, 2, 4096, 16, 16, 0, causal=0, seed=3),
    custom(2, 6, 2, 1024, 16, 8, 0, causal=0, seed=6),
    custom(1, 4, 2, 16 * 65, 16, 4, 32, seed=14),   # N not a multiple of 64
    custom(1, 4, 2, 2048, 16, 6, 48, seed=19),      # odd W / bs
    custom(2, 4, 2, 2048 + 3 * 64, 64, 32, 128, dist="topics", seed=42),  # top_k 17..32
    custom(1, 6, 2, 16 * 130, 16, 22, 32, seed=43),
    custom(1, 4, 2, 2048, 16, 28, 0, causal=0, seed=44),
]


def group_rows_of(w):
    per = w.seq_len if w.causal else w.seq_len // w.block
    return w.batch * w.kv_heads * per, per


def oracle_consensus(w, inp, kbar_o, rows=None):
    """Oracle group routes, gaps, scores and candidate counts for group rows."""
    if rows is None:
        rows = np.arange(group_rows_of(w)[0])
    if w.causal:
        io, gap, sc = oracle.route_consensus(kbar_o, w.block, w.top_k, q=inp.q, window=w.window,
                                             causal=1, rows=rows, with_gap=True, with_scores=True)
        ncand = causal_candidates(rows % w.seq_len, w.block, w.window)
    else:
        qbar = oracle.block_means(inp.q, w.block)
        io, gap, sc = oracle.route_consensus(kbar_o, w.block, w.top_k, qbar=qbar, causal=0,
                                             rows=rows, with_gap=True, with_scores=True)
        ncand = np.full(rows.size, w.seq_len // w.block)
    return io, gap, sc, ncand


def per_query_selection(w, gidx, qrows):
    """The group route that serves each query token row."""
    g = gidx.reshape(-1, w.top_k)
    if w.causal:
        return g[oracle.consensus_rows(qrows, w.q_heads, w.kv_heads, w.seq_len)]
    nb = w.seq_len // w.block
    qb = (qrows // w.seq_len) * nb + (qrows % w.seq_len) // w.block
    return g[oracle.consensus_rows(qb, w.q_heads, w.kv_heads, nb)]


def vmax_of(w, inp, qrows):
    v = np.abs(bf16_bits_to_f32(inp.v)).max(axis=(2, 3))            # [B, Hkv]
    per_head = np.repeat(v, w.q_heads // w.kv_heads, axis=1).reshape(-1)
    return per_head[qrows // w.seq_len]


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_consensus_routing_matches_oracle(lsa, w):
    say("consensus routing", w.name)
    inp = generate(w)
    p = params_of(lsa, w, consensus=1)
    kbar = lsa.block_summarize(p, dev(inp.k))
    idx = lsa.route_topk(p, dev(inp.q), kbar)
    torch.cuda.synchronize()
    assert tuple(idx.shape) == lsa.idx_shape(p)
    io, gap, sc, ncand = oracle_consensus(w, inp, oracle.block_means(inp.k, w.block))
    bad, near, near_diff = check_routing(idx.cpu().numpy().reshape(io.shape), io, gap, sc, ncand,
                                         w.top_k)
    say("  near ties", near, "differing", near_diff)
    assert bad == 0


# rows with 4096 or more candidate blocks (fp32 group queries keep the router's
# full second pass at any length)
@pytest.mark.parametrize("w", [custom(1, 4, 2, 81920, 16, 16, 128, dist="topics", seed=24),
                               custom(1, 4, 2, 65536, 16, 8, 0, causal=0, seed=25)],
                         ids=lambda w: w.name)
def test_consensus_routing_long_rows_sampled(lsa, w):
    say("consensus routing long rows", w.name)
    inp = generate(w)
    p = params_of(lsa, w, consensus=1)
    kbar = lsa.block_summarize(p, dev(inp.k))
    idx = lsa.route_topk(p, dev(inp.q), kbar)
    torch.cuda.synchronize()
    R, per = group_rows_of(w)
    rng = np.random.default_rng(6)
    tail = np.concatenate([np.arange(g * per + per - 128, g * per + per)
                           for g in range(w.batch * w.kv_heads)])
    rows = np.unique(np.concatenate([rng.choice(R, size=2000, replace=False), tail]))
    io, gap, sc, ncand = oracle_consensus(w, inp, oracle.block_means(inp.k, w.block), rows=rows)
    ig = idx.cpu().numpy().reshape(-1, w.top_k)[rows]
    bad, near, near_diff = check_routing(ig, io.reshape(rows.size, -1), gap.reshape(-1), sc,
                                         ncand, w.top_k)
    say("  rows", rows.size, "near ties", near, "differing", near_diff)
    assert bad == 0


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_consensus_forward_matches_oracle(lsa, w):
    say("consensus forward", w.name)
    inp = generate(w)
    p = params_of(lsa, w, consensus=1)
    out, idx = lsa.forward(p, dev(inp.q), dev(inp.k), dev(inp.v))
    torch.cuda.synchronize()
    gidx = idx.cpu().numpy()
    io, gap, sc, ncand = oracle_consensus(w, inp, oracle.block_means(inp.k, w.block))
    bad, _, _ = check_routing(gidx.reshape(io.shape), io, gap, sc, ncand, w.top_k)
    assert bad == 0
    qrows = np.arange(w.batch * w.q_heads * w.seq_len)
    sel = per_query_selection(w, gidx, qrows)
    ref = oracle.attend(inp.q, inp.k, inp.v, sel, w.block, w.top_k, w.window, w.causal)
    mx, mean = check_output(out.cpu().numpy().reshape(-1, 64), ref.reshape(-1, 64),
                            vmax_of(w, inp, qrows))
    say("  max-abs", mx, "mean-abs", mean)


@pytest.mark.parametrize("w", [custom(1, 3, 3, 2048, 64, 8, 128, dist="topics"),
                               custom(1, 2, 2, 1024, 16, 4, 0, causal=0)],
                         ids=lambda w: w.name)
def test_consensus_with_one_head_per_group_is_per_head_routing(lsa, w):
    """With Hq = Hkv the consensus of a group is its only head: the layer's
    selection and output equal the per-head path's bit for bit."""
    inp = generate(w)
    q, k, v = dev(inp.q), dev(inp.k), dev(inp.v)
    o1, i1 = lsa.forward(params_of(lsa, w), q, k, v)
    o2, i2 = lsa.forward(params_of(lsa, w, consensus=1), q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(i1, i2)
    assert torch.equal(o1, o2)


@pytest.mark.parametrize("name", ["qwen05b_n128k_needles", "qwen05b_n1m_needles",
                                  "image_zorder_128x128"])
def test_consensus_full_size_sampled_rows(lsa, name):
    check_consensus_sampled_rows(lsa, WORKLOADS[name])


def check_consensus_sampled_rows(lsa, w):
    name = w.name
    say("consensus full", name, "generating")
    inp = generate(w)
    say("consensus full", name, "gpu forward")
    p = params_of(lsa, w, consensus=1)
    out, idx = lsa.forward(p, dev(inp.q), dev(inp.k), dev(inp.v))
    torch.cuda.synchronize()
    gidx = idx.cpu().numpy().reshape(-1, w.top_k)
    out = out.cpu().numpy().reshape(-1, 64)
    kbar_o = oracle.block_means(inp.k, w.block)
    rng = np.random.default_rng(321)
    R, per = group_rows_of(w)
    grows = rng.choice(R, size=min(R, 3000), replace=False)
    needle_rows = np.array([(n.b * w.kv_heads + n.h // (w.q_heads // w.kv_heads)) * w.seq_len + n.t
                            for n in inp.needles], dtype=np.int64)
    grows = np.unique(np.concatenate([grows, needle_rows]))   # every needle's group row too
    io, gap, sc, ncand = oracle_consensus(w, inp, kbar_o, grows)
    bad, near, near_diff = check_routing(gidx[grows], io, gap, sc, ncand, w.top_k)
    say("  group rows", grows.size, "near", near, "near-differing", near_diff, "clear mismatches", bad)
    assert bad == 0
    if inp.needles:
        j = np.searchsorted(grows, needle_rows)
        hits_g, hits_o, ndiff = check_needles(gidx[grows][j], io[j], gap[j], sc[j], ncand[j],
                                              [n.p // w.block for n in inp.needles], w.top_k)
        say("  needle blocks in the group route: gpu", hits_g, "oracle", hits_o, "of",
            len(inp.needles), "differing (near ties)", ndiff)
    # query rows: every head of a sample of group rows
    rep = w.q_heads // w.kv_heads
    bg, pos = grows // per, grows % per
    b, g = bg // w.kv_heads, bg % w.kv_heads
    hh = rng.integers(0, rep, grows.size)
    if w.causal:
        qrows = (b * w.q_heads + g * rep + hh) * w.seq_len + pos
    else:
        qrows = (b * w.q_heads + g * rep + hh) * w.seq_len + pos * w.block + \
            rng.integers(0, w.block, grows.size)
    sel = per_query_selection(w, gidx, qrows)
    ref = oracle.attend(inp.q, inp.k, inp.v, sel, w.block, w.top_k, w.window, w.causal, rows=qrows)
    mx, mean = check_output(out[qrows], ref, vmax_of(w, inp, qrows))
    say("  max-abs", mx, "mean-abs", mean)
