"""Parity of two-level routing (beam > 0) through the C ABI with the CPU
oracle: selections bit-exact where both the node-level and the block-level
gaps are clear, valid outcomes elsewhere; the layer's output within the
prefill tolerances; a beam that covers every node reproduces flat routing."""
import sys

import numpy as np
import pytest
import torch

import oracle
from content_routed_block_amd.workloads import WORKLOADS, Workload, bf16_bits_to_f32, generate
from tests.parity import (check_output, check_routing, check_tree_routing, causal_candidates, dev,
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


def custom(B, Hq, Hkv, N, bs, k, W, dist="normal", seed=71, topics=16):
    return Workload(f"tree_b{B}_h{Hq}x{Hkv}_n{N}_bs{bs}_k{k}_w{W}_{dist}", B, Hq, Hkv, N, 64, bs, k,
                    W, 1, dist, topics=topics if dist == "topics" else 0, seed=seed)


CASES = [
    (WORKLOADS["tiny_causal_n1024"], 2),                          # no complete node: all tail
    (custom(1, 2, 1, 16384, 16, 8, 64), 4),
    (custom(2, 4, 2, 8192 + 5 * 64, 32, 16, 128, dist="topics"), 8),
    (custom(1, 7, 1, 32768, 64, 16, 512, dist="topics", seed=5), 8),
    (custom(1, 2, 2, 32768, 128, 3, 256), 2),
    (custom(1, 3, 1, 8192, 16, 5, 32), 1),
    (custom(1, 2, 1, 16 * 1001, 16, 6, 48, seed=73), 3),   # odd W / bs, N not a multiple of 64
]


def vmax_of(w, inp, rows):
    v = np.abs(bf16_bits_to_f32(inp.v)).max(axis=(2, 3))
    per_head = np.repeat(v, w.q_heads // w.kv_heads, axis=1).reshape(-1)
    return per_head[rows // w.seq_len]


def check_rows(w, inp, beam, gi, rows):
    kbar_o = oracle.block_means(inp.k, w.block)
    io, det = oracle.route_tree(kbar_o, w.block, w.top_k, beam, q=inp.q, window=w.window,
                                rows=rows, details=True)
    bsc = oracle.route_scores(kbar_o, rows, q=inp.q, block=w.block, window=w.window, causal=1)
    ncand = causal_candidates(rows % w.seq_len, w.block, w.window)
    return check_tree_routing(gi, io, det, bsc, ncand, w.top_k, beam)


@pytest.mark.parametrize("w,beam", CASES, ids=lambda x: x.name if hasattr(x, "name") else str(x))
def test_tree_routing_matches_oracle(lsa, w, beam):
    say("tree routing", w.name, "beam", beam)
    inp = generate(w)
    p = params_of(lsa, w, beam=beam)
    kbar = lsa.block_summarize(p, dev(inp.k))
    idx = lsa.route_topk(p, dev(inp.q), kbar)
    torch.cuda.synchronize()
    R = w.batch * w.q_heads * w.seq_len
    rows = np.arange(R) if R <= 70000 else np.sort(np.random.default_rng(3).choice(R, 70000, False))
    gi = idx.cpu().numpy().reshape(-1, w.top_k)[rows]
    bad, near, near_diff = check_rows(w, inp, beam, gi, rows)
    say("  rows", rows.size, "near", near, "differing", near_diff)
    assert bad == 0


@pytest.mark.parametrize("w,beam", CASES[:4], ids=lambda x: x.name if hasattr(x, "name") else str(x))
def test_tree_forward_matches_oracle(lsa, w, beam):
    say("tree forward", w.name, "beam", beam)
    inp = generate(w)
    p = params_of(lsa, w, beam=beam)
    out, idx = lsa.forward(p, dev(inp.q), dev(inp.k), dev(inp.v))
    torch.cuda.synchronize()
    R = w.batch * w.q_heads * w.seq_len
    rows = np.sort(np.random.default_rng(4).choice(R, min(R, 20000), False))
    gi = idx.cpu().numpy().reshape(-1, w.top_k)[rows]
    bad, _, _ = check_rows(w, inp, beam, gi, rows)
    assert bad == 0
    ref = oracle.attend(inp.q, inp.k, inp.v, gi, w.block, w.top_k, w.window, 1, rows=rows)
    mx, mean = check_output(out.cpu().numpy().reshape(-1, 64)[rows], ref, vmax_of(w, inp, rows))
    say("  max-abs", mx, "mean-abs", mean)


def test_tree_with_beam_covering_every_node_is_flat_routing(lsa):
    """N = 4096, bs = 16, W = 64: at most 15 complete candidate nodes, so
    beam 15 scores every candidate and must agree with flat routing."""
    w = custom(1, 4, 2, 4096, 16, 8, 64, dist="topics", seed=72)
    inp = generate(w)
    p = params_of(lsa, w, beam=15)
    kbar = lsa.block_summarize(p, dev(inp.k))
    idx = lsa.route_topk(p, dev(inp.q), kbar)
    torch.cuda.synchronize()
    kbar_o = oracle.block_means(inp.k, w.block)
    rows = np.arange(w.q_heads * w.seq_len)
    io, gap = oracle.route_causal(inp.q, kbar_o, w.block, w.top_k, w.window, with_gap=True)
    sc = oracle.route_scores(kbar_o, rows, q=inp.q, block=w.block, window=w.window, causal=1)
    bad, _, _ = check_routing(idx.cpu().numpy().reshape(-1, w.top_k), io.reshape(-1, w.top_k),
                              gap.reshape(-1), sc, causal_candidates(rows % w.seq_len, w.block,
                                                                     w.window), w.top_k)
    assert bad == 0


@pytest.mark.parametrize("name", ["qwen05b_n128k_needles", "qwen05b_n1m_needles"])
def test_tree_full_size_sampled_rows(lsa, name):
    check_tree_sampled_rows(lsa, WORKLOADS[name], 8)


def check_tree_sampled_rows(lsa, w, beam):
    name = w.name
    say("tree full", name, "generating")
    inp = generate(w)
    say("tree full", name, "gpu forward")
    p = params_of(lsa, w, beam=beam)
    out, idx = lsa.forward(p, dev(inp.q), dev(inp.k), dev(inp.v))
    torch.cuda.synchronize()
    gi_all = idx.cpu().numpy().reshape(-1, w.top_k)
    R = w.batch * w.q_heads * w.seq_len
    rows = np.sort(np.random.default_rng(5).choice(R, 3000, False))
    bad, near, near_diff = check_rows(w, inp, beam, gi_all[rows], rows)
    say("  rows", rows.size, "near", near, "near-differing", near_diff, "clear mismatches", bad)
    assert bad == 0
    if inp.needles:
        hits = sum(int(n.p // w.block in gi_all[(n.b * w.q_heads + n.h) * w.seq_len + n.t])
                   for n in inp.needles)
        say("  needle blocks selected", hits, "of", len(inp.needles))
    ref = oracle.attend(inp.q, inp.k, inp.v, gi_all[rows], w.block, w.top_k, w.window, 1, rows=rows)
    mx, mean = check_output(out.cpu().numpy().reshape(-1, 64)[rows], ref, vmax_of(w, inp, rows))
    say("  max-abs", mx, "mean-abs", mean)
