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
from tests.parity import (GAP, check_output, check_routing, check_tree_routing, causal_candidates,
                          dev, params_of)

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
    (custom(1, 4, 2, 16384, 16, 32, 64, dist="topics", seed=74), 4),   # top_k 17..32
    (custom(1, 2, 1, 8192, 32, 20, 64, seed=75), 1),   # fewer candidates than top_k in a row
]


def vmax_of(w, inp, rows):
    v = np.abs(bf16_bits_to_f32(inp.v)).max(axis=(2, 3))
    per_head = np.repeat(v, w.q_heads // w.kv_heads, axis=1).reshape(-1)
    return per_head[rows // w.seq_len]


def check_rows(w, inp, beam, gi, rows, oracle_out=None):
    kbar_o = oracle.block_means(inp.k, w.block)
    io, det = oracle.route_tree(kbar_o, w.block, w.top_k, beam, q=inp.q, window=w.window,
                                rows=rows, details=True)
    bsc = oracle.route_scores(kbar_o, rows, q=inp.q, block=w.block, window=w.window, causal=1)
    ncand = causal_candidates(rows % w.seq_len, w.block, w.window)
    if oracle_out is not None:
        oracle_out.update(idx=io, det=det)
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
    rows = np.random.default_rng(5).choice(R, 3000, False)
    needle_rows = np.array([(n.b * w.q_heads + n.h) * w.seq_len + n.t for n in inp.needles],
                           dtype=np.int64)
    rows = np.unique(np.concatenate([rows, needle_rows]))   # every needle row is checked too
    orc = {}
    bad, near, near_diff = check_rows(w, inp, beam, gi_all[rows], rows, orc)
    say("  rows", rows.size, "near", near, "near-differing", near_diff, "clear mismatches", bad)
    assert bad == 0
    if inp.needles:
        # the needle's block is selected on the GPU exactly when the oracle
        # selects it, unless the row is near a tie at some level (then
        # check_tree_routing above has shown the GPU's set to be valid)
        j = np.searchsorted(rows, needle_rows)
        hits_g = hits_o = ndiff = 0
        for jj, n in zip(j, inp.needles):
            hg = n.p // w.block in gi_all[rows[jj]]
            ho = n.p // w.block in orc["idx"][jj]
            hits_g, hits_o = hits_g + int(hg), hits_o + int(ho)
            if hg != ho:
                ndiff += 1
                assert orc["det"]["gap1"][jj] <= GAP or orc["det"]["gap2"][jj] <= GAP, (n, jj)
        say("  needle recall gpu", hits_g, "oracle", hits_o, "of", len(inp.needles),
            "differing (near ties)", ndiff)
    ref = oracle.attend(inp.q, inp.k, inp.v, gi_all[rows], w.block, w.top_k, w.window, 1, rows=rows)
    mx, mean = check_output(out.cpu().numpy().reshape(-1, 64)[rows], ref, vmax_of(w, inp, rows))
    say("  max-abs", mx, "mean-abs", mean)


# ---------------------------------------------------------------- image mode
# Two-level routing of pooled query blocks (LLSA page, "Minimum Usage": the
# two-level kernel for sequences of 16384 tokens and more, non-causal): every
# query block scores the nodes of 16 key blocks, opens its best `beam`, and
# takes its top-k among their blocks plus the blocks of the partial last node.
def image(B, Hq, Hkv, N, k, dist="normal", seed=91, side=0):
    return Workload(f"tree_img_b{B}_h{Hq}x{Hkv}_n{N}_k{k}_{dist}", B, Hq, Hkv, N, 64, 16, k, 0, 0,
                    dist, seed=seed, image_side=side)


IMAGE_CASES = [
    (image(2, 4, 4, 4096, 8), 4),                   # 16 nodes
    (image(1, 4, 2, 16 * (16 * 5 + 7), 6), 2),      # 5 nodes and a tail of 7 blocks, GQA
    (image(1, 2, 1, 16 * 12, 4), 3),                # no complete node: the tail only
    (image(1, 2, 2, 16 * 16 * 9, 16, seed=92), 15),  # beam covers every node
    (image(1, 4, 4, 16384, 8, "grf", seed=93, side=128), 8),  # one 128 x 128 image (Z-order)
    (image(1, 2, 1, 4096, 32, seed=95), 3),                    # top_k 17..32
]


def check_image_rows(w, inp, beam, gi, qrows, oracle_out=None):
    kbar_o = oracle.block_means(inp.k, w.block)
    qbar_o = oracle.block_means(inp.q, w.block)
    io, det = oracle.route_tree(kbar_o, w.block, w.top_k, beam, qbar=qbar_o, causal=0,
                                rows=qrows, details=True)
    bsc = oracle.route_scores(kbar_o, qrows, qbar=qbar_o, block=w.block, causal=0)
    ncand = np.full(qrows.size, w.seq_len // w.block)
    if oracle_out is not None:
        oracle_out.update(idx=io, det=det)
    return check_tree_routing(gi, io, det, bsc, ncand, w.top_k, beam)


@pytest.mark.parametrize("w,beam", IMAGE_CASES, ids=lambda x: x.name if hasattr(x, "name") else str(x))
def test_image_tree_routing_matches_oracle(lsa, w, beam):
    say("image tree routing", w.name, "beam", beam)
    inp = generate(w)
    p = params_of(lsa, w, beam=beam)
    kbar = lsa.block_summarize(p, dev(inp.k))
    idx = lsa.route_topk(p, dev(inp.q), kbar)
    torch.cuda.synchronize()
    assert tuple(idx.shape) == lsa.idx_shape(p)
    nq = w.batch * w.q_heads * (w.seq_len // w.block)
    qrows = np.arange(nq) if nq <= 20000 else np.sort(np.random.default_rng(6).choice(nq, 20000, False))
    gi = idx.cpu().numpy().reshape(-1, w.top_k)[qrows]
    bad, near, near_diff = check_image_rows(w, inp, beam, gi, qrows)
    say("  query blocks", qrows.size, "near", near, "differing", near_diff)
    assert bad == 0


@pytest.mark.parametrize("w,beam", IMAGE_CASES[:3] + IMAGE_CASES[4:],
                         ids=lambda x: x.name if hasattr(x, "name") else str(x))
def test_image_tree_forward_matches_oracle(lsa, w, beam):
    say("image tree forward", w.name, "beam", beam)
    inp = generate(w)
    p = params_of(lsa, w, beam=beam)
    out, idx = lsa.forward(p, dev(inp.q), dev(inp.k), dev(inp.v))
    torch.cuda.synchronize()
    nb = w.seq_len // w.block
    nq = w.batch * w.q_heads * nb
    qrows = np.arange(nq) if nq <= 8000 else np.sort(np.random.default_rng(7).choice(nq, 8000, False))
    gi = idx.cpu().numpy().reshape(-1, w.top_k)
    bad, _, _ = check_image_rows(w, inp, beam, gi[qrows], qrows)
    assert bad == 0
    # one token row of each checked query block attends to its block's route
    rng = np.random.default_rng(8)
    bh, i = qrows // nb, qrows % nb
    rows = bh * w.seq_len + i * w.block + rng.integers(0, w.block, qrows.size)
    ref = oracle.attend(inp.q, inp.k, inp.v, gi[qrows], w.block, w.top_k, 0, 0, rows=rows)
    mx, mean = check_output(out.cpu().numpy().reshape(-1, 64)[rows], ref, vmax_of(w, inp, rows))
    say("  max-abs", mx, "mean-abs", mean)


def test_image_tree_with_beam_covering_every_node_is_flat_routing(lsa):
    """nb = 144 blocks = 9 nodes: beam 15 opens every node, so the selection
    is flat image-mode routing (checked against the oracle's flat route)."""
    w = image(1, 2, 2, 16 * 144, 8, seed=94)
    inp = generate(w)
    p = params_of(lsa, w, beam=15)
    kbar = lsa.block_summarize(p, dev(inp.k))
    idx = lsa.route_topk(p, dev(inp.q), kbar)
    torch.cuda.synchronize()
    kbar_o = oracle.block_means(inp.k, w.block)
    qbar_o = oracle.block_means(inp.q, w.block)
    nq = w.q_heads * 144
    qrows = np.arange(nq)
    io, gap = oracle.route_image(qbar_o, kbar_o, w.top_k, with_gap=True)
    sc = oracle.route_scores(kbar_o, qrows, qbar=qbar_o, block=w.block, causal=0)
    bad, _, _ = check_routing(idx.cpu().numpy().reshape(-1, w.top_k), io.reshape(-1, w.top_k),
                              gap.reshape(-1), sc, np.full(nq, 144), w.top_k)
    assert bad == 0


@pytest.mark.parametrize("name,beam", [("image_zorder_128x128", 8), ("image_zorder_256x256", 8)])
def test_image_tree_full_size_sampled_rows(lsa, name, beam):
    """The image workload (4 images of 128 x 128 tokens) and one 256 x 256
    image (65536 tokens, 256 nodes per head), the sizes at which the LLSA
    page uses its two-level kernel."""
    w = WORKLOADS[name] if name in WORKLOADS else \
        WORKLOADS["image_zorder_128x128"].replace(name=name, batch=1, seq_len=65536, image_side=256,
                                                  seed=95)
    say("image tree full", w.name, "generating")
    inp = generate(w)
    say("image tree full", w.name, "gpu forward")
    p = params_of(lsa, w, beam=beam)
    out, idx = lsa.forward(p, dev(inp.q), dev(inp.k), dev(inp.v))
    torch.cuda.synchronize()
    nb = w.seq_len // w.block
    nq = w.batch * w.q_heads * nb
    qrows = np.sort(np.random.default_rng(9).choice(nq, 3000, False))
    gi = idx.cpu().numpy().reshape(-1, w.top_k)
    bad, near, near_diff = check_image_rows(w, inp, beam, gi[qrows], qrows)
    say("  query blocks", qrows.size, "near", near, "near-differing", near_diff, "clear mismatches", bad)
    assert bad == 0
    rng = np.random.default_rng(10)
    bh, i = qrows // nb, qrows % nb
    rows = bh * w.seq_len + i * w.block + rng.integers(0, w.block, qrows.size)
    ref = oracle.attend(inp.q, inp.k, inp.v, gi[qrows], w.block, w.top_k, 0, 0, rows=rows)
    mx, mean = check_output(out.cpu().numpy().reshape(-1, 64)[rows], ref, vmax_of(w, inp, rows))
    say("  max-abs", mx, "mean-abs", mean)
