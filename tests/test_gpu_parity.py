"""Parity of the HIP path (through the C ABI) with the CPU oracle on seeded
inputs: block summaries, routing (bit-exact on rows with a clear gap, valid
on near ties), sparse attention fed the oracle's selection, the whole layer,
special cases that reduce to dense attention, determinism, and the
full-size workloads on sampled rows."""
import sys

import numpy as np
import pytest
import torch

import oracle
from content_routed_block_amd.workloads import WORKLOADS, Workload, bf16_bits_to_f32, generate, to_bf16_bits
from tests import brute
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


def custom(B, Hq, Hkv, N, bs, k, W, causal=1, dist="normal", seed=11, topics=16):
    return Workload(f"custom_b{B}_h{Hq}x{Hkv}_n{N}_bs{bs}_k{k}_w{W}_{dist}", B, Hq, Hkv, N, 64, bs, k,
                    W, causal, dist, topics=topics if dist == "topics" else 0, seed=seed)


CAUSAL_CASES = [
    WORKLOADS["tiny_causal_n1024"],
    custom(2, 4, 2, 2048 + 3 * 64, 64, 16, 128, dist="topics"),
    custom(1, 3, 1, 1536, 16, 8, 32),
    custom(1, 2, 2, 4096, 32, 5, 64),
    custom(1, 2, 1, 2048, 128, 3, 256),
    custom(1, 7, 1, 3072, 64, 16, 512, dist="topics", seed=5),
    custom(1, 1, 1, 64 * 40, 64, 1, 64),
    # N not a multiple of the 64-position attention tiles nor of the 128-row
    # routing tiles: partial last V^T tile, partial last query tile
    custom(1, 2, 1, 16 * 65, 16, 4, 32, seed=12),
    custom(3, 3, 3, 32 * 33, 32, 5, 64, dist="topics", seed=13),
    # an odd number of window blocks (W / bs = 3): odd eligible-block counts
    custom(1, 2, 1, 2048, 16, 6, 48, seed=17),
    custom(1, 2, 2, 32 * 40, 32, 3, 96, seed=18),
    # top_k 17..32 (every routing tile takes the exact pass; 32-entry lists
    # in the bucketing and the merge): a multiple of 4 and not, E(t) < k on
    # the first rows, GQA, B = 2, ragged N
    custom(2, 4, 2, 2048 + 3 * 64, 64, 24, 128, dist="topics", seed=31),
    custom(1, 3, 1, 16 * 130, 16, 32, 32, seed=32),
    custom(1, 2, 2, 32 * 70, 32, 19, 96, seed=33),
]
IMAGE_CASES = [
    custom(2, 4, 4, 1024, 16, 8, 0, causal=0),
    custom(1, 4, 2, 4096, 16, 16, 0, causal=0, seed=3),
    custom(1, 2, 2, 272, 16, 3, 0, causal=0, seed=4),
    custom(1, 2, 1, 1024, 16, 32, 0, causal=0, seed=34),
    custom(1, 4, 2, 4096, 16, 21, 0, causal=0, seed=35),
]


def run_route(lsa, w, inp):
    p = params_of(lsa, w)
    q, k = dev(inp.q), dev(inp.k)
    kbar = lsa.block_summarize(p, k)
    idx = lsa.route_topk(p, q, kbar)
    torch.cuda.synchronize()
    return kbar.cpu().numpy(), idx.cpu().numpy()


def oracle_route(w, inp, kbar_o):
    if w.causal:
        idx, gap = oracle.route_causal(inp.q, kbar_o, w.block, w.top_k, w.window, with_gap=True)
        R = w.batch * w.q_heads * w.seq_len
        rows = np.arange(R)
        scores = oracle.route_scores(kbar_o, rows, q=inp.q, block=w.block, window=w.window, causal=1)
        ncand = causal_candidates(rows % w.seq_len, w.block, w.window)
    else:
        qbar = oracle.block_means(inp.q, w.block)
        idx, gap = oracle.route_image(qbar, kbar_o, w.top_k, with_gap=True)
        nb = w.seq_len // w.block
        R = w.batch * w.q_heads * nb
        rows = np.arange(R)
        scores = oracle.route_scores(kbar_o, rows, qbar=qbar, block=w.block, causal=0)
        ncand = np.full(R, nb)
    return idx.reshape(R, -1), gap.reshape(R), scores, ncand


@pytest.mark.parametrize("w", CAUSAL_CASES + IMAGE_CASES, ids=lambda w: w.name)
def test_summary_matches_oracle(lsa, w):
    say("summary", w.name)
    inp = generate(w)
    kbar, _ = run_route(lsa, w, inp)
    np.testing.assert_array_equal(kbar, oracle.block_means(inp.k, w.block))


@pytest.mark.parametrize("w", CAUSAL_CASES + IMAGE_CASES, ids=lambda w: w.name)
def test_routing_matches_oracle(lsa, w):
    say("routing", w.name)
    inp = generate(w)
    kbar, idx = run_route(lsa, w, inp)
    io, gap, scores, ncand = oracle_route(w, inp, oracle.block_means(inp.k, w.block))
    bad, near, near_diff = check_routing(idx.reshape(io.shape), io, gap, scores, ncand, w.top_k)
    say("  near ties", near, "differing", near_diff)
    assert bad == 0


# Rows with 4096 or more candidate blocks take the router's lean second pass
# (hi-only scores, survivors rescored exactly) when the queries are bf16;
# the causal cases reach it at a modest size with 16-token blocks, the image
# case (pooled fp32 queries) checks that long fp32-query rows keep the full
# pass.
LONG_ROW_CASES = [
    custom(1, 2, 1, 81920, 16, 16, 128, dist="topics", seed=21),
    custom(1, 3, 1, 65536 + 16 * 300, 16, 7, 64, seed=22),
    custom(1, 2, 2, 65536, 16, 8, 0, causal=0, seed=23),
]


@pytest.mark.parametrize("w", LONG_ROW_CASES, ids=lambda w: w.name)
def test_routing_long_rows_sampled(lsa, w):
    """Routing parity on a sample of rows (plus the last routing tile of
    every head) for rows long enough for the lean second pass."""
    say("routing long rows", w.name)
    inp = generate(w)
    _, idx = run_route(lsa, w, inp)
    kbar_o = oracle.block_means(inp.k, w.block)
    rng = np.random.default_rng(5)
    P = w.seq_len if w.causal else w.seq_len // w.block
    R = w.batch * w.q_heads * P
    tail = np.concatenate([np.arange(h * P + P - 128, h * P + P)
                           for h in range(w.batch * w.q_heads)])
    rows = np.unique(np.concatenate([rng.choice(R, size=3000, replace=False), tail]))
    if w.causal:
        io, gap = oracle.route_causal(inp.q, kbar_o, w.block, w.top_k, w.window, rows=rows,
                                      with_gap=True)
        scores = oracle.route_scores(kbar_o, rows, q=inp.q, block=w.block, window=w.window,
                                     causal=1)
        ncand = causal_candidates(rows % w.seq_len, w.block, w.window)
    else:
        qbar = oracle.block_means(inp.q, w.block)
        io, gap = oracle.route_image(qbar, kbar_o, w.top_k, rows=rows, with_gap=True)
        scores = oracle.route_scores(kbar_o, rows, qbar=qbar, block=w.block, causal=0)
        ncand = np.full(rows.size, P)
    ig = idx.reshape(-1, w.top_k)[rows]
    bad, near, near_diff = check_routing(ig, io.reshape(rows.size, -1), gap.reshape(-1), scores,
                                         ncand, w.top_k)
    say("  rows", rows.size, "near ties", near, "differing", near_diff)
    assert bad == 0


def test_routing_all_ties_long_rows(lsa):
    """All scores equal on rows long enough for the lean second pass: every
    row overflows its survivor list, more rows than the per-row exact pass
    takes, so the queued tiles are redone whole."""
    w = custom(1, 1, 1, 81920, 16, 4, 64)
    inp = generate(w)
    inp.k[:] = to_bf16_bits(np.full(inp.k.shape, 0.25, np.float32))
    _, idx = run_route(lsa, w, inp)
    t = np.arange(w.seq_len)
    E = np.maximum(0, t // 16 - 4 + 1)
    want = np.where(np.arange(4)[None, :] < np.minimum(4, E)[:, None], np.arange(4)[None, :], -1)
    np.testing.assert_array_equal(idx.reshape(w.seq_len, 4), want)


def test_routing_all_ties_pick_lowest_blocks(lsa):
    """Constant keys make every routing score equal: every row must take the
    lowest eligible block ids (rows with more than 29 candidates overflow the
    fast path and run the exact fallback)."""
    w = custom(1, 2, 1, 4096, 64, 4, 128)
    inp = generate(w)
    inp.k[:] = to_bf16_bits(np.full(inp.k.shape, 0.25, np.float32))
    _, idx = run_route(lsa, w, inp)
    for t in range(w.seq_len):
        E = max(0, t // 64 - 1)
        m = min(4, E)
        want = list(range(m)) + [-1] * (4 - m)
        assert list(idx[0, 0, t]) == want and list(idx[0, 1, t]) == want, t


@pytest.mark.parametrize("sign", [1.0, -1.0])
def test_routing_monotone_scores(lsa, sign):
    w = custom(1, 1, 1, 4096, 64, 16, 192)
    inp = generate(w)
    K = np.zeros((1, 1, w.seq_len, 64), np.float32)
    for c in range(w.seq_len // 64):
        K[0, 0, c * 64:(c + 1) * 64, 0] = (c + 1) / 8.0
    Q = np.zeros_like(K)
    Q[..., 0] = sign
    inp.k[:] = to_bf16_bits(K)
    inp.q[:] = to_bf16_bits(Q)
    _, idx = run_route(lsa, w, inp)
    for t in range(w.seq_len):
        E = max(0, t // 64 - 3 + 1)
        n = min(16, E)
        want = list(range(E - n, E)) if sign > 0 else list(range(n))
        assert list(idx[0, 0, t]) == want + [-1] * (16 - n), t


def attend_gpu(lsa, w, inp, idx_np):
    p = params_of(lsa, w)
    idx = torch.from_numpy(np.ascontiguousarray(idx_np, dtype=np.int32)).cuda()
    out = lsa.sparse_attend(p, dev(inp.q), dev(inp.k), dev(inp.v), idx.reshape(lsa.idx_shape(p)))
    torch.cuda.synchronize()
    return out.cpu().numpy()


def per_row_selection(w, idx):
    """idx in the ABI layout -> selection per token row [B*Hq*N, k]."""
    if w.causal:
        return idx.reshape(-1, w.top_k)
    nbk = idx.reshape(w.batch * w.q_heads, w.seq_len // w.block, w.top_k)
    return np.repeat(nbk, w.block, axis=1).reshape(-1, w.top_k)


def vmax_rows(w, inp):
    v = np.abs(bf16_bits_to_f32(inp.v)).max(axis=(2, 3))            # [B, Hkv]
    rep = w.q_heads // w.kv_heads
    per_head = np.repeat(v, rep, axis=1)                              # [B, Hq]
    return np.repeat(per_head.reshape(-1), w.seq_len)


@pytest.mark.parametrize("w", CAUSAL_CASES + IMAGE_CASES, ids=lambda w: w.name)
def test_attend_with_oracle_selection(lsa, w):
    say("attend", w.name)
    inp = generate(w)
    kbar_o = oracle.block_means(inp.k, w.block)
    io, _, _, _ = oracle_route(w, inp, kbar_o)
    ref = oracle.attend(inp.q, inp.k, inp.v, per_row_selection(w, io), w.block, w.top_k, w.window,
                        w.causal)
    out = attend_gpu(lsa, w, inp, io)
    mx, mean = check_output(out.reshape(-1, 64), ref.reshape(-1, 64), vmax_rows(w, inp))
    say("  max-abs", mx, "mean-abs", mean)


def forward_gpu(lsa, w, inp):
    p = params_of(lsa, w)
    out, idx = lsa.forward(p, dev(inp.q), dev(inp.k), dev(inp.v))
    torch.cuda.synchronize()
    return out.cpu().numpy(), idx.cpu().numpy()


@pytest.mark.parametrize("w", CAUSAL_CASES + IMAGE_CASES, ids=lambda w: w.name)
def test_forward_matches_oracle(lsa, w):
    say("forward", w.name)
    inp = generate(w)
    out, idx = forward_gpu(lsa, w, inp)
    kbar_o = oracle.block_means(inp.k, w.block)
    io, gap, scores, ncand = oracle_route(w, inp, kbar_o)
    bad, _, _ = check_routing(idx.reshape(io.shape), io, gap, scores, ncand, w.top_k)
    assert bad == 0
    # the oracle attends over the GPU's own selection: on clear rows it is
    # identical to the oracle's, on near ties it was validated above
    ref = oracle.attend(inp.q, inp.k, inp.v, per_row_selection(w, idx), w.block, w.top_k, w.window,
                        w.causal)
    check_output(out.reshape(-1, 64), ref.reshape(-1, 64), vmax_rows(w, inp))


def sdpa_f64(inp, causal):
    q = torch.from_numpy(brute.widen(inp.q))
    k = torch.from_numpy(brute.widen(inp.k))
    v = torch.from_numpy(brute.widen(inp.v))
    rep = q.shape[1] // k.shape[1]
    k, v = k.repeat_interleave(rep, 1), v.repeat_interleave(rep, 1)
    return torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=causal).numpy()


@pytest.mark.parametrize("w,causal", [
    (custom(1, 4, 2, 1024, 64, 16, 128), True),     # top-k covers every eligible block
    (custom(2, 2, 1, 1024, 64, 4, 1024), True),     # window covers the sequence
    (custom(1, 2, 2, 256, 16, 16, 0, causal=0), False),  # image mode, top-k = all blocks
], ids=["topk_all", "window_ge_n", "image_all"])
def test_dense_special_cases(lsa, w, causal):
    say("dense", w.name)
    inp = generate(w)
    out, _ = forward_gpu(lsa, w, inp)
    ref = sdpa_f64(inp, causal)
    check_output(out.reshape(-1, 64), ref.reshape(-1, 64), vmax_rows(w, inp))


@pytest.mark.parametrize("over", [dict(chunk=64), dict(chunk=128), dict(chunk=512),
                                  dict(chunk=64, consensus=1), dict(chunk=256, consensus=1)],
                         ids=["c64", "c128", "c512", "c64-consensus", "c256-consensus"])
def test_forward_is_independent_of_the_attention_chunk(lsa, over):
    """Causal attention runs over chunks of query positions; forcing small
    chunks (many partial passes, ragged last chunk) changes nothing, bit for
    bit, and the result matches the oracle."""
    w = custom(2, 6, 2, 2048 + 3 * 64 + 32, 32, 8, 192, dist="topics", seed=21)
    say("chunked forward", w.name, over)
    inp = generate(w)
    q, k, v = dev(inp.q), dev(inp.k), dev(inp.v)
    base = {"consensus": over["consensus"]} if "consensus" in over else {}
    o0, i0 = lsa.forward(params_of(lsa, w, **base), q, k, v)
    o1, i1 = lsa.forward(params_of(lsa, w, **over), q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(i0, i1)
    assert torch.equal(o0.view(torch.int32), o1.view(torch.int32))
    if "consensus" in over:
        return
    out, idx = o1.cpu().numpy(), i1.cpu().numpy()
    io, gap, scores, ncand = oracle_route(w, inp, oracle.block_means(inp.k, w.block))
    bad, _, _ = check_routing(idx.reshape(io.shape), io, gap, scores, ncand, w.top_k)
    assert bad == 0
    ref = oracle.attend(inp.q, inp.k, inp.v, per_row_selection(w, idx), w.block, w.top_k,
                        w.window, w.causal)
    check_output(out.reshape(-1, 64), ref.reshape(-1, 64), vmax_rows(w, inp))


def test_forward_is_deterministic(lsa):
    w = WORKLOADS["qwen05b_n32k"].replace(seq_len=8192, name="det")
    inp = generate(w)
    o1, i1 = forward_gpu(lsa, w, inp)
    o2, i2 = forward_gpu(lsa, w, inp)
    np.testing.assert_array_equal(i1, i2)
    np.testing.assert_array_equal(o1.view(np.uint32), o2.view(np.uint32))


def test_invalid_selection_entries_are_skipped(lsa):
    w = custom(1, 2, 1, 1024, 64, 4, 128)
    inp = generate(w)
    rng = np.random.default_rng(0)
    R = w.q_heads * w.seq_len
    raw = rng.integers(-3, 20, size=(R, 4)).astype(np.int32)
    clean = np.full_like(raw, -1)
    for r in range(R):
        E = max(0, (r % w.seq_len) // 64 - 1)
        prev, used = -1, []
        for c in raw[r]:
            if prev < c < E:
                used.append(c)
                prev = c
        clean[r, :len(used)] = used
    ref = oracle.attend(inp.q, inp.k, inp.v, clean, 64, 4, 128, 1)
    out = attend_gpu(lsa, w, inp, raw)
    check_output(out.reshape(-1, 64), ref.reshape(-1, 64), vmax_rows(w, inp))


# ---------------------------------------------------------------- full size
FULL = ["qwen05b_n32k", "qwen05b_n128k_needles", "image_zorder_128x128", "qwen05b_n1m_needles"]


@pytest.mark.parametrize("name", FULL)
def test_full_size_sampled_rows(lsa, name):
    check_sampled_rows(lsa, WORKLOADS[name])


def check_sampled_rows(lsa, w, nrows=6000):
    """The whole layer on the GPU, then routing and output parity on a
    uniform sample of nrows rows (plus every needle row) against the oracle."""
    name = w.name
    say("full", name, "generating")
    inp = generate(w)
    say("full", name, "gpu forward")
    out, idx = forward_gpu(lsa, w, inp)
    kbar_o = oracle.block_means(inp.k, w.block)
    rng = np.random.default_rng(123)
    D = 64
    if w.causal:
        R = w.batch * w.q_heads * w.seq_len
        rows = np.sort(rng.choice(R, size=min(R, nrows), replace=False))
        if inp.needles:  # every needle query row is checked too
            extra = [(n.b * w.q_heads + n.h) * w.seq_len + n.t for n in inp.needles]
            rows = np.unique(np.concatenate([rows, np.array(extra)]))
        io, gap = oracle.route_causal(inp.q, kbar_o, w.block, w.top_k, w.window, rows=rows,
                                      with_gap=True)
        scores = oracle.route_scores(kbar_o, rows, q=inp.q, block=w.block, window=w.window, causal=1)
        ncand = causal_candidates(rows % w.seq_len, w.block, w.window)
        ig = idx.reshape(-1, w.top_k)[rows]
        bad, near, near_diff = check_routing(ig, io, gap, scores, ncand, w.top_k)
        say("  rows", rows.size, "near", near, "near-differing", near_diff, "clear mismatches", bad)
        assert bad == 0
        out_rows = rows
        sel = ig
        if inp.needles:
            j = np.searchsorted(rows, [(n.b * w.q_heads + n.h) * w.seq_len + n.t
                                       for n in inp.needles])
            hit_g, hit_o, ndiff = check_needles(ig[j], io[j], gap[j], scores[j], ncand[j],
                                                [n.p // w.block for n in inp.needles], w.top_k)
            say("  needle recall gpu", hit_g, "oracle", hit_o, "of", len(inp.needles),
                "differing (near ties)", ndiff)
    else:
        nb = w.seq_len // w.block
        qbar = oracle.block_means(inp.q, w.block)
        R = w.batch * w.q_heads * nb
        qrows = np.sort(rng.choice(R, size=min(R, 3000), replace=False))
        io, gap = oracle.route_image(qbar, kbar_o, w.top_k, rows=qrows, with_gap=True)
        scores = oracle.route_scores(kbar_o, qrows, qbar=qbar, block=w.block, causal=0)
        ig = idx.reshape(-1, w.top_k)[qrows]
        bad, near, near_diff = check_routing(ig, io, gap, scores, np.full(qrows.size, nb), w.top_k)
        say("  qblocks", qrows.size, "near", near, "near-differing", near_diff, "clear mismatches", bad)
        assert bad == 0
        # two token rows of every sampled query block
        bh, i = qrows // nb, qrows % nb
        out_rows = np.concatenate([bh * w.seq_len + i * w.block + rng.integers(0, w.block, qrows.size)
                                   for _ in range(2)])
        sel = np.concatenate([ig, ig])
    ref = oracle.attend(inp.q, inp.k, inp.v, sel, w.block, w.top_k, w.window, w.causal, rows=out_rows)
    got = out.reshape(-1, D)[out_rows]
    mx, mean = check_output(got, ref, vmax_rows(w, inp)[out_rows])
    say("  max-abs", mx, "mean-abs", mean)
