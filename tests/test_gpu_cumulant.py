"""Parity of routing by the second-cumulant score (lsa_route_cumulant, and
lsa_forward with beta != 0) through the C ABI with the CPU oracle: routing
bit-exact on rows with a clear gap and valid on near ties, the layer's
output within the prefill tolerances, and the beta = 0 and constant-block
reductions to the block-mean score."""
import sys

import numpy as np
import pytest
import torch

import oracle
from content_routed_block_amd.workloads import WORKLOADS, Workload, bf16_bits_to_f32, generate, to_bf16_bits
from tests.parity import check_output, check_routing, causal_candidates, dev, params_of

pytestmark = pytest.mark.gpu

BETA = 0.125   # 1/sqrt(D): the softmax scale, the weight of the cumulant expansion of log-mean-exp


@pytest.fixture(scope="module")
def lsa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from content_routed_block_amd import lsa as m
    return m


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def custom(B, Hq, Hkv, N, bs, k, W, dist="normal", seed=51, topics=16):
    return Workload(f"cum_b{B}_h{Hq}x{Hkv}_n{N}_bs{bs}_k{k}_w{W}_{dist}", B, Hq, Hkv, N, 64, bs, k,
                    W, 1, dist, topics=topics if dist == "topics" else 0, seed=seed)


CASES = [
    (WORKLOADS["tiny_causal_n1024"], BETA),
    (custom(2, 4, 2, 2048 + 3 * 64, 64, 16, 128, dist="topics"), BETA),
    (custom(1, 3, 1, 1536, 16, 8, 32), 1.0),
    (custom(1, 2, 2, 4096, 32, 5, 64), -0.5),
    (custom(1, 2, 1, 2048, 128, 3, 256), BETA),
    (custom(1, 7, 1, 3072, 64, 16, 512, dist="topics", seed=5), 0.5),
    (custom(1, 2, 1, 16 * 65, 16, 4, 32, seed=15), BETA),   # N not a multiple of 64
    (custom(1, 2, 1, 2048, 16, 6, 48, seed=16), BETA),      # odd W / bs: odd block counts
    (custom(2, 4, 2, 2048 + 3 * 64, 64, 32, 128, dist="topics", seed=53), BETA),  # top_k 17..32
    (custom(1, 3, 1, 16 * 130, 16, 23, 32, seed=54), -0.5),
]


def oracle_rows(w, inp, beta, rows):
    kbar_o = oracle.block_means(inp.k, w.block)
    io, gap, sc = oracle.route_cumulant(inp.q, inp.k, kbar_o, w.block, w.top_k, w.window, beta,
                                        rows=rows, with_gap=True, with_scores=True)
    return io, gap, sc, causal_candidates(rows % w.seq_len, w.block, w.window)


def vmax_of(w, inp, rows):
    v = np.abs(bf16_bits_to_f32(inp.v)).max(axis=(2, 3))
    per_head = np.repeat(v, w.q_heads // w.kv_heads, axis=1).reshape(-1)
    return per_head[rows // w.seq_len]


@pytest.mark.parametrize("w,beta", CASES, ids=lambda x: x.name if hasattr(x, "name") else str(x))
def test_cumulant_routing_matches_oracle(lsa, w, beta):
    say("cumulant routing", w.name, "beta", beta)
    inp = generate(w)
    p = params_of(lsa, w, beta=beta)
    idx = lsa.route_cumulant(p, dev(inp.q), dev(inp.k))
    torch.cuda.synchronize()
    rows = np.arange(w.batch * w.q_heads * w.seq_len)
    io, gap, sc, ncand = oracle_rows(w, inp, beta, rows)
    bad, near, near_diff = check_routing(idx.cpu().numpy().reshape(io.shape), io, gap, sc, ncand,
                                         w.top_k)
    say("  near ties", near, "differing", near_diff)
    assert bad == 0


@pytest.mark.parametrize("w,beta", CASES, ids=lambda x: x.name if hasattr(x, "name") else str(x))
def test_cumulant_forward_matches_oracle(lsa, w, beta):
    say("cumulant forward", w.name, "beta", beta)
    inp = generate(w)
    p = params_of(lsa, w, beta=beta)
    out, idx = lsa.forward(p, dev(inp.q), dev(inp.k), dev(inp.v))
    torch.cuda.synchronize()
    rows = np.arange(w.batch * w.q_heads * w.seq_len)
    gi = idx.cpu().numpy().reshape(-1, w.top_k)
    io, gap, sc, ncand = oracle_rows(w, inp, beta, rows)
    bad, _, _ = check_routing(gi, io, gap, sc, ncand, w.top_k)
    assert bad == 0
    ref = oracle.attend(inp.q, inp.k, inp.v, gi, w.block, w.top_k, w.window, 1)
    mx, mean = check_output(out.cpu().numpy().reshape(-1, 64), ref.reshape(-1, 64),
                            vmax_of(w, inp, rows))
    say("  max-abs", mx, "mean-abs", mean)


@pytest.mark.parametrize("beta", [0.0, 2.0])
def test_cumulant_reduces_to_block_mean_score(lsa, beta):
    """beta = 0, or keys constant within each block (no spread): the
    selection is that of the block-mean score (oracle step 2-3)."""
    w = custom(1, 4, 2, 2048, 64, 8, 128, dist="topics", seed=52)
    inp = generate(w)
    if beta != 0.0:
        kb = bf16_bits_to_f32(inp.k).reshape(1, 2, 32, 64, 64)
        inp.k[:] = to_bf16_bits(np.repeat(kb[:, :, :, :1, :], 64, axis=3).reshape(inp.k.shape))
    idx = lsa.route_cumulant(params_of(lsa, w, beta=beta), dev(inp.q), dev(inp.k))
    torch.cuda.synchronize()
    kbar_o = oracle.block_means(inp.k, w.block)
    rows = np.arange(w.q_heads * w.seq_len)
    io, gap = oracle.route_causal(inp.q, kbar_o, w.block, w.top_k, w.window, rows=rows,
                                  with_gap=True)
    sc = oracle.route_scores(kbar_o, rows, q=inp.q, block=w.block, window=w.window, causal=1)
    bad, _, _ = check_routing(idx.cpu().numpy().reshape(-1, w.top_k), io, gap, sc,
                              causal_candidates(rows % w.seq_len, w.block, w.window), w.top_k)
    assert bad == 0


@pytest.mark.parametrize("name", ["qwen05b_n32k", "qwen05b_n128k_needles"])
def test_cumulant_full_size_sampled_rows(lsa, name):
    check_cumulant_sampled_rows(lsa, WORKLOADS[name])


def check_cumulant_sampled_rows(lsa, w):
    name = w.name
    say("cumulant full", name, "generating")
    inp = generate(w)
    say("cumulant full", name, "gpu forward")
    p = params_of(lsa, w, beta=BETA)
    out, idx = lsa.forward(p, dev(inp.q), dev(inp.k), dev(inp.v))
    torch.cuda.synchronize()
    gi = idx.cpu().numpy().reshape(-1, w.top_k)
    out = out.cpu().numpy().reshape(-1, 64)
    rng = np.random.default_rng(77)
    R = w.batch * w.q_heads * w.seq_len
    rows = np.sort(rng.choice(R, size=min(R, 2000), replace=False))
    io, gap, sc, ncand = oracle_rows(w, inp, BETA, rows)
    bad, near, near_diff = check_routing(gi[rows], io, gap, sc, ncand, w.top_k)
    say("  rows", rows.size, "near", near, "near-differing", near_diff, "clear mismatches", bad)
    assert bad == 0
    ref = oracle.attend(inp.q, inp.k, inp.v, gi[rows], w.block, w.top_k, w.window, 1, rows=rows)
    mx, mean = check_output(out[rows], ref, vmax_of(w, inp, rows))
    say("  max-abs", mx, "mean-abs", mean)


@pytest.mark.parametrize("N,bs,W,k", [(4096, 64, 512, 16), (4096, 32, 64, 16), (2048, 16, 32, 8)])
def test_cumulant_tied_block_patterns(lsa, N, bs, W, k):
    """Blocks repeating two multi-token key patterns: equal blocks have equal
    means and variances, so scores tie in groups and the lower block must win
    every tie.  Compared exactly with the oracle on rows whose distinct
    scores are more than 1e-3 apart."""
    w = Workload(f"cum_ties_n{N}_bs{bs}", 1, 2, 1, N, 64, bs, k, W, 1, "normal", seed=5)
    say("cumulant tied patterns", w.name)
    inp = generate(w)
    P = np.random.default_rng(9).standard_normal((2, bs, 64)).astype(np.float32)
    K = np.concatenate([P[c % 2] for c in range(N // bs)], axis=0)
    inp.k[:] = to_bf16_bits(np.broadcast_to(K, inp.k.shape))
    beta = 0.125
    p = params_of(lsa, w, beta=beta)
    idx = lsa.route_cumulant(p, dev(inp.q), dev(inp.k)).cpu().numpy().reshape(-1, k)
    rows = np.arange(idx.shape[0])
    io, _, sc = oracle.route_cumulant(inp.q, inp.k, oracle.block_means(inp.k, bs), bs, k, W, beta,
                                      rows=rows, with_gap=True, with_scores=True)
    sc = np.asarray(sc)
    clear = np.ones(rows.size, bool)
    for r in rows:
        u = np.unique(sc[r][np.isfinite(sc[r])])
        clear[r] = u.size < 2 or np.diff(u).min() > 1e-3
    assert clear.mean() > 0.9
    bad = np.nonzero(clear & np.any(idx != np.asarray(io).reshape(-1, k), axis=1))[0]
    assert bad.size == 0, (bad[:5], idx[bad[:1]])
