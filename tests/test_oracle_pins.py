"""Pins of the CPU oracle against things other than itself: a hand-worked
example, closed forms, invariants, special cases that reduce to dense
attention (torch CPU SDPA in fp64), and an independent numpy brute force on
tiny inputs.  CPU only."""
import json
import math
import os

import numpy as np
import pytest
import torch

from content_routed_block_amd.workloads import (WORKLOADS, bf16_bits_to_f32, generate,
                                                to_bf16_bits)
from tests import brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand_bits(rng, shape, scale=1.0):
    return to_bf16_bits(scale * rng.standard_normal(shape).astype(np.float32))


def sdpa_f64(qb, kb, vb, causal, scale=None):
    """Dense attention, torch CPU, fp64.  q [B,Hq,N,D], k/v [B,Hkv,N,D] bits."""
    q = torch.from_numpy(brute.widen(qb))
    k = torch.from_numpy(brute.widen(kb))
    v = torch.from_numpy(brute.widen(vb))
    rep = q.shape[1] // k.shape[1]
    k = k.repeat_interleave(rep, dim=1)
    v = v.repeat_interleave(rep, dim=1)
    return torch.nn.functional.scaled_dot_product_attention(
        q, k, v, is_causal=bool(causal), scale=scale).numpy()


# ---------------------------------------------------------------- hand example
def test_hand_example(orc):
    g = json.load(open(os.path.join(GOLDEN, "hand_example.json")))
    bs, k, W = g["block"], g["top_k"], g["window"]
    K = to_bf16_bits(np.array(g["k"], np.float32))[None, None]
    V = to_bf16_bits(np.array(g["v"], np.float32))[None, None]
    Q = to_bf16_bits(np.array(g["q"], np.float32))[None, None]
    kbar = orc.block_means(K, bs)
    np.testing.assert_array_equal(kbar[0, 0], np.array(g["kbar"], np.float32))
    idx, gap = orc.route_causal(Q, kbar, bs, k, W, with_gap=True)
    scores = orc.route_scores(kbar, np.arange(8), q=Q, block=bs, window=W, causal=1)
    out = orc.attend(Q, K, V, idx.reshape(-1, k), bs, k, W, 1, scale=g["scale"])
    vv = np.array(g["v"], np.float64)
    for row in g["rows"]:
        t = row["t"]
        assert list(idx[0, 0, t]) == row["sel"], t
        exp_gap = math.inf if row["gap"] == "inf" else row["gap"]
        assert gap[0, 0, t] == exp_gap, t
        E = row["E"]
        np.testing.assert_array_equal(scores[t, :E], row["scores"])
        assert np.all(np.isneginf(scores[t, E:]))
        w = np.exp(np.array(row["dots"], np.float64) / math.sqrt(2.0))
        expect = (w[:, None] * vv[row["keys"]]).sum(0) / w.sum()
        np.testing.assert_allclose(out[0, 0, t], expect, rtol=1e-6, atol=1e-7)


# ---------------------------------------------------------------- block means
def test_means_constant_blocks(orc):
    rng = np.random.default_rng(0)
    bs, nb, D = 32, 6, 16
    consts = rand_bits(rng, (2, nb, D))
    x = np.repeat(consts[:, :, None, :], bs, axis=2).reshape(2, nb * bs, D)
    got = orc.block_means(x, bs)
    np.testing.assert_array_equal(got, bf16_bits_to_f32(consts))


def test_means_arithmetic_progression(orc):
    bs, D = 64, 8
    j = np.arange(bs, dtype=np.float32)[:, None]
    d = np.arange(D, dtype=np.float32)[None, :]
    x = to_bf16_bits((j + d) / 4.0)            # exact in bf16
    got = orc.block_means(x[None], bs)[0, 0]
    np.testing.assert_array_equal(got, (31.5 + np.arange(D)) / 4.0)


def test_means_permutation_invariant_and_local(orc):
    rng = np.random.default_rng(1)
    bs, nb, D = 64, 5, 64
    x = rand_bits(rng, (1, nb * bs, D))
    base = orc.block_means(x, bs)
    perm = np.concatenate([c * bs + rng.permutation(bs) for c in range(nb)])
    np.testing.assert_array_equal(orc.block_means(x[:, perm], bs), base)
    y = x.copy()
    y[0, 2 * bs + 7] = to_bf16_bits(bf16_bits_to_f32(y[0, 2 * bs + 7]) + 8.0)
    changed = orc.block_means(y, bs)
    for c in range(nb):
        if c != 2:
            np.testing.assert_array_equal(changed[0, c], base[0, c])
    np.testing.assert_allclose(
        changed[0, 2].astype(np.float64) - base[0, 2],
        (bf16_bits_to_f32(y[0, 2 * bs + 7]).astype(np.float64)
         - bf16_bits_to_f32(x[0, 2 * bs + 7])) / bs, atol=1e-6)


# ---------------------------------------------------------------- routing
def test_route_all_ties_pick_lowest_blocks(orc):
    bs, W, k, N, D = 16, 32, 3, 256, 8
    Q = to_bf16_bits(np.random.default_rng(2).standard_normal((1, 2, N, D)).astype(np.float32))
    K = to_bf16_bits(np.full((1, 1, N, D), 0.5, np.float32))
    kbar = orc.block_means(K, bs)
    idx, gap = orc.route_causal(Q, kbar, bs, k, W, with_gap=True)
    for t in range(N):
        E = max(0, t // bs - W // bs + 1)
        want = list(range(min(k, E))) + [-1] * (k - min(k, E))
        assert list(idx[0, 0, t]) == want and list(idx[0, 1, t]) == want
        assert gap[0, 0, t] == (0.0 if E > k else math.inf)


@pytest.mark.parametrize("sign", [1.0, -1.0])
def test_route_monotone_scores(orc, sign):
    bs, W, k, N, D = 16, 48, 4, 320, 8
    K = np.zeros((1, 1, N, D), np.float32)
    for c in range(N // bs):
        K[0, 0, c * bs:(c + 1) * bs, 0] = c + 1
    Q = np.zeros((1, 1, N, D), np.float32)
    Q[..., 0] = sign
    kb, qb = to_bf16_bits(K), to_bf16_bits(Q)
    idx = orc.route_causal(qb, orc.block_means(kb, bs), bs, k, W)
    for t in range(N):
        E = max(0, t // bs - W // bs + 1)
        n = min(k, E)
        want = list(range(E - n, E)) if sign > 0 else list(range(n))
        assert list(idx[0, 0, t]) == want + [-1] * (k - n), t


@pytest.mark.parametrize("bs,W,k,Hq,Hkv", [(16, 32, 3, 4, 2), (8, 8, 2, 2, 1), (32, 96, 1, 3, 3),
                                            (4, 8, 24, 2, 1)])
def test_route_matches_rank_brute_force(orc, bs, W, k, Hq, Hkv):
    rng = np.random.default_rng(bs * 100 + k)
    N, D = 256, 16
    Q = rand_bits(rng, (1, Hq, N, D))
    K = rand_bits(rng, (1, Hkv, N, D))
    kbar = orc.block_means(K, bs)
    kbar_np = brute.block_means(brute.widen(K), bs)
    np.testing.assert_array_equal(kbar, kbar_np)
    idx, gap = orc.route_causal(Q, kbar, bs, k, W, with_gap=True)
    qf = brute.widen(Q)
    rep = Hq // Hkv
    for h in range(Hq):
        for t in range(N):
            E = max(0, t // bs - W // bs + 1)
            s = [float(np.dot(qf[0, h, t], kbar_np[0, h // rep, c].astype(np.float64)))
                 for c in range(E)]
            keep = brute.rank_select(s, E, k)
            assert list(idx[0, h, t]) == keep + [-1] * (k - len(keep)), (h, t)
            if E > k:
                ss = sorted(s, reverse=True)
                assert gap[0, h, t] == pytest.approx(ss[k - 1] - ss[k], abs=1e-12)
            else:
                assert gap[0, h, t] == math.inf


def test_route_eligible_counts_tiny_config(orc):
    """With top-k >= number of blocks every eligible block is selected; the
    total candidate count of the tiny 1K config is 64 * (1 + ... + 14) per
    head, and no selected block reaches the window."""
    w = WORKLOADS["tiny_causal_n1024"]
    inp = generate(w)
    kbar = orc.block_means(inp.k, w.block)
    nb = w.seq_len // w.block
    idx = orc.route_causal(inp.q, kbar, w.block, nb, w.window)
    valid = idx >= 0
    assert valid.sum() == 2 * 64 * sum(range(15)) == 13440
    t = np.arange(w.seq_len)[None, None, :, None]
    assert np.all(np.where(valid, idx, -10**9) <= t // w.block - w.window // w.block)
    for tt in range(w.seq_len):
        E = max(0, tt // 64 - 1)
        assert list(idx[0, 0, tt, :E]) == list(range(E))


def test_route_invariant_under_signed_permutation(orc):
    """One common linear isometry of all queries and keys leaves the selected
    set unchanged (SSA page, 'Mathematical status').  A signed permutation of
    the coordinates is an isometry that is exact in bf16."""
    rng = np.random.default_rng(5)
    bs, W, k, N, D = 16, 32, 4, 512, 32
    Q = rand_bits(rng, (1, 2, N, D))
    K = rand_bits(rng, (1, 1, N, D))
    perm = rng.permutation(D)
    flip = np.where(rng.random(D) < 0.5, 0x8000, 0).astype(np.uint16)
    Q2 = Q[..., perm] ^ flip
    K2 = K[..., perm] ^ flip
    i1, g1 = orc.route_causal(Q, orc.block_means(K, bs), bs, k, W, with_gap=True)
    i2 = orc.route_causal(Q2, orc.block_means(K2, bs), bs, k, W)
    clear = g1 > 1e-9
    assert clear.mean() > 0.9
    np.testing.assert_array_equal(i1[clear], i2[clear])


def test_route_huge_needle_always_selected(orc):
    rng = np.random.default_rng(6)
    bs, W, k, N, D = 32, 64, 2, 1024, 64
    Q = rand_bits(rng, (1, 1, N, D))
    K = rand_bits(rng, (1, 1, N, D))
    rows = []
    for t, p in [(1000, 5), (700, 333), (500, 400)]:
        K[0, 0, p] = to_bf16_bits(1000.0 * bf16_bits_to_f32(Q[0, 0, t]))
        rows.append((t, p))
    idx = orc.route_causal(Q, orc.block_means(K, bs), bs, k, W)
    for t, p in rows:
        assert p // bs in idx[0, 0, t]


# ---------------------------------------------------------------- attention
def test_topk_covering_all_blocks_is_dense_causal(orc):
    rng = np.random.default_rng(7)
    bs, W, N, D = 16, 32, 256, 64
    Q, K, V = rand_bits(rng, (1, 4, N, D)), rand_bits(rng, (1, 2, N, D)), rand_bits(rng, (1, 2, N, D))
    out, sel = orc.forward(Q, K, V, bs, N // bs, W, 1)
    np.testing.assert_allclose(out, sdpa_f64(Q, K, V, True), atol=2e-7, rtol=1e-6)


def test_window_covering_sequence_is_dense_causal(orc):
    rng = np.random.default_rng(8)
    bs, k, N, D = 16, 2, 256, 32
    Q, K, V = rand_bits(rng, (2, 2, N, D)), rand_bits(rng, (2, 1, N, D)), rand_bits(rng, (2, 1, N, D))
    out, sel = orc.forward(Q, K, V, bs, k, N, 1)
    assert np.all(sel == -1)
    np.testing.assert_allclose(out, sdpa_f64(Q, K, V, True), atol=2e-7, rtol=1e-6)


def test_image_mode_full_topk_is_dense(orc):
    rng = np.random.default_rng(9)
    bs, N, D = 16, 256, 32
    Q, K, V = rand_bits(rng, (2, 2, N, D)), rand_bits(rng, (2, 2, N, D)), rand_bits(rng, (2, 2, N, D))
    out, sel = orc.forward(Q, K, V, bs, N // bs, 0, 0)
    np.testing.assert_allclose(out, sdpa_f64(Q, K, V, False), atol=2e-7, rtol=1e-6)


def test_zero_query_averages_exactly_the_selected_keys(orc):
    """q = 0 makes every logit 0, so the output is the plain mean of V over
    the attended set: routed blocks plus the window [bs*E, t]."""
    rng = np.random.default_rng(10)
    bs, W, k, N, D = 16, 48, 3, 384, 16
    Hq = 2
    Q = np.zeros((1, Hq, N, D), np.uint16)
    K, V = rand_bits(rng, (1, 1, N, D)), rand_bits(rng, (1, 1, N, D))
    nb = N // bs
    sel = np.full((Hq * N, k), -1, np.int32)
    for r in range(Hq * N):
        t = r % N
        E = max(0, t // bs - W // bs + 1)
        pick = np.sort(rng.choice(E, size=min(k, E), replace=False)) if E else []
        sel[r, :len(pick)] = pick
    out = orc.attend(Q, K, V, sel, bs, k, W, 1)
    vf = brute.widen(V)[0, 0]
    for r in range(Hq * N):
        t = r % N
        E = max(0, t // bs - W // bs + 1)
        keys = [j for c in sel[r] if c >= 0 for j in range(c * bs, c * bs + bs)]
        keys += list(range(E * bs, t + 1))
        np.testing.assert_allclose(out.reshape(-1, D)[r], vf[keys].mean(0), rtol=1e-6, atol=1e-7)
    assert nb > 0


def test_constant_values_give_that_constant(orc):
    rng = np.random.default_rng(11)
    bs, W, k, N, D = 16, 32, 2, 256, 8
    Q, K = rand_bits(rng, (1, 2, N, D)), rand_bits(rng, (1, 1, N, D))
    V = np.tile(to_bf16_bits(np.arange(D, dtype=np.float32) - 3.5), (1, 1, N, 1))
    out, _ = orc.forward(Q, K, V, bs, k, W, 1)
    np.testing.assert_allclose(out, np.broadcast_to(np.arange(D) - 3.5, out.shape), rtol=1e-6)


def test_gqa_head_reads_its_group(orc):
    rng = np.random.default_rng(12)
    bs, W, k, N, D = 16, 32, 3, 256, 16
    Q, K, V = rand_bits(rng, (1, 6, N, D)), rand_bits(rng, (1, 2, N, D)), rand_bits(rng, (1, 2, N, D))
    full, _ = orc.forward(Q, K, V, bs, k, W, 1)
    for h in range(6):
        g = h // 3
        one, _ = orc.forward(Q[:, h:h + 1], K[:, g:g + 1], V[:, g:g + 1], bs, k, W, 1)
        np.testing.assert_array_equal(one[0, 0], full[0, h])


def test_scale_acts_on_logits_only(orc):
    rng = np.random.default_rng(13)
    bs, W, k, N, D = 16, 32, 3, 256, 16
    Q, K, V = rand_bits(rng, (1, 1, N, D)), rand_bits(rng, (1, 1, N, D)), rand_bits(rng, (1, 1, N, D))
    Q2 = to_bf16_bits(2.0 * bf16_bits_to_f32(Q))
    a, sa = orc.forward(Q2, K, V, bs, k, W, 1, scale=0.125)
    b, sb = orc.forward(Q, K, V, bs, k, W, 1, scale=0.25)
    np.testing.assert_array_equal(sa, sb)
    np.testing.assert_allclose(a, b, rtol=1e-6, atol=1e-7)


@pytest.mark.parametrize("causal", [1, 0])
def test_end_to_end_matches_brute_force(orc, causal):
    rng = np.random.default_rng(14 + causal)
    bs, N, D = 16, 256, 16
    Hq, Hkv = 4, 2
    k, W = (3, 32) if causal else (4, 0)
    Q, K, V = rand_bits(rng, (1, Hq, N, D)), rand_bits(rng, (1, Hkv, N, D)), rand_bits(rng, (1, Hkv, N, D))
    out, _ = orc.forward(Q, K, V, bs, k, W, causal)
    want, _ = brute.forward(Q[0], K[0], V[0], bs, k, W, causal)
    np.testing.assert_allclose(out[0], want, rtol=1e-6, atol=2e-7)


def test_attend_rejects_invalid_selection(orc):
    rng = np.random.default_rng(15)
    bs, W, k, N, D = 16, 32, 2, 128, 8
    Q, K, V = rand_bits(rng, (1, 1, N, D)), rand_bits(rng, (1, 1, N, D)), rand_bits(rng, (1, 1, N, D))
    t = 100                                   # E = 100//16 - 2 + 1 = 5
    for bad in ([5, -1], [3, 3], [-1, 2], [4, 1], [-2, -1]):
        with pytest.raises(ValueError):
            orc.attend(Q, K, V, np.array([bad], np.int32), bs, k, W, 1, rows=[t])
    orc.attend(Q, K, V, np.array([[1, 4]], np.int32), bs, k, W, 1, rows=[t])


def test_sampled_rows_match_full_run(orc):
    rng = np.random.default_rng(16)
    bs, W, k, N, D = 16, 32, 3, 512, 32
    Q, K, V = rand_bits(rng, (2, 4, N, D)), rand_bits(rng, (2, 2, N, D)), rand_bits(rng, (2, 2, N, D))
    for causal, Wc in ((1, W), (0, 0)):
        full_o, full_s = orc.forward(Q, K, V, bs, k, Wc, causal)
        rows = rng.choice(2 * 4 * N, size=200, replace=False)
        o, s = orc.forward(Q, K, V, bs, k, Wc, causal, rows=rows)
        np.testing.assert_array_equal(o, full_o.reshape(-1, D)[rows])
        np.testing.assert_array_equal(s, full_s.reshape(-1, k)[rows])


# ---------------------------------------------------------------- consensus routing
# One route per KV group, scored by the sum of the group's query heads'
# routing scores (SSA page, "Complete 10M transformer result": a cross-head
# consensus route).

@pytest.mark.parametrize("bs,W,k,Hq,Hkv", [(16, 32, 3, 4, 2), (8, 16, 2, 3, 1), (32, 64, 1, 4, 1),
                                            (4, 8, 32, 3, 1)])
def test_consensus_matches_rank_brute_force(orc, bs, W, k, Hq, Hkv):
    rng = np.random.default_rng(bs * 10 + Hq)
    N, D = 256, 16
    Q = rand_bits(rng, (1, Hq, N, D))
    K = rand_bits(rng, (1, Hkv, N, D))
    kbar = orc.block_means(K, bs)
    kbar_np = brute.block_means(brute.widen(K), bs)
    idx, gap = orc.route_consensus(kbar, bs, k, q=Q, window=W, causal=1, with_gap=True)
    assert idx.shape == (1, Hkv, N, k)
    qf = brute.widen(Q)
    rep = Hq // Hkv
    for g in range(Hkv):
        for t in range(N):
            E = max(0, t // bs - W // bs + 1)
            s = [sum(float(np.dot(qf[0, h, t], kbar_np[0, g, c].astype(np.float64)))
                     for h in range(g * rep, (g + 1) * rep)) for c in range(E)]
            keep = brute.rank_select(s, E, k)
            assert list(idx[0, g, t]) == keep + [-1] * (k - len(keep)), (g, t)
            if E > k:
                ss = sorted(s, reverse=True)
                assert gap[0, g, t] == pytest.approx(ss[k - 1] - ss[k], abs=1e-12)
            else:
                assert gap[0, g, t] == math.inf


def test_consensus_image_matches_rank_brute_force(orc):
    rng = np.random.default_rng(31)
    bs, k, Hq, Hkv, N, D = 16, 3, 6, 2, 256, 16
    Q = rand_bits(rng, (1, Hq, N, D))
    K = rand_bits(rng, (1, Hkv, N, D))
    qbar = orc.block_means(Q, bs)
    kbar = orc.block_means(K, bs)
    idx = orc.route_consensus(kbar, bs, k, qbar=qbar, causal=0)
    nb, rep = N // bs, Hq // Hkv
    for g in range(Hkv):
        for i in range(nb):
            s = [sum(float(np.dot(qbar[0, h, i].astype(np.float64), kbar[0, g, c].astype(np.float64)))
                     for h in range(g * rep, (g + 1) * rep)) for c in range(nb)]
            assert list(idx[0, g, i]) == brute.rank_select(s, nb, k), (g, i)


def test_consensus_with_one_head_per_group_is_per_head_routing(orc):
    rng = np.random.default_rng(32)
    bs, W, k, N, D = 16, 32, 3, 512, 32
    Q, K = rand_bits(rng, (2, 3, N, D)), rand_bits(rng, (2, 3, N, D))
    kbar = orc.block_means(K, bs)
    np.testing.assert_array_equal(orc.route_consensus(kbar, bs, k, q=Q, window=W, causal=1),
                                  orc.route_causal(Q, kbar, bs, k, W))
    qbar = orc.block_means(Q, bs)
    np.testing.assert_array_equal(orc.route_consensus(kbar, bs, k, qbar=qbar, causal=0),
                                  orc.route_image(qbar, kbar, k))


def test_consensus_of_identical_heads_is_their_own_route(orc):
    """A group whose heads are copies of one query routes as that query does
    (the summed score is a positive multiple of it); groups are contiguous
    head ranges, so distinct queries per group keep distinct routes."""
    rng = np.random.default_rng(33)
    bs, W, k, N, D, rep = 16, 32, 4, 512, 32, 3
    base = rand_bits(rng, (1, 2, N, D))
    Q = np.repeat(base, rep, axis=1)                    # heads 0-2 = base 0, 3-5 = base 1
    K = rand_bits(rng, (1, 2, N, D))
    kbar = orc.block_means(K, bs)
    got = orc.route_consensus(kbar, bs, k, q=Q, window=W, causal=1)
    want = orc.route_causal(base, kbar, bs, k, W)       # one head per KV head
    np.testing.assert_array_equal(got, want)


def test_consensus_invariant_under_head_order_within_group(orc):
    rng = np.random.default_rng(34)
    bs, W, k, N, D = 16, 32, 3, 384, 16
    Q, K = rand_bits(rng, (1, 4, N, D)), rand_bits(rng, (1, 2, N, D))
    kbar = orc.block_means(K, bs)
    a = orc.route_consensus(kbar, bs, k, q=Q, window=W, causal=1)
    b = orc.route_consensus(kbar, bs, k, q=Q[:, [1, 0, 3, 2]], window=W, causal=1)
    np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("causal", [1, 0])
def test_consensus_end_to_end_matches_brute_force(orc, causal):
    rng = np.random.default_rng(35 + causal)
    bs, N, D = 16, 256, 16
    Hq, Hkv = 4, 2
    k, W = (3, 32) if causal else (4, 0)
    Q, K, V = rand_bits(rng, (1, Hq, N, D)), rand_bits(rng, (1, Hkv, N, D)), rand_bits(rng, (1, Hkv, N, D))
    out, sel = orc.forward_consensus(Q, K, V, bs, k, W, causal)
    want, mask = brute.forward(Q[0], K[0], V[0], bs, k, W, causal, consensus=True)
    np.testing.assert_allclose(out[0], want, rtol=1e-6, atol=2e-7)
    for g in range(Hkv):                                # the group shares one route
        for h in range(g * 2, g * 2 + 2):
            np.testing.assert_array_equal(sel[0, h], sel[0, g * 2])
            np.testing.assert_array_equal(mask[h], mask[g * 2])


# ---------------------------------------------------------------- second-cumulant score
# r_c(q) = <q, mu_c> + (beta/2) q^T Sigma_c q (SSA page, "Algorithm and
# complexity"), Sigma_c the bs-normalised covariance of the block's keys.

def test_cumulant_with_beta_zero_is_the_mean_score(orc):
    rng = np.random.default_rng(41)
    bs, W, k, N, D = 16, 32, 3, 512, 32
    Q, K = rand_bits(rng, (1, 4, N, D)), rand_bits(rng, (1, 2, N, D))
    kbar = orc.block_means(K, bs)
    a, ga = orc.route_cumulant(Q, K, kbar, bs, k, W, 0.0, with_gap=True)
    b, gb = orc.route_causal(Q, kbar, bs, k, W, with_gap=True)
    np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(ga, gb)


@pytest.mark.parametrize("bs,W,k,beta", [(16, 32, 3, 0.125), (8, 16, 2, 1.0), (32, 64, 4, -0.5),
                                         (8, 16, 20, 0.5)])
def test_cumulant_matches_score_variance_brute_force(orc, bs, W, k, beta):
    rng = np.random.default_rng(bs + k)
    N, D, Hq, Hkv = 256, 16, 4, 2
    Q = rand_bits(rng, (1, Hq, N, D))
    K = rand_bits(rng, (1, Hkv, N, D), scale=1.5)
    kbar = orc.block_means(K, bs)
    idx, gap, sc = orc.route_cumulant(Q, K, kbar, bs, k, W, beta, with_gap=True, with_scores=True)
    qf, kf = brute.widen(Q), brute.widen(K)
    rep, nb = Hq // Hkv, N // bs
    checked = 0
    for h in range(Hq):
        for t in range(N):
            E = max(0, t // bs - W // bs + 1)
            g = h // rep
            s = [brute.cumulant_score(qf[0, h, t], kf[0, g, c * bs:(c + 1) * bs], kbar[0, g, c], beta)
                 for c in range(E)]
            row = h * N + t
            np.testing.assert_allclose(sc[row, :E], s, rtol=1e-12, atol=1e-12)
            assert np.all(np.isneginf(sc[row, E:]))
            if E > k and gap[0, h, t] <= 1e-9:
                continue
            keep = brute.rank_select(s, E, k)
            assert list(idx[0, h, t]) == keep + [-1] * (k - len(keep)), (h, t)
            checked += 1
    assert checked > 0.9 * Hq * N


def test_cumulant_prefers_a_spread_block_with_lower_mean(orc):
    """Two candidate blocks along one direction u: block 0 has every key at
    mean score 1.0 and no spread; block 1 has mean score 0.75 with key scores
    +-1 around it (variance 1).  k = 1 picks block 1 exactly when
    0.75 + beta/2 > 1.0, i.e. beta > 0.5."""
    bs, D, W = 4, 2, 4
    N = 3 * bs                                  # query at t = 11: E = 2 candidates
    K = np.zeros((1, 1, N, D), np.float32)
    K[0, 0, 0:4, 0] = 1.0
    K[0, 0, 4:8, 0] = [1.75, -0.25, 1.75, -0.25]
    Q = np.zeros((1, 1, N, D), np.float32)
    Q[0, 0, :, 0] = 1.0
    Kb, Qb = to_bf16_bits(K), to_bf16_bits(Q)
    kbar = orc.block_means(Kb, bs)
    for beta, want in ((0.0, 0), (0.25, 0), (0.75, 1), (2.0, 1), (-1.0, 0)):
        idx, sc = orc.route_cumulant(Qb, Kb, kbar, bs, 1, W, beta, rows=[N - 1], with_scores=True)
        assert idx[0, 0] == want, (beta, idx)
        assert sc[0, 0] == pytest.approx(1.0)
        assert sc[0, 1] == pytest.approx(0.75 + beta / 2)


def test_cumulant_constant_blocks_reduce_to_the_mean_score(orc):
    rng = np.random.default_rng(42)
    bs, W, k, N, D = 16, 32, 3, 512, 16
    Q = rand_bits(rng, (1, 2, N, D))
    blocks = rng.standard_normal((1, 1, N // bs, D)).astype(np.float32)
    K = to_bf16_bits(np.repeat(blocks, bs, axis=2))   # every key of a block equal
    kbar = orc.block_means(K, bs)
    np.testing.assert_array_equal(orc.route_cumulant(Q, K, kbar, bs, k, W, 3.0),
                                  orc.route_causal(Q, kbar, bs, k, W))


# ---------------------------------------------------------------- two-level (tree) routing
# Nodes of 16 blocks summarised by the mean of their block means; the best
# `beam` complete candidate nodes are opened, plus the incomplete tail
# (SSA page, "Algorithm and complexity": hierarchical router, fanout 16).

def test_tree_with_wide_beam_is_flat_routing(orc):
    rng = np.random.default_rng(61)
    bs, W, k, N, D = 16, 32, 5, 4096, 16
    Q, K = rand_bits(rng, (1, 4, N, D)), rand_bits(rng, (1, 2, N, D))
    kbar = orc.block_means(K, bs)
    S_max = (N // bs) // 16
    np.testing.assert_array_equal(orc.route_tree(kbar, bs, k, S_max, q=Q, window=W),
                                  orc.route_causal(Q, kbar, bs, k, W))
    qbar = orc.block_means(Q, bs)
    np.testing.assert_array_equal(orc.route_tree(kbar, bs, k, S_max, qbar=qbar, causal=0),
                                  orc.route_image(qbar, kbar, k))


@pytest.mark.parametrize("bs,W,k,beam,F", [(8, 16, 4, 2, 16), (4, 8, 3, 1, 4), (8, 32, 6, 3, 8),
                                           (4, 8, 24, 2, 16)])
def test_tree_matches_rank_brute_force(orc, bs, W, k, beam, F):
    rng = np.random.default_rng(bs * 7 + beam)
    N, D, Hq, Hkv = 1024, 8, 2, 1
    Q, K = rand_bits(rng, (1, Hq, N, D)), rand_bits(rng, (1, Hkv, N, D))
    kbar = orc.block_means(K, bs)
    idx, det = orc.route_tree(kbar, bs, k, beam, q=Q, window=W, fanout=F, details=True)
    qf = brute.widen(Q)
    checked = 0
    for h in range(Hq):
        for t in range(0, N, 3):
            E = max(0, t // bs - W // bs + 1)
            row = h * N + t
            if min(det["gap1"][row], det["gap2"][row]) <= 1e-12:
                continue
            want = brute.tree_select(qf[0, h, t], kbar[0, 0], E, F, beam, k)
            assert list(idx[0, h, t]) == want + [-1] * (k - len(want)), (h, t)
            checked += 1
    assert checked > 0.9 * Hq * N / 3


def test_tree_misses_a_strong_block_in_a_weak_node(orc):
    """All blocks score 0 except: node 0 has every block at 1.0 (node mean
    1.0) and node 1 has one block at 8.0 and the rest at -1.0 (node mean
    1/16 * (8 - 15) < 1).  With beam 1 the tree opens node 0 only, so block
    16 (the 8.0) is not selected; with beam 2 it is; the flat selection
    always has it.  Tail blocks (past the last complete node) are always
    candidates."""
    bs, D, F = 1, 1, 16
    nb = 40                                  # nodes 0, 1; tail blocks 32..39
    vals = np.zeros(nb, np.float32)
    vals[0:16] = 1.0
    vals[16] = 8.0
    vals[17:32] = -1.0
    vals[35] = 4.0                           # a tail block
    kbar = vals.reshape(1, 1, nb, 1)
    qbar = np.ones((1, 1, nb, 1), np.float32)
    idx1 = orc.route_tree(kbar, bs, 2, 1, qbar=qbar, causal=0)[0, 0, 0]
    assert list(idx1) == [0, 35]             # node 0's first block (ties -> lowest) and the tail block
    idx2 = orc.route_tree(kbar, bs, 2, 2, qbar=qbar, causal=0)[0, 0, 0]
    assert list(idx2) == [16, 35]
    flat = orc.route_image(qbar, kbar, 2)[0, 0, 0]
    assert list(flat) == [16, 35]


def test_tree_node_scores_are_means_of_block_scores(orc):
    """<q, nu_s> equals the mean over the node of <q, mu_c> (linearity), up
    to the fp32 rounding of nu_s."""
    rng = np.random.default_rng(62)
    bs, W, k, N, D = 16, 32, 4, 8192, 32
    Q, K = rand_bits(rng, (1, 1, N, D)), rand_bits(rng, (1, 1, N, D))
    kbar = orc.block_means(K, bs)
    rows = np.array([N - 1, N // 2, 3000])
    _, det = orc.route_tree(kbar, bs, k, 4, q=Q, window=W, rows=rows, details=True)
    qf = brute.widen(Q)
    for i, t in enumerate(rows):
        S = max(0, t // bs - W // bs + 1) // 16
        bsc = kbar[0, 0].astype(np.float64) @ qf[0, 0, t]
        want = bsc[:S * 16].reshape(S, 16).mean(axis=1)
        np.testing.assert_allclose(det["node_scores"][i, :S], want, rtol=1e-6, atol=1e-6)
        assert np.all(np.isneginf(det["node_scores"][i, S:]))
