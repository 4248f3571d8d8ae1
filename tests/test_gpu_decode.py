"""Parity of the single-query decode path (lsa_decode, through the C ABI)
with the CPU oracle: the decode output for the query at position T-1 of a
cache holding T tokens must equal the oracle's forward row T-1 of the same
sequence (routing bit-exact on rows with a clear gap, valid on near ties;
outputs within the same tolerances as the prefill path).  The caches hold
the whole sequence, so these tests also check that nothing past T-1 is read.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from content_routed_block_amd.workloads import WORKLOADS, Workload, bf16_bits_to_f32, generate
from tests.parity import check_output, check_routing, causal_candidates, dev, params_of

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


def custom(B, Hq, Hkv, N, bs, k, W, dist="normal", seed=21, topics=16):
    return Workload(f"dec_b{B}_h{Hq}x{Hkv}_n{N}_bs{bs}_k{k}_w{W}_{dist}", B, Hq, Hkv, N, 64, bs, k,
                    W, 1, dist, topics=topics if dist == "topics" else 0, seed=seed)


CASES = [
    (WORKLOADS["tiny_causal_n1024"], [1, 64, 127, 128, 129, 640, 1023, 1024]),
    (custom(2, 4, 2, 2048, 64, 16, 128, dist="topics"), [1, 700, 1536, 2000, 2048]),
    (custom(1, 3, 1, 1536, 16, 8, 32), [17, 48, 511, 1536]),
    (custom(1, 2, 2, 4096, 32, 5, 64), [96, 2049, 4095]),
    (custom(1, 2, 1, 2048, 128, 3, 256), [300, 1280, 2048]),
    (custom(1, 4, 2, 40960, 16, 16, 128, dist="topics"), [16384, 40000, 40960]),
    (custom(1, 2, 1, 16 * 130, 16, 6, 48, seed=22), [1, 47, 49, 1000, 2080]),  # odd W / bs
    # top_k 17..32: 32-key chunk sets, one to four chunks per row
    (custom(2, 4, 2, 2048, 64, 32, 128, dist="topics", seed=24), [1, 700, 2047, 2048]),
    (custom(1, 2, 1, 40960, 16, 25, 128, seed=25), [5000, 40960]),
]


def run_decode(lsa, w, inp, T, kbar):
    """One decode step for position T-1 with the full sequence as the cache."""
    B, Hq, D = w.batch, w.q_heads, w.head_dim
    p = params_of(lsa, w, seq_len=T)
    q = dev(np.ascontiguousarray(inp.q[:, :, T - 1, :]))
    out, idx = lsa.decode(p, w.seq_len, q, dev(inp.k), dev(inp.v), kbar)
    torch.cuda.synchronize()
    return out.cpu().numpy().reshape(B * Hq, D), idx.cpu().numpy().reshape(B * Hq, w.top_k)


def check_steps(w, inp, kbar_o, Ts, out, idx):
    """out [R, D], idx [R, k] for rows (bh, T-1) over Ts (row order: T-major,
    then bh).  Routing parity by the gap rule, then the output against the
    oracle's attention over the GPU's own selection."""
    rows = np.array([bh * w.seq_len + T - 1 for T in Ts for bh in range(w.batch * w.q_heads)])
    io, gap = oracle.route_causal(inp.q, kbar_o, w.block, w.top_k, w.window, rows=rows,
                                  with_gap=True)
    scores = oracle.route_scores(kbar_o, rows, q=inp.q, block=w.block, window=w.window, causal=1)
    ncand = causal_candidates(rows % w.seq_len, w.block, w.window)
    bad, near, near_diff = check_routing(idx, io, gap, scores, ncand, w.top_k)
    assert bad == 0, bad
    ref = oracle.attend(inp.q, inp.k, inp.v, idx, w.block, w.top_k, w.window, 1, rows=rows)
    mx, _ = check_output(out, ref, np.full(rows.size, np.abs(bf16_bits_to_f32(inp.v)).max()))
    return near, near_diff, mx


@pytest.mark.parametrize("w,steps", CASES, ids=lambda x: x.name if hasattr(x, "name") else "")
def test_decode_matches_oracle(lsa, w, steps):
    say("decode", w.name, steps)
    inp = generate(w)
    kbar = lsa.block_summarize(params_of(lsa, w), dev(inp.k))   # block means of the whole cache
    kbar_o = oracle.block_means(inp.k, w.block)
    for T in steps:
        out, idx = run_decode(lsa, w, inp, T, kbar)
        near, near_diff, mx = check_steps(w, inp, kbar_o, [T], out, idx)
        say("  T", T, "near", near, "near-differing", near_diff, "max-abs", mx)


def test_decode_maintains_block_means(lsa):
    """A step at T = m*bs writes the mean of block m-1 into the cache (and
    reads only blocks that end before the window)."""
    w = custom(1, 2, 1, 1024, 64, 4, 128, seed=5)
    inp = generate(w)
    kbar_o = oracle.block_means(inp.k, w.block)               # [1, 1, 16, 64]
    kbar = torch.from_numpy(np.ascontiguousarray(kbar_o)).cuda()
    m = 9
    kbar[:, :, m - 1:, :] = 0.0                                # blocks >= m-1 not summarized yet
    T = m * w.block
    out, idx = run_decode(lsa, w, inp, T, kbar)
    got = kbar.cpu().numpy()
    assert np.array_equal(got[:, :, m - 1], kbar_o[:, :, m - 1])   # bit-exact mean
    assert np.all(got[:, :, m:] == 0.0)                          # later blocks untouched
    check_steps(w, inp, kbar_o, [T], out, idx)


def test_decode_consecutive_steps_match_prefill(lsa):
    """Consecutive steps that start from an empty block-mean cache and let
    each step summarize the block it completes reproduce the prefill rows."""
    w = custom(1, 4, 2, 768, 32, 6, 64, dist="topics", seed=9)
    inp = generate(w)
    kbar = torch.zeros((w.batch, w.kv_heads, w.seq_len // w.block, w.head_dim),
                       dtype=torch.float32, device="cuda")
    outs, idxs = [], []
    Ts = list(range(1, w.seq_len + 1))
    for T in Ts:
        out, idx = run_decode(lsa, w, inp, T, kbar)
        outs.append(out)
        idxs.append(idx)
    kbar_o = oracle.block_means(inp.k, w.block)
    assert np.array_equal(kbar.cpu().numpy(), kbar_o)
    near, near_diff, mx = check_steps(w, inp, kbar_o, Ts, np.concatenate(outs), np.concatenate(idxs))
    say("consecutive: near", near, "near-differing", near_diff, "max-abs", mx)


def test_decode_at_a_million_tokens(lsa):
    """The last position of the million-token workload: 16 chunk sets per
    row, the top-k merge over 256 keys and several attention splits."""
    w = WORKLOADS["qwen05b_n1m_needles"]
    inp = generate(w)
    kbar = lsa.block_summarize(params_of(lsa, w), dev(inp.k))
    T = w.seq_len
    out, idx = run_decode(lsa, w, inp, T, kbar)
    near, near_diff, mx = check_steps(w, inp, oracle.block_means(inp.k, w.block), [T], out, idx)
    say("  1M: near", near, "near-differing", near_diff, "max-abs", mx)


@pytest.mark.parametrize("bs,k,W", [(64, 16, 512), (16, 5, 48)])
def test_decode_equal_keys_take_the_lowest_blocks(lsa, bs, k, W):
    """Every key equal: every routing score ties, so every decode step must
    take the lowest min(k, E) blocks (the radix select over score-then-index
    keys has no capacity to overflow)."""
    w = custom(1, 2, 1, 8192, bs, k, W, seed=23)
    inp = generate(w)
    inp.k[:] = inp.k[:, :, :1, :]
    kbar = lsa.block_summarize(params_of(lsa, w), dev(inp.k))
    for T in (W + bs, 2 * W + 3, 4096, 8192):
        say("decode equal keys", w.name, T)
        _, idx = run_decode(lsa, w, inp, T, kbar)
        E = max(0, (T - 1) // bs - W // bs + 1)
        m = min(k, E)
        want = list(range(m)) + [-1] * (k - m)
        for r in range(idx.shape[0]):
            assert list(idx[r]) == want, (T, r, idx[r])
