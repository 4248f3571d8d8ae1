"""Parity over a seeded sweep of random valid shapes, for every routing
variant (per-head, consensus, second-cumulant, two-level) and for decode,
plus causal shapes long enough for the router's lean second pass.

The fixed cases in the other GPU suites pick shapes by hand; this sweep draws
them: block size, window width in blocks (odd counts included), top-k, GQA
ratio, batch, sequence length down to a single block, and the value
distribution.  Each case runs the same checks as the fixed cases (routing
bit-exact on rows with a clear gap and valid on near ties, outputs within the
prefill tolerances, block means bit-exact), through the same helpers.
"""
import numpy as np
import pytest

import tests.test_gpu_consensus as C
import tests.test_gpu_cumulant as U
import tests.test_gpu_decode as D
import tests.test_gpu_parity as P
import tests.test_gpu_tree as T
from content_routed_block_amd.workloads import Workload

pytestmark = pytest.mark.gpu

lsa = P.lsa  # the module fixture: skips without a GPU
MAX_ROWS = 120_000  # B * Hq * N per case, so the oracle finishes in about a second


def draw(n, seed, causal=True, tag="sw", kmin=1, kmax=16):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        bs = int(rng.choice([16, 32, 64, 128])) if causal else 16
        m = int(rng.integers(1, 4096 // bs + 1))            # blocks in the sequence
        N = bs * m
        W = bs * int(rng.integers(1, 9)) if causal else 0   # 1 to 8 window blocks
        k = int(rng.integers(kmin, kmax + 1))
        Hkv = int(rng.integers(1, 4))
        rep = int(rng.choice([1, 2, 3, 7]))
        B = int(rng.integers(1, 3))
        if B * Hkv * rep * N > MAX_ROWS:
            continue
        dist = "topics" if rng.random() < 0.5 else "normal"
        i = len(out)
        out.append(Workload(f"{tag}{i}_b{B}_h{Hkv * rep}x{Hkv}_n{N}_bs{bs}_k{k}_w{W}_{dist}",
                            B, Hkv * rep, Hkv, N, 64, bs, k, W, int(causal), dist,
                            topics=16 if dist == "topics" else 0, seed=seed * 100 + i))
    return out


def draw_long(n, seed, tag="long"):
    """Causal shapes whose longest rows have 4096 or more candidate blocks
    (the router's lean second pass), checked on sampled rows."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        bs = int(rng.choice([16, 32]))
        wb = int(rng.integers(1, 9))
        m = 4096 + wb - 1 + int(rng.integers(0, 1200))       # blocks: E(N-1) >= 4096
        k = int(rng.integers(1, 17))
        Hkv = int(rng.integers(1, 3))
        rep = int(rng.choice([1, 2, 3, 7]))
        dist = "topics" if rng.random() < 0.5 else "normal"
        out.append(Workload(f"{tag}{i}_h{Hkv * rep}x{Hkv}_n{bs * m}_bs{bs}_k{k}_w{bs * wb}_{dist}",
                            1, Hkv * rep, Hkv, bs * m, 64, bs, k, bs * wb, 1, dist,
                            topics=16 if dist == "topics" else 0, seed=seed * 100 + i))
    return out


FLAT = draw(64, 31) + draw(16, 32, causal=False, tag="img")
LONG = draw_long(12, 41)
CONSENSUS = draw(20, 33, tag="cons") + draw(8, 34, causal=False, tag="consimg")
CUMULANT = [(w, float(b)) for w, b in zip(draw(20, 35, tag="cum"),
                                          np.random.default_rng(40).choice([0.125, 1.0, -0.5, 2.0], 20))]
TREE = [(w, int(b)) for w, b in zip(draw(20, 36, tag="tree"),
                                    np.random.default_rng(37).integers(1, 16, 20))]
DECODE = [(w, sorted({1, w.seq_len, *np.random.default_rng(39 + i).integers(1, w.seq_len + 1, 3)
                      .tolist()}))
          for i, w in enumerate(draw(16, 38, tag="dec"))]
# top_k 17..32 through every variant
WIDE = draw(24, 42, tag="wide", kmin=17, kmax=32) + draw(8, 43, causal=False, tag="wideimg",
                                                         kmin=17, kmax=32)
WIDE_CONSENSUS = draw(6, 44, tag="widecons", kmin=17, kmax=32) + draw(
    2, 45, causal=False, tag="wideconsimg", kmin=17, kmax=32)
WIDE_CUMULANT = [(w, float(b)) for w, b in zip(draw(6, 46, tag="widecum", kmin=17, kmax=32),
                                               np.random.default_rng(47).choice([0.125, -0.5, 2.0], 6))]
WIDE_TREE = [(w, int(b)) for w, b in zip(draw(6, 48, tag="widetree", kmin=17, kmax=32),
                                         np.random.default_rng(49).integers(1, 16, 6))]
WIDE_DECODE = [(w, sorted({1, w.seq_len, *np.random.default_rng(50 + i).integers(1, w.seq_len + 1, 3)
                           .tolist()}))
               for i, w in enumerate(draw(6, 51, tag="widedec", kmin=17, kmax=32))]


def name(x):
    return x.name if hasattr(x, "name") else str(x)


@pytest.mark.parametrize("w", FLAT, ids=name)
def test_sweep_summary(lsa, w):
    P.test_summary_matches_oracle(lsa, w)


@pytest.mark.parametrize("w", FLAT, ids=name)
def test_sweep_forward(lsa, w):
    P.test_forward_matches_oracle(lsa, w)


@pytest.mark.parametrize("w", LONG, ids=name)
def test_sweep_long_rows_routing(lsa, w):
    P.test_routing_long_rows_sampled(lsa, w)


@pytest.mark.parametrize("w", CONSENSUS, ids=name)
def test_sweep_consensus_forward(lsa, w):
    C.test_consensus_forward_matches_oracle(lsa, w)


@pytest.mark.parametrize("w,beta", CUMULANT, ids=name)
def test_sweep_cumulant_forward(lsa, w, beta):
    U.test_cumulant_forward_matches_oracle(lsa, w, beta)


@pytest.mark.parametrize("w,beam", TREE, ids=name)
def test_sweep_tree_forward(lsa, w, beam):
    T.test_tree_forward_matches_oracle(lsa, w, beam)


@pytest.mark.parametrize("w,steps", DECODE, ids=name)
def test_sweep_decode(lsa, w, steps):
    D.test_decode_matches_oracle(lsa, w, steps)


@pytest.mark.parametrize("w", WIDE, ids=name)
def test_sweep_wide_forward(lsa, w):
    P.test_forward_matches_oracle(lsa, w)


@pytest.mark.parametrize("w", WIDE_CONSENSUS, ids=name)
def test_sweep_wide_consensus_forward(lsa, w):
    C.test_consensus_forward_matches_oracle(lsa, w)


@pytest.mark.parametrize("w,beta", WIDE_CUMULANT, ids=name)
def test_sweep_wide_cumulant_forward(lsa, w, beta):
    U.test_cumulant_forward_matches_oracle(lsa, w, beta)


@pytest.mark.parametrize("w,beam", WIDE_TREE, ids=name)
def test_sweep_wide_tree_forward(lsa, w, beam):
    T.test_tree_forward_matches_oracle(lsa, w, beam)


@pytest.mark.parametrize("w,steps", WIDE_DECODE, ids=name)
def test_sweep_wide_decode(lsa, w, steps):
    D.test_decode_matches_oracle(lsa, w, steps)
