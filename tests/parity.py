"""Parity helpers shared by the GPU tests: move seeded inputs to the device,
call the HIP path through the C ABI binding, compare with the CPU oracle.

Routing parity (the pages' method gives several correct answers on ties):
  * rows whose oracle gap (k-th minus (k+1)-th routing score) exceeds 1e-3
    must select bit-identical block sets;
  * other rows ("near ties") may differ, but then the GPU set must be a valid
    top-k under the oracle's fp64 scores to within 1e-3:
    min s(selected) >= max s(unselected candidates) - 1e-3, with the right
    count, ascending order and -1 padding.
Output parity: max-abs <= 2e-2 and mean-abs <= 5e-3 against the fp32 oracle,
plus a tighter bound derived from the arithmetic: bf16 rounding of the
probabilities and of the routed partial outputs perturbs each output by at
most 2^-9 * max|v| each, so |err| <= 2^-8 * max|v| per row.
"""
import numpy as np
import torch

import oracle

GAP = 1e-3
MAX_ABS, MEAN_ABS = 2e-2, 5e-3
REL_V = 2.0 ** -8


def dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda()


def params_of(lsa, w, **over):
    kw = dict(batch=w.batch, q_heads=w.q_heads, kv_heads=w.kv_heads, seq_len=w.seq_len,
              head_dim=w.head_dim, block=w.block, top_k=w.top_k, window=w.window,
              causal=w.causal)
    kw.update(over)
    return lsa.params(**kw)


def causal_candidates(t, bs, window):
    return np.maximum(0, t // bs - window // bs + 1)


def check_routing(idx_gpu, idx_orc, gap, scores, ncand, k):
    """idx_gpu / idx_orc: [R, k]; gap: [R]; scores: [R, nb] oracle scores
    (-inf off the candidate set); ncand: [R].  Returns (n_clear_mismatch,
    n_near, n_near_differing).  Raises AssertionError on an invalid set."""
    idx_gpu = np.asarray(idx_gpu)
    idx_orc = np.asarray(idx_orc)
    clear = gap > GAP
    differ = np.any(idx_gpu != idx_orc, axis=1)
    bad_clear = int(np.sum(differ & clear))
    near_rows = np.nonzero(differ & ~clear)[0]
    for r in near_rows:
        sel = idx_gpu[r]
        m = min(k, int(ncand[r]))
        assert np.all(sel[m:] == -1), (r, sel)
        chosen = sel[:m]
        assert np.all(chosen >= 0) and np.all(chosen < ncand[r]), (r, sel)
        assert np.all(np.diff(chosen) > 0), (r, sel)
        s = scores[r]
        rest = np.setdiff1d(np.arange(int(ncand[r])), chosen)
        if rest.size:
            assert s[chosen].min() >= s[rest].max() - GAP, (r, s[chosen].min(), s[rest].max())
    return bad_clear, int(np.sum(~clear)), len(near_rows)


def check_needles(sel_gpu, sel_orc, gap, scores, ncand, needle_blocks, k):
    """Needle rows.  Mean-pooled block summaries can lose an isolated key (SSA
    page, "The retrieval law"), so a needle's selection is measured, not
    assumed, and the GPU must agree with the oracle row by row: the needle's
    block is in the GPU set exactly when it is in the oracle's.  Where the two
    differ the row must be a near tie (gap <= GAP) and the needle block's
    oracle score must lie within GAP of the row's k-th best score, so that
    either choice is a valid top-k.  sel_*: [R, k] sets of the needle rows;
    gap: [R]; scores: [R, nb] oracle scores; ncand: [R]; needle_blocks: [R].
    Returns (recall_gpu, recall_oracle, n_differing)."""
    hits_g = hits_o = differing = 0
    for r in range(len(needle_blocks)):
        c = int(needle_blocks[r])
        hg, ho = c in sel_gpu[r], c in sel_orc[r]
        hits_g += int(hg)
        hits_o += int(ho)
        if hg != ho:
            differing += 1
            assert gap[r] <= GAP, (r, c, gap[r])
            s = np.asarray(scores[r][:int(ncand[r])], np.float64)
            kth = np.sort(s)[::-1][min(k, s.size) - 1]
            assert abs(s[c] - kth) <= GAP, (r, c, s[c], kth)
    return hits_g, hits_o, differing


def check_output(out_gpu, out_ref, vmax_row):
    """out_*: [R, D] float; vmax_row: [R] max |v| over the row's keys (or a
    global bound).  Returns (max_abs, mean_abs)."""
    err = np.abs(np.asarray(out_gpu, np.float64) - np.asarray(out_ref, np.float64))
    max_abs, mean_abs = float(err.max()), float(err.mean())
    assert max_abs <= MAX_ABS, max_abs
    assert mean_abs <= MEAN_ABS, mean_abs
    row_err = err.max(axis=1)
    worst = float(np.max(row_err / np.maximum(vmax_row, 1e-30)))
    assert worst <= REL_V, worst
    return max_abs, mean_abs


def check_tree_routing(idx_gpu, idx_orc, det, block_scores, ncand, k, beam, fanout=16):
    """Two-level routing parity.  Rows whose node-level and block-level gaps
    both exceed GAP must match the oracle bit for bit.  Any other row that
    differs must be a valid outcome: some beam B* of min(beam, S) complete
    candidate nodes, holding every node that beats the beam-th node score by
    more than GAP and only nodes within GAP of it otherwise, for which the
    GPU set is a valid top-k (within GAP) of B*'s blocks plus the tail.
    det: the oracle's details (gap1, gap2, node_scores); block_scores: [R, nb]
    fp64 oracle block scores.  Returns (n_clear_mismatch, n_near,
    n_near_differing)."""
    idx_gpu = np.asarray(idx_gpu)
    idx_orc = np.asarray(idx_orc)
    clear = (det["gap1"] > GAP) & (det["gap2"] > GAP)
    differ = np.any(idx_gpu != idx_orc, axis=1)
    bad_clear = int(np.sum(differ & clear))
    near_rows = np.nonzero(differ & ~clear)[0]
    for r in near_rows:
        E = int(ncand[r])
        S = E // fanout
        nb_keep = min(beam, S)
        ns = det["node_scores"][r][:S]
        s = block_scores[r]
        order = np.sort(ns)[::-1]
        th = order[nb_keep - 1] if S > nb_keep else -np.inf
        certain = [x for x in range(S) if ns[x] > th + GAP] if S > nb_keep else list(range(S))
        maybe = [x for x in range(S) if abs(ns[x] - th) <= GAP and x not in certain] \
            if S > nb_keep else []
        sel = idx_gpu[r]
        tail = list(range(S * fanout, E))
        m = min(k, fanout * nb_keep + len(tail))
        assert np.all(sel[m:] == -1), (r, sel)
        chosen = sel[:m]
        assert np.all(chosen >= 0) and np.all(chosen < E) and np.all(np.diff(chosen) > 0), (r, sel)
        nodes = set(int(c) // fanout for c in chosen if c < S * fanout)
        assert nodes <= set(certain) | set(maybe), (r, sorted(nodes), certain, maybe)
        used_maybe = nodes - set(certain)
        free = nb_keep - len(certain) - len(used_maybe)
        assert free >= 0, (r, len(certain), len(used_maybe), nb_keep)
        lo = s[chosen].min() if m else np.inf
        opened = set(certain) | used_maybe
        rest = [c for x in opened for c in range(x * fanout, x * fanout + fanout)] + tail
        rest = np.setdiff1d(np.array(rest, dtype=np.int64), chosen)
        if rest.size:
            assert s[rest].max() <= lo + GAP, (r, s[rest].max(), lo)
        harmless = [x for x in maybe if x not in used_maybe
                    and s[x * fanout:(x + 1) * fanout].max() <= lo + GAP]
        assert len(harmless) >= free, (r, len(harmless), free)
    return bad_clear, int(np.sum(~clear)), len(near_rows)
