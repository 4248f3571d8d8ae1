"""Brute-force numpy reference for tiny inputs, written independently of the
oracle (different algorithms: rank counting instead of sorting, an explicit
dense N x N mask instead of key ranges) so that the two can pin each other.

Everything is fp64; bf16 inputs arrive as uint16 bit patterns.
"""
import numpy as np

from content_routed_block_amd.workloads import bf16_bits_to_f32


def widen(x_bits):
    return bf16_bits_to_f32(x_bits).astype(np.float64)


def block_means(xf, bs):
    """xf: float64 [..., N, D] -> float32 [..., N/bs, D] (fp64 mean, one rounding)."""
    *lead, N, D = xf.shape
    return xf.reshape(*lead, N // bs, bs, D).mean(axis=-2).astype(np.float32)


def rank_select(scores, ncand, k):
    """Selection by rank counting: candidate c is kept when fewer than k
    candidates beat it, where c' beats c if s[c'] > s[c], or s[c'] == s[c]
    and c' < c.  Returns the kept block ids in ascending order."""
    keep = []
    for c in range(ncand):
        beaten = 0
        for c2 in range(ncand):
            if scores[c2] > scores[c] or (scores[c2] == scores[c] and c2 < c):
                beaten += 1
        if beaten < k:
            keep.append(c)
    return keep


def _router_heads(h, rep, consensus):
    """The query heads whose scores are summed to route head h: itself, or,
    with consensus routing, every head of its KV group."""
    g = h // rep
    return range(g * rep, (g + 1) * rep) if consensus else [h]


def causal_mask(N, bs, window, top_k, q_f64, kbar, rep, consensus=False):
    """Dense boolean mask [Hq, N, N] of the keys each causal query attends to.
    q_f64: [Hq, N, D]; kbar: float32 [Hkv, nb, D]."""
    Hq = q_f64.shape[0]
    mask = np.zeros((Hq, N, N), dtype=bool)
    wb = window // bs
    for h in range(Hq):
        g = h // rep
        for t in range(N):
            ncand = max(0, t // bs - wb + 1)
            s = [sum(float(np.dot(q_f64[hh, t], kbar[g, c].astype(np.float64)))
                     for hh in _router_heads(h, rep, consensus)) for c in range(ncand)]
            for c in rank_select(s, ncand, top_k):
                mask[h, t, c * bs:(c + 1) * bs] = True
            mask[h, t, ncand * bs:t + 1] = True
    return mask


def image_mask(N, bs, top_k, qbar, kbar, rep, consensus=False):
    Hq = qbar.shape[0]
    nb = N // bs
    mask = np.zeros((Hq, N, N), dtype=bool)
    for h in range(Hq):
        g = h // rep
        for i in range(nb):
            s = [sum(float(np.dot(qbar[hh, i].astype(np.float64), kbar[g, c].astype(np.float64)))
                     for hh in _router_heads(h, rep, consensus)) for c in range(nb)]
            for c in rank_select(s, nb, top_k):
                mask[h, i * bs:(i + 1) * bs, c * bs:(c + 1) * bs] = True
    return mask


def masked_softmax_attention(q_f64, k_f64, v_f64, mask, rep, scale):
    """q [Hq,N,D], k/v [Hkv,N,D], mask [Hq,N,N] -> [Hq,N,D] fp64."""
    Hq, N, D = q_f64.shape
    out = np.empty((Hq, N, D))
    for h in range(Hq):
        g = h // rep
        logits = (q_f64[h] @ k_f64[g].T) * scale
        logits = np.where(mask[h], logits, -np.inf)
        m = logits.max(axis=1, keepdims=True)
        p = np.exp(logits - m)
        out[h] = (p @ v_f64[g]) / p.sum(axis=1, keepdims=True)
    return out


def forward(q_bits, k_bits, v_bits, bs, top_k, window, causal, scale=None, consensus=False):
    """End-to-end brute force for one batch element: q [Hq,N,D], k/v [Hkv,N,D].
    consensus: route once per KV group by the sum of its heads' scores."""
    qf, kf, vf = widen(q_bits), widen(k_bits), widen(v_bits)
    Hq, N, D = qf.shape
    rep = Hq // kf.shape[0]
    scale = 1.0 / np.sqrt(D) if scale is None else scale
    kbar = block_means(kf, bs)
    if causal:
        mask = causal_mask(N, bs, window, top_k, qf, kbar, rep, consensus)
    else:
        mask = image_mask(N, bs, top_k, block_means(qf, bs), kbar, rep, consensus)
    return masked_softmax_attention(qf, kf, vf, mask, rep, scale), mask


def cumulant_score(q_f64, keys_f64, mu_f32, beta):
    """Second-cumulant routing score of one block, computed from the spread
    of the block's raw scores instead of a covariance matrix:
    <q, mu> + (beta/2) * (population variance over the block of q . k_j)."""
    s = keys_f64 @ q_f64
    return float(np.dot(q_f64, mu_f32.astype(np.float64))) + 0.5 * beta * float(np.var(s))


def tree_select(q_f64, kbar_g, E, F, beam, k):
    """Two-level selection for one row by rank counting: node summaries are
    the fp32-rounded fp64 means of F consecutive block means; the best beam
    of the floor(E/F) complete nodes are kept; top-k over their blocks plus
    blocks [F*floor(E/F), E).  kbar_g: float32 [nb, D]."""
    S = E // F
    nu = [kbar_g[s * F:(s + 1) * F].astype(np.float64).mean(axis=0).astype(np.float32)
          for s in range(S)]
    ns = [float(np.dot(q_f64, nu[s].astype(np.float64))) for s in range(S)]
    kept = rank_select(ns, S, beam)
    cands = [s * F + x for s in kept for x in range(F)] + list(range(S * F, E))
    cs = [float(np.dot(q_f64, kbar_g[c].astype(np.float64))) for c in cands]
    # rank over the candidate set (ties to the lower block id)
    keep = []
    for a, ca in enumerate(cands):
        beaten = sum(1 for b, cb in enumerate(cands)
                     if cs[b] > cs[a] or (cs[b] == cs[a] and cb < ca))
        if beaten < k:
            keep.append(ca)
    return sorted(keep)
