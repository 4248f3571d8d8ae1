"""Seeded generators: determinism, bf16 rounding, Z-order, needle placement."""
import numpy as np

from content_routed_block_amd.workloads import (WORKLOADS, bf16_bits_to_f32, generate,
                                                to_bf16_bits, zorder_permutation)


def test_bf16_round_to_nearest_even():
    one = np.float32(1.0)
    ulp = np.float32(2.0 ** -7)
    vals = np.array([1.0, one + ulp / 2, one + 3 * ulp / 2, one + ulp / 4,
                     -2.5, 3.0e38, 1e-40], np.float32)
    got = to_bf16_bits(vals)
    assert got[0] == 0x3F80
    assert got[1] == 0x3F80          # tie -> even
    assert got[2] == 0x3F82          # tie -> even (up)
    assert got[3] == 0x3F80
    assert got[4] == 0xC020
    back = bf16_bits_to_f32(got)
    assert back[4] == -2.5


def test_generation_is_deterministic():
    w = WORKLOADS["tiny_causal_n1024"]
    a, b = generate(w), generate(w)
    for x, y in ((a.q, b.q), (a.k, b.k), (a.v, b.v)):
        assert x.dtype == np.uint16
        np.testing.assert_array_equal(x, y)
    c = generate(w, seed=99)
    assert not np.array_equal(a.q, c.q)
    assert a.q.shape == (1, 2, 1024, 64) and a.k.shape == (1, 1, 1024, 64)


def test_zorder_squares():
    side = 16
    perm = zorder_permutation(side)
    assert sorted(perm) == list(range(side * side))
    rows, cols = perm // side, perm % side
    for run in (4, 16, 64):
        s = int(np.sqrt(run))
        for start in range(0, side * side, run):
            r, c = rows[start:start + run], cols[start:start + run]
            assert r.max() - r.min() == s - 1 and c.max() - c.min() == s - 1
            assert r.min() % s == 0 and c.min() % s == 0
    # the row bit sits above the column bit: slots 0..3 are (0,0),(0,1),(1,0),(1,1)
    assert list(perm[:4]) == [0, 1, side, side + 1]


def test_topic_mixture_and_needles():
    w = WORKLOADS["qwen05b_n32k"].replace(seq_len=4096, needles=8, name="small")
    inp = generate(w)
    q = bf16_bits_to_f32(inp.q).astype(np.float64)
    k = bf16_bits_to_f32(inp.k).astype(np.float64)
    # same token, same group: query and key share a topic direction (2*U, |U|=1)
    same = np.einsum("nd,nd->n", q[0, 0], k[0, 0]).mean()
    assert 3.0 < same < 5.0
    for nd in inp.needles:
        assert nd.h // (w.q_heads // w.kv_heads) == nd.g
        assert nd.p <= nd.t - w.window - w.block
        np.testing.assert_array_equal(
            bf16_bits_to_f32(inp.k[nd.b, nd.g, nd.p]), 4.0 * bf16_bits_to_f32(inp.q[nd.b, nd.h, nd.t]))
    blocks = {(n.b, n.g, n.p // w.block) for n in inp.needles}
    assert len(blocks) == len(inp.needles)


def test_image_field_is_smooth_in_zorder():
    w = WORKLOADS["image_zorder_128x128"].replace(batch=1, q_heads=2, kv_heads=2,
                                                   seq_len=1024, image_side=32, name="small")
    inp = generate(w)
    k = bf16_bits_to_f32(inp.k[0, 0]).astype(np.float64)
    near = np.mean(np.sum(k[0::2] * k[1::2], axis=1))       # Z-order neighbours
    far = np.mean(np.sum(k[:512] * k[512:], axis=1))
    assert near > 0.5 * np.mean(np.sum(k * k, axis=1)) and abs(far) < near
