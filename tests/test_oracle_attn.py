"""Pins of the decode-attention oracle (CPU): closed forms, invariants and a scalar brute-force
loop, each chosen so that a plausible mistake (a wrong group index, a missing scale or max
shift, a transposed operand, a wrong block/row in the cache gather) fails at least one."""
import math

import numpy as np
import pytest

import synth
from oracle import attn_oracle as A
from oracle import moe_oracle as O


def _bits(a):
    return synth.f32_to_bf16_bits(np.asarray(a, np.float32))


def test_single_key_returns_its_value():
    """S = 1: the only key gets weight 1 whatever the scores, so out_h = V_g(h)[0]."""
    rng = np.random.default_rng(1)
    q = rng.standard_normal((8, 16))
    k = rng.standard_normal((2, 1, 16))
    v = rng.standard_normal((2, 1, 16))
    out = A.attention(q, k, v, 0.37)
    for h in range(8):
        assert np.array_equal(out[h], v[h // 4, 0])


def test_equal_keys_and_zero_scale_give_the_mean_value():
    rng = np.random.default_rng(2)
    q = rng.standard_normal((4, 8))
    v = rng.standard_normal((2, 5, 8))
    k_same = np.repeat(rng.standard_normal((2, 1, 8)), 5, axis=1)   # every key equal
    k_rand = rng.standard_normal((2, 5, 8))
    for k, scale in ((k_same, 0.5), (k_rand, 0.0)):
        out = A.attention(q, k, v, scale)
        for h in range(4):
            assert np.allclose(out[h], v[h // 2].mean(axis=0), rtol=1e-14, atol=1e-15)


def test_dominant_key_selects_its_value_and_scale_matters():
    """A key aligned with q far more than the others takes almost all the weight; the closed
    form of two keys pins the scale: p_0 = 1 / (1 + exp(scale * (s1 - s0)))."""
    D = 8
    q = np.zeros((2, D))
    q[:, 0] = 1.0
    k = np.zeros((1, 2, D))
    k[0, 0, 0], k[0, 1, 0] = 3.0, 1.0           # raw scores 3 and 1
    v = np.zeros((1, 2, D))
    v[0, 0, 1], v[0, 1, 2] = 1.0, 1.0
    for scale in (0.25, 1.0, 40.0):
        out = A.attention(q, k, v, scale)
        p0 = 1.0 / (1.0 + math.exp(scale * (1.0 - 3.0)))
        assert abs(out[0, 1] - p0) < 1e-15 and abs(out[0, 2] - (1 - p0)) < 1e-15
        assert np.array_equal(out[0], out[1])
    assert A.attention(q, k, v, 40.0)[0, 2] < 1e-30   # exp(-80): the other key vanishes


def test_group_mapping_of_query_heads():
    """Hq = 6, Hkv = 3: heads 2h and 2h+1 read KV head h. With identical queries, heads of one
    group agree and heads of different groups read their own values."""
    rng = np.random.default_rng(3)
    q = np.repeat(rng.standard_normal((1, 8)), 6, axis=0)
    k = rng.standard_normal((3, 7, 8))
    v = np.stack([np.full((7, 8), float(g)) for g in range(3)])   # KV head g holds value g
    out = A.attention(q, k, v, 0.3)
    for h in range(6):
        assert np.allclose(out[h], h // 2, rtol=0, atol=1e-15)


def test_token_order_and_block_placement_do_not_matter():
    """Permuting the tokens (keys and values together) or scattering the blocks over the cache
    leaves the output unchanged; the gather itself is checked against a contiguous copy."""
    shape = synth.AttnShape(4, 2, 16, 4)
    q, kc, vc, table, lens = synth.make_attn_inputs(shape, [13], seed=5, spare_blocks=2)
    out = A.decode_attention(q, kc, vc, table, lens, shape.block_size, 0.25)
    k = A.gather_kv(kc, table[0], 13, 4)
    v = A.gather_kv(vc, table[0], 13, 4)
    # the gather against an explicit block copy
    blocks = [O.bf16_to_f64(kc[b]) for b in table[0][:4]]
    contig = np.concatenate(blocks, axis=1)[:, :13, :]
    assert np.array_equal(k, contig)
    perm = np.random.default_rng(0).permutation(13)
    q0 = O.bf16_to_f64(q[0])
    assert np.allclose(A.attention(q0, k[:, perm], v[:, perm], 0.25), out[0], rtol=1e-13, atol=1e-15)
    # the same tokens in a cache with other physical blocks (a different permutation)
    n_phys = kc.shape[0]
    new_pos = np.random.default_rng(9).permutation(n_phys)
    kc2, vc2 = np.empty_like(kc), np.empty_like(vc)
    kc2[new_pos], vc2[new_pos] = kc, vc
    table2 = np.where(table >= 0, new_pos[np.maximum(table, 0)], -1).astype(np.int32)
    out2 = A.decode_attention(q, kc2, vc2, table2, lens, 4, 0.25)
    assert np.array_equal(out2, out)


def test_against_scalar_loops():
    """Every sum written out as a Python loop over tokens and dimensions (tiny sizes)."""
    shape = synth.AttnShape(4, 2, 8, 4)
    q, kc, vc, table, lens = synth.make_attn_inputs(shape, [1, 6, 9], seed=7)
    scale = 1.0 / math.sqrt(8)
    got = A.decode_attention(q, kc, vc, table, lens, 4, scale)
    f = lambda bits: float(O.bf16_to_f64(np.array([bits], np.uint16))[0])  # noqa: E731
    for b in range(3):
        for h in range(4):
            g = h // 2
            s = []
            for j in range(int(lens[b])):
                blk, row = int(table[b, j // 4]), j % 4
                s.append(scale * sum(f(q[b, h, d]) * f(kc[blk, g, row, d]) for d in range(8)))
            m = max(s)
            w = [math.exp(x - m) for x in s]
            tot = sum(w)
            for d in range(8):
                want = sum(w[j] * f(vc[int(table[b, j // 4]), g, j % 4, d])
                           for j in range(len(s))) / tot
                assert abs(got[b, h, d] - want) <= 1e-13 * max(1.0, abs(want))


def test_weights_sum_to_one_and_output_is_a_convex_combination():
    rng = np.random.default_rng(11)
    q = rng.standard_normal((2, 32))
    k = rng.standard_normal((1, 300, 32)) * 3
    v = rng.standard_normal((1, 300, 32))
    out = A.attention(q, k, v, 1.0 / math.sqrt(32))
    assert np.all(out <= v[0].max(axis=0) + 1e-12) and np.all(out >= v[0].min(axis=0) - 1e-12)
    # linear in V
    out2 = A.attention(q, k, 2 * v + 1, 1.0 / math.sqrt(32))
    assert np.allclose(out2, 2 * out + 1, rtol=1e-12, atol=1e-12)


def test_empty_sequence_gives_zero():
    q = np.ones((4, 8))
    out = A.attention(q, np.zeros((2, 0, 8)), np.zeros((2, 0, 8)), 0.5)
    assert out.shape == (4, 8) and np.all(out == 0)


def test_generator_layout():
    shape = synth.ATTN_SHAPES["full"]
    q, kc, vc, table, lens = synth.make_attn_inputs(shape, [100, 1, 64], seed=0)
    assert q.shape == (3, 16, 128) and kc.shape[1:] == (2, 64, 128) and kc.dtype == np.uint16
    assert table.shape == (3, 2) and table[1, 1] == -1 and table[2, 1] == -1
    used = table[table >= 0]
    assert len(set(used.tolist())) == used.size      # distinct physical blocks
