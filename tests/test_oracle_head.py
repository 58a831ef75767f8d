"""Pins of the greedy-step oracle (oracle/head_oracle.py) against closed forms, a scalar loop with
its own unpacking and rounding, and hand-made ties."""
import numpy as np

import synth
from oracle import head_oracle as Hd
from synth.moe_inputs import f32_to_bf16_bits


def _bf16_value(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _scalar_logits(x_bits, head):
    """logits by loops: each nibble unpacked with shifts, w = s*q + b in fp32 (exact), rounded to
    bf16 through the fp32 bit pattern, then summed in fp64."""
    q, s, b = head
    x = _bf16_value(x_bits)
    T, H = x.shape
    V = q.shape[1]
    out = np.zeros((T, V))
    for v in range(V):
        w = np.empty(H)
        for i in range(H):
            nib = (int(q[0, v, i // 8]) >> (4 * (i % 8))) & 15
            sv = np.float32(_bf16_value(s[0, v, i // 64]))
            bv = np.float32(_bf16_value(b[0, v, i // 64]))
            w[i] = _bf16_value(f32_to_bf16_bits(np.array([sv * np.float32(nib) + bv], np.float32)))[0]
        for t in range(T):
            out[t, v] = sum(x[t, i] * w[i] for i in range(H))
    return out


def test_argmax_takes_the_lowest_index_among_equal_maxima():
    lg = np.array([[1.0, 3.0, 3.0, 2.0], [-1.0, -1.0, -5.0, -1.0], [0.0, 0.0, 0.0, 7.0]])
    assert Hd.greedy(lg).tolist() == [1, 0, 3]


def test_near_tie_reports_close_top_two():
    lg = np.array([[1.0, 1.00005, 0.0], [1.0, 2.0, 0.0]])
    assert Hd.near_tie(lg).tolist() == [0]
    assert Hd.near_tie(np.array([[3.0], [1.0]])).tolist() == []   # one entry: no rival


def test_logits_match_a_scalar_loop():
    w = synth.make_head(7, 128, seed=3)
    x = synth.make_tokens(synth.SHAPES["tiny"], 2, seed=5)[:, :128]
    np.testing.assert_allclose(Hd.lm_logits(x, w["head"]), _scalar_logits(x, w["head"]), rtol=1e-12, atol=1e-12)


def test_logits_closed_form_with_constant_nibbles():
    """All nibbles 9 and bias -8*scale: every weight equals its group's scale, so a logit is the
    scale-weighted sum of the token's group sums."""
    V, H = 5, 256
    w = synth.make_head(V, H, seed=1)["head"]
    q = np.full_like(w[0], 0x99999999)
    head = (q, w[1], w[2])
    x = synth.make_tokens(synth.SHAPES["tiny"], 3, seed=2)
    xv = _bf16_value(x)
    gs = xv.reshape(3, H // 64, 64).sum(axis=2)
    want = gs @ _bf16_value(w[1][0]).T
    np.testing.assert_allclose(Hd.lm_logits(x, head), want, rtol=1e-12, atol=1e-12)


def test_embedding_rows_are_the_rounded_dequantised_values():
    V, H = 4, 128
    q, s, b = synth.make_head(V, H, seed=7)["embed"]
    q = q.copy()
    q[0, 1, :] = 0x76543210      # nibbles 0..7 in order
    q[0, 2, :] = 0x88888888      # q = 8 with b = -8 s: all zero
    e = Hd.embed(np.array([1, 2, 1]), (q, s, b))
    sv = _bf16_value(s[0, 1]).astype(np.float32)
    bv = _bf16_value(b[0, 1]).astype(np.float32)
    vals = np.repeat(sv, 64) * np.tile(np.arange(8, dtype=np.float32), H // 8) + np.repeat(bv, 64)
    assert np.array_equal(e[0], f32_to_bf16_bits(vals.astype(np.float32)))
    assert np.array_equal(e[2], e[0])
    assert np.all(_bf16_value(e[1]) == 0.0)


def test_greedy_step_takes_the_argmax_token_and_its_embedding():
    w = synth.make_head(11, 128, seed=4)
    x = synth.make_tokens(synth.SHAPES["tiny"], 2, seed=9)[:, :128]
    tok, nxt, lg = Hd.greedy_step(x, w["head"], w["embed"])
    ref = _scalar_logits(x, w["head"])
    assert tok.tolist() == [int(np.argmax(r)) for r in ref]
    assert np.array_equal(nxt, Hd.embed(tok, w["embed"]))
    # the bf16 profile differs from the exact one only through the weights' rounding
    ex = Hd.lm_logits(x, w["head"], "exact")
    assert np.abs(ex - lg).max() > 0 and np.abs(ex - lg).max() < 1e-2 * np.abs(lg).max()
