"""Pins of the gated delta-rule oracle (CPU): closed forms, the delta rule's defining property
and a scalar brute-force loop, chosen so that a plausible mistake (a missing decay or beta, a
transposed outer product, the state multiplied on the wrong side, a wrong head mapping, an
unnormalised key) fails at least one."""
import math

import numpy as np

import synth
from oracle import delta_oracle as Dn
from oracle import moe_oracle as O


def _bits(a):
    return synth.f32_to_bf16_bits(np.asarray(a, np.float32))


def _inputs(shape, B, T, seed=0, zero_state=False):
    return synth.make_delta_inputs(shape, B, T, seed, zero_state)


def test_no_write_is_pure_decay():
    """beta = 0: S_t = alpha_t S_{t-1}, so S_T = (prod alpha) S_0 and o_t = (prod_{u<=t} alpha_u) S_0 qh_t."""
    shape = synth.DeltaShape(2, 2, 8, 4)
    q, k, v, g, beta, s0 = _inputs(shape, 1, 5, seed=1)
    beta = np.zeros_like(beta)
    o, S = Dn.recurrence(q, k, v, g, beta, s0)
    decay = np.exp(np.cumsum(g.astype(np.float64), axis=1))          # [B, T, Hv]
    qh = Dn.l2_normalise(O.bf16_to_f64(q)) / math.sqrt(8)
    for t in range(5):
        for j in range(2):
            want = decay[0, t, j] * (s0[0, j].astype(np.float64) @ qh[0, t, j])
            assert np.allclose(o[0, t, j], want, rtol=1e-12, atol=1e-15)
    assert np.allclose(S[0], decay[0, -1][:, None, None] * s0[0], rtol=1e-12, atol=1e-15)


def test_first_step_from_zero_state():
    """S_0 = 0: S_1 = beta v kh^T and o_1 = beta (kh . qh) v, for every head."""
    shape = synth.DeltaShape(2, 4, 16, 8)
    q, k, v, g, beta, s0 = _inputs(shape, 2, 1, seed=2, zero_state=True)
    o, S = Dn.recurrence(q, k, v, g, beta, s0)
    for b in range(2):
        for j in range(4):
            i = j // 2
            kh = Dn.l2_normalise(O.bf16_to_f64(k[b, 0, i]))
            qh = Dn.l2_normalise(O.bf16_to_f64(q[b, 0, i])) / 4.0
            vv = O.bf16_to_f64(v[b, 0, j])
            bt = float(beta[b, 0, j])
            assert np.allclose(S[b, j], bt * np.outer(vv, kh), rtol=1e-13, atol=1e-16)
            assert np.allclose(o[b, 0, j], bt * float(kh @ qh) * vv, rtol=1e-12, atol=1e-16)


def test_delta_rule_writes_the_value_under_its_key():
    """alpha = 1, beta = 1: the step replaces what the state returned for kh by v, so
    S_t kh_t = v_t exactly (up to the eps in the key normalisation)."""
    shape = synth.DeltaShape(1, 1, 16, 8)
    q, k, v, g, beta, s0 = _inputs(shape, 1, 6, seed=3)
    g, beta = np.zeros_like(g), np.ones_like(beta)
    for t in range(1, 7):
        _, S = Dn.recurrence(q[:, :t], k[:, :t], v[:, :t], g[:, :t], beta[:, :t], s0)
        kh = Dn.l2_normalise(O.bf16_to_f64(k[0, t - 1, 0]), eps=0.0)
        assert np.allclose(S[0, 0] @ kh, O.bf16_to_f64(v[0, t - 1, 0]), rtol=1e-6, atol=1e-6)


def test_orthogonal_keys_are_all_retrievable():
    """Orthogonal unit keys written with alpha = beta = 1 into a zero state do not disturb each
    other: afterwards S e_i = v_i for every written key e_i."""
    Dk, Dv, T = 8, 4, 5
    kk = np.zeros((1, T, 1, Dk), np.float32)
    for t in range(T):
        kk[0, t, 0, t] = 2.0                      # orthogonal, normalised by the oracle
    rng = np.random.default_rng(4)
    q = _bits(rng.standard_normal((1, T, 1, Dk)))
    vv = _bits(rng.standard_normal((1, T, 1, Dv)))
    g = np.zeros((1, T, 1), np.float32)
    beta = np.ones((1, T, 1), np.float32)
    _, S = Dn.recurrence(q, _bits(kk), vv, g, beta, np.zeros((1, 1, Dv, Dk), np.float32), eps=0.0)
    for t in range(T):
        assert np.allclose(S[0, 0][:, t], O.bf16_to_f64(vv[0, t, 0]), rtol=1e-14, atol=1e-15)
    assert np.all(S[0, 0][:, T:] == 0)


def test_two_pieces_equal_one_run():
    shape = synth.DeltaShape(2, 4, 16, 16)
    q, k, v, g, beta, s0 = _inputs(shape, 2, 9, seed=5)
    o, S = Dn.recurrence(q, k, v, g, beta, s0)
    o1, S1 = Dn.recurrence(q[:, :4], k[:, :4], v[:, :4], g[:, :4], beta[:, :4], s0)
    o2, S2 = Dn.recurrence(q[:, 4:], k[:, 4:], v[:, 4:], g[:, 4:], beta[:, 4:], S1)
    assert np.allclose(np.concatenate([o1, o2], axis=1), o, rtol=1e-13, atol=1e-14)
    assert np.allclose(S2, S, rtol=1e-13, atol=1e-14)


def test_value_heads_share_their_key_head():
    """Hv = 2 Hk: value heads 2i and 2i+1 read q/k head i; with equal v, g, beta and state they
    give equal outputs, and heads of different groups differ."""
    shape = synth.DeltaShape(2, 4, 8, 8)
    q, k, v, g, beta, s0 = _inputs(shape, 1, 3, seed=6)
    v[:, :, 1], g[:, :, 1], beta[:, :, 1], s0[:, 1] = v[:, :, 0], g[:, :, 0], beta[:, :, 0], s0[:, 0]
    v[:, :, 2], g[:, :, 2], beta[:, :, 2], s0[:, 2] = v[:, :, 0], g[:, :, 0], beta[:, :, 0], s0[:, 0]
    o, _ = Dn.recurrence(q, k, v, g, beta, s0)
    assert np.array_equal(o[:, :, 0], o[:, :, 1])
    assert not np.allclose(o[:, :, 0], o[:, :, 2])


def test_against_scalar_loops():
    """The update written element by element: S[r, c] <- a (S[r, c] - b (sum_m S[r, m] kh[m]) kh[c])
    + b v[r] kh[c], then o[r] = sum_c S[r, c] qh[c]."""
    shape = synth.DeltaShape(1, 2, 4, 3)
    q, k, v, g, beta, s0 = _inputs(shape, 1, 4, seed=7)
    o, S = Dn.recurrence(q, k, v, g, beta, s0)
    f = lambda x: [float(t) for t in O.bf16_to_f64(x)]  # noqa: E731
    for j in range(2):
        St = [[float(s0[0, j, r, c]) for c in range(4)] for r in range(3)]
        for t in range(4):
            kk, qq, vv = f(k[0, t, 0]), f(q[0, t, 0]), f(v[0, t, j])
            nk = math.sqrt(sum(x * x for x in kk) + 1e-6)
            nq = math.sqrt(sum(x * x for x in qq) + 1e-6)
            kh = [x / nk for x in kk]
            qh = [x / nq / 2.0 for x in qq]          # scale = 1/sqrt(4)
            a, b = math.exp(float(g[0, t, j])), float(beta[0, t, j])
            for r in range(3):
                u = sum(St[r][m] * kh[m] for m in range(4))
                for c in range(4):
                    St[r][c] = a * (St[r][c] - b * u * kh[c]) + b * vv[r] * kh[c]
            for r in range(3):
                want = sum(St[r][c] * qh[c] for c in range(4))
                assert abs(o[0, t, j, r] - want) <= 1e-12 * max(1.0, abs(want))
        for r in range(3):
            for c in range(4):
                assert abs(S[0, j, r, c] - St[r][c]) <= 1e-12 * max(1.0, abs(St[r][c]))
