"""Pins for the fp64 oracle: closed forms, brute force and invariants (CPU only).

Each test names what fixes the expected value; none of them re-calls the oracle's own
formula to produce its expectation.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import moe_oracle as O
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]


def _all_finite_bf16():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    exp = (bits >> 7) & 0xFF
    return bits[exp != 0xFF]


def _bf16_exact(bits: int) -> Fraction:
    """IEEE-style decode of a bf16 pattern with Python integers (independent of numpy)."""
    sign = -1 if bits & 0x8000 else 1
    e = (bits >> 7) & 0xFF
    m = bits & 0x7F
    if e == 0:
        return sign * Fraction(m, 128) * Fraction(1, 2 ** 126)
    return sign * (1 + Fraction(m, 128)) * (Fraction(2) ** (e - 127))


# ------------------------------------------------------------------ numbers and formats
def test_bf16_decode_golden():
    for bits, val in _golden_lines("bf16_values.txt"):
        got = O.bf16_to_f64(np.array([int(bits, 16)], np.uint16))[0]
        assert Fraction(got) == Fraction(val), bits


def test_bf16_decode_matches_integer_decode_everywhere():
    bits = _all_finite_bf16()
    vals = O.bf16_to_f64(bits)
    rng = np.random.default_rng(1)
    for b in rng.choice(bits, 2000, replace=False):
        assert Fraction(vals[np.searchsorted(bits, b)]) == _bf16_exact(int(b))


def test_round_to_bf16_ties_to_even():
    one = 1.0
    u = 2.0 ** -7                                      # bf16 spacing on [1, 2)
    cases = [
        (one + u / 2, one),                            # tie, 1.0 has an even fraction
        (one + 3 * u / 2, one + 2 * u),                # tie, 1+2u has the even fraction
        (one + u / 2 + 2.0 ** -30, one + u),           # just above the tie
        (one + u / 2 - 2.0 ** -30, one),               # just below the tie
        (-(one + 3 * u / 2), -(one + 2 * u)),
        (2.0 - u / 4, 2.0),
        (2.0 - 3 * u / 4, 2.0 - u),
        (2.0 - u / 2, 2.0),                            # tie into the next binade (even)
        (0.0, 0.0),
        (2.0 ** -140, 0.0),                            # below half the smallest subnormal
        (3 * 2.0 ** -134, 2.0 ** -132),                # subnormal tie -> even
    ]
    for v, want in cases:
        assert O.round_to_bf16(np.array([v]))[0] == want, v


def test_round_to_bf16_is_nearest_by_brute_force():
    """Against a search over every finite bf16 value (nearest, ties to even fraction)."""
    bits = _all_finite_bf16()
    vals = O.bf16_to_f64(bits)
    order = np.argsort(vals, kind="stable")
    sv, sb = vals[order], bits[order]
    # keep +0 only (drop -0) so neighbours are distinct
    keep = ~((sv == 0) & (sb == 0x8000))
    sv, sb = sv[keep], sb[keep]
    rng = np.random.default_rng(2)
    v = np.concatenate([rng.normal(0, 1, 3000), rng.normal(0, 1e-3, 1000),
                        rng.uniform(-300, 300, 1000)])
    got = O.round_to_bf16(v)
    for x, g in zip(v, got):
        i = np.searchsorted(sv, x)
        lo, hi = sv[i - 1], sv[i]
        dlo, dhi = x - lo, hi - x
        if dlo < dhi:
            want = lo
        elif dhi < dlo:
            want = hi
        else:
            want = lo if (sb[i - 1] & 1) == 0 else hi
        assert g == want


def test_round_to_bf16_fixes_every_bf16_value():
    vals = O.bf16_to_f64(_all_finite_bf16())
    assert np.array_equal(O.round_to_bf16(vals), vals)


def test_unpack_nibbles_golden():
    for row in _golden_lines("nibble_unpack.txt"):
        word = np.array([int(row[0], 16)], np.uint32)
        assert O.unpack_nibbles(word).tolist() == [int(v) for v in row[1:]]


def test_unpack_nibbles_roundtrip_with_independent_packer():
    rng = np.random.default_rng(3)
    q = rng.integers(0, 16, size=(5, 7, 64))
    words = np.zeros((5, 7, 8), np.uint64)
    for j in range(8):                                 # pack with integer arithmetic
        words += q[..., j::8].astype(np.uint64) * (16 ** j)
    assert np.array_equal(O.unpack_nibbles(words.astype(np.uint32)), q)


def _bits(v):
    return synth.f32_to_bf16_bits(np.asarray(v, np.float32))


def test_dequant_special_cases():
    s = _bits([[0.015625, 0.01171875]])               # two groups (exact bf16 values)
    b = _bits([[-8 * 0.015625, -8 * 0.01171875]])
    q8 = np.full((1, 16), 0x88888888, np.uint32)       # q = 8 everywhere -> w = 0
    assert np.all(O.dequant(q8, s, b) == 0.0)
    q9 = np.full((1, 16), 0x99999999, np.uint32)       # q = 9 -> w = s of its group
    w = O.dequant(q9, s, b)
    assert np.all(w[0, :64] == 0.015625) and np.all(w[0, 64:] == 0.01171875)
    # s = 1, b = 0 gives the nibbles themselves; s = 0.5, b = -1 gives q/2 - 1
    s2 = _bits([[1.0, 0.5]])
    b2 = _bits([[0.0, -1.0]])
    words = np.full((1, 16), 0x76543210, np.uint32)
    w2 = O.dequant(words, s2, b2)
    assert w2[0, :8].tolist() == [0, 1, 2, 3, 4, 5, 6, 7]
    assert w2[0, 64:72].tolist() == [-1.0, -0.5, 0.0, 0.5, 1.0, 1.5, 2.0, 2.5]


def test_dequant_exact_rational_on_generated_layer():
    """w = s*q + b checked in exact rational arithmetic on the generator's distribution."""
    L = synth.make_layer(synth.SHAPES["tiny"], seed=0)
    q, s, b = L["gate"]
    w = O.dequant(q[3], s[3], b[3])
    rng = np.random.default_rng(4)
    for n, i in zip(rng.integers(0, q.shape[1], 300), rng.integers(0, q.shape[2] * 8, 300)):
        nib = (int(q[3, n, i // 8]) >> (4 * (i % 8))) & 0xF
        want = _bf16_exact(int(s[3, n, i // 64])) * nib + _bf16_exact(int(b[3, n, i // 64]))
        assert Fraction(w[n, i]) == want
    # the bf16 profile is the nearest bf16 of that exact value
    wb = O.dequant(q[3], s[3], b[3], "bf16")
    assert np.array_equal(O.round_to_bf16(wb), wb)
    assert np.all(np.abs(wb - w) <= np.abs(w) * 2.0 ** -8 + 1e-300)
    frac_changed = np.mean(wb != w)
    assert 0.2 < frac_changed < 0.5                    # the rounding is real on this layer


# ------------------------------------------------------------------------- routing
def test_router_logits_integer_brute_force():
    rng = np.random.default_rng(5)
    T, H, E = 3, 64, 5
    xi = rng.integers(-4, 5, size=(T, H))
    wi = rng.integers(-3, 4, size=(E, H))
    bias = np.array([0.5, -1.0, 0.0, 2.0, -0.25])
    got = O.router_logits(_bits(xi), wi.astype(np.float32), bias.astype(np.float32))
    for t in range(T):
        for e in range(E):
            want = sum(int(xi[t, h]) * int(wi[e, h]) for h in range(H)) + float(bias[e])
            assert got[t, e] == want


def test_topk_matches_full_sort_with_ties():
    rng = np.random.default_rng(6)
    T, E, K = 200, 32, 6
    l = np.round(rng.normal(0, 1, (T, E)), 1)          # many exact ties
    idx, p = O.select_topk(l, K)
    for t in range(T):
        full = sorted(range(E), key=lambda e: (-l[t, e], e))
        assert idx[t].tolist() == full[:K]
    assert np.allclose(p.sum(axis=1), 1.0, atol=1e-12, rtol=0)
    assert np.all(np.diff(p, axis=1) <= 1e-15)         # rank order -> non-increasing weights


def test_topk_softmax_closed_forms():
    K = 4
    l = np.full((2, 10), -5.0)
    l[0, [2, 7, 4, 9]] = np.log([4.0, 3.0, 2.0, 1.0])  # weights proportional to 4:3:2:1
    l[1, :K] = 0.7                                     # equal logits -> 1/K each, low index first
    idx, p = O.select_topk(l, K)
    assert idx[0].tolist() == [2, 7, 4, 9]
    assert np.allclose(p[0], [0.4, 0.3, 0.2, 0.1], rtol=0, atol=1e-15)
    assert idx[1].tolist() == [0, 1, 2, 3]
    assert np.allclose(p[1], 0.25, rtol=0, atol=1e-15)


def test_router_bias_forces_selection():
    L = synth.make_layer(synth.SHAPES["tiny"], seed=1)
    x = synth.make_tokens(synth.SHAPES["tiny"], 6, seed=1)
    bias = np.zeros(16, np.float32)
    bias[[11, 3]] = [100.0, 105.0]
    idx, _ = O.select_topk(O.router_logits(x, L["router_w"], bias), 2)
    assert np.all(idx[:, 0] == 3) and np.all(idx[:, 1] == 11)


def test_shared_gate_closed_forms():
    x = _bits(np.eye(4, 64))                           # one-hot tokens
    wg = np.zeros(64, np.float32)
    assert np.allclose(O.shared_gate(x, wg), 0.5, atol=0, rtol=0)
    wg[0] = np.float32(math.log(3.0))                  # sigmoid(ln 3) = 3/4
    wg[1] = np.float32(-math.log(3.0))                 # sigmoid(-ln 3) = 1/4
    g = O.shared_gate(x, wg)
    assert abs(g[0] - 0.75) < 1e-7 and abs(g[1] - 0.25) < 1e-7 and g[2] == 0.5


def test_near_ties_flags_small_gaps_only():
    l = np.array([[5.0, 4.0, 3.0, 2.0, 2.0 - 5e-5, 0.0],
                  [5.0, 4.0, 3.0, 2.0, 2.0 - 2e-4, 0.0],
                  [5.0, 5.0 - 1e-5, 3.0, 2.0, 1.0, 0.0]])
    assert O.near_ties(l, 4).tolist() == [0, 2]    # ranks 1..5 matter for a top-4
    assert O.near_ties(l, 3).tolist() == [2]       # the rank-4/5 gap cannot change a top-3


# ----------------------------------------------------------------------- permutation
def test_permute_brute_force_and_invariants():
    rng = np.random.default_rng(7)
    for T, E, K in ((1, 16, 2), (37, 8, 3), (300, 32, 4)):
        idx = np.stack([rng.choice(E, K, replace=False) for _ in range(T)])
        counts, offsets, sorted_slots, slot_pos = O.permute(idx, E)
        buckets = [[] for _ in range(E)]
        for s in range(T * K):                          # brute-force stable bucketing
            buckets[idx[s // K, s % K]].append(s)
        assert counts.tolist() == [len(bk) for bk in buckets]
        assert sorted_slots.tolist() == [s for bk in buckets for s in bk]
        assert offsets[0] == 0 and offsets[-1] == T * K
        assert np.array_equal(np.diff(offsets), counts)
        assert np.array_equal(slot_pos[sorted_slots], np.arange(T * K))


# ------------------------------------------------------------------------------- FFN
def test_silu_closed_forms():
    z = np.array([0.0, math.log(3.0), -math.log(3.0), 800.0, -800.0])
    got = O.silu(z)
    assert got[0] == 0.0
    assert abs(got[1] - 0.75 * math.log(3.0)) < 1e-15
    assert abs(got[2] + 0.25 * math.log(3.0)) < 1e-15
    assert got[3] == 800.0 and got[4] == 0.0 and np.all(np.isfinite(got))


def _const_proj(n_out, k_in, c):
    """A projection whose every weight equals c: q = 9 and b = -8s with s = c."""
    q = np.full((1, n_out, k_in // 8), 0x99999999, np.uint32)
    s = np.full((1, n_out, k_in // 64), _bits([c])[0], np.uint16)
    b = np.full_like(s, _bits([-8 * c])[0])
    return q, s, b


def test_expert_ffn_constant_weight_closed_form():
    H, F = 128, 64
    cg, cu, cd = 0.015625, 0.0078125, 0.03125            # bf16-exact constants
    x = np.array([[1.0] * 64 + [-0.5] * 64, [2.0] * 128])
    wg = O.dequant(*[a[0] for a in _const_proj(F, H, cg)])
    wu = O.dequant(*[a[0] for a in _const_proj(F, H, cu)])
    wd = O.dequant(*[a[0] for a in _const_proj(H, F, cd)])
    y = O.expert_ffn(x, wg, wu, wd)
    for t in range(2):
        sx = float(x[t].sum())
        g, u = cg * sx, cu * sx
        a = g / (1 + math.exp(-g)) * u
        assert np.allclose(y[t], F * cd * a, rtol=1e-14, atol=0)


def _rne_bf16_via_f32_bits(v: float) -> float:
    """Nearest bf16 of a value that fp32 holds exactly, by integer rounding of its fp32 bits
    (ties to even): an implementation independent of the oracle's frexp-based rounding."""
    b = int(np.array([v], np.float32).view(np.uint32)[0])
    assert float(np.array([b], np.uint32).view(np.float32)[0]) == v
    r = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16) << 16
    return float(np.array([r], np.uint32).view(np.float32)[0])


def test_expert_ffn_bf16_profile_closed_form():
    """bf16 profile: the SwiGLU output A, the input of the down projection's tensor operation,
    is rounded to bf16, and the expert output is not ([P1 "The Model ..."]: weights rebuilt
    into bf16 for the tensor operations, fp32 accumulation; nothing is said of the outputs).
    Constant weights give y = F*cd*bf16(a) exactly; F*cd = 1.5 makes that value need nine
    significant bits for at least one token, so a stray rounding of the output (to bf16) would
    change it, and a missing rounding of A would leave y = F*cd*a instead."""
    H, F = 128, 64
    cg, cu, cd = 0.015625, 0.0078125, 0.0234375          # bf16-exact constants, F*cd = 1.5
    x = np.array([[1.0] * 64 + [-0.5] * 64, [2.0] * 128, [0.75] * 128])
    wg = O.dequant(*[a[0] for a in _const_proj(F, H, cg)], "bf16")
    wu = O.dequant(*[a[0] for a in _const_proj(F, H, cu)], "bf16")
    wd = O.dequant(*[a[0] for a in _const_proj(H, F, cd)], "bf16")
    y = O.expert_ffn(x, wg, wu, wd, "bf16")
    y_exact = O.expert_ffn(x, wg, wu, wd)
    needs_nine_bits = False
    a_rounded = False
    for t in range(x.shape[0]):
        sx = float(x[t].sum())
        g, u = cg * sx, cu * sx
        a64 = g / (1 + math.exp(-g)) * u
        a_b = _rne_bf16_via_f32_bits(float(np.float32(a64)))
        # going through fp32 first decides the same bf16 as rounding a64 directly unless a64
        # lies within one fp32 step of a bf16 midpoint
        ulp_bf16 = 2.0 ** (math.frexp(a_b)[1] - 8)
        mid = a_b + math.copysign(ulp_bf16 / 2, a64 - a_b)
        assert abs(a64 - mid) > 2.0 ** (math.frexp(a64)[1] - 23)
        want = F * cd * a_b                                  # exact in fp64, not rounded
        assert np.all(y[t] == want), (t, y[t][:2], want)
        needs_nine_bits |= _rne_bf16_via_f32_bits(want) != want
        a_rounded |= a_b != a64
        assert np.allclose(y[t], y_exact[t], rtol=2.0 ** -8, atol=0)
    assert needs_nine_bits and a_rounded


def _tiny_layer_with(routed_zero=False, identical=False, seed=0):
    shape = synth.SHAPES["tiny"]
    L = synth.make_layer(shape, seed=seed)
    if routed_zero:
        for name in ("gate", "up", "down"):
            q, s, b = L[name]
            L[name] = (q, np.zeros_like(s), np.zeros_like(b))
    if identical:
        for name in ("gate", "up", "down"):
            q, s, b = L[name]
            L[name] = (np.repeat(q[:1], q.shape[0], 0), np.repeat(s[:1], s.shape[0], 0),
                       np.repeat(b[:1], b.shape[0], 0))
    return shape, L


def test_layer_zero_routed_weights_returns_shared_term_only():
    shape, L = _tiny_layer_with(routed_zero=True)
    x = synth.make_tokens(shape, 5, seed=2)
    y = O.layer_forward(L, x, shape.K)
    xf = O.bf16_to_f64(x)
    sg = 1 / (1 + np.exp(-(xf @ L["shared_gate_w"].astype(np.float64))))
    ws = [O.dequant(*[a[0] for a in L[n]]) for n in ("sh_gate", "sh_up", "sh_down")]
    a = (xf @ ws[0].T) / (1 + np.exp(-(xf @ ws[0].T))) * (xf @ ws[1].T)
    assert np.allclose(y, sg[:, None] * (a @ ws[2].T), rtol=1e-12, atol=1e-12)
    L["sh_gate"] = L["sh_up"] = L["sh_down"] = None    # no shared expert -> exactly zero
    assert np.all(O.layer_forward(L, x, shape.K) == 0.0)


def test_layer_identical_experts_routing_invariant():
    shape, L = _tiny_layer_with(identical=True)
    x = synth.make_tokens(shape, 7, seed=3)
    y = O.layer_forward(L, x, shape.K)
    L2 = dict(L)
    L2["router_w"] = np.random.default_rng(9).normal(0, 1, L["router_w"].shape).astype(np.float32)
    y2 = O.layer_forward(L2, x, shape.K)               # any routing gives the same output
    assert np.allclose(y, y2, rtol=1e-12, atol=1e-12)


def test_layer_constant_weights_closed_form():
    """Every weight constant: each expert's FFN is known in closed form, so the whole layer is."""
    H, E, K, F, Fs = 128, 4, 2, 64, 64
    L = {"router_w": np.zeros((E, H), np.float32), "router_bias": np.array([0, 1, 2, 3], np.float32),
         "shared_gate_w": np.zeros(H, np.float32)}
    cs = [0.015625, 0.0078125, 0.03125, 0.0625]
    for name, n_out, k_in in (("gate", F, H), ("up", F, H), ("down", H, F)):
        parts = [_const_proj(n_out, k_in, c) for c in cs]
        L[name] = tuple(np.concatenate([p[i] for p in parts]) for i in range(3))
    L["sh_gate"], L["sh_up"], L["sh_down"] = (_const_proj(Fs, H, 0.03125), _const_proj(Fs, H, 0.03125),
                                              _const_proj(H, Fs, 0.0078125))
    x = _bits([[0.25] * H, [-0.5] * 64 + [1.0] * 64])
    y = O.layer_forward(L, x, K)
    for t in range(2):
        sx = float(O.bf16_to_f64(x[t]).sum())
        # logits are the bias (router weights are zero): experts 3 then 2, p = e^3/(e^3+e^2), ...
        p3 = math.exp(3) / (math.exp(3) + math.exp(2))
        want = 0.0
        for e, p in ((3, p3), (2, 1 - p3)):
            g = u = cs[e] * sx
            want += p * F * cs[e] * (g / (1 + math.exp(-g)) * u)
        g = u = 0.03125 * sx
        want += 0.5 * Fs * 0.0078125 * (g / (1 + math.exp(-g)) * u)
        assert np.allclose(y[t], want, rtol=1e-13, atol=0)


def _brute_force_layer(L, x_bits, K):
    """Scalar Python reference for tiny layers: integer bit decoding, explicit loops."""
    def bf(bits):
        return float(_bf16_exact(int(bits)))

    def wval(proj, e, n, i):
        q, s, b = proj
        nib = (int(q[e, n, i // 8]) >> (4 * (i % 8))) & 0xF
        return bf(s[e, n, i // 64]) * nib + bf(b[e, n, i // 64])

    def ffn(proj3, e, x):
        g, u, d = proj3
        F, H = g[0].shape[1], len(x)
        a = []
        for f in range(F):
            gf = sum(x[i] * wval(g, e, f, i) for i in range(H))
            uf = sum(x[i] * wval(u, e, f, i) for i in range(H))
            a.append(gf / (1 + math.exp(-gf)) * uf)
        return [sum(a[f] * wval(d, e, h, f) for f in range(F)) for h in range(H)]

    E, H = L["router_w"].shape
    out = []
    for t in range(x_bits.shape[0]):
        x = [bf(v) for v in x_bits[t]]
        l = [sum(x[i] * float(L["router_w"][e, i]) for i in range(H)) for e in range(E)]
        sel = sorted(range(E), key=lambda e: (-l[e], e))[:K]
        den = sum(math.exp(l[e] - l[sel[0]]) for e in sel)
        y = [0.0] * H
        for e in sel:
            pe = math.exp(l[e] - l[sel[0]]) / den
            fe = ffn((L["gate"], L["up"], L["down"]), e, x)
            y = [a + pe * b for a, b in zip(y, fe)]
        gl = sum(x[i] * float(L["shared_gate_w"][i]) for i in range(H))
        fs = ffn((L["sh_gate"], L["sh_up"], L["sh_down"]), 0, x)
        y = [a + b / (1 + math.exp(-gl)) for a, b in zip(y, fs)]
        out.append(y)
    return np.array(out)


def test_layer_matches_scalar_brute_force():
    shape = synth.LayerShape(64, 6, 2, 64, 64)
    L = synth.make_layer(shape, seed=11)
    x = synth.make_tokens(shape, 2, seed=11)
    want = _brute_force_layer(L, x, shape.K)
    got = O.layer_forward(L, x, shape.K)
    assert np.allclose(got, want, rtol=1e-11, atol=1e-11)


def test_layer_grouped_equals_per_token_loop():
    shape = synth.SHAPES["tiny"]
    L = synth.make_layer(shape, seed=0)
    x = synth.make_tokens(shape, 4, seed=0)
    for prof in O.PROFILES:
        a = O.layer_forward(L, x, shape.K, prof)
        b = O.layer_forward_per_token(L, x, shape.K, prof)
        assert np.allclose(a, b, rtol=1e-12, atol=1e-12)


def test_layer_token_independence_and_order():
    shape = synth.SHAPES["mid"]
    L = synth.make_layer(shape, seed=4)
    x = synth.make_tokens(shape, 24, seed=4)
    y = O.layer_forward(L, x, shape.K, "bf16")
    perm = np.random.default_rng(0).permutation(24)
    assert np.allclose(O.layer_forward(L, x[perm], shape.K, "bf16"), y[perm], rtol=1e-12, atol=1e-12)
    sub = np.array([3, 17, 5])
    assert np.allclose(O.layer_forward(L, x, shape.K, "bf16", tokens=sub), y[sub], rtol=1e-12, atol=1e-12)


def test_layer_scales_linearly_with_down_weights():
    shape = synth.SHAPES["tiny"]
    L = synth.make_layer(shape, seed=5)
    x = synth.make_tokens(shape, 3, seed=5)
    y = O.layer_forward(L, x, shape.K)
    L2 = dict(L)
    for name in ("down", "sh_down"):                   # s, b -> 2s, 2b (exact: exponent + 1)
        q, s, b = L[name]
        L2[name] = (q, s + np.uint16(1 << 7), b + np.uint16(1 << 7))
    assert np.allclose(O.layer_forward(L2, x, shape.K), 2 * y, rtol=1e-13, atol=1e-13)


def test_bf16_profile_close_to_exact_and_forced_routing():
    shape = synth.SHAPES["tiny"]
    L = synth.make_layer(shape, seed=0)
    x = synth.make_tokens(shape, 4, seed=0)
    ye = O.layer_forward(L, x, shape.K, "exact")
    yb = O.layer_forward(L, x, shape.K, "bf16")
    st = O.error_stats(yb, ye)
    assert 0 < st["max_rel"] < 2e-2
    # forcing the routing the oracle itself picks changes nothing
    idx, _ = O.select_topk(O.router_logits(x, L["router_w"], L["router_bias"]), shape.K)
    assert np.array_equal(O.layer_forward(L, x, shape.K, "bf16", topk_idx=idx), yb)


def test_rms_norm_and_error_stats():
    r = np.array([[3.0, 4.0], [2.0, 2.0]])
    n = O.rms_norm(r, eps=0.0)
    assert np.allclose(n[0], [3 / math.sqrt(12.5), 4 / math.sqrt(12.5)], rtol=1e-15)
    assert np.allclose(n[1], [1.0, 1.0], rtol=1e-15)
    st = O.error_stats(np.array([[1.0, 2.0], [0.0, 4.5]]), np.array([[1.0, 2.5], [0.0, 4.0]]))
    assert st["max_rel"] == pytest.approx(0.2) and st["mean_abs"] == pytest.approx(0.25)


def test_generator_recipe():
    shape = synth.SHAPES["full"]
    L = synth.make_layer(shape, seed=0)
    q, s, b = L["gate"]
    sv, bv = O.bf16_to_f64(s), O.bf16_to_f64(b)
    assert np.all(bv == -8 * sv) and sv.min() >= 0.00498 and sv.max() <= 0.02005
    nib = O.unpack_nibbles(q[0, :64])
    assert abs(nib.mean() - 7.5) < 0.05 and nib.min() == 0 and nib.max() == 15
    assert abs(L["router_w"].std() - 0.02) < 2e-4
    x = O.bf16_to_f64(synth.make_tokens(shape, 64))
    assert abs(x.std() - 1.0) < 0.02
    # per-tensor streams: one expert regenerates alone and identically
    L1 = synth.make_layer(synth.SHAPES["full"], seed=0)
    assert np.array_equal(L1["down"][0][17], L["down"][0][17])
    skew = synth.make_layer(synth.SHAPES["full_skew"], seed=0)["router_bias"]
    assert np.allclose(skew, -1.2 * np.log(np.arange(1, 257)), rtol=1e-6)


# ------------------------------------------------------------------ stack glue
def test_residual_rmsnorm_closed_forms():
    # y = -r: the stream cancels and the normalised input is exactly zero (eps > 0)
    r = np.array([[1.5, -2.0, 0.25, 8.0]])
    r2, x = O.residual_rmsnorm(r, -r)
    assert np.all(r2 == 0) and np.all(x == 0)
    # a constant row c: x = c / sqrt(c^2 + eps), rounded to bf16 (hand value for c = 3)
    c = 3.0
    _, x = O.residual_rmsnorm(np.full((1, 64), c), None, eps=1e-6)
    want = c / math.sqrt(c * c + 1e-6)            # 0.99999994..., rounds to 1.0 in bf16
    assert np.all(O.bf16_to_f64(x) == 1.0) and abs(want - 1.0) < 2 ** -9
    # with eps = 0 a power-of-two scaling of the row changes nothing at all
    rng = np.random.default_rng(3)
    row = rng.standard_normal((2, 128))
    _, xa = O.residual_rmsnorm(row, None, eps=0.0)
    _, xb = O.residual_rmsnorm(row * 1024.0, None, eps=0.0)
    assert np.array_equal(xa, xb)
    # mean of squares of the normalised row is 1 before rounding (eps = 0)
    assert abs(np.mean(O.rms_norm(row, 0.0) ** 2) - 1.0) < 1e-12


def test_bf16_bits_round_trip():
    bits = _all_finite_bf16()
    assert np.array_equal(O.bf16_bits(O.bf16_to_f64(bits)), bits)
    with pytest.raises(AssertionError):
        O.bf16_bits(np.array([1.0 + 2 ** -10]))


def test_stack_of_zero_layers_keeps_the_stream():
    """Layers whose routed and shared weights are all zero output zero, so the residual stream
    stays the input exactly and the final input is the normalised tokens."""
    shape = synth.LayerShape(128, 4, 2, 64, 64)
    layer = synth.make_layer(shape, seed=5)
    for name in ("gate", "up", "down", "sh_gate", "sh_up", "sh_down"):
        q, sc, b = layer[name]
        layer[name] = (q, np.zeros_like(sc), np.zeros_like(b))
    x = synth.make_tokens(shape, 3, seed=5)
    r, xl = O.stack_forward([layer, layer], x, shape.K)
    assert np.array_equal(r, O.bf16_to_f64(x))
    # the hand-computed normalisation of token 0
    row = O.bf16_to_f64(x[0])
    want = O.round_to_bf16(row / math.sqrt(float(np.mean(row * row)) + 1e-6))
    assert np.array_equal(O.bf16_to_f64(xl[0]), want)
