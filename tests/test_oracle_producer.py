"""Pins of the producer and quantizer oracles: exact rational / high-precision
decimal brute force on small rows, closed-form rows (constant, one-hot, zero,
w = -1 columns), the per-row invariants and the dequantization error bound."""
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np

from oracle import producer, quant, codecs
from tests import exact

FP8_MAX = 448.0


def _bf16_bits(vals):
    import torch
    return torch.tensor(vals, dtype=torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_residual_add_brute_force():
    g = np.random.default_rng(20)
    y = (g.standard_normal((4, 64)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    r = (g.standard_normal((4, 64)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    # adversarial ties: 1 + 2**-8 (tie -> 1), (1 + 2**-7) + 2**-8 (tie -> 1 + 2**-6)
    y[0, :2] = _bf16_bits([1.0, 1.0 + 2.0 ** -7])
    r[0, :2] = _bf16_bits([2.0 ** -8, 2.0 ** -8])
    w = np.zeros(64, np.uint16)
    _, _, r_bits = producer.add_rms_quant(y, r, w)
    Y = exact.bf16_values(y)
    R = exact.bf16_values(r)
    want = [exact.fraction_to_bf16_bits(exact.bf16_round(a + b)) for a, b in zip(Y, R)]
    assert r_bits.reshape(-1).tolist() == want
    assert codecs.decode_bf16(r_bits[0, :2]).tolist() == [1.0, 1.0 + 2.0 ** -6]


def exact_fp32(f):
    """Fraction -> nearest fp32 value as a Fraction (RNE), by comparing the
    two fp32 neighbours of the fp64 approximation."""
    x = np.float32(float(f))
    cands = [np.nextafter(x, np.float32(-np.inf)), x, np.nextafter(x, np.float32(np.inf))]
    best = min(cands, key=lambda c: (abs(Fraction(float(c)) - f), int(np.array(c).view(np.uint32)) & 1))
    return Fraction(float(best))


def _decimal_producer_row(y, r, w, eps):
    """High-precision reference of one row: returns (h list of Decimals, amax)."""
    getcontext().prec = 60
    Y = [Decimal(Fraction(v).numerator) / Decimal(Fraction(v).denominator) for v in exact.bf16_values(y)]
    R = [Decimal(Fraction(v).numerator) / Decimal(Fraction(v).denominator) for v in exact.bf16_values(r)]
    Wt = [Decimal(Fraction(v).numerator) / Decimal(Fraction(v).denominator) for v in exact.bf16_values(w)]
    rr = []
    for a, b in zip(Y, R):
        f = exact.bf16_round(Fraction(a) + Fraction(b))
        rr.append(Decimal(f.numerator) / Decimal(f.denominator))
    ms = sum(x * x for x in rr) / len(rr)
    inv = 1 / (ms + Decimal(eps)).sqrt()
    h = [x * inv * (1 + wk) for x, wk in zip(rr, Wt)]
    return h, max(abs(x) for x in h)


def test_producer_decimal_brute_force():
    g = np.random.default_rng(21)
    M, K = 6, 96
    y = (g.standard_normal((M, K)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    r = (g.standard_normal((M, K)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    w = ((g.standard_normal(K) * 0.1).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    y[5] = _bf16_bits(list(g.standard_normal(K) * 1e-5))      # ms << eps: eps matters
    q, s, _, h = producer.add_rms_quant(y, r, w, eps=1e-6, return_h=True)
    for m in range(M):
        hd, amax = _decimal_producer_row(y[m], r[m], w, 1e-6)
        hm = np.array([float(x) for x in hd])
        assert np.allclose(h[m], hm, rtol=1e-13, atol=0)
        # scale: amax of the fp32-rounded h, then the exact quotient rounded once to fp32
        amax32 = Fraction(float(np.float32(float(amax))))
        s_want = max(amax32 / 448, Fraction(1, 448 * 512))
        assert Fraction(float(s[m])) == exact_fp32(s_want)
        # codes: e4m3 of fp32(fp32(h)/s) with the clamp; compare away from rounding midpoints
        v = (hm.astype(np.float32) / np.float32(s[m])).astype(np.float64)
        v = np.clip(v, -FP8_MAX, FP8_MAX)
        for k in range(K):
            want = exact.e4m3_round(Fraction(float(v[k])))
            assert Fraction(float(codecs.decode_e4m3(q[m, k]))) == want


def test_producer_closed_form_rows():
    K = 256
    c = 0.75
    y = np.tile(_bf16_bits([c]), (1, K))
    zeros = np.zeros((1, K), np.uint16)
    w0 = np.zeros(K, np.uint16)
    q, s, r = producer.add_rms_quant(y, zeros, w0)
    assert np.all(q == 0x7E)                                   # every |h| equals the max
    h = c / np.sqrt(c * c + 1e-6)
    assert float(s[0]) == float(np.float32(h / 448.0))
    # negative constant
    q, s, _ = producer.add_rms_quant(np.tile(_bf16_bits([-c]), (1, K)), zeros, w0)
    assert np.all(q == 0xFE)
    # one-hot row
    y1 = np.zeros((1, K), np.uint16)
    y1[0, 17] = _bf16_bits([-3.0])[0]
    q, s, _ = producer.add_rms_quant(y1, zeros, w0)
    assert q[0, 17] == 0xFE and np.all(np.delete(q[0], 17) == 0)
    # all-zero row: min scale, zero codes
    q, s, r = producer.add_rms_quant(zeros, zeros, w0)
    assert np.all(q == 0) and float(s[0]) == float(np.float32(1.0 / (448 * 512)))
    # Gemma offset: w = -1 zeroes the column, w = 0 is the plain RMSNorm
    g = np.random.default_rng(22)
    yr = (g.standard_normal((3, K)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    wm = np.zeros(K, np.uint16)
    wm[::7] = _bf16_bits([-1.0])[0]
    q, s, r, h = producer.add_rms_quant(yr, np.zeros_like(yr), wm, return_h=True)
    assert np.all(h[:, ::7] == 0) and np.all((q[:, ::7] & 0x7F) == 0)
    rv = codecs.decode_bf16(r)
    plain = rv / np.sqrt(np.mean(rv * rv, axis=1, keepdims=True) + 1e-6)
    mask = np.ones(K, bool)
    mask[::7] = False
    assert np.allclose(h[:, mask], plain[:, mask], rtol=1e-14)


def test_producer_invariants_and_dequant_bound():
    g = np.random.default_rng(23)
    M, K = 32, 5120
    y = (g.standard_normal((M, K)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    r = (g.standard_normal((M, K)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    w = ((g.standard_normal(K) * 0.1).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    q, s, _, h = producer.add_rms_quant(y, r, w, return_h=True)
    assert np.all(np.any((q & 0x7F) == 0x7E, axis=1))          # every row reaches the max code
    deq = codecs.decode_e4m3(q) * s.astype(np.float64)[:, None]
    v = np.abs(h) / s.astype(np.float64)[:, None]
    e = np.maximum(np.floor(np.log2(np.maximum(v, 2.0 ** -6))), -6)
    half_ulp = np.exp2(e - 3) / 2
    slack = 1e-6 * np.abs(h) / s.astype(np.float64)[:, None]    # fp32 rounding of h and h/s
    assert np.all(np.abs(deq - h) / s.astype(np.float64)[:, None] <= half_ulp + slack)


def test_quant_per_token_and_group_fixtures():
    g = np.random.default_rng(24)
    x = (g.standard_normal((4, 512)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    q, s = quant.quant_per_token_bf16(x)
    xv = codecs.decode_bf16(x)
    for m in range(4):
        amax = Fraction(float(np.abs(xv[m]).max()))
        assert float(s[m]) == float(np.float32(float(amax / 448)))
        assert (q[m] & 0x7F).max() == 0x7E
    qg, sg = quant.quant_group128_bf16(x)
    assert sg.shape == (4, 4)
    for gi in range(4):
        blk = xv[:, gi * 128:(gi + 1) * 128]
        assert np.array_equal(sg[:, gi], (np.abs(blk).max(axis=1) / 448).astype(np.float32))
        assert np.all((qg[:, gi * 128:(gi + 1) * 128] & 0x7F).max(axis=1) == 0x7E)
    wq, ws = quant.quant_block128_bf16(np.tile(x, (64, 1)))       # [256, 512]
    assert ws.shape == (2, 4)
    # tiny row: the minimum scale clamp
    tiny = _bf16_bits([1e-7] * 128).reshape(1, 128)
    qt, st = quant.quant_per_token_bf16(tiny)
    assert float(st[0]) == float(np.float32(1.0 / (448 * 512)))
    assert np.all(codecs.decode_e4m3(qt) * float(st[0]) <= 2e-7)


# ----------------------------------------------------------------- silu_mul_quant
def _decimal_silu_row(g_bits, u_bits):
    """SiLU(gate) * up at 60 digits with Decimal's own exp: an evaluation that
    shares nothing with numpy's exp."""
    getcontext().prec = 60
    G = [Decimal(Fraction(v).numerator) / Decimal(Fraction(v).denominator) for v in exact.bf16_values(g_bits)]
    U = [Decimal(Fraction(v).numerator) / Decimal(Fraction(v).denominator) for v in exact.bf16_values(u_bits)]
    return [gk / (1 + (-gk).exp()) * uk for gk, uk in zip(G, U)]


def test_silu_mul_quant_decimal_brute_force():
    g = np.random.default_rng(25)
    M, N = 5, 64
    gu = (g.standard_normal((M, 2 * N)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    gu[1, :8] = _bf16_bits([0.0, -0.0, 30.0, -30.0, 88.0, -88.0, 120.0, -120.0])
    gu[2, :N] = _bf16_bits(list(g.standard_normal(N) * 8.0))   # saturated and vanishing SiLU
    gu[4, N:] = _bf16_bits(list(g.standard_normal(N) * 1e-4))  # small up: tiny row maximum
    q, s, h = producer.silu_mul_quant(gu, return_h=True)
    assert q.shape == (M, N) and s.shape == (M,)
    for m in range(M):
        hd = _decimal_silu_row(gu[m, :N], gu[m, N:])
        hm = np.array([float(x) for x in hd])
        assert np.allclose(h[m], hm, rtol=1e-13, atol=1e-300)
        amax = max(abs(x) for x in hd)
        amax32 = Fraction(float(np.float32(float(amax))))
        s_want = max(amax32 / 448, Fraction(1, 448 * 512))
        assert Fraction(float(s[m])) == exact_fp32(s_want)
        v = (hm.astype(np.float32) / np.float32(s[m])).astype(np.float64)
        v = np.clip(v, -FP8_MAX, FP8_MAX)
        for k in range(N):
            assert Fraction(float(codecs.decode_e4m3(q[m, k]))) == exact.e4m3_round(Fraction(float(v[k])))


def test_silu_mul_quant_closed_forms():
    g = np.random.default_rng(26)
    N = 256
    up = (g.standard_normal((1, N)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    # gate = 30: sigmoid is 1 - 9.4e-14, below half an fp32 ulp, so fp32(h) is exactly 30 * up
    # (an fp32 number: 8 + 5 significant bits); a swapped half would give 30 * SiLU(up) instead
    gate = np.tile(_bf16_bits([30.0]), (1, N))
    q, s, h = producer.silu_mul_quant(np.concatenate([gate, up], axis=1), return_h=True)
    want = 30.0 * codecs.decode_bf16(up)
    assert np.array_equal(h.astype(np.float32), want.astype(np.float32))
    q2, s2 = quant.quant_per_token(want.astype(np.float32))
    assert np.array_equal(q, q2) and np.array_equal(s, s2)
    # gate = 0: SiLU(0) = 0, the minimum scale and zero codes (negative zeros as 0x80 or 0)
    q, s = producer.silu_mul_quant(np.concatenate([np.zeros((1, N), np.uint16), up], axis=1))
    assert np.all((q & 0x7F) == 0) and float(s[0]) == float(np.float32(1.0 / (448 * 512)))
    # up = 1: h is SiLU itself; SiLU(x) - SiLU(-x) = x and SiLU(x) + SiLU(-x) = x * tanh(x / 2)
    x = (g.standard_normal((1, N)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    one = np.tile(_bf16_bits([1.0]), (1, N))
    _, _, hp = producer.silu_mul_quant(np.concatenate([x, one], axis=1), return_h=True)
    _, _, hn = producer.silu_mul_quant(np.concatenate([x ^ np.uint16(0x8000), one], axis=1), return_h=True)
    xv = codecs.decode_bf16(x)
    assert np.allclose(hp - hn, xv, rtol=1e-14, atol=1e-15)
    assert np.allclose(hp + hn, xv * np.tanh(xv / 2), rtol=1e-13, atol=1e-15)
    # the logistic function from scipy: SiLU(x) = x * expit(x)
    from scipy.special import expit
    assert np.allclose(hp, xv * expit(xv), rtol=1e-14, atol=0)
    # large negative gate: SiLU vanishes, the row maximum comes from the other columns
    gate = np.tile(_bf16_bits([-60.0]), (1, N))
    gate[0, 5] = _bf16_bits([2.0])[0]
    q, s, h = producer.silu_mul_quant(np.concatenate([gate, one], axis=1), return_h=True)
    assert q[0, 5] == 0x7E and np.all((np.delete(q[0], 5) & 0x7F) == 0)
    h2 = np.float32(2.0 / (1.0 + float((-Decimal(2)).exp())))
    assert float(s[0]) == float(np.float32(float(h2) / 448.0))       # amax rounded to fp32 first


def test_silu_mul_quant_dequant_bound():
    g = np.random.default_rng(27)
    M, N = 16, 2048
    gu = (g.standard_normal((M, 2 * N)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    q, s, h = producer.silu_mul_quant(gu, return_h=True)
    assert np.all(np.any((q & 0x7F) == 0x7E, axis=1))
    sd = s.astype(np.float64)[:, None]
    deq = codecs.decode_e4m3(q) * sd
    v = np.abs(h) / sd
    e = np.maximum(np.floor(np.log2(np.maximum(v, 2.0 ** -6))), -6)
    half_ulp = np.exp2(e - 3) / 2
    assert np.all(np.abs(deq - h) / sd <= half_ulp + 1e-6 * v)


# ----------------------------------------------------------------- group-scale producer
def test_group_producer_reduces_to_per_token_at_one_group():
    g = np.random.default_rng(28)
    y = (g.standard_normal((5, 128)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    r = (g.standard_normal((5, 128)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    w = ((g.standard_normal(128) * 0.1).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    q1, s1, r1 = producer.add_rms_quant(y, r, w)
    qg, sg, rg = producer.add_rms_quant_group128(y, r, w)
    assert np.array_equal(q1, qg) and np.array_equal(s1, sg[:, 0]) and np.array_equal(r1, rg)


def test_group_producer_decimal_brute_force():
    g = np.random.default_rng(29)
    M, K = 3, 384
    y = (g.standard_normal((M, K)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    r = (g.standard_normal((M, K)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    w = ((g.standard_normal(K) * 0.1).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    y[1, 128:256] = _bf16_bits(list(g.standard_normal(128) * 1e-3))   # a quiet group: its own small scale
    q, s, rb = producer.add_rms_quant_group128(y, r, w)
    _, _, rb1 = producer.add_rms_quant(y, r, w)
    assert np.array_equal(rb, rb1) and s.shape == (M, K // 128)
    for m in range(M):
        hd, _ = _decimal_producer_row(y[m], r[m], w, 1e-6)
        hm = np.array([float(x) for x in hd])
        for gi in range(K // 128):
            blk = hm[gi * 128:(gi + 1) * 128]
            amax32 = Fraction(float(np.float32(float(max(abs(x) for x in hd[gi * 128:(gi + 1) * 128])))))
            assert Fraction(float(s[m, gi])) == exact_fp32(max(amax32 / 448, Fraction(1, 448 * 512)))
            v = np.clip((blk.astype(np.float32) / np.float32(s[m, gi])).astype(np.float64), -FP8_MAX, FP8_MAX)
            for k in range(128):
                assert Fraction(float(codecs.decode_e4m3(q[m, gi * 128 + k]))) == exact.e4m3_round(Fraction(float(v[k])))
            assert (q[m, gi * 128:(gi + 1) * 128] & 0x7F).max() == 0x7E        # every group reaches the top code


def test_group_producer_constant_rows_and_bound():
    K = 512
    y = np.tile(_bf16_bits([0.75]), (1, K))
    y[0, 128:256] = _bf16_bits([-0.5])[0]
    zeros = np.zeros((1, K), np.uint16)
    q, s, _ = producer.add_rms_quant_group128(y, zeros, np.zeros(K, np.uint16))
    assert np.all(q[0, :128] == 0x7E) and np.all(q[0, 128:256] == 0xFE) and np.all(q[0, 256:] == 0x7E)
    assert s[0, 1] < s[0, 0] and s[0, 0] == s[0, 2] == s[0, 3]
    g = np.random.default_rng(30)
    M, K = 8, 1024
    y = (g.standard_normal((M, K)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    r = (g.standard_normal((M, K)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    w = ((g.standard_normal(K) * 0.1).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    q, s, _, h = producer.add_rms_quant_group128(y, r, w, return_h=True)
    sd = np.repeat(s.astype(np.float64), 128, axis=1)
    deq = codecs.decode_e4m3(q) * sd
    v = np.abs(h) / sd
    e = np.maximum(np.floor(np.log2(np.maximum(v, 2.0 ** -6))), -6)
    assert np.all(np.abs(deq - h) / sd <= np.exp2(e - 3) / 2 + 1e-6 * v)
