"""Pins of the oracle's GEMM definitions: exact rational brute force on tiny
shapes (spanning several scale groups and N blocks so a wrong scale index or a
transposed operand shows), one-hot weights, integer-valued cases and the
e2m1 x e8m0 sweep whose results are exact powers-of-two multiples of the
page's table."""
from fractions import Fraction

import numpy as np

from oracle import gemm, codecs, checks
from tests import exact


def _fp8_brute(a, asc, w, wsc):
    M, K = a.shape
    N = w.shape[0]
    A = np.array(exact.e4m3_values(a), dtype=object).reshape(M, K)
    W = np.array(exact.e4m3_values(w), dtype=object).reshape(N, K)
    out = np.empty((M, N), dtype=object)
    for m in range(M):
        for n in range(N):
            tot = Fraction(0)
            for g in range(K // 128):
                part = sum((A[m, k] * W[n, k] for k in range(128 * g, 128 * g + 128)), Fraction(0))
                tot += Fraction(float(asc[m, g])) * Fraction(float(wsc[n // 128, g])) * part
            out[m, n] = tot
    return out


def test_fp8_block_brute_force():
    g = np.random.default_rng(10)
    M, N, K = 2, 256, 256
    a = g.integers(0, 256, (M, K), dtype=np.uint8)
    w = g.integers(0, 256, (N, K), dtype=np.uint8)
    a[(a & 0x7F) == 0x7F] = 0x3C          # no NaN codes
    w[(w & 0x7F) == 0x7F] = 0x41
    asc = g.uniform(0.01, 2, (M, K // 128)).astype(np.float32)
    wsc = g.uniform(0.001, 0.1, (N // 128, K // 128)).astype(np.float32)
    c_bits, c_exact, abs_sum = gemm.fp8_block_gemm(a, asc, w, wsc)
    brute = _fp8_brute(a, asc, w, wsc)
    for m in range(M):
        for n in range(N):
            want = exact.bf16_round(brute[m, n])
            assert Fraction(float(codecs.decode_bf16(c_bits[m, n]))) == want, (m, n)
            # fp64 rounding of the scale products and group sums only: far below the bf16 quantum
            assert abs(Fraction(float(c_exact[m, n])) - brute[m, n]) <= Fraction(float(abs_sum[m, n])) * Fraction(1, 2 ** 48)
    # the single-element form agrees with the full form
    rows = np.array([0, 1, 1, 0])
    cols = np.array([0, 127, 128, 255])
    cb, ce, asum = gemm.fp8_block_gemm_at(a, asc, w, wsc, rows, cols)
    assert np.array_equal(cb, c_bits[rows, cols])
    assert np.allclose(asum, abs_sum[rows, cols], rtol=1e-12)


def test_fp8_block_one_hot_weight():
    g = np.random.default_rng(11)
    M, N, K = 5, 256, 384
    a = g.integers(0, 0x7F, (M, K), dtype=np.uint8) | (g.integers(0, 2, (M, K), dtype=np.uint8) << 7)
    perm = g.permutation(K)[:N]
    w = np.zeros((N, K), np.uint8)
    w[np.arange(N), perm] = 0x38                    # e4m3 1.0
    asc = np.ones((M, K // 128), np.float32)
    wsc = np.ones((N // 128, K // 128), np.float32)
    c_bits, _, _ = gemm.fp8_block_gemm(a, asc, w, wsc)
    vals = exact.e4m3_values(a[:, perm])
    want = [exact.fraction_to_bf16_bits(v) for v in vals]   # e4m3 values are exact in bf16
    assert c_bits.reshape(-1).tolist() == want


def test_fp8_block_integer_valued():
    g = np.random.default_rng(12)
    M, N, K = 3, 128, 256
    ints = np.array([0x00, 0x38, 0x40, 0x44, 0x48, 0x4A, 0x4C, 0x4E, 0xB8, 0xC0], np.uint8)  # 0,1,2,3,4,5,6,7,-1,-2
    ival = np.array([0, 1, 2, 3, 4, 5, 6, 7, -1, -2])
    ia = g.integers(0, len(ints), (M, K))
    iw = g.integers(0, len(ints), (N, K))
    c_bits, c_exact, _ = gemm.fp8_block_gemm(ints[ia], np.ones((M, 2), np.float32), ints[iw],
                                             np.ones((1, 2), np.float32))
    want = ival[ia] @ ival[iw].T
    assert np.array_equal(c_exact, want.astype(np.float64))


def _fp4_value(code, lut):
    return Fraction(lut[code & 15]).limit_denominator(2)


def test_w4a8_brute_force(golden):
    lut = golden["e2m1_lut"]["value"]
    g = np.random.default_rng(13)
    M, N, K = 2, 16, 256
    a = g.integers(0, 256, (M, K), dtype=np.uint8)
    a[(a & 0x7F) == 0x7F] = 0x30
    wp = g.integers(0, 256, (N, K // 2), dtype=np.uint8)
    e = g.integers(117, 131, (N, K // 32), dtype=np.uint8)
    asc = g.uniform(0.001, 0.02, M).astype(np.float32)
    c_bits, c_exact, _ = gemm.w4a8_mxfp4_gemm(a, asc, wp, e)
    A = np.array(exact.e4m3_values(a), dtype=object).reshape(M, K)
    for m in range(M):
        for n in range(N):
            tot = Fraction(0)
            for k in range(K):
                byte = int(wp[n, k // 2])
                code = byte & 15 if k % 2 == 0 else byte >> 4
                tot += A[m, k] * _fp4_value(code, lut) * exact.e8m0_value(e[n, k // 32])
            tot *= Fraction(float(asc[m]))
            assert Fraction(float(codecs.decode_bf16(c_bits[m, n]))) == exact.bf16_round(tot), (m, n)
    rows = np.array([0, 1])
    cols = np.array([15, 3])
    cb, _, _ = gemm.w4a8_mxfp4_gemm_at(a, asc, wp, e, rows, cols)
    assert np.array_equal(cb, c_bits[rows, cols])


def test_w4a8_code_scale_sweep(golden):
    """Every e2m1 code x e8m0 in 100..154 against A = 1.0: C is that table value
    times a power of two, exact in bf16."""
    lut = golden["e2m1_lut"]["value"]
    exps = np.arange(100, 155, dtype=np.uint8)
    N = 16 * len(exps)
    K = 128
    wp = np.zeros((N, K // 2), np.uint8)
    e = np.full((N, K // 32), 127, np.uint8)
    for i, ex in enumerate(exps):
        for c in range(16):
            n = i * 16 + c
            wp[n, 0] = c                 # element k=0 (low nibble)
            e[n, 0] = ex
    a = np.zeros((1, K), np.uint8)
    a[0, 0] = 0x38
    c_bits, _, _ = gemm.w4a8_mxfp4_gemm(a, np.ones(1, np.float32), wp, e)
    for i, ex in enumerate(exps):
        for c in range(16):
            want = Fraction(lut[c]).limit_denominator(2) * exact.e8m0_value(ex)
            got = codecs.decode_bf16(c_bits[0, i * 16 + c])
            assert Fraction(float(got)) == want
    # high nibble carries element k=1
    wp2 = np.zeros((16, K // 2), np.uint8)
    wp2[:, 0] = np.arange(16, dtype=np.uint8) << 4
    a2 = np.zeros((1, K), np.uint8)
    a2[0, 1] = 0x38
    c2, _, _ = gemm.w4a8_mxfp4_gemm(a2, np.ones(1, np.float32), wp2, np.full((16, 4), 127, np.uint8))
    assert codecs.decode_bf16(c2[0]).tolist() == lut


def test_bf16_gemm_brute_force_and_one_hot():
    g = np.random.default_rng(14)
    M, N, K = 3, 5, 64
    x = (g.standard_normal((M, K)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    w = (g.standard_normal((N, K)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    c_bits, _, _ = gemm.bf16_gemm(x, w)
    X = np.array(exact.bf16_values(x), dtype=object).reshape(M, K)
    W = np.array(exact.bf16_values(w), dtype=object).reshape(N, K)
    for m in range(M):
        for n in range(N):
            want = exact.bf16_round(sum((X[m, k] * W[n, k] for k in range(K)), Fraction(0)))
            assert Fraction(float(codecs.decode_bf16(c_bits[m, n]))) == want
    perm = g.permutation(K)[:N]
    onehot = np.zeros((N, K), np.uint16)
    onehot[np.arange(N), perm] = 0x3F80          # bf16 1.0
    c1, _, _ = gemm.bf16_gemm(x, onehot)
    assert np.array_equal(c1, x[:, perm])


def test_tolerance_check_accepts_and_rejects():
    c_exact = np.array([1.0, 100.0, -3.0])
    abs_sum = np.array([1.0, 100.0, 3.0])
    good = codecs.round_to_bf16(c_exact)
    bad, _ = checks.gemm_violations(good, c_exact, abs_sum)
    assert not bad.any()
    worse = codecs.round_to_bf16(c_exact * (1 + 2.0 ** -5))
    bad, _ = checks.gemm_violations(worse, c_exact, abs_sum)
    assert bad.all()
