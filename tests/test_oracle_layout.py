"""Pins of the pre-layout index maps: exact inverses, byte permutations, and
agreement with the per-element offset formulas evaluated one byte at a time."""
import numpy as np

from oracle import layout


def test_fp8_block_layout_roundtrip_and_formula():
    g = np.random.default_rng(30)
    N, K = 48, 384
    w = g.integers(0, 256, (N, K), dtype=np.uint8)
    pre = layout.prelayout_fp8_block(w)
    assert pre.size == N * K
    assert np.array_equal(layout.unprelayout_fp8_block(pre, N, K), w)
    assert np.array_equal(np.sort(pre), np.sort(w.reshape(-1)))
    KS = K // 128
    for n in range(N):
        for k in range(K):
            nt, ks, kk = n // 16, k // 128, k % 128
            lane = n % 16 + 16 * (kk // 32)
            off = ((nt * KS + ks) * 2 + (kk % 32) // 16) * 1024 + lane * 16 + kk % 16
            assert pre[off] == w[n, k]


def test_mxfp4_layout_roundtrip_and_formula():
    g = np.random.default_rng(31)
    for N, K in [(32, 640), (16, 512), (48, 128)]:
        wp = g.integers(0, 256, (N, K // 2), dtype=np.uint8)
        e = g.integers(0, 256, (N, K // 32), dtype=np.uint8)
        pc = layout.prelayout_mxfp4_codes(wp)
        ps = layout.prelayout_mxfp4_scales(e)
        assert pc.size == N * K // 2 and ps.size == layout.mxfp4_scale_bytes(N, K)
        assert np.array_equal(layout.unprelayout_mxfp4_codes(pc, N, K), wp)
        assert np.array_equal(layout.unprelayout_mxfp4_scales(ps, N, K), e)
        KS = K // 128
        KQ = (KS + 3) // 4
        for n in range(N):
            for p in range(K // 2):
                kk = (2 * p) % 128
                lane = n % 16 + 16 * (kk // 32)
                off = ((n // 16) * KS + (2 * p) // 128) * 1024 + lane * 16 + (kk % 32) // 2
                assert pc[off] == wp[n, p]
            for k32 in range(K // 32):
                ks = k32 // 4
                lane = n % 16 + 16 * (k32 % 4)
                off = (((n // 16) * KQ + ks // 4) * 64 + lane) * 4 + ks % 4
                assert ps[off] == e[n, k32]
        # padding bytes of a partly used scale dword
        used = np.zeros(ps.size, bool)
        for n in range(N):
            for k32 in range(K // 32):
                ks = k32 // 4
                used[(((n // 16) * KQ + ks // 4) * 64 + n % 16 + 16 * (k32 % 4)) * 4 + ks % 4] = True
        assert np.all(ps[~used] == layout.E8M0_PAD)
