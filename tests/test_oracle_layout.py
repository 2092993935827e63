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


def test_activation_tiling_roundtrip_and_operand_order():
    """The activation-tiled order against the 32x32x64 MFMA 8-bit operand
    order read lane by lane (row l % 32; bytes 0..15 hold K = 16*(l//32)+b
    and bytes 16..31 K = 32 + 16*(l//32) + b - 16 of each 64-wide half):
    every byte of the tiled buffer is found at the (row, K) that order names."""
    g = np.random.default_rng(32)
    for M, K in [(32, 128), (45, 384), (70, 256)]:
        q = g.integers(0, 256, (M, K), dtype=np.uint8)
        t = layout.tile_activation(q)
        Mp = -(-M // 32) * 32
        assert t.size == layout.tiled_activation_bytes(M, K) == Mp * K
        assert np.array_equal(layout.untile_activation(t, M, K), q)
        KS = K // 128
        for rb in range(Mp // 32):
            for ks in range(KS):
                for h in range(2):
                    base = ((rb * KS + ks) * 2 + h) * 2048
                    for lane in range(64):
                        m = 32 * rb + lane % 32
                        for b in range(32):
                            kk = 16 * (lane // 32) + b if b < 16 else 32 + 16 * (lane // 32) + b - 16
                            want = q[m, 128 * ks + 64 * h + kk] if m < M else 0
                            assert t[base + lane * 32 + b] == want
