"""Weight pre-layout into gfx950 MFMA fragment order: the index maps and inverses.

Test infrastructure (see the package docstring); never used by the product path.

The pages re-lay weights once at load so that the hot loop reads contiguous
bytes, and insist that this is a permutation, not a re-quantisation, with an
exact inverse (radiance_mxfp4.py page, the WPERM comment and
``permute_w`` / ``unpermute_w``; radiance_kernels.py page, ``install_load_hook``).
The order itself here is for gfx950's 16x16x128 8-bit/4-bit MFMA operand:
lane l of a 64-lane wave holds row n = l % 16 of a 16-row tile and the 32
consecutive K values starting at 32*(l // 16) of a 128-wide K step.

Block-FP8 codes (uint8 e4m3 [N, K], N % 16 == 0, K % 128 == 0):
    W[n, k] goes to byte  ((nt*KS + ks)*2 + h)*1024 + lane*16 + j
    with nt = n//16, ks = k//128, kk = k%128, lane = n%16 + 16*(kk//32),
         h = (kk%32)//16, j = kk%16, KS = K/128.
  i.e. each (16-row tile, 128-K step) is 2 KiB: two 1 KiB halves, each half
  one 16-byte load per lane.

MXFP4 codes (uint8 [N, K/2], element 2j = low nibble of byte j):
    packed byte p = W[n, 2j..2j+1] goes to  (nt*KS + ks)*1024 + lane*16 + b
    with k = 2p, ks = k//128, kk = k%128, lane = n%16 + 16*(kk//32),
         b = (kk%32)//2; nibble order inside the byte is kept.
  i.e. 1 KiB per (tile, step), one 16-byte load per lane.

MXFP4 e8m0 scales (uint8 [N, K/32]):
    E[n, k32] goes to  ((nt*KQ + ks//4)*64 + lane)*4 + ks%4
    with ks = k32//4, lane = n%16 + 16*(k32%4), KQ = ceil(KS/4);
  i.e. one dword per lane holds the scales of four consecutive K steps.
  Bytes of a final, partly used dword are 0x7F (scale 1.0, never read).

Activation-tiled producer output (e4m3 codes [M, K], K % 128 == 0): the
A-fragment order of gfx950's 32x32x64 MFMA with an 8-bit operand, whose lane
l holds row l % 32 and, of each 64-wide half of a 128-K step, the K values
16*(l//32) .. +15 in bytes 0..15 and 32 + 16*(l//32) .. +15 in bytes 16..31.
Rows are padded to a multiple of 32:
    A[m, k] goes to byte  ((rb*KS + ks)*2 + h)*2048 + lane*32 + c*16 + j
    with rb = m//32, ks = k//128, h = (k%128)//64, k' = k%64 = 32c + 16g + j,
         lane = m%32 + 32g;
  i.e. each (32-row block, 128-K step) is 4 KiB: two 2 KiB halves, each the
  32 bytes of every lane of one MFMA operand (radiance_mxfp4.py page, the
  A_TILED_MIN_M comment: the producer writes fragment-tiled activations with
  rows padded, so the consumer reads fragments without re-laying them out).
"""
import numpy as np

E8M0_PAD = 0x7F
A_TILE_ROWS = 32


def prelayout_fp8_block(w):
    w = np.asarray(w, np.uint8)
    N, K = w.shape
    assert N % 16 == 0 and K % 128 == 0
    nt, KS = N // 16, K // 128
    # [nt][row][ks][g][h][j] -> [nt][ks][h][g][row][j]; lane = row + 16 g
    t = w.reshape(nt, 16, KS, 4, 2, 16).transpose(0, 2, 4, 3, 1, 5)
    return np.ascontiguousarray(t).reshape(-1)


def unprelayout_fp8_block(pre, N, K):
    nt, KS = N // 16, K // 128
    t = np.asarray(pre, np.uint8).reshape(nt, KS, 2, 4, 16, 16)     # [nt][ks][h][g][row][j]
    return np.ascontiguousarray(t.transpose(0, 4, 1, 3, 2, 5)).reshape(N, K)


def prelayout_mxfp4_codes(wp):
    wp = np.asarray(wp, np.uint8)
    N, Kh = wp.shape
    K = Kh * 2
    assert N % 16 == 0 and K % 128 == 0
    nt, KS = N // 16, K // 128
    # [nt][row][ks][g][b] -> [nt][ks][g][row][b]
    t = wp.reshape(nt, 16, KS, 4, 16).transpose(0, 2, 3, 1, 4)
    return np.ascontiguousarray(t).reshape(-1)


def unprelayout_mxfp4_codes(pre, N, K):
    nt, KS = N // 16, K // 128
    t = np.asarray(pre, np.uint8).reshape(nt, KS, 4, 16, 16)      # [nt][ks][g][row][b]
    return np.ascontiguousarray(t.transpose(0, 3, 1, 2, 4)).reshape(N, K // 2)


def mxfp4_scale_bytes(N, K):
    KS = K // 128
    return (N // 16) * ((KS + 3) // 4) * 256


def prelayout_mxfp4_scales(e):
    e = np.asarray(e, np.uint8)
    N, K32 = e.shape
    K = K32 * 32
    nt, KS = N // 16, K // 128
    KQ = (KS + 3) // 4
    padded = np.full((N, KQ * 16), E8M0_PAD, np.uint8)
    padded[:, :K32] = e
    # [nt][row][kq][r][g] -> [nt][kq][g][row][r]; lane = row + 16 g, ks = 4 kq + r
    t = padded.reshape(nt, 16, KQ, 4, 4).transpose(0, 2, 4, 1, 3)
    return np.ascontiguousarray(t).reshape(-1)


def unprelayout_mxfp4_scales(pre, N, K):
    nt, KS = N // 16, K // 128
    KQ = (KS + 3) // 4
    t = np.asarray(pre, np.uint8).reshape(nt, KQ, 4, 16, 4)       # [nt][kq][g][row][r]
    full = np.ascontiguousarray(t.transpose(0, 3, 1, 4, 2)).reshape(N, KQ * 16)
    return full[:, : K // 32].copy()


def tiled_activation_bytes(M, K):
    return -(-M // A_TILE_ROWS) * A_TILE_ROWS * K


def tile_activation(q):
    """[M, K] e4m3 codes -> the activation-tiled byte order (pad rows are 0)."""
    q = np.asarray(q, np.uint8)
    M, K = q.shape
    assert K % 128 == 0
    Mp = -(-M // A_TILE_ROWS) * A_TILE_ROWS
    padded = np.zeros((Mp, K), np.uint8)
    padded[:M] = q
    RB, KS = Mp // 32, K // 128
    # [rb][r][ks][h][c][g][j] -> [rb][ks][h][g][r][c][j]; lane = r + 32 g
    t = padded.reshape(RB, 32, KS, 2, 2, 2, 16).transpose(0, 2, 3, 5, 1, 4, 6)
    return np.ascontiguousarray(t).reshape(-1)


def untile_activation(t, M, K):
    """Inverse of tile_activation: the first M rows back in row-major order."""
    Mp = -(-M // A_TILE_ROWS) * A_TILE_ROWS
    RB, KS = Mp // 32, K // 128
    a = np.asarray(t, np.uint8)[: Mp * K].reshape(RB, KS, 2, 2, 32, 2, 16)   # [rb][ks][h][g][r][c][j]
    return np.ascontiguousarray(a.transpose(0, 4, 1, 2, 5, 3, 6)).reshape(Mp, K)[:M].copy()
