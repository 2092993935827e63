"""Seeded synthetic inputs for the five workloads of the block-scaled linear layer.

This module is the only code shared by the parity tests (oracle side) and the
HIP side (tests, smoke, bench).  It draws random numbers and nothing else: it
holds none of the method's arithmetic (no quantization, no rounding, no
decoding).  bf16 draws are the top 16 bits of a float32 normal sample
(truncation), so no rounding rule is shared with either side.

Workloads (sizes of the pages' production shapes; the pages' own datasets are
not used):
  fp8_block_small   block-FP8 W8A8, M=16 N=512 K=1024
  skinny_bf16       x[M,K] . W[N,K]^T, M in {6,8,16,32,64},
                    (N,K) in {(256,2048), (96,5120)}  (MoE gate, b/a projection)
  fp8_block_decode  block-FP8 W8A8, M in {8,32,64},
                    (N,K) in {(5120,5120), (10240,5120), (5120,17408)};
                    W ~ N(0, 0.02) with 1% outliers x10
  w4a8_prefill      MXFP4 W4A8, M in {256,2048,8192},
                    (N,K) in {(10240,5120), (34816,5120), (5120,17408)};
                    codes uniform bytes, e8m0 uniform in 117..130
  fused_chain       add + Gemma RMSNorm + per-token quant at K=5120,
                    M in {8,4096}, feeding W4A8 with N=17408
  silu_chain        SiLU(gate) * up + per-token quant of the gate/up
                    projection's output [M, 2*17408], M in {8,4096},
                    feeding the W4A8 down projection (K=17408)
  fp8_block_prefill block-FP8 W8A8 at large M: M in {2048, 8192} with the
                    decode workload's (N,K) shapes and distributions; the
                    group-scale chain: add + Gemma RMSNorm + per-128 quant at
                    K=5120, M=4096, feeding block-FP8 with N=10240
Seeds: 100 * workload index + case index.
"""
import numpy as np

WORKLOADS = {
    0: ("fp8_block_small", [(16, 512, 1024)]),
    1: ("skinny_bf16", [(m, n, k) for (n, k) in [(256, 2048), (96, 5120)] for m in (6, 8, 16, 32, 64)]),
    2: ("fp8_block_decode", [(m, n, k) for (n, k) in [(5120, 5120), (10240, 5120), (5120, 17408)]
                             for m in (8, 32, 64)]),
    3: ("w4a8_prefill", [(m, n, k) for (n, k) in [(10240, 5120), (34816, 5120), (5120, 17408)]
                         for m in (256, 2048, 8192)]),
    4: ("fused_chain", [(8, 17408, 5120), (4096, 17408, 5120)]),
    5: ("silu_chain", [(8, 17408), (4096, 17408)]),
    6: ("fp8_block_prefill", [(m, n, k) for (n, k) in [(5120, 5120), (10240, 5120), (5120, 17408)]
                              for m in (2048, 8192)] + [(4096, 10240, 5120)]),
}


def seed_of(workload, case):
    return 100 * workload + case


def rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def bf16_normal(g, shape, std=1.0, outlier_p=0.0, outlier_factor=10.0):
    """bf16 bit patterns of N(0, std) draws; with outlier_p > 0 a Bernoulli
    mask (drawn after the values) multiplies that fraction by outlier_factor."""
    x = g.standard_normal(shape, dtype=np.float32) * np.float32(std)
    if outlier_p > 0:
        mask = g.random(shape, dtype=np.float32) < outlier_p
        x = np.where(mask, x * np.float32(outlier_factor), x).astype(np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def uniform_bytes(g, shape):
    return g.integers(0, 256, size=shape, dtype=np.uint8)


def uniform_exponents(g, shape, lo=117, hi=130):
    return g.integers(lo, hi + 1, size=shape, dtype=np.uint8)


# ------------------------------------------------------------ per-workload raw draws
def fp8_block_raw(workload, case, M, N, K, w_std=0.02, outliers=False):
    """Raw bf16 draws for a block-FP8 GEMM: activations N(0,1) [M,K] and
    weights N(0, w_std) [N,K] (1% outliers x10 for the decode workload)."""
    g = rng(seed_of(workload, case))
    a = bf16_normal(g, (M, K), 1.0)
    w = bf16_normal(g, (N, K), w_std, outlier_p=0.01 if outliers else 0.0)
    return a, w


def skinny_raw(case, M, N, K):
    g = rng(seed_of(1, case))
    return bf16_normal(g, (M, K), 1.0), bf16_normal(g, (N, K), 0.02)


def mxfp4_weight_raw(workload, case, N, K):
    """Packed e2m1 codes [N, K/2] (two uniform nibbles per byte) and e8m0
    exponents [N, K/32] uniform in 117..130."""
    g = rng(seed_of(workload, case) * 7 + 1)
    return uniform_bytes(g, (N, K // 2)), uniform_exponents(g, (N, K // 32))


def activation_raw(workload, case, M, K):
    """bf16 N(0,1) activations [M, K] to be quantized per token."""
    g = rng(seed_of(workload, case) * 7 + 2)
    return bf16_normal(g, (M, K), 1.0)


def producer_raw(case, M, K):
    """(y partial, residual, norm weight): bf16 N(0,1), N(0,1), N(0,0.1)."""
    g = rng(seed_of(4, case))
    return bf16_normal(g, (M, K), 1.0), bf16_normal(g, (M, K), 1.0), bf16_normal(g, (K,), 0.1)


def silu_raw(case, M, N):
    """gate/up projection output gu bf16 [M, 2N]: N(0,1) with 0.1% outliers x8."""
    g = rng(seed_of(5, case))
    return bf16_normal(g, (M, 2 * N), 1.0, outlier_p=0.001, outlier_factor=8.0)


def group_chain_raw(M, K):
    """(y partial, residual, norm weight) of the group-scale chain: bf16 N(0,1),
    N(0,1), N(0,0.1) (the fused chain's distributions)."""
    g = rng(seed_of(6, 6) * 7 + 3)
    return bf16_normal(g, (M, K), 1.0), bf16_normal(g, (M, K), 1.0), bf16_normal(g, (K,), 0.1)
