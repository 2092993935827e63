"""Helpers for the GPU parity tests: move numpy arrays to the device and back,
and build each workload's inputs (seeded draws from the shared generator
module, quantized by the oracle's fixture quantizers so the HIP path and the
oracle see the very same bytes)."""
import numpy as np
import torch

from block_scaled_precision_04_amd import synth
from oracle import quant

DEV = "cuda"


def dev_u8(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.uint8)).to(DEV)


def dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).to(DEV).view(torch.bfloat16)


def dev_f32(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(DEV)


def host_bits16(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def host_u8(t):
    return t.view(torch.uint8).cpu().numpy()


def fp8_block_inputs(workload, case, M, N, K, outliers=False):
    """Block-FP8 inputs: activations N(0,1) quantized per token per 128-K
    group, weights N(0, 0.02) (optionally 1% outliers x10) per 128x128 block."""
    a_bits, w_bits = synth.fp8_block_raw(workload, case, M, N, K, outliers=outliers)
    aq, asc = quant.quant_group128_bf16(a_bits)
    wq, wsc = quant.quant_block128_bf16(w_bits)
    return aq, asc, wq, wsc


def w4a8_inputs(workload, case, M, N, K):
    """MXFP4 W4A8 inputs: uniform codes, e8m0 in 117..130, activations N(0,1)
    quantized per token."""
    wp, e = synth.mxfp4_weight_raw(workload, case, N, K)
    x = synth.activation_raw(workload, case, M, K)
    aq, asc = quant.quant_per_token_bf16(x)
    return aq, asc, wp, e


def sample_grid(M, N, nrows, ncols, seed):
    """Rows and columns to check at sizes too large for the full oracle:
    the first and last of each, tile edges, and random picks."""
    g = np.random.default_rng(seed)
    rows = {0, M - 1, min(M - 1, 31), min(M - 1, 32), min(M - 1, 127), min(M - 1, 128)}
    cols = {0, N - 1, min(N - 1, 15), min(N - 1, 16), min(N - 1, 127), min(N - 1, 128)}
    rows |= set(g.integers(0, M, nrows).tolist())
    cols |= set(g.integers(0, N, ncols).tolist())
    r = np.array(sorted(rows))
    c = np.array(sorted(cols))
    rr, cc = np.meshgrid(r, c, indexing="ij")
    return rr.reshape(-1), cc.reshape(-1)


def block_samples(M, N, block, seed):
    """One random element in every block x block cell of an [M, N] output.
    Every tile of every tiled launch (256x256 or 128x128 tiles, column strips
    starting at multiples of 128) contains whole cells, so each tile of each
    launch is checked at least once."""
    g = np.random.default_rng(seed)
    r0, c0 = np.meshgrid(np.arange(0, M, block), np.arange(0, N, block), indexing="ij")
    r = np.minimum(r0 + g.integers(0, block, r0.shape), M - 1)
    c = np.minimum(c0 + g.integers(0, block, c0.shape), N - 1)
    return r.reshape(-1), c.reshape(-1)


def oracle_at(fn, rows, cols, *args, chunk=2048):
    """fn(*args, rows, cols) evaluated in chunks of samples (bounded host
    memory at K = 17408); returns (c_exact, abs_sum) over all samples."""
    ce, asum = [], []
    for i in range(0, len(rows), chunk):
        _, c, a = fn(*args, rows[i:i + chunk], cols[i:i + chunk])
        ce.append(c)
        asum.append(a)
    return np.concatenate(ce), np.concatenate(asum)
