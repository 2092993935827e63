"""CPU oracle for the block-scaled linear layer and its fused producer.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library (no kernels, headers, tables or helpers) and imports nothing from it.

Everything here is plain, slow and written to be checked by eye against the
source pages (the five "vllm-sly-radiance" module pages: radiance_kernels.py,
radiance_gemm.py, radiance_mxfp4.py, radiance_arnq.py).  Floating point is
fp64 unless the pages fix a precision; every GEMM reaches a plain definition
(exact decode, exact scale application, fp64 accumulation, one rounding to
bf16), so the oracle is that definition written out.

Modules
  codecs    exact decoders (e4m3fn, e2m1, e8m0, bf16) and RNE encoders
  gemm      the three GEMM definitions and the per-element error budget
  producer  residual add -> Gemma RMSNorm -> per-token e4m3 quant, step by step
  quant     the pages' per-token quant and the block / group fixture quantizers
  layout    the weight pre-layout index maps (gfx950 MFMA fragment order)
  checks    the tolerance checks used by the parity tests

Parity pins live in tests/test_oracle_*.py.  Every function here is pinned to
something other than itself (closed forms, the pages' printed tables,
library conversions, exact rational brute force); none is "parity unpinned".
"""
from . import codecs, gemm, producer, quant, layout, checks  # noqa: F401
