"""Checks on the gfx950 assembly of every kernel of the library (hipcc
cross-compiles without a GPU; each source is compiled once per session).

* Register budget: no VGPR/SGPR spills and no per-lane scratch.  A spill puts
  a kernel's registers in scratch memory (private segment) -- an extra memory
  round trip inside loops that are built to keep every operand in registers,
  and a per-dispatch scratch allocation.  The launch bounds and occupancy
  targets (e.g. two 256-thread workgroups per CU for the 128x128 prefill
  tile, i.e. at most 256 registers per lane) leave little room, so a source
  change that adds live values can tip one over without any test failing on
  numbers.
* M0: the direct-to-LDS loads set M0 (the LDS destination base) in inline
  assembly that lists M0 as clobbered.  The compiler does not preserve a
  reserved register across such a statement, so the library is correct only
  while the compiler itself never keeps a value in M0: every write of M0 must
  be the DMA pattern (s_mov_b32 m0 -> s_nop 0 -> global_load_lds).
* Scaled 16x16x128 MFMA accumulating in AGPRs: the one kernel ever built that
  way (an MXFP4 decode configuration with four waves, whose small register
  demand per workgroup let the compiler keep the accumulator in AGPRs) gave
  wrong results on the GPU, with exact indexing and the compiler's documented
  wait states in place; every kernel in use writes that MFMA's result to
  ordinary VGPRs, and this scan keeps it so.
* Decode-kernel load order: each wave issues its activation DMA, then the
  scale loads, then all of its weight loads, and waits before the first
  barrier only until the DMA has landed -- at most weight_loads() newer loads
  may still be outstanding.  If the compiler sinks a scale load below the
  weight loads, the wait before the LDS store of the scales covers the whole
  weight stream and the kernel serialises load and compute.
* Prefill K loop shape: the MXFP4 prefill kernels issue each half step's
  MFMAs with the next stages' direct-to-LDS loads between them.  MFMAs have
  no memory effects, so the compiler may move them across the loop's
  barriers and branches; a wave-dependent branch in the loop (e.g. a load
  that only some waves issue) once let it gather the MFMAs of three K steps
  into one run after the last barrier, which serialised loads and compute
  and cost 10-17% on the 128x128 tile.  No run of back-to-back MFMAs may be
  longer than one half step's, and the loads must sit between MFMAs.
"""
import functools
import glob
import os
import re
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "block_scaled_precision_04_amd", "csrc")
SOURCES = sorted(os.path.basename(p) for p in glob.glob(os.path.join(CSRC, "*.hip")))


def _hipcc():
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return None


pytestmark = pytest.mark.skipif(_hipcc() is None, reason="hipcc not available")


@functools.lru_cache(maxsize=None)
def _asm(src):
    """Device assembly of one source, compiled with the library's flags."""
    import tempfile
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, src + ".s")
        cmd = [_hipcc(), "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
               "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-I", CSRC, "--cuda-device-only", "-S",
               os.path.join(CSRC, src), "-o", out]
        res = subprocess.run(cmd, capture_output=True, text=True)
        assert res.returncode == 0, res.stderr[-2000:]
        with open(out) as f:
            return f.read()


def _kernels(text):
    """(mangled name, list of instruction lines) per kernel body."""
    out = []
    for chunk in re.split(r"\n(?=_Z[^\s:]*:)", text)[1:]:
        name = chunk.split(":", 1)[0]
        body = chunk.split("\n")
        end = next((i for i, ln in enumerate(body) if ln.strip().startswith(".Lfunc_end")), len(body))
        instrs = []
        for ln in body[1:end]:
            s = ln.split(";", 1)[0].strip()
            if s and not s.startswith(".") and not s.endswith(":"):
                instrs.append(s)
        out.append((name, instrs))
    return out


@pytest.mark.parametrize("src", SOURCES)
def test_no_spills(src):
    text = _asm(src)
    kernels = re.findall(r"\.name:\s+(\S+)", text)
    for key in ("vgpr_spill_count", "sgpr_spill_count", "private_segment_fixed_size"):
        vals = [int(v) for v in re.findall(rf"\.{key}:\s+(\d+)", text)]
        assert all(v == 0 for v in vals), f"{src}: {key} = {vals} (kernels {kernels})"


@pytest.mark.parametrize("src", SOURCES)
def test_m0_written_only_by_the_dma_pattern(src):
    for name, ins in _kernels(_asm(src)):
        for i, s in enumerate(ins):
            if not re.search(r"\bm0\b", s):
                continue
            assert re.fullmatch(r"s_mov_b32\s+m0,\s*s\d+", s), f"{name}: M0 used outside the DMA pattern: {s}"
            assert i + 2 < len(ins) and ins[i + 1] == "s_nop 0" and ins[i + 2].startswith("global_load_lds_"), \
                f"{name}: M0 write not followed by s_nop 0 + global_load_lds: {ins[i:i + 3]}"


def _vmcnt(s):
    m = re.search(r"vmcnt\((\d+)\)", s)
    return int(m.group(1)) if m else None


def test_decode_waits_only_for_the_activation_dma():
    ks = _kernels(_asm("gemm_decode.hip"))
    seen = 0
    for name, ins in ks:
        m = re.search(r"k_decodeILb([01])ELi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)E", name)
        if not m:
            continue
        mx, mb, tw, kw, t, r = (int(x) for x in m.groups())
        allowed = t * r + t * ((r + 3) // 4) if mx else 2 * t * r + 1   # weight_loads<MX, T, R>()
        # block-FP8 also loads its share of the slice's activation scales (kSPer per lane) before them
        scale_loads = 0 if mx else -(-(kw * r * 16 * mb) // (tw * kw * 64))
        bar = next(i for i, s in enumerate(ins) if s.startswith("s_barrier"))
        last_dma = max(i for i, s in enumerate(ins[:bar]) if s.startswith("global_load_lds"))
        loads_after = sum(1 for s in ins[last_dma + 1:bar] if s.startswith("global_load"))
        assert loads_after == allowed + scale_loads, \
            f"{name}: {loads_after} loads after the DMA, expected {allowed + scale_loads}"
        waits = [_vmcnt(s) for s in ins[last_dma + 1:bar] if s.startswith("s_waitcnt")]
        waits = [w for w in waits if w is not None]
        assert waits and min(waits) == allowed, f"{name}: vmcnt waits {waits} before the barrier, want {allowed}"
        seen += 1
    assert seen >= 10, f"only {seen} decode instantiations found"


@pytest.mark.parametrize("src", SOURCES)
def test_scaled_16x16x128_mfma_accumulates_in_vgprs(src):
    for name, ins in _kernels(_asm(src)):
        for s in ins:
            if s.startswith("v_mfma_scale_f32_16x16x128_f8f6f4"):
                dst = s.split()[1]
                assert dst.startswith("v["), f"{name}: scaled 16x16x128 MFMA writes {dst}: {s}"


def test_prefill_k_loop_keeps_mfmas_and_loads_interleaved():
    seen = 0
    for name, ins in _kernels(_asm("gemm_prefill.hip")):
        m = re.search(r"k_w4a8_prefillILi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)E", name)
        if not m:
            continue
        bm, bn, wm, wn = (int(x) for x in m.groups())
        half = (bm // wm // 32) * (bn // wn // 32)   # MFMAs per wave per 64-K half step
        dma = (bm * 128 + bn * 64) // (64 * wm * wn * 16) + -(-(bn * 16) // (64 * wm * wn * 16))
        run = longest = interleaved = 0
        for i, s in enumerate(ins):
            if s.startswith("v_mfma"):
                run += 1
                longest = max(longest, run)
                nxt = next((j for j in range(i + 1, len(ins)) if ins[j].startswith("v_mfma")), len(ins))
                if any(x.startswith("global_load_lds") for x in ins[i + 1:nxt]):
                    interleaved += 1
            elif not s.startswith(("s_waitcnt", "s_nop")):
                run = 0
        assert longest <= half, f"{name}: {longest} back-to-back MFMAs, one half step has {half}"
        # the three unrolled steps of the loop each put min(half, loads) loads right after MFMAs
        assert interleaved >= 3 * min(half, dma), f"{name}: only {interleaved} MFMAs followed by a load"
        seen += 1
    # 256x256 (4 waves), 128x128 as 4 waves of 64x64 and as 2 waves of 64x128, each
    # for row-major and activation-tiled input
    assert seen == 6, f"{seen} prefill instantiations found"


def test_split_k_handoff_uses_device_scope_instructions():
    seen = 0
    for src in ("gemm_skinny.hip", "gemm_decode.hip", "gemm_prefill.hip"):
        for name, ins in _kernels(_asm(src)):
            atoms = [i for i, s in enumerate(ins) if s.startswith("global_atomic_add")]
            if not atoms:
                continue
            a = atoms[0]
            stores = [i for i, s in enumerate(ins[:a]) if s.startswith("global_store")]
            assert stores, f"{name}: no partial store before the counter"
            # the partial stores are the device-scope ones of the path
            dev = [i for i in stores if re.search(r"\bsc1\b", ins[i])]
            assert dev, f"{name}: partial stores without sc1: {[ins[i] for i in stores[-4:]]}"
            last = dev[-1]
            waits = [s for s in ins[last + 1:a] if s.startswith("s_waitcnt") and "vmcnt(0)" in s]
            assert waits, f"{name}: counter bumped before the partial stores are acknowledged"
            assert "sc0" in ins[a], f"{name}: counter atomic does not return its value: {ins[a]}"
            loads = [s for s in ins[a + 1:] if s.startswith("global_load") and re.search(r"\bsc1\b", s)]
            assert loads, f"{name}: the partials are not read back with device-scope loads"
            assert not any(s.startswith(("buffer_wbl2", "buffer_inv")) for s in ins), \
                f"{name}: cache maintenance in the hand-off (it costs microseconds per workgroup)"
            seen += 1
    assert seen >= 10, f"only {seen} kernels with a split-K hand-off found"
