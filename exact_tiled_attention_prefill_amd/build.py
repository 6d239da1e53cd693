"""Build libfa.so (the HIP kernels and the C ABI of include/fa.h) for gfx950.

Each .hip source is compiled to an object with hipcc (in parallel), then
linked into exact_tiled_attention_prefill_amd/libfa.so.  The device assembly
of every library source is generated as well and checked for hazards the
compiler does not guard around the kernels' inline-asm LDS copies
(isa_check.py); a violation fails the build.  The hardware-ceiling
probes the benchmark reports beside the nominal peaks are linked separately
into libfa_probes.so (not part of the attention ABI).  Intermediate objects
go to _build/ at the repository root.  Run `python -m
exact_tiled_attention_prefill_amd.build` or call build().
"""

import concurrent.futures
import os
import shutil
import subprocess
import sys

try:
    from . import isa_check
except ImportError:  # run as a script
    import isa_check

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libfa.so")
PROBE_LIB = os.path.join(PKG, "libfa_probes.so")

SOURCES = ["fa_api.hip", "prefill_bf16.hip", "prefill_f32.hip", "decode.hip", "backward_bf16.hip"]
PROBE_SOURCES = ["ceiling_probes.hip"]
# Per-source flags.  The MFMA prefill keeps its accumulators in the VGPR form
# of the MFMA instructions, which lets the allocator use the AGPR half of the
# register file as overflow instead of scratch memory.
# prefill_bf16.hip: no NaN can arise inside the bf16 prefill kernel (every row
# sees a key in its first tile, so the running max is finite and masked
# scores give exp2(-inf) = 0), and -fno-honor-nans lets the row maxima compile
# to bare v_max3_f32 instead of quieting every MFMA result first.  The decode
# source keeps full NaN semantics.
SOURCE_FLAGS = {"prefill_bf16.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1", "-fno-honor-nans"]}

ARCH = "gfx950"
# Packed-fp32 VALU forms are disabled for all device code: hipcc would
# otherwise emit v_pk_{add,mul,fma}_f32 from ordinary float code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# The kernels reinterpret LDS and register data between element types (bf16
# pairs, 16-byte vectors); strict-aliasing based reordering is turned off so
# such accesses keep their program order.
COMMON_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
                "-Wno-unused-function", "-fno-strict-aliasing", "-I", INCLUDE] + DEVICE_FLAGS


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def _compile(src, extra):
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *COMMON_FLAGS, *SOURCE_FLAGS.get(src, []), *extra, "-c", os.path.join(CSRC, src),
           "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj, r.stderr


def _device_asm(src, extra):
    """The device assembly hipcc generates for src with the same flags."""
    out = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".s")
    cmd = [hipcc(), *COMMON_FLAGS, *SOURCE_FLAGS.get(src, []), *extra, "--cuda-device-only", "-S",
           os.path.join(CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc -S failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    with open(out) as f:
        return f.read()


def check_device_code(srcs=None, extra=()):
    """Generate each source's device assembly and raise if isa_check finds a hazard."""
    srcs = SOURCES if srcs is None else srcs
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(srcs)) as ex:
        asms = dict(zip(srcs, ex.map(lambda s: _device_asm(s, list(extra)), srcs)))
    bad = []
    for src, asm in asms.items():
        bad += [f"{src}: {fn}: {insn}: {rule}" for fn, insn, rule in isa_check.check_asm(asm)]
    if bad:
        raise RuntimeError("device code hazard around an inline-asm LDS copy:\n" + "\n".join(bad[:20]))


def _link(objs, lib):
    tmp = lib + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose=False, extra_flags=()):
    """Compile every kernel source, link libfa.so and libfa_probes.so; returns libfa.so's path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = SOURCES + PROBE_SOURCES
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(srcs)) as ex:
        results = dict(zip(srcs, ex.map(lambda s: _compile(s, list(extra_flags)), srcs)))
    if verbose:
        for _, err in results.values():
            if err.strip():
                print(err, file=sys.stderr)
    check_device_code(SOURCES, extra_flags)
    _link([results[s][0] for s in SOURCES], LIB)
    _link([results[s][0] for s in PROBE_SOURCES], PROBE_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
