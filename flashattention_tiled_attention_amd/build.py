"""Build the HIP attention library (libattn.so) and the three microbenchmarks, the
LDS transpose one (liblds_transpose.so), the matrix-core rate one (libmfma_rate.so)
and the instruction-issue one (libissue_rate.so), in-tree for gfx950 with hipcc."""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libattn.so")
SOURCES = ["attn_api.hip", "attn_fwd.hip", "attn_bwd.hip", "attn_sparse.hip"]
LDS_LIB = os.path.join(HERE, "liblds_transpose.so")
LDS_SOURCES = ["lds_transpose.hip"]
MFMA_LIB = os.path.join(HERE, "libmfma_rate.so")
MFMA_SOURCES = ["mfma_rate.hip"]
ISSUE_LIB = os.path.join(HERE, "libissue_rate.so")
ISSUE_SOURCES = ["issue_rate.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# Packed fp32 VALU instructions are disabled for all device code.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", INCLUDE, "-I", CSRC]
# Per-source flags. fwd1_kernel and dkv1_kernel run one wave per SIMD, so they may use
# 512 registers; for such kernels the compiler otherwise puts every MFMA accumulator in
# AGPRs, and the vector code then moves each value it reads or writes in and out of
# them with extra instructions. This flag makes it keep MFMA results in VGPRs (spilling
# cold values to AGPRs). It changes no other kernel of those files: kernels with two
# waves per SIMD (256 registers) already get that form.
_VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form=true"]
SOURCE_FLAGS = {"attn_fwd.hip": _VGPR_FORM, "attn_bwd.hip": _VGPR_FORM}


def _compile(src, obj, extra):
    cmd = [HIPCC] + FLAGS + SOURCE_FLAGS.get(src, []) + extra + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the device-only target feature; that warning is harmless
    noise = [ln for ln in r.stderr.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
    return r.returncode, cmd, "\n".join(noise)


def build(extra=None, verbose=False):
    """Compile every source and link libattn.so and the three microbenchmark libraries;
    raises on any compiler error. Returns the path of libattn.so."""
    extra = list(extra or [])
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    srcs = SOURCES + LDS_SOURCES + MFMA_SOURCES + ISSUE_SOURCES
    objs = [os.path.join(objdir, s.replace(".hip", ".o")) for s in srcs]
    with ThreadPoolExecutor(max_workers=len(srcs)) as ex:
        results = list(ex.map(lambda so: _compile(so[0], so[1], extra), zip(srcs, objs)))
    for rc, cmd, err in results:
        if err and (verbose or rc):
            sys.stderr.write(err + "\n")
        if rc:
            raise RuntimeError("hipcc failed: " + " ".join(cmd))
    n1 = len(SOURCES)
    n2 = n1 + len(LDS_SOURCES)
    n3 = n2 + len(MFMA_SOURCES)
    for lib, members in ((LIB, objs[:n1]), (LDS_LIB, objs[n1:n2]), (MFMA_LIB, objs[n2:n3]), (ISSUE_LIB, objs[n3:])):
        tmp = lib + ".tmp%d" % os.getpid()
        cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + members
        subprocess.run(cmd, check=True)
        os.replace(tmp, lib)
    return LIB


if __name__ == "__main__":
    print(build(sys.argv[1:], verbose=True))
