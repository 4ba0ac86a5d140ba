"""Build liblsa.so (the C-ABI library of the LSA hot path) for gfx950.

Every translation unit under csrc/ is compiled by hipcc for gfx950 only and
linked into long_context_sparse_lsa_amd/liblsa.so. Objects go to _build/ at
the repository root. Run `python -m long_context_sparse_lsa_amd.build`.
"""
import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "liblsa.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

CFLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-I" + INCLUDE, "-I" + CSRC,
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
    # packed fp32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


# Per-file flags. The indexer and attention kernels keep their MFMA
# accumulators in ordinary VGPRs, which their VALU epilogues read directly
# (no copies between accumulation and vector registers in the loops).
_VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]
# The softmax takes no NaN inputs (scores of finite bf16 rows, -inf for
# masked keys) and never depends on the sign of a zero sum, so its max and
# sum chains need no NaN quieting or -0 handling.
_NO_NAN = ["-fno-honor-nans", "-fno-signed-zeros"]
FILE_FLAGS = {"index_prefill.hip": _VGPR_FORM, "index_decode.hip": _VGPR_FORM,
              "attention.hip": _VGPR_FORM + _NO_NAN, "attention_bwd.hip": _VGPR_FORM, "kl.hip": _VGPR_FORM,
              "hi_step.hip": _VGPR_FORM + _NO_NAN}


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *CFLAGS, *FILE_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj]
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{p.stderr}")
    # hipcc's host pass warns that it does not know the packed-fp32 feature
    msgs = [ln for ln in p.stderr.splitlines() if "packed-fp32-ops" not in ln]
    return obj, "\n".join(msgs)


def build(verbose=True, jobs=None):
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(len(srcs), max(1, (os.cpu_count() or 4) // 2), 8)
    with cf.ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(_compile, srcs))
    for obj, msg in results:
        if verbose and msg.strip():
            print(msg, file=sys.stderr)
    objs = [o for o, _ in results]
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", f"--offload-arch={ARCH}", "-fPIC", *objs, "-o", tmp]
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"link failed:\n{p.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
