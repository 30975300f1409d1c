"""Build the HIP library ``libmiconv.so`` in-tree with hipcc for gfx950.

Always recompiles.  Objects are compiled in parallel, then linked into one
shared library next to this file.  Packed-fp32 VALU instructions are disabled
for all device code.  The compiler's per-kernel resource report is read for
every device kernel; a kernel with a nonzero scratch (private memory) size,
i.e. register spills or a stack, fails the build.
"""
import os
import re
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmiconv.so")
SOURCES = ["igemm.hip", "patch.hip", "bwdf16.hip", "pointwise.hip", "tinyc.hip", "noalloc.hip", "bwd_bias.hip",
           "convnd.hip", "plan.cpp", "ndplan.cpp", "abi.cpp"]
ARCH = "gfx950"
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return "hipcc"


def compile_flags():
    return ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I" + os.path.join(ROOT, "include"), "-I" + CSRC]


_REMARK = re.compile(r"remark: .*?(Function Name|ScratchSize \[bytes/lane\]): (\S+)")


def scratch_kernels(lines):
    """(kernel, bytes per lane) of every kernel whose resource report (the
    -Rpass-analysis=kernel-resource-usage remarks) shows a nonzero scratch size."""
    found, name = [], None
    for line in lines:
        m = _REMARK.search(line)
        if not m:
            continue
        if m.group(1) == "Function Name":
            name = m.group(2)
        elif int(m.group(2)) != 0:
            found.append((name, int(m.group(2))))
    return found


def build(verbose: bool = False) -> str:
    hipcc = _hipcc()
    with tempfile.TemporaryDirectory(prefix="miconv_build_") as tmp:
        procs, objs = [], []
        for src in SOURCES:
            obj = os.path.join(tmp, src + ".o")
            if src.endswith(".hip"):
                cmd = [hipcc] + compile_flags() + ["-Rpass-analysis=kernel-resource-usage", "-x", "hip"]
            else:  # host-only C++ (no device code)
                cmd = [hipcc, "-x", "c++", "-O2", "-std=c++17", "-fPIC", "-D__HIP_PLATFORM_AMD__",
                       "-I" + os.path.join(ROCM, "include"), "-I" + os.path.join(ROOT, "include"),
                       "-I" + CSRC]
            cmd = cmd + ["-c", os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
            objs.append(obj)
        failed, scratch = [], []
        for src, pr in procs:
            out, _ = pr.communicate()
            lines = out.decode(errors="replace").splitlines()
            scratch += scratch_kernels(lines)
            text = "\n".join(l for l in lines if "packed-fp32-ops" not in l and "remark:" not in l)
            if pr.returncode != 0:
                failed.append(src)
                sys.stderr.write(text + "\n")
            elif verbose and text.strip():
                print(text)
        if failed:
            raise RuntimeError("hipcc failed for " + ", ".join(failed))
        if scratch:
            raise RuntimeError("device kernels use scratch memory (register spills or a stack): "
                               + "; ".join("%s: %d bytes/lane" % k for k in scratch))
        tmp_lib = LIB + ".tmp"
        cmd = [hipcc, "--offload-arch=" + ARCH, "-shared", "-fPIC"] + objs + ["-o", tmp_lib]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        os.replace(tmp_lib, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
