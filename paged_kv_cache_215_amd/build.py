"""Build libpa.so (the HIP library behind include/pa.h) for gfx950, in-tree.

    python -m paged_kv_cache_215_amd.build [--asm DIR]

Every source is compiled with hipcc for gfx950 with packed-FP32 instructions
disabled, then linked into paged_kv_cache_215_amd/libpa.so. ``--asm DIR`` also
writes each kernel file's device assembly to DIR for inspection.
"""

import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libpa.so")
SOURCES = ["pa_api.cpp", "pa_block_manager.cpp", "pa_scheduler.cpp", "pa_engine.cpp",
           "pa_scatter.hip",
           "pa_copy.hip",
           "pa_decode.hip", "pa_prefill.hip"]
ARCH = "gfx950"


def hipcc():
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found: the HIP library cannot be built")
    return exe


def common_flags():
    return [
        f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-I", INCLUDE, "-I", CSRC,
        # packed FP32 VALU forms are kept out of every kernel
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
    ]


# Per-source code-generation flags. The prefill kernel keeps its MFMA
# accumulators in ordinary VGPRs: with the accumulation registers the compiler
# copied all 64 accumulators to VGPRs and back on every key tile so that the
# softmax rescale could scale them.
EXTRA_FLAGS = {"pa_prefill.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def _run(cmd):
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(line for line in proc.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in line)
    if proc.returncode != 0:
        raise RuntimeError(f"command failed ({proc.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(asm_dir=None, jobs=8, verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    objs = []

    def compile_one(src):
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        extra = EXTRA_FLAGS.get(src, [])
        cmd = [cc] + common_flags() + extra + ["-c", os.path.join(CSRC, src), "-o", obj]
        if src.endswith(".cpp"):
            cmd[1:1] = ["-x", "hip"]
        out = _run(cmd)
        if asm_dir and src.endswith(".hip"):
            os.makedirs(asm_dir, exist_ok=True)
            _run([cc] + common_flags() + extra + ["-S", "--cuda-device-only", os.path.join(CSRC, src),
                                          "-o", os.path.join(asm_dir, src + ".s")])
        return obj, out

    with ThreadPoolExecutor(max_workers=jobs) as ex:
        for obj, out in ex.map(compile_one, SOURCES):
            objs.append(obj)
            if verbose and out.strip():
                print(out)
    tmp = LIB + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs)
    os.replace(tmp, LIB)
    return LIB


def kernel_resources(lib_path=LIB):
    """Per-kernel resource metadata of the gfx950 code objects inside the
    built library: {kernel name: {field: int}} with private (scratch) segment
    size, VGPR / AGPR / SGPR counts, spill counts and LDS size. Reads the
    library this build made (llvm-objdump --offloading, llvm-readelf --notes)."""
    import re
    import tempfile
    llvm = "/opt/rocm/llvm/bin"
    out = {}
    with tempfile.TemporaryDirectory() as tmp:
        copy = os.path.join(tmp, "lib.so")
        shutil.copyfile(lib_path, copy)
        _run([os.path.join(llvm, "llvm-objdump"), "--offloading", copy])
        for fn in sorted(os.listdir(tmp)):
            if "amdgcn" not in fn:
                continue
            notes = _run([os.path.join(llvm, "llvm-readelf"), "--notes", os.path.join(tmp, fn)])
            # Each kernel is one list item of amdhsa.kernels ("  - .field: ..."
            # opens it); its fields are sorted by name, so some come before
            # its .name and the item is stored when the next one opens.
            fields, name = None, None
            def flush():
                if fields is not None and name:
                    out[name] = dict(fields)
            for line in notes.splitlines():
                if re.match(r"  - \.", line):
                    flush()
                    fields, name = {}, None
                if fields is None:
                    continue
                m = re.match(r"\s+(?:- )?\.name:\s+(\S+)", line)
                if m:
                    name = m.group(1)
                    continue
                m = re.match(r"\s+(?:- )?\.(private_segment_fixed_size|vgpr_count|agpr_count|"
                             r"sgpr_count|vgpr_spill_count|sgpr_spill_count|"
                             r"group_segment_fixed_size):\s+(\d+)", line)
                if m:
                    fields[m.group(1)] = int(m.group(2))
            flush()
    return out


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--asm", default=None, help="write device assembly here")
    ap.add_argument("-v", "--verbose", action="store_true")
    args = ap.parse_args(argv)
    print(build(asm_dir=args.asm, verbose=args.verbose))


if __name__ == "__main__":
    sys.exit(main())
