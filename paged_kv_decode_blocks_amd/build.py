"""Build libpkv.so (the HIP kernels and the C ABI) in-tree for gfx950 with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(HERE, "libpkv.so")

SOURCES = ["api.cpp", "block_manager.cpp", "step_graphs.cpp", "decoder.cpp", "cu_streams.cpp", "kv_append.hip", "kv_append_fp8.hip", "decode_fp8.hip", "kv_append_mxfp4.hip", "decode_mxfp4.hip", "decode_mxfp4_mfma.hip", "block_copy.hip", "decode_mha.hip", "decode_gqa.hip", "lse_merge.hip", "probe.hip", "debug_checks.hip"]

# Packed-fp32 instructions are switched off for all device code.
HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + INCLUDE, "-I" + CSRC,
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.isabs(cand) and os.path.exists(cand) or not os.path.isabs(cand)):
            return cand
    return "hipcc"


def build(verbose: bool = False, jobs: int = 0) -> str:
    """Compile every source to an object, then link libpkv.so.  Always rebuilds."""
    obj_dir = os.path.join(HERE, "_build")
    os.makedirs(obj_dir, exist_ok=True)
    hipcc = _hipcc()
    objs, procs = [], []
    for src in SOURCES:
        obj = os.path.join(obj_dir, os.path.splitext(src)[0] + ".o")
        cmd = [hipcc, *HIPCC_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        if src.endswith(".cpp"):
            cmd.insert(1, "-x")
            cmd.insert(2, "hip")
        objs.append(obj)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        if verbose or p.returncode:
            # the host pass does not know the packed-fp32 target feature; that warning is expected
            lines = [ln for ln in out.splitlines() if "packed-fp32-ops" not in ln and "not a recognized feature" not in ln]
            if lines:
                sys.stderr.write("\n".join(lines) + "\n")
        if p.returncode:
            failed.append(src)
    if failed:
        raise RuntimeError("hipcc failed for: " + ", ".join(failed))
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    subprocess.run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs], check=True)
    os.replace(tmp, LIB_PATH)
    _build_programs(hipcc, obj_dir)
    return LIB_PATH


# Standalone programs linked against libpkv.so (found next to them at run time).
PROGRAMS = {"pkv_cumask": ("pkv_cumask.cpp", ["-lrocblas"])}


def _build_programs(hipcc: str, obj_dir: str):
    for name, (src, libs) in PROGRAMS.items():
        obj = os.path.join(obj_dir, os.path.splitext(src)[0] + ".o")
        subprocess.run([hipcc, "-x", "hip", *HIPCC_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj], check=True,
                       stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
        out = os.path.join(HERE, name)
        tmp = out + ".tmp%d" % os.getpid()
        subprocess.run([hipcc, "--offload-arch=gfx950", "-o", tmp, obj, "-L" + HERE, "-lpkv", *libs,
                        "-Wl,-rpath,$ORIGIN", "-Wl,-rpath,/opt/rocm/lib"], check=True)
        os.replace(tmp, out)


def kernel_resource_usage(sources=None) -> dict:
    """Per-kernel register, scratch and LDS use of the device code, from the compiler's
    kernel-resource-usage remarks (device pass only; nothing is linked).

    Returns {demangled kernel name: {"VGPRs", "AGPRs", "ScratchSize", "Occupancy", "LDS", ...}}.
    """
    import re
    srcs = sources or [s for s in SOURCES if s.endswith(".hip")]
    hipcc = _hipcc()
    procs = []
    for src in srcs:
        cmd = [hipcc, *HIPCC_FLAGS, "--offload-device-only", "-c", os.path.join(CSRC, src), "-o", os.devnull,
               "-Rpass-analysis=kernel-resource-usage"]
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
    raw = {}
    for src, p in procs:
        out, _ = p.communicate()
        if p.returncode:
            raise RuntimeError(f"hipcc failed for {src}:\n{out}")
        name = None
        for line in out.splitlines():
            m = re.search(r"remark: Function Name: (\S+)", line)
            if m:
                name = m.group(1)
                raw[name] = {"source": src}
                continue
            m = re.search(r"remark:\s+([A-Za-z ]+?)(?: \[[^\]]*\])?: (\d+) \[-Rpass", line)
            if m and name:
                key = {"LDS Size": "LDS", "ScratchSize": "ScratchSize"}.get(m.group(1).strip(), m.group(1).strip())
                raw[name][key] = int(m.group(2))
    names = list(raw)
    dem = subprocess.run(["c++filt"], input="\n".join(names), stdout=subprocess.PIPE, text=True).stdout.splitlines()
    return {d: raw[n] for n, d in zip(names, dem)}


if __name__ == "__main__":
    print(build(verbose=True))
