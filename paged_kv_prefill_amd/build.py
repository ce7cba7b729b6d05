"""Build libpaged_kv_prefill.so (gfx950) in-tree with hipcc.

    python -m paged_kv_prefill_amd.build     (or build() from Python)

Every HIP source is compiled for gfx950 only, with packed-fp32 instruction
selection disabled, no fast-math (IEEE division and rounding are needed for
bit-exact int8 codes and fp8 dequant), and a build id made of the sources'
hash and the flags.
"""
from __future__ import annotations

import concurrent.futures as cf
import hashlib
import os
import re
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libpaged_kv_prefill.so")
SOURCES = ["pa_attention.hip", "pa_images.hip", "pa_passes.hip", "pa_probe.hip", "pa_noalloc.hip",
           "pa_verify.hip", "pa_api.cpp"]
HEADERS = ["pa_device.h", "pa_kernels.h", "pa_layout.h"]
PUBLIC_HEADER = os.path.join(ROOT, "include", "paged_kv_prefill.h")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         # the ILP-first machine scheduler issues LDS operand reads ahead of the
         # MFMAs that consume them (the default one serialises read -> wait -> MFMA)
         "-mllvm", "--amdgpu-sched-strategy=iterative-ilp",
         "-Wall", "-Wno-unused-function", "-Wno-unused-variable"]


def _source_hash() -> str:
    h = hashlib.sha256()
    for f in SOURCES + HEADERS:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    with open(PUBLIC_HEADER, "rb") as fh:
        h.update(fh.read())
    h.update(" ".join(FLAGS).encode())
    return h.hexdigest()[:16]


def _resources(stderr: str) -> dict:
    """Per-kernel figures of clang's kernel-resource-usage remarks."""
    out, name = {}, None
    for line in stderr.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            out[name] = {}
            continue
        m = re.search(r"remark:\s+([A-Za-z][^:]*): (\d+) \[-Rpass-analysis", line)
        if m and name:
            out[name][m.group(1).strip()] = int(m.group(2))
    return out


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    bid = f"paged_kv_prefill gfx950 src={_source_hash()}"
    defs = [f'-DPA_BUILD_ID="{bid}"']

    def compile_one(src):
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        cmd = [HIPCC] + FLAGS + defs + ["-c", os.path.join(CSRC, src), "-o", obj]
        if src.endswith(".hip"):
            cmd.append("-Rpass-analysis=kernel-resource-usage")
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{res.stdout}\n{res.stderr}")
        msgs = "\n".join(l for l in res.stderr.splitlines()
                         if "packed-fp32-ops" not in l and "kernel-resource-usage" not in l
                         and not re.match(r"\s*(\d+ )?\|", l) and not l.strip() == "^")
        if verbose and msgs.strip():
            print(msgs)
        return obj, _resources(res.stderr)

    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        done = list(ex.map(compile_one, SOURCES))
    objs = [o for o, _ in done]
    usage = {k: v for _, r in done for k, v in r.items()}
    with open(os.path.join(BUILD, "kernel_resources.txt"), "w") as fh:
        for name in sorted(usage):
            fh.write(f"{name} {usage[name]}\n")
    # per-lane scratch in a kernel here is always a defect (an outlined helper
    # taking the address of the by-value parameter block, or a dynamically
    # indexed private array), and a costly one: refuse to build
    bad = sorted(n for n, u in usage.items() if u.get("ScratchSize [bytes/lane]", 0) > 0)
    if bad:
        raise RuntimeError("kernels using scratch memory: " + ", ".join(bad))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    import time
    t = time.time()
    print(build(verbose=True), f"{time.time() - t:.1f}s")
