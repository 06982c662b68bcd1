"""Build libgmla.so (the HIP kernels and their C ABI) for gfx950 with hipcc.

    python -m causal_softmax_attention_gmla_amd.build

Each translation unit is compiled to an object in parallel, then linked into
``causal_softmax_attention_gmla_amd/libgmla.so`` next to this file.  The build
always recompiles.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
LIB = os.path.join(HERE, "libgmla.so")
PROBE_LIB = os.path.join(HERE, "libgmla_probe.so")
ARCH = "gfx950"

SOURCES = ["gmla_api.hip", "prefill_bf16.hip", "prefill_simple.hip", "decode.hip", "decode_latent.hip", "gemm.hip", "gemm_lds.hip"]
# measurement aids for the benchmark, linked into their own library
PROBE_SOURCES = ["probe.hip"]

# -packed-fp32-ops: never emit packed float32 VALU instructions (v_pk_fma_f32 and
# friends); the host pass prints a harmless "not a recognized feature" warning.
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wno-unused-command-line-argument"]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def _compile(src: str, obj: str, extra: list[str]) -> None:
    cmd = [hipcc(), *HIP_FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    noise = [ln for ln in r.stderr.splitlines()
             if ln.strip() and "packed-fp32-ops" not in ln]
    if noise:
        sys.stderr.write("\n".join(noise) + "\n")


def _link(objs: list[str], out: str) -> str:
    tmp = out + f".tmp{os.getpid()}"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs,
           "-Wl,-rpath,/opt/rocm/lib"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, out)
    return out


def build(out: str = LIB, extra: list[str] | None = None, jobs: int = 8,
          probe_out: str | None = PROBE_LIB) -> str:
    """Compile and link libgmla.so (and, unless probe_out is None, libgmla_probe.so)."""
    extra = list(extra or [])
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    srcs = SOURCES + (PROBE_SOURCES if probe_out else [])
    objs = {s: os.path.join(objdir, s.replace(".hip", ".o")) for s in srcs}
    with cf.ThreadPoolExecutor(max_workers=min(jobs, len(srcs))) as ex:
        futs = [ex.submit(_compile, s, objs[s], extra) for s in srcs]
        for f in futs:
            f.result()
    _link([objs[s] for s in SOURCES], out)
    if probe_out:
        _link([objs[s] for s in PROBE_SOURCES], probe_out)
    return out


if __name__ == "__main__":
    print(build())
