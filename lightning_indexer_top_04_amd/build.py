"""Build liblsi.so in-tree with hipcc for gfx950.

    python -m lightning_indexer_top_04_amd.build        # compile and link

Every HIP source under csrc/ is compiled to an object in csrc/_build/ (in
parallel), then linked into lightning_indexer_top_04_amd/liblsi.so.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "liblsi.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed-fp32 VALU forms are disabled on purpose: ordinary float code is
# compiled to scalar-per-lane VALU instead.
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-munsafe-fp-atomics", "-Wall", "-Wno-unused-result",
]

SOURCES = ["api.hip", "scan.hip", "topk.hip", "attn.hip", "prefill.hip"]

# The score kernels take ReLU of MFMA results; NaN inputs (fp8 NaN codes) are
# invalid by contract, so these files skip NaN canonicalisation before max().
EXTRA = {"scan.hip": ["-fno-honor-nans"], "prefill.hip": ["-fno-honor-nans"]}


def _compile(src: str, obj: str) -> None:
    cmd = [HIPCC, *FLAGS, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")


def build(verbose: bool = True) -> str:
    bdir = os.path.join(CSRC, "_build")
    os.makedirs(bdir, exist_ok=True)
    objs = [os.path.join(bdir, s.replace(".hip", ".o")) for s in SOURCES]
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        list(ex.map(lambda p: _compile(*p), zip(SOURCES, objs)))
    tmp = OUT + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT}")
    return OUT


if __name__ == "__main__":
    build()
    sys.exit(0)
