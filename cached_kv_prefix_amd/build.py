"""Builds libflashblock.so (the attention library) and libfb_ceiling.so (the measured-ceiling
kernels the bench sets beside the published peaks) in-tree with hipcc for gfx950
(cross-compiles without a GPU).

    python -m cached_kv_prefix_amd.build
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
OBJ = os.path.join(ROOT, "_build", "obj")
LIB = os.path.join(HERE, "libflashblock.so")
CEILING_LIB = os.path.join(HERE, "libfb_ceiling.so")
CEILING_SOURCES = ["fb_ceiling.hip"]
SOURCES = ["fb_attn.hip", "fb_stream.hip", "fb_fa.hip", "fb_combine.hip", "fb_losa.hip", "fb_residual.hip", "fb_lifecycle.hip", "fb_api.hip", "fb_noalloc.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed-fp32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def _compile(src: str, obj_dir: str = OBJ, defines=()) -> str:
    obj = os.path.join(obj_dir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *[f"-D{d}" for d in defines], "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def _link(objs, out: str) -> None:
    tmp = out + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, out)


def build(verbose: bool = False, out: str = LIB, defines=()) -> str:
    """Compile every source and link `out`; `defines` are extra -D macros (tuning knobs).
    The default build also links the measured-ceiling library."""
    obj_dir = OBJ if out == LIB else out + ".obj"
    os.makedirs(obj_dir, exist_ok=True)
    both = out == LIB and not defines
    sources = SOURCES + (CEILING_SOURCES if both else [])
    with cf.ThreadPoolExecutor(max_workers=min(4, len(sources))) as ex:
        objs = dict(zip(sources, ex.map(lambda s: _compile(s, obj_dir, defines), sources)))
    _link([objs[s] for s in SOURCES], out)
    if verbose:
        print(f"built {out}")
    if both:
        _link([objs[s] for s in CEILING_SOURCES], CEILING_LIB)
        if verbose:
            print(f"built {CEILING_LIB}")
    return out


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
