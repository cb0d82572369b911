"""Builds libdsa.so (the HIP/gfx950 DSA library) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libdsa.so")
SOURCES = ["dsa_api.cpp", "indexer.hip", "topk.hip", "sparse_mla.hip", "indexer_kl.hip", "sparse_mla_bwd.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # no packed fp32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


# Per-source extra flags: VGPR-form MFMAs.  The attention kernel keeps its
# logit accumulators in VGPRs so that its 256 output accumulators alone fill
# the accumulation registers; the indexer's epilogue (also run by the fused
# prefill's top-k when it rescores keys) reads every accumulator with VALU
# instructions, which cannot read accumulation registers directly.
_VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]
SOURCE_FLAGS = {"sparse_mla.hip": _VGPR_FORM, "indexer.hip": _VGPR_FORM, "indexer_kl.hip": _VGPR_FORM,
                "topk.hip": _VGPR_FORM}


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(" ".join(cmd) + "\n" + r.stdout + r.stderr)
        raise RuntimeError("hipcc failed building libdsa.so")
    return r


def build(verbose: bool = False, extra=(), out: str | None = None, link_extra=()) -> str:
    """Compiles every source and links libdsa.so into `out` (default: in-tree)."""
    import concurrent.futures
    import tempfile
    inc = ["-I", os.path.join(ROOT, "include")]
    with tempfile.TemporaryDirectory(prefix="dsa_build_") as tmpdir:
        objs, cmds = [], []
        for src in SOURCES:
            obj = os.path.join(tmpdir, src.replace(".", "_") + ".o")
            objs.append(obj)
            flags = [f for f in HIPCC_FLAGS if f != "-shared"]
            cmds.append(["hipcc", *flags, *SOURCE_FLAGS.get(src, []), *extra, *inc, "-x", "hip", "-c",
                         os.path.join(CSRC, src), "-o", obj])
        with concurrent.futures.ThreadPoolExecutor(max_workers=len(cmds)) as ex:
            results = list(ex.map(_run, cmds))
        out = out or LIB
        tmp = out + ".tmp"
        link = ["hipcc", "--offload-arch=gfx950", "-fPIC", "-shared", *link_extra, *objs, "-o", tmp]
        results.append(_run(link))
    if verbose:
        for r in results:
            sys.stderr.write(r.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
