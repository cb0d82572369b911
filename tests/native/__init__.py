"""Test-only native helpers (built by __graft_entry__.build())."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
PROBE_SRC = os.path.join(HERE, "mfma_probe.hip")
PROBE_LIB = os.path.join(HERE, "libmfma_probe.so")


def build() -> str:
    cmd = ["hipcc", "--offload-arch=gfx950", "-O2", "-fPIC", "-shared", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", PROBE_SRC, "-o", PROBE_LIB + ".tmp"]
    subprocess.run(cmd, check=True, stdout=subprocess.DEVNULL, stderr=subprocess.DEVNULL)
    os.replace(PROBE_LIB + ".tmp", PROBE_LIB)
    return PROBE_LIB
