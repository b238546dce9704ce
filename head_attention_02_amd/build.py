"""Build libmi_attn.so in-tree with hipcc for gfx950.

    python -m head_attention_02_amd.build

All HIP sources under csrc/ go into one shared library next to this file.  Packed fp32
VALU instructions are disabled for the device code (-packed-fp32-ops); the host pass of
hipcc warns that it does not know that feature, which is harmless.
"""
from __future__ import annotations

import os
import subprocess
import sys
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
INCLUDE = ROOT / "include"
LIBRARY = PKG / "libmi_attn.so"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"


def sources() -> list[Path]:
    return sorted(CSRC.glob("*.hip"))


def command(output: Path = LIBRARY) -> list[str]:
    return [HIPCC, f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wno-unused-result", f"-I{INCLUDE}", f"-I{CSRC}",
            "-o", str(output), *map(str, sources())]


def build(verbose: bool = False) -> Path:
    """Compile every source into LIBRARY (always recompiles)."""
    tmp = LIBRARY.with_suffix(".so.tmp")
    proc = subprocess.run(command(tmp), capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = "\n".join(l for l in (proc.stdout + proc.stderr).splitlines() if noise not in l)
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed ({proc.returncode}):\n{msgs}")
    if verbose and msgs.strip():
        print(msgs, file=sys.stderr)
    tmp.replace(LIBRARY)
    return LIBRARY


if __name__ == "__main__":
    print(build(verbose=True))
