"""Writes config1_digest.txt: the oracle's NVFP4 codes/scales/tensor scale and a
few layer outputs for the 256x512 single-layer workload (seeded inputs), as a
regression anchor for the oracle.  Calls only the oracle and the seeded input
generators.  Run from the repository root:  python tests/golden/make_config1_digest.py
"""
import hashlib
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import synth  # noqa: E402
from oracle import gemm, nvfp4  # noqa: E402


def digest():
    c = synth.config1()
    codes, scales, S = nvfp4.quantize(c["w"])
    y = gemm.forward_nvfp4(c["x"], codes, scales, S, c["a"], c["b"], c["lora_scale"])
    lines = [
        "# oracle regression anchor for the 256x512 NVFP4 layer (x 4x512, LoRA rank 8, s=2)",
        "# written by tests/golden/make_config1_digest.py (oracle + seeded inputs only)",
        f"codes_sha256 {hashlib.sha256(codes.tobytes()).hexdigest()}",
        f"scales_sha256 {hashlib.sha256(scales.tobytes()).hexdigest()}",
        f"S_hex {np.float32(S).view(np.uint32):08x}",
    ]
    for (m, n) in [(0, 0), (1, 17), (2, 128), (3, 255)]:
        lines.append(f"y {m} {n} {y[m, n].hex()}")
    return "\n".join(lines) + "\n"


if __name__ == "__main__":
    with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "config1_digest.txt"), "w") as f:
        f.write(digest())
