"""Writes recip_trap_cases.json: int8 groups on which a reciprocal-multiply
quantiser (x * (1/s)) stores different codes from the rule's division x / s.

Calls only the CPU oracle (for the rule) and NumPy (for the planted mistake).
Run from the repository root:  python tests/golden/make_recip_trap_cases.py
"""
import json
import os
import sys

import numpy as np

sys.path.insert(0, os.path.abspath(os.path.join(os.path.dirname(__file__), "..", "..")))
from oracle import quantize_q8  # noqa: E402


def reciprocal_variant(x):
    g = x.reshape(-1, 64)
    s = (np.abs(g).max(-1) / np.float32(127)).astype(np.float16).astype(np.float32)
    inv = (np.float32(1) / s)[:, None]
    return np.clip(np.rint(g * inv), -127, 127).astype(np.int8).reshape(x.shape)


def main():
    rng = np.random.default_rng(20240611)
    found = []
    for _ in range(40):
        x = rng.standard_normal((200000, 64), dtype=np.float32)
        x *= np.exp2(rng.integers(-6, 7, size=(200000, 1))).astype(np.float32)
        c, _ = quantize_q8(x)
        cr = reciprocal_variant(x)
        bad = np.nonzero((c != cr).any(-1))[0]
        for b in bad[: 8 - len(found)]:
            found.append([f"0x{int(v):08x}" for v in x[b].view(np.uint32)])
        if len(found) >= 8:
            break
    out = {
        "source": "Division rule of PR #3084 \"FP16 K/V cache by default, int8 with --kv-q8\", section What changed (code = rint(x / scale)); groups found by searching seeded normal data for disagreement with a reciprocal-multiply quantiser. Values are float32 bit patterns.",
        "groups_f32_bits": found,
    }
    path = os.path.join(os.path.dirname(__file__), "recip_trap_cases.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(f"wrote {len(found)} groups to {path}")


if __name__ == "__main__":
    main()
