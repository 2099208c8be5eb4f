"""Reader for the hand-worked fixtures in tests/golden/ (see README.txt there)."""

import glob
import os
import re

import numpy as np

GOLDEN_DIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _hex_bytes(text: str) -> bytes:
    out = bytearray()
    for tok in text.split():
        m = re.fullmatch(r"([0-9A-Fa-f]+)(?:\*(\d+))?", tok)
        if not m or len(m.group(1)) % 2:
            raise ValueError(f"bad hex token {tok!r}")
        out += bytes.fromhex(m.group(1)) * int(m.group(2) or 1)
    return bytes(out)


def load(path: str) -> dict:
    rec = {"set": [], "stream": []}
    with open(path) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, val = (s.strip() for s in line.split(":", 1))
            if key in ("set", "stream"):
                rec[key].append(val)
            else:
                rec[key] = val
    esz, n = int(rec["esz"]), int(rec["n"])
    dt = np.uint32 if esz == 4 else np.uint16
    x = np.zeros(n, dtype=dt)
    for s in rec["set"]:
        rng, hx = s.split(":")
        lo, hi = (int(v) for v in rng.split("-"))
        x[lo: hi + 1] = int(hx, 16)
    stream = np.frombuffer(_hex_bytes(" ".join(rec["stream"])), dtype=np.uint8)
    return dict(name=os.path.basename(path), algo=rec["algo"], esz=esz, n=n,
                x=x, stream=stream, size=int(rec["size"]))


def all_cases():
    return [load(p) for p in sorted(glob.glob(os.path.join(GOLDEN_DIR, "*_*.txt")))
            if not p.endswith("README.txt")]
