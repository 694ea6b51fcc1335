"""Reader for the `key = value` fixtures under tests/golden/."""

from __future__ import annotations

from pathlib import Path

GOLDEN = Path(__file__).resolve().parent / "golden"


def load(name: str) -> dict:
    out = {}
    for raw in (GOLDEN / name).read_text().splitlines():
        line = raw.split("#", 1)[0].strip()
        if not line:
            continue
        key, val = (s.strip() for s in line.split("=", 1))
        parts = val.split()
        conv = []
        for p in parts:
            try:
                conv.append(int(p))
            except ValueError:
                conv.append(float(p))
        out[key] = conv if len(conv) > 1 else conv[0]
    return out
