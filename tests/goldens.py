"""Reader for the small text fixtures under tests/golden/ (``key: values`` lines,
``#`` comments). Each fixture states the page and section its values come from."""
from __future__ import annotations

import os

GOLDEN_DIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load(name: str) -> dict:
    out = {}
    with open(os.path.join(GOLDEN_DIR, name), encoding="utf-8") as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, _, val = line.partition(":")
            out[key.strip()] = val.strip()
    return out


def numbers(s: str):
    return [float(v) if any(ch in v for ch in ".e") else int(v) for v in s.split()]
