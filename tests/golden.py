"""Reader for the small text fixtures under tests/golden/ (values printed on the pages)."""

import os

GOLDEN_DIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load(name: str) -> dict:
    """Parse `key = v1 v2 ...` lines; '#' starts a comment. Values stay strings."""
    out = {}
    with open(os.path.join(GOLDEN_DIR, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            k, v = line.split("=", 1)
            out[k.strip()] = v.split()
    return out


def floats(d: dict, key: str) -> list:
    return [float(v) for v in d[key]]


def ints(d: dict, key: str) -> list:
    return [int(v, 0) for v in d[key]]
