"""Tiny text fixtures taken from the pages, each with its citation.

Format: '#' lines are comments (the first ones cite the passage); every
other line is 'name: v1 v2 ...'."""
import os

_HERE = os.path.dirname(os.path.abspath(__file__))


def load(name: str) -> dict:
    out = {}
    with open(os.path.join(_HERE, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, vals = line.split(":", 1)
            out[key.strip()] = [float(x) if any(c in x for c in ".e") else int(x)
                                for x in vals.split()]
    return out
