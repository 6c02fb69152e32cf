"""Readers for the small text fixtures in this folder."""
import os

HERE = os.path.dirname(os.path.abspath(__file__))


def read_kv(name):
    """Parse 'key value...' lines (comments start with '#')."""
    out = {}
    with open(os.path.join(HERE, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *vals = line.split()
            out[key] = vals if len(vals) != 1 else vals[0]
    return out
