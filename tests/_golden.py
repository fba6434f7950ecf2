"""Reader for the text fixtures under tests/golden/ (name = value | title | section)."""
import os

_DIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load(name: str) -> dict:
    out = {}
    with open(os.path.join(_DIR, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, rest = line.split("=", 1)
            value = rest.split("|", 1)[0].strip()
            out[key.strip()] = float(value)
    return out
