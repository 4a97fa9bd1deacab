"""Reader for the hand-worked fixtures in tests/golden/ (key: values lines)."""
import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def read_golden(name):
    """Return {key: [list of whitespace-split token lists, one per line]}."""
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, _, rest = line.partition(":")
            out.setdefault(key.strip(), []).append(rest.split())
    return out
