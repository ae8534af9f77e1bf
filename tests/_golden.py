"""Reader for the small text fixtures under tests/golden/ (citations are in each file)."""
import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def read_pairs(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append(line.split())
    return rows


def read_kv(name):
    return {r[0]: r[1:] for r in read_pairs(name)}
