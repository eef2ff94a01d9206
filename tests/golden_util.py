"""Reader for the small text fixtures under tests/golden/ (values from the pages)."""
import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def rows(name):
    """Non-comment lines, split on whitespace."""
    out = []
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                out.append(line.split())
    return out


def keyed(name):
    """'key v1 v2 ...' lines as {key: [numbers]} (ints where integral)."""
    d = {}
    for r in rows(name):
        vals = []
        for v in r[1:]:
            x = float(v)
            vals.append(int(x) if x.is_integer() and "." not in v else x)
        d[r[0]] = vals if len(vals) != 1 else vals[0]
    return d
