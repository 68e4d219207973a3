"""Reader for the small text fixtures under tests/golden/.

Format: ``key = value [value ...]`` per line, ``#`` starts a comment.  Values
are floats; a value written ``a/b`` is the fraction a/b.
"""
import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _num(tok):
    if "/" in tok:
        a, b = tok.split("/")
        return float(a) / float(b)
    return float(tok)


def load(name):
    """Return a list of records; records are separated by blank lines."""
    recs, cur = [], {}
    with open(os.path.join(GOLDEN, name)) as f:
        for raw in f:
            line = raw.split("#", 1)[0].strip()
            if not line:
                if cur:
                    recs.append(cur)
                    cur = {}
                continue
            key, val = (s.strip() for s in line.split("=", 1))
            vals = [_num(t) for t in val.split()]
            cur[key] = vals if len(vals) > 1 else vals[0]
    if cur:
        recs.append(cur)
    return recs
