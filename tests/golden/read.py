"""Readers for the small text fixtures in this folder."""
import os

HERE = os.path.dirname(os.path.abspath(__file__))


def cases(fname):
    """Parse 'case NAME' blocks of 'key v1 v2 ...' lines; '#' starts a comment."""
    out, cur = [], None
    with open(os.path.join(HERE, fname)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *vals = line.split()
            if key == "case":
                cur = {"name": vals[0]}
                out.append(cur)
            else:
                cur[key] = [float(v) for v in vals]
    return out


def constants(fname="page_constants.txt"):
    out = {}
    with open(os.path.join(HERE, fname)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            left, src = line.split("|", 1)
            name, val = left.split()
            out[name] = (int(val), src.strip())
    return out
