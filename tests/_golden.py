"""Reader for the small text fixtures under tests/golden/ (key: value lines,
'#' comments, '|' separates rows, repeated keys collect into a list)."""
import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, _, val = line.partition(":")
            key, val = key.strip(), val.strip()
            if key in out:
                if not isinstance(out[key], list) or not out.get("_multi_" + key):
                    out[key] = [out[key]]
                    out["_multi_" + key] = True
                out[key].append(val)
            else:
                out[key] = val
    return out


def nums(s, typ=float):
    return [typ(v) for v in s.split()]


def rows(s, typ=float):
    return [nums(r, typ) for r in s.split("|")]
