"""Readers for the text fixtures under tests/golden/."""
import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                yield line


def e2m1_table():
    rows = []
    for line in _lines("e2m1_ocp.txt"):
        c, s, e, m, v = line.split()
        rows.append((int(c), int(s), int(e), int(m), float(v)))
    return rows


def total_order_cases():
    cases, cur = [], None
    for line in _lines("total_order_cases.txt"):
        if line.startswith("case "):
            cur = {"name": line.split()[1]}
        elif line == "end":
            cases.append(cur)
            cur = None
        else:
            k, v = line.split(":", 1)
            vals = v.split()
            if k == "scores":
                cur[k] = [int(x, 16) for x in vals]
            else:
                cur[k] = [int(x) for x in vals]
    for c in cases:
        c["start"] = c["start"][0]
        c["K"] = c["K"][0]
    return cases


def short_rows():
    out = []
    for line in _lines("short_rows.txt"):
        v = [int(x) for x in line.split()]
        out.append((v[0], v[1], v[2], v[3:]))
    return out


def geometry():
    pairs, dense = [], None
    for line in _lines("geometry.txt"):
        v = line.split()
        if v[0] == "dense":
            dense = dict(c4=int(v[1]), bytes_per_row=int(v[2]), mib_per_row=float(v[3]),
                         rows=int(v[4]), mib_total=float(v[5]))
        else:
            pairs.append((int(v[0]), int(v[1])))
    return pairs, dense
