"""Readers for the hand-written fixtures under tests/golden/ (no arithmetic of the method)."""
import math
import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _lines(name):
    with open(os.path.join(GOLDEN, name)) as fh:
        for line in fh:
            line = line.strip()
            if line and not line.startswith("#"):
                yield line


def _num(tok):
    return math.nan if tok == "nan" else float(tok)


def e2m1_table():
    return {int(c, 16): _num(v) for c, v in (l.split() for l in _lines("e2m1.txt"))}


def mx_bytes():
    out = []
    for l in _lines("mx_bytes.txt"):
        b, s, v0, v1 = l.split()
        out.append((int(b, 16), int(s, 16), _num(v0), _num(v1)))
    return out


def e4m3_cases():
    return [(int(t[1], 16), _num(t[2])) for t in (l.split() for l in _lines("e4m3_nvfp4.txt")) if t[0] == "e4m3"]


def nvfp4_cases():
    return [(int(t[1], 16), int(t[2], 16), float(t[3]), _num(t[4]))
            for t in (l.split() for l in _lines("e4m3_nvfp4.txt")) if t[0] == "nvfp4"]


def router_cases():
    out = []
    for l in _lines("router_cases.txt"):
        logits, k, ids, ws = [p.strip() for p in l.split("|")]
        out.append(([float(v) for v in logits.split()], int(k), [int(v) for v in ids.split()],
                    [float(v) for v in ws.split()]))
    return out
