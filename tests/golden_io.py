"""Readers for the text fixtures under tests/golden/ (each file states its source)."""
import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                yield line.split()


def code_value_table(name):
    """[(code, value)] from a 'hex value' fixture."""
    return [(int(c, 16), float(v)) for c, v in _lines(name)]


def value_code_table(name):
    return [(float(v), int(c, 16)) for v, c in _lines(name)]


def worked_example(name):
    """Dict with per-row 'w', 'fp8' (input E4M3 codes), 'codes', 'scales' /
    'scale' and optional 'g'."""
    out = {"w": {}, "codes": {}, "scales": {}, "scale": {}, "fp8": {}}
    for tok in _lines(name):
        key = tok[0]
        if key == "g":
            out["g"] = float(tok[1])
        elif key == "w":
            out["w"][int(tok[1])] = [float(v) for v in tok[2:]]
        elif key == "codes":
            out["codes"][int(tok[1])] = [int(v, 16) for v in tok[2:]]
        elif key == "scales":
            out["scales"][int(tok[1])] = [int(v, 16) for v in tok[2:]]
        elif key == "fp8":
            out["fp8"][int(tok[1])] = [int(v, 16) for v in tok[2:]]
        elif key == "scale":
            out["scale"][int(tok[1])] = float(tok[2])
    return out
