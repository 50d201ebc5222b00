"""Readers of the hand-derived fixtures under tests/golden."""

import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def parse_float(v):
    return float.fromhex(v) if v.lstrip("-").startswith("0x") else float(v)


def e4m3_cases():
    out = []
    with open(os.path.join(GOLDEN, "e4m3_cases.txt")) as f:
        for ln in f:
            ln = ln.strip()
            if not ln or ln.startswith("#"):
                continue
            v, code, *_ = ln.split()
            out.append((parse_float(v), int(code, 16)))
    return out


def quant_cases():
    """List of dicts: name, x (128 floats), S (float), q (128 codes)."""
    cases, cur = [], None
    with open(os.path.join(GOLDEN, "quant_cases.txt")) as f:
        for ln in f:
            ln = ln.split("#")[0].strip()
            if not ln:
                continue
            key, *rest = ln.split()
            if key == "case":
                cur = {"name": rest[0], "x": [0.0] * 128, "q": [0] * 128}
                cases.append(cur)
            elif key == "x":
                for a in rest:
                    i, v = a.split("=")
                    cur["x"][int(i)] = parse_float(v)
            elif key == "S":
                cur["S"] = parse_float(rest[0])
            elif key == "q":
                for a in rest:
                    i, v = a.split("=")
                    cur["q"][int(i)] = int(v, 16)
    return cases
