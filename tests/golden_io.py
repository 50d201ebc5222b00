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


def rmsnorm_cases():
    """List of dicts: name, K, eps, x, gamma (K floats), rstd_bits, S_bits,
    q and q_swapped (K codes)."""
    cases, cur = [], None

    def expand(rest, k, conv):
        vals = None
        for a in rest:
            i, v = a.split("=")
            if i == "default":
                vals = [conv(v)] * k
            else:
                vals[int(i)] = conv(v)
        return vals

    with open(os.path.join(GOLDEN, "rmsnorm_cases.txt")) as f:
        for ln in f:
            ln = ln.split("#")[0].strip()
            if not ln:
                continue
            key, *rest = ln.split()
            if key == "case":
                cur = {"name": rest[0]}
                cases.append(cur)
            elif key == "K":
                cur["K"] = int(rest[0])
            elif key == "eps":
                cur["eps"] = float(rest[0])
            elif key in ("x", "gamma"):
                cur[key] = expand(rest, cur["K"], parse_float)
            elif key in ("q", "q_swapped"):
                cur[key] = expand(rest, cur["K"], lambda v: int(v, 16))
            elif key in ("rstd_bits", "S_bits"):
                cur[key] = int(rest[0], 16)
    return cases
