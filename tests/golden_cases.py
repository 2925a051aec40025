"""Reader for tests/golden/hand_examples.txt (hand-worked streams)."""
from __future__ import annotations

import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "hand_examples.txt")


def _input(spec: list[str]) -> bytes:
    if "concat" == spec[0]:
        rest = " ".join(spec[1:]).split(";")
        return b"".join(_input(part.split()) for part in rest)
    kind = spec[0]
    if kind == "const":
        v, n = int(spec[1]), int(spec[2])
        return np.full(n, v, dtype="<u4").tobytes()
    if kind == "ramp":
        n = int(spec[1])
        return (np.arange(n, dtype="<u4") + 1).tobytes()
    if kind == "mod":
        p, n = int(spec[1]), int(spec[2])
        return (np.arange(n, dtype="<u4") % p + 1).astype("<u4").tobytes()
    if kind == "bytes":
        head = b"" if spec[1] == "-" else bytes.fromhex(spec[1])
        pad = int(spec[2])
        return head + bytes(pad - len(head))
    raise ValueError(spec)


def _b5_payload(data: bytes) -> bytes:
    # 64 literals, then (255,40), (193,80); 66 items -> 9 flag bytes, bits 64, 65 set
    flags = bytes(8) + bytes([0x03])
    return flags + data[: 64 * 4] + bytes([255, 40, 193, 80])


def load():
    cases = []
    cur = None
    with open(GOLDEN) as fh:
        for line in fh:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, _, val = line.partition(" ")
            if key == "case":
                cur = {"name": val}
            elif key in ("cs", "ws", "level"):
                cur[key] = int(val)
            elif key == "input":
                cur["input"] = _input(val.split())
            elif key == "stream":
                parts = val.split()
                out = b""
                for p in parts:
                    if p == "+INPUT":
                        out += cur["input"]
                    elif p == "+B5PAYLOAD":
                        out += _b5_payload(cur["input"])
                    else:
                        out += bytes.fromhex(p)
                cur["stream"] = out
            elif key == "end":
                cases.append(cur)
                cur = None
    return cases


SPLIT_GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "split_examples.txt")


def _port(tokens: list[str], data: bytes) -> bytes:
    out = b""
    for p in tokens:
        if p == "-":
            continue
        if p == "+INPUT":
            out += data
        elif p == "+INPUT64W":
            out += data[: 64 * 4]
        else:
            out += bytes.fromhex(p)
    return out


def load_split():
    """Cases of tests/golden/split_examples.txt: dicts with cs, ws, level,
    input and the four ports lit / lens / offs / meta (bytes)."""
    cases, cur = [], None
    with open(SPLIT_GOLDEN) as fh:
        for line in fh:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, _, val = line.partition(" ")
            if key == "case":
                if cur is not None:
                    cases.append(cur)
                cur = {"name": val}
            elif key in ("cs", "ws", "level"):
                cur[key] = int(val)
            elif key == "input":
                cur["input"] = _input(val.split())
            elif key in ("lit", "lens", "offs", "meta"):
                cur[key] = _port(val.split(), cur["input"])
    if cur is not None:
        cases.append(cur)
    return cases
