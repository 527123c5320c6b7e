"""Reader of ``golden/quantize_examples.txt`` (hand-worked quantisation cases)."""
from __future__ import annotations

import os
from dataclasses import dataclass, field

import numpy as np

import exact

_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "quantize_examples.txt")


@dataclass
class Case:
    name: str
    fmt: str
    rule: str
    K: int
    x: dict = field(default_factory=dict)        # position -> float
    sf: list = field(default_factory=list)       # one byte per block
    packed: list = field(default_factory=list)   # int16 words (as unsigned)
    codes: dict = field(default_factory=dict)    # e4m3: element -> code; e2m1: byte -> byte

    def x_bits(self) -> np.ndarray:
        row = np.zeros((1, self.K), dtype=np.uint16)
        for pos, v in self.x.items():
            row[0, pos] = exact.bf16_bits(v)
        return row

    def expected_codes(self) -> np.ndarray:
        width = self.K if self.fmt == "e4m3" else self.K // 2
        row = np.zeros((1, width), dtype=np.uint8)
        for pos, c in self.codes.items():
            row[0, pos] = c
        return row


def _float(tok: str) -> float:
    t = tok.lstrip("+-")
    if t.startswith("0x"):
        v = float.fromhex(t)
        return -v if tok.startswith("-") else v
    return float(tok)


def cases() -> list[Case]:
    out, cur = [], None
    with open(_PATH) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            tok = line.split()
            if tok[0] == "case":
                cur = Case(tok[1], tok[2], tok[3], int(tok[4]))
            elif tok[0] == "x":
                cur.x[int(tok[1])] = _float(tok[2])
            elif tok[0] == "sf":
                cur.sf = [int(t, 16) for t in tok[1:]]
            elif tok[0] == "packed":
                cur.packed = [int(t, 16) for t in tok[1:]]
            elif tok[0] in ("code", "byte"):
                cur.codes[int(tok[1])] = int(tok[2], 16)
            elif tok[0] == "end":
                out.append(cur)
                cur = None
            else:
                raise ValueError(f"bad fixture line: {line}")
    return out
