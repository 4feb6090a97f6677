"""Parsers for the hand-written fixtures under tests/golden/."""

from __future__ import annotations

import os
import re

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for raw in f:
            line = raw.split("#", 1)[0].strip()
            if line:
                yield line


def e4m3_points():
    """[(code, value)] from e4m3fn_points.txt."""
    out = []
    for line in _lines("e4m3fn_points.txt"):
        code, val = line.split()
        out.append((int(code, 16), float(val)))
    return out


def _expand_runs(text):
    codes = []
    for m in re.finditer(r"\(([^)]*)\)\*(\d+)|(0x[0-9A-Fa-f]+)\*(\d+)", text):
        if m.group(1) is not None:
            group = [int(t, 16) for t in m.group(1).split()]
            codes += group * int(m.group(2))
        else:
            codes += [int(m.group(3), 16)] * int(m.group(4))
    return codes


def worked_gemm():
    """The hand-worked GEMM example: dict with g, a8, b8, sa, sb, ref, bf16."""
    kv = {}
    for line in _lines("worked_gemm_g64.txt"):
        key, rest = line.split(None, 1)
        kv[key] = rest
    g, M, N, K = (int(kv[k]) for k in ("g", "M", "N", "K"))
    a8 = np.array([_expand_runs(kv["A%d" % i]) for i in range(M)], dtype=np.uint8)
    b8 = np.array([_expand_runs(kv["B%d" % j]) for j in range(N)], dtype=np.uint8)
    assert a8.shape == (M, K) and b8.shape == (N, K)
    sa = np.array([float(t) for t in kv["sa"].split()], dtype=np.float32).reshape(1, K // g)
    sb = np.array([float(t) for t in kv["sb"].split()], dtype=np.float32).reshape(1, K // g)
    ref = np.array([float(t) for t in kv["ref"].split()]).reshape(M, N)
    bf16 = np.array([float(t) for t in kv["bf16"].split()]).reshape(M, N)
    return dict(g=g, M=M, N=N, K=K, a8=a8, b8=b8, sa=sa, sb=sb, ref=ref, bf16=bf16)


def worked_quant():
    """The hand-worked quantisation example: dict with g, x, codes, scale."""
    head = {}
    entries = []
    for line in _lines("worked_quant_g64.txt"):
        parts = line.split()
        if len(parts) == 2:
            head[parts[0]] = parts[1]
        else:
            entries.append((int(parts[0]), int(parts[1]), float(parts[2]), int(parts[3], 16)))
    rows, cols = int(head["rows"]), int(head["cols"])
    x = np.zeros((rows, cols), dtype=np.float32)
    codes = np.zeros((rows, cols), dtype=np.uint8)
    for r, c, v, code in entries:
        x[r, c] = v
        codes[r, c] = code
    return dict(g=int(head["g"]), x=x, codes=codes, scale=float(head["scale"]))
