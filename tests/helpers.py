"""Small helpers shared by the tests (no product or oracle arithmetic)."""
from __future__ import annotations

import os

import numpy as np
from numpy.lib.stride_tricks import as_strided

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def view(storage: np.ndarray, batch: int, rows: int, cols: int, strides) -> np.ndarray:
    """Read-only [batch, rows, cols] numpy view of a flat float32 storage
    under element strides (batch, row, col)."""
    return as_strided(storage, (batch, rows, cols), tuple(4 * int(s) for s in strides),
                      writeable=False)


def load_golden(name: str) -> dict:
    """Parse a `key: value` fixture; '#' lines are the citation and comments."""
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, _, val = line.partition(":")
            out[key.strip()] = val.strip()
    return out


def ints(text: str):
    return [int(t) for t in text.split()]


def floats(text: str):
    return [float(t) for t in text.split()]


def column_major_strides(ld: int):
    """(row, col) element strides of a column-major matrix with leading
    dimension `ld`: element (r, c) sits at r + c*ld."""
    return (1, ld)


def view4(storage: np.ndarray, shape, strides) -> np.ndarray:
    """Read-only 4-D numpy view of a flat float32 storage under element
    strides (two batch levels, then row and column)."""
    return as_strided(storage, tuple(int(s) for s in shape), tuple(4 * int(s) for s in strides),
                      writeable=False)
