"""Small helpers shared by the test modules (no method arithmetic here)."""
from __future__ import annotations

import numpy as np


def ulp_dist_bf16(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """|ord(a) - ord(b)| for bf16 bit patterns on a monotone integer line (+-0 -> 0)."""
    def ordv(h):
        h = np.asarray(h).astype(np.int64)
        return np.where(h & 0x8000, -(h & 0x7FFF), h & 0x7FFF)
    return np.abs(ordv(a) - ordv(b))


def sweep_rows(exponents, pad_to=None):
    """Rows [a, x...] for every bf16 mantissa of a in each given binade and every
    bf16 x with |x| <= a in the 9 binades that can give a nonzero code (both
    signs, bf16 subnormals included where the binade reaches them); entries
    with |x| > a are replaced by 0.  Returns uint16 [len(exponents)*128, C]."""
    out = []
    for E in exponents:
        a_bits = (np.uint32(E) << 7) | np.arange(128, dtype=np.uint32)
        es = np.arange(E - 8, E + 1)
        es = es[es >= 0]
        cand = ((es[:, None].astype(np.uint32) << 7) | np.arange(128, dtype=np.uint32)[None, :]).ravel()
        keep = cand[None, :] <= a_bits[:, None]
        pos = np.where(keep, cand[None, :], 0)
        neg = np.where(keep, cand[None, :] | 0x8000, 0)
        rows = np.concatenate([a_bits[:, None], pos, neg], axis=1)
        width = 1 + 2 * 9 * 128
        if rows.shape[1] < width:
            rows = np.pad(rows, ((0, 0), (0, width - rows.shape[1])))
        out.append(rows)
    r = np.concatenate(out, axis=0).astype(np.uint16)
    if pad_to is not None and pad_to > r.shape[1]:
        r = np.pad(r, ((0, 0), (0, pad_to - r.shape[1])))
    return r
