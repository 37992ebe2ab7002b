"""Constructed activation blocks for the quantizer's rounding edge.

halfway_after_rounding(): blocks in which some elements x have an fp32
product x*id that rounds to exactly c + 1/2 while the exact product is below
c + 1/2.  Rounding the fp32 product half away from zero gives c + 1; taking
the fractional part of the unrounded product (a fused multiply-add) gives c.
"""
from __future__ import annotations

import numpy as np


def halfway_after_rounding(seed: int, n_blocks: int = 64):
    """Returns (x [n_blocks*32] fp32, hits: list of (index, expected_code))."""
    rng = np.random.default_rng(seed)
    f32 = np.float32
    x = np.zeros((n_blocks, 32), np.float32)
    hits = []
    for b in range(n_blocks):
        while True:
            amax = f32(rng.uniform(0.5, 4.0))
            d = f32(amax / f32(127.0))
            idv = f32(f32(1.0) / d)
            if idv != f32(2.0) ** np.floor(np.log2(idv)):
                break
        x[b, 0] = amax
        j = 1
        for c in rng.permutation(np.arange(2, 126)):
            if j >= 32:
                break
            h = float(c) + 0.5
            x0 = f32(h / float(idv))
            for cand in (np.nextafter(x0, f32(0)), x0, np.nextafter(x0, f32(np.inf))):
                cand = f32(cand)
                v32 = f32(cand * idv)
                v64 = float(cand) * float(idv)  # exact: 24 + 24 bits
                if float(v32) == h and v64 < h and abs(cand) < amax:
                    sgn = 1 if rng.integers(0, 2) else -1
                    x[b, j] = sgn * cand
                    hits.append((b * 32 + j, sgn * (int(c) + 1)))
                    j += 1
                    break
        # fill the rest with ordinary values below amax
        if j < 32:
            x[b, j:] = (rng.uniform(-1, 1, 32 - j) * float(amax) * 0.99).astype(np.float32)
    return x.reshape(-1), hits
