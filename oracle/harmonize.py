"""Fused-group scale harmonisation.  TEST INFRASTRUCTURE ONLY.

[P1] "접근 방법" and "개발자 관점", and the abstract on [P2]: per-module
calibrated NVFP4 checkpoints clash with serving kernels that fuse modules
(qkv|z, b|a) into one GEMM with one global scale; the fix rewrites the
per-module globals to one shared global and folds each module's ratio into
its block scales.  Readings where the pages are silent:

  * the shared global is g* = max_i g_i (the only choice under which no
    folded scale e4m3(s) * g_i / g* can exceed e4m3(s) <= 448);
  * each scale becomes RNE_SAT_E4M3(e4m3(s) * g_i / g*), the quotient exact,
    ties to even; modules with g_i == g* are left exactly as they are;
  * the 4-bit codes are not re-encoded (a checkpoint has no originals);
  * the fused weight is the row concatenation of the modules.

float64 tier exactness: e4m3(s) * g_i has <= 28 significant bits (exact in
float64); the midpoint test of the quotient against an E4M3 midpoint t
(<= 5 bits) is decided by one correctly rounded float64 division for the
same reason as in quantize.py.
"""
from fractions import Fraction

import numpy as np

from .formats import e4m3_decode, e4m3_decode_table, e4m3_rne_sat_exact
from .quantize import _rne_sat_codes

_E4M3 = e4m3_decode_table()[:127]


def harmonize(scales, row_offsets, module_globals):
    """Return (new_scales, g_star) for a fused [n_total, K/16] scale array
    whose module i owns rows row_offsets[i]:row_offsets[i+1]."""
    scales = np.asarray(scales, dtype=np.uint8)
    gs = [np.float32(g) for g in module_globals]
    if len(row_offsets) != len(gs) + 1 or row_offsets[0] != 0 \
            or row_offsets[-1] != scales.shape[0]:
        raise ValueError("row_offsets must partition the rows")
    if np.any(scales == 0x7F) or np.any(scales & 0x80):
        raise ValueError("scales must be non-negative finite E4M3")
    g_star = max(gs)
    out = scales.copy()
    for i, gi in enumerate(gs):
        r0, r1 = row_offsets[i], row_offsets[i + 1]
        if gi == g_star:
            continue
        num = _E4M3[scales[r0:r1].astype(np.int64)] * float(gi)   # exact
        v = num / float(g_star)
        out[r0:r1] = _rne_sat_codes(v, _E4M3).astype(np.uint8)
    return out, np.float32(g_star)


def harmonize_exact(scales, row_offsets, module_globals):
    """Fraction-exact version of harmonize() for small inputs."""
    scales = np.asarray(scales, dtype=np.uint8)
    gs = [Fraction(float(np.float32(g))) for g in module_globals]
    g_star = max(gs)
    out = scales.copy()
    for i, gi in enumerate(gs):
        if gi == g_star:
            continue
        for r in range(row_offsets[i], row_offsets[i + 1]):
            for j in range(scales.shape[1]):
                d = e4m3_decode(int(scales[r, j]))
                out[r, j] = e4m3_rne_sat_exact(d * gi / g_star)
    return out, np.float32(float(g_star))
