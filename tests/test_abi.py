"""The C-ABI library loads, exports every symbol the header declares, and
rejects invalid arguments on the host before any device work.  Runs on the
CPU: every call below is invalid in at least one argument, so nothing is
ever launched."""
import ctypes
import os
import re

import pytest

import nvfp4_w4a4_quantized_03_amd as nv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nvfp4_w4a4.h")

OK, INVALID, UNSUPPORTED, MISALIGNED = 0, 1, 2, 3
P = 0x7F0000000000          # a 256-byte aligned fake address, never touched


def _declared_functions():
    text = open(HEADER).read()
    return re.findall(r"^\s*(?:int|const char\*)\s+(\w+)\s*\(", text,
                      re.MULTILINE)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(nv.LIB_PATH):
        pytest.fail("library not built: run __graft_entry__.build()")
    return nv.library()


def test_exports_every_declared_symbol(lib):
    names = _declared_functions()
    assert set(names) >= {"nvfp4_quantize", "nvfp4_harmonize_group",
                          "w4a4_gemm", "w4a4_gemm_gdn_gates",
                          "nvfp4_dequantize", "fp8_kv_amax_update",
                          "fp8_kv_scale_from_amax", "fp8_kv_cast",
                          "nvfp4_error_stats", "nvfp4_status_string",
                          "nvfp4_abi_version", "w4a4_gemm_quantize_a"}
    for name in names:
        assert hasattr(lib, name), name
    assert lib.nvfp4_abi_version() == 3
    for s in range(6):
        assert lib.nvfp4_status_string(s)


def q(lib, x=P, dt=1, rows=4, k=32, ldx=32, codes=P + 0x100000,
      scales=P + 0x200000, g=P + 0x300000, mode=0):
    return lib.nvfp4_quantize(x, dt, rows, k, ldx, codes, scales, g, mode,
                              None)


def test_quantize_validation(lib):
    assert q(lib, x=None) == INVALID
    assert q(lib, codes=None) == INVALID
    assert q(lib, scales=None) == INVALID
    assert q(lib, g=None) == INVALID
    assert q(lib, rows=0) == INVALID
    assert q(lib, k=0, ldx=0) == INVALID
    assert q(lib, k=24, ldx=24) == INVALID            # k % 16 != 0
    assert q(lib, ldx=16) == INVALID                  # ldx < k
    assert q(lib, rows=1 << 41) == INVALID
    assert q(lib, dt=7) == UNSUPPORTED
    assert q(lib, mode=5) == UNSUPPORTED
    assert q(lib, x=P + 8) == MISALIGNED              # x not 16-byte aligned
    assert q(lib, ldx=36) == MISALIGNED               # bf16 row stride 72 B
    assert q(lib, codes=P + 0x100004) == MISALIGNED
    assert q(lib, g=P + 0x300002) == MISALIGNED
    assert q(lib, codes=P + 16) == INVALID            # codes overlap x
    assert q(lib, scales=P + 0x100010) == INVALID     # scales overlap codes


def h(lib, scales=P, k=64, offs=(0, 8, 12), glob=P + 0x100000,
      shared=P + 0x200000):
    arr = (ctypes.c_int64 * len(offs))(*offs)
    return lib.nvfp4_harmonize_group(scales, k, arr, len(offs) - 1, glob,
                                     shared, None)


def test_harmonize_validation(lib):
    assert h(lib, scales=None) == INVALID
    assert h(lib, glob=None) == INVALID
    assert h(lib, shared=None) == INVALID
    assert h(lib, k=40) == INVALID
    assert h(lib, offs=(1, 8, 12)) == INVALID         # must start at 0
    assert h(lib, offs=(0, 8, 8)) == INVALID          # empty module
    assert h(lib, offs=(0,)) == INVALID               # no module
    assert h(lib, offs=tuple(range(0, 66))) == INVALID  # > 64 modules
    assert h(lib, shared=P + 0x100000) == INVALID     # aliases the globals
    assert h(lib, shared=P + 4) == INVALID            # inside the scales
    assert h(lib, glob=P + 0x100002) == MISALIGNED
    assert h(lib, scales=P + 1) == MISALIGNED         # scales not 16-byte aligned
    assert h(lib, scales=P + 8) == MISALIGNED
    assert lib.nvfp4_harmonize_group(P, 64, None, 1, P + 0x100000,
                                     P + 0x200000, None) == INVALID


def gm(lib, a=P, sa=P + 0x100000, ga=P + 0x200000, m=4, b=P + 0x300000,
       sb=P + 0x400000, gb=P + 0x500000, n=8, k=64, out=P + 0x600000, od=0,
       ldo=8, epi=0):
    return lib.w4a4_gemm(a, sa, ga, m, b, sb, gb, n, k, out, od, ldo, epi,
                         None)


def test_gemm_validation(lib):
    for kw in ("a", "sa", "ga", "b", "sb", "gb", "out"):
        assert gm(lib, **{kw: None}) == INVALID, kw
    assert gm(lib, m=0) == INVALID
    assert gm(lib, n=0) == INVALID
    assert gm(lib, k=8) == INVALID
    assert gm(lib, k=72) == INVALID
    assert gm(lib, ldo=4) == INVALID                  # ldo < n
    assert gm(lib, m=1 << 41) == INVALID
    assert gm(lib, od=3) == UNSUPPORTED
    assert gm(lib, epi=9) == UNSUPPORTED
    assert gm(lib, a=P + 8) == MISALIGNED
    assert gm(lib, b=P + 0x300008) == MISALIGNED
    assert gm(lib, sa=P + 0x100001) == MISALIGNED     # scale arrays 16-byte aligned
    assert gm(lib, sb=P + 0x400008) == MISALIGNED
    assert gm(lib, out=P + 0x600002) == MISALIGNED
    assert gm(lib, out=P + 0x300010) == INVALID       # out overlaps b codes
    assert gm(lib, out=P + 0x200000 - 8) == INVALID   # out covers a_global


def fq(lib, x=P, dt=1, m=4, k=256, ldx=256, xc=P + 0x100000, xs=P + 0x200000,
       xg=P + 0x300000, mode=0, wc=P + 0x400000, ws=P + 0x500000,
       wg=P + 0x600000, n=8, out=P + 0x700000, od=1, ldo=8):
    return lib.w4a4_gemm_quantize_a(x, dt, m, k, ldx, xc, xs, xg, mode, wc, ws,
                                    wg, n, out, od, ldo, None)


def test_gemm_quantize_a_validation(lib):
    for kw in ("x", "xc", "xs", "xg", "wc", "ws", "wg", "out"):
        assert fq(lib, **{kw: None}) == INVALID, kw
    assert fq(lib, m=0) == INVALID
    assert fq(lib, n=0) == INVALID
    assert fq(lib, k=8, ldx=8) == INVALID
    assert fq(lib, ldx=128) == INVALID                # ldx < k
    assert fq(lib, ldo=4) == INVALID                  # ldo < n
    assert fq(lib, dt=5) == UNSUPPORTED
    assert fq(lib, mode=2) == UNSUPPORTED
    assert fq(lib, od=3) == UNSUPPORTED
    assert fq(lib, m=65) == UNSUPPORTED               # not a small-M shape
    assert fq(lib, k=272, ldx=272) == UNSUPPORTED     # k % 128 != 0
    assert fq(lib, x=P + 8) == MISALIGNED
    assert fq(lib, xs=P + 0x200008) == MISALIGNED
    assert fq(lib, ws=P + 0x500004) == MISALIGNED
    assert fq(lib, out=P + 0x700002) == MISALIGNED
    assert fq(lib, xc=P + 0x40) == INVALID            # codes overlap x
    assert fq(lib, out=P + 0x400010) == INVALID       # out overlaps w codes
    assert fq(lib, xg=P + 0x200004) == INVALID        # global inside scales
    assert fq(lib, out=P + 0x100000 + 0x100) == INVALID   # out overlaps codes


def gg(lib, xc=P, xs=P + 0x100000, xg=P + 0x200000, m=4, wc=P + 0x300000,
       ws=P + 0x400000, wg=P + 0x500000, nb=8, na=8, k=128, al=P + 0x600000,
       dt=P + 0x700000, bo=P + 0x800000, ldb=8, ao=P + 0x900000, lda=8):
    return lib.w4a4_gemm_gdn_gates(xc, xs, xg, m, wc, ws, wg, nb, na, k, al, dt,
                                   bo, ldb, ao, lda, None)


def test_gdn_gates_validation(lib):
    for kw in ("xc", "xs", "xg", "wc", "ws", "wg", "al", "dt", "bo", "ao"):
        assert gg(lib, **{kw: None}) == INVALID, kw
    assert gg(lib, nb=0, na=0) == INVALID
    assert gg(lib, m=0) == INVALID
    assert gg(lib, nb=-1) == INVALID
    assert gg(lib, k=24) == INVALID
    assert gg(lib, ldb=4) == INVALID                  # ld_beta < n_beta
    assert gg(lib, lda=4) == INVALID
    assert gg(lib, k=192) == UNSUPPORTED              # k % 128 != 0
    assert gg(lib, nb=200, na=100, ldb=200, lda=100) == UNSUPPORTED
    assert gg(lib, xs=P + 0x100008) == MISALIGNED     # scales not 16-byte aligned
    assert gg(lib, ao=P + 0x900002) == MISALIGNED
    assert gg(lib, ao=P + 0x800010) == INVALID        # alpha overlaps beta
    assert gg(lib, bo=P + 0x300000) == INVALID        # beta over the weight codes


def dq(lib, codes=P, scales=P + 0x100000, g=P + 0x200000, rows=4, k=32,
       out=P + 0x300000, od=1, ldo=32):
    return lib.nvfp4_dequantize(codes, scales, g, rows, k, out, od, ldo, None)


def test_dequantize_validation(lib):
    for kw in ("codes", "scales", "g", "out"):
        assert dq(lib, **{kw: None}) == INVALID, kw
    assert dq(lib, rows=0) == INVALID
    assert dq(lib, k=24, ldo=24) == INVALID
    assert dq(lib, ldo=16) == INVALID                 # ldo < k
    assert dq(lib, od=4) == UNSUPPORTED
    assert dq(lib, codes=P + 4) == MISALIGNED
    assert dq(lib, out=P + 0x300008) == MISALIGNED
    assert dq(lib, ldo=36) == MISALIGNED              # bf16 row stride 72 B
    assert dq(lib, out=P + 0x100000) == INVALID       # out covers the scales


def es(lib, x=P, dt=1, rows=4, k=32, ldx=32, codes=P + 0x100000,
       scales=P + 0x200000, g=P + 0x300000, stats=P + 0x400000):
    return lib.nvfp4_error_stats(x, dt, rows, k, ldx, codes, scales, g,
                                 stats, None)


def test_error_stats_validation(lib):
    for kw in ("x", "codes", "scales", "g", "stats"):
        assert es(lib, **{kw: None}) == INVALID, kw
    assert es(lib, rows=0) == INVALID
    assert es(lib, k=40, ldx=40) == INVALID
    assert es(lib, ldx=16) == INVALID
    assert es(lib, dt=2) == UNSUPPORTED
    assert es(lib, x=P + 8) == MISALIGNED
    assert es(lib, stats=P + 0x400004) == MISALIGNED
    assert es(lib, stats=P + 0x100000) == INVALID     # stats covers codes


def kv(lib, x=P, dt=1, rows=4, k=32, ldx=32, scale=P + 0x100000,
       out=P + 0x200000, ldo=32):
    return lib.fp8_kv_cast(x, dt, rows, k, ldx, scale, out, ldo, None)


def test_fp8_kv_validation(lib):
    for kw in ("x", "scale", "out"):
        assert kv(lib, **{kw: None}) == INVALID, kw
    assert kv(lib, rows=0) == INVALID
    assert kv(lib, k=24, ldx=24, ldo=24) == INVALID
    assert kv(lib, ldo=16) == INVALID                 # ldo < k
    assert kv(lib, dt=5) == UNSUPPORTED
    assert kv(lib, x=P + 8) == MISALIGNED
    assert kv(lib, out=P + 0x200008) == MISALIGNED
    assert kv(lib, ldo=40) == MISALIGNED              # ldo % 16 != 0
    assert kv(lib, out=P + 16) == INVALID             # out overlaps x
    assert lib.fp8_kv_amax_update(P, 1, 4, 32, 32, None, None) == INVALID
    assert lib.fp8_kv_amax_update(P, 1, 4, 32, 32, P + 2, None) == MISALIGNED
    assert lib.fp8_kv_scale_from_amax(None, P, None) == INVALID
    assert lib.fp8_kv_scale_from_amax(P, P + 1, None) == MISALIGNED


def test_binding_rejects_cpu_tensors():
    import torch
    with pytest.raises(ValueError):
        nv.quantize(torch.zeros(4, 32))
