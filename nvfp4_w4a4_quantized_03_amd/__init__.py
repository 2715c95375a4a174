"""NVFP4 W4A4 hot path for MI355X (gfx950): Python binding.

A thin ctypes layer over libnvfp4_w4a4.so (C ABI in include/nvfp4_w4a4.h).
It only marshals arguments: torch tensors provide device memory and the
current HIP stream; every step of the computation runs in the library's
HIP kernels.  Importing works without a GPU; calling needs the built library
and a GPU, and fails loudly otherwise.

    q = quantize(x)                        # NVFP4(codes, scales, global_scale)
    q = quantize(x, global_scale=g)        # calibrated static global
    g_star = harmonize_group(scales, k, row_offsets, module_globals)
    y = gemm(a, b, out_dtype=torch.bfloat16, epilogue="none")
"""
import ctypes
import os
from collections import namedtuple

import torch

__all__ = ["NVFP4", "quantize", "harmonize_group", "gemm", "gemm_quantize_a",
           "gdn_gates",
           "dequantize", "fp8_kv_calibrate", "fp8_kv_cast",
           "fake_quantize", "error_stats", "library",
           "LIB_PATH", "NVFP4Error"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)),
                        "libnvfp4_w4a4.so")

# Enumerations of the C ABI.
DTYPE_F32, DTYPE_BF16 = 0, 1
GLOBAL_COMPUTE, GLOBAL_GIVEN = 0, 1
EPILOGUES = {"none": 0, "alpha": 1, "beta": 2}

NVFP4 = namedtuple("NVFP4", ["codes", "scales", "global_scale"])
NVFP4.__doc__ = """A packed NVFP4 tensor: codes uint8 [rows, k/2] (element 2j
in the low nibble of byte j), scales uint8 [rows, k/16] (OCP E4M3), and
global_scale float32 [1] (decode scale: value = e2m1 * e4m3 * g)."""


class NVFP4Error(RuntimeError):
    """A nonzero nvfp4_status returned by the library."""


_lib = None


def library():
    """Load libnvfp4_w4a4.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            "libnvfp4_w4a4.so is not built (expected at %s); run "
            "python -c 'import __graft_entry__; __graft_entry__.build()'"
            % LIB_PATH)
    L = ctypes.CDLL(LIB_PATH)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    L.nvfp4_quantize.argtypes = [vp, i32, i64, i64, i64, vp, vp, vp, i32, vp]
    L.nvfp4_quantize.restype = i32
    L.nvfp4_harmonize_group.argtypes = [vp, i64, ctypes.POINTER(i64), i32,
                                        vp, vp, vp]
    L.nvfp4_harmonize_group.restype = i32
    L.w4a4_gemm.argtypes = [vp, vp, vp, i64, vp, vp, vp, i64, i64, vp, i32,
                            i64, i32, vp]
    L.w4a4_gemm.restype = i32
    L.w4a4_gemm_gdn_gates.argtypes = [vp, vp, vp, i64, vp, vp, vp, i64, i64,
                                      i64, vp, vp, vp, i64, vp, i64, vp]
    L.w4a4_gemm_gdn_gates.restype = i32
    L.fp8_kv_amax_update.argtypes = [vp, i32, i64, i64, i64, vp, vp]
    L.fp8_kv_amax_update.restype = i32
    L.fp8_kv_scale_from_amax.argtypes = [vp, vp, vp]
    L.fp8_kv_scale_from_amax.restype = i32
    L.fp8_kv_cast.argtypes = [vp, i32, i64, i64, i64, vp, vp, i64, vp]
    L.fp8_kv_cast.restype = i32
    L.w4a4_gemm_quantize_a.argtypes = [vp, i32, i64, i64, i64, vp, vp, vp, i32,
                                       vp, vp, vp, i64, vp, i32, i64, vp]
    L.w4a4_gemm_quantize_a.restype = i32
    L.nvfp4_dequantize.argtypes = [vp, vp, vp, i64, i64, vp, i32, i64, vp]
    L.nvfp4_dequantize.restype = i32
    L.nvfp4_error_stats.argtypes = [vp, i32, i64, i64, i64, vp, vp, vp, vp,
                                    vp]
    L.nvfp4_error_stats.restype = i32
    L.nvfp4_status_string.argtypes = [i32]
    L.nvfp4_status_string.restype = ctypes.c_char_p
    L.nvfp4_abi_version.argtypes = []
    L.nvfp4_abi_version.restype = i32
    _lib = L
    return L


def _check(rc, what=""):
    if rc != 0:
        raise NVFP4Error(library().nvfp4_status_string(rc).decode() +
                         (" [%s]" % what if what else ""))


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _device_tensor(t, name, dtype=None, numel=None, device=None):
    """Refuse anything but a GPU tensor (optionally of one dtype, element
    count and device) before any pointer reaches the library: a host or
    mistyped buffer would otherwise be read or written by a kernel."""
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError("%s must be a torch tensor on a GPU" % name)
    if dtype is not None and t.dtype != dtype:
        raise ValueError("%s must be %s, not %s" % (name, dtype, t.dtype))
    if numel is not None and t.numel() != numel:
        raise ValueError("%s must hold %d element(s), not %d"
                         % (name, numel, t.numel()))
    if device is not None and t.device != device:
        raise ValueError("%s is on %s, the other operands on %s"
                         % (name, t.device, device))


def _global_tensor(t, name, device):
    """A float32 device scalar (one element) on the operands' device."""
    _device_tensor(t, name, torch.float32, 1, device)


def quantize(x, global_scale=None, out=None):
    """NVFP4-quantise a [rows, k] float32 or bfloat16 GPU tensor.

    global_scale=None: the tensor's own global g = fp32(amax / 2688) is
    computed on the device (self-calibration).  Otherwise global_scale is a
    float32 GPU tensor of one element used as given (a calibrated static
    global).  out=(codes, scales) lets the caller pick the output buffers
    (for example row slices of a fused weight).  Returns NVFP4.
    """
    _device_tensor(x, "x")
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with unit stride along k")
    if x.dtype == torch.float32:
        dt = DTYPE_F32
    elif x.dtype == torch.bfloat16:
        dt = DTYPE_BF16
    else:
        raise ValueError("x must be float32 or bfloat16")
    rows, k = x.shape
    # a one-row tensor's row stride is arbitrary (numpy/torch may report 0)
    ldx = x.stride(0) if rows > 1 else k
    # every caller-supplied buffer is checked before anything is allocated
    if global_scale is not None:
        _global_tensor(global_scale, "global_scale", x.device)
    if out is not None:
        codes, scales = out
        _device_tensor(codes, "out codes", torch.uint8, device=x.device)
        _device_tensor(scales, "out scales", torch.uint8, device=x.device)
        if codes.shape != (rows, k // 2) or scales.shape != (rows, k // 16) \
                or not codes.is_contiguous() or not scales.is_contiguous():
            raise ValueError("out buffers have the wrong shape or layout")
    else:
        codes = torch.empty((rows, k // 2), dtype=torch.uint8, device=x.device)
        scales = torch.empty((rows, k // 16), dtype=torch.uint8,
                             device=x.device)
    if global_scale is None:
        g = torch.empty(1, dtype=torch.float32, device=x.device)
        mode = GLOBAL_COMPUTE
    else:
        g = global_scale
        mode = GLOBAL_GIVEN
    _check(library().nvfp4_quantize(_ptr(x), dt, rows, k, ldx,
                                    _ptr(codes), _ptr(scales), _ptr(g), mode,
                                    _stream(x)),
           "quantize x=%#x dtype=%d rows=%d k=%d ldx=%d codes=%#x "
           "scales=%#x global=%#x" % (x.data_ptr(), dt, rows, k, ldx,
                                      codes.data_ptr(), scales.data_ptr(),
                                      g.data_ptr()))
    return NVFP4(codes, scales, g)


def harmonize_group(scales, k, row_offsets, module_globals,
                    shared_global=None):
    """Rewrite the scales of a fused group in place to one shared global.

    scales: uint8 GPU tensor [n_total, k/16]; module i owns rows
    row_offsets[i]:row_offsets[i+1] (a host sequence of ints starting at 0);
    module_globals: float32 GPU tensor [n_modules].  Returns the shared
    global (float32 GPU tensor [1]).
    """
    _device_tensor(scales, "scales", torch.uint8)
    n_mod = len(row_offsets) - 1
    _device_tensor(module_globals, "module_globals", torch.float32, n_mod,
                   scales.device)
    if not module_globals.is_contiguous():
        raise ValueError("module_globals must be float32 [n_modules]")
    if not scales.is_contiguous() or \
            scales.shape != (row_offsets[-1], k // 16):
        raise ValueError("scales must be contiguous uint8 [n_total, k/16]")
    if shared_global is None:
        shared_global = torch.empty(1, dtype=torch.float32,
                                    device=scales.device)
    else:
        _global_tensor(shared_global, "shared_global", scales.device)
    offs = (ctypes.c_int64 * (n_mod + 1))(*[int(v) for v in row_offsets])
    _check(library().nvfp4_harmonize_group(_ptr(scales), k, offs, n_mod,
                                           _ptr(module_globals),
                                           _ptr(shared_global),
                                           _stream(scales)))
    return shared_global


def gemm(a, b, out_dtype=torch.bfloat16, epilogue="none", out=None):
    """Y = g_a g_b * A_hat B_hat^T for NVFP4 operands a [m, k] and b [n, k]
    (weights, K-major).  epilogue: "none", "alpha" (exp(-softplus(y))) or
    "beta" (sigmoid(y)).  Returns a [m, n] float32 or bfloat16 tensor."""
    ac, as_, ag = _nvfp4_parts(a, "a")
    bc, bs, bg = _nvfp4_parts(b, "b", ac.device)
    m, k = ac.shape[0], ac.shape[1] * 2
    n = bc.shape[0]
    if bc.shape[1] * 2 != k or as_.shape != (m, k // 16) or \
            bs.shape != (n, k // 16):
        raise ValueError("operand shapes disagree")
    if out_dtype == torch.float32:
        od = DTYPE_F32
    elif out_dtype == torch.bfloat16:
        od = DTYPE_BF16
    else:
        raise ValueError("out_dtype must be float32 or bfloat16")
    if epilogue not in EPILOGUES:
        raise ValueError("epilogue must be one of %s" % sorted(EPILOGUES))
    if out is None:
        out = torch.empty((m, n), dtype=out_dtype, device=ac.device)
    else:
        _device_tensor(out, "out", out_dtype, device=ac.device)
        if out.dim() != 2 or out.shape != (m, n) or out.stride(1) != 1:
            raise ValueError("out has the wrong shape or layout")
    _check(library().w4a4_gemm(_ptr(ac), _ptr(as_), _ptr(ag), m, _ptr(bc),
                               _ptr(bs), _ptr(bg), n, k, _ptr(out), od,
                               out.stride(0) if m > 1 else n,
                               EPILOGUES[epilogue],
                               _stream(ac)))
    return out


def gemm_quantize_a(x, w, global_scale=None, out_dtype=torch.bfloat16,
                    out=None):
    """Small-M (rows <= 64) activation quantisation and W4A4 GEMM in one
    launch: quantize(x, global_scale), then gemm(that, w).  x: float32 or
    bfloat16 GPU tensor [m, k] (k % 128 == 0); w: NVFP4 weights [n, k].
    global_scale as for quantize (None: self-calibrated).  Returns
    (NVFP4 of x, Y [m, n] of out_dtype), both bit-identical to the two
    separate calls."""
    dt, m, k, ldx = _x_args(x)
    wc, ws, wg = _nvfp4_parts(w, "w", x.device)
    n = wc.shape[0]
    if wc.shape[1] * 2 != k or ws.shape != (n, k // 16):
        raise ValueError("operand shapes disagree")
    od = {torch.float32: DTYPE_F32, torch.bfloat16: DTYPE_BF16}.get(out_dtype)
    if od is None:
        raise ValueError("out_dtype must be float32 or bfloat16")
    if global_scale is not None:
        _global_tensor(global_scale, "global_scale", x.device)
    if out is not None:
        _device_tensor(out, "out", out_dtype, device=x.device)
        if out.dim() != 2 or out.shape != (m, n) or out.stride(1) != 1:
            raise ValueError("out has the wrong shape or layout")
    codes = torch.empty((m, k // 2), dtype=torch.uint8, device=x.device)
    scales = torch.empty((m, k // 16), dtype=torch.uint8, device=x.device)
    if global_scale is None:
        g = torch.empty(1, dtype=torch.float32, device=x.device)
        mode = GLOBAL_COMPUTE
    else:
        g = global_scale
        mode = GLOBAL_GIVEN
    if out is None:
        out = torch.empty((m, n), dtype=out_dtype, device=x.device)
    _check(library().w4a4_gemm_quantize_a(
        _ptr(x), dt, m, k, ldx, _ptr(codes), _ptr(scales), _ptr(g), mode,
        _ptr(wc), _ptr(ws), _ptr(wg), n, _ptr(out), od,
        out.stride(0) if m > 1 else n, _stream(x)),
        "gemm_quantize_a m=%d n=%d k=%d" % (m, n, k))
    return NVFP4(codes, scales, g), out


def _nvfp4_parts(q, name, device=None):
    """Codes (uint8 [rows, k/2]), scales (uint8 [rows, k/16]) and global
    (float32 [1]) of an NVFP4 operand, checked to be contiguous GPU tensors
    of those types on one device (`device` when given)."""
    codes, scales, g = q
    _device_tensor(codes, name + ".codes", torch.uint8, device=device)
    device = codes.device
    _device_tensor(scales, name + ".scales", torch.uint8, device=device)
    _global_tensor(g, name + ".global_scale", device)
    for t, nm in ((codes, name + ".codes"), (scales, name + ".scales")):
        if t.dim() != 2 or not t.is_contiguous():
            raise ValueError("%s must be a contiguous 2-D tensor" % nm)
    return codes, scales, g


def dequantize(q, out_dtype=torch.bfloat16, out=None):
    """Values of an NVFP4 tensor q ([rows, k]): sign * E2M1 * E4M3 * g,
    each rounded once to out_dtype (float32 or bfloat16).  Returns a
    [rows, k] GPU tensor (or fills out, which may be a row-strided view)."""
    codes, scales, g = _nvfp4_parts(q, "q")
    rows, k = codes.shape[0], codes.shape[1] * 2
    od = {torch.float32: DTYPE_F32, torch.bfloat16: DTYPE_BF16}.get(out_dtype)
    if od is None:
        raise ValueError("out_dtype must be float32 or bfloat16")
    if out is None:
        out = torch.empty((rows, k), dtype=out_dtype, device=codes.device)
    else:
        _device_tensor(out, "out", out_dtype, device=codes.device)
        if out.dim() != 2 or out.shape != (rows, k) or out.stride(1) != 1:
            raise ValueError("out must be [rows, k] of out_dtype with unit "
                             "column stride")
    ldo = out.stride(0) if rows > 1 else k
    _check(library().nvfp4_dequantize(_ptr(codes), _ptr(scales), _ptr(g), rows,
                                      k, _ptr(out), od, ldo, _stream(codes)),
           "dequantize rows=%d k=%d ldo=%d" % (rows, k, ldo))
    return out


def fake_quantize(x, global_scale=None, out_dtype=None):
    """Quantise then dequantise ([P1] 접근 방법: exactly the 4-bit rounding
    error, nothing else).  Two launches: nvfp4_quantize and
    nvfp4_dequantize.  out_dtype defaults to x's dtype."""
    q = quantize(x, global_scale)
    return dequantize(q, out_dtype or x.dtype)


def error_stats(x, q):
    """Per-row float64 statistics of x and of its NVFP4 form q:
    [rows, 3] = (sum x^2, sum (x - x_hat)^2, max |x|), x_hat the exact
    dequantised value.  Relative error = sqrt(sum col 1 / sum col 0);
    max/RMS of a row = col 2 / sqrt(col 0 / k)."""
    _device_tensor(x, "x")
    codes, scales, g = _nvfp4_parts(q, "q", x.device)
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with unit stride along k")
    dt = {torch.float32: DTYPE_F32, torch.bfloat16: DTYPE_BF16}.get(x.dtype)
    if dt is None:
        raise ValueError("x must be float32 or bfloat16")
    rows, k = x.shape
    if codes.shape != (rows, k // 2) or scales.shape != (rows, k // 16):
        raise ValueError("q does not match x's shape")
    ldx = x.stride(0) if rows > 1 else k
    stats = torch.empty((rows, 3), dtype=torch.float64, device=x.device)
    _check(library().nvfp4_error_stats(_ptr(x), dt, rows, k, ldx, _ptr(codes),
                                       _ptr(scales), _ptr(g), _ptr(stats),
                                       _stream(x)),
           "error_stats rows=%d k=%d ldx=%d" % (rows, k, ldx))
    return stats


def gdn_gates(x, w_ba, n_beta, a_log, dt_bias, out=None):
    """Gate pair of a Gated DeltaNet layer from its fused b|a projection:
    w_ba is the NVFP4 weight [W_b; W_a] (n_beta + n_alpha rows, one shared
    global), x the NVFP4 activations [m, k].  Returns (beta [m, n_beta],
    alpha [m, n_alpha]) float32 with beta = sigmoid(b) and
    alpha = exp(-exp(A_log) * softplus(a + dt_bias)); a_log and dt_bias are
    float32 GPU tensors [n_alpha].  out=(beta, alpha) supplies buffers."""
    xc, xs, xg = _nvfp4_parts(x, "x")
    wc, ws, wg = _nvfp4_parts(w_ba, "w_ba", xc.device)
    m, k = xc.shape[0], xc.shape[1] * 2
    n = wc.shape[0]
    n_alpha = n - n_beta
    if wc.shape[1] * 2 != k or not 0 <= n_beta <= n:
        raise ValueError("x and w_ba disagree in k, or n_beta is out of range")
    for t, nm in ((a_log, "a_log"), (dt_bias, "dt_bias")):
        _device_tensor(t, nm, torch.float32, n_alpha, xc.device)
        if not t.is_contiguous():
            raise ValueError("%s must be float32 [n_alpha]" % nm)
    if out is None:
        beta = torch.empty((m, n_beta), dtype=torch.float32, device=xc.device)
        alpha = torch.empty((m, n_alpha), dtype=torch.float32, device=xc.device)
    else:
        beta, alpha = out
    for t, nm, cols in ((beta, "beta", n_beta), (alpha, "alpha", n_alpha)):
        _device_tensor(t, nm, torch.float32, device=xc.device)
        if t.dim() != 2 or t.shape != (m, cols) or t.stride(1) != 1:
            raise ValueError("%s must be float32 [m, %d] with unit column stride" % (nm, cols))
    ldb = beta.stride(0) if m > 1 else max(n_beta, 1)
    lda = alpha.stride(0) if m > 1 else max(n_alpha, 1)
    _check(library().w4a4_gemm_gdn_gates(
        _ptr(xc), _ptr(xs), _ptr(xg), m, _ptr(wc), _ptr(ws), _ptr(wg), n_beta,
        n_alpha, k, _ptr(a_log), _ptr(dt_bias),
        _ptr(beta) if n_beta else None, ldb,
        _ptr(alpha) if n_alpha else None, lda, _stream(xc)),
        "gdn_gates m=%d n_beta=%d n_alpha=%d k=%d" % (m, n_beta, n_alpha, k))
    return beta, alpha


def _x_args(x, name="x", device=None):
    _device_tensor(x, name, device=device)
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("%s must be 2-D with unit stride along k" % name)
    dt = {torch.float32: DTYPE_F32, torch.bfloat16: DTYPE_BF16}.get(x.dtype)
    if dt is None:
        raise ValueError("%s must be float32 or bfloat16" % name)
    rows, k = x.shape
    return dt, rows, k, (x.stride(0) if rows > 1 else k)


def fp8_kv_calibrate(tensors, amax=None):
    """Static per-tensor FP8 KV scale from calibration tensors (float32 or
    bfloat16 GPU tensors [rows, k]): the running max |x| is accumulated on
    the device (pass amax, a float32 [1] GPU tensor, to continue an earlier
    calibration), then scale = fp32(amax / 448).  Returns (scale, amax)."""
    first = tensors[0]
    _device_tensor(first, "calibration tensor")
    args = [_x_args(t, "calibration tensor", first.device) for t in tensors]
    if amax is None:
        amax = torch.zeros(1, dtype=torch.float32, device=first.device)
    else:
        _global_tensor(amax, "amax", first.device)
    for t, (dt, rows, k, ldx) in zip(tensors, args):
        _check(library().fp8_kv_amax_update(_ptr(t), dt, rows, k, ldx, _ptr(amax),
                                            _stream(t)), "fp8_kv_amax_update")
    scale = torch.empty(1, dtype=torch.float32, device=first.device)
    _check(library().fp8_kv_scale_from_amax(_ptr(amax), _ptr(scale), _stream(first)),
           "fp8_kv_scale_from_amax")
    return scale, amax


def fp8_kv_cast(x, scale, out=None):
    """OCP E4M3 codes (uint8 [rows, k]) of x under the static decode scale
    (float32 [1] GPU tensor): sign | E4M3(|x| / scale), one rounding."""
    dt, rows, k, ldx = _x_args(x)
    _global_tensor(scale, "scale", x.device)
    if out is None:
        out = torch.empty((rows, k), dtype=torch.uint8, device=x.device)
    else:
        _device_tensor(out, "out", torch.uint8, device=x.device)
        if out.dim() != 2 or out.shape != (rows, k) or out.stride(1) != 1:
            raise ValueError("out must be uint8 [rows, k] with unit column "
                             "stride")
    ldo = out.stride(0) if rows > 1 else k
    _check(library().fp8_kv_cast(_ptr(x), dt, rows, k, ldx, _ptr(scale), _ptr(out),
                                 ldo, _stream(x)),
           "fp8_kv_cast rows=%d k=%d ldx=%d ldo=%d" % (rows, k, ldx, ldo))
    return out
