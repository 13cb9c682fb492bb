"""Thin Python binding over libmx355 (C ABI in include/mx.h).

Argument marshalling only: every step of the path runs in the HIP kernels of
libmx355.so.  PyTorch supplies device memory (tensors are passed as raw device
pointers) and the current HIP stream.  There is no fallback: if the library
or a GPU is missing, calls raise.
"""
from __future__ import annotations

import ctypes
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmx355.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "mx.h")

MX_F32, MX_BF16 = 0, 1
RNE, SR = 0, 1
# scale storage orders (include/mx.h): 2D B scales; staged ([stage][row][8 bytes]);
# column-wise groups padded to 256 tokens
SCALES_B_2D, SCALES_STAGED, GROUPS_PAD256 = 1, 2, 4
STATUS = {0: "MX_OK", 1: "MX_ERR_NULL", 2: "MX_ERR_SHAPE", 3: "MX_ERR_ALIGN",
          4: "MX_ERR_DTYPE", 5: "MX_ERR_UNSUPPORTED", 6: "MX_ERR_LAUNCH"}


class MXError(RuntimeError):
    def __init__(self, fn, code):
        super().__init__("%s returned %s" % (fn, STATUS.get(code, code)))
        self.code = code


_lib = None


def lib():
    """Load libmx355.so (built in-tree by __graft_entry__.build())."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libmx355.so is not built; run "
                               "python -m mxfp4_precision_numerics_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        P, i64, u64, u32, i32, c_int = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64,
                                        ctypes.c_uint32, ctypes.c_int32, ctypes.c_int)
        L.mx_version.restype = c_int
        L.mx_status_str.argtypes = [c_int]
        L.mx_status_str.restype = ctypes.c_char_p
        L.mx_rht_sign_mask.argtypes = [u64]
        L.mx_rht_sign_mask.restype = u32
        L.mx_rht.argtypes = [P, c_int, P, i64, i64, u32, c_int, P]
        L.mx_quantize_1d.argtypes = [P, c_int, i64, i64, c_int, P, i32, i64, P, c_int, u32, c_int,
                                     u64, u32, u64, P, i64, P, P]
        L.mx_quantize_2d.argtypes = [P, c_int, i64, i64, i64, P, i64, P, P, i64, P, P]
        L.mx_quantize_2d_deosc.argtypes = [P, c_int, i64, i64, i64, P, i64, P, c_int, P, i64, P, P, i64, P,
                                           P, P]
        L.mx_dequantize.argtypes = [P, i64, P, i64, i64, i64, c_int, P, c_int, P]
        L.mx_quantize_1d_dual.argtypes = [P, c_int, i64, i64, P, i32, i64, c_int, u32, c_int, u32, u64, P, P,
                                          c_int, u32, u64, P, i64, P, u64, c_int, P]
        L.mx_quantize_1d_ex.argtypes = [P, c_int, i64, i64, c_int, u32, c_int, u64, u32, u64,
                                        ctypes.c_float, i64, P, P, P, P]
        L.mx_dequantize_1d_ex.argtypes = [P, P, P, i64, i64, i64, P, P]
        L.mx_grouped_gemm.argtypes = [P, i64, P, P, P, i64, P, c_int, P, i32, c_int, i64, i64, i64,
                                      ctypes.c_float, P, c_int, P]
        L.mx_grouped_gemm_q.argtypes = [P, i64, P, P, P, i64, P, c_int, P, i32, i64, i64, i64,
                                        ctypes.c_float, P, P, i64, P, P]
        for name in ("mx_rht", "mx_quantize_1d", "mx_quantize_2d", "mx_quantize_2d_deosc", "mx_dequantize",
                     "mx_quantize_1d_ex", "mx_dequantize_1d_ex", "mx_quantize_1d_dual",
                     "mx_grouped_gemm", "mx_grouped_gemm_q"):
            getattr(L, name).restype = c_int
        _lib = L
    return _lib


def declared_functions():
    """Function names declared in include/mx.h."""
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*[A-Za-z_][\w\s\*]*?\b(mx_\w+)\s*\(", text, re.M)))


def _check(fn, code):
    if code != 0:
        raise MXError(fn, code)


# ---------------------------------------------------------------------------
# torch plumbing
# ---------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream():
    return _torch().cuda.current_stream().cuda_stream


def _dtype_code(t):
    torch = _torch()
    if t.dtype == torch.float32:
        return MX_F32
    if t.dtype == torch.bfloat16:
        return MX_BF16
    raise TypeError("expected float32 or bfloat16, got %s" % t.dtype)


def _dev(t, name):
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t


def _codes(t, name):
    """A code tensor [..., rows, row_bytes] whose rows may be padded: its
    rows are contiguous and any row pitch (stride between rows, in bytes) is
    allowed, and leading dimensions are contiguous over pitched rows (a
    row-slice view t = buf[..., :row_bytes] of a wider buffer).  Returns the
    row pitch to pass to the library, 0 when the rows are contiguous."""
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if t.dtype.itemsize != 1 or t.dim() < 2 or t.stride(-1) != 1:
        raise ValueError("%s must be uint8 [..., rows, bytes] with contiguous rows" % name)
    ld = t.stride(-2)
    expect = ld * t.shape[-2]
    for d in range(t.dim() - 3, -1, -1):
        if t.shape[d] > 1 and t.stride(d) != expect:
            raise ValueError("%s: leading dimensions must be contiguous over its rows" % name)
        expect *= t.shape[d]
    return 0 if ld == t.shape[-1] else ld


def _shaped(t, shape, dtype, name, pitched=False):
    """Check a tensor against the extent the library reads or writes: this
    shape (a leading batch of 1 may be left out) and dtype, on the device,
    contiguous, or for a code array with rows that may be padded.  Returns
    the code rows' pitch (0 when unpadded or not a code array)."""
    shape = tuple(int(v) for v in shape)
    got = tuple(t.shape)
    if got != shape and not (len(shape) == 3 and shape[0] == 1 and got == shape[1:]):
        raise ValueError("%s: expected shape %s, got %s" % (name, shape, got))
    if t.dtype != dtype:
        raise TypeError("%s: expected %s, got %s" % (name, dtype, t.dtype))
    if pitched:
        return _codes(t, name)
    _dev(t, name)
    return 0


def rht_sign_mask(seed: int) -> int:
    return int(lib().mx_rht_sign_mask(seed))


def _index_vector(t, name, min_numel=0):
    """A device int32 vector (offsets, row indices): a tensor of another type
    would be read as int32 words and mis-group silently."""
    torch = _torch()
    if t.dtype != torch.int32 or t.dim() != 1 or t.numel() < min_numel:
        raise ValueError("%s must be a 1-D int32 tensor%s" %
                         (name, " of at least %d elements" % min_numel if min_numel else ""))
    return _dev(t, name)


def rht(x, sign_mask: int, inverse: bool = False, out=None):
    torch = _torch()
    _dev(x, "x")
    rows, cols = x.shape
    if out is None:
        out = torch.empty((rows, cols), dtype=torch.float32, device=x.device)
    else:
        _shaped(out, (rows, cols), torch.float32, "out")
    _check("mx_rht", lib().mx_rht(_ptr(x), _dtype_code(x), _ptr(out), rows, cols, sign_mask,
                                  int(inverse), _stream()))
    return out


def _scale_flags(b_scale_2d, staged):
    return (SCALES_B_2D if b_scale_2d else 0) | (SCALES_STAGED if staged else 0)


def padded_capacity(rows: int, num_groups: int, group_pad: int = 32) -> int:
    """A token capacity that holds any grouping of `rows` tokens into
    `num_groups` groups each padded to a multiple of group_pad (32 or 256),
    rounded up to a multiple of 256 tokens: every row of the column-wise
    codes is then a whole number of 128-byte lines, and the number of
    32-token blocks is even (the grouped GEMM moves scale bytes in pairs)."""
    return (rows + (group_pad - 1) * num_groups + 255) // 256 * 256


def quantize_1d(x, block_axis: int = 1, group_offsets=None, kp: int = 0, use_rht: bool = False,
                sign_mask: int = 0, rnd: int = RNE, seed: int = 0, stream_id: int = 0,
                index_base: int = 0, codes=None, scales=None, row_index=None, staged: bool = False,
                group_pad: int = 32):
    """Returns (codes, scales) uint8 device tensors; see mx_quantize_1d.
    row_index (column-wise only): gather x's rows through it; the grouped
    positions then number row_index.numel().  A row-wise codes output may
    have padded rows, e.g. buf[:, :cols // 2] of a wider buffer (its row
    stride, a multiple of 16, is passed as the pitch; the padding is not
    written).  staged: scales in the staged order (include/mx.h), row-wise
    [ceil(cols / 256), rows, 8], column-wise [kp // 256 + groups, cols, 8].
    group_pad (column-wise): 32, or 256 to start every group on a whole K
    stage of the weight-gradient GEMM."""
    torch = _torch()
    _dev(x, "x")
    rows, cols = x.shape
    if row_index is not None:
        _index_vector(row_index, "row_index")
        rows = row_index.numel()
    ng = 0
    if block_axis == 1:
        shape_c, shape_s = (rows, cols // 2), (rows, cols // 32)
        if staged:
            shape_s = ((cols + 255) // 256, rows, 8)
    else:
        _index_vector(group_offsets, "group_offsets", min_numel=2)
        ng = group_offsets.numel() - 1
        if group_pad not in (32, 256):
            raise ValueError("group_pad is 32 or 256")
        if not kp:
            kp = padded_capacity(rows, ng, group_pad)
        shape_c, shape_s = (cols, kp // 2), (cols, kp // 32)
        if staged:
            shape_s = (kp // 256 + ng, cols, 8)
    if codes is None:
        codes = torch.empty(shape_c, dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(shape_s, dtype=torch.uint8, device=x.device)
    # codes may be a row-slice view of a wider buffer (padded rows)
    codes_ld = _shaped(codes, shape_c, torch.uint8, "codes", pitched=True)
    _shaped(scales, shape_s, torch.uint8, "scales")
    _check("mx_quantize_1d", lib().mx_quantize_1d(
        _ptr(x), _dtype_code(x), rows, cols,
        block_axis | (SCALES_STAGED if staged else 0) | (GROUPS_PAD256 if group_pad == 256 else 0),
        _ptr(group_offsets), ng, kp,
        _ptr(row_index), int(use_rht), sign_mask, rnd, seed, stream_id, index_base, _ptr(codes), codes_ld,
        _ptr(scales), _stream()))
    return codes, scales


def quantize_1d_dual(x, group_offsets, kp: int = 0, use_rht: bool = False, sign_mask: int = 0,
                     col_rnd: int = RNE, col_stream_id: int = 0, row_rnd: int = RNE, row_stream_id: int = 0,
                     seed: int = 0, col_index_base: int = 0, row_index_base: int = 0, col_codes=None,
                     col_scales=None, row_codes=None, row_scales=None, staged: bool = False, group_pad: int = 32):
    """Column-wise (grouped, transposed, optional RHT) and row-wise (no RHT)
    1x32 quantization of x from one read (see mx_quantize_1d_dual).
    Returns (col_codes, col_scales, row_codes, row_scales); row_codes may
    have padded rows (a row-slice view of a wider buffer).  staged: both
    outputs' scales in the staged order (column-wise [kp // 256 + groups,
    cols, 8], row-wise [ceil(cols / 256), rows, 8]); group_pad: the
    column-wise output's group padding, 32 or 256 tokens."""
    torch = _torch()
    _dev(x, "x")
    rows, cols = x.shape
    _index_vector(group_offsets, "group_offsets", min_numel=2)
    ng = group_offsets.numel() - 1
    if group_pad not in (32, 256):
        raise ValueError("group_pad is 32 or 256")
    kp = kp or padded_capacity(rows, ng, group_pad)
    u8, dev = torch.uint8, x.device
    shape_cs = (kp // 256 + ng, cols, 8) if staged else (cols, kp // 32)
    shape_rs = ((cols + 255) // 256, rows, 8) if staged else (rows, cols // 32)
    col_codes = col_codes if col_codes is not None else torch.empty((cols, kp // 2), dtype=u8, device=dev)
    col_scales = col_scales if col_scales is not None else torch.empty(shape_cs, dtype=u8, device=dev)
    row_codes = row_codes if row_codes is not None else torch.empty((rows, cols // 2), dtype=u8, device=dev)
    row_scales = row_scales if row_scales is not None else torch.empty(shape_rs, dtype=u8, device=dev)
    _shaped(col_codes, (cols, kp // 2), u8, "col_codes")
    _shaped(col_scales, shape_cs, u8, "col_scales")
    ld = _shaped(row_codes, (rows, cols // 2), u8, "row_codes", pitched=True)
    _shaped(row_scales, shape_rs, u8, "row_scales")
    flags = (SCALES_STAGED if staged else 0) | (GROUPS_PAD256 if group_pad == 256 else 0)
    _check("mx_quantize_1d_dual", lib().mx_quantize_1d_dual(
        _ptr(x), _dtype_code(x), rows, cols, _ptr(group_offsets), ng, kp, int(use_rht), sign_mask, col_rnd,
        col_stream_id, col_index_base, _ptr(col_codes), _ptr(col_scales), row_rnd, row_stream_id,
        row_index_base, _ptr(row_codes), ld, _ptr(row_scales), seed, flags, _stream()))
    return col_codes, col_scales, row_codes, row_scales


def quantize_2d(w, layout=True, transposed=True):
    """w [batch x rows x cols] or [rows x cols]; returns (codes, scales,
    codes_t, scales_t), None for a layout not asked for."""
    torch = _torch()
    _dev(w, "w")
    b, r, c = (1,) + tuple(w.shape) if w.dim() == 2 else tuple(w.shape)
    dev = w.device
    codes = torch.empty((b, r, c // 2), dtype=torch.uint8, device=dev) if layout else None
    scales = torch.empty((b, r // 32, c // 32), dtype=torch.uint8, device=dev) if layout else None
    codes_t = torch.empty((b, c, r // 2), dtype=torch.uint8, device=dev) if transposed else None
    scales_t = torch.empty((b, c // 32, r // 32), dtype=torch.uint8, device=dev) if transposed else None
    return quantize_2d_into(w, codes, scales, codes_t, scales_t)


def quantize_2d_into(w, codes, scales, codes_t, scales_t):
    """As quantize_2d, into caller-provided buffers (either pair may be None).
    codes and codes_t may have padded rows (row-slice views of wider buffers)."""
    torch = _torch()
    _dev(w, "w")
    squeeze = w.dim() == 2
    w3 = w.unsqueeze(0) if squeeze else w
    b, r, c = w3.shape
    u8 = torch.uint8
    ld = 0 if codes is None else _shaped(codes, (b, r, c // 2), u8, "codes", pitched=True)
    ld_t = 0 if codes_t is None else _shaped(codes_t, (b, c, r // 2), u8, "codes_t", pitched=True)
    if scales is not None:
        _shaped(scales, (b, r // 32, c // 32), u8, "scales")
    if scales_t is not None:
        _shaped(scales_t, (b, c // 32, r // 32), u8, "scales_t")
    _check("mx_quantize_2d", lib().mx_quantize_2d(
        _ptr(w3), _dtype_code(w3), b, r, c, _ptr(codes), ld, _ptr(scales), _ptr(codes_t), ld_t,
        _ptr(scales_t), _stream()))
    out = [codes, scales, codes_t, scales_t]
    if squeeze:
        out = [t[0] if t is not None and t.dim() == 3 else t for t in out]
    return tuple(out)


def quantize_1d_ex(x, use_rht: bool = False, sign_mask: int = 0, rnd: int = RNE, seed: int = 0,
                   stream_id: int = 0, index_base: int = 0, clip_ratio: float = 1.0, macro_block: int = 0,
                   codes=None, scales=None, macro_r=None):
    """Row-wise 1x32 quantization with outlier clipping and macro-block
    scaling (see mx_quantize_1d_ex).  Returns (codes, scales, macro_r or
    None)."""
    torch = _torch()
    _dev(x, "x")
    rows, cols = x.shape
    dev = x.device
    codes = codes if codes is not None else torch.empty((rows, cols // 2), dtype=torch.uint8, device=dev)
    scales = scales if scales is not None else torch.empty((rows, cols // 32), dtype=torch.uint8, device=dev)
    _shaped(codes, (rows, cols // 2), torch.uint8, "codes")
    _shaped(scales, (rows, cols // 32), torch.uint8, "scales")
    if macro_block:
        if cols % macro_block:
            raise ValueError("macro_block must divide cols")
        macro_r = macro_r if macro_r is not None else torch.empty((rows, cols // macro_block),
                                                                  dtype=torch.float32, device=dev)
        _shaped(macro_r, (rows, cols // macro_block), torch.float32, "macro_r")
    else:
        macro_r = None
    _check("mx_quantize_1d_ex", lib().mx_quantize_1d_ex(
        _ptr(x), _dtype_code(x), rows, cols, int(use_rht), sign_mask, rnd, seed, stream_id, index_base,
        float(clip_ratio), int(macro_block), _ptr(codes), _ptr(scales), _ptr(macro_r), _stream()))
    return codes, scales, macro_r


def dequantize_1d_ex(codes, scales, macro_r=None, macro_block: int = 0, out=None):
    """fp32 decode of quantize_1d_ex's output: deq(code, scale) / r."""
    torch = _torch()
    _dev(codes, "codes")
    rows, half = codes.shape
    cols = half * 2
    _shaped(scales, (rows, cols // 32), torch.uint8, "scales")
    if macro_block:
        _shaped(macro_r, (rows, cols // macro_block), torch.float32, "macro_r")
    out = out if out is not None else torch.empty((rows, cols), dtype=torch.float32, device=codes.device)
    _shaped(out, (rows, cols), torch.float32, "out")
    _check("mx_dequantize_1d_ex", lib().mx_dequantize_1d_ex(
        _ptr(codes), _ptr(scales), _ptr(macro_r) if macro_block else None, rows, cols, int(macro_block),
        _ptr(out), _stream()))
    return out


def quantize_2d_deosc(w, prev_codes, prev_scales, margin64: int, codes=None, scales=None,
                      codes_t=None, scales_t=None, transposed=True, flips=True):
    """32x32 quantization with the de-oscillation band against the previous
    step's as-given codes and scales (see mx_quantize_2d_deosc).  codes /
    scales default to new tensors; passing prev_codes / prev_scales again
    updates them in place.  Returns (codes, scales, codes_t, scales_t,
    flips), None for what was not asked for."""
    torch = _torch()
    _dev(w, "w")
    squeeze = w.dim() == 2
    w3 = w.unsqueeze(0) if squeeze else w
    b, r, c = w3.shape
    u8, dev = torch.uint8, w.device

    def as3(t):
        return t.unsqueeze(0) if t is not None and t.dim() == 2 else t

    prev_codes, prev_scales = as3(prev_codes), as3(prev_scales)
    codes = as3(codes) if codes is not None else torch.empty((b, r, c // 2), dtype=u8, device=dev)
    scales = as3(scales) if scales is not None else torch.empty((b, r // 32, c // 32), dtype=u8, device=dev)
    if transposed:
        codes_t = as3(codes_t) if codes_t is not None else torch.empty((b, c, r // 2), dtype=u8, device=dev)
        scales_t = as3(scales_t) if scales_t is not None else torch.empty((b, c // 32, r // 32), dtype=u8,
                                                                          device=dev)
    else:
        codes_t = scales_t = None
    fl = torch.empty((b, r // 32, c // 32), dtype=torch.int16, device=dev) if flips else None
    pld = _shaped(prev_codes, (b, r, c // 2), u8, "prev_codes", pitched=True)
    _shaped(prev_scales, (b, r // 32, c // 32), u8, "prev_scales")
    ld = _shaped(codes, (b, r, c // 2), u8, "codes", pitched=True)
    _shaped(scales, (b, r // 32, c // 32), u8, "scales")
    ld_t = 0 if codes_t is None else _shaped(codes_t, (b, c, r // 2), u8, "codes_t", pitched=True)
    if scales_t is not None:
        _shaped(scales_t, (b, c // 32, r // 32), u8, "scales_t")
    _check("mx_quantize_2d_deosc", lib().mx_quantize_2d_deosc(
        _ptr(w3), _dtype_code(w3), b, r, c, _ptr(prev_codes), pld, _ptr(prev_scales), int(margin64),
        _ptr(codes), ld, _ptr(scales), _ptr(codes_t), ld_t, _ptr(scales_t), _ptr(fl), _stream()))
    out = [codes, scales, codes_t, scales_t, fl]
    if squeeze:
        out = [t[0] if t is not None and t.dim() == 3 else t for t in out]
    return tuple(out)


def dequantize(codes, scales, block_rows: int = 1, out_dtype=None, out=None):
    """Per mx_dequantize; codes may have padded rows."""
    torch = _torch()
    ld = _codes(codes, "codes")
    out_dtype = out_dtype or torch.float32
    squeeze = codes.dim() == 2
    c3 = codes.unsqueeze(0) if squeeze else codes
    b, r, half = c3.shape
    _shaped(scales, (b, r // block_rows, half * 2 // 32), torch.uint8, "scales")
    if out is None:
        out = torch.empty((b, r, half * 2), dtype=out_dtype, device=codes.device)
    else:
        _shaped(out, (b, r, half * 2), out.dtype, "out")
    _check("mx_dequantize", lib().mx_dequantize(
        _ptr(c3), ld, _ptr(scales), b, r, half * 2, block_rows, _ptr(out), _dtype_code(out),
        _stream()))
    return out[0] if squeeze and out.dim() == 3 else out


def _gemm_operands(a_codes, a_scales, a_row_index, b_codes, b_scales, group_offsets, M, N, K,
                   b_scale_2d, group_dim_k, staged=False):
    """Check A, B and their scales against M, N, K and the group count (the
    extents the kernel reads); returns (a_ld, b_ld, G).  Staged scales are
    [stages, rows, 8]: K // 256 + G stages with groups along K, ceil(K / 256)
    along M."""
    torch = _torch()
    u8 = torch.uint8
    _index_vector(group_offsets, "group_offsets", min_numel=2)
    G = group_offsets.numel() - 1
    a_rows = M
    if a_row_index is not None:
        _index_vector(a_row_index, "a_row_index")
        if a_row_index.numel() != M:
            raise ValueError("a_row_index must be int32 [M]")
        a_rows = a_codes.shape[0]
    a_ld = _shaped(a_codes, (a_rows, K // 2), u8, "a_codes", pitched=True)
    stages = (K // 256 + G) if group_dim_k else (K + 255) // 256
    _shaped(a_scales, (stages, a_rows, 8) if staged else (a_rows, K // 32), u8, "a_scales")
    if group_dim_k:
        b_ld = _shaped(b_codes, (N, K // 2), u8, "b_codes", pitched=True)
        _shaped(b_scales, (stages, N, 8) if staged else (N, K // 32), u8, "b_scales")
    else:
        b_ld = _shaped(b_codes, (G, N, K // 2), u8, "b_codes", pitched=True)
        _shaped(b_scales, (G, N // 32, K // 32) if b_scale_2d else (G, N, K // 32), u8, "b_scales")
    return a_ld, b_ld, G


def grouped_gemm(a_codes, a_scales, b_codes, b_scales, group_offsets, M, N, K,
                 a_row_index=None, b_scale_2d=False, group_dim_k=False, alpha=1.0,
                 out_dtype=None, out=None, staged=False):
    """C (bf16 by default, or out_dtype float32) per mx_grouped_gemm.  a_codes
    and b_codes may have padded rows (row-slice views of wider buffers); rows
    padded to whole 128-byte lines are read fastest."""
    torch = _torch()
    a_ld, b_ld, G = _gemm_operands(a_codes, a_scales, a_row_index, b_codes, b_scales, group_offsets,
                                   M, N, K, b_scale_2d, group_dim_k, staged)
    shape = (G, M, N) if group_dim_k else (M, N)
    if out is None:
        out = torch.empty(shape, dtype=out_dtype or torch.bfloat16, device=a_codes.device)
    else:
        _shaped(out, shape, out_dtype or out.dtype, "out")
    _check("mx_grouped_gemm", lib().mx_grouped_gemm(
        _ptr(a_codes), a_ld, _ptr(a_scales), _ptr(a_row_index), _ptr(b_codes), b_ld, _ptr(b_scales),
        _scale_flags(b_scale_2d, staged), _ptr(group_offsets), G, int(bool(group_dim_k)), M, N, K,
        float(alpha), _ptr(out), _dtype_code(out), _stream()))
    return out


def grouped_gemm_q(a_codes, a_scales, b_codes, b_scales, group_offsets, M, N, K,
                   a_row_index=None, b_scale_2d=False, alpha=1.0, with_bf16=True,
                   out=None, codes=None, scales=None, staged=False):
    """Grouped GEMM (groups split M) whose bf16 output is also written as
    row-wise MXFP4 (1x32 along N, RTNE) by the GEMM's epilogue.  Returns
    (c or None, codes [M x N/2], scales [M x N/32]); out / codes / scales
    are optional preallocated outputs."""
    torch = _torch()
    a_ld, b_ld, G = _gemm_operands(a_codes, a_scales, a_row_index, b_codes, b_scales, group_offsets,
                                   M, N, K, b_scale_2d, False, staged)
    dev = a_codes.device
    c = None
    if with_bf16:
        c = out if out is not None else torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        _shaped(c, (M, N), torch.bfloat16, "out")
    codes = codes if codes is not None else torch.empty((M, N // 2), dtype=torch.uint8, device=dev)
    c_ld = _shaped(codes, (M, N // 2), torch.uint8, "codes", pitched=True)
    scales = scales if scales is not None else torch.empty((M, N // 32), dtype=torch.uint8, device=dev)
    _shaped(scales, (M, N // 32), torch.uint8, "scales")
    _check("mx_grouped_gemm_q", lib().mx_grouped_gemm_q(
        _ptr(a_codes), a_ld, _ptr(a_scales), _ptr(a_row_index), _ptr(b_codes), b_ld, _ptr(b_scales),
        _scale_flags(b_scale_2d, staged), _ptr(group_offsets), G, M, N, K, float(alpha),
        _ptr(c), _ptr(codes), c_ld, _ptr(scales), _stream()))
    return c, codes, scales
