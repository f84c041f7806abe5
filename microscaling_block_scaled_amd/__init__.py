"""libmxfp8 for MI355X: MXFP8 block-scaled quantization and the block-scaled
matrix product, as hand-written HIP kernels behind a C ABI (include/mxfp8.h).

This package is the thin Python binding: each function has the name of the C
entry point it calls, takes torch tensors on the GPU (torch provides device
memory and the current stream), allocates outputs when none are given, and
raises MXError on any non-OK status. Nothing here computes; there is no CPU
fallback.

Layouts (row-major, unit stride along the last dimension):
  * codes  uint8 [rows, cols]; E8M0 scales uint8 [rows, cols/32];
  * mx_quantize_colwise returns the codes and scales of X^T (blocks down the
    columns of X), i.e. [cols, rows] and [cols, rows/32];
  * mx_gemm(a, sa, b, sb) computes y = A * B^T for A [M, K], B [N, K];
  * MX_E2M1 (MXFP4) codes are packed two per byte, so their arrays are
    [rows, cols/2]; K is then taken from the scales.
"""
import ctypes
import functools

from ._lib import (BLOCK, MX_ACCUM_AUTO, MX_ACCUM_FP8, MX_ACCUM_FP32, MX_BCAST_1X128, MX_BCAST_128X128, MX_BF16,
                   MX_BLOCKS_1D, MX_BLOCKS_2D, MX_E2M1, MX_E4M3, MX_E5M2, MX_F32, MX_SCALE_CEIL, MX_SCALE_FLOOR,
                   MXError, check, lib, mx_attention_desc_t, mx_gemm_desc_t, mx_grouped_gemm_desc_t,
                   mx_quantize_desc_t)

__all__ = [
    "MX_E4M3", "MX_E5M2", "MX_E2M1", "MX_F32", "MX_BF16", "BLOCK", "MXError",
    "MX_ACCUM_AUTO", "MX_ACCUM_FP8", "MX_ACCUM_FP32", "MX_SCALE_FLOOR", "MX_SCALE_CEIL",
    "MX_BLOCKS_1D", "MX_BLOCKS_2D", "MX_BCAST_1X128", "MX_BCAST_128X128",
    "mx_quantize", "mx_quantize_colwise", "mx_quantize_ex", "mx_scale_broadcast", "mx_dequantize", "mx_kv_quant_write", "mx_gemm",
    "mx_gemm_desc", "mx_grouped_gemm", "mx_paged_scores", "mx_paged_attention", "mx_status_string",
    "mx_query_support",
]


def _torch():
    import torch
    return torch


def _on_device_of_first_tensor(fn):
    """Runs an entry point with its first tensor's GPU as the current device,
    so that the library's device checks and the default stream
    (torch.cuda.current_stream()) refer to the GPU that holds the data."""
    @functools.wraps(fn)
    def wrapper(t, *args, **kwargs):
        if getattr(t, "is_cuda", False):
            with _torch().cuda.device(t.device):
                return fn(t, *args, **kwargs)
        return fn(t, *args, **kwargs)
    return wrapper


def _stream(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dtype_code(t):
    torch = _torch()
    if t.dtype == torch.float32:
        return MX_F32
    if t.dtype == torch.bfloat16:
        return MX_BF16
    raise TypeError("expected float32 or bfloat16, got %s" % t.dtype)


def _rowmajor(t, name, ndim=2):
    if t.dim() != ndim:
        raise ValueError("%s must be %d-D" % (name, ndim))
    if t.stride(-1) != 1 and t.numel() > 0:
        raise ValueError("%s must have unit stride along its last dimension" % name)
    if not t.is_cuda:
        raise ValueError("%s must be a GPU tensor" % name)


def _buf(t, name, shape, dtype, like=None):
    """Checks a buffer the kernels read or write through a bare pointer: its
    exact shape and dtype, unit stride along the last dimension, rows that do
    not overlap, and (with `like`) the same GPU as `like`. A smaller tensor
    would otherwise let a kernel run past its end."""
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if t.numel() > 0:
        if t.stride(-1) != 1:
            raise ValueError("%s must have unit stride along its last dimension" % name)
        for i in range(t.dim() - 1):
            if t.shape[i] > 1 and t.stride(i) < t.shape[i + 1] * t.stride(i + 1):
                raise ValueError("%s has overlapping rows" % name)
    if not t.is_cuda:
        raise ValueError("%s must be a GPU tensor" % name)
    if like is not None and t.device != like.device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, like.device))


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


def _ld(t):
    """Row pitch of a 2-D tensor; a single row may carry any stride, so its
    pitch is taken as its length."""
    return t.stride(0) if t.shape[0] > 1 else t.shape[1]


@_on_device_of_first_tensor
def mx_quantize(x, fmt=MX_E4M3, q=None, s=None, stream=None):
    """Rowwise MX quantization of x [rows, cols] -> (codes, scales); E2M1
    codes are [rows, cols/2] (two per byte)."""
    torch = _torch()
    _rowmajor(x, "x")
    rows, cols = x.shape
    cb = cols // 2 if fmt == MX_E2M1 else cols
    q = torch.empty((rows, cb), dtype=torch.uint8, device=x.device) if q is None else q
    s = torch.empty((rows, cols // BLOCK), dtype=torch.uint8, device=x.device) if s is None else s
    _buf(q, "q", (rows, cb), torch.uint8, x)
    _buf(s, "s", (rows, cols // BLOCK), torch.uint8, x)
    check("mx_quantize", lib().mx_quantize(_p(x), _dtype_code(x), rows, cols, _ld(x), fmt, _p(q), _ld(q),
                                           _p(s), _ld(s), _stream(stream)))
    return q, s


@_on_device_of_first_tensor
def mx_quantize_colwise(x, fmt=MX_E4M3, qt=None, st=None, stream=None):
    """Colwise MX quantization of x [rows, cols] (blocks of 32 down each
    column), stored transposed -> (codes [cols, rows] (E2M1: [cols, rows/2],
    two per byte), scales [cols, rows/32])."""
    torch = _torch()
    _rowmajor(x, "x")
    rows, cols = x.shape
    rb = rows // 2 if fmt == MX_E2M1 else rows
    qt = torch.empty((cols, rb), dtype=torch.uint8, device=x.device) if qt is None else qt
    st = torch.empty((cols, rows // BLOCK), dtype=torch.uint8, device=x.device) if st is None else st
    _buf(qt, "qt", (cols, rb), torch.uint8, x)
    _buf(st, "st", (cols, rows // BLOCK), torch.uint8, x)
    check("mx_quantize_colwise", lib().mx_quantize_colwise(_p(x), _dtype_code(x), rows, cols, _ld(x), fmt,
                                                           _p(qt), _ld(qt), _p(st), _ld(st),
                                                           _stream(stream)))
    return qt, st


@_on_device_of_first_tensor
def mx_quantize_ex(x, fmt=MX_E4M3, rule=MX_SCALE_FLOOR, blocks=MX_BLOCKS_1D, rowwise=True, colwise=False,
                   q=None, s=None, qt=None, st=None, stream=None):
    """Quantization with a scale rule (MX_SCALE_FLOOR / MX_SCALE_CEIL) and a
    block shape (MX_BLOCKS_1D: 1x32 rowwise and 32x1 colwise blocks;
    MX_BLOCKS_2D: one scale per 32x32 block, repeated in the MXFP8 scale
    layout). Returns (q, s, qt, st); the outputs not asked for are None."""
    torch = _torch()
    _rowmajor(x, "x")
    rows, cols = x.shape
    u8 = dict(dtype=torch.uint8, device=x.device)
    d = mx_quantize_desc_t(x=_p(x).value, xdt=_dtype_code(x), rows=rows, cols=cols, ldx=_ld(x), fmt=fmt, rule=rule,
                           blocks=blocks)
    if rowwise:
        q = torch.empty((rows, cols // 2 if fmt == MX_E2M1 else cols), **u8) if q is None else q
        s = torch.empty((rows, cols // BLOCK), **u8) if s is None else s
        _buf(q, "q", (rows, cols // 2 if fmt == MX_E2M1 else cols), torch.uint8, x)
        _buf(s, "s", (rows, cols // BLOCK), torch.uint8, x)
        d.q, d.ldq, d.s, d.lds = _p(q).value, _ld(q), _p(s).value, _ld(s)
    else:
        q = s = None
    if colwise:
        rb = rows // 2 if fmt == MX_E2M1 else rows
        qt = torch.empty((cols, rb), **u8) if qt is None else qt
        st = torch.empty((cols, rows // BLOCK), **u8) if st is None else st
        _buf(qt, "qt", (cols, rb), torch.uint8, x)
        _buf(st, "st", (cols, rows // BLOCK), torch.uint8, x)
        d.qt, d.ldqt, d.st, d.ldst = _p(qt).value, _ld(qt), _p(st).value, _ld(st)
    else:
        qt = st = None
    check("mx_quantize_ex", lib().mx_quantize_ex(ctypes.byref(d), _stream(stream)))
    return q, s, qt, st


@_on_device_of_first_tensor
def mx_scale_broadcast(s_in, rows, cols, layout=MX_BCAST_1X128, out=None, stream=None):
    """Power-of-two FP32 scales of 128-element blocks (layout MX_BCAST_1X128:
    s_in [rows, cols/128]; MX_BCAST_128X128: [ceil(rows/128), cols/128]) ->
    E8M0 scales [rows, cols/32] for the same FP8 codes."""
    torch = _torch()
    _rowmajor(s_in, "s_in")
    if s_in.dtype != torch.float32:
        raise TypeError("s_in must be float32")
    out = torch.empty((rows, cols // BLOCK), dtype=torch.uint8, device=s_in.device) if out is None else out
    src_rows = rows if layout == MX_BCAST_1X128 else (rows + 127) // 128
    _buf(s_in, "s_in", (src_rows, cols // 128), torch.float32)
    _buf(out, "out", (rows, cols // BLOCK), torch.uint8, s_in)
    check("mx_scale_broadcast", lib().mx_scale_broadcast(_p(s_in), _ld(s_in), layout, rows, cols, _p(out), _ld(out),
                                                         _stream(stream)))
    return out


@_on_device_of_first_tensor
def mx_dequantize(q, s, fmt=MX_E4M3, out_dtype=None, y=None, stream=None):
    """x_hat = scale * code -> y [rows, cols] in float32 or bfloat16."""
    torch = _torch()
    _rowmajor(q, "q")
    rows, cols = q.shape[0], s.shape[1] * BLOCK
    _buf(q, "q", (rows, cols // 2 if fmt == MX_E2M1 else cols), torch.uint8)
    _buf(s, "s", (rows, cols // BLOCK), torch.uint8, q)
    if y is None:
        y = torch.empty((rows, cols), dtype=out_dtype or torch.float32, device=q.device)
    _buf(y, "y", (rows, cols), y.dtype, q)
    check("mx_dequantize", lib().mx_dequantize(_p(q), _ld(q), _p(s), _ld(s), fmt, rows, cols, _p(y),
                                               _dtype_code(y), _ld(y), _stream(stream)))
    return y


@_on_device_of_first_tensor
def mx_kv_quant_write(k, v, slot_mapping, k_cache, k_scale, v_cache, v_scale, stream=None):
    """Fused E4M3 quantize + paged write of k, v [T, H, D] into
    k_cache / v_cache [pages, page_size, H, D] and k_scale / v_scale
    [pages, page_size, H, D/32] at slot_mapping [T] (int64)."""
    torch = _torch()
    if k.shape != v.shape or k.dim() != 3 or k.stride() != v.stride():
        raise ValueError("k and v must be [T, H, D] with equal strides")
    T, H, D = k.shape
    if k.stride(2) != 1 or k.stride(1) != D:
        raise ValueError("k/v must be contiguous within a token")
    if not k.is_cuda or v.device != k.device:
        raise ValueError("k and v must be on one GPU")
    _buf(slot_mapping, "slot_mapping", (T,), torch.int64, k)
    pages, page_size = k_cache.shape[0], k_cache.shape[1]
    for c, n in ((k_cache, "k_cache"), (v_cache, "v_cache")):
        if tuple(c.shape) != (pages, page_size, H, D) or not c.is_contiguous():
            raise ValueError("%s must be contiguous [pages, page_size, H, D]" % n)
        _buf(c, n, (pages, page_size, H, D), torch.uint8, k)
    for c, n in ((k_scale, "k_scale"), (v_scale, "v_scale")):
        if tuple(c.shape) != (pages, page_size, H, D // BLOCK) or not c.is_contiguous():
            raise ValueError("%s must be contiguous [pages, page_size, H, D/32]" % n)
        _buf(c, n, (pages, page_size, H, D // BLOCK), torch.uint8, k)
    check("mx_kv_quant_write", lib().mx_kv_quant_write(_p(k), _p(v), _dtype_code(k), T, H, D, k.stride(0),
                                                       _p(slot_mapping), _p(k_cache), _p(k_scale), _p(v_cache),
                                                       _p(v_scale), page_size, pages, _stream(stream)))


def mx_gemm_desc(desc, stream=None):
    """Call mx_gemm with a filled mx_gemm_desc_t."""
    check("mx_gemm", lib().mx_gemm(ctypes.byref(desc), _stream(stream)))


@_on_device_of_first_tensor
def mx_gemm(a, sa, b, sb, a_fmt=MX_E4M3, b_fmt=MX_E4M3, out_dtype=None, y=None, stream=None, accum=MX_ACCUM_AUTO):
    """y [M, N] = block-scaled A [M, K] * B [N, K]^T with FP32 accumulation
    (accum selects the matrix-instruction path; see include/mxfp8.h)."""
    torch = _torch()
    for t, n in ((a, "a"), (sa, "sa"), (b, "b"), (sb, "sb")):
        _rowmajor(t, n)
    M, N = a.shape[0], b.shape[0]
    K = sa.shape[1] * BLOCK
    kb_a = K // 2 if a_fmt == MX_E2M1 else K
    kb_b = K // 2 if b_fmt == MX_E2M1 else K
    if a.shape[1] != kb_a or b.shape[1] != kb_b or sb.shape != (N, K // BLOCK) or sa.shape[0] != M:
        raise ValueError("shape mismatch: a %s sa %s b %s sb %s" % (tuple(a.shape), tuple(sa.shape), tuple(b.shape),
                                                                    tuple(sb.shape)))
    for t, n, shp in ((a, "a", (M, kb_a)), (sa, "sa", (M, K // BLOCK)), (b, "b", (N, kb_b)),
                      (sb, "sb", (N, K // BLOCK))):
        _buf(t, n, shp, torch.uint8, a)
    if y is None:
        y = torch.empty((M, N), dtype=out_dtype or torch.bfloat16, device=a.device)
    _buf(y, "y", (M, N), y.dtype, a)
    d = mx_gemm_desc_t()
    d.M, d.N, d.K = M, N, K
    d.a, d.lda, d.sa, d.ldsa, d.a_fmt = a.data_ptr(), _ld(a), sa.data_ptr(), _ld(sa), a_fmt
    d.b, d.ldb, d.sb, d.ldsb, d.b_fmt = b.data_ptr(), _ld(b), sb.data_ptr(), _ld(sb), b_fmt
    d.y, d.ldy, d.y_dtype = y.data_ptr(), _ld(y), _dtype_code(y)
    d.accum = accum
    mx_gemm_desc(d, stream)
    return y


@_on_device_of_first_tensor
def mx_grouped_gemm(a, sa, b, sb, group_offsets, a_fmt=MX_E4M3, b_fmt=MX_E4M3, out_dtype=None, y=None,
                    stream=None, accum=MX_ACCUM_AUTO):
    """Per-group block-scaled products: rows off[q] .. off[q+1]-1 of A [total_m,
    K] times group q's B [N, K]^T. b [G, N, K] and sb [G, N, K/32] (E2M1: b is
    [G, N, K/2]); group_offsets int64 [G+1] on the device. Rows of y outside
    every group are left as they are (zeros when y is allocated here)."""
    torch = _torch()
    for t, n in ((a, "a"), (sa, "sa")):
        _rowmajor(t, n)
    if b.dim() != 3 or sb.dim() != 3 or not b.is_contiguous() or not sb.is_contiguous():
        raise ValueError("b and sb must be contiguous [G, N, ...] tensors")
    if group_offsets.dtype != torch.int64 or not group_offsets.is_cuda or group_offsets.shape != (b.shape[0] + 1,):
        raise ValueError("group_offsets must be a device int64 tensor of groups + 1 entries")
    G, N = b.shape[0], b.shape[1]
    M = a.shape[0]
    K = sa.shape[1] * BLOCK
    if sb.shape != (G, N, K // BLOCK):
        raise ValueError("sb must be [G, N, K/32]")
    kb_a = K // 2 if a_fmt == MX_E2M1 else K
    kb_b = K // 2 if b_fmt == MX_E2M1 else K
    for t, n, shp in ((a, "a", (M, kb_a)), (sa, "sa", (M, K // BLOCK)), (b, "b", (G, N, kb_b)),
                      (sb, "sb", (G, N, K // BLOCK))):
        _buf(t, n, shp, torch.uint8, a)
    _buf(group_offsets, "group_offsets", (G + 1,), torch.int64, a)
    if y is None:
        y = torch.zeros((M, N), dtype=out_dtype or torch.bfloat16, device=a.device)
    _buf(y, "y", (M, N), y.dtype, a)
    d = mx_grouped_gemm_desc_t()
    d.groups, d.total_m, d.N, d.K = G, M, N, K
    d.group_offsets = group_offsets.data_ptr()
    d.a, d.lda, d.sa, d.ldsa, d.a_fmt = a.data_ptr(), _ld(a), sa.data_ptr(), _ld(sa), a_fmt
    d.b, d.ldb, d.sb, d.ldsb, d.b_fmt = b.data_ptr(), b.shape[2], sb.data_ptr(), sb.shape[2], b_fmt
    d.stride_b, d.stride_sb = N * b.shape[2], N * sb.shape[2]
    d.y, d.ldy, d.y_dtype = y.data_ptr(), _ld(y), _dtype_code(y)
    d.accum = accum
    check("mx_grouped_gemm", lib().mx_grouped_gemm(ctypes.byref(d), _stream(stream)))
    return y


@_on_device_of_first_tensor
def mx_paged_scores(q_codes, q_scales, k_cache, k_scale, page_table, seq_len, out=None, stream=None,
                    accum=MX_ACCUM_AUTO):
    """QK^T scores per (sequence, head) with K read through a page table.

    q_codes [S*seq_len, H, D] / q_scales [S*seq_len, H, D/32] (rowwise E4M3
    along D); k_cache [pages, page_size, H, D] / k_scale [..., D/32];
    page_table int32 [S, seq_len/page_size]. Returns f32 [S, H, seq_len,
    seq_len] with out[s, h, i, j] = q(s, i, h) . k(s, j, h), the block-scaled
    product over D."""
    torch = _torch()
    tokens, H, D = q_codes.shape
    S = page_table.shape[0]
    page_size = k_cache.shape[1]
    if tokens != S * seq_len or page_table.shape[1] * page_size < seq_len:
        raise ValueError("inconsistent query/page-table sizes")
    if not (q_codes.is_contiguous() and q_scales.is_contiguous() and k_cache.is_contiguous()
            and k_scale.is_contiguous() and page_table.is_contiguous()):
        raise ValueError("inputs must be contiguous")
    if page_table.dtype != torch.int32:
        raise TypeError("page_table must be int32")
    pages = k_cache.shape[0]
    for t, n, shp in ((q_codes, "q_codes", (tokens, H, D)), (q_scales, "q_scales", (tokens, H, D // BLOCK)),
                      (k_cache, "k_cache", (pages, page_size, H, D)),
                      (k_scale, "k_scale", (pages, page_size, H, D // BLOCK))):
        _buf(t, n, shp, torch.uint8, q_codes)
    _buf(page_table, "page_table", (S, page_table.shape[1]), torch.int32, q_codes)
    if out is None:
        out = torch.empty((S, H, seq_len, seq_len), dtype=torch.float32, device=q_codes.device)
    if not out.is_contiguous():
        raise ValueError("out must be contiguous")
    _buf(out, "out", (S, H, seq_len, seq_len), torch.float32, q_codes)
    d = mx_gemm_desc_t()
    d.M, d.N, d.K = seq_len, seq_len, D
    d.a, d.lda, d.sa, d.ldsa, d.a_fmt = q_codes.data_ptr(), H * D, q_scales.data_ptr(), H * (D // BLOCK), MX_E4M3
    d.b, d.ldb, d.sb, d.ldsb, d.b_fmt = k_cache.data_ptr(), H * D, k_scale.data_ptr(), H * (D // BLOCK), MX_E4M3
    d.y, d.ldy, d.y_dtype = out.data_ptr(), seq_len, MX_F32
    d.batch_outer, d.batch_inner = S, H
    d.stride_a_outer, d.stride_a_inner = seq_len * H * D, D
    d.stride_sa_outer, d.stride_sa_inner = seq_len * H * (D // BLOCK), D // BLOCK
    d.stride_b_inner, d.stride_sb_inner = D, D // BLOCK
    d.stride_y_outer, d.stride_y_inner = H * seq_len * seq_len, seq_len * seq_len
    d.b_page_table = page_table.data_ptr()
    d.b_pages_per_seq = page_table.shape[1]
    d.b_page_rows = page_size
    d.b_page_stride = page_size * H * D
    d.b_page_stride_s = page_size * H * (D // BLOCK)
    d.accum = accum
    mx_gemm_desc(d, stream)
    return out


@_on_device_of_first_tensor
def mx_paged_attention(q_codes, q_scales, k_cache, k_scale, v_cache, v_scale, page_table, kv_lens, q_len,
                       sm_scale=None, causal=False, out=None, out_dtype=None, lse=None, stream=None):
    """Attention of MXFP8 queries over the paged MXFP8 KV cache.

    q_codes [S*q_len, Hq, D] / q_scales [S*q_len, Hq, D/32] (rowwise E4M3
    along D); k_cache, v_cache [pages, page_size, Hkv, D] and k_scale,
    v_scale [pages, page_size, Hkv, D/32] as mx_kv_quant_write fills them;
    page_table int32 [S, pages_per_seq]; kv_lens int32 [S] (device).
    sm_scale defaults to 1/sqrt(D). Returns out [S*q_len, Hq, D] (bf16 unless
    out / out_dtype say f32); `lse` (f32 [S*q_len, Hq]) is filled when given."""
    torch = _torch()
    T, Hq, D = q_codes.shape
    S = page_table.shape[0]
    Hkv = k_cache.shape[2]
    if T != S * q_len or kv_lens.shape != (S,):
        raise ValueError("inconsistent query / sequence sizes")
    for name, t in (("q_codes", q_codes), ("q_scales", q_scales), ("k_cache", k_cache), ("k_scale", k_scale),
                    ("v_cache", v_cache), ("v_scale", v_scale), ("page_table", page_table), ("kv_lens", kv_lens)):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("%s must be a contiguous GPU tensor" % name)
    if page_table.dtype != torch.int32 or kv_lens.dtype != torch.int32:
        raise TypeError("page_table and kv_lens must be int32")
    pages, page_size = k_cache.shape[0], k_cache.shape[1]
    for t, n, shp in ((q_codes, "q_codes", (T, Hq, D)), (q_scales, "q_scales", (T, Hq, D // BLOCK)),
                      (k_cache, "k_cache", (pages, page_size, Hkv, D)),
                      (k_scale, "k_scale", (pages, page_size, Hkv, D // BLOCK)),
                      (v_cache, "v_cache", (pages, page_size, Hkv, D)),
                      (v_scale, "v_scale", (pages, page_size, Hkv, D // BLOCK))):
        _buf(t, n, shp, torch.uint8, q_codes)
    _buf(page_table, "page_table", (S, page_table.shape[1]), torch.int32, q_codes)
    _buf(kv_lens, "kv_lens", (S,), torch.int32, q_codes)
    if out is None:
        dt = torch.bfloat16 if out_dtype in (None, MX_BF16, torch.bfloat16) else torch.float32
        out = torch.empty((T, Hq, D), dtype=dt, device=q_codes.device)
    if out.shape != (T, Hq, D) or not out.is_contiguous():
        raise ValueError("out must be a contiguous [S*q_len, Hq, D] tensor")
    _buf(out, "out", (T, Hq, D), out.dtype, q_codes)
    if lse is not None and (lse.shape != (T, Hq) or lse.dtype != torch.float32 or not lse.is_contiguous()):
        raise ValueError("lse must be a contiguous float32 [S*q_len, Hq] tensor")
    if lse is not None:
        _buf(lse, "lse", (T, Hq), torch.float32, q_codes)
    d = mx_attention_desc_t()
    d.num_seqs, d.q_len, d.num_q_heads, d.num_kv_heads, d.head_dim = S, q_len, Hq, Hkv, D
    d.q, d.ld_q, d.q_scale, d.ld_qs = q_codes.data_ptr(), Hq * D, q_scales.data_ptr(), Hq * (D // BLOCK)
    d.k_cache, d.k_scale, d.v_cache, d.v_scale = (k_cache.data_ptr(), k_scale.data_ptr(), v_cache.data_ptr(),
                                                  v_scale.data_ptr())
    d.page_size = k_cache.shape[1]
    d.page_table, d.pages_per_seq = page_table.data_ptr(), page_table.shape[1]
    d.kv_lens = kv_lens.data_ptr()
    d.sm_scale = float(D ** -0.5 if sm_scale is None else sm_scale)
    d.causal = 1 if causal else 0
    d.out, d.ld_o, d.out_dtype = out.data_ptr(), Hq * D, _dtype_code(out)
    d.lse = lse.data_ptr() if lse is not None else None
    check("mx_paged_attention", lib().mx_paged_attention(ctypes.byref(d), _stream(stream)))
    return out


def mx_status_string(status):
    return lib().mx_status_string(status).decode()


def mx_query_support(device=0):
    """(ok: bool, reason: str) for `device`."""
    r = ctypes.c_char_p()
    st = lib().mx_query_support(device, ctypes.byref(r))
    return st == 0, (r.value.decode() if r.value else "")
