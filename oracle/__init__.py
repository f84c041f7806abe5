"""CPU oracle for MXFP8 block-scaled quantization and the block-scaled product.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package. It is independent of
the HIP library: it neither imports it nor shares any code, table or helper
with it. The arithmetic lives in ``mx_oracle.c`` (plain C, fp64); this module
only marshals numpy arrays into it.

Array conventions (host numpy arrays):
  * f32 inputs are ``np.float32``; bf16 inputs are their 16-bit patterns as
    ``np.uint16``;
  * codes and E8M0 scales are ``np.uint8``;
  * formats: ``E4M3 = 0``, ``E5M2 = 1``, ``E2M1 = 2`` (MXFP4). E2M1 codes are
    packed two per byte, element 2i in the low nibble, so an E2M1 code array
    of K elements per row is K/2 bytes wide.
"""
import ctypes
import os

import numpy as np

E4M3 = 0
E5M2 = 1
E2M1 = 2
RULE_FLOOR = 0  # X = 2^(floor(log2 amax) - emax_elem)
RULE_CEIL = 1   # smallest power of two with amax / X <= largest finite element
F32 = 0
BF16 = 1
BLOCK = 32

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libmxoracle.so")
_lib = None

_i64 = ctypes.c_int64
_p = ctypes.c_void_p


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _b
        _b.build()
    lib = ctypes.CDLL(_LIB_PATH)
    lib.mxo_decode.restype = ctypes.c_double
    lib.mxo_decode.argtypes = [ctypes.c_int, ctypes.c_uint]
    lib.mxo_decode_e8m0.restype = ctypes.c_double
    lib.mxo_decode_e8m0.argtypes = [ctypes.c_uint]
    lib.mxo_encode.restype = ctypes.c_uint
    lib.mxo_encode.argtypes = [ctypes.c_int, ctypes.c_double]
    lib.mxo_scale_code.restype = ctypes.c_uint
    lib.mxo_scale_code.argtypes = [ctypes.c_int, _p, _i64]
    lib.mxo_double_to_bf16.restype = ctypes.c_uint16
    lib.mxo_double_to_bf16.argtypes = [ctypes.c_double]
    lib.mxo_dequant_value.restype = ctypes.c_double
    lib.mxo_dequant_value.argtypes = [ctypes.c_int, ctypes.c_uint, ctypes.c_uint]
    lib.mxo_quantize_rows.argtypes = [_p, ctypes.c_int, _i64, _i64, _i64, ctypes.c_int, _p, _i64, _p, _i64]
    lib.mxo_quantize_cols.argtypes = [_p, ctypes.c_int, _i64, _i64, _i64, ctypes.c_int, _p, _i64, _p, _i64]
    lib.mxo_kv_quant_write.argtypes = [_p, _p, ctypes.c_int, _i64, _i64, _i64, _i64, _p, _p, _p, _p, _p, _i64, _i64]
    lib.mxo_dequantize.argtypes = [_p, _i64, _p, _i64, ctypes.c_int, _i64, _i64, _p, ctypes.c_int, _i64]
    lib.mxo_gemm.argtypes = [_i64, _i64, _i64, _p, _i64, _p, _i64, ctypes.c_int, _p, _i64, _p, _i64, ctypes.c_int,
                             _p, _i64, _p, _i64]
    lib.mxo_gemm_at.argtypes = [_i64, _p, _i64, _p, _i64, ctypes.c_int, _p, _i64, _p, _i64, ctypes.c_int, _p, _p,
                                _i64, _p, _p]
    lib.mxo_paged_attention.argtypes = [_p, _p, _i64, _i64, _p, _p, _p, _p, _p, _i64, _p, _i64, _i64, _i64, _i64,
                                        _i64, _i64, ctypes.c_double, ctypes.c_int, _p, _i64, _p, _p, _p, _p]
    lib.mxo_scale_code_rule.restype = ctypes.c_uint
    lib.mxo_scale_code_rule.argtypes = [ctypes.c_int, _p, _i64, ctypes.c_int]
    lib.mxo_quantize_rows_rule.argtypes = [_p, ctypes.c_int, _i64, _i64, _i64, ctypes.c_int, ctypes.c_int, _p, _i64, _p,
                                           _i64]
    lib.mxo_quantize_cols_rule.argtypes = [_p, ctypes.c_int, _i64, _i64, _i64, ctypes.c_int, ctypes.c_int, _p, _i64, _p,
                                           _i64]
    lib.mxo_quantize_2d.argtypes = [_p, ctypes.c_int, _i64, _i64, _i64, ctypes.c_int, ctypes.c_int, _p, _i64, _p, _i64,
                                    _p, _i64, _p, _i64]
    lib.mxo_scale_broadcast.argtypes = [_p, _i64, ctypes.c_int, _i64, _i64, _p, _i64]
    lib.mxo_num_threads.restype = ctypes.c_int
    lib.mxo_set_num_threads.argtypes = [ctypes.c_int]
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def _in_dtype(x: np.ndarray) -> int:
    if x.dtype == np.float32:
        return F32
    if x.dtype == np.uint16:
        return BF16
    raise TypeError("oracle inputs are float32 or bf16 bit patterns (uint16), got %s" % x.dtype)


def _check(rc: int):
    if rc != 0:
        raise ValueError("oracle rejected the shape (status %d)" % rc)


# ---- scalar helpers -------------------------------------------------------
def decode(fmt: int, code: int) -> float:
    return _load().mxo_decode(fmt, code)


def decode_e8m0(e: int) -> float:
    return _load().mxo_decode_e8m0(e)


def encode(fmt: int, y: float) -> int:
    return _load().mxo_encode(fmt, float(y))


def scale_code(fmt: int, block, rule: int = RULE_FLOOR) -> int:
    v = np.ascontiguousarray(block, dtype=np.float64)
    return _load().mxo_scale_code_rule(fmt, _ptr(v), v.size, rule)


def double_to_bf16(v: float) -> int:
    return _load().mxo_double_to_bf16(float(v))


def dequant_value(fmt: int, code: int, scale: int) -> float:
    return _load().mxo_dequant_value(fmt, code, scale)


def decode_table(fmt: int) -> np.ndarray:
    n = 16 if fmt == E2M1 else 256
    return np.array([decode(fmt, c) for c in range(n)], dtype=np.float64)


def code_bytes(fmt: int, n: int) -> int:
    """Bytes holding n codes of the format."""
    return n // 2 if fmt == E2M1 else n


# ---- array operations -----------------------------------------------------
def quantize_rows(x: np.ndarray, fmt: int, rule: int = RULE_FLOOR):
    """Rowwise MX quantization: returns (codes [R, C] uint8 (E2M1: [R, C/2]
    packed), scales [R, C/32] uint8)."""
    x = np.ascontiguousarray(x)
    rows, cols = x.shape
    cb = code_bytes(fmt, cols)
    q = np.empty((rows, cb), np.uint8)
    s = np.empty((rows, cols // BLOCK), np.uint8)
    _check(_load().mxo_quantize_rows_rule(_ptr(x), _in_dtype(x), rows, cols, cols, fmt, rule, _ptr(q), cb, _ptr(s),
                                          cols // BLOCK))
    return q, s


def quantize_cols(x: np.ndarray, fmt: int, rule: int = RULE_FLOOR):
    """Colwise MXFP8 (blocks down columns), stored transposed:
    returns (codes^T [C, R] uint8, scales^T [C, R/32] uint8)."""
    x = np.ascontiguousarray(x)
    rows, cols = x.shape
    rb = code_bytes(fmt, rows)
    qt = np.empty((cols, rb), np.uint8)
    st = np.empty((cols, rows // BLOCK), np.uint8)
    _check(_load().mxo_quantize_cols_rule(_ptr(x), _in_dtype(x), rows, cols, cols, fmt, rule, _ptr(qt), rb, _ptr(st),
                                          rows // BLOCK))
    return qt, st


def quantize_2d(x: np.ndarray, fmt: int, rule: int = RULE_FLOOR):
    """One scale per 32 x 32 block: returns (q [R, C], s [R, C/32], qt [C, R],
    st [C, R/32]) with s and st the block scales expanded to the MXFP8 layout."""
    x = np.ascontiguousarray(x)
    rows, cols = x.shape
    q = np.empty((rows, cols), np.uint8)
    s = np.empty((rows, cols // BLOCK), np.uint8)
    qt = np.empty((cols, rows), np.uint8)
    st = np.empty((cols, rows // BLOCK), np.uint8)
    _check(_load().mxo_quantize_2d(_ptr(x), _in_dtype(x), rows, cols, cols, fmt, rule, _ptr(q), cols, _ptr(s),
                                   cols // BLOCK, _ptr(qt), rows, _ptr(st), rows // BLOCK))
    return q, s, qt, st


def scale_broadcast(s_in: np.ndarray, layout: int, rows: int, cols: int) -> np.ndarray:
    """Power-of-two FP32 block scales (layout 0: [rows, cols/128] for 1 x 128
    blocks; layout 1: [ceil(rows/128), cols/128] for 128 x 128 blocks) ->
    E8M0 scales [rows, cols/32]."""
    s_in = np.ascontiguousarray(s_in, dtype=np.float32)
    out = np.empty((rows, cols // BLOCK), np.uint8)
    _check(_load().mxo_scale_broadcast(_ptr(s_in), s_in.shape[1], layout, rows, cols, _ptr(out), cols // BLOCK))
    return out


def kv_quant_write(k: np.ndarray, v: np.ndarray, slot_mapping: np.ndarray, page_size: int, num_pages: int,
                   k_cache=None, k_scale=None, v_cache=None, v_scale=None):
    """Fused quantize + paged write of K and V [T, H, D] into the caches.

    Caches are [num_pages, page_size, H, D] uint8 and scales
    [num_pages, page_size, H, D/32] uint8; pass existing arrays to update them
    in place (slots not named by slot_mapping keep their contents)."""
    k = np.ascontiguousarray(k)
    v = np.ascontiguousarray(v)
    assert k.shape == v.shape and k.dtype == v.dtype
    T, H, D = k.shape
    shape_c = (num_pages, page_size, H, D)
    shape_s = (num_pages, page_size, H, D // BLOCK)
    k_cache = np.zeros(shape_c, np.uint8) if k_cache is None else k_cache
    v_cache = np.zeros(shape_c, np.uint8) if v_cache is None else v_cache
    k_scale = np.zeros(shape_s, np.uint8) if k_scale is None else k_scale
    v_scale = np.zeros(shape_s, np.uint8) if v_scale is None else v_scale
    sm = np.ascontiguousarray(slot_mapping, dtype=np.int64)
    _check(_load().mxo_kv_quant_write(_ptr(k), _ptr(v), _in_dtype(k), T, H, D, H * D, _ptr(sm), _ptr(k_cache),
                                      _ptr(k_scale), _ptr(v_cache), _ptr(v_scale), page_size, num_pages))
    return k_cache, k_scale, v_cache, v_scale


def dequantize(q: np.ndarray, s: np.ndarray, fmt: int, out: str = "f32") -> np.ndarray:
    """x_hat = s * q rounded to f32 (np.float32) or bf16 (np.uint16 patterns)."""
    q = np.ascontiguousarray(q, dtype=np.uint8)
    s = np.ascontiguousarray(s, dtype=np.uint8)
    rows, cols = q.shape[0], s.shape[1] * BLOCK
    assert q.shape[1] == code_bytes(fmt, cols)
    if out == "f32":
        y = np.empty((rows, cols), np.float32)
        ydt = F32
    else:
        y = np.empty((rows, cols), np.uint16)
        ydt = BF16
    _check(_load().mxo_dequantize(_ptr(q), q.shape[1], _ptr(s), s.shape[1], fmt, rows, cols, _ptr(y), ydt, cols))
    return y


def gemm(a: np.ndarray, sa: np.ndarray, afmt: int, b: np.ndarray, sb: np.ndarray, bfmt: int):
    """Block-scaled product y = A * B^T with A [M, K], B [N, K] codes (E2M1
    operands packed: [M, K/2] bytes); K is taken from the scales.

    Returns (y [M, N] float64, t [M, N] float64) with t = sum_k |a_k b_k|."""
    a = np.ascontiguousarray(a, dtype=np.uint8)
    b = np.ascontiguousarray(b, dtype=np.uint8)
    sa = np.ascontiguousarray(sa, dtype=np.uint8)
    sb = np.ascontiguousarray(sb, dtype=np.uint8)
    M, N = a.shape[0], b.shape[0]
    K = sa.shape[1] * BLOCK
    assert a.shape[1] == code_bytes(afmt, K) and b.shape[1] == code_bytes(bfmt, K) and sb.shape == (N, K // BLOCK)
    y = np.empty((M, N), np.float64)
    t = np.empty((M, N), np.float64)
    _check(_load().mxo_gemm(M, N, K, _ptr(a), a.shape[1], _ptr(sa), K // BLOCK, afmt, _ptr(b), b.shape[1], _ptr(sb),
                            K // BLOCK, bfmt, _ptr(y), N, _ptr(t), N))
    return y, t


def gemm_at(a: np.ndarray, sa: np.ndarray, afmt: int, b: np.ndarray, sb: np.ndarray, bfmt: int,
            mi: np.ndarray, ni: np.ndarray):
    """The block-scaled product at output coordinates (mi[i], ni[i]) only."""
    a = np.ascontiguousarray(a, dtype=np.uint8)
    b = np.ascontiguousarray(b, dtype=np.uint8)
    sa = np.ascontiguousarray(sa, dtype=np.uint8)
    sb = np.ascontiguousarray(sb, dtype=np.uint8)
    K = sa.shape[1] * BLOCK
    assert a.shape[1] == code_bytes(afmt, K) and b.shape[1] == code_bytes(bfmt, K)
    mi = np.ascontiguousarray(mi, dtype=np.int64)
    ni = np.ascontiguousarray(ni, dtype=np.int64)
    assert mi.shape == ni.shape
    assert mi.size == 0 or (0 <= mi.min() and mi.max() < a.shape[0] and 0 <= ni.min() and ni.max() < b.shape[0])
    y = np.empty(mi.shape, np.float64)
    t = np.empty(mi.shape, np.float64)
    _check(_load().mxo_gemm_at(K, _ptr(a), a.shape[1], _ptr(sa), sa.shape[1], afmt, _ptr(b), b.shape[1], _ptr(sb),
                               sb.shape[1], bfmt, _ptr(mi), _ptr(ni), mi.size, _ptr(y), _ptr(t)))
    return y, t


def paged_scores_at(q_codes, q_scales, k_cache, k_scale, page_table, seq_len, page_size, head, seq, i, j):
    """QK^T score of query token i against key token j of sequence `seq`, head
    `head`, reading K through the page table. q_codes [T, H, D] with token
    index seq*seq_len + i; k_cache [P, page_size, H, D]."""
    D = q_codes.shape[2]
    page = page_table[seq, j // page_size]
    krow = k_cache[page, j % page_size, head][None, :]
    ks = k_scale[page, j % page_size, head][None, :]
    qrow = q_codes[seq * seq_len + i, head][None, :]
    qs = q_scales[seq * seq_len + i, head][None, :]
    y, t = gemm(qrow, qs, E4M3, krow, ks, E4M3)
    return float(y[0, 0]), float(t[0, 0])


def paged_attention(q_codes, q_scales, k_cache, k_scale, v_cache, v_scale, page_table, kv_lens, q_len,
                    sm_scale, causal=False, rows=None):
    """Attention of MXFP8 queries over the paged MXFP8 KV cache (see
    mxo_paged_attention in mx_oracle.c for the definition).

    q_codes [S*q_len, Hq, D] / q_scales [S*q_len, Hq, D/32]; k_cache, v_cache
    [pages, page_size, Hkv, D] / k_scale, v_scale [pages, page_size, Hkv,
    D/32]; page_table int32 [S, pages_per_seq]; kv_lens int32 [S]. `rows`:
    optional flat (token * Hq + head) indices to evaluate; default all.

    Returns (o, w, lse, tmax): o and w [n, D] float64 (w = sum_j P_j |Vb_j|),
    lse and tmax [n] float64, n = len(rows) or S*q_len*Hq (token-major)."""
    q_codes = np.ascontiguousarray(q_codes, dtype=np.uint8)
    q_scales = np.ascontiguousarray(q_scales, dtype=np.uint8)
    k_cache = np.ascontiguousarray(k_cache, dtype=np.uint8)
    k_scale = np.ascontiguousarray(k_scale, dtype=np.uint8)
    v_cache = np.ascontiguousarray(v_cache, dtype=np.uint8)
    v_scale = np.ascontiguousarray(v_scale, dtype=np.uint8)
    page_table = np.ascontiguousarray(page_table, dtype=np.int32)
    kv_lens = np.ascontiguousarray(kv_lens, dtype=np.int32)
    T, Hq, D = q_codes.shape
    n_pages, page_size, Hkv, D2 = k_cache.shape
    S, pps = page_table.shape
    assert D2 == D and v_cache.shape == k_cache.shape and T == S * q_len and kv_lens.shape == (S,)
    assert q_scales.shape == (T, Hq, D // BLOCK) and k_scale.shape == v_scale.shape == (n_pages, page_size, Hkv, D // BLOCK)
    assert page_table.size == 0 or (page_table.min() >= 0 and page_table.max() < n_pages)
    if rows is None:
        n, rp = T * Hq, None
    else:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        assert rows.size == 0 or (rows.min() >= 0 and rows.max() < T * Hq)
        n, rp = rows.size, _ptr(rows)
    o = np.empty((n, D), np.float64)
    w = np.empty((n, D), np.float64)
    lse = np.empty(n, np.float64)
    tmax = np.empty(n, np.float64)
    _check(_load().mxo_paged_attention(_ptr(q_codes), _ptr(q_scales), Hq * D, Hq * (D // BLOCK), _ptr(k_cache),
                                       _ptr(k_scale), _ptr(v_cache), _ptr(v_scale), _ptr(page_table), pps,
                                       _ptr(kv_lens), S, q_len, Hq, Hkv, D, page_size, float(sm_scale), int(causal),
                                       rp, n, _ptr(o), _ptr(w), _ptr(lse), _ptr(tmax)))
    return o, w, lse, tmax


def num_threads() -> int:
    return _load().mxo_num_threads()


def set_num_threads(n: int):
    _load().mxo_set_num_threads(n)
