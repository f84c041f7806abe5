"""ctypes binding of libmxfp8 (include/mxfp8.h).

Argument marshalling only: every step runs in the HIP library. torch supplies
device memory and the current stream. There is no fallback: if the library is
not built, or a call returns an error, this module raises.
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmxfp8.so")

MX_OK = 0
MX_E4M3 = 0
MX_E5M2 = 1
MX_E2M1 = 2  # MXFP4: codes packed two per byte, element 2i in the low nibble
MX_F32 = 0
MX_BF16 = 1
MX_ACCUM_AUTO = 0
MX_ACCUM_FP8 = 1
MX_ACCUM_FP32 = 2
MX_SCALE_FLOOR = 0
MX_SCALE_CEIL = 1
MX_BLOCKS_1D = 0
MX_BLOCKS_2D = 1
MX_BCAST_1X128 = 0
MX_BCAST_128X128 = 1
BLOCK = 32

_i64 = ctypes.c_int64
_i32 = ctypes.c_int32
_p = ctypes.c_void_p


class MXError(RuntimeError):
    def __init__(self, func, status, text):
        super().__init__("%s failed: %s (%d)" % (func, text, status))
        self.status = status


class mx_gemm_desc_t(ctypes.Structure):
    _fields_ = [
        ("M", _i64), ("N", _i64), ("K", _i64),
        ("a", _p), ("lda", _i64), ("sa", _p), ("ldsa", _i64), ("a_fmt", ctypes.c_int),
        ("b", _p), ("ldb", _i64), ("sb", _p), ("ldsb", _i64), ("b_fmt", ctypes.c_int),
        ("y", _p), ("ldy", _i64), ("y_dtype", ctypes.c_int),
        ("batch_outer", _i64), ("batch_inner", _i64),
        ("stride_a_outer", _i64), ("stride_a_inner", _i64), ("stride_sa_outer", _i64), ("stride_sa_inner", _i64),
        ("stride_b_outer", _i64), ("stride_b_inner", _i64), ("stride_sb_outer", _i64), ("stride_sb_inner", _i64),
        ("stride_y_outer", _i64), ("stride_y_inner", _i64),
        ("b_page_table", _p),
        ("b_pages_per_seq", _i64), ("b_page_rows", _i64), ("b_page_stride", _i64), ("b_page_stride_s", _i64),
        ("accum", ctypes.c_int),
    ]


class mx_attention_desc_t(ctypes.Structure):
    _fields_ = [
        ("num_seqs", _i64), ("q_len", _i64), ("num_q_heads", _i64), ("num_kv_heads", _i64), ("head_dim", _i64),
        ("q", _p), ("ld_q", _i64), ("q_scale", _p), ("ld_qs", _i64),
        ("k_cache", _p), ("k_scale", _p), ("v_cache", _p), ("v_scale", _p),
        ("page_size", _i64),
        ("page_table", _p), ("pages_per_seq", _i64),
        ("kv_lens", _p),
        ("sm_scale", ctypes.c_float), ("causal", ctypes.c_int32),
        ("out", _p), ("ld_o", _i64), ("out_dtype", ctypes.c_int),
        ("lse", _p),
    ]


class mx_grouped_gemm_desc_t(ctypes.Structure):
    _fields_ = [
        ("groups", _i64), ("total_m", _i64), ("N", _i64), ("K", _i64),
        ("group_offsets", _p),
        ("a", _p), ("lda", _i64), ("sa", _p), ("ldsa", _i64), ("a_fmt", ctypes.c_int),
        ("b", _p), ("ldb", _i64), ("sb", _p), ("ldsb", _i64), ("b_fmt", ctypes.c_int),
        ("stride_b", _i64), ("stride_sb", _i64),
        ("y", _p), ("ldy", _i64), ("y_dtype", ctypes.c_int),
        ("accum", ctypes.c_int),
    ]


class mx_quantize_desc_t(ctypes.Structure):
    _fields_ = [
        ("x", _p), ("xdt", ctypes.c_int), ("rows", _i64), ("cols", _i64), ("ldx", _i64),
        ("fmt", ctypes.c_int), ("rule", ctypes.c_int), ("blocks", ctypes.c_int),
        ("q", _p), ("ldq", _i64), ("s", _p), ("lds", _i64),
        ("qt", _p), ("ldqt", _i64), ("st", _p), ("ldst", _i64),
    ]


_lib = None

# name -> (restype, argtypes)
SIGNATURES = {
    "mx_quantize": (_i32, [_p, ctypes.c_int, _i64, _i64, _i64, ctypes.c_int, _p, _i64, _p, _i64, _p]),
    "mx_quantize_colwise": (_i32, [_p, ctypes.c_int, _i64, _i64, _i64, ctypes.c_int, _p, _i64, _p, _i64, _p]),
    "mx_quantize_ex": (_i32, [ctypes.POINTER(mx_quantize_desc_t), _p]),
    "mx_scale_broadcast": (_i32, [_p, _i64, ctypes.c_int, _i64, _i64, _p, _i64, _p]),
    "mx_dequantize": (_i32, [_p, _i64, _p, _i64, ctypes.c_int, _i64, _i64, _p, ctypes.c_int, _i64, _p]),
    "mx_kv_quant_write": (_i32, [_p, _p, ctypes.c_int, _i64, _i64, _i64, _i64, _p, _p, _p, _p, _p, _i64, _i64, _p]),
    "mx_gemm": (_i32, [ctypes.POINTER(mx_gemm_desc_t), _p]),
    "mx_paged_attention": (_i32, [ctypes.POINTER(mx_attention_desc_t), _p]),
    "mx_grouped_gemm": (_i32, [ctypes.POINTER(mx_grouped_gemm_desc_t), _p]),
    "mx_status_string": (ctypes.c_char_p, [_i32]),
    "mx_query_support": (_i32, [ctypes.c_int, ctypes.POINTER(ctypes.c_char_p)]),
}


def lib():
    """Load libmxfp8.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libmxfp8.so is not built: run `python -m microscaling_block_scaled_amd.build` "
                              "(or __graft_entry__.build())")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(l, name)
            f.restype = res
            f.argtypes = args
        _lib = l
    return _lib


def check(func, status):
    if status != MX_OK:
        raise MXError(func, status, lib().mx_status_string(status).decode())
