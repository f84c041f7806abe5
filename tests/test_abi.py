"""CPU checks of the C ABI boundary (no GPU, no compute calls)."""
import ctypes
import os
import re
import subprocess

import pytest

from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "mxfp8.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+char\s*\*|mx_status_t)\s+(mx_\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def libmx():
    from microscaling_block_scaled_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from microscaling_block_scaled_amd import build
        build.build()
    return ctypes.CDLL(_lib.LIB_PATH)


def test_header_declares_the_five_operations_and_status_api():
    names = declared_functions()
    for n in ("mx_quantize", "mx_quantize_colwise", "mx_dequantize", "mx_gemm", "mx_kv_quant_write",
              "mx_paged_attention", "mx_status_string", "mx_query_support"):
        assert n in names, n


def test_library_exports_every_declared_symbol(libmx):
    from microscaling_block_scaled_amd import _lib
    names = declared_functions()
    assert names
    for n in names:
        assert hasattr(libmx, n), "libmxfp8.so does not export %s" % n
        assert n in _lib.SIGNATURES, "the Python binding does not declare %s" % n


def test_status_strings_without_gpu(libmx):
    libmx.mx_status_string.restype = ctypes.c_char_p
    libmx.mx_status_string.argtypes = [ctypes.c_int32]
    for code in (0, -1, -2, -3, -4, -5, -6):
        s = libmx.mx_status_string(code).decode()
        assert s.startswith("MX_")
    assert "unknown" in libmx.mx_status_string(12345).decode()


@pytest.mark.parametrize("name", ["mx_gemm_desc_t", "mx_attention_desc_t", "mx_grouped_gemm_desc_t",
                                  "mx_quantize_desc_t"])
def test_ctypes_descriptor_matches_c_layout(tmp_path, name):
    """Compile a probe against the real header with gcc and compare field
    offsets and size with the ctypes mirror used by the binding."""
    from microscaling_block_scaled_amd import _lib
    desc = getattr(_lib, name)
    fields = [f for f, _ in desc._fields_]
    src = tmp_path / "layout.c"
    src.write_text(
        '#include <stdio.h>\n#include <stddef.h>\n#include "mxfp8.h"\nint main(void){\n'
        + 'printf("size %%zu\\n", sizeof(%s));\n' % name
        + "".join('printf("%s %%zu\\n", offsetof(%s, %s));\n' % (f, name, f) for f in fields)
        + "return 0;}\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
                    str(src), "-o", str(exe)], check=True)
    out = dict(line.split() for line in subprocess.run([str(exe)], capture_output=True, text=True,
                                                       check=True).stdout.splitlines())
    assert int(out["size"]) == ctypes.sizeof(desc)
    for f in fields:
        assert int(out[f]) == getattr(desc, f).offset, f


def test_attention_argument_errors_without_gpu(libmx):
    """Host-side validation of mx_paged_attention runs before any device call;
    the pointers below are never dereferenced."""
    from microscaling_block_scaled_amd import _lib
    f = libmx.mx_paged_attention
    f.restype, f.argtypes = _lib.SIGNATURES["mx_paged_attention"]

    def desc(**kw):
        d = _lib.mx_attention_desc_t()
        base = dict(num_seqs=2, q_len=64, num_q_heads=4, num_kv_heads=2, head_dim=128, q=0x10000, ld_q=512,
                    q_scale=0x20000, ld_qs=16, k_cache=0x30000, k_scale=0x40000, v_cache=0x50000, v_scale=0x60000,
                    page_size=128, page_table=0x70000, pages_per_seq=4, kv_lens=0x80000, sm_scale=0.088, causal=0,
                    out=0x90000, ld_o=512, out_dtype=1, lse=None)
        base.update(kw)
        for k, v in base.items():
            setattr(d, k, v)
        return d

    assert f(None, None) == -1
    assert f(ctypes.byref(desc(q=None)), None) == -1
    assert f(ctypes.byref(desc(head_dim=64, ld_q=256, ld_qs=8, ld_o=256)), None) == -2
    assert f(ctypes.byref(desc(page_size=64)), None) == -2
    assert f(ctypes.byref(desc(num_kv_heads=3)), None) == -2
    assert f(ctypes.byref(desc(sm_scale=0.0)), None) == -2
    assert f(ctypes.byref(desc(sm_scale=float("nan"))), None) == -2
    assert f(ctypes.byref(desc(ld_q=256)), None) == -2
    assert f(ctypes.byref(desc(q=0x10008)), None) == -3
    assert f(ctypes.byref(desc(k_scale=0x40002)), None) == -3
    assert f(ctypes.byref(desc(out=0x90004)), None) == -3
    assert f(ctypes.byref(desc(out_dtype=7)), None) == -4
    # empty problems launch nothing and succeed
    assert f(ctypes.byref(desc(num_seqs=0)), None) == 0
    assert f(ctypes.byref(desc(q_len=0, q=None)), None) == 0


def test_mxfp4_argument_errors_without_gpu(libmx):
    """MXFP4 limits are checked on the host before any device call."""
    from microscaling_block_scaled_amd import _lib
    g = libmx.mx_gemm
    g.restype, g.argtypes = _lib.SIGNATURES["mx_gemm"]

    def desc(**kw):
        d = _lib.mx_gemm_desc_t()
        base = dict(M=512, N=512, K=2048, a=0x10000, lda=1024, sa=0x20000, ldsa=64, a_fmt=2, b=0x30000, ldb=1024,
                    sb=0x40000, ldsb=64, b_fmt=2, y=0x50000, ldy=512, y_dtype=1, accum=0)
        base.update(kw)
        for k, v in base.items():
            setattr(d, k, v)
        return d

    assert g(ctypes.byref(desc(accum=3)), None) == -4               # no such accumulation mode
    assert g(ctypes.byref(desc(a_fmt=3)), None) == -4               # no such element format
    assert g(ctypes.byref(desc(lda=512)), None) == -2               # pitch below K/2 bytes
    assert g(ctypes.byref(desc(b_fmt=0, ldb=1024)), None) == -2     # an E4M3 B row holds K bytes
    assert g(ctypes.byref(desc(K=2064, lda=1040, ldb=1040, ldsa=65, ldsb=65)), None) == -2  # K % 32
    q = libmx.mx_quantize_colwise
    q.restype, q.argtypes = _lib.SIGNATURES["mx_quantize_colwise"]
    assert q(0x10000, 1, 64, 64, 64, 2, 0x20000, 16, 0x30000, 2, None) == -2  # pitch below rows/2 bytes
    assert q(0x10000, 1, 64, 64, 64, 2, 0x20008, 32, 0x30000, 2, None) == -3  # codes 16-byte aligned
    assert q(0x10000, 1, 64, 64, 64, 3, 0x20000, 32, 0x30000, 2, None) == -4  # no such element format


def test_scale_variant_argument_errors_without_gpu(libmx):
    """mx_quantize_ex and mx_scale_broadcast check rule, block shape, shapes
    and alignment on the host before any device call."""
    from microscaling_block_scaled_amd import _lib
    f = libmx.mx_quantize_ex
    f.restype, f.argtypes = _lib.SIGNATURES["mx_quantize_ex"]

    def desc(**kw):
        d = _lib.mx_quantize_desc_t()
        base = dict(x=0x10000, xdt=1, rows=64, cols=64, ldx=64, fmt=0, rule=1, blocks=1, q=0x20000, ldq=64,
                    s=0x30000, lds=2, qt=0x40000, ldqt=64, st=0x50000, ldst=2)
        base.update(kw)
        for k, v in base.items():
            setattr(d, k, v)
        return d

    assert f(None, None) == -1
    assert f(ctypes.byref(desc(x=None)), None) == -1
    assert f(ctypes.byref(desc(q=None, s=None, qt=None, st=None)), None) == -1  # no output asked for
    assert f(ctypes.byref(desc(s=None)), None) == -1                          # half an output pair
    assert f(ctypes.byref(desc(rule=2)), None) == -4
    assert f(ctypes.byref(desc(blocks=3)), None) == -4
    assert f(ctypes.byref(desc(fmt=2)), None) == -4                           # 2-D MXFP4 not offered
    assert f(ctypes.byref(desc(blocks=0, fmt=2, q=None, s=None, ldqt=16)), None) == -2  # colwise MXFP4: rows/2 bytes
    assert f(ctypes.byref(desc(rows=48, ldqt=48)), None) == -2                # rows % 32
    assert f(ctypes.byref(desc(qt=0x40008)), None) == -3                      # transposed codes 16-aligned
    assert f(ctypes.byref(desc(ldq=32)), None) == -2
    assert f(ctypes.byref(desc(ldst=1)), None) == -2
    assert f(ctypes.byref(desc(q=0x20008)), None) == -3
    assert f(ctypes.byref(desc(x=0x10004)), None) == -3
    b = libmx.mx_scale_broadcast
    b.restype, b.argtypes = _lib.SIGNATURES["mx_scale_broadcast"]
    assert b(None, 2, 0, 64, 256, 0x20000, 8, None) == -1
    assert b(0x10000, 2, 2, 64, 256, 0x20000, 8, None) == -4                  # layout
    assert b(0x10000, 2, 0, 64, 224, 0x20000, 8, None) == -2                  # cols % 128
    assert b(0x10000, 1, 0, 64, 256, 0x20000, 8, None) == -2                  # ld_in below cols / 128
    assert b(0x10000, 2, 0, 64, 256, 0x20000, 4, None) == -2                  # ld_out below cols / 32
    assert b(0x10002, 2, 0, 64, 256, 0x20000, 8, None) == -3
    assert b(0x10000, 2, 0, 64, 256, 0x20000, 10, None) == -3                 # ld_out % 4


def test_binding_checks_buffers_before_any_call():
    """The binding knows each tensor's size, the C ABI only its pointer: a
    buffer of the wrong shape, dtype or layout is refused in Python."""
    import torch
    from microscaling_block_scaled_amd import _buf
    u8 = torch.uint8
    with pytest.raises(ValueError, match="shape"):
        _buf(torch.empty((63, 96), dtype=u8), "q", (64, 96), u8)
    with pytest.raises(TypeError, match="uint8"):
        _buf(torch.empty((64, 96), dtype=torch.int8), "q", (64, 96), u8)
    with pytest.raises(ValueError, match="unit stride"):
        _buf(torch.empty((96, 64), dtype=u8).t(), "q", (64, 96), u8)
    with pytest.raises(ValueError, match="overlapping"):
        _buf(torch.empty((1, 96), dtype=u8).expand(64, 96), "q", (64, 96), u8)
    with pytest.raises(ValueError, match="GPU"):
        _buf(torch.empty((64, 96), dtype=u8), "q", (64, 96), u8)
    # a padded pitch and an empty buffer pass the layout checks
    with pytest.raises(ValueError, match="GPU"):
        _buf(torch.empty((64, 128), dtype=u8)[:, :96], "q", (64, 96), u8)
    with pytest.raises(ValueError, match="GPU"):
        _buf(torch.empty((0, 96), dtype=u8), "q", (0, 96), u8)
