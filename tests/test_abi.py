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
              "mx_status_string", "mx_query_support"):
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


def test_ctypes_descriptor_matches_c_layout(tmp_path):
    """Compile a probe against the real header with gcc and compare field
    offsets and size with the ctypes mirror used by the binding."""
    from microscaling_block_scaled_amd._lib import mx_gemm_desc_t
    fields = [f for f, _ in mx_gemm_desc_t._fields_]
    src = tmp_path / "layout.c"
    src.write_text(
        '#include <stdio.h>\n#include <stddef.h>\n#include "mxfp8.h"\nint main(void){\n'
        + 'printf("size %zu\\n", sizeof(mx_gemm_desc_t));\n'
        + "".join('printf("%s %%zu\\n", offsetof(mx_gemm_desc_t, %s));\n' % (f, f) for f in fields)
        + "return 0;}\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
                    str(src), "-o", str(exe)], check=True)
    out = dict(line.split() for line in subprocess.run([str(exe)], capture_output=True, text=True,
                                                       check=True).stdout.splitlines())
    assert int(out["size"]) == ctypes.sizeof(mx_gemm_desc_t)
    for f in fields:
        assert int(out[f]) == getattr(mx_gemm_desc_t, f).offset, f
