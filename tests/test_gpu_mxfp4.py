"""GPU parity of the MXFP4 path (E2M1 codes, E8M0 scale per 32) against the oracle.

Codes (two per byte, element 2i in the low nibble) and scales must match the
oracle bit for bit; dequantized values too. The product y = A * B^T of two
MXFP4 operands must satisfy |y_gpu - y_ref| <= 1e-5 * sum_k |a_k b_k| per
element (f32 output; bf16 output adds its own rounding, 2^-8 of |y|).
"""
import numpy as np
import pytest

from gpu_util import assert_bitexact, assert_gemm_bound, bf16_to_f64, dev, host
from microscaling_block_scaled_amd import inputs

pytestmark = pytest.mark.gpu

E2M1 = 2


@pytest.fixture(scope="module")
def mx():
    import torch
    import microscaling_block_scaled_amd as m
    assert torch.cuda.is_available()
    ok, reason = m.mx_query_support(0)
    assert ok, reason
    return m


@pytest.mark.parametrize("rows,cols,seed", [(1, 32, 1), (7, 96, 2), (300, 4096, 3), (1031, 160, 4)])
@pytest.mark.parametrize("f32", [False, True])
def test_quantize_rowwise_mxfp4(mx, oracle, rows, cols, seed, f32):
    x = inputs.normal_bf16(300 + seed, (rows, cols))
    x[:, ::37] = inputs.f32_to_bf16_bits(inputs.bf16_bits_to_f32(x[:, ::37]) * np.float32(2.0 ** 9))
    if f32:
        x = inputs.bf16_bits_to_f32(x) * np.float32(1.0 + 2.0 ** -12)  # values between bf16 points
    q, s = mx.mx_quantize(dev(x, bf16=not f32), E2M1)
    qo, so = oracle.quantize_rows(x, E2M1)
    assert_bitexact(host(q), qo, "E2M1 codes")
    assert_bitexact(host(s), so, "E2M1 scales")


def test_quantize_mxfp4_every_bf16_value_and_special_blocks(mx, oracle):
    """Every finite bf16 magnitude under every scale the rule can produce
    (blocks anchored at 2^(c - 127 + 2)), both signs; then NaN / Inf blocks
    (scale 0xFF, codes 0) and zero blocks."""
    bits = np.arange(0x7F80, dtype=np.uint16)
    mag = inputs.bf16_bits_to_f32(bits).astype(np.float64)
    rows = []
    for c in range(0, 127 + 127 - 2 + 1, 3):
        anchor = 2.0 ** (c - 127 + 2)
        sel = bits[mag < 2 * anchor]
        sel = np.concatenate([sel, sel | np.uint16(0x8000)])
        pad = (-len(sel)) % 31
        sel = np.concatenate([sel, np.zeros(pad, np.uint16)]).reshape(-1, 31)
        anc = np.full((sel.shape[0], 1), inputs.f32_to_bf16_bits(np.float32([anchor]))[0], np.uint16)
        rows.append(np.concatenate([anc, sel], axis=1))
    x = np.concatenate(rows)
    x = np.concatenate([x, np.zeros(((-len(x)) % 4, 32), np.uint16)]).reshape(-1, 128)
    special = inputs.normal_bf16(310, (4, 128))
    special[0, 5] = 0x7FC0   # NaN
    special[1, 70] = 0x7F80  # +Inf
    special[2, 100] = 0xFF80  # -Inf
    special[3, :] = 0         # zeros
    x = np.concatenate([x, special])
    q, s = mx.mx_quantize(dev(x, bf16=True), E2M1)
    qo, so = oracle.quantize_rows(x, E2M1)
    assert_bitexact(host(s), so, "E2M1 scales (all values)")
    assert_bitexact(host(q), qo, "E2M1 codes (all values)")


@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_dequantize_mxfp4(mx, oracle, out):
    import torch
    x = inputs.normal_bf16(320, (257, 512))
    x[3, 40] = 0x7FC0
    qo, so = oracle.quantize_rows(x, E2M1)
    y = mx.mx_dequantize(dev(qo), dev(so), E2M1, out_dtype=torch.float32 if out == "f32" else torch.bfloat16)
    want = oracle.dequantize(qo, so, E2M1, out)
    got = host(y)
    assert_bitexact(got.view(np.uint32) if out == "f32" else got, want.view(np.uint32) if out == "f32" else want,
                    "E2M1 dequantize " + out)


SHAPES = [(256, 256, 1024), (300, 257, 1024), (513, 1000, 2048), (1024, 512, 4096)]


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_gemm_mxfp4(mx, oracle, M, N, K):
    import torch
    a = inputs.normal_bf16(330 + M, (M, K))
    b = inputs.normal_bf16(331 + N, (N, K))
    qa, sa = mx.mx_quantize(dev(a, bf16=True), E2M1)
    qb, sb = mx.mx_quantize(dev(b, bf16=True), E2M1)
    qa_o, sa_o = oracle.quantize_rows(a, E2M1)
    qb_o, sb_o = oracle.quantize_rows(b, E2M1)
    assert_bitexact(host(qa), qa_o, "A codes")
    assert_bitexact(host(qb), qb_o, "B codes")
    y_ref, t_ref = oracle.gemm(qa_o, sa_o, E2M1, qb_o, sb_o, E2M1)
    y = mx.mx_gemm(qa, sa, qb, sb, a_fmt=E2M1, b_fmt=E2M1, out_dtype=torch.float32)
    worst = assert_gemm_bound(host(y).astype(np.float64), y_ref, t_ref, "mxfp4 %dx%dx%d f32" % (M, N, K))
    print("mxfp4 %dx%dx%d: worst |err|/T = %.3g" % (M, N, K, worst))
    yb = mx.mx_gemm(qa, sa, qb, sb, a_fmt=E2M1, b_fmt=E2M1, out_dtype=torch.bfloat16)
    assert_gemm_bound(bf16_to_f64(host(yb)), y_ref, t_ref, "mxfp4 bf16", bf16_out=True)


def test_gemm_mxfp4_varied_scales_and_extreme_codes(mx, oracle):
    """Codes drawn uniformly from all 16 values and scales from a wide range:
    every (code, scale) combination reaches the instruction."""
    import torch
    g = inputs.rng(340)
    M, N, K = 384, 512, 2048
    qa = g.integers(0, 256, (M, K // 2), dtype=np.uint8)
    qb = g.integers(0, 256, (N, K // 2), dtype=np.uint8)
    sa = g.integers(100, 150, (M, K // 32), dtype=np.uint8)
    sb = g.integers(100, 150, (N, K // 32), dtype=np.uint8)
    y_ref, t_ref = oracle.gemm(qa, sa, E2M1, qb, sb, E2M1)
    y = mx.mx_gemm(dev(qa), dev(sa), dev(qb), dev(sb), a_fmt=E2M1, b_fmt=E2M1, out_dtype=torch.float32)
    assert_gemm_bound(host(y).astype(np.float64), y_ref, t_ref, "mxfp4 random codes")


@pytest.mark.slow
def test_gemm_mxfp4_8192_cubed_sampled(mx, oracle):
    """M = N = K = 8192 MXFP4 (the GEMM workload's inputs quantized to E2M1),
    bf16 output as timed; 4000 sampled outputs against the oracle."""
    import torch
    xa, xb = inputs.gemm_inputs()
    qa, sa = mx.mx_quantize(dev(xa, bf16=True), E2M1)
    qb, sb = mx.mx_quantize(dev(xb, bf16=True), E2M1)
    qa_o, sa_o = oracle.quantize_rows(xa, E2M1)
    qb_o, sb_o = oracle.quantize_rows(xb, E2M1)
    assert_bitexact(host(qa), qa_o, "A codes")
    y = mx.mx_gemm(qa, sa, qb, sb, a_fmt=E2M1, b_fmt=E2M1, out_dtype=torch.float32)
    g = inputs.rng(341)
    mi, ni = g.integers(0, 8192, 4000), g.integers(0, 8192, 4000)
    y_ref, t_ref = oracle.gemm_at(qa_o, sa_o, E2M1, qb_o, sb_o, E2M1, mi, ni)
    got = host(y[dev(mi), dev(ni)]).astype(np.float64)
    worst = assert_gemm_bound(got, y_ref, t_ref, "mxfp4 8192^3")
    print("mxfp4 8192^3: worst |err|/T = %.3g" % worst)
