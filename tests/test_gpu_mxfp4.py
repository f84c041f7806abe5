"""GPU parity of the MXFP4 path (E2M1 codes, E8M0 scale per 32) against the oracle.

Codes (two per byte, element 2i in the low nibble) and scales must match the
oracle bit for bit, rowwise and colwise (stored transposed); dequantized
values too. The product y = A * B^T of two MXFP4 operands must satisfy
|y_gpu - y_ref| <= 1e-5 * sum_k |a_k b_k| per element (f32 output; bf16
output adds its own rounding, 2^-8 of |y|), on the large-tile kernel and on
every other shape (general kernel), on the scaled instruction and in the
FP32-accumulation mode. A product of E2M1 with E4M3 / E5M2 is held to
1e-5 * sum |a b| in the FP32-accumulation mode (AUTO's choice for it) and
to the grouped bound 2^-10 * sum |a b| on the scaled instruction; the worst
ratios found are printed.
"""
import numpy as np
import pytest

from gpu_util import FP8_GROUPED_REL, REL_T, assert_bitexact, assert_gemm_bound, bf16_to_f64, dev, host
from microscaling_block_scaled_amd import inputs

pytestmark = pytest.mark.gpu

E4M3, E5M2, E2M1 = 0, 1, 2
AUTO, FP8, FP32 = 0, 1, 2


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


def test_gemm_mxfp4_walk(mx, oracle):
    """4352 x 4096 x 1024 MXFP4: 272 whole tiles, more than a 256-CU part
    has CUs, so the large-tile kernel walks tiles (16 work-groups take a
    second one); every column of the first and last row of each row tile
    and of 3 others against the oracle, f32 and bf16 out."""
    import torch
    M, N, K = 4352, 4096, 1024
    a = inputs.normal_bf16(380, (M, K))
    b = inputs.normal_bf16(381, (N, K))
    qa_o, sa_o = oracle.quantize_rows(a, E2M1)
    qb_o, sb_o = oracle.quantize_rows(b, E2M1)
    g = inputs.rng(382)
    rows = sorted({r for t0 in range(0, M, 256) for r in [t0, t0 + 255] + list(g.integers(t0, t0 + 256, 3))})
    rows = np.array(rows)
    y_ref, t_ref = oracle.gemm(qa_o[rows], sa_o[rows], E2M1, qb_o, sb_o, E2M1)
    qa, sa, qb, sb = dev(qa_o), dev(sa_o), dev(qb_o), dev(sb_o)
    y = host(mx.mx_gemm(qa, sa, qb, sb, a_fmt=E2M1, b_fmt=E2M1, out_dtype=torch.float32))[rows]
    worst = assert_gemm_bound(y.astype(np.float64), y_ref, t_ref, "mxfp4 walk f32")
    yb = host(mx.mx_gemm(qa, sa, qb, sb, a_fmt=E2M1, b_fmt=E2M1, out_dtype=torch.bfloat16))[rows]
    assert_gemm_bound(bf16_to_f64(yb), y_ref, t_ref, "mxfp4 walk bf16", bf16_out=True)
    print("mxfp4 walk %dx%dx%d: worst |err|/T = %.3g" % (M, N, K, worst))


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


# --------------------------------------------------------------------------- colwise MXFP4
@pytest.mark.parametrize("rows,cols,seed", [(32, 8, 1), (64, 96, 2), (4096, 296, 3), (160, 1032, 4)])
@pytest.mark.parametrize("f32", [False, True])
def test_quantize_colwise_mxfp4(mx, oracle, rows, cols, seed, f32):
    """Blocks of 32 down each column, stored transposed [cols, rows/2]: the
    codes and scales of the oracle's colwise quantization, bit for bit (NaN,
    Inf and all-zero column blocks included; column counts off the 128-column
    tile; x's pitch 16-byte aligned as the colwise call requires)."""
    x = inputs.normal_bf16(350 + seed, (rows, cols))
    x[::29, :] = inputs.f32_to_bf16_bits(inputs.bf16_bits_to_f32(x[::29, :]) * np.float32(2.0 ** 9))
    x[3, 0] = 0x7FC0                 # NaN in column block (0, 0)
    if cols > 5:
        x[rows - 1, 5] = 0x7F80      # +Inf in the last block of column 5
        x[:32, cols - 1] = 0         # an all-zero block
    if f32:
        x = inputs.bf16_bits_to_f32(x) * np.float32(1.0 + 2.0 ** -12)
    qt, st = mx.mx_quantize_colwise(dev(x, bf16=not f32), E2M1)
    qo, so = oracle.quantize_cols(x, E2M1)
    assert host(qt).shape == (cols, rows // 2)
    assert_bitexact(host(st), so, "E2M1 colwise scales")
    assert_bitexact(host(qt), qo, "E2M1 colwise codes")


def test_quantize_ex_both_orientations_mxfp4(mx, oracle):
    """mx_quantize_ex with both 1-D outputs in E2M1 (one pass per output)."""
    x = inputs.normal_bf16(360, (256, 160))
    q, s, qt, st = mx.mx_quantize_ex(dev(x, bf16=True), E2M1, rowwise=True, colwise=True)
    qo, so = oracle.quantize_rows(x, E2M1)
    qto, sto = oracle.quantize_cols(x, E2M1)
    assert_bitexact(host(q), qo, "rowwise codes")
    assert_bitexact(host(s), so, "rowwise scales")
    assert_bitexact(host(qt), qto, "colwise codes")
    assert_bitexact(host(st), sto, "colwise scales")


def test_gemm_colwise_mxfp4_operands(mx, oracle):
    """A weight-gradient-shaped product of two colwise MXFP4 operands:
    dW [N, M] = G^T X with G [K, N] and X [K, M], both quantized down their
    columns (K-contiguous after the transpose)."""
    import torch
    K, N, M = 1024, 320, 192
    gx = inputs.normal_bf16(361, (K, N))
    xx = inputs.normal_bf16(362, (K, M))
    qg, sg = mx.mx_quantize_colwise(dev(gx, bf16=True), E2M1)
    qx, sx = mx.mx_quantize_colwise(dev(xx, bf16=True), E2M1)
    qgo, sgo = oracle.quantize_cols(gx, E2M1)
    qxo, sxo = oracle.quantize_cols(xx, E2M1)
    assert_bitexact(host(qg), qgo, "G^T codes")
    assert_bitexact(host(qx), qxo, "X^T codes")
    y_ref, t_ref = oracle.gemm(qgo, sgo, E2M1, qxo, sxo, E2M1)
    y = mx.mx_gemm(qg, sg, qx, sx, a_fmt=E2M1, b_fmt=E2M1, out_dtype=torch.float32)
    worst = assert_gemm_bound(host(y).astype(np.float64), y_ref, t_ref, "colwise mxfp4 product")
    print("colwise MXFP4 G^T X %dx%dx%d: worst |err|/T = %.3g" % (N, M, K, worst))


# --------------------------------------------------------------------------- MXFP4 products of any shape
GENERAL_SHAPES = [(1, 1, 32), (64, 64, 128), (100, 37, 96), (130, 129, 160), (300, 257, 1056), (200, 600, 2048)]


@pytest.mark.parametrize("M,N,K", GENERAL_SHAPES)
@pytest.mark.parametrize("accum", [AUTO, FP8, FP32])
def test_gemm_mxfp4_any_shape(mx, oracle, M, N, K, accum):
    """Shapes the large-tile kernel does not take (K % 1024 != 0, M or N
    below 256): the general kernel, on the instruction (exact up to the f32
    sum) and in the FP32-accumulation mode."""
    import torch
    a = inputs.normal_bf16(370 + M + K, (M, K))
    b = inputs.normal_bf16(371 + N + K, (N, K))
    qa, sa = oracle.quantize_rows(a, E2M1)
    qb, sb = oracle.quantize_rows(b, E2M1)
    y_ref, t_ref = oracle.gemm(qa, sa, E2M1, qb, sb, E2M1)
    what = "mxfp4 %dx%dx%d accum %d" % (M, N, K, accum)
    y = mx.mx_gemm(dev(qa), dev(sa), dev(qb), dev(sb), a_fmt=E2M1, b_fmt=E2M1, out_dtype=torch.float32, accum=accum)
    worst = assert_gemm_bound(host(y).astype(np.float64), y_ref, t_ref, what + " f32")
    yb = mx.mx_gemm(dev(qa), dev(sa), dev(qb), dev(sb), a_fmt=E2M1, b_fmt=E2M1, out_dtype=torch.bfloat16,
                    accum=accum)
    assert_gemm_bound(bf16_to_f64(host(yb)), y_ref, t_ref, what + " bf16", bf16_out=True)
    print("%s: worst |err|/T = %.3g" % (what, worst))


# --------------------------------------------------------------------------- E2M1 x E4M3 / E5M2
MIXED = [(E2M1, E4M3), (E2M1, E5M2), (E4M3, E2M1), (E5M2, E2M1)]
MIXED_SHAPES = [(64, 64, 128), (300, 200, 96), (256, 512, 1024), (513, 1000, 2048)]


@pytest.mark.parametrize("afmt,bfmt", MIXED)
@pytest.mark.parametrize("M,N,K", MIXED_SHAPES)
def test_gemm_e2m1_times_fp8(mx, oracle, afmt, bfmt, M, N, K):
    import torch
    a = inputs.normal_bf16(380 + M + 3 * afmt, (M, K))
    b = inputs.normal_bf16(381 + N + 3 * bfmt, (N, K))
    qa, sa = mx.mx_quantize(dev(a, bf16=True), afmt)
    qb, sb = mx.mx_quantize(dev(b, bf16=True), bfmt)
    qa_o, sa_o = oracle.quantize_rows(a, afmt)
    qb_o, sb_o = oracle.quantize_rows(b, bfmt)
    assert_bitexact(host(qa), qa_o, "A codes")
    assert_bitexact(host(qb), qb_o, "B codes")
    y_ref, t_ref = oracle.gemm(qa_o, sa_o, afmt, qb_o, sb_o, bfmt)
    worst = {}
    for accum in (AUTO, FP8, FP32):
        rel = FP8_GROUPED_REL if accum == FP8 else REL_T
        what = "%d x %d %dx%dx%d accum %d" % (afmt, bfmt, M, N, K, accum)
        y = mx.mx_gemm(qa, sa, qb, sb, a_fmt=afmt, b_fmt=bfmt, out_dtype=torch.float32, accum=accum)
        worst[accum] = assert_gemm_bound(host(y).astype(np.float64), y_ref, t_ref, what + " f32", rel=rel)
        yb = mx.mx_gemm(qa, sa, qb, sb, a_fmt=afmt, b_fmt=bfmt, out_dtype=torch.bfloat16, accum=accum)
        assert_gemm_bound(bf16_to_f64(host(yb)), y_ref, t_ref, what + " bf16", bf16_out=True, rel=rel)
    print("E2M1 mixed %d x %d %dx%dx%d: worst |err|/T AUTO %.3g FP8 %.3g FP32 %.3g" % (
        afmt, bfmt, M, N, K, worst[AUTO], worst[FP8], worst[FP32]))


@pytest.mark.parametrize("afmt,bfmt", MIXED)
def test_gemm_e2m1_times_fp8_random_codes(mx, oracle, afmt, bfmt):
    """Codes drawn uniformly from every finite value of both formats and
    scales from a wide range."""
    import torch
    g = inputs.rng(390 + afmt + 4 * bfmt)
    M, N, K = 192, 320, 512

    def codes(fmt, rows):
        if fmt == E2M1:
            return g.integers(0, 256, (rows, K // 2), dtype=np.uint8)
        c = g.integers(0, 256, (rows, K), dtype=np.uint8)
        bad = (c & 0x7F) == 0x7F if fmt == E4M3 else (c & 0x7F) >= 0x7C  # NaN (and E5M2 Inf) codes
        c[bad] ^= 0x08
        return c

    qa, qb = codes(afmt, M), codes(bfmt, N)
    sa = g.integers(100, 150, (M, K // 32), dtype=np.uint8)
    sb = g.integers(100, 150, (N, K // 32), dtype=np.uint8)
    y_ref, t_ref = oracle.gemm(qa, sa, afmt, qb, sb, bfmt)
    worst = {}
    for accum in (AUTO, FP8):
        y = mx.mx_gemm(dev(qa), dev(sa), dev(qb), dev(sb), a_fmt=afmt, b_fmt=bfmt, out_dtype=torch.float32,
                       accum=accum)
        worst[accum] = assert_gemm_bound(host(y).astype(np.float64), y_ref, t_ref, "mixed random codes",
                                         rel=FP8_GROUPED_REL if accum == FP8 else REL_T)
    print("E2M1 mixed %d x %d random codes: worst |err|/T AUTO %.3g FP8 %.3g" % (afmt, bfmt, worst[AUTO], worst[FP8]))


def test_gemm_e2m1_paged_b(mx, oracle):
    """An E4M3 A against an E2M1 B read through a page table (rows of B in
    pages of 64, pages out of order), N ragged."""
    import ctypes
    import torch
    from microscaling_block_scaled_amd import _lib
    M, N, K, page_rows = 96, 300, 256, 64
    pages_per_seq = (N + page_rows - 1) // page_rows
    n_pages = pages_per_seq + 3
    g = inputs.rng(395)
    table = g.permutation(n_pages)[:pages_per_seq].astype(np.int32)
    a = inputs.normal_bf16(396, (M, K))
    bpages = inputs.normal_bf16(397, (n_pages * page_rows, K))
    qa, sa = oracle.quantize_rows(a, E4M3)
    qbp, sbp = oracle.quantize_rows(bpages, E2M1)
    rows = table[np.arange(N) // page_rows].astype(np.int64) * page_rows + np.arange(N) % page_rows
    y_ref, t_ref = oracle.gemm(qa, sa, E4M3, np.ascontiguousarray(qbp[rows]), np.ascontiguousarray(sbp[rows]), E2M1)
    dqa, dsa, dqb, dsb, dtab = dev(qa), dev(sa), dev(qbp), dev(sbp), dev(table)
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    d = mx.mx_gemm_desc_t()
    d.M, d.N, d.K = M, N, K
    d.a, d.lda, d.sa, d.ldsa, d.a_fmt = dqa.data_ptr(), K, dsa.data_ptr(), K // 32, E4M3
    d.b, d.ldb, d.sb, d.ldsb, d.b_fmt = dqb.data_ptr(), K // 2, dsb.data_ptr(), K // 32, E2M1
    d.y, d.ldy, d.y_dtype = y.data_ptr(), N, 0
    d.b_page_table = dtab.data_ptr()
    d.b_pages_per_seq, d.b_page_rows = pages_per_seq, page_rows
    d.b_page_stride, d.b_page_stride_s = page_rows * (K // 2), page_rows * (K // 32)
    d.accum = AUTO
    mx.mx_gemm_desc(d)
    torch.cuda.synchronize()
    worst = assert_gemm_bound(host(y).astype(np.float64), y_ref, t_ref, "paged E2M1 B")
    print("paged E4M3 x E2M1: worst |err|/T = %.3g" % worst)
