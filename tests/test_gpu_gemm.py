"""GPU parity of the block-scaled matrix product against the oracle.

Bound (per output element): |y_gpu - y_ref| <= 1e-5 * sum_k |a_k b_k| for
f32 output; bf16 output adds its own rounding, 2^-8 of the magnitude. The
oracle quantizes the bf16 inputs itself and computes y_ref in fp64; the GPU
quantizes the same inputs with its own kernels (the codes are compared
bit for bit as well) and multiplies.
"""
import numpy as np
import pytest

from conftest import load_golden
from gpu_util import FP8_GROUPED_REL, REL_T, assert_bitexact, assert_gemm_bound, bf16_to_f64, check_every_output, dev, host
from microscaling_block_scaled_amd import inputs

pytestmark = pytest.mark.gpu

E4M3, E5M2 = 0, 1
AUTO, FP8, FP32 = 0, 1, 2


@pytest.fixture(scope="module")
def mx():
    import torch
    import microscaling_block_scaled_amd as m
    assert torch.cuda.is_available()
    ok, reason = m.mx_query_support(0)
    assert ok, reason
    return m


def _torch():
    import torch
    return torch


# --------------------------------------------------------------------------- page examples
@pytest.mark.parametrize("accum", [FP8, FP32])
def test_block_dot_example(mx, oracle, accum):
    """[NVFP4 page, section 7.2] q . p = 5.25, and with s_A s_B = 4, 21."""
    torch = _torch()
    ex = load_golden("block_dot_example.json")
    a = np.zeros((1, 128), np.uint8)
    b = np.zeros((1, 128), np.uint8)
    a[0, :4] = [oracle.encode(E4M3, v) for v in ex["q"]]
    b[0, :4] = [oracle.encode(E4M3, v) for v in ex["p"]]
    for sc, want in ((127, ex["dot"]), (128, ex["dot"] * 4)):
        s = np.full((1, 4), sc, np.uint8)
        y = host(mx.mx_gemm(dev(a), dev(s), dev(b), dev(s), out_dtype=torch.float32, accum=accum))
        assert y[0, 0] == want


@pytest.mark.parametrize("accum", [FP8, FP32])
def test_scales_stay_inside_the_sum(mx, oracle, accum):
    """[MXFP8 SM120 software support, section 0.3]: with different scales
    per block, the result is sum_b s_A s_B d_b, not one scale pair applied
    to the whole sum."""
    torch = _torch()
    a = np.zeros((16, 128), np.uint8)
    b = np.zeros((16, 128), np.uint8)
    one = oracle.encode(E4M3, 1.0)
    a[:, 0::32] = one
    b[:, 0::32] = one
    sa = np.tile(np.array([[130, 120, 127, 140]], np.uint8), (16, 1))
    sb = np.tile(np.array([[127, 127, 100, 110]], np.uint8), (16, 1))
    y = host(mx.mx_gemm(dev(a), dev(sa), dev(b), dev(sb), out_dtype=torch.float32, accum=accum))
    want = 2.0 ** 3 + 2.0 ** -7 + 2.0 ** -27 + 2.0 ** -4
    assert np.all(y == np.float32(want))


# --------------------------------------------------------------------------- tiny config
def test_tiny_config(mx, oracle):
    """v64 and A [64, 128] x B [128, 64] f32 ~ N(0,1): A rowwise, B colwise
    (blocks along K = 128), every output checked."""
    torch = _torch()
    t = inputs.tiny()
    A, B = t["A"], t["B"]
    qa, sa = mx.mx_quantize(dev(A), E4M3)
    qb, sb = mx.mx_quantize_colwise(dev(B), E4M3)
    qa_o, sa_o = oracle.quantize_rows(A, E4M3)
    qb_o, sb_o = oracle.quantize_cols(B, E4M3)
    assert_bitexact(host(qa), qa_o, "A codes")
    assert_bitexact(host(sa), sa_o, "A scales")
    assert_bitexact(host(qb), qb_o, "B^T codes")
    assert_bitexact(host(sb), sb_o, "B^T scales")
    y_ref, t_ref = oracle.gemm(qa_o, sa_o, E4M3, qb_o, sb_o, E4M3)
    y32 = host(mx.mx_gemm(qa, sa, qb, sb, out_dtype=torch.float32))
    assert_gemm_bound(y32, y_ref, t_ref, "tiny f32")
    ybf = host(mx.mx_gemm(qa, sa, qb, sb, out_dtype=torch.bfloat16))
    assert_gemm_bound(bf16_to_f64(ybf), y_ref, t_ref, "tiny bf16", bf16_out=True)
    # the worked vector against itself: 2^25 + 2^-19, which rounds to 2^25 in f32
    v = t["v64"]
    qv, sv = mx.mx_quantize(dev(v), E4M3)
    pad_q = torch.zeros((1, 128), dtype=torch.uint8, device="cuda")
    pad_s = torch.full((1, 4), 127, dtype=torch.uint8, device="cuda")
    pad_q[:, :64] = qv
    pad_s[:, :2] = sv
    yv = host(mx.mx_gemm(pad_q, pad_s, pad_q, pad_s, out_dtype=torch.float32))
    assert yv[0, 0] == np.float32(2.0 ** 25 + 2.0 ** -19)


# --------------------------------------------------------------------------- ragged shapes
SHAPES = [(1, 1, 32), (17, 33, 96), (130, 129, 160), (64, 64, 128), (257, 300, 416), (128, 256, 1024),
          (300, 17, 8192)]


@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("afmt,bfmt", [(E4M3, E4M3), (E5M2, E4M3), (E4M3, E5M2), (E5M2, E5M2)])
@pytest.mark.parametrize("accum", [AUTO, FP8, FP32])
def test_ragged_shapes(mx, oracle, M, N, K, afmt, bfmt, accum):
    torch = _torch()
    xa = inputs.normal_bf16(100 + M, (M, K))
    xb = inputs.normal_bf16(200 + N, (N, K), sigma=0.02)
    qa, sa = mx.mx_quantize(dev(xa, bf16=True), afmt)
    qb, sb = mx.mx_quantize(dev(xb, bf16=True), bfmt)
    qa_o, sa_o = oracle.quantize_rows(xa, afmt)
    qb_o, sb_o = oracle.quantize_rows(xb, bfmt)
    assert_bitexact(host(qa), qa_o, "A codes")
    assert_bitexact(host(qb), qb_o, "B codes")
    y_ref, t_ref = oracle.gemm(qa_o, sa_o, afmt, qb_o, sb_o, bfmt)
    rel = FP8_GROUPED_REL if accum == FP8 else 1e-5
    y = host(mx.mx_gemm(qa, sa, qb, sb, afmt, bfmt, out_dtype=torch.float32, accum=accum))
    assert_gemm_bound(y, y_ref, t_ref, "f32 %s" % ((M, N, K),), rel=rel)
    yb = host(mx.mx_gemm(qa, sa, qb, sb, afmt, bfmt, out_dtype=torch.bfloat16, accum=accum))
    assert_gemm_bound(bf16_to_f64(yb), y_ref, t_ref, "bf16 %s" % ((M, N, K),), bf16_out=True, rel=rel)


# shapes that take the 256 x 256 pipelined kernel (M, N >= 256, K % 512 == 0,
# 16-byte aligned scale rows), including ragged M / N, a single scale group
# and odd group counts; K = 256 falls back to the general kernel
BIG_SHAPES = [(256, 256, 256), (256, 256, 512), (300, 257, 512), (513, 1000, 1536), (1024, 512, 2048),
              (640, 384, 8192)]


@pytest.mark.parametrize("M,N,K", BIG_SHAPES)
@pytest.mark.parametrize("afmt,bfmt", [(E4M3, E4M3), (E5M2, E4M3)])
def test_large_tile_kernel(mx, oracle, M, N, K, afmt, bfmt):
    torch = _torch()
    xa = inputs.normal_bf16(300 + M, (M, K))
    xb = inputs.normal_bf16(400 + N, (N, K))
    qa_o, sa_o = oracle.quantize_rows(xa, afmt)
    qb_o, sb_o = oracle.quantize_rows(xb, bfmt)
    y_ref, t_ref = oracle.gemm(qa_o, sa_o, afmt, qb_o, sb_o, bfmt)
    qa, sa, qb, sb = dev(qa_o), dev(sa_o), dev(qb_o), dev(sb_o)
    y = host(mx.mx_gemm(qa, sa, qb, sb, afmt, bfmt, out_dtype=torch.float32, accum=FP8))
    assert_gemm_bound(y, y_ref, t_ref, "fp8 f32 %s" % ((M, N, K),), rel=FP8_GROUPED_REL)
    yb = host(mx.mx_gemm(qa, sa, qb, sb, afmt, bfmt, out_dtype=torch.bfloat16, accum=FP8))
    assert_gemm_bound(bf16_to_f64(yb), y_ref, t_ref, "fp8 bf16 %s" % ((M, N, K),), bf16_out=True, rel=FP8_GROUPED_REL)
    if afmt == E4M3 and K >= 2048:
        # N(0,1) data: the grouped error cancels and stays inside 1e-5
        assert_gemm_bound(y, y_ref, t_ref, "fp8 on N(0,1) data %s" % ((M, N, K),))
    # the same kernel in FP32-accumulation mode (bf16 MFMA on decoded codes)
    y = host(mx.mx_gemm(qa, sa, qb, sb, afmt, bfmt, out_dtype=torch.float32, accum=FP32))
    assert_gemm_bound(y, y_ref, t_ref, "fp32-accum f32 %s" % ((M, N, K),))
    yb = host(mx.mx_gemm(qa, sa, qb, sb, afmt, bfmt, out_dtype=torch.bfloat16, accum=FP32))
    assert_gemm_bound(bf16_to_f64(yb), y_ref, t_ref, "fp32-accum bf16 %s" % ((M, N, K),), bf16_out=True)


# Whole-tile shapes with more tiles than a 256-CU part has CUs, so the FP8
# and FP4 modes walk tiles with one work-group per CU: 272 tiles leave 16
# work-groups with a second tile. K = 512 is a single scale group per tile
# (its last group is also its first), K = 1536 an odd number of groups.
WALK_SHAPES = [(4352, 4096, 512), (4096, 4352, 1536)]


def _sampled_rows(M, per_tile=3, seed=7):
    """The first and last row of every 256-row tile and a few others."""
    rng = np.random.default_rng(seed)
    rows = set()
    for t0 in range(0, M, 256):
        t1 = min(M, t0 + 256)
        rows.update([t0, t1 - 1])
        rows.update(int(r) for r in rng.integers(t0, t1, per_tile))
    return np.array(sorted(rows))


@pytest.mark.parametrize("M,N,K", WALK_SHAPES)
@pytest.mark.parametrize("afmt,bfmt", [(E4M3, E4M3), (E5M2, E4M3)])
def test_large_tile_kernel_walk(mx, oracle, M, N, K, afmt, bfmt):
    """Every column of sampled rows of every row tile, against the oracle,
    in the FP8 mode (walking) and the FP32-accumulation mode (one tile per
    work-group), f32 and bf16 out."""
    torch = _torch()
    xa = inputs.normal_bf16(700 + K, (M, K))
    xb = inputs.normal_bf16(800 + K, (N, K))
    qa_o, sa_o = oracle.quantize_rows(xa, afmt)
    qb_o, sb_o = oracle.quantize_rows(xb, bfmt)
    rows = _sampled_rows(M)
    y_ref, t_ref = oracle.gemm(qa_o[rows], sa_o[rows], afmt, qb_o, sb_o, bfmt)
    qa, sa, qb, sb = dev(qa_o), dev(sa_o), dev(qb_o), dev(sb_o)
    for accum, rel in ((FP8, FP8_GROUPED_REL), (FP32, REL_T)):
        y = host(mx.mx_gemm(qa, sa, qb, sb, afmt, bfmt, out_dtype=torch.float32, accum=accum))[rows]
        assert_gemm_bound(y, y_ref, t_ref, "walk f32 accum %d %s" % (accum, (M, N, K)), rel=rel)
        yb = host(mx.mx_gemm(qa, sa, qb, sb, afmt, bfmt, out_dtype=torch.bfloat16, accum=accum))[rows]
        assert_gemm_bound(bf16_to_f64(yb), y_ref, t_ref, "walk bf16 accum %d %s" % (accum, (M, N, K)),
                          bf16_out=True, rel=rel)


@pytest.mark.parametrize("afmt,bfmt", [(E4M3, E5M2), (E5M2, E5M2)])
def test_large_tile_kernel_walk_padded(mx, oracle, afmt, bfmt):
    """A walking shape (4352 x 4096 x 1024, 272 tiles) with every pitch
    padded: codes and scales of A and B and the output rows (f32 and bf16);
    sampled rows of every row tile against the oracle and the padding left
    as it was."""
    torch = _torch()
    M, N, K = 4352, 4096, 1024
    xa = inputs.normal_bf16(900, (M, K))
    xb = inputs.normal_bf16(901, (N, K))
    qa_o, sa_o = oracle.quantize_rows(xa, afmt)
    qb_o, sb_o = oracle.quantize_rows(xb, bfmt)
    u8 = dict(dtype=torch.uint8, device="cuda")
    A = torch.zeros((M, K + 64), **u8); B = torch.zeros((N, K + 128), **u8)
    SA = torch.zeros((M, K // 32 + 16), **u8); SB = torch.zeros((N, K // 32 + 32), **u8)
    A[:, :K] = dev(qa_o); B[:, :K] = dev(qb_o); SA[:, :K // 32] = dev(sa_o); SB[:, :K // 32] = dev(sb_o)
    rows = _sampled_rows(M)
    y_ref, t_ref = oracle.gemm(qa_o[rows], sa_o[rows], afmt, qb_o, sb_o, bfmt)
    for dt in (torch.float32, torch.bfloat16):
        Y = torch.full((M, N + 64), -7.0, dtype=dt, device="cuda")
        mx.mx_gemm(A[:, :K], SA[:, :K // 32], B[:, :K], SB[:, :K // 32], afmt, bfmt, y=Y[:, :N], accum=FP8)
        Yh = host(Y)
        got = bf16_to_f64(Yh[rows, :N]) if dt == torch.bfloat16 else Yh[rows, :N]
        assert_gemm_bound(got, y_ref, t_ref, "walk padded %s" % dt, bf16_out=dt == torch.bfloat16,
                          rel=FP8_GROUPED_REL)
        pad = bf16_to_f64(Yh[:, N:]) if dt == torch.bfloat16 else Yh[:, N:]
        assert np.all(pad == -7.0)


def test_large_tile_kernel_batched(mx, oracle):
    """Two problems of 256 x 512 x 512 in one call (batch strides)."""
    torch = _torch()
    Bt, M, N, K = 2, 256, 512, 512
    xa = inputs.normal_bf16(51, (Bt * M, K))
    xb = inputs.normal_bf16(52, (Bt * N, K))
    qa_o, sa_o = oracle.quantize_rows(xa, E4M3)
    qb_o, sb_o = oracle.quantize_rows(xb, E4M3)
    qa, sa, qb, sb = dev(qa_o), dev(sa_o), dev(qb_o), dev(sb_o)
    y = torch.empty((Bt, M, N), dtype=torch.float32, device="cuda")
    d = mx.mx_gemm_desc_t()
    d.M, d.N, d.K = M, N, K
    d.a, d.lda, d.sa, d.ldsa, d.a_fmt = qa.data_ptr(), K, sa.data_ptr(), K // 32, E4M3
    d.b, d.ldb, d.sb, d.ldsb, d.b_fmt = qb.data_ptr(), K, sb.data_ptr(), K // 32, E4M3
    d.y, d.ldy, d.y_dtype = y.data_ptr(), N, mx.MX_F32
    d.batch_outer, d.batch_inner = Bt, 1
    d.stride_a_outer, d.stride_sa_outer = M * K, M * K // 32
    d.stride_b_outer, d.stride_sb_outer = N * K, N * K // 32
    d.stride_y_outer = M * N
    d.accum = FP8
    mx.mx_gemm_desc(d)
    yh = host(y)
    for b in range(Bt):
        y_ref, t_ref = oracle.gemm(qa_o[b * M:(b + 1) * M], sa_o[b * M:(b + 1) * M], E4M3,
                                   qb_o[b * N:(b + 1) * N], sb_o[b * N:(b + 1) * N], E4M3)
        assert_gemm_bound(yh[b], y_ref, t_ref, "batch %d" % b, rel=FP8_GROUPED_REL)


def test_large_tile_kernel_batched_whole_tiles(mx, oracle):
    """Two problems of 4352 x 4096 x 512 in one call: whole tiles and more
    of them than a 256-CU part has CUs, but a batch does not walk (one tile
    per work-group); sampled rows of every row tile of both problems."""
    torch = _torch()
    Bt, M, N, K = 2, 4352, 4096, 512
    xa = inputs.normal_bf16(53, (Bt * M, K))
    xb = inputs.normal_bf16(54, (Bt * N, K))
    qa_o, sa_o = oracle.quantize_rows(xa, E4M3)
    qb_o, sb_o = oracle.quantize_rows(xb, E4M3)
    qa, sa, qb, sb = dev(qa_o), dev(sa_o), dev(qb_o), dev(sb_o)
    y = torch.empty((Bt, M, N), dtype=torch.bfloat16, device="cuda")
    d = mx.mx_gemm_desc_t()
    d.M, d.N, d.K = M, N, K
    d.a, d.lda, d.sa, d.ldsa, d.a_fmt = qa.data_ptr(), K, sa.data_ptr(), K // 32, E4M3
    d.b, d.ldb, d.sb, d.ldsb, d.b_fmt = qb.data_ptr(), K, sb.data_ptr(), K // 32, E4M3
    d.y, d.ldy, d.y_dtype = y.data_ptr(), N, mx.MX_BF16
    d.batch_outer, d.batch_inner = Bt, 1
    d.stride_a_outer, d.stride_sa_outer = M * K, M * K // 32
    d.stride_b_outer, d.stride_sb_outer = N * K, N * K // 32
    d.stride_y_outer = M * N
    d.accum = FP8
    mx.mx_gemm_desc(d)
    yh = host(y)
    rows = _sampled_rows(M)
    for b in range(Bt):
        y_ref, t_ref = oracle.gemm(qa_o[b * M + rows], sa_o[b * M + rows], E4M3,
                                   qb_o[b * N:(b + 1) * N], sb_o[b * N:(b + 1) * N], E4M3)
        assert_gemm_bound(bf16_to_f64(yh[b][rows]), y_ref, t_ref, "batch %d" % b, bf16_out=True, rel=FP8_GROUPED_REL)


def test_padded_pitches_and_unaligned_scale_rows(mx, oracle):
    """Leading dimensions larger than the rows, and K/32 not a multiple of 4
    (scale rows not dword aligned)."""
    torch = _torch()
    M, N, K = 70, 50, 224
    xa = inputs.normal_bf16(5, (M, K))
    xb = inputs.normal_bf16(6, (N, K))
    qa_o, sa_o = oracle.quantize_rows(xa, E4M3)
    qb_o, sb_o = oracle.quantize_rows(xb, E4M3)
    A = torch.zeros((M, K + 32), dtype=torch.uint8, device="cuda")
    B = torch.zeros((N, K + 48), dtype=torch.uint8, device="cuda")
    SA = torch.zeros((M, K // 32 + 3), dtype=torch.uint8, device="cuda")
    SB = torch.zeros((N, K // 32 + 1), dtype=torch.uint8, device="cuda")
    A[:, :K] = dev(qa_o); B[:, :K] = dev(qb_o); SA[:, :K // 32] = dev(sa_o); SB[:, :K // 32] = dev(sb_o)
    Y = torch.full((M, N + 12), -7.0, dtype=torch.float32, device="cuda")
    mx.mx_gemm(A[:, :K], SA[:, :K // 32], B[:, :K], SB[:, :K // 32], y=Y[:, :N])
    y_ref, t_ref = oracle.gemm(qa_o, sa_o, E4M3, qb_o, sb_o, E4M3)
    Yh = host(Y)
    assert_gemm_bound(Yh[:, :N], y_ref, t_ref, "padded")
    assert np.all(Yh[:, N:] == -7.0)


@pytest.mark.parametrize("L,page", [(96, 32), (96, 24), (100, 24), (90, 48), (90, 128)])
def test_batched_paged_scores_small(mx, oracle, L, page):
    """Paged QK^T: 3 sequences x 2 heads on pages of `page` rows, including
    page sizes that are not powers of two and a last page left partly empty
    (the kernel splits row indices into (page, offset) by multiply-high)."""
    torch = _torch()
    S, H, D = 3, 2, 64
    pages_per_seq = -(-L // page)
    n_pages = S * pages_per_seq + 3
    k = inputs.normal_bf16(71, (S * L, H, D))
    q = inputs.normal_bf16(72, (S * L, H, D))
    perm = inputs.rng(73).permutation(n_pages)
    table = perm[:S * pages_per_seq].reshape(S, pages_per_seq).astype(np.int32)
    t = np.arange(S * L)
    slots = (table[t // L, (t % L) // page].astype(np.int64) * page + (t % L) % page)
    kc = torch.zeros((n_pages, page, H, D), dtype=torch.uint8, device="cuda")
    ks = torch.zeros((n_pages, page, H, D // 32), dtype=torch.uint8, device="cuda")
    vc, vs = torch.zeros_like(kc), torch.zeros_like(ks)
    mx.mx_kv_quant_write(dev(k, bf16=True), dev(k, bf16=True), dev(slots), kc, ks, vc, vs)
    qq, qs = mx.mx_quantize(dev(q.reshape(S * L * H, D), bf16=True), E4M3)
    out = host(mx.mx_paged_scores(qq.view(S * L, H, D), qs.view(S * L, H, D // 32), kc, ks, dev(table), L))
    qo, qso = oracle.quantize_rows(q.reshape(S * L * H, D), E4M3)
    ko, kso = oracle.quantize_rows(k.reshape(S * L * H, D), E4M3)
    qo = qo.reshape(S, L, H, D); qso = qso.reshape(S, L, H, D // 32)
    ko = ko.reshape(S, L, H, D); kso = kso.reshape(S, L, H, D // 32)
    for s in range(S):
        for h in range(H):
            y_ref, t_ref = oracle.gemm(qo[s, :, h], qso[s, :, h], E4M3, ko[s, :, h], kso[s, :, h], E4M3)
            assert_gemm_bound(out[s, h], y_ref, t_ref, "scores s=%d h=%d" % (s, h))


# --------------------------------------------------------------------------- workload sizes
@pytest.mark.slow
def test_gemm_8192_cubed(mx, oracle):
    """M = N = K = 8192, E4M3 x E4M3, inputs ~ N(0,1) quantized rowwise along
    K. Every one of the 67.1 M outputs is compared with the oracle: bf16 and
    f32 output of the scaled FP8 instruction (the timed configuration), and
    f32 output of the FP32-accumulation mode (the default)."""
    torch = _torch()
    xa, xb = inputs.gemm_inputs()
    qa, sa = mx.mx_quantize(dev(xa, bf16=True), E4M3)
    qb, sb = mx.mx_quantize(dev(xb, bf16=True), E4M3)
    qa_o, sa_o = oracle.quantize_rows(xa, E4M3)
    qb_o, sb_o = oracle.quantize_rows(xb, E4M3)
    del xa, xb
    assert_bitexact(host(qa), qa_o, "A codes")
    assert_bitexact(host(qb), qb_o, "B codes")
    assert_bitexact(host(sa), sa_o, "A scales")
    assert_bitexact(host(sb), sb_o, "B scales")
    y = mx.mx_gemm(qa, sa, qb, sb, out_dtype=torch.bfloat16, accum=FP8)
    y32 = mx.mx_gemm(qa, sa, qb, sb, out_dtype=torch.float32, accum=FP8)
    # bf16 output is the f32 result rounded once
    assert torch.equal(y, y32.to(torch.bfloat16))
    y_auto = mx.mx_gemm(qa, sa, qb, sb, out_dtype=torch.bfloat16)
    y_exact = mx.mx_gemm(qa, sa, qb, sb, out_dtype=torch.float32, accum=FP32)
    assert torch.equal(y_auto, y_exact.to(torch.bfloat16))
    worst = check_every_output(oracle, [("bf16 FP8", y, REL_T), ("f32 FP8", y32, REL_T),
                                        ("f32 FP32-accum", y_exact, REL_T)],
                               qa_o, sa_o, E4M3, qb_o, sb_o, E4M3, "8192^3")
    print("8192^3 worst |err|/T over all outputs: %s" % worst)


@pytest.mark.slow
def test_training_linear_fwd(mx, oracle):
    """fwd Y = X W^T: X [16384, 4096] E4M3, W [14336, 4096] E4M3 (rowwise), on
    the scaled FP8 instruction as the bench times it; every one of the
    234.9 M outputs, bf16 (the timed output) and f32."""
    torch = _torch()
    x, w, _ = inputs.training_inputs(with_grad=False)
    qx, sx = mx.mx_quantize(dev(x, bf16=True), E4M3)
    qw, sw = mx.mx_quantize(dev(w, bf16=True), E4M3)
    qx_o, sx_o = oracle.quantize_rows(x, E4M3)
    qw_o, sw_o = oracle.quantize_rows(w, E4M3)
    assert_bitexact(host(qx), qx_o, "X codes")
    assert_bitexact(host(qw), qw_o, "W codes")
    y = mx.mx_gemm(qx, sx, qw, sw, out_dtype=torch.bfloat16, accum=FP8)
    y32 = mx.mx_gemm(qx, sx, qw, sw, out_dtype=torch.float32, accum=FP8)
    worst = check_every_output(oracle, [("bf16", y, REL_T), ("f32", y32, REL_T)], qx_o, sx_o, E4M3, qw_o, sw_o, E4M3,
                               "fwd", chunk_rows=2048)
    print("training fwd worst |err|/T over all outputs: %s" % worst)


@pytest.mark.slow
def test_training_linear_dgrad(mx, oracle):
    """dgrad dX = G W: G [16384, 14336] E5M2 rowwise x W colwise E4M3
    [4096, 14336] (requantized from bf16); every one of the 67.1 M outputs."""
    torch = _torch()
    _, w, g = inputs.training_inputs()
    gd, wd = dev(g, bf16=True), dev(w, bf16=True)
    qg, sg = mx.mx_quantize(gd, E5M2)
    qwt, swt = mx.mx_quantize_colwise(wd, E4M3)
    qg_o, sg_o = oracle.quantize_rows(g, E5M2)
    qwt_o, swt_o = oracle.quantize_cols(w, E4M3)
    del g, w, gd, wd
    assert_bitexact(host(qg), qg_o, "G codes")
    assert_bitexact(host(sg), sg_o, "G scales")
    assert_bitexact(host(qwt), qwt_o, "W colwise codes")
    assert_bitexact(host(swt), swt_o, "W colwise scales")
    dx = mx.mx_gemm(qg, sg, qwt, swt, E5M2, E4M3, out_dtype=torch.bfloat16)
    dx32 = mx.mx_gemm(qg, sg, qwt, swt, E5M2, E4M3, out_dtype=torch.float32)
    worst = check_every_output(oracle, [("bf16", dx, REL_T), ("f32", dx32, REL_T)], qg_o, sg_o, E5M2, qwt_o, swt_o,
                               E4M3, "dgrad", chunk_rows=2048)
    print("training dgrad worst |err|/T over all outputs: %s" % worst)


@pytest.mark.slow
def test_training_linear_wgrad(mx, oracle):
    """wgrad dW = G^T X [14336, 4096]: G [16384, 14336] quantized colwise in
    E5M2 and X [16384, 4096] colwise in E4M3 (blocks along the 16384 tokens,
    the reduction), then the block-scaled product over K = 16384; every one of
    the 58.7 M outputs."""
    torch = _torch()
    x, _, g = inputs.training_inputs()
    qgt, sgt = mx.mx_quantize_colwise(dev(g, bf16=True), E5M2)
    qxt, sxt = mx.mx_quantize_colwise(dev(x, bf16=True), E4M3)
    qgt_o, sgt_o = oracle.quantize_cols(g, E5M2)
    qxt_o, sxt_o = oracle.quantize_cols(x, E4M3)
    del x, g
    assert_bitexact(host(sgt), sgt_o, "G colwise scales")
    assert_bitexact(host(qgt), qgt_o, "G colwise codes")
    assert_bitexact(host(sxt), sxt_o, "X colwise scales")
    assert_bitexact(host(qxt), qxt_o, "X colwise codes")
    dw = mx.mx_gemm(qgt, sgt, qxt, sxt, E5M2, E4M3, out_dtype=torch.float32)
    worst = check_every_output(oracle, [("f32", dw, REL_T)], qgt_o, sgt_o, E5M2, qxt_o, sxt_o, E4M3, "wgrad",
                               chunk_rows=2048)
    print("training wgrad worst |err|/T over all outputs: %s" % worst)


@pytest.mark.slow
def test_kv_cache_scores_full_size(mx, oracle):
    """32768 tokens x 8 heads x 128 written to 256 pages of 128, then QK^T
    for 64 sequences x 512 tokens per head, f32 output; every one of the
    134.2 M scores is compared with the oracle's product of the same codes."""
    torch = _torch()
    k, v, q = inputs.kv_inputs()
    slots, table = inputs.kv_layout()
    kc = torch.empty((256, 128, 8, 128), dtype=torch.uint8, device="cuda")
    ks = torch.empty((256, 128, 8, 4), dtype=torch.uint8, device="cuda")
    vc, vs = torch.empty_like(kc), torch.empty_like(ks)
    mx.mx_kv_quant_write(dev(k, bf16=True), dev(v, bf16=True), dev(slots), kc, ks, vc, vs)
    qq, qs = mx.mx_quantize(dev(q.reshape(-1, 128), bf16=True), E4M3)
    scores = mx.mx_paged_scores(qq.view(32768, 8, 128), qs.view(32768, 8, 4), kc, ks, dev(table), 512)
    qo, qso = oracle.quantize_rows(q.reshape(-1, 128), E4M3)
    ko, kso = oracle.quantize_rows(k.reshape(-1, 128), E4M3)
    kco, kso_c, _, _ = oracle.kv_quant_write(k, v, slots, 128, 256)
    assert_bitexact(host(kc), kco, "K cache")
    assert_bitexact(host(ks), kso_c, "K cache scales")
    assert_bitexact(host(qq), qo, "Q codes")
    qo, qso = qo.reshape(32768, 8, 128), qso.reshape(32768, 8, 4)
    ko, kso = ko.reshape(32768, 8, 128), kso.reshape(32768, 8, 4)
    worst = 0.0
    for s in range(64):
        got = host(scores[s]).astype(np.float64)  # [8, 512, 512]
        rows = slice(512 * s, 512 * (s + 1))
        for h in range(8):
            y_ref, t_ref = oracle.gemm(qo[rows, h], qso[rows, h], E4M3, ko[rows, h], kso[rows, h], E4M3)
            worst = max(worst, assert_gemm_bound(got[h], y_ref, t_ref, "kv scores seq %d head %d" % (s, h)))
    print("kv scores worst |err|/T over all 134.2 M outputs: %.3g" % worst)


def test_gemm_repeat_runs_identical(mx):
    torch = _torch()
    g = inputs.rng(3)
    a = torch.from_numpy(g.integers(0, 0x7E, (384, 512), dtype=np.uint8)).cuda()
    b = torch.from_numpy(g.integers(0, 0x7E, (256, 512), dtype=np.uint8)).cuda()
    sa = torch.full((384, 16), 120, dtype=torch.uint8, device="cuda")
    sb = torch.full((256, 16), 125, dtype=torch.uint8, device="cuda")
    y1 = mx.mx_gemm(a, sa, b, sb, out_dtype=torch.float32)
    y2 = mx.mx_gemm(a, sa, b, sb, out_dtype=torch.float32)
    assert torch.equal(y1, y2)


def test_binding_refuses_short_buffers(mx):
    """Buffers the kernels would run past are refused before any launch."""
    import torch
    u8 = dict(dtype=torch.uint8, device="cuda")
    a, sa = torch.zeros((256, 512), **u8), torch.zeros((256, 16), **u8)
    with pytest.raises(ValueError, match="shape"):
        mx.mx_gemm(a, sa[:200], a, sa)
    with pytest.raises(ValueError, match="shape"):
        mx.mx_gemm(a, sa, a, sa, y=torch.empty((256, 200), dtype=torch.bfloat16, device="cuda"))
    with pytest.raises(ValueError, match="shape"):
        mx.mx_dequantize(a[:100], sa, y=None)
    torch.cuda.synchronize()
