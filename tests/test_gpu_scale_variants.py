"""GPU parity of the scale variants against the oracle: the round-up scale
rule, 32 x 32 two-dimensional blocks, and the broadcast of power-of-two
128-block scales into E8M0 [MXFP8 SM120 software support, §1.3].

All three produce integers (codes and scales), so every case is bit-exact.
Inputs plant block maxima whose significands sit on both sides of the point
where the round-up rule moves one E8M0 step above the floor rule (1.75 for
FP8, 1.5 for E2M1), across a range of exponents, so both outcomes of the rule
are exercised in every block orientation.
"""
import numpy as np
import pytest

from gpu_util import assert_bitexact, dev, host
from microscaling_block_scaled_amd import inputs

pytestmark = pytest.mark.gpu

E4M3, E5M2, E2M1 = 0, 1, 2
FLOOR, CEIL = 0, 1
# significands around the round-up thresholds, all exact in bf16
SIGNIFICANDS = np.array([1.0, 1.4921875, 1.5, 1.5078125, 1.7421875, 1.75, 1.7578125, 1.9921875])


@pytest.fixture(scope="module")
def mx():
    import torch
    import microscaling_block_scaled_amd as m
    assert torch.cuda.is_available()
    ok, reason = m.mx_query_support(0)
    assert ok, reason
    return m


def planted(seed, shape, f32=False):
    """Normal bf16 data with every 13th element replaced by a significand from
    SIGNIFICANDS times 2^e, e in [-4, 9], random sign; optional f32 values
    between bf16 points elsewhere."""
    g = inputs.rng(seed)
    x = inputs.bf16_bits_to_f32(inputs.normal_bf16(seed, shape)).astype(np.float32)
    flat = x.reshape(-1)
    idx = np.arange(g.integers(0, 13), flat.size, 13)
    mags = SIGNIFICANDS[g.integers(0, len(SIGNIFICANDS), idx.size)] * np.exp2(g.integers(-4, 10, idx.size))
    flat[idx] = (mags * np.where(g.random(idx.size) < 0.5, -1.0, 1.0)).astype(np.float32)
    if f32:
        # between bf16 points except for the planted maxima
        keep = np.zeros(flat.size, bool)
        keep[idx] = True
        flat[~keep] *= np.float32(1.0 + 2.0 ** -12)
        return x
    return inputs.f32_to_bf16_bits(x)


def to_dev(x):
    return dev(x, bf16=x.dtype == np.uint16)


@pytest.mark.parametrize("fmt", [E4M3, E5M2, E2M1])
@pytest.mark.parametrize("f32", [False, True])
@pytest.mark.parametrize("rows,cols,seed", [(1, 32, 1), (37, 96, 2), (300, 4128, 3)])
def test_round_up_rule_rowwise(mx, oracle, fmt, f32, rows, cols, seed):
    x = planted(700 + seed, (rows, cols), f32)
    q, s, _, _ = mx.mx_quantize_ex(to_dev(x), fmt, rule=CEIL)
    qo, so = oracle.quantize_rows(x, fmt, oracle.RULE_CEIL)
    assert_bitexact(host(s), so, "round-up scales")
    assert_bitexact(host(q), qo, "round-up codes")
    # the planted maxima must reach both outcomes of the rule
    qf, sf = oracle.quantize_rows(x, fmt, oracle.RULE_FLOOR)
    if rows * cols >= 4096:
        assert (so != sf).any() and (so == sf).any()


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
@pytest.mark.parametrize("f32", [False, True])
@pytest.mark.parametrize("rows,cols,seed", [(32, 8, 4), (96, 200, 5), (416, 1000, 6)])
def test_round_up_rule_colwise(mx, oracle, fmt, f32, rows, cols, seed):
    x = planted(710 + seed, (rows, cols), f32)
    _, _, qt, st = mx.mx_quantize_ex(to_dev(x), fmt, rule=CEIL, rowwise=False, colwise=True)
    qo, so = oracle.quantize_cols(x, fmt, oracle.RULE_CEIL)
    assert_bitexact(host(st), so, "round-up colwise scales")
    assert_bitexact(host(qt), qo, "round-up colwise codes")


@pytest.mark.parametrize("rule", [FLOOR, CEIL])
@pytest.mark.parametrize("fmt", [E4M3, E5M2])
@pytest.mark.parametrize("f32", [False, True])
@pytest.mark.parametrize("rows,cols,seed", [(256, 640, 0), (96, 224, 1), (160, 8224, 2)])
def test_1d_both_orientations_in_one_call(mx, oracle, rule, fmt, f32, rows, cols, seed):
    """Both 1-D orientations from one pass over x (the tile kernel's rowwise
    mode), against the oracle's rowwise and colwise quantizations; (160, 8224)
    has more than 64 column tiles, so its tiles run down the columns."""
    x = planted(720 + seed, (rows, cols), f32)
    q, s, qt, st = mx.mx_quantize_ex(to_dev(x), fmt, rule=rule, rowwise=True, colwise=True)
    qo, so = oracle.quantize_rows(x, fmt, rule)
    qto, sto = oracle.quantize_cols(x, fmt, rule)
    assert_bitexact(host(q), qo, "rowwise codes")
    assert_bitexact(host(s), so, "rowwise scales")
    assert_bitexact(host(qt), qto, "colwise codes")
    assert_bitexact(host(st), sto, "colwise scales")


def test_1d_both_orientations_special_blocks(mx, oracle):
    """NaN, Inf and all-zero blocks in the one-pass rowwise + colwise mode."""
    x = inputs.normal_bf16(722, (128, 256))
    x[5, 40] = 0x7FC0      # NaN
    x[70, 200] = 0xFF80    # -Inf
    x[96:128, 0:64] = 0    # zero blocks in both orientations
    q, s, qt, st = mx.mx_quantize_ex(dev(x, bf16=True), E4M3, rowwise=True, colwise=True)
    qo, so = oracle.quantize_rows(x, E4M3)
    qto, sto = oracle.quantize_cols(x, E4M3)
    for g, w, n in ((q, qo, "q"), (s, so, "s"), (qt, qto, "qt"), (st, sto, "st")):
        assert_bitexact(host(g), w, n)


def test_floor_rule_matches_mx_quantize(mx):
    """MX_SCALE_FLOOR with 1-D blocks is the rule of mx_quantize and
    mx_quantize_colwise."""
    x = dev(inputs.normal_bf16(721, (128, 384)), bf16=True)
    q, s, qt, st = mx.mx_quantize_ex(x, E5M2, rule=FLOOR, colwise=True)
    q0, s0 = mx.mx_quantize(x, E5M2)
    qt0, st0 = mx.mx_quantize_colwise(x, E5M2)
    for a, b, n in ((q, q0, "q"), (s, s0, "s"), (qt, qt0, "qt"), (st, st0, "st")):
        assert_bitexact(host(a), host(b), n)


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
@pytest.mark.parametrize("rule", [FLOOR, CEIL])
@pytest.mark.parametrize("f32", [False, True])
@pytest.mark.parametrize("rows,cols,seed", [(32, 32, 1), (96, 320, 2), (256, 1056, 3), (160, 8224, 4)])
def test_2d_blocks(mx, oracle, fmt, rule, f32, rows, cols, seed):
    x = planted(730 + seed, (rows, cols), f32)
    q, s, qt, st = mx.mx_quantize_ex(to_dev(x), fmt, rule=rule, blocks=mx.MX_BLOCKS_2D, colwise=True)
    qo, so, qto, sto = oracle.quantize_2d(x, fmt, rule)
    assert_bitexact(host(s), so, "2-D row-layout scales")
    assert_bitexact(host(q), qo, "2-D rowwise codes")
    assert_bitexact(host(st), sto, "2-D column-layout scales")
    assert_bitexact(host(qt), qto, "2-D transposed codes")


def test_2d_single_outputs_and_special_blocks(mx, oracle):
    """Only one orientation asked for; blocks holding NaN, Inf or only zeros."""
    x = inputs.normal_bf16(740, (128, 256))
    x[3, 40] = 0x7FC0      # NaN in block (0, 1)
    x[70, 200] = 0x7F80    # +Inf in block (2, 6)
    x[96:128, 0:32] = 0    # a zero block
    qo, so, qto, sto = oracle.quantize_2d(x, E4M3, CEIL)
    q, s, _, _ = mx.mx_quantize_ex(dev(x, bf16=True), E4M3, rule=CEIL, blocks=mx.MX_BLOCKS_2D)
    assert_bitexact(host(q), qo, "2-D codes, rowwise only")
    assert_bitexact(host(s), so, "2-D scales, rowwise only")
    _, _, qt, st = mx.mx_quantize_ex(dev(x, bf16=True), E4M3, rule=CEIL, blocks=mx.MX_BLOCKS_2D, rowwise=False,
                                     colwise=True)
    assert_bitexact(host(qt), qto, "2-D codes, colwise only")
    assert_bitexact(host(st), sto, "2-D scales, colwise only")


def test_2d_strided_outputs(mx, oracle):
    """Pitches above the minimum: only the named bytes are written."""
    import torch
    x = planted(741, (64, 96))
    qo, so, qto, sto = oracle.quantize_2d(x, E4M3, FLOOR)
    big = lambda r, c: torch.full((r, c), 0xA5, dtype=torch.uint8, device="cuda")
    q, s, qt, st = big(64, 128), big(64, 8), big(96, 80), big(96, 5)
    mx.mx_quantize_ex(dev(x, bf16=True), E4M3, blocks=mx.MX_BLOCKS_2D, colwise=True, q=q[:, :96], s=s[:, :3],
                      qt=qt[:, :64], st=st[:, :2])
    assert_bitexact(host(q[:, :96]), qo, "codes")
    assert_bitexact(host(s[:, :3]), so, "scales")
    assert_bitexact(host(qt[:, :64]), qto, "transposed codes")
    assert_bitexact(host(st[:, :2]), sto, "transposed scales")
    for t, c in ((q, 96), (s, 3), (qt, 64), (st, 2)):
        assert (host(t[:, c:]) == 0xA5).all()


@pytest.mark.slow
def test_2d_blocks_weight_size(mx, oracle):
    """An 8192 x 8192 bf16 weight (the GEMM workload's operand), 2-D blocks,
    both outputs, compared whole."""
    xa, _ = inputs.gemm_inputs()
    q, s, qt, st = mx.mx_quantize_ex(dev(xa, bf16=True), E4M3, blocks=mx.MX_BLOCKS_2D, colwise=True)
    qo, so, qto, sto = oracle.quantize_2d(xa, E4M3, FLOOR)
    assert_bitexact(host(s), so, "scales")
    assert_bitexact(host(q), qo, "codes")
    assert_bitexact(host(st), sto, "transposed scales")
    assert_bitexact(host(qt), qto, "transposed codes")


def broadcast_scales(seed, shape):
    """Powers of two 2^k, k in [-127, 127] (2^-127 is an f32 subnormal), with
    a few entries that E8M0 cannot hold."""
    g = inputs.rng(seed)
    s = np.ldexp(np.float32(1.0), g.integers(-127, 128, shape)).astype(np.float32)
    flat = s.reshape(-1)
    bad = np.array([3.0, 0.0, -0.0, -2.0, np.inf, np.nan, 2.0 ** -128, 2.0 ** -149, 1.5 * 2.0 ** -127,
                    np.float32(1.0000001)], np.float32)
    pos = g.choice(flat.size, min(flat.size, len(bad)), replace=False)
    flat[pos] = bad[:len(pos)]
    flat[g.integers(0, flat.size)] = np.float32(2.0 ** 127)
    flat[g.integers(0, flat.size)] = np.float32(2.0 ** -127)
    return s


@pytest.mark.parametrize("layout", [0, 1])
@pytest.mark.parametrize("rows,cols", [(1, 128), (200, 384), (1024, 4096)])
def test_scale_broadcast(mx, oracle, layout, rows, cols):
    sr = rows if layout == 0 else (rows + 127) // 128
    s_in = broadcast_scales(750 + rows + layout, (sr, cols // 128))
    out = mx.mx_scale_broadcast(dev(s_in), rows, cols, layout=layout)
    want = oracle.scale_broadcast(s_in, layout, rows, cols)
    assert_bitexact(host(out), want, "broadcast E8M0 scales")


def test_scale_broadcast_strided(mx, oracle):
    import torch
    s_in = broadcast_scales(760, (64, 6))
    out = torch.full((64, 20), 0x5A, dtype=torch.uint8, device="cuda")
    mx.mx_scale_broadcast(dev(s_in)[:, :4], 64, 512, out=out[:, :16])
    want = oracle.scale_broadcast(s_in[:, :4], 0, 64, 512)
    assert_bitexact(host(out[:, :16]), want, "broadcast into a wider array")
    assert (host(out[:, 16:]) == 0x5A).all()


def test_scale_broadcast_strided_four_per_thread(mx, oracle):
    """Padded pitches on the path that converts 4 source scales per thread
    (a multiple of 4 scales per row, 4-scale and 16-byte pitches): both
    layouts, bytes past the output pitch untouched."""
    import torch
    for layout in (0, 1):
        rows = 300
        sr = rows if layout == 0 else (rows + 127) // 128
        s_in = broadcast_scales(770 + layout, (sr, 36))
        out = torch.full((rows, 144), 0x5A, dtype=torch.uint8, device="cuda")
        mx.mx_scale_broadcast(dev(s_in)[:, :32], rows, 32 * 128, layout=layout, out=out[:, :128])
        want = oracle.scale_broadcast(s_in[:, :32], layout, rows, 32 * 128)
        assert_bitexact(host(out[:, :128]), want, "broadcast, 4 per thread, layout %d" % layout)
        assert (host(out[:, 128:]) == 0x5A).all()
