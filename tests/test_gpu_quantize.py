"""GPU parity of the quantize / KV-write / dequantize kernels against the
oracle: codes, scales and dequantized values must match bit for bit."""
import numpy as np
import pytest

from conftest import load_golden
from gpu_util import assert_bitexact, dev, host
from microscaling_block_scaled_amd import inputs

pytestmark = pytest.mark.gpu

E4M3, E5M2 = 0, 1


@pytest.fixture(scope="module")
def mx():
    import torch
    import microscaling_block_scaled_amd as m
    assert torch.cuda.is_available()
    ok, reason = m.mx_query_support(0)
    assert ok, reason
    return m


def assorted_bits(seed, rows, cols):
    """bf16 patterns mixing normal data, per-block magnitude jumps, exact
    ties, zeros, subnormals, huge values, and raw random bit patterns
    (which include NaN/Inf, so some blocks take the NaN path)."""
    width = cols
    cols = (cols + 31) // 32 * 32
    g = inputs.rng(seed)
    x = (g.standard_normal((rows, cols)) * np.exp2(g.integers(-30, 30, (rows, cols // 32)).repeat(32, 1)))
    bits = inputs.f32_to_bf16_bits(x.astype(np.float32))
    kind = g.integers(0, 10, (rows, cols // 32)).repeat(32, 1)
    raw = g.integers(0, 1 << 16, (rows, cols), dtype=np.uint32).astype(np.uint16)
    bits = np.where(kind == 0, raw, bits)                                   # random patterns
    bits = np.where(kind == 1, np.uint16(0), bits)                          # all-zero blocks
    bits = np.where((kind == 2) & (g.random((rows, cols)) < 0.5), np.uint16(0x8000), bits)  # -0
    bits = np.where(kind == 3, (raw & np.uint16(0x807F)), bits)             # bf16 subnormals
    bits = np.where(kind == 4, (raw | np.uint16(0x7E00)) & np.uint16(0xFF7F), bits)  # near the bf16 max
    # ties: values exactly halfway between E4M3 grid points relative to a power-of-two amax
    tie = inputs.f32_to_bf16_bits(np.float32(1.0625) * np.ones((rows, cols), np.float32))
    bits = np.where((kind == 5) & (g.random((rows, cols)) < 0.3), tie, bits)
    return np.ascontiguousarray(bits[:, :width])


def f32_from(bits, seed=0):
    """f32 values with the given bf16 top halves and random low mantissa bits
    (zeros stay zero), so the f32 path sees full-precision inputs."""
    low = inputs.rng(seed).integers(0, 1 << 16, bits.shape, dtype=np.uint32)
    hi = bits.astype(np.uint32) << np.uint32(16)
    keep_exact = (bits & np.uint16(0x7FFF)) == 0
    return np.where(keep_exact, hi, hi | low).view(np.float32)


# --------------------------------------------------------------------------- worked example
def test_worked_example_on_gpu(mx, oracle):
    ex = load_golden("worked_example_v64.json")
    v = inputs.tiny()["v64"]
    q, s = mx.mx_quantize(dev(v), E4M3)
    q, s = host(q), host(s)
    qo, so = oracle.quantize_rows(v, E4M3)
    assert_bitexact(q, qo, "codes")
    assert_bitexact(s, so, "scales")
    assert [int(c) - 127 for c in s[0]] == ex["per_block"]["scale_exponents"]
    back = host(mx.mx_dequantize(dev(q), dev(s), E4M3))
    assert np.array_equal(back, v)


# --------------------------------------------------------------------------- rowwise
ROW_SHAPES = [(1, 32, 0), (3, 96, 8), (7, 160, 0), (33, 4096 + 32, 24), (130, 512, 0), (257, 96, 64)]


@pytest.mark.parametrize("rows,cols,pad", ROW_SHAPES)
@pytest.mark.parametrize("fmt", [E4M3, E5M2])
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_rowwise_matches_oracle(mx, oracle, rows, cols, pad, fmt, dt):
    bits = assorted_bits(1000 + rows + cols + fmt, rows, cols + pad)
    x = bits if dt == "bf16" else f32_from(bits, rows)
    xd = dev(x, bf16=(dt == "bf16"))[:, :cols]
    q, s = mx.mx_quantize(xd, fmt)
    qo, so = oracle.quantize_rows(np.ascontiguousarray(x[:, :cols]), fmt)
    assert_bitexact(host(s), so, "scales")
    assert_bitexact(host(q), qo, "codes")


def test_rowwise_writes_only_its_region(mx, oracle):
    import torch
    rows, cols = 40, 96
    x = inputs.normal_bf16(3, (rows, cols))
    q = torch.full((rows, 128), 0xA5, dtype=torch.uint8, device="cuda")
    s = torch.full((rows, 8), 0x5A, dtype=torch.uint8, device="cuda")
    mx.mx_quantize(dev(x, bf16=True), E4M3, q=q[:, :cols], s=s[:, :3])
    qh, sh = host(q), host(s)
    qo, so = oracle.quantize_rows(x, E4M3)
    assert_bitexact(qh[:, :cols], qo, "codes")
    assert_bitexact(sh[:, :3], so, "scales")
    assert np.all(qh[:, cols:] == 0xA5) and np.all(sh[:, 3:] == 0x5A)


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_every_bf16_input_under_every_scale(mx, oracle, fmt):
    """Every finite bf16 magnitude (both signs) under every scale code the
    rule can choose, each block anchored so that it selects that code."""
    emax = 8 if fmt == E4M3 else 15
    bits = np.arange(0x7F80, dtype=np.uint16)
    mag = inputs.bf16_bits_to_f32(bits).astype(np.float64)
    rows = []
    for c in range(0, 127 + 127 - emax + 1):
        anchor = 2.0 ** (c - 127 + emax)
        sel = bits[mag < 2 * anchor]
        sel = np.concatenate([sel, sel | np.uint16(0x8000)])
        sel = np.concatenate([sel, np.zeros((-len(sel)) % 31, np.uint16)]).reshape(-1, 31)
        anc = np.full((sel.shape[0], 1), inputs.f32_to_bf16_bits(np.float32([anchor]))[0], np.uint16)
        rows.append(np.concatenate([anc, sel], axis=1))
    x = np.concatenate(rows)
    pad = (-x.shape[0]) % 4
    x = np.concatenate([x, np.zeros((pad, 32), np.uint16)]).reshape(-1, 128)
    q, s = mx.mx_quantize(dev(x, bf16=True), fmt)
    qo, so = oracle.quantize_rows(x, fmt)
    assert_bitexact(host(s), so, "scales")
    assert_bitexact(host(q), qo, "codes")


# --------------------------------------------------------------------------- colwise
# (96, 8200) and (288, 8192) have 64 or more column tiles, where the tiles
# are ordered down the columns
COL_SHAPES = [(32, 1, 8), (64, 7, 1), (96, 65, 7), (160, 100, 4), (128, 64, 0), (256, 1000, 8), (4096, 96, 0),
              (160, 1024, 0), (96, 2043, 5), (384, 1032, 0), (96, 8200, 3), (288, 8192, 0)]


@pytest.mark.parametrize("rows,cols,pad", COL_SHAPES)
@pytest.mark.parametrize("fmt", [E4M3, E5M2])
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_colwise_matches_oracle(mx, oracle, rows, cols, pad, fmt, dt):
    bits = assorted_bits(2000 + rows + cols + fmt, rows, cols + pad)
    x = bits if dt == "bf16" else f32_from(bits, cols)
    ld_align = 8 if dt == "bf16" else 4
    ld = (cols + pad + ld_align - 1) // ld_align * ld_align
    xp = np.zeros((rows, ld), x.dtype)
    xp[:, :cols] = x[:, :cols]
    xd = dev(xp, bf16=(dt == "bf16"))[:, :cols]
    qt, st = mx.mx_quantize_colwise(xd, fmt)
    qo, so = oracle.quantize_cols(np.ascontiguousarray(x[:, :cols]), fmt)
    assert_bitexact(host(st), so, "scales")
    assert_bitexact(host(qt), qo, "codes")


# --------------------------------------------------------------------------- workload sizes
@pytest.mark.slow
def test_quantize_workload_full_size(mx, oracle):
    """X bf16 [8192, 4096] ~ N(0,1) with 4 outlier channels x 2^12, E4M3,
    rowwise and colwise, every code and scale compared."""
    x, channels = inputs.quantize_input()
    xd = dev(x, bf16=True)
    q, s = mx.mx_quantize(xd, E4M3)
    qt, st = mx.mx_quantize_colwise(xd, E4M3)
    qo, so = oracle.quantize_rows(x, E4M3)
    assert_bitexact(host(s), so, "rowwise scales")
    assert_bitexact(host(q), qo, "rowwise codes")
    qto, sto = oracle.quantize_cols(x, E4M3)
    assert_bitexact(host(st), sto, "colwise scales")
    assert_bitexact(host(qt), qto, "colwise codes")
    # the outlier channels' colwise scales sit 12 binades above their neighbours'
    assert np.all(host(st)[channels].astype(int).mean(axis=1) > host(st)[channels ^ 1].astype(int).mean(axis=1) + 10)


@pytest.mark.slow
def test_training_quantize_full_size(mx, oracle):
    """Training linear layer: X and W rowwise E4M3, W colwise E4M3 (the
    dgrad operand), G rowwise E5M2, each compared in full."""
    x, w, g = inputs.training_inputs()
    for name, arr, fmt in (("X", x, E4M3), ("W", w, E4M3), ("G", g, E5M2)):
        q, s = mx.mx_quantize(dev(arr, bf16=True), fmt)
        qo, so = oracle.quantize_rows(arr, fmt)
        assert_bitexact(host(s), so, name + " scales")
        assert_bitexact(host(q), qo, name + " codes")
        del q, s, qo, so
    qt, st = mx.mx_quantize_colwise(dev(w, bf16=True), E4M3)
    qto, sto = oracle.quantize_cols(w, E4M3)
    assert_bitexact(host(st), sto, "W colwise scales")
    assert_bitexact(host(qt), qto, "W colwise codes")


# --------------------------------------------------------------------------- KV write
def _kv_run(mx, k, v, slots, pages, page_size):
    import torch
    T, H, D = k.shape
    kc = torch.full((pages, page_size, H, D), 0x33, dtype=torch.uint8, device="cuda")
    vc = torch.full_like(kc, 0x33)
    ks = torch.full((pages, page_size, H, D // 32), 0x44, dtype=torch.uint8, device="cuda")
    vs = torch.full_like(ks, 0x44)
    mx.mx_kv_quant_write(dev(k, bf16=True), dev(v, bf16=True), dev(slots), kc, ks, vc, vs)
    return host(kc), host(ks), host(vc), host(vs)


def test_kv_write_small_with_padding_and_bad_slots(mx, oracle):
    T, H, D, pages, page_size = 200, 3, 96, 5, 64
    k = assorted_bits(31, T * H, D).reshape(T, H, D)
    v = assorted_bits(32, T * H, D).reshape(T, H, D)
    slots = inputs.rng(33).permutation(pages * page_size)[:T].astype(np.int64)
    slots[::17] = -1                 # padding tokens
    slots[5] = pages * page_size + 3  # out of range: ignored
    got = _kv_run(mx, k, v, slots, pages, page_size)
    ok_slots = np.where((slots >= 0) & (slots < pages * page_size), slots, -1)
    init = [np.full((pages, page_size, H, D), 0x33, np.uint8), np.full((pages, page_size, H, D // 32), 0x44, np.uint8)]
    want = oracle.kv_quant_write(k, v, ok_slots, page_size, pages, k_cache=init[0].copy(), k_scale=init[1].copy(),
                                 v_cache=init[0].copy(), v_scale=init[1].copy())
    for g_, w_, n in zip(got, want, ("k_cache", "k_scale", "v_cache", "v_scale")):
        assert_bitexact(g_, w_, n)


@pytest.mark.slow
def test_kv_write_full_size(mx, oracle):
    k, v, _ = inputs.kv_inputs()
    slots, _ = inputs.kv_layout()
    got = _kv_run(mx, k, v, slots, 256, 128)
    want = oracle.kv_quant_write(k, v, slots, 128, 256)
    for g_, w_, n in zip(got, want, ("k_cache", "k_scale", "v_cache", "v_scale")):
        assert_bitexact(g_, w_, n)


# --------------------------------------------------------------------------- dequantize
@pytest.mark.parametrize("fmt", [E4M3, E5M2])
@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("rows,cols", [(1, 32), (37, 96), (256, 1024)])
def test_dequantize_matches_oracle(mx, oracle, fmt, out, rows, cols):
    import torch
    g = inputs.rng(40 + rows + fmt)
    q = g.integers(0, 256, (rows, cols), dtype=np.uint8)
    s = g.integers(0, 256, (rows, cols // 32), dtype=np.uint8)  # every code incl. 0xFF (NaN) and the extremes
    y = host(mx.mx_dequantize(dev(q), dev(s), fmt, out_dtype=torch.float32 if out == "f32" else torch.bfloat16))
    want = oracle.dequantize(q, s, fmt, out)
    if out == "f32":
        assert_bitexact(y.view(np.uint32), want.view(np.uint32), "dequant f32 bits")
    else:
        assert_bitexact(y, want, "dequant bf16 bits")


# --------------------------------------------------------------------------- determinism, errors
def test_repeat_runs_are_byte_identical(mx):
    x = dev(inputs.normal_bf16(7, (512, 1024)), bf16=True)
    a = [host(t) for t in mx.mx_quantize(x, E4M3)] + [host(t) for t in mx.mx_quantize_colwise(x, E4M3)]
    b = [host(t) for t in mx.mx_quantize(x, E4M3)] + [host(t) for t in mx.mx_quantize_colwise(x, E4M3)]
    for u, w in zip(a, b):
        assert np.array_equal(u, w)


def test_argument_errors_are_returned_not_launched(mx):
    import torch
    x = torch.zeros((64, 96), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(mx.MXError) as e:
        mx.mx_quantize(x[:, :40], E4M3)                 # cols % 32 != 0
    assert e.value.status == -2
    with pytest.raises(mx.MXError) as e:
        mx.mx_quantize(x[:, 1:33], E4M3)                # base not 16-byte aligned
    assert e.value.status == -3
    with pytest.raises(mx.MXError) as e:
        mx.mx_quantize(x, 7)                            # unknown format
    assert e.value.status == -4
    with pytest.raises(mx.MXError) as e:
        mx.mx_quantize_colwise(x[:48], E4M3)            # rows % 32 != 0
    assert e.value.status == -2
    u8 = dict(dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError, match="shape"):     # an output one row short
        mx.mx_quantize(x, E4M3, q=torch.empty((63, 96), **u8))
    with pytest.raises(ValueError, match="shape"):
        mx.mx_quantize_colwise(x, E4M3, st=torch.empty((96, 1), **u8))
    with pytest.raises(TypeError):
        mx.mx_quantize_ex(x, E4M3, colwise=True, qt=torch.empty((96, 64), dtype=torch.int16, device="cuda"))
    torch.cuda.synchronize()


# --------------------------------------------------------------------------- empty problems
def test_empty_problems_are_no_ops(mx):
    """A zero dimension writes nothing and succeeds, although torch hands
    over NULL for the empty buffers."""
    import torch
    for shape in ((0, 64), (64, 0)):
        x = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
        q, s = mx.mx_quantize(x, E4M3)
        assert q.numel() == 0 and s.numel() == 0
        qt, st = mx.mx_quantize_colwise(x, E5M2)
        assert qt.numel() == 0 and st.numel() == 0
        q, s, qt, st = mx.mx_quantize_ex(x, E4M3, rule=mx.MX_SCALE_CEIL, blocks=mx.MX_BLOCKS_2D, colwise=True)
        assert q.numel() == 0 and qt.numel() == 0
        y = mx.mx_dequantize(torch.empty((shape[0], shape[1]), dtype=torch.uint8, device="cuda"),
                             torch.empty((shape[0], shape[1] // 32), dtype=torch.uint8, device="cuda"), E4M3)
        assert y.numel() == 0
    assert mx.mx_quantize(torch.empty((0, 64), dtype=torch.bfloat16, device="cuda"), mx.MX_E2M1)[0].shape == (0, 32)
    e8 = mx.mx_scale_broadcast(torch.empty((0, 2), dtype=torch.float32, device="cuda"), 0, 256)
    assert e8.shape == (0, 8)
    # KV write of zero tokens leaves the cache untouched
    kc = torch.full((2, 128, 2, 64), 0xA5, dtype=torch.uint8, device="cuda")
    ks = torch.full((2, 128, 2, 2), 0x5A, dtype=torch.uint8, device="cuda")
    vc, vs = kc.clone(), ks.clone()
    kv = torch.empty((0, 2, 64), dtype=torch.bfloat16, device="cuda")
    mx.mx_kv_quant_write(kv, kv, torch.empty((0,), dtype=torch.int64, device="cuda"), kc, ks, vc, vs)
    assert bool((kc == 0xA5).all()) and bool((ks == 0x5A).all()) and bool((vc == 0xA5).all())
    # products with no rows or no columns
    a = torch.empty((0, 512), dtype=torch.uint8, device="cuda")
    sa = torch.empty((0, 16), dtype=torch.uint8, device="cuda")
    b = torch.zeros((64, 512), dtype=torch.uint8, device="cuda")
    sb = torch.full((64, 16), 127, dtype=torch.uint8, device="cuda")
    assert mx.mx_gemm(a, sa, b, sb).shape == (0, 64)
    assert mx.mx_gemm(b, sb, a, sa).shape == (64, 0)


@pytest.mark.slow
def test_launch_split_at_two_to_the_30_chunks(mx, oracle):
    """Rowwise quantize and dequantize split a problem into launches of at
    most 2^30 work items (chunks of 8 elements; for a bf16 dequantize, pieces
    of 8). A 2^27 + 96 row x 128 column bf16 input (32 GiB) is quantized and
    dequantized in three launches each (rows 0, 2^26, 2^27); rows on both
    sides of every boundary, and the first and last rows, are compared with
    the oracle bit for bit."""
    import torch
    rows, cols = (1 << 27) + 96, 128
    g = torch.Generator(device="cuda").manual_seed(21)
    x = torch.randn((rows, cols), device="cuda", dtype=torch.bfloat16, generator=g)
    q, s = mx.mx_quantize(x, E4M3)
    y = mx.mx_dequantize(q, s, E4M3, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    pick = np.concatenate([np.arange(0, 8), np.arange((1 << 26) - 40, (1 << 26) + 40),
                           np.arange((1 << 27) - 40, (1 << 27) + 40), np.arange(rows - 40, rows)])
    pick = np.unique(pick[pick < rows])
    idx = torch.from_numpy(pick).cuda()
    xs = x[idx].view(torch.int16).cpu().numpy().view(np.uint16)
    qo, so = oracle.quantize_rows(xs, E4M3)
    assert_bitexact(host(q[idx]), qo, "codes around the launch splits")
    assert_bitexact(host(s[idx]), so, "scales around the launch splits")
    assert_bitexact(host(y[idx]), oracle.dequantize(qo, so, E4M3, "bf16"), "dequantized rows around the splits")
    del x, q, s, y
    torch.cuda.empty_cache()


@pytest.mark.slow
def test_kv_write_launch_split(mx, oracle):
    """The fused KV write splits at 2^30 work items too: with 8 heads of 128,
    every 2^23 tokens. 2^23 + 64 tokens (K and V 17 GiB each) are written
    through a shuffled slot mapping; the cache slots of tokens on both sides
    of the split, and the last ones, are compared with the oracle."""
    import torch
    T, H, D, page = (1 << 23) + 64, 8, 128, 128
    pages = -(-T // page)
    g = torch.Generator(device="cuda").manual_seed(22)
    k = torch.randn((T, H, D), device="cuda", dtype=torch.bfloat16, generator=g)
    v = torch.randn((T, H, D), device="cuda", dtype=torch.bfloat16, generator=g)
    slots = torch.randperm(pages * page, device="cuda", generator=g)[:T].contiguous()
    kc = torch.empty((pages, page, H, D), dtype=torch.uint8, device="cuda")
    ks = torch.empty((pages, page, H, D // 32), dtype=torch.uint8, device="cuda")
    vc, vs = torch.empty_like(kc), torch.empty_like(ks)
    mx.mx_kv_quant_write(k, v, slots, kc, ks, vc, vs)
    torch.cuda.synchronize()
    pick = np.unique(np.concatenate([np.arange(0, 4), np.arange((1 << 23) - 32, (1 << 23) + 32), np.arange(T - 16, T)]))
    idx = torch.from_numpy(pick).cuda()
    sl = slots[idx]
    for src, cache, scale, name in ((k, kc, ks, "K"), (v, vc, vs, "V")):
        xs = src[idx].reshape(-1, D).view(torch.int16).cpu().numpy().view(np.uint16)
        qo, so = oracle.quantize_rows(xs, E4M3)
        got_q = cache.view(-1, H, D)[sl].reshape(-1, D)
        got_s = scale.view(-1, H, D // 32)[sl].reshape(-1, D // 32)
        assert_bitexact(host(got_q), qo, name + " cache codes around the launch split")
        assert_bitexact(host(got_s), so, name + " cache scales around the launch split")
    del k, v, kc, ks, vc, vs
    torch.cuda.empty_cache()
