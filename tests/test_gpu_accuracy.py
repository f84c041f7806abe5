"""GPU accuracy of the block-scaled product and of paged attention on data
that stresses them, checked against the oracle on every output.

1. The accumulation modes on data whose rounding errors cannot cancel:
   same-sign operands (|N(0,1)|) and heavy tails (Student-t, nu = 3), at
   K = 2048 and K = 8192 with E4M3 operands. AUTO and FP32 must meet the
   product bound |y - y_ref| <= 1e-5 * sum_k |a_k b_k| on every output;
   forced FP8 is held to its own grouped bound (2^-10).

2. The full E8M0 range [MXFP8 SM120 software support, §0.1: a finite scale
   is 2^k with -127 <= k <= 127]. Blocks with scale codes at both ends
   (E4M3: 0..3 and 246, 247, 254; E5M2: 0..10 and 239..254) are mixed with
   ordinary ones across the A and B operands (high scales of one operand
   meet low ones of the other, so the products stay in f32 range), in all
   three accumulation modes and on every kernel (row-panel, general,
   large-tile). The bound applies wherever the f32 result is representable
   at the bound's resolution: 2^-100 <= sum |a b| <= 2^120 (smaller sums fall
   below the f32 grid, larger ones may overflow a partial sum).

3. The NaN scale code [same section: E8M0 has one NaN code besides the
   finite scales]: a block under 0xFF is NaN, so every output it enters is
   NaN, also when its element codes are all zero.

4. Paged attention with Q, K and V scales from both ends of the range, and
   the NaN code in Q, K and V.

5. The exact pass in the grouped product (large-tile kernel) and with B
   read through a page table (row-panel and general kernels).
"""
import numpy as np
import pytest

from gpu_util import FP8_GROUPED_REL, REL_T, assert_gemm_bound, bf16_to_f64, dev, host
from microscaling_block_scaled_amd import inputs

pytestmark = pytest.mark.gpu

E4M3, E5M2, E2M1 = 0, 1, 2
AUTO, FP8, FP32 = 0, 1, 2
MODE_NAME = {AUTO: "AUTO", FP8: "FP8", FP32: "FP32"}


@pytest.fixture(scope="module")
def mx():
    import torch
    import microscaling_block_scaled_amd as m
    assert torch.cuda.is_available()
    ok, reason = m.mx_query_support(0)
    assert ok, reason
    return m


def _gemm(mx, qa, sa, qb, sb, afmt, bfmt, accum, f32=True):
    import torch
    y = mx.mx_gemm(dev(qa), dev(sa), dev(qb), dev(sb), afmt, bfmt,
                   out_dtype=torch.float32 if f32 else torch.bfloat16, accum=accum)
    y = host(y)
    return y.astype(np.float64) if f32 else bf16_to_f64(y)


# --------------------------------------------------------------------------- 1. data that does not cancel
def _dist(name, seed, shape):
    if name == "normal":
        return inputs.normal_bf16(seed, shape)
    if name == "same_sign":
        return inputs.abs_normal_bf16(seed, shape)
    if name == "student_t":
        return inputs.student_t_bf16(seed, shape, scale=1.0)
    raise ValueError(name)


@pytest.mark.parametrize("K", [2048, 8192])
@pytest.mark.parametrize("dist", ["normal", "same_sign", "student_t"])
def test_accumulation_modes_on_hard_data(mx, oracle, dist, K):
    M = N = 512
    xa = _dist(dist, 7100 + K, (M, K))
    xb = _dist(dist, 7200 + K, (N, K))
    qa, sa = oracle.quantize_rows(xa, E4M3)
    qb, sb = oracle.quantize_rows(xb, E4M3)
    y_ref, t_ref = oracle.gemm(qa, sa, E4M3, qb, sb, E4M3)
    worst = {}
    for accum in (AUTO, FP32, FP8):
        rel = FP8_GROUPED_REL if accum == FP8 else REL_T
        what = "%s K=%d %s" % (dist, K, MODE_NAME[accum])
        y = _gemm(mx, qa, sa, qb, sb, E4M3, E4M3, accum)
        worst[MODE_NAME[accum]] = assert_gemm_bound(y, y_ref, t_ref, what + " f32", rel=rel)
        yb = _gemm(mx, qa, sa, qb, sb, E4M3, E4M3, accum, f32=False)
        assert_gemm_bound(yb, y_ref, t_ref, what + " bf16", bf16_out=True, rel=rel)
    print("%s K=%d worst |err|/T: %s" % (dist, K, " ".join("%s %.3g" % kv for kv in worst.items())))


# --------------------------------------------------------------------------- 2. the whole E8M0 range


def _finite_codes(g, fmt, shape, small=False):
    """Random element codes of finite values (no NaN / Inf codes); `small`
    keeps magnitudes <= 0.25 (E2M1: <= 1) so that blocks under the largest
    scales stay in f32 range. E2M1: `shape` counts elements, two per byte."""
    if fmt == E2M1:
        pool = np.arange(16, dtype=np.uint8)
        if small:
            pool = pool[(pool & 7) <= 2]
        shp = tuple(shape[:-1]) + (shape[-1] // 2,) if len(shape) > 0 else shape
        lo = pool[g.integers(0, pool.size, shp)]
        hi = pool[g.integers(0, pool.size, shp)]
        return (lo | (hi << 4)).astype(np.uint8)
    if fmt == E4M3:
        pool = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
        lim = 0x28  # 0.25
    else:
        pool = np.array([c for c in range(256) if (c & 0x7F) < 0x7C], np.uint8)
        lim = 0x34  # 0.25
    if small:
        pool = pool[(pool & 0x7F) <= lim]
    return pool[g.integers(0, pool.size, shape)]


LOW = {E4M3: [0, 1, 2, 3], E5M2: list(range(0, 11)), E2M1: [0, 1, 2]}
HIGH = {E4M3: [246, 247, 254], E5M2: list(range(239, 255)), E2M1: [252, 253, 254]}


def _attention_v(g, vs_shape):
    """E4M3 V scales and codes for the attention case. Per key and 32-wide
    block the scale is low (0..3, 9, 10), high (246..254) or ordinary
    (100..154), so most keys hold blocks from both ends; the high blocks hold
    zero codes except for one element in 64 with a tiny magnitude (2^-9 ..
    2^-7), so that an output column meets about one nonzero high value and W
    stays within the range of the kernel's unnormalised sum."""
    u = g.random(vs_shape)
    vs = g.integers(100, 155, vs_shape).astype(np.uint8)
    low = u < 0.3
    high = (u >= 0.3) & (u < 0.55)
    vs[low] = np.array([0, 1, 2, 3, 9, 10], np.uint8)[g.integers(0, 6, int(low.sum()))]
    vs[high] = g.integers(246, 255, int(high.sum()))
    vc = _finite_codes(g, E4M3, vs_shape[:-1] + (vs_shape[-1] * 32,))
    big = np.repeat(high, 32, axis=-1)
    nz = big & (g.random(big.shape) < 1 / 64)
    tiny = np.array([1, 2, 3, 4, 0x81, 0x82, 0x83, 0x84], np.uint8)  # +-2^-9 .. +-2^-7
    vc[big] = 0
    vc[nz] = tiny[g.integers(0, tiny.size, int(nz.sum()))]
    return vs, vc


def _pick(g, shape, choices):
    """Per element, a code drawn from one of the (probability, code list) choices."""
    out = np.empty(shape, np.uint8)
    u = g.random(shape)
    acc = 0.0
    for p, codes in choices:
        sel = (u >= acc) & (u < acc + p)
        codes = np.asarray(codes, np.uint8)
        out[sel] = codes[g.integers(0, codes.size, int(sel.sum()))]
        acc += p
    return out


def _extreme_pair(g, afmt, bfmt, M, N, K):
    """Codes and scales of A [M, K] and B [N, K] whose blocks use both ends of
    the E8M0 range. Each 32-wide block column is one of three kinds: ordinary
    (both operands ordinary or low), A-high (A's rows high, low or ordinary,
    every B row low) or B-high (the mirror), so that high scales only ever
    meet low ones and the products of the blocks stay inside f32 range. Within
    one block column an operand's codes can span nearly the whole range."""
    kb = K // 32
    kind = g.choice(3, size=kb, p=[0.4, 0.3, 0.3])
    norm = list(range(100, 155))
    sa = np.empty((M, kb), np.uint8)
    sb = np.empty((N, kb), np.uint8)
    for b in range(kb):
        if kind[b] == 0:
            sa[:, b] = _pick(g, M, [(0.7, norm), (0.3, LOW[afmt])])
            sb[:, b] = _pick(g, N, [(0.7, norm), (0.3, LOW[bfmt])])
        elif kind[b] == 1:
            sa[:, b] = _pick(g, M, [(0.4, HIGH[afmt]), (0.2, LOW[afmt]), (0.4, norm)])
            sb[:, b] = _pick(g, N, [(1.0, LOW[bfmt])])
        else:
            sa[:, b] = _pick(g, M, [(1.0, LOW[afmt])])
            sb[:, b] = _pick(g, N, [(0.4, HIGH[bfmt]), (0.2, LOW[bfmt]), (0.4, norm)])

    def codes(fmt, s, rows):
        q = _finite_codes(g, fmt, (rows, K))
        # blocks under scales whose 2^(s - 127) * 448 (57344, 6) would overflow f32 get small codes
        per = 16 if fmt == E2M1 else 32  # code bytes per block
        big = np.repeat(s >= {E4M3: 240, E5M2: 232, E2M1: 250}[fmt], per, axis=1)
        q[big] = _finite_codes(g, fmt, (int(big.sum()) * (2 if fmt == E2M1 else 1),), small=True)
        return q

    return codes(afmt, sa, M), sa, codes(bfmt, sb, N), sb


def _mode_rel(afmt, bfmt, accum):
    """The bound a product is held to: 1e-5 * sum|a b| in the FP32-
    accumulation mode (AUTO's choice except for MXFP4 x MXFP4) and for
    MXFP4 x MXFP4 on the instruction (exact), the grouped bound 2^-10 on the
    scaled FP8 instruction otherwise."""
    fp4 = afmt == E2M1 and bfmt == E2M1
    on_instruction = accum == FP8 or (accum == AUTO and fp4)
    return FP8_GROUPED_REL if on_instruction and not fp4 else REL_T


def _representable(y_ref, t_ref):
    return (t_ref >= 2.0 ** -100) & (t_ref <= 2.0 ** 120)


# one shape per kernel: row-panel (K <= 128, N <= 512, FP32-accumulation
# mode), the general kernel, the large-tile kernel (K % 512 == 0, M, N >= 256)
EXTREME_SHAPES = [(300, 200, 96), (130, 129, 160), (256, 512, 512), (512, 256, 2048)]


@pytest.mark.parametrize("M,N,K", EXTREME_SHAPES)
@pytest.mark.parametrize("afmt,bfmt", [(E4M3, E4M3), (E5M2, E4M3), (E4M3, E5M2), (E5M2, E5M2), (E2M1, E2M1),
                                       (E2M1, E4M3), (E5M2, E2M1)])
@pytest.mark.parametrize("accum", [AUTO, FP8, FP32])
def test_extreme_scale_codes(mx, oracle, M, N, K, afmt, bfmt, accum):
    g = inputs.rng(7300 + M + N + K + 10 * afmt + 20 * bfmt)
    qa, sa, qb, sb = _extreme_pair(g, afmt, bfmt, M, N, K)
    y_ref, t_ref = oracle.gemm(qa, sa, afmt, qb, sb, bfmt)
    keep = _representable(y_ref, t_ref)
    assert keep.mean() > 0.5, "too few representable outputs: %.2f" % keep.mean()
    rel = _mode_rel(afmt, bfmt, accum)
    what = "%s x %s %s %s" % (afmt, bfmt, MODE_NAME[accum], (M, N, K))
    y = _gemm(mx, qa, sa, qb, sb, afmt, bfmt, accum)
    worst = assert_gemm_bound(y[keep], y_ref[keep], t_ref[keep], what + " f32", rel=rel)
    yb = _gemm(mx, qa, sa, qb, sb, afmt, bfmt, accum, f32=False)
    ok_b = keep & (np.abs(y_ref) < 2.0 ** 126)
    assert_gemm_bound(yb[ok_b], y_ref[ok_b], t_ref[ok_b], what + " bf16", bf16_out=True, rel=rel)
    print("%s: worst |err|/T %.3g over %d representable outputs" % (what, worst, int(keep.sum())))


# --------------------------------------------------------------------------- 3. the NaN scale code
NAN_CASES = [(a, b, m) for a, b in [(E4M3, E4M3), (E5M2, E4M3), (E2M1, E2M1), (E2M1, E4M3), (E4M3, E2M1)]
             for m in (AUTO, FP8, FP32)]


@pytest.mark.parametrize("M,N,K", EXTREME_SHAPES)
@pytest.mark.parametrize("afmt,bfmt,accum", NAN_CASES)
def test_nan_scale_code(mx, oracle, M, N, K, afmt, bfmt, accum):
    g = inputs.rng(7500 + M + N + K + afmt + 3 * bfmt)
    qa, sa = oracle.quantize_rows(inputs.normal_bf16(7501 + K + afmt, (M, K)), afmt)
    qb, sb = oracle.quantize_rows(inputs.normal_bf16(7502 + K + bfmt, (N, K)), bfmt)
    kb = K // 32
    ra, ba = g.choice(M, 3, replace=False), g.integers(0, kb, 3)
    rb, bb = g.choice(N, 3, replace=False), g.integers(0, kb, 3)
    sa[ra, ba] = 0xFF
    sb[rb, bb] = 0xFF
    wa, wb = (16 if afmt == E2M1 else 32), (16 if bfmt == E2M1 else 32)  # code bytes per block
    qa[ra[0], wa * ba[0]:wa * ba[0] + wa] = 0  # NaN scale over zero codes
    qb[rb[0], wb * bb[0]:wb * bb[0] + wb] = 0
    y_ref, t_ref = oracle.gemm(qa, sa, afmt, qb, sb, bfmt)
    nan_ref = np.isnan(y_ref)
    assert nan_ref.sum() == 3 * N + 3 * M - 9  # three whole rows and three whole columns
    what = "NaN scale %s x %s %s %s" % (afmt, bfmt, MODE_NAME[accum], (M, N, K))
    rel = _mode_rel(afmt, bfmt, accum)
    for f32 in (True, False):
        y = _gemm(mx, qa, sa, qb, sb, afmt, bfmt, accum, f32=f32)
        bad = np.isnan(y) != nan_ref
        assert not bad.any(), "%s f32 %d: NaN pattern differs at %d outputs, first %s (got %r)" % (
            what, f32, bad.sum(), tuple(np.argwhere(bad)[0]), y[bad][0])
        assert_gemm_bound(y[~nan_ref], y_ref[~nan_ref], t_ref[~nan_ref], what + (" f32" if f32 else " bf16"),
                          bf16_out=not f32, rel=rel)


# --------------------------------------------------------------------------- 4. attention over the whole E8M0 range
@pytest.mark.parametrize("causal", [False, True])
def test_attention_extreme_scale_codes(mx, oracle, causal):
    """V blocks with scale codes from both ends of the E8M0 range mixed with
    ordinary ones, within every key and across keys; Q and K blocks at the
    ends of the range in pairs whose products stay moderate (query block b at
    code c_b, key block b near 242 - c_b), so the scores are ordinary numbers
    computed from extreme operands. Checked on every output element whose
    W = sum_j P_j |Vb_jd| satisfies 2^-100 <= W <= 2^110: the kernel forms the
    unnormalised sum of P_j * V_jd with weights up to 2^8, so with at most
    333 keys that sum stays below 2^8 * 2^8.4 * 2^110 < 2^127."""
    import math
    from attn_util import assert_attention_bound, quantized_case, run_attention, small_weight_mass
    S, ql, lens, page, hq, hkv = 2, 200, [333, 256], 128, 2, 1
    c = quantized_case(oracle, 7400, S, ql, lens, page, hq, hkv, 128)
    g = inputs.rng(7401)
    c["vs"], c["vc"] = _attention_v(g, c["vs"].shape)
    qbase = np.array([0, 2, 240, 242], np.int64)[g.integers(0, 4, 4)]
    jq = g.integers(0, 3, c["qs"].shape)
    jk = g.integers(0, 3, c["ks"].shape)
    c["qs"] = np.where(qbase < 128, qbase + jq, qbase - jq).astype(np.uint8)
    kbase = 242 - qbase
    c["ks"] = np.where(kbase < 128, kbase + jk, kbase - jk).astype(np.uint8)
    sm = 1.0 / math.sqrt(128)
    ref = oracle.paged_attention(c["qc"], c["qs"], c["kc"], c["ks"], c["vc"], c["vs"], c["table"], c["kv_lens"], ql,
                                 sm, causal)
    o_ref, w_ref = ref[0], ref[1]
    keep = (w_ref >= 2.0 ** -100) & (w_ref <= 2.0 ** 110)
    assert keep.mean() > 0.9, "too few representable outputs: %.2f" % keep.mean()
    small = small_weight_mass(oracle, c, sm, causal)
    for out_f32 in (True, False):
        o, lse = run_attention(mx, c, sm, causal, out_f32)
        k = keep if out_f32 else keep & (np.abs(o_ref) < 2.0 ** 126)
        worst = assert_attention_bound(o, lse, ref, sm, "extreme scales causal %d f32 %d" % (causal, out_f32),
                                       out_f32=out_f32, keep=k, abs_extra=small)
        print("extreme scales causal %d f32 %d: worst |err|/W = %.3g" % (causal, out_f32, worst))


@pytest.mark.parametrize("causal", [False, True])
def test_attention_nan_scale_codes(mx, oracle, causal):
    """Scale code 0xFF in Q, K and V. A NaN query block makes its row NaN; a
    NaN key block makes NaN every row that sees the key; a NaN value block
    makes NaN its 32 output columns in every row that sees the key, and may
    also do so in the rows of the same 128-query tile that the causal mask
    hides it from (its zero weight times NaN is NaN inside the matrix
    instruction). Every other output keeps the attention bound."""
    import math
    from attn_util import assert_attention_bound, quantized_case, run_attention
    S, ql, lens, page, hq, hkv, D = 2, 200, [333, 256], 128, 2, 1, 128
    c = quantized_case(oracle, 7600, S, ql, lens, page, hq, hkv, D)

    def slot(s, j):
        return int(c["table"][s, j // page]) * page + j % page

    vs = c["vs"].reshape(-1, hkv, D // 32)
    ks = c["ks"].reshape(-1, hkv, D // 32)
    vkey, vblk = (0, 300), 1    # seen by queries >= 167 of sequence 0 under the mask
    vs[slot(*vkey), 0, vblk] = 0xFF
    ks[slot(1, 100), 0, 2] = 0xFF
    c["qs"][7, 1, 0] = 0xFF     # token 7 (sequence 0), head 1
    sm = 1.0 / math.sqrt(D)
    ref = oracle.paged_attention(c["qc"], c["qs"], c["kc"], c["ks"], c["vc"], c["vs"], c["table"], c["kv_lens"], ql,
                                 sm, causal)
    o_ref, w_ref, lse_ref, tmax = ref
    nan_ref = np.isnan(o_ref)
    # where the kernel may also give NaN: the value block's columns in every
    # row of a query tile that reads the key
    T = S * ql
    may = nan_ref.copy()
    s, j = vkey
    L = int(c["kv_lens"][s])
    for qt in range((ql + 127) // 128):
        q_last = min(qt * 128 + 127, ql - 1)
        kmax = min(L, L - ql + q_last + 1) if causal else L
        if j < kmax:
            for tok in range(s * ql + qt * 128, s * ql + q_last + 1):
                for h in range(hq):
                    may[tok * hq + h, 32 * vblk:32 * vblk + 32] = True
    assert nan_ref[:, 32 * vblk:32 * vblk + 32].any() and np.isnan(lse_ref).sum() > 0
    rows_ok = ~np.isnan(lse_ref)
    for out_f32 in (True, False):
        o, lse = run_attention(mx, c, sm, causal, out_f32)
        what = "NaN scale codes causal %d f32 %d" % (causal, out_f32)
        got = np.isnan(o)
        assert not (nan_ref & ~got).any(), "%s: %d outputs should be NaN, first %s" % (
            what, (nan_ref & ~got).sum(), tuple(np.argwhere(nan_ref & ~got)[0]))
        assert not (got & ~may).any(), "%s: %d outputs NaN where they should not be, first %s" % (
            what, (got & ~may).sum(), tuple(np.argwhere(got & ~may)[0]))
        assert np.all(np.isnan(lse[~rows_ok])), what + ": rows with a NaN score must have lse = NaN"
        sub = (o_ref[rows_ok], w_ref[rows_ok], lse_ref[rows_ok], tmax[rows_ok])
        assert_attention_bound(o[rows_ok], lse[rows_ok], sub, sm, what, out_f32=out_f32, keep=~may[rows_ok])


# --------------------------------------------------------------------------- the whole range in grouped and paged products
@pytest.mark.parametrize("bfmt", [E4M3, E5M2])
@pytest.mark.parametrize("accum", [AUTO, FP32])
def test_grouped_extreme_scale_codes(mx, oracle, bfmt, accum):
    """The exact pass of the large-tile kernel in grouped mode: each group's
    rows and its own B drawn like the extreme-range pairs above, ragged and
    empty groups, every representable output of every group."""
    import torch
    sizes, N, K, afmt = [300, 0, 17, 257, 40], 256, 1024, E4M3
    g = inputs.rng(7700 + bfmt + 4 * accum)
    parts = [_extreme_pair(g, afmt, bfmt, max(m, 1), N, K) for m in sizes]
    qa = np.concatenate([p[0][:m] for p, m in zip(parts, sizes)])
    sa = np.concatenate([p[1][:m] for p, m in zip(parts, sizes)])
    qb = np.concatenate([p[2] for p in parts])
    sb = np.concatenate([p[3] for p in parts])
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    G = len(sizes)
    for f32 in (True, False):
        dt = torch.float32 if f32 else torch.bfloat16
        y = torch.zeros((int(off[-1]), N), dtype=dt, device="cuda")
        mx.mx_grouped_gemm(dev(qa), dev(sa), dev(qb).view(G, N, K), dev(sb).view(G, N, K // 32), dev(off), a_fmt=afmt,
                           b_fmt=bfmt, y=y, accum=accum)
        yh = host(y)
        yh = yh.astype(np.float64) if f32 else bf16_to_f64(yh)
        for q in range(G):
            r0, r1 = int(off[q]), int(off[q + 1])
            if r1 == r0:
                continue
            y_ref, t_ref = oracle.gemm(qa[r0:r1], sa[r0:r1], afmt, qb[q * N:(q + 1) * N], sb[q * N:(q + 1) * N], bfmt)
            keep = _representable(y_ref, t_ref)
            if not f32:
                keep &= np.abs(y_ref) < 2.0 ** 126
            assert_gemm_bound(yh[r0:r1][keep], y_ref[keep], t_ref[keep], "grouped extreme group %d f32 %d" % (q, f32),
                              bf16_out=not f32)


@pytest.mark.parametrize("K,N", [(96, 300), (160, 129)])
@pytest.mark.parametrize("afmt,bfmt", [(E4M3, E4M3), (E5M2, E4M3)])
def test_paged_extreme_scale_codes(mx, oracle, K, N, afmt, bfmt):
    """The exact pass with B read through a page table (the row-panel kernel
    at K = 96, the general kernel at K = 160), FP32-accumulation mode."""
    import torch
    M, page_rows = 200, 64
    pages_per_seq = (N + page_rows - 1) // page_rows
    n_pages = pages_per_seq + 2
    g = inputs.rng(7800 + K + N + afmt)
    qa, sa, qbp, sbp = _extreme_pair(g, afmt, bfmt, M, n_pages * page_rows, K)
    table = g.permutation(n_pages)[:pages_per_seq].astype(np.int32)
    rows = table[np.arange(N) // page_rows].astype(np.int64) * page_rows + np.arange(N) % page_rows
    y_ref, t_ref = oracle.gemm(qa, sa, afmt, np.ascontiguousarray(qbp[rows]), np.ascontiguousarray(sbp[rows]), bfmt)
    keep = _representable(y_ref, t_ref)
    assert keep.mean() > 0.5
    dqa, dsa, dqb, dsb, dtab = dev(qa), dev(sa), dev(qbp), dev(sbp), dev(table)
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    d = mx.mx_gemm_desc_t()
    d.M, d.N, d.K = M, N, K
    d.a, d.lda, d.sa, d.ldsa, d.a_fmt = dqa.data_ptr(), K, dsa.data_ptr(), K // 32, afmt
    d.b, d.ldb, d.sb, d.ldsb, d.b_fmt = dqb.data_ptr(), K, dsb.data_ptr(), K // 32, bfmt
    d.y, d.ldy, d.y_dtype = y.data_ptr(), N, 0
    d.b_page_table = dtab.data_ptr()
    d.b_pages_per_seq, d.b_page_rows = pages_per_seq, page_rows
    d.b_page_stride, d.b_page_stride_s = page_rows * K, page_rows * (K // 32)
    d.accum = FP32
    mx.mx_gemm_desc(d)
    torch.cuda.synchronize()
    worst = assert_gemm_bound(host(y).astype(np.float64)[keep], y_ref[keep], t_ref[keep], "paged extreme K=%d" % K)
    print("paged extreme K=%d N=%d %d x %d: worst |err|/T %.3g" % (K, N, afmt, bfmt, worst))
