"""GPU parity of mx_paged_attention against the oracle.

Tolerance, per output element (t, h, d), derived from the arithmetic:
  * scores: the scaled FP8 instruction may lose up to 2^-10 * T_j of a score
    (T_j = sum_d |q_hat k_hat_j|, the grouped-accumulation bound the GEMM tests
    use), so every logit moves by at most eps = sm_scale * 2^-10 * max_j T_j,
    and each normalised weight by a factor within exp(+-2 eps): the output
    moves by at most (exp(2 eps) - 1) * W with W = sum_j P_j |Vb_jd|;
  * P is rounded to bf16 for the matrix instruction. bf16 keeps 8
    significant bits, so each weight moves by at most 2^-8 of itself and the
    output by at most 2^-8 * W; as much again is allowed for the f32
    exponentials, sums and the final division;
  * bf16 output adds its own rounding, 2^-8 of |O| <= 2^-8 * W.
lse: |lse_gpu - lse_ref| <= eps + 1e-5 * (1 + |lse_ref|).
Inputs are quantized by the oracle on the CPU and the same codes are handed
to the GPU; the full-size case runs the GPU's own KV write and checks its
cache bit for bit against the oracle's first.
"""
import math

import numpy as np
import pytest

from attn_util import assert_attention_bound, quantized_case, run_attention
from gpu_util import assert_bitexact, bf16_to_f64, dev, host
from microscaling_block_scaled_amd import inputs

pytestmark = pytest.mark.gpu

E4M3 = 0


@pytest.fixture(scope="module")
def mx():
    import torch
    import microscaling_block_scaled_amd as m
    assert torch.cuda.is_available()
    ok, reason = m.mx_query_support(0)
    assert ok, reason
    return m


CASES = [
    # (n_seqs, q_len, kv_lens, page_size, q_heads, kv_heads)
    (2, 128, [128, 128], 128, 2, 2),        # one tile, one block
    (3, 200, [333, 70, 512], 128, 4, 2),    # ragged queries and keys, GQA
    (2, 1, [1000, 5], 256, 4, 1),           # decode, pages of 256
    (2, 50, [0, 300], 128, 2, 1),           # an empty sequence
    (1, 300, [140], 384, 1, 1),             # more queries than keys
]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("case", range(len(CASES)))
def test_attention_matches_oracle(mx, oracle, case, causal):
    S, ql, lens, page, hq, hkv = CASES[case]
    c = quantized_case(oracle, 8100 + case, S, ql, lens, page, hq, hkv, 128)
    sm = 1.0 / math.sqrt(128)
    ref = oracle.paged_attention(c["qc"], c["qs"], c["kc"], c["ks"], c["vc"], c["vs"], c["table"], c["kv_lens"], ql,
                                 sm, causal)
    for out_f32 in (True, False):
        o, lse = run_attention(mx, c, sm, causal, out_f32)
        worst = assert_attention_bound(o, lse, ref, sm, "case %d causal %d f32 %d" % (case, causal, out_f32),
                                       out_f32=out_f32)
        print("case %d causal %d f32 %d: worst |err|/W = %.3g" % (case, causal, out_f32, worst))


def _exact_score_case(oracle, seed, S, ql, lens, page, hq, hkv):
    """Q and K codes from {0, +-0.5, +-1, +-2} with block scales near 1: every
    group of 8 products is a multiple of 2^-2 below 2^5 in magnitude, so the
    scaled FP8 instruction sums it exactly and the GPU scores are exact."""
    c = quantized_case(oracle, seed, S, ql, lens, page, hq, hkv, 128)
    g = inputs.rng(seed + 50)
    vals = np.array([0x00, 0x30, 0xB0, 0x38, 0xB8, 0x40, 0xC0], dtype=np.uint8)
    for k in ("qc", "kc"):
        c[k] = vals[g.integers(0, len(vals), c[k].shape)]
    for k in ("qs", "ks"):
        c[k] = g.integers(125, 130, c[k].shape).astype(np.uint8)
    return c


@pytest.mark.parametrize("causal", [False, True])
def test_attention_exact_scores_and_one_hot(mx, oracle, causal):
    S, ql, lens, page, hq, hkv = 3, 160, [400, 160, 129], 128, 2, 1
    c = _exact_score_case(oracle, 8200, S, ql, lens, page, hq, hkv)
    sm = 1.0 / math.sqrt(128)
    ref = oracle.paged_attention(c["qc"], c["qs"], c["kc"], c["ks"], c["vc"], c["vs"], c["table"], c["kv_lens"], ql,
                                 sm, causal)
    o, lse = run_attention(mx, c, sm, causal, True)
    worst = assert_attention_bound(o, lse, ref, sm, "exact scores", score_rel=0.0)
    print("exact scores: worst |err|/W = %.3g" % worst)
    # one-hot: a softmax scale so large that every weight but the top key's
    # underflows to 0. Most rows then reduce to one key's bf16 V, so the
    # bound (exact scores: 2^-7 of |V_top|) pins the key order of P against V
    # at every key position; a wrong pairing misses by the size of V itself.
    big = 2000.0
    ref1 = oracle.paged_attention(c["qc"], c["qs"], c["kc"], c["ks"], c["vc"], c["vs"], c["table"], c["kv_lens"], ql,
                                  big, causal)
    o1, l1 = run_attention(mx, c, big, causal, True)
    # rows whose reference is a single key's value lie on the bf16 grid (an
    # f32 value whose low 16 bits are zero); rows mixing nearly tied keys do not
    f32 = ref1[0].astype(np.float32)
    one = np.all((f32.astype(np.float64) == ref1[0]) & ((f32.view(np.uint32) & 0xFFFF) == 0), axis=1)
    assert one.sum() > 0.5 * len(one)
    worst = assert_attention_bound(o1, l1, ref1, big, "one-hot", score_rel=0.0)
    print("one-hot: %d of %d rows single-key, worst |err|/W = %.3g" % (one.sum(), len(one), worst))


@pytest.mark.slow
def test_attention_kv_workload(mx, oracle):
    """64 sequences x 512 tokens x 8 heads x 128 on pages of 128: the GPU KV
    write fills the cache (checked bit for bit against the oracle's), the GPU
    quantizes Q, and sampled (token, head) rows of the attention output are
    compared with the oracle, non-causal (the timed configuration) and causal."""
    import torch
    k, v, q = inputs.kv_inputs()
    slots, table = inputs.kv_layout()
    T, H, D = k.shape
    kc = torch.zeros((256, 128, H, D), dtype=torch.uint8, device="cuda")
    ks = torch.zeros((256, 128, H, D // 32), dtype=torch.uint8, device="cuda")
    vc, vs = torch.zeros_like(kc), torch.zeros_like(ks)
    mx.mx_kv_quant_write(dev(k, bf16=True), dev(v, bf16=True), dev(slots), kc, ks, vc, vs)
    qq, qs = mx.mx_quantize(dev(q.reshape(-1, D), bf16=True), E4M3)
    kco, kso, vco, vso = oracle.kv_quant_write(k, v, slots, 128, 256)
    qo, qso = oracle.quantize_rows(q.reshape(-1, D), E4M3)
    assert_bitexact(host(kc), kco, "K cache")
    assert_bitexact(host(vc), vco, "V cache")
    assert_bitexact(host(ks), kso, "K scales")
    assert_bitexact(host(vs), vso, "V scales")
    assert_bitexact(host(qq), qo, "Q codes")
    lens = np.full(64, 512, np.int32)
    sm = 1.0 / math.sqrt(D)
    rows = inputs.rng(8300).choice(T * H, 1500, replace=False)
    for causal in (False, True):
        for out_dtype in (torch.bfloat16, torch.float32):
            lse = torch.empty((T, H), dtype=torch.float32, device="cuda")
            out = mx.mx_paged_attention(qq.view(T, H, D), qs.view(T, H, D // 32), kc, ks, vc, vs, dev(table),
                                        dev(lens), 512, sm_scale=sm, causal=causal, out_dtype=out_dtype, lse=lse)
            o = host(out.view(T * H, D)[dev(rows)])
            o = o.astype(np.float64) if out_dtype == torch.float32 else bf16_to_f64(o)
            l = host(lse.view(-1)[dev(rows)]).astype(np.float64)
            ref = oracle.paged_attention(qo.reshape(T, H, D), qso.reshape(T, H, D // 32), kco, kso, vco, vso, table,
                                         lens, 512, sm, causal, rows=rows)
            worst = assert_attention_bound(o, l, ref, sm, "kv workload causal %d" % causal,
                                           out_f32=out_dtype == torch.float32)
            print("kv workload causal %d %s: worst |err|/W = %.3g" % (causal, out_dtype, worst))


def test_attention_repeat_runs_identical(mx, oracle):
    c = quantized_case(oracle, 8400, 2, 256, [256, 200], 128, 2, 2, 128)
    a, la = run_attention(mx, c, 0.1, True, True)
    b, lb = run_attention(mx, c, 0.1, True, True)
    assert np.array_equal(a, b) and np.array_equal(la, lb)


def random_case(i):
    """Seeded random configuration i: sequences, queries, ragged kv_lens
    (zero allowed), page size, query/KV heads and the causal flag."""
    g = inputs.rng(8500 + i)
    S = int(g.integers(1, 4))
    ql = int(g.integers(1, 261))
    lens = [int(v) for v in g.integers(0, 901, S)]
    page = int(g.choice([128, 256, 384]))
    hq, hkv = [(1, 1), (2, 1), (4, 2), (8, 8), (8, 2), (6, 3)][int(g.integers(0, 6))]
    return S, ql, lens, page, hq, hkv, bool(g.integers(0, 2))


@pytest.mark.parametrize("i", range(16))
def test_attention_random_configurations(mx, oracle, i):
    S, ql, lens, page, hq, hkv, causal = random_case(i)
    c = quantized_case(oracle, 8600 + i, S, ql, lens, page, hq, hkv, 128)
    sm = 1.0 / math.sqrt(128)
    ref = oracle.paged_attention(c["qc"], c["qs"], c["kc"], c["ks"], c["vc"], c["vs"], c["table"], c["kv_lens"], ql,
                                 sm, causal)
    o, lse = run_attention(mx, c, sm, causal, True)
    assert_attention_bound(o, lse, ref, sm, "random case %d %s" % (i, (S, ql, lens, page, hq, hkv, causal)))
