"""Shared set-up of paged-attention cases (seeded bf16 inputs quantized to
MXFP8 E4M3 codes and scales by the CPU oracle, rowwise along the head
dimension, as the KV write stores them), the GPU call, and the per-element
bound the attention tests hold the output to."""
import numpy as np

from gpu_util import bf16_to_f64, dev, host
from microscaling_block_scaled_amd import inputs

E4M3 = 0
SCORE_REL = 2.0 ** -10
P_REL = 2.0 ** -7
BF16_OUT_REL = 2.0 ** -8


def run_attention(mx, c, sm, causal, out_f32):
    import torch
    T, Hq, D = c["qc"].shape
    lse = torch.empty((T, Hq), dtype=torch.float32, device="cuda")
    out = mx.mx_paged_attention(dev(c["qc"]), dev(c["qs"]), dev(c["kc"]), dev(c["ks"]), dev(c["vc"]), dev(c["vs"]),
                                dev(c["table"]), dev(c["kv_lens"]), c["q_len"], sm_scale=sm, causal=causal,
                                out_dtype=torch.float32 if out_f32 else torch.bfloat16, lse=lse)
    torch.cuda.synchronize()
    o = host(out)
    o = o.astype(np.float64) if out_f32 else bf16_to_f64(o)
    return o.reshape(T * Hq, D), host(lse).astype(np.float64).reshape(-1)


def assert_attention_bound(o, lse, ref, sm, what, out_f32=True, score_rel=SCORE_REL, keep=None, abs_extra=None):
    """Per-element bound (module docstring of the attention tests); `keep`
    (bool [rows, D]) restricts the output check to those elements;
    `abs_extra` ([rows, D]) is added to the bound (see small_weight_mass)."""
    o_ref, w_ref, lse_ref, tmax = ref
    eps = sm * score_rel * tmax
    rel = P_REL + np.expm1(2.0 * eps) + (0.0 if out_f32 else BF16_OUT_REL)
    bound = rel[:, None] * w_ref
    if abs_extra is not None:
        bound = bound + (1.0 + rel[:, None]) * abs_extra
    err = np.abs(o - o_ref)
    bad = ~(err <= bound)
    if keep is not None:
        bad &= keep
    assert not bad.any(), "%s: %d elements out of bound; first at %s: got %r want %r bound %r" % (
        what, bad.sum(), tuple(np.argwhere(bad)[0]), o[bad][0], o_ref[bad][0], bound[bad][0])
    live = np.isfinite(lse_ref)
    assert np.all(np.isneginf(lse[~live])), what + ": rows without keys must have lse = -inf"
    assert np.all(o[~live] == 0.0), what + ": rows without keys must be zero"
    lerr = np.abs(lse[live] - lse_ref[live])
    lb = eps[live] + 1e-5 * (1 + np.abs(lse_ref[live]))
    assert np.all(lerr <= lb), "%s: lse error %g > %g" % (what, lerr.max(), lb[np.argmax(lerr - lb)])
    with np.errstate(invalid="ignore", divide="ignore"):
        r = np.where((w_ref > 0) & (True if keep is None else keep), err / w_ref, 0.0)
    return float(r.max(initial=0.0))


def quantized_case(oracle, seed, n_seqs, q_len, kv_lens, page_size, q_heads, kv_heads, head_dim):
    """Returns dict(qc, qs, kc, ks, vc, vs, table, kv_lens, q_len) of numpy arrays."""
    q, k, v, table, lens = inputs.attention_case(seed, n_seqs, q_len, kv_lens, page_size, q_heads, kv_heads,
                                                 head_dim)
    D = head_dim

    def quant(x):
        c, s = oracle.quantize_rows(x.reshape(-1, D), E4M3)
        return c.reshape(x.shape), s.reshape(x.shape[:-1] + (D // 32,))

    qc, qs = quant(q)
    kc, ks = quant(k)
    vc, vs = quant(v)
    return dict(qc=qc, qs=qs, kc=kc, ks=ks, vc=vc, vs=vs, table=table, kv_lens=lens, q_len=q_len)


SMALL_WEIGHT = 2.0 ** -116


def small_weight_mass(oracle, c, sm, causal, tau=SMALL_WEIGHT):
    """Per output [rows, D]: sum over the keys j with softmax weight P_j < tau
    of P_j |V_jd|, in f64 from the dequantized operands. The kernel rounds
    its weights to bf16 after moving up to 2^10 of a key's V scale onto them,
    so a weight under 2^-116 may fall below bf16's normal range and be
    flushed or rounded coarsely; those terms are outside the relative bound
    and this mass bounds them."""
    tab = oracle.decode_table(E4M3)

    def deq(codes, scales):
        return np.ldexp(tab[codes], np.repeat(scales.astype(np.int64) - 127, 32, axis=-1))

    T, Hq, D = c["qc"].shape
    _, page, Hkv, _ = c["kc"].shape
    S, ql = c["table"].shape[0], c["q_len"]
    q = deq(c["qc"], c["qs"])
    k = deq(c["kc"], c["ks"]).reshape(-1, Hkv, D)
    v = np.abs(deq(c["vc"], c["vs"])).reshape(-1, Hkv, D)
    out = np.zeros((T * Hq, D))
    for s in range(S):
        L = int(c["kv_lens"][s])
        j = np.arange(L)
        slot = c["table"][s, j // page].astype(np.int64) * page + j % page
        for h in range(Hq):
            hk = h // (Hq // Hkv)
            sc = q[s * ql:(s + 1) * ql, h] @ k[slot, hk].T * sm
            if causal:
                sc[j[None, :] > (L - ql + np.arange(ql))[:, None]] = -np.inf
            live = np.isfinite(sc.max(axis=1))
            p = np.zeros_like(sc)
            p[live] = np.exp(sc[live] - sc[live].max(axis=1, keepdims=True))
            p[live] /= p[live].sum(axis=1, keepdims=True)
            out[(s * ql + np.arange(ql)) * Hq + h] = np.where(p < tau, p, 0.0) @ v[slot, hk]
    return out
