"""Shared set-up of paged-attention cases: seeded bf16 inputs quantized to
MXFP8 E4M3 codes and scales by the CPU oracle (rowwise along the head
dimension, as the KV write stores them)."""
from microscaling_block_scaled_amd import inputs

E4M3 = 0


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
