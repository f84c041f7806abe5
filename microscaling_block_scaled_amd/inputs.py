"""Seeded synthetic inputs for the five workloads (no MX arithmetic here).

Both the HIP path and the CPU oracle are fed from these generators; the module
itself quantizes nothing. Every array is produced by numpy's PCG64 generator
from a fixed seed, drawn in float32 (float64 for Student-t) and rounded to
bfloat16 with round-to-nearest-even on the host. bf16 tensors are returned as
their 16-bit patterns (``np.uint16``).

Workloads (sizes as given for the method's headline runs):
  * tiny:     64-element vector of 32 x 2^10 then 32 x 2^-12 (f32); A [64, 128]
              and B [128, 64] f32 ~ N(0, 1), seeds 1001 / 1002.
  * quantize: X bf16 [8192, 4096] ~ N(0, 1) (seed 2001) with 4 outlier
              channels multiplied by 2^12, one per distinct 32-column block
              (seed 2002).
  * gemm:     A bf16 [8192, 8192], B bf16 [N=8192, K=8192] ~ N(0, 1),
              seeds 3001 / 3002.
  * training: X bf16 [16384, 4096] ~ N(0, 1) (4001); W bf16 [N=14336,
              K=4096] ~ N(0, 0.02) (4002); G bf16 [16384, 14336] ~ Student-t
              (nu = 3) * 1e-3 (4003).
  * kv:       K, V, Q bf16 [32768 tokens, 8 heads, 128] ~ N(0, 1) (5001 /
              5002 / 5003); 64 sequences of 512 tokens on pages of 128 tokens;
              sequence s owns logical pages 4s..4s+3, mapped to physical pages
              by a seeded permutation of 0..255 (5004).
  * moe:      32768 rows (16384 tokens x top-2) split over 8 experts by
              `moe_group_sizes` (seed 6001); X bf16 [32768, 4096] ~ N(0, 1)
              (6002), expert weights bf16 [8 x 4096, 4096] ~ N(0, 0.02) (6003).
  * attention: the kv workload read back as paged attention: the query of
              every token (seed 5003) attends over its sequence's 512 cached
              keys. Smaller cases (`attention_case`) draw a ragged mix of
              sequence lengths and a shuffled page table from one seed.
All sizes can be scaled down (same distributions) for tests that must finish
quickly on the CPU.
"""
import numpy as np


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); returns the
    16-bit patterns. Inputs here are finite and far from the bf16 limits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_bf16(seed: int, shape, sigma: float = 1.0, chunk_rows: int = 1024) -> np.ndarray:
    """bf16 patterns of N(0, sigma^2) float32 draws, generated row-chunk by
    row-chunk so that large tensors never hold a float64 copy."""
    g = rng(seed)
    shape = tuple(shape)
    out = np.empty(shape, np.uint16)
    flat = out.reshape(shape[0], -1)
    for r0 in range(0, shape[0], chunk_rows):
        r1 = min(shape[0], r0 + chunk_rows)
        x = g.standard_normal((r1 - r0, flat.shape[1]), dtype=np.float32)
        if sigma != 1.0:
            x *= np.float32(sigma)
        flat[r0:r1] = f32_to_bf16_bits(x)
    return out


def student_t_bf16(seed: int, shape, df: float = 3.0, scale: float = 1e-3, chunk_rows: int = 512) -> np.ndarray:
    g = rng(seed)
    out = np.empty(tuple(shape), np.uint16)
    for r0 in range(0, shape[0], chunk_rows):
        r1 = min(shape[0], r0 + chunk_rows)
        x = (g.standard_t(df, size=(r1 - r0, shape[1])) * scale).astype(np.float32)
        out[r0:r1] = f32_to_bf16_bits(x)
    return out


def abs_normal_bf16(seed: int, shape, chunk_rows: int = 1024) -> np.ndarray:
    """bf16 patterns of |N(0, 1)| float32 draws: same-sign data, for which the
    rounding errors of a sum cannot cancel between terms."""
    out = normal_bf16(seed, shape, chunk_rows=chunk_rows)
    return out & np.uint16(0x7FFF)


# ---------------------------------------------------------------- workloads
def tiny():
    v64 = np.concatenate([np.full(32, 2.0 ** 10, np.float32), np.full(32, 2.0 ** -12, np.float32)])[None, :]
    a = rng(1001).standard_normal((64, 128), dtype=np.float32)
    b = rng(1002).standard_normal((128, 64), dtype=np.float32)
    return {"v64": v64, "A": a, "B": b}


def quantize_input(rows: int = 8192, cols: int = 4096, n_outliers: int = 4, outlier_scale: float = 2.0 ** 12):
    """X with `n_outliers` outlier channels, each in a different 32-column
    block, multiplied by `outlier_scale` (a power of two, exact in bf16)."""
    x = normal_bf16(2001, (rows, cols))
    g = rng(2002)
    blocks = g.choice(cols // 32, size=n_outliers, replace=False)
    channels = np.sort(blocks * 32 + g.integers(0, 32, size=n_outliers))
    xf = bf16_bits_to_f32(x[:, channels]) * np.float32(outlier_scale)
    x[:, channels] = f32_to_bf16_bits(xf)
    return x, channels


def gemm_inputs(m: int = 8192, n: int = 8192, k: int = 8192):
    return normal_bf16(3001, (m, k)), normal_bf16(3002, (n, k))


def training_inputs(tokens: int = 16384, d_in: int = 4096, d_out: int = 14336, with_grad: bool = True):
    x = normal_bf16(4001, (tokens, d_in))
    w = normal_bf16(4002, (d_out, d_in), sigma=0.02)
    gr = student_t_bf16(4003, (tokens, d_out)) if with_grad else None
    return x, w, gr


def kv_layout(n_seqs: int = 64, seq_len: int = 512, page_size: int = 128, n_pages: int = 256):
    """Slot mapping (int64 [n_seqs*seq_len]) and page table (int32
    [n_seqs, seq_len/page_size]) for sequences laid out on shuffled pages."""
    pages_per_seq = seq_len // page_size
    assert n_seqs * pages_per_seq <= n_pages
    perm = rng(5004).permutation(n_pages).astype(np.int64)
    page_table = perm[: n_seqs * pages_per_seq].reshape(n_seqs, pages_per_seq)
    t = np.arange(n_seqs * seq_len, dtype=np.int64)
    seq, pos = t // seq_len, t % seq_len
    slot = page_table[seq, pos // page_size] * page_size + pos % page_size
    return slot, page_table.astype(np.int32)


def kv_inputs(tokens: int = 32768, heads: int = 8, head_dim: int = 128):
    k = normal_bf16(5001, (tokens, heads, head_dim))
    v = normal_bf16(5002, (tokens, heads, head_dim))
    q = normal_bf16(5003, (tokens, heads, head_dim))
    return k, v, q


def attention_case(seed: int, n_seqs: int, q_len: int, kv_lens, page_size: int, q_heads: int, kv_heads: int,
                   head_dim: int, spare_pages: int = 3):
    """Inputs of a paged-attention case: bf16 queries [n_seqs*q_len, q_heads,
    head_dim], bf16 cache contents for every slot [pages, page_size, kv_heads,
    head_dim] (K and V), an int32 page table [n_seqs, pages_per_seq] drawn as a
    shuffled subset of the pages, and int32 kv_lens. All values ~ N(0, 1)."""
    kv_lens = np.asarray(kv_lens, dtype=np.int32)
    assert kv_lens.shape == (n_seqs,)
    pps = max(1, -(-int(kv_lens.max(initial=0)) // page_size))
    n_pages = n_seqs * pps + spare_pages
    table = rng(seed).permutation(n_pages)[: n_seqs * pps].reshape(n_seqs, pps).astype(np.int32)
    q = normal_bf16(seed + 1, (n_seqs * q_len, q_heads, head_dim))
    k = normal_bf16(seed + 2, (n_pages, page_size, kv_heads, head_dim))
    v = normal_bf16(seed + 3, (n_pages, page_size, kv_heads, head_dim))
    return q, k, v, table, kv_lens


def moe_group_sizes(rows: int = 32768, groups: int = 8, seed: int = 6001):
    """Rows per expert for a skewed routing: shares drawn from a Dirichlet(1)
    (seeded), rounded to integers that sum to `rows`."""
    share = rng(seed).dirichlet(np.ones(groups))
    sizes = np.floor(share * rows).astype(np.int64)
    sizes[np.argmax(sizes)] += rows - sizes.sum()
    return sizes
