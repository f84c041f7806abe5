"""Host-side model of how mx_grouped_gemm deals its row tiles (the kernel
scans the group offsets 64 groups at a time with a prefix sum): with any
offsets every tile stays inside [0, total_m); with nondecreasing offsets the
tiles cover every group's rows exactly once within a grid of
ceil(total_m / 256) + groups row tiles."""
import numpy as np

TILE = 256


def decode(off, M, G, t):
    prefix = 0
    for q0 in range(0, G, 64):
        q = np.arange(q0, q0 + 64)
        valid = q < G
        lo = np.where(valid, np.clip(off[np.minimum(q, G - 1)], 0, M), 0)
        hi = np.where(valid, np.clip(off[np.minimum(q + 1, G)], lo, M), 0)
        nt = (hi - lo + TILE - 1) // TILE
        incl = np.cumsum(nt)
        if t < prefix + incl[-1]:
            src = int(np.argmax((t >= prefix + incl - nt) & (t < prefix + incl)))
            return lo[src] + (t - (prefix + incl[src] - nt[src])) * TILE, hi[src]
        prefix += incl[-1]
    return None


def test_grouped_tiles_in_bounds_and_covering():
    rng = np.random.default_rng(0)
    for trial in range(120):
        G, M = int(rng.integers(1, 150)), int(rng.integers(0, 3000))
        wellformed = trial % 2 == 0
        if wellformed:
            off = np.concatenate([[0], np.sort(rng.integers(0, M + 1, G - 1)), [M]]).astype(np.int64)
        else:
            off = rng.integers(-500, M + 500, G + 1).astype(np.int64)
        covered = np.zeros(M, np.int64)
        for t in range((M + TILE - 1) // TILE + G):
            r = decode(off, M, G, t)
            if r is None:
                continue
            m0, m_end = r
            assert 0 <= m0 < m_end <= M
            covered[m0:min(m0 + TILE, m_end)] += 1
        if wellformed:
            assert np.all(covered == 1) or M == 0
