"""Helpers shared by the GPU parity tests (host/device transfer, bounds)."""
import numpy as np

# |y_gpu - y_ref| <= REL_T * sum_k |a_k b_k| per output element (f32 output)
REL_T = 1e-5
# Forced MX_ACCUM_FP8 on small K: the scaled FP8 instruction sums each group
# of 8 products with ~14 significant bits aligned to the group's largest
# product, so each group may lose up to 7 * 2^-13 of its largest product
# (< 2^-10 of the group's sum of magnitudes). Index or layout mistakes give
# errors of order 1 and still fail this bound.
FP8_GROUPED_REL = 2.0 ** -10
# extra term for bf16 output: bf16 keeps 8 significant bits, so rounding an
# f32 result to it moves it by at most 2^-8 of its magnitude
BF16_REL = 2.0 ** -8


def torch_mod():
    import torch
    return torch


def dev(a: np.ndarray, bf16: bool = False):
    """numpy -> cuda tensor. bf16 data is passed as uint16 bit patterns."""
    torch = torch_mod()
    if bf16:
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    elif a.dtype == np.uint16:
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16))
    else:
        t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to("cuda")


def host(t) -> np.ndarray:
    torch = torch_mod()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def assert_bitexact(got: np.ndarray, want: np.ndarray, what: str):
    assert got.shape == want.shape, (what, got.shape, want.shape)
    bad = np.argwhere(got != want)
    assert bad.size == 0, "%s: %d mismatches, first at %s: got %#x want %#x" % (
        what, len(bad), tuple(bad[0]), int(got[tuple(bad[0])]), int(want[tuple(bad[0])]))


def assert_gemm_bound(y: np.ndarray, y_ref: np.ndarray, t_ref: np.ndarray, what: str, bf16_out: bool = False,
                      rel: float = REL_T):
    y = y.astype(np.float64)
    err = np.abs(y - y_ref)
    bound = rel * t_ref
    if bf16_out:
        bound = bound + BF16_REL * (np.abs(y_ref) + rel * t_ref)
    ok = err <= bound
    if not ok.all():
        i = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError("%s: %d of %d outputs outside the bound; worst at %s: gpu %r ref %r |err| %g bound %g "
                             "(err/T %g)" % (what, int((~ok).sum()), ok.size, i, y[i], y_ref[i], err[i], bound[i],
                                             err[i] / max(t_ref[i], 1e-300)))
    return float(np.max(err / np.maximum(t_ref, 1e-300)))


def check_every_output(oracle, outputs, qa, sa, afmt, qb, sb, bfmt, what, chunk_rows=1024):
    """Compare every element of each GPU product in `outputs` -- a list of
    (name, device tensor [M, N] of f32 or bf16, rel) -- with the oracle's
    y = A * B^T, computed row chunk by row chunk so that y_ref and sum|a b|
    never have to be held for the whole output at once. Returns the worst
    |err| / sum|a b| of each output."""
    import torch
    M = qa.shape[0]
    worst = {name: 0.0 for name, _, _ in outputs}
    for r0 in range(0, M, chunk_rows):
        r1 = min(M, r0 + chunk_rows)
        y_ref, t_ref = oracle.gemm(qa[r0:r1], sa[r0:r1], afmt, qb, sb, bfmt)
        for name, y, rel in outputs:
            bf = y.dtype == torch.bfloat16
            yc = host(y[r0:r1])
            yc = bf16_to_f64(yc) if bf else yc.astype(np.float64)
            w = assert_gemm_bound(yc, y_ref, t_ref, "%s %s rows %d-%d" % (what, name, r0, r1), bf16_out=bf, rel=rel)
            worst[name] = max(worst[name], w)
    return worst
