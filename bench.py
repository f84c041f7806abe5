#!/usr/bin/env python3
"""Benchmark of the MXFP8 hot path on one MI355X (gfx950).

One step = one pass of the metric's workload with inputs resident in HBM:
  1. mx_quantize          bf16 X [8192, 4096] -> E4M3 codes + E8M0 scales (rowwise)
  2. mx_quantize_colwise  the same X, blocks down the columns, stored transposed
  3. mx_gemm              8192 x 8192 x 8192, E4M3 x E4M3 (pre-quantized rowwise
                          along K), FP32 accumulation, bf16 output
Before each kernel a 512 MiB read evicts the caches (L2 and MALL) with clean
lines, outside the kernel's timing: the inputs come from HBM and no write-back
of unrelated data lands in the kernel's time. Kernel durations come from HIP events recorded on the
stream the kernels run on; ms_per_step is wall time per step including the
fills.

`value` is the GEMM's TFLOP/s (2*M*N*K per launch / mean launch time; the
median is printed beside it as gemm_us_median, and us_median per quantizer); the
quantizers' GB/s (algorithmic bytes: read 2RC, write RC + RC/32) are reported
beside it, and the other rows of the path (paged KV write, paged QK^T scores,
dequantize, training linear fwd / dgrad / wgrad) unless --quick. cpu_baseline times
the CPU oracle on a bounded sample of the same GEMM.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--quick]
       [--no-cpu-baseline] [--copy-calibration]
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MXFP8 GEMM TFLOP/s @8192³ + quantize GB/s, each as % of MI355X peak"
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, 8 TB/s
MFMA_FP8_PEAK_TFLOPS = 5000.0   # MI355X dense FP8 / MXFP8 matrix peak
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak
MFMA_FP4_PEAK_TFLOPS = 10100.0  # MI355X dense FP4 / MXFP4 matrix peak
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_gemm_8192_quantize_8192x4096.json")
_CSRC = os.path.join(ROOT, "microscaling_block_scaled_amd", "csrc")
# the sources each measured kernel is built from (its file and the shared header)
GEMM_SOURCE = [os.path.join(_CSRC, "gemm.hip"), os.path.join(_CSRC, "mx_common.hpp")]
QUANT_SOURCE = [os.path.join(_CSRC, "quantize.hip"), os.path.join(_CSRC, "mx_common.hpp")]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class Timer:
    """Accumulates HIP-event durations of kernels launched on one stream.

    The events are created through the HIP runtime with
    hipEventDisableSystemFence: recording them then skips the system-scope
    cache release, which adds ~1-2 us to every recorded interval and would
    distort kernels that run for ~20 us."""

    HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self, torch, stream):
        import ctypes
        self.ct = ctypes
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.torch, self.stream, self.pairs = torch, stream, {}
        self.sp = ctypes.c_void_p(stream.cuda_stream)

    def _event(self):
        e = self.ct.c_void_p()
        if self.hip.hipEventCreateWithFlags(self.ct.byref(e), self.HIP_EVENT_DISABLE_SYSTEM_FENCE) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")
        return e

    def run(self, name, fn, record=True):
        if not record:
            fn()
            return
        e0, e1 = self._event(), self._event()
        if self.hip.hipEventRecord(e0, self.sp) != 0:
            raise RuntimeError("hipEventRecord failed")
        fn()
        if self.hip.hipEventRecord(e1, self.sp) != 0:
            raise RuntimeError("hipEventRecord failed")
        self.pairs.setdefault(name, []).append((e0, e1))

    def times_ms(self, name):
        self.torch.cuda.synchronize()
        ts = []
        for e0, e1 in self.pairs[name]:
            ms = self.ct.c_float()
            if self.hip.hipEventElapsedTime(self.ct.byref(ms), e0, e1) != 0:
                raise RuntimeError("hipEventElapsedTime failed")
            ts.append(ms.value)
        return ts

    def mean_ms(self, name):
        ts = self.times_ms(name)
        return sum(ts) / len(ts)

    def median_ms(self, name):
        ts = sorted(self.times_ms(name))
        n = len(ts)
        return ts[n // 2] if n % 2 else 0.5 * (ts[n // 2 - 1] + ts[n // 2])

    def release(self):
        for pairs in self.pairs.values():
            for e0, e1 in pairs:
                self.hip.hipEventDestroy(e0)
                self.hip.hipEventDestroy(e1)
        self.pairs = {}


def dev_bf16(torch, bits):
    import numpy as np
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def copy_calibration(torch, steps):
    """Plain device copy of a known size, for scaling the HBM byte counters."""
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": {"bytes_read": n, "bytes_written": n, "launches": steps}}))


def _sha256(paths):
    """sha256 over the concatenated bytes of the files, in order."""
    h = hashlib.sha256()
    for path in paths:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def committed_traffic(key, source, sha_field):
    """HBM bytes per launch of one kernel from the committed counter summary,
    or None if that kernel's source changed since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
        if t.get(sha_field) != _sha256(source):
            return None
        return t[key]["bytes_per_launch"]
    except (OSError, KeyError, ValueError):
        return None


def cpu_baseline(xa, xb, xq, budget_s=10.0):
    """The oracle, as it is, on a bounded sample of the 8192^3 GEMM: quantize
    the sampled rows of A and B and compute a square block of outputs over
    the full K; plus the oracle's rowwise quantize of the full 8192 x 4096
    input."""
    import numpy as np
    import oracle
    K = xa.shape[1]

    def run(n):
        qa, sa = oracle.quantize_rows(np.ascontiguousarray(xa[:n]), oracle.E4M3)
        qb, sb = oracle.quantize_rows(np.ascontiguousarray(xb[:n]), oracle.E4M3)
        t0 = time.perf_counter()
        oracle.gemm(qa, sa, oracle.E4M3, qb, sb, oracle.E4M3)
        return time.perf_counter() - t0

    # size the square sample for ~budget_s: a first guess from a tiny run
    # (dominated by start-up), then one correction from a run of that size
    n = 32
    t = run(n)
    n = int(min(8192, max(32, n * (budget_s / 4 / max(t, 1e-3)) ** 0.5)))
    t = run(n)
    if t < budget_s / 2 and n < 8192:
        n = int(min(8192, n * (budget_s / max(t, 1e-3)) ** 0.5))
        t = run(n)
    flop = 2.0 * n * n * K
    t0 = time.perf_counter()
    oracle.quantize_rows(xq, oracle.E4M3)
    tq = time.perf_counter() - t0
    R, C = xq.shape
    qbytes = 2 * R * C + R * C + R * C // 32
    return {"value": round(flop / t / 1e12, 6), "unit": "TFLOP/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": "%d x %d outputs of the 8192^3 product over the full K=%d (%.2f s, fp64); quantize: the "
                      "full 8192 x 4096 input rowwise (%.2f s)" % (n, n, K, t, tq),
            "quantize_GB/s": round(qbytes / tq / 1e9, 3)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--quick", action="store_true", help="only the metric's workload (quantize + 8192^3 GEMM)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--kv-only", action="store_true",
                    help="only the KV-cache rows (write, scores, attention), for profiling them alone")
    ap.add_argument("--quantize-only", action="store_true",
                    help="only the quantize-family kernels on the 8192 x 4096 input, for profiling them alone")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (each rank's work would be the "
              "single-GPU kernel at its full shape); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import microscaling_block_scaled_amd as mx
    from microscaling_block_scaled_amd import inputs

    if args.copy_calibration:
        copy_calibration(torch, args.steps)
        return
    ok, reason = mx.mx_query_support(0)
    if not ok:
        raise SystemExit("libmxfp8 cannot run here: " + reason)
    stream = torch.cuda.current_stream()
    flush_buf = torch.ones((512 << 20) // 4, dtype=torch.float32, device="cuda")

    def flush():
        flush_buf.sum()

    if args.kv_only:
        print(json.dumps({"kv_rows": other_rows(torch, mx, inputs, np, flush, stream, args.steps, kv_only=True)}))
        return
    if args.quantize_only:
        print(json.dumps({"quantize_rows": quantize_rows_only(torch, mx, inputs, flush, stream, args.steps)}))
        return

    # ---- inputs (generated on the host, resident in HBM before timing)
    log("generating inputs")
    xq, _ = inputs.quantize_input()
    xa, xb = inputs.gemm_inputs()
    X = dev_bf16(torch, xq)
    R, C = X.shape
    q = torch.empty((R, C), dtype=torch.uint8, device="cuda")
    s = torch.empty((R, C // 32), dtype=torch.uint8, device="cuda")
    qt = torch.empty((C, R), dtype=torch.uint8, device="cuda")
    st = torch.empty((C, R // 32), dtype=torch.uint8, device="cuda")
    A, SA = mx.mx_quantize(dev_bf16(torch, xa), mx.MX_E4M3)
    B, SB = mx.mx_quantize(dev_bf16(torch, xb), mx.MX_E4M3)
    M, K = A.shape
    N = B.shape[0]
    Y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    torch.cuda.synchronize()

    tm = Timer(torch, stream)

    def step(record):
        flush()
        tm.run("quantize_rowwise", lambda: mx.mx_quantize(X, mx.MX_E4M3, q=q, s=s), record)
        flush()
        tm.run("quantize_colwise", lambda: mx.mx_quantize_colwise(X, mx.MX_E4M3, qt=qt, st=st), record)
        flush()
        tm.run("gemm_8192", lambda: mx.mx_gemm(A, SA, B, SB, y=Y, accum=mx.MX_ACCUM_FP8), record)

    log("warmup")
    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    log("timing %d steps" % args.steps)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    gemm_ms = tm.mean_ms("gemm_8192")
    gemm_tflops = 2.0 * M * N * K / (gemm_ms * 1e-3) / 1e12
    qbytes = 2 * R * C + R * C + R * C // 32
    quant = {}
    for name in ("quantize_rowwise", "quantize_colwise"):
        ms = tm.mean_ms(name)
        gbps = qbytes / (ms * 1e-3) / 1e9
        quant[name] = {"us": round(ms * 1e3, 2), "us_median": round(tm.median_ms(name) * 1e3, 2), "GB/s": round(gbps, 1),
                       "frac_of_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4), "algorithmic_bytes": qbytes}

    result = {
        "metric": METRIC, "value": round(gemm_tflops, 1), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp8",
        "data": "synthetic (seeded N(0,1) bf16, quantized to MXFP8 E4M3 on the GPU)",
        "config": {"workload": "MXFP8 GEMM M=N=K=8192 E4M3 x E4M3, FP32 accumulate, bf16 out; "
                               "quantize bf16 [8192 x 4096] (4 outlier channels x 2^12) to E4M3 rowwise and colwise",
                   "gemm_accumulation": "MX_ACCUM_FP8: scaled FP8 MFMA; every output of this workload is checked "
                                        "within 1e-5 * sum|a b| by the GPU tests"},
        "roofline": {"bound": "mfma", "achieved": round(gemm_tflops, 1), "peak": MFMA_FP8_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(gemm_tflops / MFMA_FP8_PEAK_TFLOPS, 4),
                     "traffic": committed_traffic("gemm_big_kernel (FP8 mode) 8192^3", GEMM_SOURCE, "gemm_source_sha256")},
        "roofline_quantize": {"bound": "hbm", "achieved": quant["quantize_rowwise"]["GB/s"], "peak": HBM_PEAK_GBPS,
                              "unit": "GB/s", "frac": quant["quantize_rowwise"]["frac_of_hbm_peak"],
                              "traffic": committed_traffic("quant_rows_kernel 8192x4096 bf16 E4M3", QUANT_SOURCE,
                                                           "quantize_source_sha256")},
        "gemm_us": round(gemm_ms * 1e3, 2),
        "gemm_us_median": round(tm.median_ms("gemm_8192") * 1e3, 2),
        "quantize": quant,
    }

    if not args.quick:
        result["other_rows"] = other_rows(torch, mx, inputs, np, flush, stream, args.steps)

    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        result["cpu_baseline"] = cpu_baseline(xa, xb, xq)
    print(json.dumps(result))


def quantize_rows_only(torch, mx, inputs, flush, stream, steps):
    """The quantize-family kernels on the quantize input [8192 x 4096] bf16,
    each after a cache-evicting read: rowwise, colwise, both in one pass,
    32 x 32 blocks (both outputs), MXFP4 rowwise, dequantize to bf16."""
    tm = Timer(torch, stream)
    xq, _ = inputs.quantize_input()
    X = dev_bf16(torch, xq)
    R, C = X.shape
    u8 = dict(dtype=torch.uint8, device="cuda")
    q, s = torch.empty((R, C), **u8), torch.empty((R, C // 32), **u8)
    qt, st = torch.empty((C, R), **u8), torch.empty((C, R // 32), **u8)
    q4 = torch.empty((R, C // 2), **u8)
    y = torch.empty((R, C), dtype=torch.bfloat16, device="cuda")
    # a plain device copy moving as many bytes as a quantizer (reads and
    # writes 51 MB): the rate this part sustains on a pure stream
    cn = (3 * R * C + R * C // 32) // 2
    csrc, cdst = torch.empty(cn, **u8), torch.empty(cn, **u8)
    calls = {
        "device_copy_same_bytes": (lambda: cdst.copy_(csrc), 2 * cn),
        "rowwise": (lambda: mx.mx_quantize(X, mx.MX_E4M3, q=q, s=s), 3 * R * C + R * C // 32),
        "colwise": (lambda: mx.mx_quantize_colwise(X, mx.MX_E4M3, qt=qt, st=st), 3 * R * C + R * C // 32),
        "rows_and_cols_one_pass": (lambda: mx.mx_quantize_ex(X, mx.MX_E4M3, colwise=True, q=q, s=s, qt=qt, st=st),
                                   4 * R * C + R * C // 16),
        "blocks_32x32_both": (lambda: mx.mx_quantize_ex(X, mx.MX_E4M3, blocks=mx.MX_BLOCKS_2D, colwise=True, q=q, s=s,
                                                        qt=qt, st=st), 4 * R * C + R * C // 16),
        "mxfp4_rowwise": (lambda: mx.mx_quantize(X, mx.MX_E2M1, q=q4, s=s), 2 * R * C + R * C // 2 + R * C // 32),
        "dequantize_bf16": (lambda: mx.mx_dequantize(q, s, mx.MX_E4M3, y=y), 3 * R * C + R * C // 32),
    }
    out = {}
    for _ in range(3):  # every kernel and the evicting read, three times over, before any is timed
        for fn, _ in calls.values():
            flush()
            fn()
    torch.cuda.synchronize()
    for name, (fn, nbytes) in calls.items():
        for _ in range(max(3, steps)):
            flush()
            tm.run(name, fn)
        torch.cuda.synchronize()
        ms = tm.mean_ms(name)
        out[name] = {"us": round(ms * 1e3, 2), "us_median": round(tm.median_ms(name) * 1e3, 2),
                     "GB/s": round(nbytes / ms / 1e6, 1),
                     "frac_of_hbm_peak": round(nbytes / ms / 1e6 / HBM_PEAK_GBPS, 4), "algorithmic_bytes": nbytes}
    return out


def other_rows(torch, mx, inputs, np, flush, stream, steps, kv_only=False):
    """The remaining rows of the path, each timed like the metric's kernels."""
    out = {}
    tm = Timer(torch, stream)
    reps = max(3, steps // 4)

    def timed(name, fn, n=reps):
        fn()
        torch.cuda.synchronize()
        for _ in range(n):
            flush()
            tm.run(name, fn)
        torch.cuda.synchronize()
        return tm.mean_ms(name)

    # paged KV write + paged QK^T scores (32768 tokens x 8 heads x 128, pages of 128)
    log("kv rows")
    k, v, qv = inputs.kv_inputs()
    slots, table = inputs.kv_layout()
    T, H, D = k.shape
    Kd, Vd = dev_bf16(torch, k), dev_bf16(torch, v)
    slots_d = torch.from_numpy(slots).cuda()
    kc = torch.empty((256, 128, H, D), dtype=torch.uint8, device="cuda")
    ks = torch.empty((256, 128, H, D // 32), dtype=torch.uint8, device="cuda")
    vc, vs = torch.empty_like(kc), torch.empty_like(ks)
    ms = timed("kv_write", lambda: mx.mx_kv_quant_write(Kd, Vd, slots_d, kc, ks, vc, vs))
    kv_bytes = 2 * T * H * D * 2 + T * 8 + 2 * (T * H * D + T * H * D // 32)
    out["kv_quant_write"] = {"us": round(ms * 1e3, 2), "GB/s": round(kv_bytes / ms / 1e6, 1),
                             "frac_of_hbm_peak": round(kv_bytes / ms / 1e6 / HBM_PEAK_GBPS, 4),
                             "algorithmic_bytes": kv_bytes}
    Qc, Qs = mx.mx_quantize(dev_bf16(torch, qv.reshape(-1, D)), mx.MX_E4M3)
    Qc, Qs = Qc.view(T, H, D), Qs.view(T, H, D // 32)
    table_d = torch.from_numpy(table).cuda()
    S = torch.empty((64, H, 512, 512), dtype=torch.float32, device="cuda")
    ms = timed("paged_scores", lambda: mx.mx_paged_scores(Qc, Qs, kc, ks, table_d, 512, out=S))
    sc_bytes = 2 * T * H * (D + D // 32) + 64 * H * 512 * 512 * 4
    sc_flop = 2.0 * 64 * H * 512 * 512 * D
    out["paged_scores"] = {"us": round(ms * 1e3, 2), "GB/s": round(sc_bytes / ms / 1e6, 1),
                           "frac_of_hbm_peak": round(sc_bytes / ms / 1e6 / HBM_PEAK_GBPS, 4),
                           "TFLOP/s": round(sc_flop / ms / 1e9, 1), "algorithmic_bytes": sc_bytes,
                           "accumulation": "AUTO (FP32-accumulation mode, K = 128)"}
    del S
    # paged attention over the same cache: every token's query attends over
    # the 512 keys of its sequence (bf16 out); non-causal, and causal prefill
    lens_d = torch.full((64,), 512, dtype=torch.int32, device="cuda")
    O = torch.empty((T, H, D), dtype=torch.bfloat16, device="cuda")
    at_bytes = 3 * T * H * (D + D // 32) + T * H * D * 2
    for causal in (False, True):
        name = "paged_attention_causal" if causal else "paged_attention"
        ms = timed(name, lambda: mx.mx_paged_attention(Qc, Qs, kc, ks, vc, vs, table_d, lens_d, 512, causal=causal,
                                                       out=O))
        pairs = 64 * H * (512 * 513 // 2 if causal else 512 * 512)
        flop = 4.0 * pairs * D  # QK^T (scaled FP8) and PV (bf16), 2 flops per multiply-add each
        t_mfma = 2.0 * pairs * D / (MFMA_FP8_PEAK_TFLOPS * 1e12) + 2.0 * pairs * D / (MFMA_BF16_PEAK_TFLOPS * 1e12)
        out[name] = {"us": round(ms * 1e3, 2), "TFLOP/s": round(flop / ms / 1e9, 1),
                     "frac_of_mfma_bound": round(t_mfma * 1e3 / ms, 4),
                     "GB/s": round(at_bytes / ms / 1e6, 1), "frac_of_hbm_peak": round(at_bytes / ms / 1e6 / HBM_PEAK_GBPS, 4),
                     "algorithmic_bytes": at_bytes, "flop": flop,
                     "shape": "64 seq x 512 queries x 8 heads x 128, 512 keys, pages of 128, bf16 out"}
    del O, Qc, Qs, Kd, Vd, kc, ks, vc, vs
    if kv_only:
        return out
    # dequantize the 8192 x 4096 codes to bf16
    log("dequant row")
    xq, _ = inputs.quantize_input()
    q, s = mx.mx_quantize(dev_bf16(torch, xq), mx.MX_E4M3)
    yd = torch.empty(q.shape, dtype=torch.bfloat16, device="cuda")
    ms = timed("dequant", lambda: mx.mx_dequantize(q, s, mx.MX_E4M3, y=yd))
    dq_bytes = q.numel() + s.numel() + 2 * q.numel()
    out["dequantize_bf16"] = {"us": round(ms * 1e3, 2), "GB/s": round(dq_bytes / ms / 1e6, 1),
                              "frac_of_hbm_peak": round(dq_bytes / ms / 1e6 / HBM_PEAK_GBPS, 4),
                              "algorithmic_bytes": dq_bytes}
    # the quantize input in both 1-D orientations from one read of x
    Xq2 = dev_bf16(torch, xq)
    q1, s1 = torch.empty_like(q), torch.empty_like(s)
    qt1 = torch.empty((Xq2.shape[1], Xq2.shape[0]), dtype=torch.uint8, device="cuda")
    st1 = torch.empty((Xq2.shape[1], Xq2.shape[0] // 32), dtype=torch.uint8, device="cuda")
    ms = timed("quantize_both", lambda: mx.mx_quantize_ex(Xq2, mx.MX_E4M3, colwise=True, q=q1, s=s1, qt=qt1, st=st1))
    b_bytes = 2 * Xq2.numel() + 2 * (Xq2.numel() + Xq2.numel() // 32)
    out["quantize_rows_and_cols_one_pass"] = {"us": round(ms * 1e3, 2), "GB/s": round(b_bytes / ms / 1e6, 1),
                                              "frac_of_hbm_peak": round(b_bytes / ms / 1e6 / HBM_PEAK_GBPS, 4),
                                              "algorithmic_bytes": b_bytes,
                                              "shape": "the quantize input [8192 x 4096] bf16, E4M3"}
    del Xq2, q1, s1, qt1, st1
    # MXFP4: the quantize input to E2M1 rowwise, and the 8192^3 product of
    # the GEMM workload's inputs quantized to E2M1 (bf16 out)
    log("mxfp4 rows")
    Xq = dev_bf16(torch, xq)
    q4 = torch.empty((Xq.shape[0], Xq.shape[1] // 2), dtype=torch.uint8, device="cuda")
    s4 = torch.empty((Xq.shape[0], Xq.shape[1] // 32), dtype=torch.uint8, device="cuda")
    ms = timed("quantize_mxfp4", lambda: mx.mx_quantize(Xq, mx.MX_E2M1, q=q4, s=s4))
    q4_bytes = 2 * Xq.numel() + Xq.numel() // 2 + Xq.numel() // 32
    out["quantize_mxfp4_rowwise"] = {"us": round(ms * 1e3, 2), "GB/s": round(q4_bytes / ms / 1e6, 1),
                                     "frac_of_hbm_peak": round(q4_bytes / ms / 1e6 / HBM_PEAK_GBPS, 4),
                                     "algorithmic_bytes": q4_bytes}
    del Xq, q4, s4
    xa, xb = inputs.gemm_inputs()
    A4, SA4 = mx.mx_quantize(dev_bf16(torch, xa), mx.MX_E2M1)
    B4, SB4 = mx.mx_quantize(dev_bf16(torch, xb), mx.MX_E2M1)
    del xa, xb
    Y4 = torch.empty((8192, 8192), dtype=torch.bfloat16, device="cuda")
    ms = timed("gemm_mxfp4", lambda: mx.mx_gemm(A4, SA4, B4, SB4, a_fmt=mx.MX_E2M1, b_fmt=mx.MX_E2M1, y=Y4))
    tf = 2.0 * 8192 ** 3 / ms / 1e9
    out["gemm_mxfp4_8192"] = {"us": round(ms * 1e3, 2), "TFLOP/s": round(tf, 1),
                              "frac_of_fp4_peak": round(tf / MFMA_FP4_PEAK_TFLOPS, 4),
                              "shape": [8192, 8192, 8192], "operands": "E2M1 x E2M1, bf16 out"}
    del A4, SA4, B4, SB4, Y4
    # MoE grouped GEMM: 32768 routed rows (16384 tokens x top-2) over 8
    # experts, hidden 4096 -> 4096, E4M3 x E4M3, bf16 out
    log("moe grouped row")
    sizes = inputs.moe_group_sizes(32768, 8)
    off = torch.from_numpy(np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)).cuda()
    Xm, SXm = mx.mx_quantize(dev_bf16(torch, inputs.normal_bf16(6002, (32768, 4096))), mx.MX_E4M3)
    Wm, SWm = mx.mx_quantize(dev_bf16(torch, inputs.normal_bf16(6003, (8 * 4096, 4096), sigma=0.02)), mx.MX_E4M3)
    Ym = torch.empty((32768, 4096), dtype=torch.bfloat16, device="cuda")
    ms = timed("moe_grouped", lambda: mx.mx_grouped_gemm(Xm, SXm, Wm.view(8, 4096, 4096), SWm.view(8, 4096, 128), off,
                                                         y=Ym, accum=mx.MX_ACCUM_FP8))
    tf = 2.0 * 32768 * 4096 * 4096 / ms / 1e9
    out["moe_grouped_gemm"] = {"us": round(ms * 1e3, 2), "TFLOP/s": round(tf, 1),
                               "frac_of_fp8_peak": round(tf / MFMA_FP8_PEAK_TFLOPS, 4),
                               "groups": [int(v) for v in sizes], "shape": "32768 rows x 4096 -> 4096, 8 experts",
                               "accumulation": "MX_ACCUM_FP8 (scaled FP8 MFMA, E4M3 x E4M3, K = 4096)"}
    del Xm, SXm, Wm, SWm, Ym, off
    del q, s, yd
    # training linear layer: fwd (E4M3 x E4M3, K = 4096) and dgrad (E5M2 x E4M3, K = 14336)
    log("training rows")
    x, w, g = inputs.training_inputs()
    Xd, Wd, Gd = dev_bf16(torch, x), dev_bf16(torch, w), dev_bf16(torch, g)
    del x, w, g
    M, Kf = Xd.shape
    N = Wd.shape[0]
    qg = torch.empty(Gd.shape, dtype=torch.uint8, device="cuda")
    sg = torch.empty((Gd.shape[0], Gd.shape[1] // 32), dtype=torch.uint8, device="cuda")
    ms = timed("quantize_G_e5m2", lambda: mx.mx_quantize(Gd, mx.MX_E5M2, q=qg, s=sg))
    g_bytes = 3 * Gd.numel() + Gd.numel() // 32
    out["quantize_G_e5m2_rowwise"] = {"us": round(ms * 1e3, 2), "GB/s": round(g_bytes / ms / 1e6, 1),
                                      "frac_of_hbm_peak": round(g_bytes / ms / 1e6 / HBM_PEAK_GBPS, 4),
                                      "algorithmic_bytes": g_bytes}
    qwt = torch.empty((Wd.shape[1], Wd.shape[0]), dtype=torch.uint8, device="cuda")
    swt = torch.empty((Wd.shape[1], Wd.shape[0] // 32), dtype=torch.uint8, device="cuda")
    ms = timed("quantize_W_colwise", lambda: mx.mx_quantize_colwise(Wd, mx.MX_E4M3, qt=qwt, st=swt))
    w_bytes = 3 * Wd.numel() + Wd.numel() // 32
    out["quantize_W_colwise"] = {"us": round(ms * 1e3, 2), "GB/s": round(w_bytes / ms / 1e6, 1),
                                 "frac_of_hbm_peak": round(w_bytes / ms / 1e6 / HBM_PEAK_GBPS, 4),
                                 "algorithmic_bytes": w_bytes}
    # scale variants on the same weight: 32 x 32 blocks with the round-up
    # rule, both orientations in one pass
    qw2 = torch.empty(Wd.shape, dtype=torch.uint8, device="cuda")
    sw2 = torch.empty((Wd.shape[0], Wd.shape[1] // 32), dtype=torch.uint8, device="cuda")
    qwt2, swt2 = torch.empty_like(qwt), torch.empty_like(swt)
    ms = timed("quantize_W_2d", lambda: mx.mx_quantize_ex(Wd, mx.MX_E4M3, rule=mx.MX_SCALE_CEIL,
                                                          blocks=mx.MX_BLOCKS_2D, colwise=True, q=qw2, s=sw2,
                                                          qt=qwt2, st=swt2))
    w2_bytes = 4 * Wd.numel() + Wd.numel() // 16
    out["quantize_W_2d_both"] = {"us": round(ms * 1e3, 2), "GB/s": round(w2_bytes / ms / 1e6, 1),
                                 "frac_of_hbm_peak": round(w2_bytes / ms / 1e6 / HBM_PEAK_GBPS, 4),
                                 "algorithmic_bytes": w2_bytes, "rule": "round-up, 32x32 blocks"}
    del qw2, sw2, qwt2, swt2
    # FP32 power-of-two scales of 1 x 128 blocks of G -> E8M0 per 32
    sb_rows, sb_cols = Gd.shape
    s128 = torch.ones((sb_rows, sb_cols // 128), dtype=torch.float32, device="cuda")
    sg8 = torch.empty_like(sg)
    ms = timed("scale_broadcast", lambda: mx.mx_scale_broadcast(s128, sb_rows, sb_cols, out=sg8))
    sb_bytes = 4 * s128.numel() + sg8.numel()
    out["scale_broadcast_1x128"] = {"us": round(ms * 1e3, 2), "GB/s": round(sb_bytes / ms / 1e6, 1),
                                    "frac_of_hbm_peak": round(sb_bytes / ms / 1e6 / HBM_PEAK_GBPS, 4),
                                    "algorithmic_bytes": sb_bytes}
    del s128, sg8
    # X [16384 x 4096] quantized in both 1-D orientations from one read
    # (forward operand and wgrad operand of the same activation)
    qxr = torch.empty(Xd.shape, dtype=torch.uint8, device="cuda")
    sxr = torch.empty((Xd.shape[0], Xd.shape[1] // 32), dtype=torch.uint8, device="cuda")
    qxc = torch.empty((Xd.shape[1], Xd.shape[0]), dtype=torch.uint8, device="cuda")
    sxc = torch.empty((Xd.shape[1], Xd.shape[0] // 32), dtype=torch.uint8, device="cuda")
    ms = timed("quantize_X_both", lambda: mx.mx_quantize_ex(Xd, mx.MX_E4M3, colwise=True, q=qxr, s=sxr, qt=qxc, st=sxc))
    xb_bytes = 2 * Xd.numel() + 2 * (Xd.numel() + Xd.numel() // 32)
    ms_r = timed("quantize_X_rows", lambda: mx.mx_quantize(Xd, mx.MX_E4M3, q=qxr, s=sxr))
    ms_c = timed("quantize_X_cols", lambda: mx.mx_quantize_colwise(Xd, mx.MX_E4M3, qt=qxc, st=sxc))
    out["quantize_X_rows_and_cols_one_pass"] = {"us": round(ms * 1e3, 2), "GB/s": round(xb_bytes / ms / 1e6, 1),
                                                "frac_of_hbm_peak": round(xb_bytes / ms / 1e6 / HBM_PEAK_GBPS, 4),
                                                "algorithmic_bytes": xb_bytes,
                                                "two_calls_us": round((ms_r + ms_c) * 1e3, 2)}
    del qxr, sxr, qxc, sxc
    qx, sx = mx.mx_quantize(Xd, mx.MX_E4M3)
    qw, sw = mx.mx_quantize(Wd, mx.MX_E4M3)
    Yf = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    ms = timed("fwd", lambda: mx.mx_gemm(qx, sx, qw, sw, y=Yf, accum=mx.MX_ACCUM_FP8))
    flop = 2.0 * M * N * Kf
    out["training_fwd"] = {"us": round(ms * 1e3, 2), "TFLOP/s": round(flop / ms / 1e9, 1),
                           "frac_of_fp8_peak": round(flop / ms / 1e9 / MFMA_FP8_PEAK_TFLOPS, 4),
                           "shape": [M, N, Kf], "accumulation": "MX_ACCUM_FP8 (scaled FP8 MFMA)"}
    del Yf
    dX = torch.empty((M, Kf), dtype=torch.bfloat16, device="cuda")
    ms = timed("dgrad", lambda: mx.mx_gemm(qg, sg, qwt, swt, mx.MX_E5M2, mx.MX_E4M3, y=dX))
    out["training_dgrad"] = {"us": round(ms * 1e3, 2), "TFLOP/s": round(flop / ms / 1e9, 1),
                             "frac_of_bf16_peak": round(flop / ms / 1e9 / MFMA_BF16_PEAK_TFLOPS, 4),
                             "frac_of_fp8_peak": round(flop / ms / 1e9 / MFMA_FP8_PEAK_TFLOPS, 4),
                             "shape": [M, Kf, N], "accumulation": "AUTO (FP32-accumulation mode: bf16 MFMA on decoded codes)"}
    del dX, qwt, swt, qx, sx, qw, sw
    # wgrad dW = G^T X: both quantized colwise (blocks along the 16384 tokens)
    qgt = torch.empty((Gd.shape[1], Gd.shape[0]), dtype=torch.uint8, device="cuda")
    sgt = torch.empty((Gd.shape[1], Gd.shape[0] // 32), dtype=torch.uint8, device="cuda")
    qxt = torch.empty((Xd.shape[1], Xd.shape[0]), dtype=torch.uint8, device="cuda")
    sxt = torch.empty((Xd.shape[1], Xd.shape[0] // 32), dtype=torch.uint8, device="cuda")
    ms = timed("quantize_G_colwise", lambda: mx.mx_quantize_colwise(Gd, mx.MX_E5M2, qt=qgt, st=sgt))
    out["quantize_G_e5m2_colwise"] = {"us": round(ms * 1e3, 2), "GB/s": round(g_bytes / ms / 1e6, 1),
                                      "frac_of_hbm_peak": round(g_bytes / ms / 1e6 / HBM_PEAK_GBPS, 4),
                                      "algorithmic_bytes": g_bytes}
    mx.mx_quantize_colwise(Xd, mx.MX_E4M3, qt=qxt, st=sxt)
    dW = torch.empty((N, Kf), dtype=torch.bfloat16, device="cuda")
    ms = timed("wgrad", lambda: mx.mx_gemm(qgt, sgt, qxt, sxt, mx.MX_E5M2, mx.MX_E4M3, y=dW))
    out["training_wgrad"] = {"us": round(ms * 1e3, 2), "TFLOP/s": round(flop / ms / 1e9, 1),
                             "frac_of_bf16_peak": round(flop / ms / 1e9 / MFMA_BF16_PEAK_TFLOPS, 4),
                             "shape": [N, Kf, M], "accumulation": "AUTO (FP32-accumulation mode: bf16 MFMA on decoded codes)"}
    return out


if __name__ == "__main__":
    main()
