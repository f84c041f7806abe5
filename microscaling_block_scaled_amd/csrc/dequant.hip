// dequant.hip -- x_hat = s_b * q_i [MXFP8 SM120 software support, §0.1]:
// FP8 (or packed E2M1) codes times the block's E8M0 scale, exact in f32,
// written as f32 or as bf16 rounded to nearest even. HBM-bound, and the
// output is most of the traffic, so the kernel is laid out around its stores.
#include "mx_common.hpp"

namespace {
using namespace mx;

constexpr int kThreads = 256;

template <int FMT>
__device__ __forceinline__ v2f32 decode2(uint32_t w, float scale, bool hi) {
  if constexpr (FMT == MX_E5M2)
    return hi ? __builtin_amdgcn_cvt_scalef32_pk_f32_bf8(w, scale, true)
              : __builtin_amdgcn_cvt_scalef32_pk_f32_bf8(w, scale, false);
  else
    return hi ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, scale, true)
              : __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, scale, false);
}

// One piece is E = 16 / sizeof(output) consecutive elements of a row: one
// 16-byte store. Piece g of a launch is piece g % (cols / E) of row
// g / (cols / E). Consecutive lanes take consecutive pieces (a thread's
// pieces are kThreads apart), so every load and store instruction of a wave
// covers one contiguous run: a 16-byte store per lane, and 8, 4 or 2 bytes
// of codes per lane.
// pieces per thread (measured on 8192 x 4096: 4 for bf16 out, 2 for f32 out)
__host__ __device__ constexpr int dq_unroll(bool bf16out) { return bf16out ? 4 : 2; }

template <int FMT, bool BF16OUT>
__global__ __launch_bounds__(kThreads) void dequant_kernel(const uint8_t* __restrict__ q, int64_t ldq,
                                                           const uint8_t* __restrict__ s, int64_t lds,
                                                           void* __restrict__ y, int64_t ldy, uint32_t npieces,
                                                           FastDiv per_row) {
  constexpr int E = BF16OUT ? 8 : 4;                    // elements per piece
  constexpr int kCodeBytes = FMT == MX_E2M1 ? E / 2 : E;  // code bytes per piece
  constexpr int kDqUnroll = dq_unroll(BF16OUT);
  uint32_t w0[kDqUnroll], w1[kDqUnroll], sc[kDqUnroll], row[kDqUnroll], col[kDqUnroll];
  bool ok[kDqUnroll];
#pragma unroll
  for (int u = 0; u < kDqUnroll; ++u) {
    const uint32_t g = blockIdx.x * (kThreads * kDqUnroll) + u * kThreads + threadIdx.x;
    ok[u] = g < npieces;
    row[u] = per_row.div(g);
    col[u] = g - row[u] * per_row.d;
    w0[u] = w1[u] = sc[u] = 0;
    if (!ok[u]) continue;
    const uint8_t* p = q + (int64_t)row[u] * ldq + (int64_t)col[u] * kCodeBytes;
    if constexpr (kCodeBytes == 8) {
      const uint2 t = *(const uint2*)p;
      w0[u] = t.x;
      w1[u] = t.y;
    } else if constexpr (kCodeBytes == 4) {
      w0[u] = *(const uint32_t*)p;
    } else {
      w0[u] = *(const uint16_t*)p;
    }
    sc[u] = s[(int64_t)row[u] * lds + col[u] / (kBlock / E)];
  }
#pragma unroll
  for (int u = 0; u < kDqUnroll; ++u) {
    if (!ok[u]) continue;
    // 2^(sc - 127) as an f32; code 0 is the subnormal 2^-127
    const float scale = __uint_as_float(sc[u] ? (sc[u] << 23) : 0x00400000u);
    float v[E];
    if constexpr (FMT == MX_E2M1) {
      // byte i holds elements 2i (low nibble) and 2i + 1
#pragma unroll
      for (int i = 0; i < E / 2; ++i) {
        const v2f32 d = i == 0 ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w0[u], scale, 0)
                        : i == 1 ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w0[u], scale, 1)
                        : i == 2 ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w0[u], scale, 2)
                                 : __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w0[u], scale, 3);
        v[2 * i] = d[0];
        v[2 * i + 1] = d[1];
      }
    } else {
#pragma unroll
      for (int i = 0; i < E / 4; ++i) {
        const uint32_t w = i == 0 ? w0[u] : w1[u];
        const v2f32 lo = decode2<FMT>(w, scale, false), hi = decode2<FMT>(w, scale, true);
        v[4 * i] = lo[0]; v[4 * i + 1] = lo[1]; v[4 * i + 2] = hi[0]; v[4 * i + 3] = hi[1];
      }
    }
    const bool nan_block = sc[u] == 0xFFu;
#pragma unroll
    for (int i = 0; i < E; ++i) v[i] = nan_block ? __uint_as_float(0x7FC00000u) : canon_nan(v[i]);
    if constexpr (BF16OUT) {
      uint32_t p[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) p[i] = f32_to_bf16_rne(v[2 * i]) | (f32_to_bf16_rne(v[2 * i + 1]) << 16);
      *(uint4*)((uint16_t*)y + (int64_t)row[u] * ldy + (int64_t)col[u] * E) = make_uint4(p[0], p[1], p[2], p[3]);
    } else {
      *(float4*)((float*)y + (int64_t)row[u] * ldy + (int64_t)col[u] * E) = make_float4(v[0], v[1], v[2], v[3]);
    }
  }
}

}  // namespace

extern "C" mx_status_t mx_dequantize(const uint8_t* q, int64_t ldq, const uint8_t* s, int64_t lds, mx_fmt_t fmt,
                                     int64_t rows, int64_t cols, void* y, mx_dtype_t ydt, int64_t ldy,
                                     hipStream_t stream) {
  if (fmt != MX_E4M3 && fmt != MX_E5M2 && fmt != MX_E2M1) return MX_ERR_FORMAT;
  if (ydt != MX_F32 && ydt != MX_BF16) return MX_ERR_FORMAT;
  if (rows == 0 || cols == 0) return rows < 0 || cols < 0 ? MX_ERR_SHAPE : mx_host::check_device();  // empty
  if (!q || !s || !y) return MX_ERR_NULL;
  if (rows < 0 || cols < 0 || cols % kBlock != 0 || ldq < (fmt == MX_E2M1 ? cols / 2 : cols) ||
      lds < cols / kBlock || ldy < cols)
    return MX_ERR_SHAPE;
  const int64_t esz = ydt == MX_F32 ? 4 : 2;
  if (!mx_host::aligned16(q) || ldq % 16 != 0 || !mx_host::aligned16(y) || (ldy * esz) % 16 != 0)
    return MX_ERR_ALIGN;
  mx_status_t st;
  if ((st = mx_host::check_device()) != MX_OK) return st;
  if (rows == 0 || cols == 0) return MX_OK;
  const int64_t cpr = cols / (ydt == MX_BF16 ? 8 : 4);  // pieces per row
  if (cpr >= ((int64_t)1 << 30)) return MX_ERR_SHAPE;
  const FastDiv per_row = FastDiv::make((uint32_t)cpr);
  const int64_t rows_per_launch = std::max<int64_t>(1, ((int64_t)1 << 30) / cpr);
  for (int64_t r0 = 0; r0 < rows; r0 += rows_per_launch) {
    const int64_t nr = std::min(rows_per_launch, rows - r0);
    const uint32_t n = (uint32_t)(nr * cpr);
    const uint32_t per_block = kThreads * dq_unroll(ydt == MX_BF16);
    const dim3 grid((n + per_block - 1) / per_block);
    const uint8_t* qq = q + r0 * ldq;
    const uint8_t* ss = s + r0 * lds;
    void* yy = (uint8_t*)y + r0 * ldy * esz;
    if (fmt == MX_E2M1) {
      if (ydt == MX_BF16)
        hipLaunchKernelGGL((dequant_kernel<MX_E2M1, true>), grid, dim3(kThreads), 0, stream, qq, ldq, ss, lds, yy, ldy, n, per_row);
      else
        hipLaunchKernelGGL((dequant_kernel<MX_E2M1, false>), grid, dim3(kThreads), 0, stream, qq, ldq, ss, lds, yy, ldy, n, per_row);
    } else if (fmt == MX_E5M2) {
      if (ydt == MX_BF16)
        hipLaunchKernelGGL((dequant_kernel<MX_E5M2, true>), grid, dim3(kThreads), 0, stream, qq, ldq, ss, lds, yy, ldy, n, per_row);
      else
        hipLaunchKernelGGL((dequant_kernel<MX_E5M2, false>), grid, dim3(kThreads), 0, stream, qq, ldq, ss, lds, yy, ldy, n, per_row);
    } else {
      if (ydt == MX_BF16)
        hipLaunchKernelGGL((dequant_kernel<MX_E4M3, true>), grid, dim3(kThreads), 0, stream, qq, ldq, ss, lds, yy, ldy, n, per_row);
      else
        hipLaunchKernelGGL((dequant_kernel<MX_E4M3, false>), grid, dim3(kThreads), 0, stream, qq, ldq, ss, lds, yy, ldy, n, per_row);
    }
    if (mx_host::launch_status() != MX_OK) return MX_ERR_HIP;
  }
  return MX_OK;
}
