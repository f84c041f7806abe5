// dequant.hip -- x_hat = s_b * q_i [MXFP8 SM120 software support, §0.1]:
// FP8 (or packed E2M1) codes times the block's E8M0 scale, exact in f32,
// written as f32 or as bf16 rounded to nearest even. HBM-bound: each thread
// turns 16 codes (half a block: 16 bytes, or 8 for E2M1) into 64 bytes of f32
// or 32 bytes of bf16.
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

template <int FMT, bool BF16OUT>
__global__ __launch_bounds__(kThreads) void dequant_kernel(const uint8_t* __restrict__ q, int64_t ldq,
                                                           const uint8_t* __restrict__ s, int64_t lds,
                                                           void* __restrict__ y, int64_t ldy, uint32_t nchunks,
                                                           FastDiv per_row) {
  const uint32_t g = blockIdx.x * kThreads + threadIdx.x;
  if (g >= nchunks) return;
  const uint32_t row = per_row.div(g);
  const uint32_t c16 = g - row * per_row.d;
  const uint32_t sc = s[(int64_t)row * lds + c16 / 2];
  // 2^(sc - 127) as an f32; code 0 is the subnormal 2^-127
  const float scale = __uint_as_float(sc ? (sc << 23) : 0x00400000u);
  float v[16];
  if constexpr (FMT == MX_E2M1) {
    // 16 codes are 8 bytes; byte i holds elements 2i (low nibble) and 2i + 1
    const uint2 codes = *(const uint2*)(q + (int64_t)row * ldq + (int64_t)c16 * 8);
    const v2f32 d[8] = {__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes.x, scale, 0),
                        __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes.x, scale, 1),
                        __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes.x, scale, 2),
                        __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes.x, scale, 3),
                        __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes.y, scale, 0),
                        __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes.y, scale, 1),
                        __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes.y, scale, 2),
                        __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes.y, scale, 3)};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      v[2 * i] = d[i][0];
      v[2 * i + 1] = d[i][1];
    }
  } else {
    const uint4 codes = *(const uint4*)(q + (int64_t)row * ldq + (int64_t)c16 * 16);
    const uint32_t w[4] = {codes.x, codes.y, codes.z, codes.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v2f32 lo = decode2<FMT>(w[i], scale, false), hi = decode2<FMT>(w[i], scale, true);
      v[4 * i] = lo[0]; v[4 * i + 1] = lo[1]; v[4 * i + 2] = hi[0]; v[4 * i + 3] = hi[1];
    }
  }
  const bool nan_block = sc == 0xFFu;
#pragma unroll
  for (int i = 0; i < 16; ++i) v[i] = nan_block ? __uint_as_float(0x7FC00000u) : canon_nan(v[i]);
  if constexpr (BF16OUT) {
    uint32_t p[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) p[i] = f32_to_bf16_rne(v[2 * i]) | (f32_to_bf16_rne(v[2 * i + 1]) << 16);
    uint4* dst = (uint4*)((uint16_t*)y + (int64_t)row * ldy + (int64_t)c16 * 16);
    dst[0] = make_uint4(p[0], p[1], p[2], p[3]);
    dst[1] = make_uint4(p[4], p[5], p[6], p[7]);
  } else {
    float4* dst = (float4*)((float*)y + (int64_t)row * ldy + (int64_t)c16 * 16);
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[i] = make_float4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
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
  const int64_t cpr = cols / 16;
  if (cpr >= ((int64_t)1 << 30)) return MX_ERR_SHAPE;
  const FastDiv per_row = FastDiv::make((uint32_t)cpr);
  const int64_t rows_per_launch = std::max<int64_t>(1, ((int64_t)1 << 30) / cpr);
  for (int64_t r0 = 0; r0 < rows; r0 += rows_per_launch) {
    const int64_t nr = std::min(rows_per_launch, rows - r0);
    const uint32_t n = (uint32_t)(nr * cpr);
    const dim3 grid((n + kThreads - 1) / kThreads);
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
