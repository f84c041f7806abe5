// mx_common.hpp -- helpers shared by the libmxfp8 kernels (gfx950 only).
//
// Hardware facts these helpers rely on (established by exhaustive on-device
// checks over every bf16 input pattern and every E8M0 scale):
//  * v_cvt_scalef32_pk_{fp8,bf8}_{bf16,f32} compute RNE(x / scale) exactly,
//    subnormal results and signed zeros included, but do NOT saturate: a
//    magnitude past the largest finite value becomes NaN (E4M3) or Inf
//    (E5M2). fix_overflow_* below turns those bytes into the saturated code.
//  * v_cvt_scalef32_pk_f32_{fp8,bf8} compute code * scale exactly in f32.
//  * v_mfma_scale_f32_16x16x128_f8f6f4 takes, per lane l (row r = l % 16,
//    group g = l / 16), 32 bytes: bytes 0-15 hold k = 16g .. 16g+15 and bytes
//    16-31 hold k = 64+16g .. 64+16g+15 of the 128-wide K slice; the 32-bit
//    scale operand of lane l is the E8M0 scale of (row r, k-block g). The
//    result D[i][j] sits in lane j + 16*(i/4), element i % 4.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mxfp8.h"

namespace mx {

typedef short v2i16 __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf16 __attribute__((ext_vector_type(2)));
typedef float v2f32 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

constexpr int kBlock = 32;  // elements per MX block

// ---------------------------------------------------------------- scales
// E8M0 code from the largest |x| bit pattern of a block, for the rule
// X = 2^(floor(log2 amax) - emax_elem): code = max(E - emax_elem, 0) with E
// the biased exponent field of amax (subnormal and zero amax have E = 0, so
// they clamp to code 0); E = 255 (Inf/NaN present) gives 0xFF.
template <int FMT>
__device__ __forceinline__ uint32_t scale_code_from_exp(uint32_t E) {
  constexpr uint32_t emax = FMT == MX_E5M2 ? 15u : FMT == MX_E2M1 ? 2u : 8u;
  uint32_t c = E > emax ? E - emax : 0u;
  return E == 255u ? 0xFFu : c;
}

// Scale code from the largest |x| bit pattern (MBITS significand bits: 7 for
// bf16, 23 for f32) under either rule. The floor rule is scale_code_from_exp.
// The round-up rule (the smallest power of two X with amax / X <= the largest
// finite element) is one step higher exactly when amax's significand exceeds
// the largest element's: 1.75 for E4M3 and E5M2 (448 = 1.75 * 2^8, 57344 =
// 1.75 * 2^15), 1.5 for E2M1 (6 = 1.5 * 2^2).
template <int FMT, int MBITS>
__device__ __forceinline__ uint32_t scale_code_bits(uint32_t amax_bits, uint32_t round_up) {
  constexpr uint32_t emax = FMT == MX_E5M2 ? 15u : FMT == MX_E2M1 ? 2u : 8u;
  constexpr uint32_t thr = (FMT == MX_E2M1 ? 2u : 3u) << (MBITS - 2);
  const uint32_t E = amax_bits >> MBITS;
  uint32_t code = scale_code_from_exp<FMT>(E);
  if (round_up && E != 255u && (amax_bits & ((1u << MBITS) - 1u)) > thr && E + 1u > emax) code = E + 1u - emax;
  return code;
}

// The divisor 2^(code - 127) as an f32 (code 0 -> the subnormal 2^-127).
__device__ __forceinline__ float scale_divisor(uint32_t code) {
  return __uint_as_float(code ? (code << 23) : 0x00400000u);
}

// ---------------------------------------------------------------- encode
// Saturate the bytes the conversion overflowed: E4M3 NaN (0x7F/0xFF) becomes
// +-448 (0x7E/0xFE); E5M2 Inf (0x7C/0xFC) becomes +-57344 (0x7B/0xFB). Only
// valid for codes of finite inputs (no other byte reaches these patterns).
__device__ __forceinline__ uint32_t fix_overflow_e4m3(uint32_t d) {
  uint32_t t = (d & 0x7F7F7F7Fu) + 0x01010101u;
  return d - ((t >> 7) & 0x01010101u);
}
__device__ __forceinline__ uint32_t fix_overflow_e5m2(uint32_t d) {
  uint32_t t = (d & 0x7F7F7F7Fu) + 0x04040404u;
  return d - ((t >> 7) & 0x01010101u);
}
template <int FMT>
__device__ __forceinline__ uint32_t fix_overflow(uint32_t d) {
  return FMT == MX_E5M2 ? fix_overflow_e5m2(d) : fix_overflow_e4m3(d);
}

// Four bf16 values (two packed words) -> four codes in one dword.
template <int FMT>
__device__ __forceinline__ uint32_t encode4_bf16(uint32_t w01, uint32_t w23, float div) {
  v2i16 r = {0, 0};
  if constexpr (FMT == MX_E5M2) {
    r = __builtin_amdgcn_cvt_scalef32_pk_bf8_bf16(r, __builtin_bit_cast(v2bf16, w01), div, false);
    r = __builtin_amdgcn_cvt_scalef32_pk_bf8_bf16(r, __builtin_bit_cast(v2bf16, w23), div, true);
  } else {
    r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r, __builtin_bit_cast(v2bf16, w01), div, false);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r, __builtin_bit_cast(v2bf16, w23), div, true);
  }
  return fix_overflow<FMT>(__builtin_bit_cast(uint32_t, r));
}

// Four f32 values -> four codes in one dword.
template <int FMT>
__device__ __forceinline__ uint32_t encode4_f32(float a, float b, float c, float d, float div) {
  v2i16 r = {0, 0};
  if constexpr (FMT == MX_E5M2) {
    r = __builtin_amdgcn_cvt_scalef32_pk_bf8_f32(r, a, b, div, false);
    r = __builtin_amdgcn_cvt_scalef32_pk_bf8_f32(r, c, d, div, true);
  } else {
    r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(r, a, b, div, false);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(r, c, d, div, true);
  }
  return fix_overflow<FMT>(__builtin_bit_cast(uint32_t, r));
}

// Eight bf16 / f32 values -> eight E2M1 codes in one dword, element 2i in
// the low nibble of byte i. v_cvt_scalef32_pk_fp4_* round to nearest even and
// saturate at +-6 (checked on the device over every bf16 input), so no fix-up
// is needed; Inf becomes +-6 and NaN 6, which the callers override for NaN
// blocks.
__device__ __forceinline__ uint32_t encode8_fp4_bf16(uint4 w, float div) {
  uint32_t r = 0;
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(v2bf16, w.x), div, 0);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(v2bf16, w.y), div, 1);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(v2bf16, w.z), div, 2);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(v2bf16, w.w), div, 3);
  return r;
}
__device__ __forceinline__ uint32_t encode8_fp4_f32(uint4 a, uint4 b, float div) {
  uint32_t r = 0;
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, __uint_as_float(a.x), __uint_as_float(a.y), div, 0);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, __uint_as_float(a.z), __uint_as_float(a.w), div, 1);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, __uint_as_float(b.x), __uint_as_float(b.y), div, 2);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, __uint_as_float(b.z), __uint_as_float(b.w), div, 3);
  return r;
}

// ---------------------------------------------------------------- reductions
// Packed 16-bit unsigned max of two words (v_pk_max_u16).
__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b) {
  u16x2 r = __builtin_elementwise_max(__builtin_bit_cast(u16x2, a), __builtin_bit_cast(u16x2, b));
  return __builtin_bit_cast(uint32_t, r);
}
__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }

// DPP lane moves inside a row of 16 lanes.
#define MX_DPP_QUAD_XOR1 0xB1   // quad_perm [1,0,3,2]
#define MX_DPP_QUAD_XOR2 0x4E   // quad_perm [2,3,0,1]
#define MX_DPP_HALF_MIRROR 0x141  // reverse within each group of 8 lanes
#define MX_DPP_ROW_MIRROR 0x140   // reverse within each group of 16 lanes
template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, false);
}
// max over the 4 lanes of a quad (32-bit values)
__device__ __forceinline__ uint32_t quad_max_u32(uint32_t v) {
  v = umax(v, dpp<MX_DPP_QUAD_XOR1>(v));
  return umax(v, dpp<MX_DPP_QUAD_XOR2>(v));
}
// packed-u16 max over the 8 lanes of an aligned group of 8
__device__ __forceinline__ uint32_t oct_max_pk_u16(uint32_t v) {
  v = pk_max_u16(v, dpp<MX_DPP_QUAD_XOR1>(v));
  v = pk_max_u16(v, dpp<MX_DPP_QUAD_XOR2>(v));
  return pk_max_u16(v, dpp<MX_DPP_HALF_MIRROR>(v));
}
// packed-u16 max over the 4 lanes of a quad
__device__ __forceinline__ uint32_t quad_max_pk_u16(uint32_t v) {
  v = pk_max_u16(v, dpp<MX_DPP_QUAD_XOR1>(v));
  return pk_max_u16(v, dpp<MX_DPP_QUAD_XOR2>(v));
}
__device__ __forceinline__ uint32_t oct_max_u32(uint32_t v) {
  v = umax(v, dpp<MX_DPP_QUAD_XOR1>(v));
  v = umax(v, dpp<MX_DPP_QUAD_XOR2>(v));
  return umax(v, dpp<MX_DPP_HALF_MIRROR>(v));
}
// max over the 16 lanes of a DPP row
__device__ __forceinline__ uint32_t row16_max_u32(uint32_t v) {
  v = oct_max_u32(v);
  return umax(v, dpp<MX_DPP_ROW_MIRROR>(v));
}

// ---------------------------------------------------------------- division
// n / d for 0 <= n < 2^31 and 1 <= d < 2^31 by multiply-high: for d not a
// power of two, l = ceil(log2 d), m = ceil(2^(31+l) / d) (fits in 32 bits)
// and n / d = mulhi(n, m) >> (l - 1); powers of two use a shift.
struct FastDiv {
  uint32_t d, m, s;  // m == 0 -> shift by s
  __host__ static FastDiv make(uint32_t d) {
    FastDiv f{d, 0, 0};
    uint32_t l = 0;
    while ((1ull << l) < d) ++l;
    if ((1ull << l) == d) {
      f.s = l;
    } else {
      unsigned __int128 num = (unsigned __int128)1 << (31 + l);
      f.m = (uint32_t)((num + d - 1) / d);
      f.s = l - 1;
    }
    return f;
  }
  __device__ __forceinline__ uint32_t div(uint32_t n) const {
    return m ? (__umulhi(n, m) >> s) : (n >> s);
  }
};

// ---------------------------------------------------------------- vectors
typedef int v8i32 __attribute__((ext_vector_type(8)));
typedef float v4f32 __attribute__((ext_vector_type(4)));
typedef float v16f32 __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf16 __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------- decode
// 2^(code - 127) as an f32 multiplier; code 0xFF (NaN scale) gives NaN.
__device__ __forceinline__ float scale_value(uint32_t code) {
  return code == 0xFFu ? __uint_as_float(0x7FC00000u) : __uint_as_float(code ? (code << 23) : 0x00400000u);
}

// Eight codes -> eight bf16 values times the block scale: two dwords of
// FP8 codes, or (E2M1) the eight nibbles of w.x, element 2i in the low
// nibble of byte i.
template <int FMT>
__device__ __forceinline__ v8bf16 decode8_bf16(uint2 w, float scale) {
  v2bf16 r0, r1, r2, r3;
  if constexpr (FMT == MX_E2M1) {
    r0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w.x, scale, 0);
    r1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w.x, scale, 1);
    r2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w.x, scale, 2);
    r3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w.x, scale, 3);
  } else if constexpr (FMT == MX_E5M2) {
    r0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8((int)w.x, scale, false);
    r1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8((int)w.x, scale, true);
    r2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8((int)w.y, scale, false);
    r3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8((int)w.y, scale, true);
  } else {
    r0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w.x, scale, false);
    r1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w.x, scale, true);
    r2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w.y, scale, false);
    r3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w.y, scale, true);
  }
  return v8bf16{r0[0], r0[1], r1[0], r1[1], r2[0], r2[1], r3[0], r3[1]};
}

// ---------------------------------------------------------------- exact scaling
// The FP32-accumulation paths fold a block's E8M0 scale into its bf16
// operands. q * 2^(s - 127) is an exact *normal* bf16 for every finite code q
// exactly when s lies in [fold_lo, fold_hi]: E4M3 values run from 2^-9 to
// 448 = 1.75 * 2^8, so 2^-9 * 2^(s - 127) >= 2^-126 needs s >= 10 and
// 448 * 2^(s - 127) < 2^128 needs s <= 246; E5M2 values run from 2^-16 to
// 1.75 * 2^15, giving [17, 239]; E2M1 values run from 2^-1 to 6 = 1.5 * 2^2,
// giving [2, 252]. The main loops fold every block; the terms
// of blocks outside the window are replaced afterwards by an exact pass
// (below).
template <int FMT>
constexpr uint32_t fold_lo() { return FMT == MX_E5M2 ? 17u : FMT == MX_E2M1 ? 2u : 10u; }
template <int FMT>
constexpr uint32_t fold_hi() { return FMT == MX_E5M2 ? 239u : FMT == MX_E2M1 ? 252u : 246u; }
// The bits of a code word that hold element magnitudes (a zero element of
// either sign has none set): FP8 bytes, or E2M1 nibbles.
template <int FMT>
constexpr uint32_t code_mag_mask() { return FMT == MX_E2M1 ? 0x77777777u : 0x7F7F7F7Fu; }

// A scale outside the fold window, the NaN code 0xFF included: its block's
// terms are replaced by the exact pass. (Rows are left out of a pass by
// zeroing their codes: the scaled conversions read only the exponent field
// of their f32 scale operand, so a scale of 0.0 would act as 2^-127, not as 0.)
template <int FMT>
__device__ __forceinline__ bool fold_excluded(uint32_t s) {
  return s - fold_lo<FMT>() > fold_hi<FMT>() - fold_lo<FMT>();
}
// Non-zero when a block must go through the exact pass: its scale lies
// outside the window and it holds a non-zero code (codes_or: the OR of some
// of its code dwords), or its scale is the NaN code, which makes every
// output it enters NaN whatever its codes.
template <int FMT>
__device__ __forceinline__ uint32_t exact_flag(uint32_t s, uint32_t codes_or) {
  return fold_excluded<FMT>(s) ? (s == 0xFFu ? 1u : codes_or & code_mag_mask<FMT>()) : 0u;
}

// ---- the exact pass over blocks the fold leaves out.
// Scale codes fall in 7 classes: 0 below the fold window, 1 its first codes
// [lo, 33], 2-5 four near-equal parts of [34, hi], 6 above it. A term of a block pairs an A
// row of class x with a B row of class y; the main loop's fold is exact for
// the pairs with x and y in 1..5. The pass takes back the main loop's terms
// of every other pair (two passes of the folded operands, negated) and adds
// their exact values cell by cell: A rows of class x folded with
// 2^(sa - w - 127), B rows of class y with 2^(sb + w - 127), every other
// row's codes zeroed, so each pair lands in exactly one cell and its product
// is unchanged. For every cell some shift w keeps both
// folds inside their windows (checked at compile time below), except cells
// whose terms cannot matter: all of them below 2^-160 (far under any f32
// result they could change), or all of them beyond the f32 range. Rows
// under the NaN code take no cell: the take-back passes give them NaN
// operands, which make their outputs NaN.
template <int FMT>
constexpr int exact_class_start(int c) {  // first code of class c (0..6); 7 -> 255
  return c == 0 ? 0 : c == 1 ? (int)fold_lo<FMT>() : c == 6 ? (int)fold_hi<FMT>() + 1 : c == 7 ? 255
       : 34 + ((c - 2) * ((int)fold_hi<FMT>() + 1 - 34) + 2) / 4;
}
template <int FMT>
__device__ __forceinline__ uint32_t exact_class(uint32_t s) {
  return (uint32_t)(s >= (uint32_t)exact_class_start<FMT>(1)) + (s >= (uint32_t)exact_class_start<FMT>(2)) +
         (s >= (uint32_t)exact_class_start<FMT>(3)) + (s >= (uint32_t)exact_class_start<FMT>(4)) +
         (s >= (uint32_t)exact_class_start<FMT>(5)) + (s >= (uint32_t)exact_class_start<FMT>(6));
}
// log2 bounds of the largest and smallest non-zero element magnitude
template <int FMT>
constexpr int elem_log2_max() { return FMT == MX_E5M2 ? 16 : FMT == MX_E2M1 ? 3 : 9; }
template <int FMT>
constexpr int elem_log2_min() { return FMT == MX_E5M2 ? -16 : FMT == MX_E2M1 ? -1 : -9; }

struct ExactCell { int x, y, w; };
template <int AF, int BF>
struct ExactCells {
  ExactCell cell[49];
  int n;
  constexpr ExactCells() : cell(), n(0) {
    for (int x = 0; x < 7; ++x)
      for (int y = 0; y < 7; ++y) {
        if (x != 0 && x != 6 && y != 0 && y != 6) continue;  // folded by the main loop
        const int a1 = exact_class_start<AF>(x), a2 = exact_class_start<AF>(x + 1) - 1;
        const int b1 = exact_class_start<BF>(y), b2 = exact_class_start<BF>(y + 1) - 1;
        // every term of the cell: |sum of 32 products| * 2^(sa + sb - 254)
        if (5 + elem_log2_max<AF>() + elem_log2_max<BF>() + a2 + b2 - 254 < -160) continue;
        if (elem_log2_min<AF>() + elem_log2_min<BF>() + a1 + b1 - 254 > 128) continue;
        const int wlo = max_i(a2 - (int)fold_hi<AF>(), (int)fold_lo<BF>() - b1);
        const int whi = min_i(a1 - (int)fold_lo<AF>(), (int)fold_hi<BF>() - b2);
        cell[n++] = ExactCell{x, y, wlo <= whi ? (wlo + whi) / 2 : -1000};
      }
  }
  static constexpr int max_i(int a, int b) { return a > b ? a : b; }
  static constexpr int min_i(int a, int b) { return a < b ? a : b; }
  constexpr bool feasible() const {
    for (int i = 0; i < n; ++i)
      if (cell[i].w == -1000) return false;
    return true;
  }
};

// The scale operand the main loops fold a block with: 2^(min(s, hi) - 127)
// as an f32 whose only non-zero field is the exponent (s = 0 gives 0.0,
// which the scaled conversions take as 2^-127). Inside the window the fold
// is exact; outside it (the NaN code included) the block is folded
// inexactly but never enlarged past the window, and the exact pass replaces
// its terms.
template <int FMT>
__device__ __forceinline__ float fold_scale(uint32_t s) {
  return __uint_as_float(min(s, fold_hi<FMT>()) << 23);
}
// Eight codes of one block decoded with fold_scale.
template <int FMT>
__device__ __forceinline__ v8bf16 fold_decode8(uint2 w, uint32_t s) {
  return decode8_bf16<FMT>(w, fold_scale<FMT>(s));
}
// An operand of the exact pass's take-back: the block as the main loop
// folded it when `take`, else zeros (zero codes and a neutral scale); a
// block under the NaN scale code gives NaN.
template <int FMT>
__device__ __forceinline__ v8bf16 exact_operand(uint2 w, uint32_t s, bool take) {
  const v8bf16 v = decode8_bf16<FMT>(take ? w : make_uint2(0u, 0u), take ? fold_scale<FMT>(s) : 1.f);
  const uint4 nan = make_uint4(0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u);
  return take && s == 0xFFu ? __builtin_bit_cast(v8bf16, nan) : v;
}

// Nonzero when some byte of w is below lo (lo <= 128): the borrow of a byte
// that underflows sets its top bit where the byte's own top bit was clear.
__device__ __forceinline__ uint32_t any_byte_below(uint32_t w, uint32_t lo) {
  return (w - lo * 0x01010101u) & ~w & 0x80808080u;
}
// Nonzero when some byte of w lies outside [lo, hi] (lo <= 128, hi >= 127).
__device__ __forceinline__ uint32_t any_byte_outside(uint32_t w, uint32_t lo, uint32_t hi) {
  return any_byte_below(w, lo) | any_byte_below(~w, 255u - hi);
}
// Some of the element codes in the given dwords encode a non-zero value
// (0x00 and 0x80 are the two zeros of E4M3 and E5M2).
__device__ __forceinline__ bool codes_nonzero(uint32_t a, uint32_t b) { return ((a | b) & 0x7F7F7F7Fu) != 0u; }

// ---------------------------------------------------------------- LDS staging
// 16-byte chunk permutation of a 128-byte LDS row: chunk ^ fperm(row) with
// fperm = ((row >> 1) & 7) ^ ((row & 1) << 2). The 16 (or 8) lanes that a
// ds_read_b128 serves together read 16 (8) consecutive rows at one logical
// chunk; fperm gives them distinct bank groups whether the LDS serves 16
// lanes over 64 banks or 8 lanes over 32 banks. It depends only on row bits
// 0-3, so rows 32 apart share it.
__device__ __forceinline__ uint32_t fperm(uint32_t row) { return ((row >> 1) & 7u) ^ ((row & 1u) << 2); }

// LDS byte offset of a __shared__ object (the low half of its flat address).
__device__ __forceinline__ uint32_t lds_off(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Direct global->LDS loads: lane i's 16 (dma16) or 4 (dma4) bytes land at
// M0 + 16i (4i). The address is a wave-uniform base (SGPR pair) plus a
// per-lane 32-bit offset. They are issued as inline assembly so that the
// compiler does not add its own drain of every outstanding load before each
// LDS read; completion is tracked explicitly with wait_vmcnt before the
// barrier that publishes the data. Nothing else in the kernels that use them
// touches M0. An LDS-DMA load that reads M0 right after a scalar write of it
// needs one wait state, which the compiler cannot insert inside the asm:
// hence the s_nop.
__device__ __forceinline__ void dma16(uint32_t lds, uint32_t off, const void* base) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds), "v"(off), "s"(base) : "memory");
}
__device__ __forceinline__ void dma4(uint32_t lds, uint32_t off, const void* base) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2" ::"s"(lds), "v"(off), "s"(base) : "memory");
}
// dma16 with the LDS address given as a wave-uniform base plus an offset
// that folds to a constant at compile time (an unrolled index): M0 is formed
// inside the asm, so the compiler keeps no scalar register per distinct
// address.
__device__ __forceinline__ void dma16_at(uint32_t lds_base, uint32_t imm, uint32_t off, const void* base) {
  asm volatile("s_add_u32 m0, %0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %2, %3" ::"s"(lds_base), "i"(imm), "v"(off),
               "s"(base)
               : "memory", "scc");
}
// A pointer that is the same in every lane, moved to SGPRs once, so that
// the per-stage address arithmetic stays on the scalar unit.
__device__ __forceinline__ const uint8_t* uniform_ptr(const uint8_t* p) {
  const uint64_t b = (uint64_t)p;
  return (const uint8_t*)((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b) |
                          ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32)) << 32));
}
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ void wait_lgkmcnt0() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void barrier() { asm volatile("s_barrier" ::: "memory"); }

// ---------------------------------------------------------------- bf16 out
// f32 -> bf16, round to nearest even; NaN inputs must already be canonical.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ float canon_nan(float f) { return f != f ? __uint_as_float(0x7FC00000u) : f; }

}  // namespace mx

// ---------------------------------------------------------------- host side
namespace mx_host {
mx_status_t check_device();  // MX_OK when the current device is gfx950
int cu_count();              // compute units of the current device (0 if unknown); cached with the check
inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
inline mx_status_t launch_status() {
  return hipGetLastError() == hipSuccess ? MX_OK : MX_ERR_HIP;
}
}  // namespace mx_host
