// gemm.hip -- block-scaled matrix product on gfx950 scaled-FP8 MFMA.
//
//   y[m][n] = sum_b sa[m][b] * sb[n][b] * sum_{i<32} a[m][32b+i] * b[n][32b+i]
//
// [MXFP8 SM120 software support, §0.3; NVFP4 如何用 4 bit 实现高精度, §7.1,
// §7.4]: every 32-element block carries its own pair of scales, so the scales
// cannot be pulled out of the whole sum; the matrix instruction applies them
// per block inside the multiply-accumulate. On gfx950 that instruction is
// v_mfma_scale_f32_16x16x128_f8f6f4: 128 K per issue = 4 blocks, with each
// lane supplying the E8M0 scale of one (row, block) pair; accumulation is
// FP32.
//
// Tiling: a workgroup of 4 waves computes a BM x BN tile; the waves form a
// 2 x 2 grid of (BM/2) x (BN/2) sub-tiles built from 16 x 16 MFMA tiles.
// K advances 128 bytes (4 blocks) per step through a double-buffered LDS
// stage. The MFMA's first operand is the B fragment and its second the A
// fragment, so each lane ends up owning 4 consecutive output columns of one
// row and the epilogue stores 8 (bf16) or 16 (f32) contiguous bytes.
// LDS rows are 128 bytes; their 16-byte chunks are XOR-swizzled by row so
// that the fragment reads (16 rows at one K offset) hit distinct banks.
//
// Two accumulation modes share the staging:
//  * kModeFP8: one v_mfma_scale_f32_16x16x128_f8f6f4 per 128 K on the raw
//    codes. Inside the instruction each group of 8 consecutive k is summed
//    with only ~14 significant bits aligned to the group's largest product.
//  * kModeBF16: per 32-K block, the codes are decoded to bf16 with the block
//    scale folded in (v_cvt_scalef32_pk_bf16_{fp8,bf8}; exact for the scale
//    range the quantizer produces), then v_mfma_f32_16x16x32_bf16, whose
//    accumulation is FP32-level. Half the peak rate.
#include "mx_common.hpp"

namespace {
using namespace mx;


constexpr int kModeFP8 = 0;
constexpr int kModeBF16 = 1;
constexpr int kModeFP4 = 2;  // both operands E2M1 (MXFP4), large-tile kernel only
constexpr int kMfmaFP4 = 4;  // the f8f6f4 instructions' format code for E2M1
// an element format's code for the f8f6f4 instructions (E4M3 0, E5M2 1, E2M1 4)
template <int FMT>
constexpr int mfma_fmt() { return FMT == MX_E2M1 ? kMfmaFP4 : FMT; }

constexpr int kThreads = 256;
constexpr int kBK = 128;  // K bytes per step = 4 MX blocks

struct GemmArgs {
  int64_t M, N, K;
  const uint8_t* a; int64_t lda; const uint8_t* sa; int64_t ldsa;
  const uint8_t* b; int64_t ldb; const uint8_t* sb; int64_t ldsb;
  void* y; int64_t ldy;
  int64_t batch_inner;
  int64_t sa_o, sa_i, ssa_o, ssa_i, sb_o, sb_i, ssb_o, ssb_i, sy_o, sy_i;
  const int32_t* page_table; int64_t pages_per_seq, page_rows, page_stride, page_stride_s;
  FastDiv page_div;  // row -> (page, offset) for row indices below 2^30 (the row-panel kernel's)
  uint32_t tiles_m, tiles_n;
  uint32_t scales_dword;  // 1: every row's 4 scale bytes of a K step can be read as one aligned dword
  uint32_t y_vec;         // 1: output rows allow 8/16-byte vector stores
  // grouped mode (large-tile kernel): group q owns rows [off[q], off[q+1])
  // of A and y and uses B + q * sb_o; row tiles are dealt group by group
  const int64_t* group_off; uint32_t groups;
};

__device__ __forceinline__ uint32_t swz(uint32_t row, uint32_t chunk) {
  return row * kBK + (((chunk ^ row) & 7u) << 4);
}

// Four E8M0 scale bytes (blocks 4kt .. 4kt+3) of one operand row; blocks
// past K read as 127 (scale 1.0) so the zero codes there contribute 0.
__device__ __forceinline__ uint32_t load_scales4(const uint8_t* p, int64_t kt, int64_t kblocks, bool dword_ok) {
  const int64_t b0 = 4 * kt;
  if (dword_ok && b0 + 4 <= kblocks) return *(const uint32_t*)(p + b0);
  uint32_t v = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) v |= (b0 + j < kblocks ? (uint32_t)p[b0 + j] : 127u) << (8 * j);
  return v;
}

// FP32-accumulation mode: the per-lane record of a block that needs the
// exact pass (exact_flag); the terms of such blocks are replaced after the
// main loop (exact_block16 / the large-tile kernel's pass).
template <int FMT>
__device__ __forceinline__ uint32_t unfolded_codes(uint32_t scale, uint2 w) {
  return exact_flag<FMT>(scale, w.x | w.y);
}

// -v, elementwise (sign bits flipped; exact)
__device__ __forceinline__ v8bf16 neg_bf16x8(v8bf16 v) {
  uint4 u = __builtin_bit_cast(uint4, v);
  u.x ^= 0x80008000u; u.y ^= 0x80008000u; u.z ^= 0x80008000u; u.w ^= 0x80008000u;
  return __builtin_bit_cast(v8bf16, u);
}

// The exact pass for one 32-K block of a wave's 4 x 4 tiles of 16 x 16
// outputs (v_mfma_f32_16x16x32_bf16: lane (r, g) supplies row r of a fragment
// and k = 8 g .. 8 g + 7 of the block; its outputs lie on its A row and on B
// rows 4 g .. 4 g + 3 of a tile). qa / ca: the lane's codes and scale of A
// row tile i; qb / cb: those of B row tile j. The terms of pairs with an A
// or B scale outside the fold window are replaced: the main loop's folded
// terms are taken back and the exact ones added cell by cell (ExactCells).
template <int AF, int BF>
__device__ __forceinline__ void exact_block16(const uint2 (&qa)[4], const uint32_t (&ca)[4], const uint2 (&qb)[4],
                                              const uint32_t (&cb)[4], v4f32 (&acc)[4][4]) {
  constexpr ExactCells<AF, BF> cells{};
  static_assert(cells.feasible(), "a cell of the exact pass has no common shift");
  uint32_t nz = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) nz |= unfolded_codes<AF>(ca[i], qa[i]) | unfolded_codes<BF>(cb[i], qb[i]);
  if (__builtin_amdgcn_ballot_w64(nz != 0u) == 0) return;
  // take back the main loop's (folded) terms of the pairs the fold does not
  // cover: R1 = left-out A rows x every B row, R2 = the other A rows x
  // left-out B rows
  bool exa[4], exb[4];
  v8bf16 b_all[4], b_ex[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    exa[i] = fold_excluded<AF>(ca[i]);
    exb[i] = fold_excluded<BF>(cb[i]);
    b_all[i] = exact_operand<BF>(qb[i], cb[i], true);
    b_ex[i] = exact_operand<BF>(qb[i], cb[i], exb[i]);
  }
  const bool any_exb = __builtin_amdgcn_ballot_w64(exb[0] || exb[1] || exb[2] || exb[3]) != 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (__builtin_amdgcn_ballot_w64(exa[i]) != 0) {
      const v8bf16 a1 = neg_bf16x8(exact_operand<AF>(qa[i], ca[i], exa[i]));
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b_all[j], a1, acc[i][j], 0, 0, 0);
    }
    if (any_exb) {
      const v8bf16 a2 = neg_bf16x8(exact_operand<AF>(qa[i], ca[i], !exa[i]));
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b_ex[j], a2, acc[i][j], 0, 0, 0);
    }
  }
  // and add their exact values, cell by cell
  uint32_t xa[4], xb[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    xa[i] = exact_class<AF>(ca[i]);
    xb[i] = exact_class<BF>(cb[i]);
  }
  for (int c = 0; c < cells.n; ++c) {
    const int cx = cells.cell[c].x, cy = cells.cell[c].y, w = cells.cell[c].w;
    v8bf16 bf[4];
    bool bon[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bool in = xb[j] == (uint32_t)cy && cb[j] != 0xFFu;
      bon[j] = __builtin_amdgcn_ballot_w64(in) != 0;
      // rows outside the cell: zero codes and a neutral scale (their shifted
      // code could reach the NaN exponent)
      bf[j] = decode8_bf16<BF>(in ? qb[j] : make_uint2(0u, 0u), in ? __uint_as_float((uint32_t)((int)cb[j] + w) << 23) : 1.f);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool in = xa[i] == (uint32_t)cx && ca[i] != 0xFFu;
      if (__builtin_amdgcn_ballot_w64(in) == 0) continue;
      const v8bf16 af = decode8_bf16<AF>(in ? qa[i] : make_uint2(0u, 0u), in ? __uint_as_float((uint32_t)((int)ca[i] - w) << 23) : 1.f);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (bon[j]) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf[j], af, acc[i][j], 0, 0, 0);
    }
  }
}

template <int BM, int BN, int AFMT, int BFMT, bool BF16OUT, bool PAGED, int MODE>
__global__ __launch_bounds__(kThreads) void gemm_kernel(GemmArgs g) {
  constexpr int WM = BM / 2, WN = BN / 2;   // wave sub-tile
  constexpr int FM = WM / 16, FN = WN / 16; // MFMA tiles per wave
  constexpr int CA = BM * 8 / kThreads;     // 16-byte A chunks per thread per step
  constexpr int CB = BN * 8 / kThreads;
  static_assert(CA >= 1 && CB >= 1, "tile too small");

  __shared__ __attribute__((aligned(16))) uint8_t As[2][BM * kBK];
  __shared__ __attribute__((aligned(16))) uint8_t Bs[2][BN * kBK];
  __shared__ uint32_t sAs[2][BM];
  __shared__ uint32_t sBs[2][BN];

  // ---- which tile: groups of 8 tile rows, walked column-major inside a group
  const uint32_t pid = blockIdx.x;
  const uint32_t group_size = 8;
  const uint32_t per_group = group_size * g.tiles_n;
  const uint32_t first_m = (pid / per_group) * group_size;
  const uint32_t gm = min(g.tiles_m - first_m, group_size);
  const uint32_t tile_m = first_m + (pid % per_group) % gm;
  const uint32_t tile_n = (pid % per_group) / gm;
  const int64_t m0 = (int64_t)tile_m * BM, n0 = (int64_t)tile_n * BN;

  // ---- which problem of the batch
  const int64_t p = blockIdx.y;
  const int64_t po = p / g.batch_inner, pi = p % g.batch_inner;
  const uint8_t* A = g.a + po * g.sa_o + pi * g.sa_i;
  const uint8_t* SA = g.sa + po * g.ssa_o + pi * g.ssa_i;
  const uint8_t* B = g.b + pi * g.sb_i;
  const uint8_t* SB = g.sb + pi * g.ssb_i;
  if (!PAGED) {
    B += po * g.sb_o;
    SB += po * g.ssb_o;
  }

  const int tid = threadIdx.x;
  const int64_t kblocks = g.K / kBlock;
  const int64_t ksteps = (g.K + kBK - 1) / kBK;
  const bool dword_ok = g.scales_dword != 0;

  // ---- per-thread global row pointers (fixed for the whole K loop)
  const uint8_t* a_row[CA];
  const uint8_t* b_row[CB];
  uint32_t a_lds[CA], b_lds[CB], a_ch[CA], b_ch[CB];
#pragma unroll
  for (int i = 0; i < CA; ++i) {
    const uint32_t id = tid + kThreads * i, row = id >> 3, ch = id & 7;
    a_row[i] = (m0 + row < g.M) ? A + (m0 + row) * g.lda : nullptr;
    a_lds[i] = swz(row, ch);
    a_ch[i] = ch;
  }
  auto b_row_ptr = [&](int64_t n, const uint8_t* base, int64_t ld, int64_t pstride) -> const uint8_t* {
    if (PAGED) {
      const int32_t page = g.page_table[po * g.pages_per_seq + n / g.page_rows];
      return base + (int64_t)page * pstride + (n % g.page_rows) * ld;
    }
    return base + n * ld;
  };
#pragma unroll
  for (int i = 0; i < CB; ++i) {
    const uint32_t id = tid + kThreads * i, row = id >> 3, ch = id & 7;
    b_row[i] = (n0 + row < g.N) ? b_row_ptr(n0 + row, B, g.ldb, g.page_stride) : nullptr;
    b_lds[i] = swz(row, ch);
    b_ch[i] = ch;
  }
  // scale rows: thread t serves A row t (t < BM) and B row t (t < BN)
  const uint8_t* sa_row = (tid < BM && m0 + tid < g.M) ? SA + (m0 + tid) * g.ldsa : nullptr;
  const uint8_t* sb_row = (tid < BN && n0 + tid < g.N) ? b_row_ptr(n0 + tid, SB, g.ldsb, g.page_stride_s) : nullptr;

  uint4 ra[CA], rb[CB];
  uint32_t rsa = 0, rsb = 0;
  // A step covers kBK = 128 elements (4 blocks). An FP8 operand row gives
  // them as 8 chunks of 16 bytes; an E2M1 one (two codes per byte) as
  // chunks 0-3, one block each, and leaves chunks 4-7 unused.
  auto load_chunk = [&](const uint8_t* row, int64_t kt, uint32_t ch, bool half) -> uint4 {
    const int64_t e0 = kt * kBK + ch * (half ? 32 : 16);  // first element of the chunk
    const int64_t off = half ? kt * (kBK / 2) + ch * 16 : e0;
    return (row && (!half || ch < 4) && e0 < g.K) ? *(const uint4*)(row + off) : make_uint4(0, 0, 0, 0);
  };
  auto load_global = [&](int64_t kt) {
#pragma unroll
    for (int i = 0; i < CA; ++i) ra[i] = load_chunk(a_row[i], kt, a_ch[i], AFMT == MX_E2M1);
#pragma unroll
    for (int i = 0; i < CB; ++i) rb[i] = load_chunk(b_row[i], kt, b_ch[i], BFMT == MX_E2M1);
    rsa = sa_row ? load_scales4(sa_row, kt, kblocks, dword_ok) : 0x7F7F7F7Fu;
    rsb = sb_row ? load_scales4(sb_row, kt, kblocks, dword_ok) : 0x7F7F7F7Fu;
  };
  auto store_lds = [&](int buf) {
#pragma unroll
    for (int i = 0; i < CA; ++i) *(uint4*)(&As[buf][a_lds[i]]) = ra[i];
#pragma unroll
    for (int i = 0; i < CB; ++i) *(uint4*)(&Bs[buf][b_lds[i]]) = rb[i];
    if (tid < BM) sAs[buf][tid] = rsa;
    if (tid < BN) sBs[buf][tid] = rsb;
  };

  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const uint32_t lr = lane & 15, lg = lane >> 4;

  v4f32 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = v4f32{0.f, 0.f, 0.f, 0.f};

  // FP32-accumulation mode: nonzero once a decoded block with a scale
  // outside the fold window held a non-zero code (exact pass below)
  uint32_t unfolded = 0;

  load_global(0);
  store_lds(0);
  __syncthreads();

  for (int64_t kt = 0; kt < ksteps; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < ksteps) load_global(kt + 1);

    if constexpr (MODE == kModeFP8) {
      // Lane (r, g) supplies the scale of block g of its row. FP8 operand:
      // k = 16g .. 16g+15 and 64+16g .. +15 (chunks g and g+4); E2M1
      // operand: block g whole (chunk g, four of the eight registers).
      auto frag = [&](const uint8_t* base, uint32_t row, bool half) -> v8i32 {
        const uint4 lo = *(const uint4*)(base + swz(row, lg));
        if (half) return v8i32{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, 0, 0, 0, 0};
        const uint4 hi = *(const uint4*)(base + swz(row, lg + 4));
        return v8i32{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      };
      v8i32 bf[FN];
      int bsc[FN];
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const uint32_t row = wn * WN + j * 16 + lr;
        bf[j] = frag(&Bs[buf][0], row, BFMT == MX_E2M1);
        bsc[j] = (int)(sBs[buf][row] >> (8 * lg));
      }
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const uint32_t row = wm * WM + i * 16 + lr;
        const v8i32 af = frag(&As[buf][0], row, AFMT == MX_E2M1);
        const int asc = (int)(sAs[buf][row] >> (8 * lg));
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf[j], af, acc[i][j], mfma_fmt<BFMT>(),
                                                                       mfma_fmt<AFMT>(), 0, bsc[j], 0, asc);
      }
    } else {
      // one 32-K block per MFMA: lane (r, g) takes k = 32*kb + 8g .. +7, i.e.
      // bytes 8*(g & 1) .. +7 of 16-byte chunk 2*kb + g/2 of its row (E2M1:
      // bytes 4g .. 4g+3 of chunk kb, the upper word zero)
      auto codes8 = [&](const uint8_t* base, uint32_t row, int kb, bool half) -> uint2 {
        if (half) return make_uint2(*(const uint32_t*)(base + swz(row, kb) + 4 * lg), 0u);
        return *(const uint2*)(base + swz(row, 2 * kb + (lg >> 1)) + 8 * (lg & 1));
      };
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        v8bf16 bf[FN];
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const uint32_t row = wn * WN + j * 16 + lr;
          const uint2 w = codes8(&Bs[buf][0], row, kb, BFMT == MX_E2M1);
          const uint32_t sc = (sBs[buf][row] >> (8 * kb)) & 0xFFu;
          unfolded |= unfolded_codes<BFMT>(sc, w);
          bf[j] = fold_decode8<BFMT>(w, sc);
        }
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          const uint32_t row = wm * WM + i * 16 + lr;
          const uint2 w = codes8(&As[buf][0], row, kb, AFMT == MX_E2M1);
          const uint32_t sc = (sAs[buf][row] >> (8 * kb)) & 0xFFu;
          unfolded |= unfolded_codes<AFMT>(sc, w);
          const v8bf16 af = fold_decode8<AFMT>(w, sc);
#pragma unroll
          for (int j = 0; j < FN; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf[j], af, acc[i][j], 0, 0, 0);
        }
      }
    }
    if (kt + 1 < ksteps) store_lds(buf ^ 1);
    __syncthreads();
  }

  // ---- FP32-accumulation mode, exact pass over the blocks with a scale
  // outside the fold window, one 32-K block at a time (codes and scales read
  // again from global memory; rows past M or N read as zero codes)
  if constexpr (MODE == kModeBF16 && FM == 4 && FN == 4) {
    if (__builtin_amdgcn_ballot_w64(unfolded != 0u) != 0) {
      const uint8_t* ar[4];
      const uint8_t* br[4];
      const uint8_t* sar[4];
      const uint8_t* sbr[4];
      // a lane's 8 codes of block b: 8 bytes at 32 b + 8 lg (E2M1: 4 bytes
      // at 16 b + 4 lg)
      constexpr int kAW = AFMT == MX_E2M1 ? 4 : 8, kBW = BFMT == MX_E2M1 ? 4 : 8;
      auto codes_at = [](const uint8_t* p, int64_t b, int w) -> uint2 {
        return w == 4 ? make_uint2(*(const uint32_t*)(p + 16 * b), 0u) : *(const uint2*)(p + 32 * b);
      };
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t m = m0 + wm * WM + i * 16 + lr, n = n0 + wn * WN + i * 16 + lr;
        ar[i] = m < g.M ? A + m * g.lda + kAW * lg : nullptr;
        sar[i] = m < g.M ? SA + m * g.ldsa : nullptr;
        br[i] = n < g.N ? b_row_ptr(n, B, g.ldb, g.page_stride) + kBW * lg : nullptr;
        sbr[i] = n < g.N ? b_row_ptr(n, SB, g.ldsb, g.page_stride_s) : nullptr;
      }
      for (int64_t b = 0; b < kblocks; ++b) {
        uint2 qa[4], qb[4];
        uint32_t ca[4], cb[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          qa[i] = ar[i] ? codes_at(ar[i], b, kAW) : make_uint2(0, 0);
          ca[i] = sar[i] ? sar[i][b] : 127u;
          qb[i] = br[i] ? codes_at(br[i], b, kBW) : make_uint2(0, 0);
          cb[i] = sbr[i] ? sbr[i][b] : 127u;
        }
        exact_block16<AFMT, BFMT>(qa, ca, qb, cb, acc);
      }
    }
  }

  // ---- epilogue: lane owns y[m][n .. n+3]
  uint8_t* Y = (uint8_t*)g.y + (po * g.sy_o + pi * g.sy_i) * (BF16OUT ? 2 : 4);
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int64_t m = m0 + wm * WM + i * 16 + lr;
    if (m >= g.M) continue;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int64_t n = n0 + wn * WN + j * 16 + 4 * lg;
      const v4f32 v = acc[i][j];
      if constexpr (BF16OUT) {
        uint16_t* row = (uint16_t*)Y + m * g.ldy;
        if (g.y_vec && n + 3 < g.N) {
          *(uint2*)(row + n) = make_uint2(f32_to_bf16_rne(canon_nan(v[0])) | (f32_to_bf16_rne(canon_nan(v[1])) << 16),
                                          f32_to_bf16_rne(canon_nan(v[2])) | (f32_to_bf16_rne(canon_nan(v[3])) << 16));
        } else {
          for (int e = 0; e < 4; ++e)
            if (n + e < g.N) row[n + e] = (uint16_t)f32_to_bf16_rne(canon_nan(v[e]));
        }
      } else {
        float* row = (float*)Y + m * g.ldy;
        if (g.y_vec && n + 3 < g.N) {
          *(float4*)(row + n) = make_float4(v[0], v[1], v[2], v[3]);
        } else {
          for (int e = 0; e < 4; ++e)
            if (n + e < g.N) row[n + e] = v[e];
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Row-panel kernel for short reductions (K <= 128, FP32-accumulation mode),
// e.g. attention scores over one head: the output is large and the work per
// output small, so the kernel is bound by writing y. A work-group takes 256
// rows of A and up to 512 rows of B of one problem: B (codes and scales,
// gathered through the page table when paged) is loaded into LDS once,
// each wave keeps its 64 rows of A decoded in registers, and then walks the
// columns in chunks of 64, storing each chunk as soon as it is computed.
// Each wave holds 64 rows of A (4 MFMA row tiles), so every decoded B
// fragment feeds 4 MFMAs.
// No load follows the first store, so the stores stream out without being
// waited on. Work-groups of one problem are placed on one XCD so its B rows
// are read from that XCD's L2.
// ---------------------------------------------------------------------------
constexpr int kRPTiles = 4;                  // 16-row MFMA tiles of A per wave
constexpr int kRPRows = 4 * 16 * kRPTiles;   // A rows per work-group
constexpr int kRPMaxN = 512;   // B rows held in LDS

template <int AFMT, int BFMT, bool BF16OUT, bool PAGED>
__global__ __launch_bounds__(kThreads) void gemm_rowpanel_kernel(GemmArgs g, uint32_t row_blocks, uint32_t nprob) {
  __shared__ __attribute__((aligned(16))) uint8_t Bs[kRPMaxN * kBK];
  __shared__ uint32_t sBs[kRPMaxN];
  __shared__ int32_t sPage[PAGED ? kRPMaxN : 1];

  // work-group -> (problem, row block); with 8 or more problems and a
  // problem count divisible by 8, the row blocks of problem p run on XCD p % 8
  uint32_t prob, rb;
  if (nprob % 8 == 0) {
    const uint32_t x = blockIdx.x % 8, r = blockIdx.x / 8;
    prob = x + 8 * (r / row_blocks);
    rb = r % row_blocks;
  } else {
    prob = blockIdx.x / row_blocks;
    rb = blockIdx.x % row_blocks;
  }
  const int64_t po = prob / g.batch_inner, pi = prob % g.batch_inner;
  const uint8_t* A = g.a + po * g.sa_o + pi * g.sa_i;
  const uint8_t* SA = g.sa + po * g.ssa_o + pi * g.ssa_i;
  const uint8_t* B = g.b + pi * g.sb_i;
  const uint8_t* SB = g.sb + pi * g.ssb_i;
  if (!PAGED) {
    B += po * g.sb_o;
    SB += po * g.ssb_o;
  }
  const int tid = threadIdx.x;
  // Paged B: the problem's page-table entries (at most N <= 512) go to LDS
  // first, so every row address below is one LDS read and a multiply-high
  // split instead of a dependent global load and a 64-bit division each
  // (that chain made the loads of a thread go out one round trip at a time).
  if (PAGED) {
    const uint32_t npages = g.page_div.div((uint32_t)g.N - 1u) + 1u;  // host: <= pages_per_seq
    for (uint32_t i = tid; i < npages; i += kThreads) sPage[i] = g.page_table[po * g.pages_per_seq + i];
    __syncthreads();
  }
  auto b_row_ptr = [&](int64_t n, const uint8_t* base, int64_t ld, int64_t pstride) -> const uint8_t* {
    if (PAGED) {
      const uint32_t pg = g.page_div.div((uint32_t)n);
      return base + (int64_t)sPage[pg] * pstride + (int64_t)((uint32_t)n - pg * g.page_div.d) * ld;
    }
    return base + n * ld;
  };
  const int64_t kblocks = g.K / kBlock;  // 1 .. 4
  const bool dword_ok = g.scales_dword != 0;

  // ---- B into LDS: row n, 16-byte chunk c at swz(n, c); chunks past K are
  // zero. All of a thread's loads are issued before any LDS store.
  const int64_t nrows = g.N;  // <= kRPMaxN
  constexpr int kPer = kRPMaxN * 8 / kThreads;  // 16 chunks per thread
  uint4 bv[kPer];
#pragma unroll
  for (int it = 0; it < kPer; ++it) {
    const uint32_t id = tid + kThreads * it, c = id & 7;
    const int64_t n = id >> 3;
    bv[it] = make_uint4(0, 0, 0, 0);
    if (n < nrows && (int64_t)c * 16 < g.K) bv[it] = *(const uint4*)(b_row_ptr(n, B, g.ldb, g.page_stride) + c * 16);
  }
  uint32_t sv[kRPMaxN / kThreads];
#pragma unroll
  for (int it = 0; it < kRPMaxN / kThreads; ++it) {
    const int64_t n = tid + kThreads * it;
    sv[it] = n < nrows ? load_scales4(b_row_ptr(n, SB, g.ldsb, g.page_stride_s), 0, kblocks, dword_ok) : 0u;
  }
#pragma unroll
  for (int it = 0; it < kPer; ++it) {
    const uint32_t id = tid + kThreads * it;
    if ((int64_t)(id >> 3) < nrows) *(uint4*)(&Bs[swz(id >> 3, id & 7)]) = bv[it];
  }
#pragma unroll
  for (int it = 0; it < kRPMaxN / kThreads; ++it) {
    const int64_t n = tid + kThreads * it;
    if (n < nrows) sBs[n] = sv[it];
  }

  // ---- this wave's 64 rows of A, decoded: lane (r, q) of tile t takes row
  // 16 t + r and, for block kb, k = 32 kb + 8 q .. +7
  const int wave = tid >> 6, lane = tid & 63;
  const uint32_t lr = lane & 15, lg = lane >> 4;
  const int64_t mw = (int64_t)rb * kRPRows + wave * 16 * kRPTiles + lr;  // + 16 t
  v8bf16 af[kRPTiles][4];
  uint32_t sa4s[kRPTiles];
  // nonzero once a block with a scale outside the fold window holds a
  // non-zero code: that chunk then takes the exact pass before its store
  uint32_t unfolded_a = 0;
#pragma unroll
  for (int t = 0; t < kRPTiles; ++t) {
    const int64_t m = mw + 16 * t;
    const bool mok = m < g.M;
    const uint8_t* arow = A + (mok ? m : 0) * g.lda;
    sa4s[t] = mok ? load_scales4(SA + m * g.ldsa, 0, kblocks, dword_ok) : 0x7F7F7F7Fu;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      uint2 w = make_uint2(0, 0);
      if (mok && kb < kblocks) w = *(const uint2*)(arow + 32 * kb + 8 * lg);
      const uint32_t sc = (sa4s[t] >> (8 * kb)) & 0xFFu;
      unfolded_a |= unfolded_codes<AFMT>(sc, w);
      af[t][kb] = fold_decode8<AFMT>(w, sc);
    }
  }
  __syncthreads();

  // ---- columns in chunks of 64 (4 tiles of 16); lane owns y[m][n .. n+3]
  uint8_t* Y = (uint8_t*)g.y + (po * g.sy_o + pi * g.sy_i) * (BF16OUT ? 2 : 4);
  for (int64_t n0 = 0; n0 < nrows; n0 += 64) {
    v4f32 acc[kRPTiles][4];
#pragma unroll
    for (int t = 0; t < kRPTiles; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[t][j] = v4f32{0.f, 0.f, 0.f, 0.f};
    uint32_t unfolded = unfolded_a;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      if (kb < kblocks) {
        const uint32_t chunk = 2 * kb + (lg >> 1), off = 8 * (lg & 1);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t row = (uint32_t)min(n0 + j * 16 + lr, (int64_t)kRPMaxN - 1);
          const uint2 w = *(const uint2*)(&Bs[swz(row, chunk) + off]);
          const uint32_t sc = (sBs[row] >> (8 * kb)) & 0xFFu;
          if (n0 + j * 16 + lr < nrows) unfolded |= unfolded_codes<BFMT>(sc, w);
          const v8bf16 bf = fold_decode8<BFMT>(w, sc);
#pragma unroll
          for (int t = 0; t < kRPTiles; ++t)
            acc[t][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf, af[t][kb], acc[t][j], 0, 0, 0);
        }
      }
    }
    // exact pass over the blocks outside the fold window (A codes read again from
    // global memory, B codes and scales from LDS)
    if (__builtin_amdgcn_ballot_w64(unfolded != 0u) != 0) {
      for (int kb = 0; kb < kblocks; ++kb) {
        const uint32_t chunk = 2 * kb + (lg >> 1), off = 8 * (lg & 1);
        uint2 qa[4], qb[4];
        uint32_t ca[4], cb[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int64_t m = mw + 16 * t;
          qa[t] = m < g.M ? *(const uint2*)(A + m * g.lda + 32 * kb + 8 * lg) : make_uint2(0, 0);
          ca[t] = (sa4s[t] >> (8 * kb)) & 0xFFu;
          const uint32_t row = (uint32_t)min(n0 + t * 16 + lr, (int64_t)kRPMaxN - 1);
          qb[t] = *(const uint2*)(&Bs[swz(row, chunk) + off]);
          cb[t] = (sBs[row] >> (8 * kb)) & 0xFFu;
        }
        exact_block16<AFMT, BFMT>(qa, ca, qb, cb, acc);
      }
    }
#pragma unroll
    for (int t = 0; t < kRPTiles; ++t) {
      const int64_t m = mw + 16 * t;
      if (m >= g.M) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t n = n0 + j * 16 + 4 * lg;
        const v4f32 v = acc[t][j];
        if constexpr (BF16OUT) {
          uint16_t* row = (uint16_t*)Y + m * g.ldy;
          if (g.y_vec && n + 3 < g.N) {
            *(uint2*)(row + n) =
                make_uint2(f32_to_bf16_rne(canon_nan(v[0])) | (f32_to_bf16_rne(canon_nan(v[1])) << 16),
                           f32_to_bf16_rne(canon_nan(v[2])) | (f32_to_bf16_rne(canon_nan(v[3])) << 16));
          } else {
            for (int e = 0; e < 4; ++e)
              if (n + e < g.N) row[n + e] = (uint16_t)f32_to_bf16_rne(canon_nan(v[e]));
          }
        } else {
          float* row = (float*)Y + m * g.ldy;
          if (g.y_vec && n + 3 < g.N) {
            *(float4*)(row + n) = make_float4(v[0], v[1], v[2], v[3]);
          } else {
            for (int e = 0; e < 4; ++e)
              if (n + e < g.N) row[n + e] = v[e];
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Main-loop kernel for large aligned problems, in the FP8, FP32-accumulation
// and FP4 modes.
//
// Tile 256 x 256 per workgroup, 4 waves of 128 x 128, built from
// v_mfma_scale_f32_32x32x64_f8f6f4 (K = 64 per issue = 2 MX blocks). K
// advances 128 bytes per stage -- whole 128-byte cache lines of every operand
// row -- through two LDS stages of 64 KB (A and B) filled by direct
// global->LDS loads; scales arrive 16 bytes per row (4 stages' worth) at a
// time into two 8 KB buffers, so a scale line is fetched once per 4 stages.
// Operand layout of the 32x32x64 instruction: lane l (row l % 32, half
// g = l / 32) holds k = 16g .. 16g+15 in bytes 0-15 and k = 32+16g .. +15 in
// bytes 16-31, and supplies the scale of (row, block g). The result D[i][j]
// sits in lane j + 32 * ((i / 4) % 2), element 4 * (i / 8) + i % 4.
// Rows are 128 bytes; their 16-byte chunks are XOR-permuted by row (fperm)
// so the fragment reads are free of bank conflicts. Rows past M or N are
// clamped to the last row for loading and skipped on store. Work-groups are
// dealt round-robin to the 8 XCDs, so tile ids are remapped to give each XCD
// a contiguous band of tiles (shared panels stay in that XCD's L2). With
// whole tiles the FP8 and FP4 modes run one work-group per CU, each walking
// tiles (see "Persistent walk" in the kernel).
// Requires K % 512 == 0 and 16-byte aligned scale rows.
//
// FP4 mode (both operands MXFP4, codes two per byte): a 128-byte stage holds
// 256 K. For E2M1 the instruction takes 16 bytes per lane, k = 32g .. 32g+31
// of its 64 (checked on the device), so the two 16-byte chunks a lane reads
// for a K half are the operands of two instructions (the upper half of each
// 8-register operand is left undefined and the compiler narrows it to 4
// registers). A stage has 8 scale blocks, so its scale groups hold 2 stages
// (16 bytes per row) instead of 4. Requires K % 1024 == 0.
// ---------------------------------------------------------------------------
// Two f32 -> two bf16 in one v_cvt_pk_bf16_f32 (round to nearest even; checked
// on the device against the integer rounding for every non-NaN f32 pattern).
typedef float mx_f2 __attribute__((ext_vector_type(2)));
typedef __bf16 mx_b2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2_hw(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((mx_f2){a, b}, mx_b2));
}
constexpr int kFBM = 256, kFBN = 256, kFBK = 128;
constexpr uint32_t kCodeStage = kFBM * kFBK;   // bytes per operand per stage
constexpr uint32_t kScaleRow = 16;             // scale bytes per row per scale group (4 FP8 / 2 FP4 stages)
constexpr uint32_t kScaleBuf = kFBM * kScaleRow;

// Origin of a large-tile work-group's 256 x 256 output tile. Work-groups
// are dealt round-robin to the 8 XCDs, so tile ids are remapped to give each
// XCD a contiguous band of tiles (shared panels stay in that XCD's L2),
// walked in groups of 4 tile rows. In the grouped mode the grid has
// ceil(M / 256) + groups row tiles; row tile t belongs to the group whose
// tiles (ceil(rows / 256) each, offsets clamped to [0, M]) cover it, found
// by every wave with a prefix sum over the groups, 64 at a time. Returns
// false for the tiles past the last group's (their work-groups return
// before any load or barrier).
struct BigTile {
  int64_t m0, n0, m_end, po, pi;
  uint32_t tile_m, tile_n;
};
// (tile_m, tile_n) of work-group bid: XCD bands, then groups of 4 tile rows
__device__ __forceinline__ void big_tile_coords(const GemmArgs& g, uint32_t bid, uint32_t& tile_m, uint32_t& tile_n) {
  const uint32_t ntiles = g.tiles_m * g.tiles_n;
  uint32_t lid = bid;
  if (ntiles % 8 == 0) lid = (lid % 8) * (ntiles / 8) + lid / 8;
  const uint32_t group = 4;
  const uint32_t per_group = group * g.tiles_n;
  const uint32_t first_m = (lid / per_group) * group;
  const uint32_t gm = min(g.tiles_m - first_m, group);
  tile_m = first_m + (lid % per_group) % gm;
  tile_n = (lid % per_group) / gm;
}
__device__ __forceinline__ bool big_tile(const GemmArgs& g, int lane, BigTile& r) {
  big_tile_coords(g, blockIdx.x, r.tile_m, r.tile_n);
  r.n0 = (int64_t)r.tile_n * kFBN;
  if (g.group_off == nullptr) {
    r.m0 = (int64_t)r.tile_m * kFBM;
    r.m_end = g.M;
    const int64_t p = blockIdx.y;
    r.po = p / g.batch_inner;
    r.pi = p % g.batch_inner;
    return true;
  }
  const uint32_t t = r.tile_m;
  int64_t found = -1, lo_f = 0, hi_f = 0, first_tile = 0, prefix = 0;
  for (uint32_t q0 = 0; q0 < g.groups && found < 0; q0 += 64) {
    const uint32_t q = q0 + lane;
    int64_t lo = 0, hi = 0;
    if (q < g.groups) {
      lo = min(max(g.group_off[q], (int64_t)0), g.M);
      hi = min(max(g.group_off[q + 1], lo), g.M);
    }
    const int64_t nt = (hi - lo + kFBM - 1) / kFBM;
    int64_t incl = nt;  // inclusive prefix of the tile counts across the wave
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int64_t v = __shfl_up(incl, d);
      if (lane >= d) incl += v;
    }
    const int64_t chunk = __shfl(incl, 63);
    if ((int64_t)t < prefix + chunk) {
      const bool mine = (int64_t)t >= prefix + incl - nt && (int64_t)t < prefix + incl;
      const int src = __ffsll((unsigned long long)__ballot(mine)) - 1;
      found = q0 + src;
      lo_f = __shfl(lo, src);
      hi_f = __shfl(hi, src);
      first_tile = prefix + __shfl(incl - nt, src);
    }
    prefix += chunk;
  }
  if (found < 0) return false;
  r.m0 = lo_f + ((int64_t)t - first_tile) * kFBM;
  r.m_end = hi_f;
  r.po = found;
  r.pi = 0;
  return true;
}

// Store one 32 x 32 accumulator tile of v_mfma_*_32x32x* (lane (lr, lg)
// holds row lr, columns 8 q + 4 lg .. +3 in elements 4 q .. 4 q + 3) at
// output row m, columns nb .. nb + 31. Every lane takes part (the bf16 path
// swaps dwords across lane halves); only lanes with mok store, and columns
// at or past N are skipped.
template <bool BF16OUT>
__device__ __forceinline__ void store_tile32(const GemmArgs& g, uint8_t* Y, const v16f32& acc, int64_t m, bool mok,
                                             int64_t nb, uint32_t lg) {
  if constexpr (BF16OUT) {
    uint16_t* row = (uint16_t*)Y + m * g.ldy;
    uint32_t w[4][2];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      w[q][0] = pack_bf16x2_hw(acc[4 * q], acc[4 * q + 1]);
      w[q][1] = pack_bf16x2_hw(acc[4 * q + 2], acc[4 * q + 3]);
    }
    if (g.y_vec && nb + 32 <= g.N) {
      // Lanes l and l + 32 (same row) hold columns 16p + 4 lg .. and
      // 16p + 8 + 4 lg ..; one lane swap per dword gives lane lg the 8
      // consecutive columns 16p + 8 lg .. +7, stored as 16 bytes.
#pragma unroll
      for (int pq = 0; pq < 2; ++pq) {
        const auto r0 = __builtin_amdgcn_permlane32_swap(w[2 * pq][0], w[2 * pq + 1][0], false, false);
        const auto r1 = __builtin_amdgcn_permlane32_swap(w[2 * pq][1], w[2 * pq + 1][1], false, false);
        if (mok) *(uint4*)(row + nb + 16 * pq + 8 * lg) = make_uint4(r0[0], r1[0], r0[1], r1[1]);
      }
    } else if (mok) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t n = nb + 8 * q + 4 * lg;
        if (g.y_vec && n + 3 < g.N) {
          *(uint2*)(row + n) = make_uint2(w[q][0], w[q][1]);
        } else {
          for (int e = 0; e < 4; ++e)
            if (n + e < g.N) row[n + e] = (uint16_t)(w[q][e >> 1] >> (16 * (e & 1)));
        }
      }
    }
  } else if (mok) {
    float* row = (float*)Y + m * g.ldy;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t n = nb + 8 * q + 4 * lg;
      const float v0 = acc[4 * q], v1 = acc[4 * q + 1], v2 = acc[4 * q + 2], v3 = acc[4 * q + 3];
      if (g.y_vec && n + 3 < g.N) {
        *(float4*)(row + n) = make_float4(v0, v1, v2, v3);
      } else {
        const float vv[4] = {v0, v1, v2, v3};
        for (int e = 0; e < 4; ++e)
          if (n + e < g.N) row[n + e] = vv[e];
      }
    }
  }
}

template <int AFMT, int BFMT, bool BF16OUT, int MODE>
__global__ __launch_bounds__(kThreads, 1) void gemm_big_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(1024))) uint8_t As[2][kCodeStage];
  __shared__ __attribute__((aligned(1024))) uint8_t Bs[2][kCodeStage];
  __shared__ __attribute__((aligned(16))) uint8_t sAs[2][kScaleBuf];
  __shared__ __attribute__((aligned(16))) uint8_t sBs[2][kScaleBuf];
  constexpr bool kFP4 = MODE == kModeFP4;
  // stages per scale group: 16 scale bytes per row hold 4 FP8 stages (4 blocks
  // each) or 2 FP4 stages (8 blocks each)
  constexpr int kG = kFP4 ? 2 : 4;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;

  BigTile tl;
  if (!big_tile(g, lane, tl)) return;
  int64_t m0 = tl.m0, n0 = tl.n0;
  const int64_t m_end = tl.m_end, po = tl.po, pi = tl.pi;
  uint32_t tile_m = tl.tile_m, tile_n = tl.tile_n;
  const uint8_t* A = g.a + po * g.sa_o + pi * g.sa_i;
  const uint8_t* SA = g.sa + po * g.ssa_o + pi * g.ssa_i;
  const uint8_t* B = g.b + po * g.sb_o + pi * g.sb_i;
  const uint8_t* SB = g.sb + po * g.ssb_o + pi * g.ssb_i;

  const int64_t nsteps = (kFP4 ? g.K / 2 : g.K) / kFBK;  // a multiple of 4

  // ---- loads. Codes: per stage and operand, 8 instructions per wave, each
  // 8 rows x 128 bytes (lane i: row i / 8, LDS chunk i % 8, which holds the
  // row's logical chunk (i % 8) ^ fperm(row)). Scales: per group of 4
  // stages and operand, one instruction per wave, 64 rows x 16 bytes. Rows
  // past M / N are clamped to the last row.
  const uint8_t* a_base = uniform_ptr(A + m0 * g.lda);
  const uint8_t* b_base = uniform_ptr(B + n0 * g.ldb);
  const uint8_t* sa_base = uniform_ptr(SA + m0 * g.ldsa);
  const uint8_t* sb_base = uniform_ptr(SB + n0 * g.ldsb);
  const int64_t a_last = m_end - 1 - m0, b_last = g.N - 1 - n0;
  uint32_t a_off[8], b_off[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const uint32_t row = wave * 64 + t * 8 + (lane >> 3);
    const uint32_t chunk16 = (((uint32_t)lane & 7u) ^ fperm(row)) << 4;
    a_off[t] = (uint32_t)min((int64_t)row, a_last) * (uint32_t)g.lda + chunk16;
    b_off[t] = (uint32_t)min((int64_t)row, b_last) * (uint32_t)g.ldb + chunk16;
  }
  const uint32_t srow = wave * 64 + lane;
  const uint32_t sa_off = (uint32_t)min((int64_t)srow, a_last) * (uint32_t)g.ldsa;
  const uint32_t sb_off = (uint32_t)min((int64_t)srow, b_last) * (uint32_t)g.ldsb;
  const uint32_t a_dst = lds_off(&As[0][0]) + wave * 64 * kFBK, b_dst = lds_off(&Bs[0][0]) + wave * 64 * kFBK;
  const uint32_t sa_dst = lds_off(&sAs[0][0]) + wave * 64 * kScaleRow;
  const uint32_t sb_dst = lds_off(&sBs[0][0]) + wave * 64 * kScaleRow;
  // L2 prefetch. The 32 work-groups that an XCD runs at once (4 tile rows x
  // 8 tile columns) walk K together, so without it every stage's lines are
  // new to that XCD's L2 and each stage's loads wait for HBM. Four stages
  // ahead, each work-group touches one dword of every 128-byte line of its
  // share of those lines (32 of the A rows its tile row shares with 8 tile
  // columns, 64 of the B rows its tile column shares with 4 tile rows) with
  // one direct-to-LDS load per wave into a sink nobody reads. It is issued
  // after the stage's code loads, and loads retire in order, so the barrier
  // waits with vmcnt(1) and leaves only the prefetch in flight (1.5 stages to
  // land). On 8192^3 after a cache-evicting read it removes 17 % of the
  // kernel's cycles (load waits 12.2k -> 3.0k, slow second halves 99.7k ->
  // 82.8k per wave). With N(0,1) operands the part is at its power limit and
  // the clock drops from 1.85 to 1.70 GHz, so the time gains ~1-8 %; with
  // less toggling operands it gains 9 %. The FP8 and FP4 modes use it; the
  // FP32-accumulation mode measured no gain (its slow second halves are not
  // load waits).
  constexpr int kPF = MODE != kModeBF16 ? 1 : 0;
  __shared__ __attribute__((aligned(16))) uint8_t pf_sink[kPF ? 256 : 16];  // 64 lanes x 4 bytes
  const uint32_t pf_dst = lds_off(&pf_sink[0]);

  // ---- Persistent walk. When every tile is whole (M and N multiples of 256,
  // not grouped, one batch entry) the host may launch fewer work-groups than
  // tiles; work-group b then computes tiles b, b + gridDim.x, ... (the same
  // XCD band as with one tile per work-group). The prefetches of a tile's
  // last 4 stages touch the next tile's first 4, and the next tile's first
  // loads go out before this tile's epilogue stores, so its prologue runs
  // under them. The load row offsets above hold for every whole tile. (The
  // FP32-accumulation mode has no registers to spare for it.)
  const bool walk = MODE != kModeBF16 && g.group_off == nullptr && gridDim.y == 1 && g.M % kFBM == 0 && g.N % kFBN == 0;
  const uint32_t ntiles_all = g.tiles_m * g.tiles_n;
  uint32_t bid = blockIdx.x;

  // Prefetch addresses: a 32-bit lane offset (row and stage) from a wave-
  // uniform base, which is the tile's first row, or when walking the
  // operand's first row (every offset fits: on that path M * lda and
  // N * ldb are below 2^32), so that the next tile needs no base of its own.
  const uint8_t* pf_base = uniform_ptr(walk ? (wave < 2 ? A : B) : (wave < 2 ? a_base : b_base));
  // the offset of this lane's prefetch row in tile (tm, tn) whose first rows
  // are tm0 of A and tn0 of B
  auto pf_row_off = [&](uint32_t tm, uint32_t tn, int64_t tm0, int64_t tn0) -> uint32_t {
    const uint32_t r = wave < 2 ? (tn % 8) * 32 + 16 * wave + (lane & 15) : (tm % 4) * 64 + 32 * (wave - 2) + (lane & 31);
    const int64_t origin = walk ? (wave < 2 ? tm0 : tn0) : 0;
    return (uint32_t)(origin + min((int64_t)r, wave < 2 ? a_last : b_last)) * (uint32_t)(wave < 2 ? g.lda : g.ldb);
  };
  uint32_t pf_off = pf_row_off(tile_m, tile_n, m0, n0);
  auto issue_pf = [&](int64_t src) {
    if constexpr (kPF) dma4(pf_dst, pf_off + (uint32_t)src * kFBK, pf_base);
  };

  // Codes of stage `src`, rows 16q .. 16q + 15 of each wave's 64 for
  // q in [q0, q1), into LDS buffer `buf` (buf, q0 and q1 are unrolled
  // constants at every call, so each LDS address is a base plus an
  // immediate).
  auto issue_rows = [&](int64_t src, uint32_t buf, int q0, int q1) {
    const uint8_t* ab = a_base + src * kFBK;
    const uint8_t* bb = b_base + src * kFBK;
#pragma unroll
    for (int t = 2 * q0; t < 2 * q1; ++t) {
      dma16_at(a_dst, buf * kCodeStage + t * 8 * kFBK, a_off[t], ab);
      dma16_at(b_dst, buf * kCodeStage + t * 8 * kFBK, b_off[t], bb);
    }
  };
  auto issue_codes = [&](int64_t src, uint32_t buf) { issue_rows(src, buf, 0, 4); };
  // a quarter of the codes of stage `src`
  auto issue_codes_part = [&](int64_t src, uint32_t buf, int q) { issue_rows(src, buf, q, q + 1); };
  // (the buffer of a scale group is a run-time value: the two addresses are
  // formed here, and pass through an empty asm so that the compiler does
  // not keep both buffers' addresses in scalar registers)
  auto issue_scales = [&](int64_t grp) {
    const uint32_t buf = (uint32_t)(grp & 1);
    uint32_t la = sa_dst + buf * kScaleBuf, lb = sb_dst + buf * kScaleBuf;
    asm volatile("" : "+s"(la), "+s"(lb));
    dma16(la, sa_off, sa_base + grp * kScaleRow);
    dma16(lb, sb_off, sb_base + grp * kScaleRow);
  };

  // ---- fragment reads: lane (lr, lg) of fragment f reads row base + 32 f;
  // the permutation term depends only on lr, so every read is a per-lane
  // base address plus a compile-time offset (carried as an immediate).
  const int wm = wave >> 1, wn = wave & 1;
  const uint32_t lr = lane & 31, lg = lane >> 5;
  const uint32_t fp = fperm(lr);
  const uint8_t* a_row = &As[0][0] + (wm * 128 + lr) * kFBK;
  const uint8_t* b_row = &Bs[0][0] + (wn * 128 + lr) * kFBK;
  const uint8_t* a_sc = &sAs[0][0] + (wm * 128 + lr) * kScaleRow;
  const uint8_t* b_sc = &sBs[0][0] + (wn * 128 + lr) * kScaleRow;
  // K half h of a stage: logical chunks 4h + lg and 4h + 2 + lg
  const uint32_t c_lo[2] = {((0 + lg) ^ fp) << 4, ((4 + lg) ^ fp) << 4};
  const uint32_t c_hi[2] = {((2 + lg) ^ fp) << 4, ((6 + lg) ^ fp) << 4};
  // Scales: once per group of 4 stages each lane reads the 16 scale bytes of
  // its 4 rows per operand (16-byte reads of consecutive rows, free of bank
  // conflicts, where byte reads of a 16-byte-pitch array are not). Word w of
  // row f holds blocks 4w .. 4w+3 of the group; shifting it right by 8 * lg
  // puts block 4w + lg in byte 0 and block 4w + 2 + lg in byte 2, so the
  // scale of (stage w, half h) is the word shifted right by 16 h (the
  // instruction reads byte 0).
  // (FP32-accumulation mode: no shift; the lane needs both blocks 2h and
  // 2h + 1, found in bytes 0 and 1 of the word shifted right by 16 h.)
  // (FP4 mode: the group's 32 bytes are words 0-3 here and 4-7 in the second
  // buffer; stage w uses words 2w and 2w + 1, K half h word 2w + h, whose
  // byte 0 (after the shift by 8 lg) is the scale of the half's first
  // instruction and byte 2 that of its second.)
  uint4 sa4[4], sb4[4];
  // FP32-accumulation mode: does some scale of the wave's rows in this group
  // of stages lie outside its fold window? (lanes of the lower half test the
  // A rows, lanes of the upper half the B rows; both halves hold the same
  // rows.) Wave-uniform; each fragment set carries the answer of the group
  // its scales came from (set_out).
  bool grp_out = false;
  bool set_out[2] = {false, false};
  auto read_scales = [&](int sbuf) {
    const uint32_t sh = MODE != kModeBF16 ? 8 * lg : 0;
    uint32_t out = 0;
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      uint4 va = *(const uint4*)(a_sc + sbuf * kScaleBuf + f * 32 * kScaleRow);
      uint4 vb = *(const uint4*)(b_sc + sbuf * kScaleBuf + f * 32 * kScaleRow);
      sa4[f] = make_uint4(va.x >> sh, va.y >> sh, va.z >> sh, va.w >> sh);
      sb4[f] = make_uint4(vb.x >> sh, vb.y >> sh, vb.z >> sh, vb.w >> sh);
      if constexpr (MODE == kModeBF16) {
        const uint4 v = lg ? vb : va;
        const uint32_t lo = lg ? fold_lo<BFMT>() : fold_lo<AFMT>(), hi = lg ? fold_hi<BFMT>() : fold_hi<AFMT>();
        out |= any_byte_outside(v.x, lo, hi) | any_byte_outside(v.y, lo, hi) | any_byte_outside(v.z, lo, hi) |
               any_byte_outside(v.w, lo, hi);
      }
    }
    if constexpr (MODE == kModeBF16) grp_out = __builtin_amdgcn_ballot_w64(out != 0u) != 0;
  };
  auto word_of = [&](const uint4& w4, int k) -> uint32_t {
    return k == 0 ? w4.x : k == 1 ? w4.y : k == 2 ? w4.z : w4.w;
  };
  auto scale_of = [&](const uint4* s4, int f, int sub, int h) -> int {
    if constexpr (kFP4) {
      return (int)word_of(s4[f], 2 * sub + h);
    } else {
      return (int)(word_of(s4[f], sub) >> (16 * h));
    }
  };
  auto read_frag = [&](const uint8_t* row_base, const uint4* s4, int buf, int sub, int h, int f,
                       v8i32& fr, int& sc) {
    const uint8_t* r = row_base + buf * kCodeStage + f * 32 * kFBK;
    const uint4 lo = *(const uint4*)(r + c_lo[h]);
    const uint4 hi = *(const uint4*)(r + c_hi[h]);
    fr = v8i32{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    sc = scale_of(s4, f, sub, h);
  };

  v16f32 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  // Fragments of one K half (4 A + 4 B) live in register set 0 (first half
  // of a stage) or 1 (second half). While one set feeds 16 MFMAs, the other
  // is refilled one A and one B fragment per group of 4 MFMAs, so LDS reads
  // are spread evenly over the stage.
  v8i32 fa[2][4], fb[2][4];
  int sa[2][4], sb[2][4];

  // FP32-accumulation mode over the whole E8M0 range. A block whose scale
  // lies outside its fold window is folded inexactly (fold_decode8); it
  // matters only if it holds a non-zero code or its scale is the NaN code,
  // and then the wave replaces its terms in the exact pass after the main
  // loop (exact_flag). Only in K halves whose group of scales has a scale
  // outside the window (set_out) do the lanes look at their scales and
  // codes, so all-zero blocks (scale code 0) never start the exact pass.
  bool needs_exact = false;
  auto check_half = [&](int set) {
    if constexpr (MODE == kModeBF16) {
      if (set_out[set]) {
        // branch-free (no short-circuit): divergent branches in the main
        // loop make the compiler move the accumulators out of registers
        uint32_t bad = 0;
#pragma unroll
        for (int f = 0; f < 4; ++f)
#pragma unroll
          for (int blk = 0; blk < 2; ++blk) {
            const v8i32 x = fa[set][f], y = fb[set][f];
            const uint32_t ora = (uint32_t)(x[4 * blk] | x[4 * blk + 1] | x[4 * blk + 2] | x[4 * blk + 3]);
            const uint32_t orb = (uint32_t)(y[4 * blk] | y[4 * blk + 1] | y[4 * blk + 2] | y[4 * blk + 3]);
            bad |= exact_flag<AFMT>(((uint32_t)sa[set][f] >> (8 * blk)) & 0xFFu, ora) |
                   exact_flag<BFMT>(((uint32_t)sb[set][f] >> (8 * blk)) & 0xFFu, orb);
          }
        needs_exact |= bad != 0u;
      }
    }
  };

  // One of the 4 MFMA groups of a K half. FP8 mode: group i is the 4
  // scaled MFMAs of A fragment i. FP32-accumulation mode: group t is K step
  // t of the half (8 of each lane's 32 codes, bytes 8t .. 8t+7, the same
  // k positions in A and B), decoded exactly to bf16 with the block scale
  // folded in (blocks 2h for t < 2, 2h + 1 after), then 16
  // v_mfma_f32_32x32x16_bf16; each decoded B fragment feeds 4 of them.
  // FP4 mode: the two instructions of a K half, on the lower and upper
  // 16 bytes of each fragment
  auto mfma_fp4 = [&](int set, int i, int j) {
    const v8i32 a_lo = __builtin_shufflevector(fa[set][i], fa[set][i], 0, 1, 2, 3, -1, -1, -1, -1);
    const v8i32 a_hi = __builtin_shufflevector(fa[set][i], fa[set][i], 4, 5, 6, 7, -1, -1, -1, -1);
    const v8i32 b_lo = __builtin_shufflevector(fb[set][j], fb[set][j], 0, 1, 2, 3, -1, -1, -1, -1);
    const v8i32 b_hi = __builtin_shufflevector(fb[set][j], fb[set][j], 4, 5, 6, 7, -1, -1, -1, -1);
    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b_lo, a_lo, acc[i][j], kMfmaFP4, kMfmaFP4, 0,
                                                                 sb[set][j], 0, sa[set][i]);
    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b_hi, a_hi, acc[i][j], kMfmaFP4, kMfmaFP4, 0,
                                                                 sb[set][j] >> 16, 0, sa[set][i] >> 16);
  };
  auto mfma_pair = [&](int set, int i, int j0) {
#pragma unroll
    for (int j = j0; j < j0 + 2; ++j) {
      if constexpr (kFP4)
        mfma_fp4(set, i, j);
      else
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb[set][j], fa[set][i], acc[i][j], BFMT, AFMT, 0,
                                                                     sb[set][j], 0, sa[set][i]);
    }
  };
  auto mfma_group = [&](int set, int i) {
    if constexpr (kFP4) {
#pragma unroll
      for (int j = 0; j < 4; ++j) mfma_fp4(set, i, j);
    } else if constexpr (MODE == kModeFP8) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb[set][j], fa[set][i], acc[i][j], BFMT, AFMT, 0,
                                                                     sb[set][j], 0, sa[set][i]);
    } else {
      const int t = i;
      v8bf16 bb[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bb[j] = fold_decode8<BFMT>(make_uint2((uint32_t)fb[set][j][2 * t], (uint32_t)fb[set][j][2 * t + 1]),
                                   ((uint32_t)sb[set][j] >> (8 * (t >> 1))) & 0xFFu);
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const v8bf16 aa = fold_decode8<AFMT>(make_uint2((uint32_t)fa[set][a][2 * t], (uint32_t)fa[set][a][2 * t + 1]),
                                             ((uint32_t)sa[set][a] >> (8 * (t >> 1))) & 0xFFu);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[a][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bb[j], aa, acc[a][j], 0, 0, 0);
      }
    }
  };

  // Pipeline. Stage s lives in LDS buffer s % 2. In the middle of stage s
  // (its second-half fragments are already in registers) one barrier
  // publishes stage s+1 and frees buffer s % 2, and the loads of stage s+2
  // go out into it during the following MFMA groups, so each stage has most
  // of a stage of MFMA work to land. The loop body has
  // no branches (a branch lets the compiler sink MFMAs past the barrier):
  // past the last stage the loads repeat the last stage into the free
  // buffer and the extra fragment reads are discarded (a walking work-group
  // then loads the next tile's first stages after the loop).
  const int64_t last = nsteps - 1;
  issue_scales(0);
  issue_codes(0, 0);
  issue_codes(1, 1);
  issue_pf(min((int64_t)3, last));
  wait_vmcnt<16 + kPF>();  // scales and stage 0 landed; stage 1 may still be in flight
  barrier();
  // a tile's first K half and scale group, from LDS buffer 0
  auto read_first = [&]() {
    read_scales(0);
    set_out[0] = grp_out;
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      read_frag(a_row, sa4, 0, 0, 0, f, fa[0][f], sa[0][f]);
      read_frag(b_row, sb4, 0, 0, 0, f, fb[0][f], sb[0][f]);
    }
  };
  read_first();

  for (;;) {  // the tiles of this work-group
  // the work-group's next tile, if any, and where the prefetches of this
  // tile's last group go: that tile's stages 0 .. 3, or else this tile's
  // last stage again
  const bool has_next = walk && bid + gridDim.x < ntiles_all;
  uint32_t ntm = 0, ntn = 0;
  if (has_next) big_tile_coords(g, bid + gridDim.x, ntm, ntn);
  const uint32_t pfn_off =
      has_next ? pf_row_off(ntm, ntn, (int64_t)ntm * kFBM, (int64_t)ntn * kFBN) : pf_off + (uint32_t)last * kFBK;
  const uint32_t pfn_step = has_next ? (uint32_t)kFBK : 0u;
  for (int64_t s0 = 0; s0 < nsteps; s0 += 4) {
    // the prefetches of this group (stages s0 + 4 .. s0 + 7), chosen here,
    // outside the scheduling regions below
    const bool lastg = s0 + 4 >= nsteps;
    const uint32_t pf_group = lastg ? pfn_off : pf_off + (uint32_t)(s0 + 4) * kFBK;
    const uint32_t pf_gstep = lastg ? pfn_step : (uint32_t)kFBK;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t s = s0 + u;
      const int buf = u & 1, sbuf = (int)((s / kG) & 1), sub = (int)(s % kG);
      // ---- first half: MFMAs on set 0; set 1 <- second half of stage s.
      // (The exactness test of a set sits where a scheduling barrier already
      // splits the loop body: a branch inside an MFMA group would keep its
      // LDS reads from interleaving with its MFMAs.)
      check_half(0);
      __builtin_amdgcn_sched_barrier(0);
      set_out[1] = grp_out;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        read_frag(a_row, sa4, buf, sub, 1, i, fa[1][i], sa[1][i]);
        read_frag(b_row, sb4, buf, sub, 1, i, fb[1][i], sb[1][i]);
        mfma_group(0, i);
        __builtin_amdgcn_sched_barrier(0);
      }
      // ---- publish stage s+1 (its loads were issued one stage ago); every
      // wave holds the rest of stage s in registers, so buffer s % 2 is free
      wait_vmcnt<kPF>();
      wait_lgkmcnt0();
      barrier();
      if ((u + 2) % kG == 0) issue_scales(min((s + 2) / kG, nsteps / kG - 1));
      // the next scale group was published by this barrier
      if (u % kG == kG - 1) read_scales(sbuf ^ 1);
      __builtin_amdgcn_sched_barrier(0);
      check_half(1);
      __builtin_amdgcn_sched_barrier(0);
      // ---- second half: MFMAs on set 1; set 0 <- first half of stage s+1.
      // The loads of stage s+2 are issued a quarter per MFMA group: a wave
      // issues in order, and 18 loads in a row would hold back its MFMAs.
      const int nbuf = buf ^ 1, nsub = (sub + 1) % kG;
      set_out[0] = grp_out;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        read_frag(a_row, sa4, nbuf, nsub, 0, i, fa[0][i], sa[0][i]);
        read_frag(b_row, sb4, nbuf, nsub, 0, i, fb[0][i], sb[0][i]);
        if constexpr (MODE != kModeBF16) {
          // the loads go out between two pairs of MFMAs, so the matrix unit
          // has queued work while the wave issues them
          mfma_pair(1, i, 0);
          __builtin_amdgcn_sched_barrier(0);
          issue_codes_part(min(s + 2, last), (uint32_t)buf, i);
          __builtin_amdgcn_sched_barrier(0);
          mfma_pair(1, i, 2);
        } else {
          issue_codes_part(min(s + 2, last), (uint32_t)buf, i);
          mfma_group(1, i);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (kPF) dma4(pf_dst, pf_group + (uint32_t)u * pf_gstep, pf_base);
    }
  }
  wait_vmcnt<0>();  // no load may still be writing LDS when the group ends

  // ---- FP32-accumulation mode, exact pass. The main loop folded every
  // block, exactly only where the scale lies inside its window; a wave that
  // met a block outside it holding a non-zero code replaces those terms
  // here, reading the blocks' scales and codes again (from L2): the folded
  // terms are taken back (two passes of the negated folded operands), and
  // the exact ones added over the cells of ExactCells, where the A rows of
  // class x and the B rows of class y are folded with scales shifted by -w
  // and +w (every other row's codes zeroed), which keeps both exact, normal
  // bf16. Every pass accumulates the block's two K steps straight into the
  // output tiles, as the main loop does. Lane (lr, lg) holds k = 16 lg .. 16 lg + 15 of a block,
  // as in the main loop, so the two steps take its dwords 0-1 and 2-3.
  if constexpr (MODE == kModeBF16) {
    if (__builtin_amdgcn_ballot_w64(needs_exact) != 0) {
      constexpr ExactCells<AFMT, BFMT> cells{};
      static_assert(cells.feasible(), "a cell of the exact pass has no common shift");
      // row offsets from the tile's (wave-uniform) bases; they fit in 32
      // bits, as the main loop's do
      uint32_t ao[4], bo[4], sao[4], sbo[4];
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        const uint32_t ra = (uint32_t)min((int64_t)(wm * 128 + f * 32 + lr), a_last);
        const uint32_t rb = (uint32_t)min((int64_t)(wn * 128 + f * 32 + lr), b_last);
        ao[f] = ra * (uint32_t)g.lda + 16 * lg;
        bo[f] = rb * (uint32_t)g.ldb + 16 * lg;
        sao[f] = ra * (uint32_t)g.ldsa;
        sbo[f] = rb * (uint32_t)g.ldsb;
      }
      const uint32_t kblocks = (uint32_t)(g.K / kBlock);
      for (uint32_t b = 0; b < kblocks; ++b) {
        uint32_t ca[4], cb[4];
        bool any = false;
#pragma unroll
        for (int f = 0; f < 4; ++f) {
          ca[f] = sa_base[sao[f] + b];
          cb[f] = sb_base[sbo[f] + b];
          any |= (fold_excluded<AFMT>(ca[f]) ? 1 : 0) | (fold_excluded<BFMT>(cb[f]) ? 1 : 0);  // no short circuit
        }
        if (__builtin_amdgcn_ballot_w64(any) == 0) continue;
        uint4 qa[4], qb[4];
        uint32_t nz = 0;
#pragma unroll
        for (int f = 0; f < 4; ++f) {
          qa[f] = *(const uint4*)(a_base + ao[f] + 32 * b);
          qb[f] = *(const uint4*)(b_base + bo[f] + 32 * b);
          nz |= exact_flag<AFMT>(ca[f], qa[f].x | qa[f].y | qa[f].z | qa[f].w);
          nz |= exact_flag<BFMT>(cb[f], qb[f].x | qb[f].y | qb[f].z | qb[f].w);
        }
        if (__builtin_amdgcn_ballot_w64(nz != 0u) == 0) continue;
        // take back the main loop's (folded) terms of the pairs the fold
        // does not cover: R1 = left-out A rows x every B row, R2 = the other
        // A rows x left-out B rows
        bool exa[4], exb[4];
        v8bf16 b0[4], b1[4];
#pragma unroll
        for (int f = 0; f < 4; ++f) {
          exa[f] = fold_excluded<AFMT>(ca[f]);
          exb[f] = fold_excluded<BFMT>(cb[f]);
          b0[f] = exact_operand<BFMT>(make_uint2(qb[f].x, qb[f].y), cb[f], true);
          b1[f] = exact_operand<BFMT>(make_uint2(qb[f].z, qb[f].w), cb[f], true);
        }
#pragma unroll
        for (int f = 0; f < 4; ++f) {
          if (__builtin_amdgcn_ballot_w64(exa[f]) == 0) continue;
          const v8bf16 a0 = neg_bf16x8(exact_operand<AFMT>(make_uint2(qa[f].x, qa[f].y), ca[f], exa[f]));
          const v8bf16 a1 = neg_bf16x8(exact_operand<AFMT>(make_uint2(qa[f].z, qa[f].w), ca[f], exa[f]));
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            acc[f][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b0[j], a0, acc[f][j], 0, 0, 0);
            acc[f][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b1[j], a1, acc[f][j], 0, 0, 0);
          }
        }
        if (__builtin_amdgcn_ballot_w64(exb[0] || exb[1] || exb[2] || exb[3]) != 0) {
          bool bon[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            bon[j] = __builtin_amdgcn_ballot_w64(exb[j]) != 0;
            b0[j] = exact_operand<BFMT>(make_uint2(qb[j].x, qb[j].y), cb[j], exb[j]);
            b1[j] = exact_operand<BFMT>(make_uint2(qb[j].z, qb[j].w), cb[j], exb[j]);
          }
#pragma unroll
          for (int f = 0; f < 4; ++f) {
            const v8bf16 a0 = neg_bf16x8(exact_operand<AFMT>(make_uint2(qa[f].x, qa[f].y), ca[f], !exa[f]));
            const v8bf16 a1 = neg_bf16x8(exact_operand<AFMT>(make_uint2(qa[f].z, qa[f].w), ca[f], !exa[f]));
#pragma unroll
            for (int j = 0; j < 4; ++j)
              if (bon[j]) {
                acc[f][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b0[j], a0, acc[f][j], 0, 0, 0);
                acc[f][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b1[j], a1, acc[f][j], 0, 0, 0);
              }
          }
        }
        // and add their exact values, cell by cell
        uint32_t xa[4], xb[4];
#pragma unroll
        for (int f = 0; f < 4; ++f) {
          xa[f] = exact_class<AFMT>(ca[f]);
          xb[f] = exact_class<BFMT>(cb[f]);
        }
        for (int c = 0; c < cells.n; ++c) {
          const int cx = cells.cell[c].x, cy = cells.cell[c].y, w = cells.cell[c].w;
          bool bon[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const bool in = xb[j] == (uint32_t)cy && cb[j] != 0xFFu;
            bon[j] = __builtin_amdgcn_ballot_w64(in) != 0;
            // rows outside the cell: zero codes and a neutral scale (their
            // shifted code could reach the NaN exponent)
            const float fs = in ? __uint_as_float((uint32_t)((int)cb[j] + w) << 23) : 1.f;
            b0[j] = decode8_bf16<BFMT>(in ? make_uint2(qb[j].x, qb[j].y) : make_uint2(0u, 0u), fs);
            b1[j] = decode8_bf16<BFMT>(in ? make_uint2(qb[j].z, qb[j].w) : make_uint2(0u, 0u), fs);
          }
#pragma unroll
          for (int f = 0; f < 4; ++f) {
            const bool in = xa[f] == (uint32_t)cx && ca[f] != 0xFFu;
            if (__builtin_amdgcn_ballot_w64(in) == 0) continue;
            const float fs = in ? __uint_as_float((uint32_t)((int)ca[f] - w) << 23) : 1.f;
            const v8bf16 a0 = decode8_bf16<AFMT>(in ? make_uint2(qa[f].x, qa[f].y) : make_uint2(0u, 0u), fs);
            const v8bf16 a1 = decode8_bf16<AFMT>(in ? make_uint2(qa[f].z, qa[f].w) : make_uint2(0u, 0u), fs);
#pragma unroll
            for (int j = 0; j < 4; ++j)
              if (bon[j]) {
                acc[f][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b0[j], a0, acc[f][j], 0, 0, 0);
                acc[f][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b1[j], a1, acc[f][j], 0, 0, 0);
              }
          }
        }
      }
    }
  }

  // ---- the next tile's first loads go out before this tile's stores,
  // once every wave is done with both LDS buffers
  const int64_t em0 = m0, en0 = n0;
  if (has_next) {
    wait_lgkmcnt0();
    barrier();
    bid += gridDim.x;
    tile_m = ntm;
    tile_n = ntn;
    m0 = (int64_t)tile_m * kFBM;
    n0 = (int64_t)tile_n * kFBN;
    a_base = uniform_ptr(A + m0 * g.lda);
    b_base = uniform_ptr(B + n0 * g.ldb);
    sa_base = uniform_ptr(SA + m0 * g.ldsa);
    sb_base = uniform_ptr(SB + n0 * g.ldsb);
    pf_off = pfn_off;
    issue_scales(0);
    issue_codes(0, 0);
    issue_codes(1, 1);
    issue_pf(min((int64_t)3, last));
  }

  // ---- epilogue: lane owns y[m][n .. n+3] for 4 groups of n
  uint8_t* Y = (uint8_t*)g.y + (po * g.sy_o + pi * g.sy_i) * (BF16OUT ? 2 : 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t m = em0 + wm * 128 + i * 32 + lr;
#pragma unroll
    for (int j = 0; j < 4; ++j) store_tile32<BF16OUT>(g, Y, acc[i][j], m, m < m_end, en0 + wn * 128 + j * 32, lg);
  }
  if (!has_next) break;

  // ---- next tile: its first loads and this tile's stores (loads and
  // stores share one counter and may complete out of order) have landed
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
  needs_exact = false;
  wait_vmcnt<0>();
  barrier();
  read_first();
  }  // tiles
}

template <int MODE>
mx_status_t launch_big(const GemmArgs& g, mx_fmt_t af, mx_fmt_t bf, bool bf16out, int64_t batch, hipStream_t st) {
  // The FP8 and FP4 modes walk the tiles with one work-group per CU (each
  // computing every gridDim.x-th tile, which keeps the XCD bands when the
  // CU count is a multiple of 8) when every tile is whole and there is one
  // batch entry -- the same condition the kernel tests; otherwise one tile
  // per work-group.
  uint32_t wgs = g.tiles_m * g.tiles_n;
  if (MODE != kModeBF16 && g.group_off == nullptr && batch == 1 && g.M % kFBM == 0 && g.N % kFBN == 0) {
    const int cus = mx_host::cu_count();
    if (cus >= 8 && cus % 8 == 0 && (uint32_t)cus < wgs) wgs = (uint32_t)cus;
  }
  const dim3 grid(wgs, (uint32_t)batch);
#define MX_BIG_LAUNCH(AF, BF, OUT) \
  hipLaunchKernelGGL((gemm_big_kernel<AF, BF, OUT, MODE>), grid, dim3(kThreads), 0, st, g)
#define MX_BIG_OUT(AF, BF) \
  do { if (bf16out) MX_BIG_LAUNCH(AF, BF, true); else MX_BIG_LAUNCH(AF, BF, false); } while (0)
  if constexpr (MODE == kModeFP4) {
    MX_BIG_OUT(MX_E2M1, MX_E2M1);
  } else {
    if (af == MX_E4M3 && bf == MX_E4M3) MX_BIG_OUT(MX_E4M3, MX_E4M3);
    else if (af == MX_E5M2 && bf == MX_E4M3) MX_BIG_OUT(MX_E5M2, MX_E4M3);
    else if (af == MX_E4M3 && bf == MX_E5M2) MX_BIG_OUT(MX_E4M3, MX_E5M2);
    else MX_BIG_OUT(MX_E5M2, MX_E5M2);
  }
#undef MX_BIG_OUT
#undef MX_BIG_LAUNCH
  return mx_host::launch_status();
}

template <bool PAGED>
mx_status_t launch_rowpanel(const GemmArgs& g, mx_fmt_t af, mx_fmt_t bf, bool bf16out, int64_t batch, hipStream_t st) {
  const int64_t row_blocks = (g.M + kRPRows - 1) / kRPRows;
  if (row_blocks * batch >= ((int64_t)1 << 31)) return MX_ERR_SHAPE;
  const dim3 grid((uint32_t)(row_blocks * batch));
  const uint32_t rbs = (uint32_t)row_blocks, np = (uint32_t)batch;
#define MX_RP_LAUNCH(AF, BF, OUT) \
  hipLaunchKernelGGL((gemm_rowpanel_kernel<AF, BF, OUT, PAGED>), grid, dim3(kThreads), 0, st, g, rbs, np)
#define MX_RP_OUT(AF, BF) \
  do { if (bf16out) MX_RP_LAUNCH(AF, BF, true); else MX_RP_LAUNCH(AF, BF, false); } while (0)
  if (af == MX_E4M3 && bf == MX_E4M3) MX_RP_OUT(MX_E4M3, MX_E4M3);
  else if (af == MX_E5M2 && bf == MX_E4M3) MX_RP_OUT(MX_E5M2, MX_E4M3);
  else if (af == MX_E4M3 && bf == MX_E5M2) MX_RP_OUT(MX_E4M3, MX_E5M2);
  else MX_RP_OUT(MX_E5M2, MX_E5M2);
#undef MX_RP_OUT
#undef MX_RP_LAUNCH
  return mx_host::launch_status();
}

template <int BM, int BN, bool PAGED, int MODE>
mx_status_t launch(const GemmArgs& g, mx_fmt_t af, mx_fmt_t bf, bool bf16out, int64_t batch, hipStream_t st) {
  const dim3 grid(g.tiles_m * g.tiles_n, (uint32_t)batch);
#define MX_GEMM_LAUNCH(AF, BF, OUT) \
  hipLaunchKernelGGL((gemm_kernel<BM, BN, AF, BF, OUT, PAGED, MODE>), grid, dim3(kThreads), 0, st, g)
#define MX_GEMM_OUT(AF, BF) \
  do { if (bf16out) MX_GEMM_LAUNCH(AF, BF, true); else MX_GEMM_LAUNCH(AF, BF, false); } while (0)
  // E2M1 operands, alone or against an FP8 format
  if (af == MX_E2M1 || bf == MX_E2M1) {
    if (af == MX_E2M1 && bf == MX_E2M1) MX_GEMM_OUT(MX_E2M1, MX_E2M1);
    else if (af == MX_E2M1 && bf == MX_E4M3) MX_GEMM_OUT(MX_E2M1, MX_E4M3);
    else if (af == MX_E2M1) MX_GEMM_OUT(MX_E2M1, MX_E5M2);
    else if (af == MX_E4M3) MX_GEMM_OUT(MX_E4M3, MX_E2M1);
    else MX_GEMM_OUT(MX_E5M2, MX_E2M1);
    return mx_host::launch_status();
  }
  if (af == MX_E4M3 && bf == MX_E4M3) MX_GEMM_OUT(MX_E4M3, MX_E4M3);
  else if (af == MX_E5M2 && bf == MX_E4M3) MX_GEMM_OUT(MX_E5M2, MX_E4M3);
  else if (af == MX_E4M3 && bf == MX_E5M2) MX_GEMM_OUT(MX_E4M3, MX_E5M2);
  else MX_GEMM_OUT(MX_E5M2, MX_E5M2);
#undef MX_GEMM_OUT
#undef MX_GEMM_LAUNCH
  return mx_host::launch_status();
}

}  // namespace

extern "C" mx_status_t mx_gemm(const mx_gemm_desc_t* d, hipStream_t stream) {
  if (!d) return MX_ERR_NULL;
  auto known = [](mx_fmt_t f) { return f == MX_E4M3 || f == MX_E5M2 || f == MX_E2M1; };
  if (!known(d->a_fmt) || !known(d->b_fmt)) return MX_ERR_FORMAT;
  // an E2M1 operand: MXFP4 x MXFP4, or against E4M3 / E5M2
  const bool e2m1 = d->a_fmt == MX_E2M1 || d->b_fmt == MX_E2M1;
  const bool fp4 = d->a_fmt == MX_E2M1 && d->b_fmt == MX_E2M1;
  if (d->y_dtype != MX_F32 && d->y_dtype != MX_BF16) return MX_ERR_FORMAT;
  const int64_t M = d->M, N = d->N, K = d->K;
  if (M < 0 || N < 0 || K < 0 || K % kBlock != 0) return MX_ERR_SHAPE;
  const int64_t bo = d->batch_outer > 0 ? d->batch_outer : 1;
  const int64_t bi = d->batch_inner > 0 ? d->batch_inner : 1;
  if (d->batch_outer < 0 || d->batch_inner < 0) return MX_ERR_SHAPE;
  const bool paged = d->b_page_table != nullptr;
  if (M == 0 || N == 0) return mx_host::check_device();
  if (!d->y) return MX_ERR_NULL;
  if (K > 0 && (!d->a || !d->b || !d->sa || !d->sb)) return MX_ERR_NULL;
  // code bytes per operand row
  const int64_t arow = d->a_fmt == MX_E2M1 ? K / 2 : K, brow = d->b_fmt == MX_E2M1 ? K / 2 : K;
  if (d->lda < arow || d->ldb < brow || d->ldsa < K / kBlock || d->ldsb < K / kBlock || d->ldy < N)
    return MX_ERR_SHAPE;
  if (paged && (d->b_page_rows <= 0 || d->b_pages_per_seq <= 0 || (N + d->b_page_rows - 1) / d->b_page_rows > d->b_pages_per_seq))
    return MX_ERR_SHAPE;
  if (d->accum != MX_ACCUM_AUTO && d->accum != MX_ACCUM_FP8 && d->accum != MX_ACCUM_FP32) return MX_ERR_FORMAT;
  const int64_t ysz = d->y_dtype == MX_F32 ? 4 : 2;
  if (!mx_host::aligned16(d->a) || !mx_host::aligned16(d->b) || d->lda % 16 || d->ldb % 16 ||
      ((uintptr_t)d->y % ysz) != 0)
    return MX_ERR_ALIGN;
  if (d->stride_a_outer % 16 || d->stride_a_inner % 16 || d->stride_b_inner % 16 || (!paged && d->stride_b_outer % 16) ||
      (paged && d->b_page_stride % 16))
    return MX_ERR_ALIGN;
  mx_status_t st;
  if ((st = mx_host::check_device()) != MX_OK) return st;
  if (bo * bi >= 65536) return MX_ERR_SHAPE;

  GemmArgs g{};
  g.M = M; g.N = N; g.K = K;
  g.a = d->a; g.lda = d->lda; g.sa = d->sa; g.ldsa = d->ldsa;
  g.b = d->b; g.ldb = d->ldb; g.sb = d->sb; g.ldsb = d->ldsb;
  g.y = d->y; g.ldy = d->ldy;
  g.batch_inner = bi;
  g.sa_o = d->stride_a_outer; g.sa_i = d->stride_a_inner; g.ssa_o = d->stride_sa_outer; g.ssa_i = d->stride_sa_inner;
  g.sb_o = d->stride_b_outer; g.sb_i = d->stride_b_inner; g.ssb_o = d->stride_sb_outer; g.ssb_i = d->stride_sb_inner;
  g.sy_o = d->stride_y_outer; g.sy_i = d->stride_y_inner;
  g.page_table = d->b_page_table; g.pages_per_seq = d->b_pages_per_seq; g.page_rows = d->b_page_rows;
  // the divider serves row indices below 2^30, for which a page of 2^30 rows
  // or more splits the same way as the real page size
  if (paged) g.page_div = FastDiv::make((uint32_t)std::min<int64_t>(d->b_page_rows, (int64_t)1 << 30));
  g.page_stride = d->b_page_stride; g.page_stride_s = d->b_page_stride_s;
  // dword scale reads need 4-byte aligned scale rows in every problem and page
  const bool sa4 = ((uintptr_t)d->sa % 4 == 0) && d->ldsa % 4 == 0 && d->stride_sa_outer % 4 == 0 && d->stride_sa_inner % 4 == 0;
  const bool sb4 = ((uintptr_t)d->sb % 4 == 0) && d->ldsb % 4 == 0 && d->stride_sb_inner % 4 == 0 &&
                   (paged ? d->b_page_stride_s % 4 == 0 : d->stride_sb_outer % 4 == 0);
  g.scales_dword = (sa4 && sb4) ? 1u : 0u;
  g.y_vec = (mx_host::aligned16(d->y) && (d->ldy * ysz) % 16 == 0 && (d->stride_y_outer * ysz) % 16 == 0 &&
             (d->stride_y_inner * ysz) % 16 == 0) ? 1u : 0u;
  // MX_ACCUM_AUTO is the FP32-accumulation mode (the scaled FP8 instruction
  // meets 1e-5 * sum|a b| only on data whose errors cancel, see mx_accum_t),
  // except for MXFP4 x MXFP4, where the instruction is exact
  const bool fp8 = d->accum == MX_ACCUM_FP8 || (d->accum == MX_ACCUM_AUTO && fp4);

  constexpr int BM = 128, BN = 128;
  g.tiles_m = (uint32_t)((M + BM - 1) / BM);
  g.tiles_n = (uint32_t)((N + BN - 1) / BN);
  if ((int64_t)g.tiles_m * g.tiles_n >= ((int64_t)1 << 31)) return MX_ERR_SHAPE;
  const bool bf16out = d->y_dtype == MX_BF16;
  // large aligned problems: the 256 x 256 pipelined kernel (either mode)
  const bool big_ok = !paged && K % (fp4 ? 1024 : 512) == 0 && K > 0 && d->lda % 16 == 0 && d->ldb % 16 == 0 &&
                      mx_host::aligned16(d->sa) && mx_host::aligned16(d->sb) && d->ldsa % 16 == 0 &&
                      d->ldsb % 16 == 0 && d->stride_sa_outer % 16 == 0 && d->stride_sa_inner % 16 == 0 &&
                      d->stride_sb_outer % 16 == 0 && d->stride_sb_inner % 16 == 0 && M >= 256 && N >= 256 &&
                      (M * d->lda) < ((int64_t)1 << 32) && (N * d->ldb) < ((int64_t)1 << 32);
  // MXFP4 x MXFP4 on the scaled instruction on the large-tile kernel where
  // it fits; every other product with an E2M1 operand on the general kernel
  if (big_ok && (!e2m1 || (fp4 && fp8))) {
    GemmArgs gb = g;
    gb.tiles_m = (uint32_t)((M + kFBM - 1) / kFBM);
    gb.tiles_n = (uint32_t)((N + kFBN - 1) / kFBN);
    if (fp4) return launch_big<kModeFP4>(gb, d->a_fmt, d->b_fmt, bf16out, bo * bi, stream);
    return fp8 ? launch_big<kModeFP8>(gb, d->a_fmt, d->b_fmt, bf16out, bo * bi, stream)
               : launch_big<kModeBF16>(gb, d->a_fmt, d->b_fmt, bf16out, bo * bi, stream);
  }
  // short reductions with at most 512 B rows: the row-panel kernel
  const bool rowpanel_ok = !fp8 && !e2m1 && K <= kBK && N <= kRPMaxN && d->lda % 8 == 0 && d->ldb % 16 == 0 &&
                           (paged ? d->b_page_stride % 16 == 0 : d->stride_b_outer % 16 == 0) &&
                           d->stride_b_inner % 16 == 0 && d->stride_a_outer % 8 == 0 && d->stride_a_inner % 8 == 0;
  if (rowpanel_ok)
    return paged ? launch_rowpanel<true>(g, d->a_fmt, d->b_fmt, bf16out, bo * bi, stream)
                 : launch_rowpanel<false>(g, d->a_fmt, d->b_fmt, bf16out, bo * bi, stream);
  if (fp8)
    return paged ? launch<BM, BN, true, kModeFP8>(g, d->a_fmt, d->b_fmt, bf16out, bo * bi, stream)
                 : launch<BM, BN, false, kModeFP8>(g, d->a_fmt, d->b_fmt, bf16out, bo * bi, stream);
  return paged ? launch<BM, BN, true, kModeBF16>(g, d->a_fmt, d->b_fmt, bf16out, bo * bi, stream)
               : launch<BM, BN, false, kModeBF16>(g, d->a_fmt, d->b_fmt, bf16out, bo * bi, stream);
}

extern "C" mx_status_t mx_grouped_gemm(const mx_grouped_gemm_desc_t* d, hipStream_t stream) {
  if (!d) return MX_ERR_NULL;
  const bool fp4 = d->a_fmt == MX_E2M1 || d->b_fmt == MX_E2M1;
  if (fp4) {
    if (d->a_fmt != MX_E2M1 || d->b_fmt != MX_E2M1 || d->accum == MX_ACCUM_FP32) return MX_ERR_FORMAT;
  } else {
    if (d->a_fmt != MX_E4M3 && d->a_fmt != MX_E5M2) return MX_ERR_FORMAT;
    if (d->b_fmt != MX_E4M3 && d->b_fmt != MX_E5M2) return MX_ERR_FORMAT;
  }
  if (d->y_dtype != MX_F32 && d->y_dtype != MX_BF16) return MX_ERR_FORMAT;
  if (d->accum != MX_ACCUM_AUTO && d->accum != MX_ACCUM_FP8 && d->accum != MX_ACCUM_FP32) return MX_ERR_FORMAT;
  const int64_t G = d->groups, M = d->total_m, N = d->N, K = d->K;
  if (G < 0 || M < 0 || N < 0 || K <= 0 || G >= ((int64_t)1 << 20)) return MX_ERR_SHAPE;
  if (G == 0 || M == 0 || N == 0) return mx_host::check_device();
  if (!d->group_offsets || !d->a || !d->sa || !d->b || !d->sb || !d->y) return MX_ERR_NULL;
  const int64_t krow = fp4 ? K / 2 : K;
  if (K % (fp4 ? 1024 : 512) != 0 || N < 256 || d->lda < krow || d->ldb < krow || d->ldsa < K / kBlock ||
      d->ldsb < K / kBlock || d->ldy < N || d->stride_b < N * d->ldb || d->stride_sb < N * d->ldsb ||
      d->lda >= ((int64_t)1 << 24) || d->ldb >= ((int64_t)1 << 24))
    return MX_ERR_SHAPE;
  const int64_t ysz = d->y_dtype == MX_F32 ? 4 : 2;
  if (!mx_host::aligned16(d->a) || !mx_host::aligned16(d->b) || d->lda % 16 || d->ldb % 16 || d->stride_b % 16 ||
      !mx_host::aligned16(d->sa) || !mx_host::aligned16(d->sb) || d->ldsa % 16 || d->ldsb % 16 ||
      d->stride_sb % 16 || ((uintptr_t)d->y % ysz) != 0 || ((uintptr_t)d->group_offsets % 8) != 0)
    return MX_ERR_ALIGN;
  mx_status_t st;
  if ((st = mx_host::check_device()) != MX_OK) return st;

  GemmArgs g{};
  g.M = M; g.N = N; g.K = K;
  g.a = d->a; g.lda = d->lda; g.sa = d->sa; g.ldsa = d->ldsa;
  g.b = d->b; g.ldb = d->ldb; g.sb = d->sb; g.ldsb = d->ldsb;
  g.y = d->y; g.ldy = d->ldy;
  g.batch_inner = 1;
  g.sb_o = d->stride_b; g.ssb_o = d->stride_sb;  // per group; A and y rows are absolute
  g.group_off = d->group_offsets;
  g.groups = (uint32_t)G;
  g.scales_dword = 1;
  g.y_vec = (mx_host::aligned16(d->y) && (d->ldy * ysz) % 16 == 0) ? 1u : 0u;
  g.tiles_n = (uint32_t)((N + kFBN - 1) / kFBN);
  // every group adds at most one partial row tile
  const int64_t tiles_m = (M + kFBM - 1) / kFBM + G;
  if (tiles_m * g.tiles_n >= ((int64_t)1 << 31)) return MX_ERR_SHAPE;
  g.tiles_m = (uint32_t)tiles_m;
  const bool bf16out = d->y_dtype == MX_BF16;
  if (fp4) return launch_big<kModeFP4>(g, d->a_fmt, d->b_fmt, bf16out, 1, stream);
  const bool fp8 = d->accum == MX_ACCUM_FP8;
  return fp8 ? launch_big<kModeFP8>(g, d->a_fmt, d->b_fmt, bf16out, 1, stream)
             : launch_big<kModeBF16>(g, d->a_fmt, d->b_fmt, bf16out, 1, stream);
}
