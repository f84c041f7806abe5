// quantize.hip -- MXFP8 quantization kernels for gfx950:
//   rowwise (1 x 32 blocks), the fused paged KV-cache write, and colwise
//   (32 x 1 blocks, stored transposed through an LDS tile). The rowwise
//   kernel also writes MXFP4 (E2M1 codes, two per byte) [NVFP4 §2.4, §5.5].
//
// Method [MXFP8 SM120 software support, §0.1-§0.2; MXFP8 quantization
// glossary]: each block of 32 consecutive values gets one E8M0 scale chosen
// from its amax, X = 2^(floor(log2 amax) - emax_elem), and every element is
// rounded to nearest-even FP8 of x / X, saturating at the largest finite
// value. All three kernels are HBM-bound: they read the input once with
// 16-byte loads and write codes with 8- or 16-byte stores.
#include "mx_common.hpp"

namespace {

using namespace mx;

constexpr int kThreads = 256;
constexpr int kRowUnroll = 2;  // 8-element chunks per thread in the rowwise kernel

// ---------------------------------------------------------------------------
// Rowwise. One thread handles chunks of 8 consecutive elements; the 4 lanes
// of a quad hold one 32-element block, reduce its amax with two DPP steps,
// convert with the scaled-FP8 instruction and store 8 codes each. Chunk g of
// a workgroup pass maps to row = g / (cols/8), chunk-in-row = g % (cols/8).
// ---------------------------------------------------------------------------
struct RowArgs {
  const void* x;      // input base
  uint8_t* q;         // codes base
  uint8_t* s;         // scales base
  int64_t ldx, ldq, lds;
  uint32_t nchunks;   // rows * cols / 8 of this launch (< 2^31)
  FastDiv per_row;    // divide by cols / 8
  // fused KV write: a row is (token, head); src/dst rows are remapped
  const int64_t* slot_mapping;
  FastDiv heads;      // divide by H
  int64_t ld_token;   // elements between tokens
  int64_t head_dim;   // D
  int64_t capacity;   // page_size * num_pages
  const void* x2;     // second tensor (V) for the fused KV write
  uint8_t* q2;
  uint8_t* s2;
  uint32_t round_up;  // 1: the round-up scale rule (see scale_code_bits)
};

template <typename InT>
struct Chunk;  // 8 input elements as raw words
template <>
struct Chunk<uint16_t> { uint4 w; };
template <>
struct Chunk<float> { uint4 w0, w1; };

template <typename InT>
__device__ __forceinline__ void load_chunk(Chunk<InT>& c, const InT* p) {
  if constexpr (sizeof(InT) == 2) {
    c.w = *(const uint4*)p;
  } else {
    c.w0 = *(const uint4*)p;
    c.w1 = *(const uint4*)(p + 4);
  }
}

// |x| bit patterns' maximum over the 8 elements (bf16: 16-bit field, f32: 31-bit)
template <typename InT>
__device__ __forceinline__ uint32_t chunk_amax_bits(const Chunk<InT>& c) {
  if constexpr (sizeof(InT) == 2) {
    uint32_t m = pk_max_u16(pk_max_u16(c.w.x & 0x7FFF7FFFu, c.w.y & 0x7FFF7FFFu),
                            pk_max_u16(c.w.z & 0x7FFF7FFFu, c.w.w & 0x7FFF7FFFu));
    return umax(m & 0xFFFFu, m >> 16);
  } else {
    uint32_t a = umax(umax(c.w0.x & 0x7FFFFFFFu, c.w0.y & 0x7FFFFFFFu), umax(c.w0.z & 0x7FFFFFFFu, c.w0.w & 0x7FFFFFFFu));
    uint32_t b = umax(umax(c.w1.x & 0x7FFFFFFFu, c.w1.y & 0x7FFFFFFFu), umax(c.w1.z & 0x7FFFFFFFu, c.w1.w & 0x7FFFFFFFu));
    return umax(a, b);
  }
}

template <typename InT, int FMT>
__device__ __forceinline__ uint2 encode_chunk(const Chunk<InT>& c, float div) {
  if constexpr (sizeof(InT) == 2) {
    return make_uint2(encode4_bf16<FMT>(c.w.x, c.w.y, div), encode4_bf16<FMT>(c.w.z, c.w.w, div));
  } else {
    return make_uint2(encode4_f32<FMT>(__uint_as_float(c.w0.x), __uint_as_float(c.w0.y), __uint_as_float(c.w0.z),
                                       __uint_as_float(c.w0.w), div),
                      encode4_f32<FMT>(__uint_as_float(c.w1.x), __uint_as_float(c.w1.y), __uint_as_float(c.w1.z),
                                       __uint_as_float(c.w1.w), div));
  }
}

template <typename InT, int FMT, bool KV>
__global__ __launch_bounds__(kThreads) void quant_rows_kernel(RowArgs a) {
  const InT* x = (const InT*)a.x;
  uint8_t* q = a.q;
  uint8_t* s = a.s;
  if (KV && blockIdx.y == 1) {
    x = (const InT*)a.x2;
    q = a.q2;
    s = a.s2;
  }
  const uint32_t base = blockIdx.x * (kThreads * kRowUnroll) + threadIdx.x;
  Chunk<InT> c[kRowUnroll];
  int64_t dst_row[kRowUnroll];
  uint32_t col8[kRowUnroll];
  bool ok[kRowUnroll];
#pragma unroll
  for (int u = 0; u < kRowUnroll; ++u) {
    const uint32_t g = base + u * kThreads;
    ok[u] = g < a.nchunks;
    const uint32_t row = a.per_row.div(g);
    col8[u] = g - row * a.per_row.d;
    int64_t src;
    if (KV) {
      const uint32_t t = a.heads.div(row);
      const uint32_t h = row - t * a.heads.d;
      int64_t slot = ok[u] ? a.slot_mapping[t] : -1;
      ok[u] = ok[u] && slot >= 0 && slot < a.capacity;
      src = (int64_t)t * a.ld_token + (int64_t)h * a.head_dim;
      dst_row[u] = slot * (int64_t)a.heads.d + h;
    } else {
      src = (int64_t)row * a.ldx;
      dst_row[u] = row;
    }
    if (ok[u]) load_chunk<InT>(c[u], x + src + (int64_t)col8[u] * 8);
  }
#pragma unroll
  for (int u = 0; u < kRowUnroll; ++u) {
    // whole quads share `ok` (cols % 32 == 0 and the chunk base is quad aligned)
    if (!ok[u]) continue;
    const uint32_t amax = quad_max_u32(chunk_amax_bits<InT>(c[u]));
    const uint32_t code = scale_code_bits<FMT, sizeof(InT) == 2 ? 7 : 23>(amax, a.round_up);
    const int64_t ldq = KV ? a.head_dim : a.ldq;
    const int64_t lds = KV ? a.head_dim / kBlock : a.lds;
    if constexpr (FMT == MX_E2M1) {
      // MXFP4: the 8 codes of the chunk are one dword (a NaN block gets 0s)
      uint32_t out;
      if constexpr (sizeof(InT) == 2) out = encode8_fp4_bf16(c[u].w, scale_divisor(code));
      else out = encode8_fp4_f32(c[u].w0, c[u].w1, scale_divisor(code));
      if (code == 0xFFu) out = 0u;
      *(uint32_t*)(q + dst_row[u] * ldq + (int64_t)col8[u] * 4) = out;
    } else {
      uint2 out = encode_chunk<InT, FMT>(c[u], scale_divisor(code));
      if (code == 0xFFu) out = make_uint2(0x7F7F7F7Fu, 0x7F7F7F7Fu);
      *(uint2*)(q + dst_row[u] * ldq + (int64_t)col8[u] * 8) = out;
    }
    if ((threadIdx.x & 3) == 0) s[dst_row[u] * lds + col8[u] / 4] = (uint8_t)code;
  }
}

// ---------------------------------------------------------------------------
// Colwise. A workgroup owns a 128-row x 128-column tile; wave w takes the
// 32-row block row w. Lane j takes the 8 columns 8*(j/4) .. +7 and the 8 rows
// 8*(j%4) .. +7, so one load instruction covers 4 rows x 16 column groups
// (256 contiguous bytes of bf16 per row) and a column's 32 values sit in the
// 4 lanes of a quad (two DPP steps reduce the amax). The codes of a column
// (8 per lane) go to an LDS tile [128 columns][128 bytes] and leave as
// 128-byte rows of the transposed output; the 4 scales of a column (one per
// block row) are gathered in LDS and leave as one 4-byte store. With few
// column tiles the tiles are ordered along the rows of x: the work-groups in
// flight then read whole rows and still write long runs of each output row.
// From 64 column tiles on they are ordered down the columns, which keeps the
// output rows' runs long (16384 x 14336: 158 -> 147 us; with 32 column tiles
// this order measured 8-17 % slower).
//
// B2D: two-dimensional blocks, one scale per 32 x 32 block [SM120 §1.3]. The
// 16 lanes of a DPP row hold one whole block (4 column groups x 4 row
// groups), so the block's amax is a 16-lane reduction and every column of the
// block takes that code. The tile's transposed codes leave as above (qt may be
// NULL), and the rowwise codes are encoded a second time along the rows and
// stored straight from registers: each store instruction writes 4 rows x 128
// contiguous bytes. The rowwise scales are 4 bytes per row (q may be NULL).
//
// ROWS: 1-D blocks in both orientations from one read of x. The colwise
// output is as above; a row's 32-column block lies in the 4 lanes j, j ^ 4,
// j ^ 8, j ^ 12 of a DPP row (the same row group, 4 column groups), so each
// of a lane's 8 rows gets its block amax from two lane exchanges, and its 8
// codes are encoded along the row and stored from registers as with B2D.
// ---------------------------------------------------------------------------
constexpr int kColTileRows = 128;
constexpr int kColTileCols = 128;

// LDS byte offset of row byte `rbyte` of column `c`: the 16-byte chunk index
// is XORed with 2 * (c / 8), which keeps both the 8-byte writes (16 lanes:
// 4 column groups x 4 row groups) and the 16-byte row reads free of bank
// conflicts.
__device__ __forceinline__ uint32_t col_lds_offset(uint32_t c, uint32_t rbyte) {
  return c * 128u + ((((rbyte >> 4) ^ (2u * (c >> 3))) & 7u) << 4) + (rbyte & 15u);
}

template <typename InT, int FMT, bool B2D, bool ROWS>
__global__ __launch_bounds__(kThreads) void quant_cols_kernel(const InT* __restrict__ x, int64_t rows, int64_t cols,
                                                              int64_t ldx, uint8_t* __restrict__ qt, int64_t ldq,
                                                              uint8_t* __restrict__ st, int64_t lds,
                                                              uint32_t col_tiles, uint32_t col_major, uint32_t round_up,
                                                              uint8_t* __restrict__ q2, int64_t ldq2,
                                                              uint8_t* __restrict__ s2, int64_t lds2) {
  __shared__ __attribute__((aligned(16))) uint8_t tile[kColTileCols * kColTileRows];
  __shared__ __attribute__((aligned(16))) uint8_t stile[kColTileCols * 4];
  // rowwise scales of the tile's 128 rows x 4 blocks (B2D / ROWS with the
  // transposed output, whose barrier publishes them): one 4-byte store per row
  __shared__ __attribute__((aligned(16))) uint8_t rstile[(B2D || ROWS) ? kColTileRows * 4 : 4];
  // (only when the rowwise output is asked for: a colwise-only call has s2 == NULL)
  const bool rs_lds = (B2D || ROWS) && qt != nullptr && s2 != nullptr;
  const uint32_t row_tiles = gridDim.x / col_tiles;  // the grid is row_tiles x col_tiles
  const uint32_t tile_r = col_major ? blockIdx.x % row_tiles : blockIdx.x / col_tiles;
  const uint32_t tile_c = col_major ? blockIdx.x / row_tiles : blockIdx.x % col_tiles;
  const int64_t r0 = (int64_t)tile_r * kColTileRows, c0 = (int64_t)tile_c * kColTileCols;
  const uint32_t wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const uint32_t k = lane >> 2, b = lane & 3;
  const int64_t rblk = r0 + 32 * wave;   // first row of this wave's block row
  const bool wave_ok = rblk < rows;      // rows % 32 == 0
  const int64_t cc = c0 + 8 * k;         // first of this lane's 8 columns
  const int ncol = cols - cc >= 8 ? 8 : (cols > cc ? (int)(cols - cc) : 0);

  if (wave_ok) {
    // v[i][p]: row 8b+i, column pair p (bf16) or column p (f32)
    constexpr int W = sizeof(InT) == 2 ? 4 : 8;
    uint32_t v[8][W];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const InT* p = x + (rblk + 8 * b + i) * ldx + cc;
      if (ncol == 8) {
        uint4 t = *(const uint4*)p;
        v[i][0] = t.x; v[i][1] = t.y; v[i][2] = t.z; v[i][3] = t.w;
        if constexpr (W == 8) {
          uint4 t2 = *(const uint4*)(p + 4);
          v[i][4] = t2.x; v[i][5] = t2.y; v[i][6] = t2.z; v[i][7] = t2.w;
        }
      } else {
#pragma unroll
        for (int w = 0; w < W; ++w) v[i][w] = 0;
        for (int e = 0; e < ncol; ++e) {
          if constexpr (W == 4) {
            uint32_t h = ((const uint16_t*)p)[e];
            v[i][e >> 1] |= h << (16 * (e & 1));
          } else {
            v[i][e] = ((const uint32_t*)p)[e];
          }
        }
      }
    }
    // per-column amax over the lane's 8 rows, then over the 4 lanes of the quad
    uint32_t codes[8];
    if constexpr (B2D) {
      // block amax: the lane's 64 values, then the 16 lanes of the block
      uint32_t m = 0;
      if constexpr (W == 4) {
        uint32_t pm = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
          for (int p = 0; p < 4; ++p) pm = pk_max_u16(pm, v[i][p] & 0x7FFF7FFFu);
        m = umax(pm & 0xFFFFu, pm >> 16);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
          for (int p = 0; p < 8; ++p) m = umax(m, v[i][p] & 0x7FFFFFFFu);
      }
      const uint32_t code = scale_code_bits<FMT, W == 4 ? 7 : 23>(row16_max_u32(m), round_up);
#pragma unroll
      for (int ci = 0; ci < 8; ++ci) codes[ci] = code;
      if (q2 && ncol == 8) {  // cols % 32 == 0: a lane's 8 columns are all in or all out
        // rowwise codes: row 8b + i, columns cc .. cc + 7
        const float div = scale_divisor(code);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          uint2 o;
          if constexpr (W == 4) {
            o.x = encode4_bf16<FMT>(v[i][0], v[i][1], div);
            o.y = encode4_bf16<FMT>(v[i][2], v[i][3], div);
          } else {
            o.x = encode4_f32<FMT>(__uint_as_float(v[i][0]), __uint_as_float(v[i][1]), __uint_as_float(v[i][2]),
                                   __uint_as_float(v[i][3]), div);
            o.y = encode4_f32<FMT>(__uint_as_float(v[i][4]), __uint_as_float(v[i][5]), __uint_as_float(v[i][6]),
                                   __uint_as_float(v[i][7]), div);
          }
          if (code == 0xFFu) o = make_uint2(0x7F7F7F7Fu, 0x7F7F7F7Fu);
          *(uint2*)(q2 + (rblk + 8 * b + i) * ldq2 + cc) = o;
        }
        // rowwise scales: the first column group of each block takes its 8 rows
        if ((k & 3u) == 0u) {
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            if (rs_lds) rstile[(32 * wave + 8 * b + i) * 4 + (k >> 2)] = (uint8_t)code;
            else s2[(rblk + 8 * b + i) * lds2 + cc / kBlock] = (uint8_t)code;
          }
        }
      }
    } else if constexpr (W == 4) {
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        uint32_t m = v[0][p] & 0x7FFF7FFFu;
#pragma unroll
        for (int i = 1; i < 8; ++i) m = pk_max_u16(m, v[i][p] & 0x7FFF7FFFu);
        m = quad_max_pk_u16(m);
        codes[2 * p] = scale_code_bits<FMT, 7>(m & 0xFFFFu, round_up);
        codes[2 * p + 1] = scale_code_bits<FMT, 7>(m >> 16, round_up);
      }
    } else {
#pragma unroll
      for (int p = 0; p < 8; ++p) {
        uint32_t m = v[0][p] & 0x7FFFFFFFu;
#pragma unroll
        for (int i = 1; i < 8; ++i) m = umax(m, v[i][p] & 0x7FFFFFFFu);
        m = quad_max_u32(m);
        codes[p] = scale_code_bits<FMT, 23>(m, round_up);
      }
    }
    if constexpr (ROWS) {
      // rowwise 1-D blocks: amax of row 8b + i over the lane's 8 columns, then
      // over the 4 column groups of its 32-column block (lanes j ^ 4, j ^ 8)
      uint32_t ram[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if constexpr (W == 4) {
          uint32_t pm = pk_max_u16(pk_max_u16(v[i][0] & 0x7FFF7FFFu, v[i][1] & 0x7FFF7FFFu),
                                   pk_max_u16(v[i][2] & 0x7FFF7FFFu, v[i][3] & 0x7FFF7FFFu));
          ram[i] = umax(pm & 0xFFFFu, pm >> 16);
        } else {
          uint32_t m = 0;
#pragma unroll
          for (int p = 0; p < 8; ++p) m = umax(m, v[i][p] & 0x7FFFFFFFu);
          ram[i] = m;
        }
      }
      if constexpr (W == 4) {
        // two rows per dword for the exchanges
#pragma unroll
        for (int i = 0; i < 8; i += 2) {
          uint32_t pk = ram[i] | (ram[i + 1] << 16);
          pk = pk_max_u16(pk, (uint32_t)__shfl_xor((int)pk, 4));
          pk = pk_max_u16(pk, (uint32_t)__shfl_xor((int)pk, 8));
          ram[i] = pk & 0xFFFFu;
          ram[i + 1] = pk >> 16;
        }
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          ram[i] = umax(ram[i], (uint32_t)__shfl_xor((int)ram[i], 4));
          ram[i] = umax(ram[i], (uint32_t)__shfl_xor((int)ram[i], 8));
        }
      }
      if (ncol == 8) {  // cols % 32 == 0: a lane's 8 columns are all in or all out
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const uint32_t rc = scale_code_bits<FMT, W == 4 ? 7 : 23>(ram[i], round_up);
          const float div = scale_divisor(rc);
          uint2 o;
          if constexpr (W == 4) {
            o.x = encode4_bf16<FMT>(v[i][0], v[i][1], div);
            o.y = encode4_bf16<FMT>(v[i][2], v[i][3], div);
          } else {
            o.x = encode4_f32<FMT>(__uint_as_float(v[i][0]), __uint_as_float(v[i][1]), __uint_as_float(v[i][2]),
                                   __uint_as_float(v[i][3]), div);
            o.y = encode4_f32<FMT>(__uint_as_float(v[i][4]), __uint_as_float(v[i][5]), __uint_as_float(v[i][6]),
                                   __uint_as_float(v[i][7]), div);
          }
          if (rc == 0xFFu) o = make_uint2(0x7F7F7F7Fu, 0x7F7F7F7Fu);
          *(uint2*)(q2 + (rblk + 8 * b + i) * ldq2 + cc) = o;
          if ((k & 3u) == 0u) rstile[(32 * wave + 8 * b + i) * 4 + (k >> 2)] = (uint8_t)rc;  // ROWS: qt given
        }
      }
    }
    // encode: column c gets two dwords = rows 8b .. 8b+3 and 8b+4 .. 8b+7
    // (E2M1: one dword, the 8 codes two per byte; a NaN block gets 0s)
#pragma unroll
    for (int ci = 0; ci < 8; ++ci) {
      if constexpr (FMT == MX_E2M1) {
        const float div = scale_divisor(codes[ci]);
        uint32_t d;
        if constexpr (W == 4) {
          const int p = ci >> 1;
          const uint32_t sel = (ci & 1) ? 0x07060302u : 0x05040100u;
          d = encode8_fp4_bf16(make_uint4(__builtin_amdgcn_perm(v[1][p], v[0][p], sel),
                                          __builtin_amdgcn_perm(v[3][p], v[2][p], sel),
                                          __builtin_amdgcn_perm(v[5][p], v[4][p], sel),
                                          __builtin_amdgcn_perm(v[7][p], v[6][p], sel)), div);
        } else {
          d = encode8_fp4_f32(make_uint4(v[0][ci], v[1][ci], v[2][ci], v[3][ci]),
                              make_uint4(v[4][ci], v[5][ci], v[6][ci], v[7][ci]), div);
        }
        if (codes[ci] == 0xFFu) d = 0u;
        const uint32_t c = 8 * k + ci;
        *(uint32_t*)(tile + col_lds_offset(c, 16 * wave + 4 * b)) = d;
        if (b == 0) stile[c * 4 + wave] = (uint8_t)codes[ci];
        continue;
      }
      if (B2D && !qt) break;
      const float div = scale_divisor(codes[ci]);
      uint32_t d[2];
#pragma unroll
      for (int hgrp = 0; hgrp < 2; ++hgrp) {
        const int i0 = 4 * hgrp;
        if constexpr (W == 4) {
          const int p = ci >> 1;
          const uint32_t sel = (ci & 1) ? 0x07060302u : 0x05040100u;  // pick the high or low halves
          uint32_t r01 = __builtin_amdgcn_perm(v[i0 + 1][p], v[i0][p], sel);
          uint32_t r23 = __builtin_amdgcn_perm(v[i0 + 3][p], v[i0 + 2][p], sel);
          d[hgrp] = encode4_bf16<FMT>(r01, r23, div);
        } else {
          d[hgrp] = encode4_f32<FMT>(__uint_as_float(v[i0][ci]), __uint_as_float(v[i0 + 1][ci]),
                                     __uint_as_float(v[i0 + 2][ci]), __uint_as_float(v[i0 + 3][ci]), div);
        }
        if (codes[ci] == 0xFFu) d[hgrp] = 0x7F7F7F7Fu;
      }
      const uint32_t c = 8 * k + ci;
      *(uint2*)(tile + col_lds_offset(c, 32 * wave + 8 * b)) = make_uint2(d[0], d[1]);
      if (b == 0) stile[c * 4 + wave] = (uint8_t)codes[ci];
    }
  }
  if (B2D && !qt) return;  // uniform over the grid: rowwise output only
  __syncthreads();
  // codes: 128 columns x 128 bytes = 1024 chunks of 16 bytes (E2M1: 64
  // bytes, 512 chunks of one 32-row block each)
  constexpr uint32_t kChunks = FMT == MX_E2M1 ? kColTileRows / 32 : kColTileRows / 16;  // per column
  constexpr uint32_t kRowsPerChunk = kColTileRows / kChunks;
#pragma unroll
  for (uint32_t it = 0; it < kColTileCols * kChunks / kThreads; ++it) {
    const uint32_t id = threadIdx.x + kThreads * it;
    const uint32_t c = id / kChunks, m = id % kChunks;
    const int64_t r = r0 + kRowsPerChunk * m;
    if (c0 + c < cols && r < rows) {
      uint4 val = *(const uint4*)(tile + col_lds_offset(c, 16 * m));
      *(uint4*)(qt + (c0 + c) * ldq + (FMT == MX_E2M1 ? r / 2 : r)) = val;
    }
  }
  // rowwise scales (B2D / ROWS): row r's 4 blocks are 4 consecutive bytes of s2 row r0 + r
  if (rs_lds && threadIdx.x >= kColTileCols && r0 + (threadIdx.x - kColTileCols) < rows) {
    const uint32_t r = threadIdx.x - kColTileCols;
    const int64_t nb = min((cols - c0) / kBlock, (int64_t)4);
    uint8_t* dst = s2 + (r0 + r) * lds2 + c0 / kBlock;
    const uint32_t sv = *(const uint32_t*)(rstile + 4 * r);
    if (nb == 4 && ((uintptr_t)dst & 3u) == 0) {
      *(uint32_t*)dst = sv;
    } else {
      for (int64_t j = 0; j < nb; ++j) dst[j] = (uint8_t)(sv >> (8 * j));
    }
  }
  // scales: column c's 4 block rows are 4 consecutive bytes of st row c0 + c
  if (threadIdx.x < kColTileCols && c0 + threadIdx.x < cols) {
    const uint32_t c = threadIdx.x;
    const int64_t nb = min((rows - r0) / kBlock, (int64_t)4);
    uint8_t* dst = st + (c0 + c) * lds + r0 / kBlock;
    const uint32_t sv = *(const uint32_t*)(stile + 4 * c);
    if (nb == 4 && ((uintptr_t)dst & 3u) == 0) {
      *(uint32_t*)dst = sv;
    } else {
      for (int64_t j = 0; j < nb; ++j) dst[j] = (uint8_t)(sv >> (8 * j));
    }
  }
}

// ---------------------------------------------------------------- host side
// ---------------------------------------------------------------------------
// Scale broadcast [SM120 §1.3]: a power-of-two FP32 scale of a 128-element
// (or 128 x 128) block becomes the E8M0 code of its four 32-element blocks.
// A positive normal power of two 2^(E - 127) has code E (its exponent field);
// 2^-127 is the f32 subnormal 0x00400000 and has code 0; anything else
// (another subnormal, a significand other than 1, zero, negative, Inf, NaN)
// gets 0xFF. A thread converts 4 consecutive source scales of a row (one
// 16-byte load and one 16-byte store of 16 codes) when the rows and pitches
// allow it, else one.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t e8m0_of_pow2_bits(uint32_t b) {
  const uint32_t E = (b >> 23) & 0xFFu, m = b & 0x7FFFFFu;
  if ((b >> 31) != 0u || E == 255u) return 0xFFu;
  if (E >= 1u) return m == 0u ? E : 0xFFu;
  return m == 0x400000u ? 0u : 0xFFu;
}

template <int V>
__global__ __launch_bounds__(kThreads) void scale_bcast_kernel(const float* __restrict__ s_in, int64_t ld_in,
                                                               uint32_t layout, uint32_t n, FastDiv per_row,
                                                               uint8_t* __restrict__ out, int64_t ld_out) {
  // thread i: V consecutive source scales of one row (group cg of row r)
  const uint32_t i = blockIdx.x * kThreads + threadIdx.x;
  if (i >= n) return;
  const uint32_t r = per_row.div(i), cg = i - r * per_row.d;
  const int64_t src_row = layout ? r / 128 : r;
  const float* src = s_in + src_row * ld_in + (int64_t)V * cg;
  uint8_t* dst = out + (int64_t)r * ld_out + 4 * (int64_t)V * cg;
  if constexpr (V == 1) {
    *(uint32_t*)dst = e8m0_of_pow2_bits(__float_as_uint(*src)) * 0x01010101u;
  } else {
    const uint4 w = *(const uint4*)src;
    *(uint4*)dst = make_uint4(e8m0_of_pow2_bits(w.x) * 0x01010101u, e8m0_of_pow2_bits(w.y) * 0x01010101u,
                              e8m0_of_pow2_bits(w.z) * 0x01010101u, e8m0_of_pow2_bits(w.w) * 0x01010101u);
  }
}

mx_status_t check_common(const void* x, mx_dtype_t xdt, mx_fmt_t fmt, int64_t rows, int64_t cols, int64_t ldx) {
  if (xdt != MX_F32 && xdt != MX_BF16) return MX_ERR_FORMAT;
  if (fmt != MX_E4M3 && fmt != MX_E5M2) return MX_ERR_FORMAT;
  if (rows < 0 || cols < 0 || ldx < cols) return MX_ERR_SHAPE;
  const int64_t esz = xdt == MX_F32 ? 4 : 2;
  if (!mx_host::aligned16(x) || (ldx * esz) % 16 != 0) return MX_ERR_ALIGN;
  return MX_OK;
}

template <typename InT, int FMT, bool KV>
mx_status_t launch_rows(RowArgs a, int64_t rows, int64_t cols, hipStream_t stream) {
  // split into launches of < 2^31 chunks so chunk indices stay 32-bit
  const int64_t cpr = cols / 8;
  const int64_t rows_per_launch = std::max<int64_t>(1, ((int64_t)1 << 30) / std::max<int64_t>(cpr, 1));
  for (int64_t r0 = 0; r0 < rows; r0 += rows_per_launch) {
    const int64_t nr = std::min(rows_per_launch, rows - r0);
    RowArgs b = a;
    b.nchunks = (uint32_t)(nr * cpr);
    if (KV) {
      b.slot_mapping = a.slot_mapping + r0 / a.heads.d;  // KV launches always start at a token boundary
    } else {
      b.x = (const InT*)a.x + r0 * a.ldx;
      b.q = a.q + r0 * a.ldq;
      b.s = a.s + r0 * a.lds;
    }
    const uint32_t blocks = (b.nchunks + kThreads * kRowUnroll - 1) / (kThreads * kRowUnroll);
    hipLaunchKernelGGL((quant_rows_kernel<InT, FMT, KV>), dim3(blocks, KV ? 2 : 1), dim3(kThreads), 0, stream, b);
    if (mx_host::launch_status() != MX_OK) return MX_ERR_HIP;
  }
  return MX_OK;
}

template <typename InT>
mx_status_t dispatch_rows(mx_fmt_t fmt, RowArgs a, int64_t rows, int64_t cols, hipStream_t st) {
  if (fmt == MX_E2M1) return launch_rows<InT, MX_E2M1, false>(a, rows, cols, st);
  return fmt == MX_E5M2 ? launch_rows<InT, MX_E5M2, false>(a, rows, cols, st)
                        : launch_rows<InT, MX_E4M3, false>(a, rows, cols, st);
}

}  // namespace

namespace {
mx_status_t quantize_rows_host(const void* x, mx_dtype_t xdt, int64_t rows, int64_t cols, int64_t ldx, mx_fmt_t fmt,
                               uint8_t* q, int64_t ldq, uint8_t* s, int64_t lds, uint32_t round_up,
                               hipStream_t stream) {
  if (rows == 0 || cols == 0) {  // empty: no buffer, pitch or alignment matters
    if (rows < 0 || cols < 0) return MX_ERR_SHAPE;
    if (xdt != MX_F32 && xdt != MX_BF16) return MX_ERR_FORMAT;
    if (fmt != MX_E4M3 && fmt != MX_E5M2 && fmt != MX_E2M1) return MX_ERR_FORMAT;
    return mx_host::check_device();
  }
  if (!x || !q || !s) return MX_ERR_NULL;
  const bool fp4 = fmt == MX_E2M1;
  mx_status_t st = check_common(x, xdt, fp4 ? MX_E4M3 : fmt, rows, cols, ldx);
  if (st != MX_OK) return st;
  if (cols % kBlock != 0 || ldq < (fp4 ? cols / 2 : cols) || lds < cols / kBlock) return MX_ERR_SHAPE;
  if (!mx_host::aligned16(q) || ldq % 16 != 0) return MX_ERR_ALIGN;
  if ((st = mx_host::check_device()) != MX_OK) return st;
  if (rows == 0 || cols == 0) return MX_OK;
  RowArgs a{};
  a.x = x; a.q = q; a.s = s; a.ldx = ldx; a.ldq = ldq; a.lds = lds;
  a.round_up = round_up;
  a.per_row = FastDiv::make((uint32_t)(cols / 8));
  if (cols / 8 >= ((int64_t)1 << 30)) return MX_ERR_SHAPE;
  return xdt == MX_BF16 ? dispatch_rows<uint16_t>(fmt, a, rows, cols, stream)
                        : dispatch_rows<float>(fmt, a, rows, cols, stream);
}
}  // namespace

extern "C" mx_status_t mx_quantize(const void* x, mx_dtype_t xdt, int64_t rows, int64_t cols, int64_t ldx,
                                   mx_fmt_t fmt, uint8_t* q, int64_t ldq, uint8_t* s, int64_t lds,
                                   hipStream_t stream) {
  return quantize_rows_host(x, xdt, rows, cols, ldx, fmt, q, ldq, s, lds, 0u, stream);
}

extern "C" mx_status_t mx_kv_quant_write(const void* k, const void* v, mx_dtype_t dt, int64_t T, int64_t H, int64_t D,
                                         int64_t ld_token, const int64_t* slot_mapping, uint8_t* k_cache,
                                         uint8_t* k_scale, uint8_t* v_cache, uint8_t* v_scale, int64_t page_size,
                                         int64_t num_pages, hipStream_t stream) {
  if (T == 0 || H == 0 || D == 0) {  // empty: no buffer, pitch or alignment matters
    if (T < 0 || H < 0 || D < 0) return MX_ERR_SHAPE;
    if (dt != MX_F32 && dt != MX_BF16) return MX_ERR_FORMAT;
    return mx_host::check_device();
  }
  if (!k || !v || !slot_mapping || !k_cache || !k_scale || !v_cache || !v_scale) return MX_ERR_NULL;
  if (dt != MX_F32 && dt != MX_BF16) return MX_ERR_FORMAT;
  if (T < 0 || H < 0 || D < 0 || page_size <= 0 || num_pages < 0 || D % kBlock != 0 || ld_token < H * D)
    return MX_ERR_SHAPE;
  if (H >= ((int64_t)1 << 31) || D >= ((int64_t)1 << 31)) return MX_ERR_SHAPE;
  const int64_t esz = dt == MX_F32 ? 4 : 2;
  if (!mx_host::aligned16(k) || !mx_host::aligned16(v) || (ld_token * esz) % 16 != 0 || (D * esz) % 16 != 0 ||
      !mx_host::aligned16(k_cache) || !mx_host::aligned16(v_cache) || D % 16 != 0)
    return MX_ERR_ALIGN;
  mx_status_t st;
  if ((st = mx_host::check_device()) != MX_OK) return st;
  if (T == 0 || H == 0 || D == 0) return MX_OK;
  RowArgs a{};
  a.x = k; a.x2 = v; a.q = k_cache; a.q2 = v_cache; a.s = k_scale; a.s2 = v_scale;
  a.slot_mapping = slot_mapping;
  a.heads = FastDiv::make((uint32_t)H);
  a.per_row = FastDiv::make((uint32_t)(D / 8));
  a.ld_token = ld_token;
  a.head_dim = D;
  a.capacity = page_size * num_pages;
  // rows of the launch are (token, head) pairs; split at token boundaries
  const int64_t cpr = D / 8;
  const int64_t tok_per_launch = std::max<int64_t>(1, ((int64_t)1 << 30) / (cpr * H));
  for (int64_t t0 = 0; t0 < T; t0 += tok_per_launch) {
    const int64_t nt = std::min(tok_per_launch, T - t0);
    RowArgs b = a;
    b.x = (const uint8_t*)k + t0 * ld_token * esz;
    b.x2 = (const uint8_t*)v + t0 * ld_token * esz;
    b.slot_mapping = slot_mapping + t0;
    b.nchunks = (uint32_t)(nt * H * cpr);
    const uint32_t blocks = (b.nchunks + kThreads * kRowUnroll - 1) / (kThreads * kRowUnroll);
    if (dt == MX_BF16)
      hipLaunchKernelGGL((quant_rows_kernel<uint16_t, MX_E4M3, true>), dim3(blocks, 2), dim3(kThreads), 0, stream, b);
    else
      hipLaunchKernelGGL((quant_rows_kernel<float, MX_E4M3, true>), dim3(blocks, 2), dim3(kThreads), 0, stream, b);
    if (mx_host::launch_status() != MX_OK) return MX_ERR_HIP;
  }
  return MX_OK;
}

namespace {
mx_status_t quantize_cols_host(const void* x, mx_dtype_t xdt, int64_t rows, int64_t cols, int64_t ldx, mx_fmt_t fmt,
                               uint8_t* qt, int64_t ldq, uint8_t* st, int64_t lds, uint32_t round_up,
                               hipStream_t stream) {
  if (rows == 0 || cols == 0) {  // empty: no buffer, pitch or alignment matters
    if (rows < 0 || cols < 0) return MX_ERR_SHAPE;
    if (xdt != MX_F32 && xdt != MX_BF16) return MX_ERR_FORMAT;
    if (fmt != MX_E4M3 && fmt != MX_E5M2 && fmt != MX_E2M1) return MX_ERR_FORMAT;
    return mx_host::check_device();
  }
  if (!x || !qt || !st) return MX_ERR_NULL;
  if (fmt != MX_E4M3 && fmt != MX_E5M2 && fmt != MX_E2M1) return MX_ERR_FORMAT;
  const bool fp4 = fmt == MX_E2M1;
  mx_status_t rc = check_common(x, xdt, fp4 ? MX_E4M3 : fmt, rows, cols, ldx);
  if (rc != MX_OK) return rc;
  if (rows % kBlock != 0 || ldq < (fp4 ? rows / 2 : rows) || lds < rows / kBlock) return MX_ERR_SHAPE;
  if (!mx_host::aligned16(qt) || ldq % 16 != 0) return MX_ERR_ALIGN;
  if ((rc = mx_host::check_device()) != MX_OK) return rc;
  if (rows == 0 || cols == 0) return MX_OK;
  const int64_t row_tiles = (rows + kColTileRows - 1) / kColTileRows;
  const int64_t col_tiles = (cols + kColTileCols - 1) / kColTileCols;
  if (row_tiles * col_tiles >= ((int64_t)1 << 31)) return MX_ERR_SHAPE;
  const dim3 grid((uint32_t)(row_tiles * col_tiles));
  const uint32_t col_major = col_tiles >= 64 ? 1u : 0u;
  // With 8 work-groups per CU, grids of up to 2048 tiles are resident all at
  // once, so every work-group reads, then writes, in step with the others.
  // Unused dynamic LDS limits how many fit per CU and staggers them: 20000
  // bytes (4 per CU) measured 8192 x 4096 (2048 tiles) 25.1 -> 24.2 us,
  // 14336 x 4096 (3584) 37.7 -> 37.3 us, 16384 x 4096 (4096) 42.5 -> 42.3 us,
  // and 1.2 % slower on 16384 x 14336 (14336 tiles); 12000 bytes (5 per CU)
  // then 24.2 -> 23.5 us and 37.8 -> 37.5 us, while 3 and 6 per CU were
  // slower. The 4096-tile threshold is measured, not derived.
  const uint32_t lds_pad = row_tiles * col_tiles <= 4096 ? 12000u : 0u;
#define MX_COLS_LAUNCH(T, F)                                                                                        \
  hipLaunchKernelGGL((quant_cols_kernel<T, F, false, false>), grid, dim3(kThreads), lds_pad, stream, (const T*)x, rows, cols, ldx, \
                     qt, ldq, st, lds, (uint32_t)col_tiles, col_major, round_up, nullptr, 0, nullptr, 0)
  if (xdt == MX_BF16) {
    if (fmt == MX_E5M2) MX_COLS_LAUNCH(uint16_t, MX_E5M2);
    else if (fmt == MX_E2M1) MX_COLS_LAUNCH(uint16_t, MX_E2M1);
    else MX_COLS_LAUNCH(uint16_t, MX_E4M3);
  } else {
    if (fmt == MX_E5M2) MX_COLS_LAUNCH(float, MX_E5M2);
    else if (fmt == MX_E2M1) MX_COLS_LAUNCH(float, MX_E2M1);
    else MX_COLS_LAUNCH(float, MX_E4M3);
  }
#undef MX_COLS_LAUNCH
  return mx_host::launch_status();
}

// One pass of the tile kernel over x: 32 x 32 blocks (B2D), or 1-D blocks in
// both orientations (rows1d; both outputs given).
mx_status_t quantize_tile_host(const mx_quantize_desc_t* d, uint32_t round_up, bool rows1d, hipStream_t stream) {
  const bool rowout = d->q != nullptr, colout = d->qt != nullptr;
  if (d->fmt != MX_E4M3 && d->fmt != MX_E5M2) return MX_ERR_FORMAT;
  mx_status_t rc = check_common(d->x, d->xdt, d->fmt, d->rows, d->cols, d->ldx);
  if (rc != MX_OK) return rc;
  if (d->rows % kBlock != 0 || d->cols % kBlock != 0) return MX_ERR_SHAPE;
  if (rowout && (d->ldq < d->cols || d->lds < d->cols / kBlock)) return MX_ERR_SHAPE;
  if (colout && (d->ldqt < d->rows || d->ldst < d->rows / kBlock)) return MX_ERR_SHAPE;
  if (rowout && (!mx_host::aligned16(d->q) || d->ldq % 16 != 0)) return MX_ERR_ALIGN;
  if (colout && (!mx_host::aligned16(d->qt) || d->ldqt % 16 != 0)) return MX_ERR_ALIGN;
  if ((rc = mx_host::check_device()) != MX_OK) return rc;
  if (d->rows == 0 || d->cols == 0) return MX_OK;
  const int64_t row_tiles = (d->rows + kColTileRows - 1) / kColTileRows;
  const int64_t col_tiles = (d->cols + kColTileCols - 1) / kColTileCols;
  if (row_tiles * col_tiles >= ((int64_t)1 << 31)) return MX_ERR_SHAPE;
  const dim3 grid((uint32_t)(row_tiles * col_tiles));
  const uint32_t col_major = col_tiles >= 64 ? 1u : 0u;
  // 4 per CU here (as first measured for the colwise call): 5 per CU measured
  // 1.7 % slower on the 2-D blocks of 14336 x 4096 and no different one-pass
  const uint32_t lds_pad = row_tiles * col_tiles <= 4096 ? 20000u : 0u;
#define MX_TILE_LAUNCH(T, F, B2D, ROWS)                                                                            \
  hipLaunchKernelGGL((quant_cols_kernel<T, F, B2D, ROWS>), grid, dim3(kThreads), lds_pad, stream, (const T*)d->x, d->rows, \
                     d->cols, d->ldx, d->qt, d->ldqt, d->st, d->ldst, (uint32_t)col_tiles, col_major, round_up,  \
                     d->q, d->ldq, d->s, d->lds)
#define MX_TILE_MODE(T, F) \
  do { if (rows1d) MX_TILE_LAUNCH(T, F, false, true); else MX_TILE_LAUNCH(T, F, true, false); } while (0)
  if (d->xdt == MX_BF16) {
    if (d->fmt == MX_E5M2) MX_TILE_MODE(uint16_t, MX_E5M2); else MX_TILE_MODE(uint16_t, MX_E4M3);
  } else {
    if (d->fmt == MX_E5M2) MX_TILE_MODE(float, MX_E5M2); else MX_TILE_MODE(float, MX_E4M3);
  }
#undef MX_TILE_MODE
#undef MX_TILE_LAUNCH
  return mx_host::launch_status();
}
}  // namespace

extern "C" mx_status_t mx_quantize_colwise(const void* x, mx_dtype_t xdt, int64_t rows, int64_t cols, int64_t ldx,
                                           mx_fmt_t fmt, uint8_t* qt, int64_t ldq, uint8_t* st, int64_t lds,
                                           hipStream_t stream) {
  return quantize_cols_host(x, xdt, rows, cols, ldx, fmt, qt, ldq, st, lds, 0u, stream);
}

extern "C" mx_status_t mx_quantize_ex(const mx_quantize_desc_t* d, hipStream_t stream) {
  if (!d) return MX_ERR_NULL;
  if (d->rule != MX_SCALE_FLOOR && d->rule != MX_SCALE_CEIL) return MX_ERR_FORMAT;
  if (d->blocks != MX_BLOCKS_1D && d->blocks != MX_BLOCKS_2D) return MX_ERR_FORMAT;
  if (d->rows < 0 || d->cols < 0) return MX_ERR_SHAPE;
  if (d->rows == 0 || d->cols == 0) {  // nothing to read or write: buffers may be NULL
    if (d->xdt != MX_F32 && d->xdt != MX_BF16) return MX_ERR_FORMAT;
    if (d->fmt != MX_E4M3 && d->fmt != MX_E5M2 && (d->fmt != MX_E2M1 || d->blocks == MX_BLOCKS_2D)) return MX_ERR_FORMAT;
    return mx_host::check_device();
  }
  const bool rowout = d->q != nullptr || d->s != nullptr, colout = d->qt != nullptr || d->st != nullptr;
  if (!d->x || (!rowout && !colout)) return MX_ERR_NULL;
  if ((rowout && (!d->q || !d->s)) || (colout && (!d->qt || !d->st))) return MX_ERR_NULL;
  const uint32_t round_up = d->rule == MX_SCALE_CEIL ? 1u : 0u;
  if (d->blocks == MX_BLOCKS_2D) return quantize_tile_host(d, round_up, false, stream);
  // both 1-D orientations: one pass over x (~134 MB instead of ~203 MB of
  // traffic for an 8192 x 4096 bf16 input); x needs rows % 32 == 0 as for
  // the colwise output alone, and cols % 32 == 0 as for the rowwise one.
  // (MXFP4 takes the two single-orientation passes.)
  if (rowout && colout && d->fmt != MX_E2M1) return quantize_tile_host(d, round_up, true, stream);
  mx_status_t rc = MX_OK;
  if (rowout)
    rc = quantize_rows_host(d->x, d->xdt, d->rows, d->cols, d->ldx, d->fmt, d->q, d->ldq, d->s, d->lds, round_up, stream);
  if (rc == MX_OK && colout)
    rc = quantize_cols_host(d->x, d->xdt, d->rows, d->cols, d->ldx, d->fmt, d->qt, d->ldqt, d->st, d->ldst, round_up,
                            stream);
  return rc;
}

extern "C" mx_status_t mx_scale_broadcast(const float* s_in, int64_t ld_in, mx_bcast_layout_t layout, int64_t rows,
                                          int64_t cols, uint8_t* out, int64_t ld_out, hipStream_t stream) {
  if (layout != MX_BCAST_1X128 && layout != MX_BCAST_128X128) return MX_ERR_FORMAT;
  if (rows == 0 || cols == 0) return rows < 0 || cols < 0 ? MX_ERR_SHAPE : mx_host::check_device();  // empty
  if (!s_in || !out) return MX_ERR_NULL;
  if (rows < 0 || cols < 0 || cols % 128 != 0 || ld_in < cols / 128 || ld_out < cols / kBlock) return MX_ERR_SHAPE;
  if (((uintptr_t)s_in & 3u) != 0 || ((uintptr_t)out & 3u) != 0 || ld_out % 4 != 0) return MX_ERR_ALIGN;
  mx_status_t rc;
  if ((rc = mx_host::check_device()) != MX_OK) return rc;
  if (rows == 0 || cols == 0) return MX_OK;
  const int64_t per_row = cols / 128;
  if (rows * per_row >= ((int64_t)1 << 31)) return MX_ERR_SHAPE;
  // four source scales per thread (one 16-byte load, one 16-byte store) when
  // the rows and pitches allow it, else one
  const bool v4 = per_row % 4 == 0 && ld_in % 4 == 0 && ld_out % 16 == 0 && mx_host::aligned16(s_in) &&
                  mx_host::aligned16(out);
  const uint32_t layout_flag = layout == MX_BCAST_128X128 ? 1u : 0u;
  if (v4) {
    const int64_t n = rows * (per_row / 4);
    hipLaunchKernelGGL(scale_bcast_kernel<4>, dim3((uint32_t)((n + kThreads - 1) / kThreads)), dim3(kThreads), 0,
                       stream, s_in, ld_in, layout_flag, (uint32_t)n, FastDiv::make((uint32_t)(per_row / 4)), out,
                       ld_out);
  } else {
    const int64_t n = rows * per_row;
    hipLaunchKernelGGL(scale_bcast_kernel<1>, dim3((uint32_t)((n + kThreads - 1) / kThreads)), dim3(kThreads), 0,
                       stream, s_in, ld_in, layout_flag, (uint32_t)n, FastDiv::make((uint32_t)per_row), out, ld_out);
  }
  return mx_host::launch_status();
}
