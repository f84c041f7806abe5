// attention.hip -- paged attention over the MXFP8 KV cache (gfx950).
//
// [SM120 §0.2]: the KV cache keeps K and V as E4M3 codes with one E8M0 scale
// per 32 values along the head dimension, and the attention kernel that reads
// it forms Q K^T as a block-scaled FP8 product, turns V back into BF16 inside
// the kernel and forms P V from that. This file is that consumer for one
// MI355X:
//
//   S   = Q K^T         v_mfma_scale_f32_32x32x64_f8f6f4 on the codes, the
//                       E8M0 scales of Q and K as the instruction's operands;
//   P   = softmax(sm_scale * S) over the allowed keys, online over blocks of
//         128 keys (running max and sum in f32), rounded to bf16;
//   O   = P V           v_mfma_f32_32x32x16_bf16, V decoded to bf16 with its
//                       block scale (v_cvt_scalef32_pk_bf16_fp8) into LDS once
//                       per work-group; a key whose scales leave the range
//                       where that is exact moves part of its scale to P
//                       (v_key_shift).
//
// Work-group: 4 waves, 128 queries (32 per wave) of one (sequence, query
// head). Each wave computes S^T for its queries (keys on the instruction's
// row side, queries on the lane side), so the softmax over keys is a
// reduction inside each lane plus one exchange between the two lane halves,
// and the S^T accumulator is already the bf16 B operand of the P V product
// once converted; the contraction order over keys inside a 16-key step is
// permuted, and V^T is stored in LDS in that same order.
//
// Per block of 128 keys: K codes (16 KB) and the K and V scales (512 B each)
// arrive by direct global->LDS loads into one of two buffers; V codes come
// into registers one block ahead, and every thread decodes 64 of them (8
// keys x 8 head-dim columns of one scale block) into the shared bf16 V^T
// tile (32 KB). Each key block lies inside one page
// (page_size % 128 == 0), so the block's rows are consecutive cache slots.
#include "mx_common.hpp"

namespace {
using namespace mx;

constexpr int kHD = 128;          // head dimension
constexpr int kQT = 128;          // queries per work-group
constexpr int kKB = 128;          // keys per block
constexpr int kAttnThreads = 256; // 4 waves
constexpr uint32_t kVTRow = kKB * 2;  // bytes per V^T row (bf16)

struct AttnArgs {
  const uint8_t* q; const uint8_t* qs; int64_t ld_q, ld_qs;
  const uint8_t* kc; const uint8_t* ks; const uint8_t* vc; const uint8_t* vs;
  const int32_t* table; const int32_t* lens;
  void* out; int64_t ld_o; float* lse;
  int64_t pages_per_seq;
  uint32_t page_size, q_len, hq, hkv, group, causal, q_tiles, total_wg;
  float c2;  // sm_scale * log2(e): scores are exponentiated with exp2
};

// 16-byte chunk permutation of a 256-byte V^T row. The PV fragment reads
// touch rows 32t + r (r = 0..15 or 16..31) at one logical chunk; the
// decoder's writes touch rows 32m + 4j + i (m, j = 0..3) at one chunk. With
// chunk ^ ((row ^ (row >> 5)) & 15) both sets land on 16 distinct 16-byte
// bank groups, so neither conflicts.
__device__ __forceinline__ uint32_t vt_perm(uint32_t row) { return (row ^ (row >> 5)) & 15u; }


// Buffer resource over [base, base + bytes): loads past the end return 0.
constexpr int kBufferWord3 = 0x00020000;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kBufferWord3);
}

// V over the whole E8M0 range. code * 2^(s - 127) is an exact normal bf16
// for every finite E4M3 code when the scale code s lies in [10, 246]. A key
// whose four head-dim scales leave that window gets a shift r (v_key_shift):
// its V^T entries hold code * 2^(clamp(s - r, 10, 246) - 127) and its weight
// P_j is multiplied by 2^r, so P_j * V_jd is unchanged. r = 0 whenever the
// scales are inside the window (the usual case: a block whose scales all
// are skips the shift computation and multiplies its weights by 1);
// otherwise r is the smallest move that brings them in. Only a key whose own
// scales span more than 236 codes cannot be brought in whole: its largest
// block is kept exact and its blocks more than 2^236 below that one are
// clamped up to the window's floor.
// The NaN code 0xFF counts as outside the window; the shift ignores it and
// the decode writes its block as NaN.
constexpr int kVFoldLo = 10, kVFoldHi = 246;
__device__ __forceinline__ int v_key_shift(uint32_t w) {
  int lo = 255, hi = -1;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int s = (int)((w >> (8 * i)) & 0xFFu);
    if (s != 0xFF) {
      lo = min(lo, s);
      hi = max(hi, s);
    }
  }
  // the largest block must stay exact: r >= hi - 246; within that, lift the
  // key as far as its smallest block needs (never past 0 from above)
  return max(hi - kVFoldHi, min(lo - kVFoldLo, 0));
}
__device__ __forceinline__ uint32_t v_fold_code(uint32_t s, int r) {
  return (uint32_t)min(max((int)s - r, kVFoldLo), kVFoldHi);
}

// Work item lid -> (query tile qt, query head h, sequence s). Without a mask
// the query tiles of one (sequence, head) share its keys, so they are kept
// on one XCD (the 8 XCDs take work-groups round-robin). Under a causal mask
// the work of a tile grows with its index, so all last tiles go first, then
// the tiles before them, in plain dispatch order, which spreads every class
// of tile evenly over the XCDs.
__device__ __forceinline__ void tile_of(const AttnArgs& g, uint32_t lid, uint32_t& qt, uint32_t& h, uint32_t& s) {
  if (g.causal) {
    const uint32_t nsh = g.total_wg / g.q_tiles;  // (sequence, head) pairs
    qt = g.q_tiles - 1 - lid / nsh;
    h = (lid % nsh) % g.hq;
    s = (lid % nsh) / g.hq;
  } else {
    const uint32_t l2 = g.total_wg % 8 == 0 ? (lid % 8) * (g.total_wg / 8) + lid / 8 : lid;
    qt = l2 % g.q_tiles;
    h = (l2 / g.q_tiles) % g.hq;
    s = l2 / (g.q_tiles * g.hq);
  }
}
// The sequence's key count L (returned), the keys the tile needs (kmax) and
// the fewest any of its rows may use (kmin). Key counts fit in 31 bits
// (checked on the host).
__device__ __forceinline__ int tile_keys(const AttnArgs& g, uint32_t qt, uint32_t s, int& kmax, int& kmin) {
  const int max_keys = (int)(g.pages_per_seq * (int64_t)g.page_size);
  int L = g.lens[s];
  L = L < 0 ? 0 : (L > max_keys ? max_keys : L);
  const int q_len = (int)g.q_len;
  const int q0 = (int)qt * kQT;
  const int q_last = min(q0 + kQT - 1, q_len - 1);
  kmax = L;
  kmin = L;
  if (g.causal) {
    kmax = min(L, L - q_len + q_last + 1);
    kmin = min(L, L - q_len + q0 + 1);
  }
  return L;
}
// some scale byte of w (the four head-dim blocks of one key) lies outside
// the fold window or is the NaN code
__device__ __forceinline__ bool v_word_outside(uint32_t w) {
  bool out = false;
#pragma unroll
  for (int i = 0; i < 4; ++i) out |= ((w >> (8 * i)) & 0xFFu) - (uint32_t)kVFoldLo > (uint32_t)(kVFoldHi - kVFoldLo);
  return out;
}

// The running softmax reference moves up only when a block's maximum
// exceeds it by more than this (log2 units); weights relative to it then
// stay below 2^8, far inside f32 and bf16 range, and most blocks skip the
// rescaling of the accumulators.
constexpr float kRescaleSlack = 8.f;

template <bool BF16OUT, bool SHIFTED>
__global__ __launch_bounds__(kAttnThreads, 2) void attn_kernel(AttnArgs g) {
  __shared__ __attribute__((aligned(1024))) uint8_t Ks[2][kKB * kHD];
  __shared__ __attribute__((aligned(16))) uint32_t KSs[2][kKB];
  __shared__ __attribute__((aligned(16))) uint32_t VSs[2][kKB];
  __shared__ __attribute__((aligned(1024))) uint8_t VT[kHD * kVTRow];
  __shared__ __attribute__((aligned(16))) float VShift[SHIFTED ? kKB : 4];  // 2^r of each key (v_key_shift)
  __shared__ __attribute__((aligned(16))) int32_t PageNext[2][64];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 31, lg = lane >> 5;

  // One tile: the 128 queries qt of (sequence s, query head h).
  auto tile = [&](uint32_t qt, uint32_t h, uint32_t s) {
  const uint32_t hk = h / g.group;

  int kmax, kmin;
  const int L = tile_keys(g, qt, s, kmax, kmin);
  const int q_len = (int)g.q_len;
  const int q0 = (int)qt * kQT;
  const int nblk = kmax > 0 ? (kmax + kKB - 1) / kKB : 0;

  // ---- this lane's query row (rows past q_len load the last row and store nothing)
  const int qi = q0 + wave * 32 + lr;
  const bool q_ok = qi < q_len;
  const int64_t tok = (int64_t)s * q_len + (q_ok ? qi : q_len - 1);
  const int lim = g.causal ? min(L, L - q_len + qi + 1) : L;  // allowed keys: j < lim

  const int64_t out_row = tok * g.ld_o + (int64_t)h * kHD;
  const int32_t* tab = g.table + (int64_t)s * g.pages_per_seq;


  if (nblk == 0) {  // no allowed key anywhere in the tile
    if (q_ok) {
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int64_t d = 32 * t + 8 * r + 4 * lg;
          if constexpr (BF16OUT) *(uint2*)((uint16_t*)g.out + out_row + d) = make_uint2(0u, 0u);
          else *(float4*)((float*)g.out + out_row + d) = make_float4(0.f, 0.f, 0.f, 0.f);
        }
      if (lg == 0 && g.lse) g.lse[tok * g.hq + h] = -__builtin_inff();
    }
    return;
  }

  // ---- Q fragments: lane (row lr, half lg) holds, for head-dim half hd,
  // bytes 64hd + 16lg .. +15 and 64hd + 32 + 16lg .. +15; its scale word is
  // shifted so that block 2hd + lg sits in byte 0 of qsc[hd].
  const uint8_t* qrow = g.q + tok * g.ld_q + (int64_t)h * kHD;
  v8i32 qf[2];
  uint32_t qsc[2];
  {
#pragma unroll
    for (int hd = 0; hd < 2; ++hd) {
      const uint4 lo = *(const uint4*)(qrow + 64 * hd + 16 * lg);
      const uint4 hi = *(const uint4*)(qrow + 64 * hd + 32 + 16 * lg);
      qf[hd] = v8i32{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
    const uint32_t w = *(const uint32_t*)(g.qs + tok * g.ld_qs + (int64_t)h * (kHD / 32)) >> (8 * lg);
    qsc[0] = w;
    qsc[1] = w >> 16;
  }

  // ---- per-block sources. Key j of the sequence sits in cache slot
  // table[j / page_size] * page_size + j % page_size; within a block the
  // slots are consecutive.
  const uint32_t slot_bytes = g.hkv * kHD;        // code bytes per cache slot
  const uint32_t slot_sbytes = g.hkv * (kHD / 32); // scale bytes per cache slot
  // The page of block b is fetched two blocks ahead, straight into LDS
  // (PageNext[b & 1], 64 copies), so no register waits on its load.
  auto page_of = [&](int b) -> int32_t { return tab[(uint32_t)b * kKB / g.page_size]; };
  auto prefetch_page = [&](int b) {
    if (wave == 0)
      dma4(lds_off(&PageNext[b & 1][0]), 0u, uniform_ptr((const uint8_t*)(tab + (uint32_t)b * kKB / g.page_size)));
  };
  auto slot0_of = [&](int b, int32_t page) -> int64_t {
    return (int64_t)page * g.page_size + ((uint32_t)b * kKB) % g.page_size;
  };

  // K code rows of this lane's 4 direct-to-LDS loads and the chunk each
  // fetches; rows past the last needed key are clamped to it (their scores
  // are masked, so their P is exactly 0).
  uint32_t k_row[4], k_chunk[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    k_row[t] = 32 * wave + 8 * t + (lane >> 3);
    k_chunk[t] = (((uint32_t)lane & 7u) ^ fperm(k_row[t])) << 4;
  }
  // V decode unit of this thread: V^T chunk pg (the 8 keys v_key + {0,1,2,3,
  // 8,9,10,11}) x head-dim columns 4gd .. 4gd+3 for gd = gd0 and gd0 + 4,
  // both in scale block db.
  const uint32_t pg = (uint32_t)tid >> 4;
  const uint32_t db = ((uint32_t)tid >> 2) & 3u;
  const uint32_t gd0 = 8 * db + ((uint32_t)tid & 3u);
  const uint32_t v_key = 32 * (pg >> 2) + 16 * ((pg >> 1) & 1) + 4 * (pg & 1);
  const uint32_t v_off0 = v_key * slot_bytes + 4 * gd0;

  uint32_t vraw[2][8];
  auto issue_block = [&](int b, int buf, int32_t page) {
    const int64_t slot0 = slot0_of(b, page);
    const uint32_t last = (uint32_t)min(kKB, kmax - b * kKB) - 1;
    const uint8_t* kbase = uniform_ptr(g.kc + (slot0 * g.hkv + hk) * kHD);
#pragma unroll
    for (int t = 0; t < 4; ++t)
      dma16(lds_off(&Ks[buf][(32 * wave + 8 * t) * kHD]), min(k_row[t], last) * slot_bytes + k_chunk[t], kbase);
    {
      // scales: waves 0-1 load K's, waves 2-3 V's, 64 rows each
      const bool is_k = wave < 2;
      const uint32_t row = 64 * (wave & 1) + lane;
      const uint8_t* sbase = uniform_ptr((is_k ? g.ks : g.vs) + (slot0 * g.hkv + hk) * (kHD / 32));
      dma4(lds_off(is_k ? &KSs[buf][64 * (wave & 1)] : &VSs[buf][64 * (wave & 1)]), min(row, last) * slot_sbytes,
           sbase);
    }
    // V codes: the buffer ends after the last needed key's row, so keys past
    // it read as 0 (their P is 0 as well)
    const __amdgpu_buffer_rsrc_t vr =
        buffer_rsrc(uniform_ptr(g.vc + (slot0 * g.hkv + hk) * kHD), last * slot_bytes + kHD);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t off = v_off0 + ((e & 3) + 8 * (e >> 2)) * slot_bytes;
      vraw[0][e] = __builtin_amdgcn_raw_buffer_load_b32(vr, (int)off, 0, 0);
      vraw[1][e] = __builtin_amdgcn_raw_buffer_load_b32(vr, (int)(off + 16), 0, 0);
    }
  };

  // decode this thread's V unit into V^T rows 4gd .. 4gd+3 (gd = gd0, gd0 + 4)
  auto decode_v = [&](int buf, bool shifted) {
    const uint4 sa = *(const uint4*)&VSs[buf][v_key];
    const uint4 sb = *(const uint4*)&VSs[buf][v_key + 8];
    const uint32_t sw[8] = {sa.x, sa.y, sa.z, sa.w, sb.x, sb.y, sb.z, sb.w};
    float sc[8];
    bool vnan[8];
    if (!shifted) {
      // scales inside the window decode exactly; a tile with any other is
      // computed again by the shifted kernel
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        sc[e] = __uint_as_float(((sw[e] >> (8 * db)) & 0xFFu) << 23);
        vnan[e] = false;
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t code = (sw[e] >> (8 * db)) & 0xFFu;
        const int r = v_key_shift(sw[e]);
        sc[e] = __uint_as_float(v_fold_code(code, r) << 23);
        vnan[e] = code == 0xFFu;
        // the threads of head-dim block 0 publish the key's 2^r
        if (db == 0) VShift[v_key + (e & 3) + 8 * (e >> 2)] = __uint_as_float((uint32_t)(127 + r) << 23);
      }
    }
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      uint32_t lo[8], hi[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        lo[e] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)vraw[x][e], sc[e], false));
        hi[e] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)vraw[x][e], sc[e], true));
        if (vnan[e]) lo[e] = hi[e] = 0x7FC07FC0u;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t* src = i < 2 ? lo : hi;
        const uint32_t sel = (i & 1) ? 0x07060302u : 0x05040100u;
        const uint4 w = make_uint4(__builtin_amdgcn_perm(src[1], src[0], sel), __builtin_amdgcn_perm(src[3], src[2], sel),
                                   __builtin_amdgcn_perm(src[5], src[4], sel), __builtin_amdgcn_perm(src[7], src[6], sel));
        const uint32_t row = 4 * (gd0 + 4 * x) + i;
        *(uint4*)(VT + row * kVTRow + ((pg ^ vt_perm(row)) << 4)) = w;
      }
    }
  };

  v16f32 o_acc[4];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int e = 0; e < 16; ++e) o_acc[t][e] = 0.f;
  float m_ref = -__builtin_inff();  // softmax reference, in units of sm_scale * log2(e) * S
  float l_run = 0.f;                 // sum of exp2(x - m_ref) over the keys so far

  const uint32_t fp = fperm(lr);

  issue_block(0, 0, page_of(0));
  if (nblk > 1) prefetch_page(1);

  for (int b = 0; b < nblk; ++b) {
    const int buf = b & 1;
    wait_vmcnt<0>();
    wait_lgkmcnt0();
    barrier();  // block b staged; V^T and buffer buf ^ 1 are free
    decode_v(buf, SHIFTED);
    if (b + 1 < nblk) {
      // (landed: wave 0 waited for all its loads before the barrier above)
      const int32_t page = __builtin_amdgcn_readfirstlane(PageNext[(b + 1) & 1][0]);
      if (b + 2 < nblk) prefetch_page(b + 2);
      issue_block(b + 1, buf ^ 1, page);
    }

    // ---- S^T for this wave's 32 queries x 128 keys: 4 tiles of 32 keys,
    // accumulated over the two head-dim halves
    v16f32 sacc[4];
    uint32_t kw[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
      for (int e = 0; e < 16; ++e) sacc[kt][e] = 0.f;
      kw[kt] = KSs[buf][32 * kt + lr] >> (8 * lg);
    }
#pragma unroll
    for (int hd = 0; hd < 2; ++hd)
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        const uint8_t* krow = &Ks[buf][(32 * kt + lr) * kHD];
        const uint4 lo = *(const uint4*)(krow + (((4 * hd + lg) ^ fp) << 4));
        const uint4 hi = *(const uint4*)(krow + (((4 * hd + 2 + lg) ^ fp) << 4));
        const v8i32 kf = v8i32{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        sacc[kt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kf, qf[hd], sacc[kt], MX_E4M3, MX_E4M3, 0,
                                                                    (int)(kw[kt] >> (16 * hd)), 0, (int)qsc[hd]);
      }

    // ---- online softmax. Element e of tile kt is key 32kt + 8(e/4) + 4lg + e%4.
    if ((b + 1) * kKB > kmin) {
      // allowed keys of this block for the row: local index < lim - 128b,
      // i.e. (local index - 4lg) < rel, a lane value against constants
      const int rel = lim - b * kKB - 4 * lg;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (32 * kt + 8 * (e >> 2) + (e & 3) >= rel) sacc[kt][e] = -__builtin_inff();
    }
    float mx = -__builtin_inff();
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = __builtin_fmaxf(mx, sacc[kt][e]);
    {
      const auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
      mx = __builtin_fmaxf(__uint_as_float(pr[0]), __uint_as_float(pr[1]));
    }
    const float x_max = mx * g.c2;
    const bool lift = x_max > m_ref + kRescaleSlack;
    if (__builtin_amdgcn_ballot_w64(lift)) {
      // lanes that do not lift keep their reference (alpha = 1; computing it
      // from m_ref - m_ref would give NaN for a reference still at -inf)
      const float alpha = lift ? __builtin_amdgcn_exp2f(m_ref - x_max) : 1.f;
      m_ref = lift ? x_max : m_ref;
      l_run *= alpha;
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int e = 0; e < 16; ++e) o_acc[t][e] *= alpha;
    }
    const float m_use = m_ref == -__builtin_inff() ? 0.f : m_ref;

    wait_lgkmcnt0();
    barrier();  // V^T of block b complete

    // ---- per tile of 32 keys: P = exp2(x - m) rounded to bf16, then
    // O^T += V^T P^T in two 16-key steps c, each over 4 head-dim tiles t.
    float ls = 0.f;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      v8bf16 pb[2];
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        float p[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          p[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kt][8 * c + e], g.c2, -m_use));
          ls += p[e];
        }
        if constexpr (SHIFTED) {
          // 2^r of each key; element e is key 32 kt + 16 c + 8 (e / 4) + 4 lg + e % 4
          const float4 s0 = *(const float4*)&VShift[32 * kt + 16 * c + 4 * lg];
          const float4 s1 = *(const float4*)&VShift[32 * kt + 16 * c + 8 + 4 * lg];
          p[0] *= s0.x; p[1] *= s0.y; p[2] *= s0.z; p[3] *= s0.w;
          p[4] *= s1.x; p[5] *= s1.y; p[6] *= s1.z; p[7] *= s1.w;
        }
        pb[c] = v8bf16{(__bf16)p[0], (__bf16)p[1], (__bf16)p[2], (__bf16)p[3],
                       (__bf16)p[4], (__bf16)p[5], (__bf16)p[6], (__bf16)p[7]};
      }
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const uint32_t row = 32 * t + lr;
          const v8bf16 vf =
              *(const v8bf16*)(VT + row * kVTRow + (((uint32_t)(4 * kt + 2 * c + lg) ^ vt_perm(row)) << 4));
          o_acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb[c], o_acc[t], 0, 0, 0);
        }
    }
    {
      const auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(ls), __float_as_uint(ls), false, false);
      ls = __uint_as_float(pr[0]) + __uint_as_float(pr[1]);
    }
    l_run += ls;
  }

  // ---- epilogue: O = acc / l; element e of tile t is head-dim column
  // 32t + 8(e/4) + 4lg + e%4. (A tile that needs the shift is written again
  // by the shifted kernel, which runs after this one on the stream.)
  if (!q_ok) return;
  const float inv = !(l_run <= 0.f) ? 1.f / l_run : 0.f;  // a NaN normaliser stays NaN
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    if constexpr (BF16OUT) {
      // Lanes l and l + 32 (the same query) hold columns 8r + 4lg .. +3 of
      // each r; one lane swap per dword gives lane lg the 8 consecutive
      // columns 16p + 8lg .. +7 of each pair p of r, stored as 16 bytes
      uint32_t w[4][2];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float v0 = o_acc[t][4 * r] * inv, v1 = o_acc[t][4 * r + 1] * inv;
        const float v2 = o_acc[t][4 * r + 2] * inv, v3 = o_acc[t][4 * r + 3] * inv;
        w[r][0] = f32_to_bf16_rne(canon_nan(v0)) | (f32_to_bf16_rne(canon_nan(v1)) << 16);
        w[r][1] = f32_to_bf16_rne(canon_nan(v2)) | (f32_to_bf16_rne(canon_nan(v3)) << 16);
      }
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const auto r0 = __builtin_amdgcn_permlane32_swap(w[2 * p][0], w[2 * p + 1][0], false, false);
        const auto r1 = __builtin_amdgcn_permlane32_swap(w[2 * p][1], w[2 * p + 1][1], false, false);
        *(uint4*)((uint16_t*)g.out + out_row + 32 * t + 16 * p + 8 * lg) = make_uint4(r0[0], r1[0], r0[1], r1[1]);
      }
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t d = 32 * t + 8 * r + 4 * lg;
        const float v0 = o_acc[t][4 * r] * inv, v1 = o_acc[t][4 * r + 1] * inv;
        const float v2 = o_acc[t][4 * r + 2] * inv, v3 = o_acc[t][4 * r + 3] * inv;
        *(float4*)((float*)g.out + out_row + d) = make_float4(v0, v1, v2, v3);
      }
    }
  }
  if (lg == 0 && g.lse)
    g.lse[tok * g.hq + h] = !(l_run <= 0.f) ? (m_ref + __log2f(l_run)) * 0.69314718055994531f : -__builtin_inff();
  };

  if constexpr (!SHIFTED) {
    uint32_t qt, h, s;
    tile_of(g, blockIdx.x, qt, h, s);
    tile(qt, h, s);
  } else {
    // One work-group per (sequence s, kv head hk): the first key j0 of the
    // sequence with a V scale outside the fold window (or the NaN code); the
    // tiles of the query heads on hk that read key j0 (kmax > j0) are the
    // ones the plain kernel decoded inexactly, and they are computed again
    // here, overwriting its output.
    __shared__ int j_first;
    const uint32_t s = blockIdx.x / g.hkv, hk = blockIdx.x % g.hkv;
    const int max_keys = (int)(g.pages_per_seq * (int64_t)g.page_size);
    int L = g.lens[s];
    L = L < 0 ? 0 : (L > max_keys ? max_keys : L);
    if (tid == 0) j_first = L;
    __syncthreads();
    const int32_t* tab = g.table + (int64_t)s * g.pages_per_seq;
    for (int j = tid; j < L; j += kAttnThreads) {
      const int64_t slot = (int64_t)tab[j / g.page_size] * g.page_size + j % g.page_size;
      if (v_word_outside(*(const uint32_t*)(g.vs + (slot * g.hkv + hk) * (kHD / 32)))) {
        atomicMin(&j_first, j);
        break;
      }
    }
    __syncthreads();
    const int j0 = j_first;
    if (j0 >= L) return;
    for (uint32_t h = hk * g.group; h < (hk + 1) * g.group; ++h)
      for (uint32_t qt = 0; qt < g.q_tiles; ++qt) {
        int kmax, kmin;
        tile_keys(g, qt, s, kmax, kmin);
        if (kmax > j0) {
          tile(qt, h, s);
          __syncthreads();  // the next tile reuses the LDS buffers
        }
      }
  }
}

}  // namespace

extern "C" mx_status_t mx_paged_attention(const mx_attention_desc_t* d, hipStream_t stream) {
  if (!d) return MX_ERR_NULL;
  if (d->num_seqs < 0 || d->q_len < 0) return MX_ERR_SHAPE;
  if (d->out_dtype != MX_F32 && d->out_dtype != MX_BF16) return MX_ERR_FORMAT;
  if (d->num_seqs == 0 || d->q_len == 0) return MX_OK;
  if (!d->q || !d->q_scale || !d->k_cache || !d->k_scale || !d->v_cache || !d->v_scale || !d->page_table ||
      !d->kv_lens || !d->out)
    return MX_ERR_NULL;
  const int64_t hq = d->num_q_heads, hkv = d->num_kv_heads;
  if (d->head_dim != kHD || hq <= 0 || hkv <= 0 || hq % hkv != 0 || d->page_size <= 0 || d->pages_per_seq <= 0)
    return MX_ERR_SHAPE;
  if (d->page_size % kKB != 0) return MX_ERR_SHAPE;
  if (d->pages_per_seq * d->page_size >= ((int64_t)1 << 31) || hq >= (1 << 16) || hkv >= (1 << 16) ||
      d->q_len >= ((int64_t)1 << 31))
    return MX_ERR_SHAPE;
  if (d->ld_q < hq * kHD || d->ld_qs < hq * (kHD / 32) || d->ld_o < hq * kHD) return MX_ERR_SHAPE;
  if (!(d->sm_scale > 0.f) || d->sm_scale == __builtin_inff()) return MX_ERR_SHAPE;
  using mx_host::aligned16;
  if (!aligned16(d->q) || !aligned16(d->k_cache) || !aligned16(d->v_cache) || d->ld_q % 16 != 0) return MX_ERR_ALIGN;
  if (((uintptr_t)d->q_scale | (uintptr_t)d->k_scale | (uintptr_t)d->v_scale) % 4 != 0 || d->ld_qs % 4 != 0)
    return MX_ERR_ALIGN;
  const uintptr_t oal = d->out_dtype == MX_F32 ? 16 : 8;
  if ((uintptr_t)d->out % oal != 0 || d->ld_o % 4 != 0 || ((uintptr_t)d->lse & 3u) != 0) return MX_ERR_ALIGN;
  const int64_t q_tiles = (d->q_len + kQT - 1) / kQT;
  const int64_t total = q_tiles * hq * d->num_seqs;
  if (total >= ((int64_t)1 << 31) || d->num_seqs * hkv >= ((int64_t)1 << 31)) return MX_ERR_SHAPE;
  const mx_status_t dev = mx_host::check_device();
  if (dev != MX_OK) return dev;

  AttnArgs g;
  g.q = d->q; g.qs = d->q_scale; g.ld_q = d->ld_q; g.ld_qs = d->ld_qs;
  g.kc = d->k_cache; g.ks = d->k_scale; g.vc = d->v_cache; g.vs = d->v_scale;
  g.table = d->page_table; g.lens = d->kv_lens;
  g.out = d->out; g.ld_o = d->ld_o; g.lse = d->lse;
  g.pages_per_seq = d->pages_per_seq;
  g.page_size = (uint32_t)d->page_size; g.q_len = (uint32_t)d->q_len;
  g.hq = (uint32_t)hq; g.hkv = (uint32_t)hkv; g.group = (uint32_t)(hq / hkv);
  g.causal = d->causal ? 1u : 0u; g.q_tiles = (uint32_t)q_tiles; g.total_wg = (uint32_t)total;
  g.c2 = d->sm_scale * 1.4426950408889634f;
  // the plain kernel computes every tile, decoding V with its scales as
  // they are; the shifted one then computes again, and overwrites, every
  // tile that reads a key with a V scale outside the fold window
  const uint32_t shift_wg = (uint32_t)(d->num_seqs * hkv);  // one per (sequence, kv head)
  if (d->out_dtype == MX_BF16) {
    hipLaunchKernelGGL((attn_kernel<true, false>), dim3((uint32_t)total), dim3(kAttnThreads), 0, stream, g);
    hipLaunchKernelGGL((attn_kernel<true, true>), dim3(shift_wg), dim3(kAttnThreads), 0, stream, g);
  } else {
    hipLaunchKernelGGL((attn_kernel<false, false>), dim3((uint32_t)total), dim3(kAttnThreads), 0, stream, g);
    hipLaunchKernelGGL((attn_kernel<false, true>), dim3(shift_wg), dim3(kAttnThreads), 0, stream, g);
  }
  return mx_host::launch_status();
}
