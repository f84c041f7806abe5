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
//                       block scale (v_cvt_scalef32_pk_bf16_fp8, exact for
//                       scale codes 3..246) into LDS once per work-group.
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
// into registers one block ahead, and every thread decodes 2 x 32 of them
// into the shared bf16 V^T tile (32 KB). Each key block lies inside one page
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
// touch 16 consecutive rows at one logical chunk, and the decoder's writes
// touch rows 4g + i for 16 consecutive g; (row ^ (row >> 4)) & 15 is
// distinct across both sets, so neither conflicts on LDS banks.
__device__ __forceinline__ uint32_t vt_perm(uint32_t row) { return (row ^ (row >> 4)) & 15u; }

__device__ __forceinline__ void dma4(uint32_t lds, uint32_t off, const void* base) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, %2" ::"s"(lds), "v"(off), "s"(base) : "memory");
}

__device__ __forceinline__ float max2(float a, float b) { return a > b ? a : b; }

template <bool BF16OUT>
__global__ __launch_bounds__(kAttnThreads, 2) void attn_kernel(AttnArgs g) {
  __shared__ __attribute__((aligned(1024))) uint8_t Ks[2][kKB * kHD];
  __shared__ __attribute__((aligned(16))) uint32_t KSs[2][kKB];
  __shared__ __attribute__((aligned(16))) uint32_t VSs[2][kKB];
  __shared__ __attribute__((aligned(1024))) uint8_t VT[kHD * kVTRow];

  // ---- work item: (sequence, head, query tile); the query tiles of one
  // (sequence, head) share its keys, so they are kept on one XCD.
  uint32_t lid = blockIdx.x;
  if (g.total_wg % 8 == 0) lid = (lid % 8) * (g.total_wg / 8) + lid / 8;
  const uint32_t qt = lid % g.q_tiles;
  const uint32_t h = (lid / g.q_tiles) % g.hq;
  const uint32_t s = lid / (g.q_tiles * g.hq);
  const uint32_t hk = h / g.group;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 31, lg = lane >> 5;

  const int64_t max_keys = g.pages_per_seq * (int64_t)g.page_size;
  int64_t L = g.lens[s];
  L = L < 0 ? 0 : (L > max_keys ? max_keys : L);
  const int64_t q_len = g.q_len;
  const int64_t q0 = (int64_t)qt * kQT;
  const int64_t q_last = min(q0 + kQT - 1, q_len - 1);
  // keys the tile needs, and the fewest any of its rows may use
  int64_t kmax = L, kmin = L;
  if (g.causal) {
    kmax = min(L, L - q_len + q_last + 1);
    kmin = min(L, L - q_len + q0 + 1);
  }
  const int nblk = kmax > 0 ? (int)((kmax + kKB - 1) / kKB) : 0;

  // ---- this lane's query row (rows past q_len load the last row and store nothing)
  const int64_t qi = q0 + wave * 32 + lr;
  const bool q_ok = qi < q_len;
  const int64_t tok = (int64_t)s * q_len + (q_ok ? qi : q_len - 1);
  const int64_t lim = g.causal ? min(L, L - q_len + qi + 1) : L;  // allowed keys: j < lim

  const int64_t out_row = tok * g.ld_o + (int64_t)h * kHD;
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
  // slots are consecutive. Rows past the tile's last needed key are clamped
  // to it (their scores are masked and their P is exactly 0).
  const uint32_t slot_bytes = g.hkv * kHD;        // code bytes per cache slot
  const uint32_t slot_sbytes = g.hkv * (kHD / 32); // scale bytes per cache slot
  const int32_t* tab = g.table + (int64_t)s * g.pages_per_seq;
  auto slot0_of = [&](int b) -> int64_t {
    const uint32_t j = (uint32_t)b * kKB;
    return (int64_t)tab[j / g.page_size] * g.page_size + j % g.page_size;
  };

  // K code rows handled by this lane's 4 DMA instructions, and its chunk
  uint32_t k_row[4], k_chunk[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    k_row[t] = 32 * wave + 8 * t + (lane >> 3);
    k_chunk[t] = (((uint32_t)lane & 7u) ^ fperm(k_row[t])) << 4;
  }
  // V decode units: unit u covers V^T chunk pg (8 keys) x head-dim columns 4gd .. 4gd+3
  const uint32_t gd = lr;
  uint32_t v_key[2];  // first key of each unit; the unit's keys are v_key + {0,1,2,3,8,9,10,11}
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const uint32_t pg = 2 * wave + lg + 8 * u;
    v_key[u] = 32 * (pg >> 2) + 16 * ((pg >> 1) & 1) + 4 * (pg & 1);
  }

  uint32_t vraw[2][8];
  auto issue_block = [&](int b, int buf) {
    const int64_t slot0 = slot0_of(b);
    const uint32_t last = (uint32_t)min((int64_t)kKB, kmax - (int64_t)b * kKB) - 1;
    const uint8_t* kbase = uniform_ptr(g.kc + (slot0 * g.hkv + hk) * kHD);
    const uint8_t* vbase = uniform_ptr(g.vc + (slot0 * g.hkv + hk) * kHD);
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
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t key = v_key[u] + (e & 3) + 8 * (e >> 2);
        vraw[u][e] = *(const uint32_t*)(vbase + min(key, last) * slot_bytes + 4 * gd);
      }
  };

  // decode this thread's two V units into V^T (rows 4gd .. 4gd+3)
  auto decode_v = [&](int buf) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const uint32_t pg = 2 * wave + lg + 8 * u;
      const uint32_t sh = 8 * (gd >> 3);  // scale byte of head-dim block gd / 8
      const uint4 sa = *(const uint4*)&VSs[buf][v_key[u]];
      const uint4 sb = *(const uint4*)&VSs[buf][v_key[u] + 8];
      const uint32_t sw[8] = {sa.x, sa.y, sa.z, sa.w, sb.x, sb.y, sb.z, sb.w};
      uint32_t lo[8], hi[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float sc = scale_value((sw[e] >> sh) & 0xFFu);
        lo[e] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)vraw[u][e], sc, false));
        hi[e] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)vraw[u][e], sc, true));
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t* src = i < 2 ? lo : hi;
        const uint32_t sel = (i & 1) ? 0x07060302u : 0x05040100u;
        const uint4 w = make_uint4(__builtin_amdgcn_perm(src[1], src[0], sel), __builtin_amdgcn_perm(src[3], src[2], sel),
                                   __builtin_amdgcn_perm(src[5], src[4], sel), __builtin_amdgcn_perm(src[7], src[6], sel));
        const uint32_t row = 4 * gd + i;
        *(uint4*)(VT + row * kVTRow + ((pg ^ vt_perm(row)) << 4)) = w;
      }
    }
  };

  v16f32 o_acc[4];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int e = 0; e < 16; ++e) o_acc[t][e] = 0.f;
  float m_run = -__builtin_inff();  // running max of sm_scale * log2(e) * S
  float l_run = 0.f;                 // running sum of exp2(x - m_run)

  const uint32_t fp = fperm(lr);
  issue_block(0, 0);

  for (int b = 0; b < nblk; ++b) {
    const int buf = b & 1;
    wait_vmcnt<0>();
    wait_lgkmcnt0();
    barrier();  // block b staged; V^T and buffer buf ^ 1 are free
    decode_v(buf);
    if (b + 1 < nblk) issue_block(b + 1, buf ^ 1);

    // ---- S^T for this wave's 32 queries x 128 keys: 4 tiles of 32 keys
    v16f32 sacc[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
      for (int e = 0; e < 16; ++e) sacc[kt][e] = 0.f;
      const uint8_t* krow = &Ks[buf][(32 * kt + lr) * kHD];
      const uint32_t kw = KSs[buf][32 * kt + lr] >> (8 * lg);
#pragma unroll
      for (int hd = 0; hd < 2; ++hd) {
        const uint4 lo = *(const uint4*)(krow + (((4 * hd + lg) ^ fp) << 4));
        const uint4 hi = *(const uint4*)(krow + (((4 * hd + 2 + lg) ^ fp) << 4));
        const v8i32 kf = v8i32{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        sacc[kt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kf, qf[hd], sacc[kt], MX_E4M3, MX_E4M3, 0,
                                                                    (int)(kw >> (16 * hd)), 0, (int)qsc[hd]);
      }
    }

    // ---- online softmax. Element e of tile kt is key 32kt + 8(e/4) + 4lg + e%4.
    if ((int64_t)(b + 1) * kKB > kmin) {
      // allowed keys of this block for the row: local index < rel, i.e.
      // (local index - 4lg) < rel - 4lg, a lane value against constants
      const int64_t rel64 = lim - (int64_t)b * kKB - 4 * lg;
      const int rel = (int)(rel64 < -1 ? -1 : (rel64 > kKB ? kKB : rel64));
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
      for (int e = 0; e < 16; ++e) mx = max2(mx, sacc[kt][e]);
    {
      const auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
      mx = max2(__uint_as_float(pr[0]), __uint_as_float(pr[1]));
    }
    const float m_new = max2(m_run, mx * g.c2);
    const float m_use = m_new == -__builtin_inff() ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    m_run = m_new;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int e = 0; e < 16; ++e) o_acc[t][e] *= alpha;

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
    l_run = l_run * alpha + ls;
  }

  // ---- epilogue: O = acc / l; element e of tile t is head-dim column
  // 32t + 8(e/4) + 4lg + e%4.
  if (!q_ok) return;
  const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t d = 32 * t + 8 * r + 4 * lg;
      const float v0 = o_acc[t][4 * r] * inv, v1 = o_acc[t][4 * r + 1] * inv;
      const float v2 = o_acc[t][4 * r + 2] * inv, v3 = o_acc[t][4 * r + 3] * inv;
      if constexpr (BF16OUT) {
        const uint32_t w0 = f32_to_bf16_rne(canon_nan(v0)) | (f32_to_bf16_rne(canon_nan(v1)) << 16);
        const uint32_t w1 = f32_to_bf16_rne(canon_nan(v2)) | (f32_to_bf16_rne(canon_nan(v3)) << 16);
        *(uint2*)((uint16_t*)g.out + out_row + d) = make_uint2(w0, w1);
      } else {
        *(float4*)((float*)g.out + out_row + d) = make_float4(v0, v1, v2, v3);
      }
    }
  if (lg == 0 && g.lse)
    g.lse[tok * g.hq + h] = l_run > 0.f ? (m_run + __log2f(l_run)) * 0.69314718055994531f : -__builtin_inff();
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
  if (total >= ((int64_t)1 << 31)) return MX_ERR_SHAPE;
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
  if (d->out_dtype == MX_BF16)
    hipLaunchKernelGGL(attn_kernel<true>, dim3((uint32_t)total), dim3(kAttnThreads), 0, stream, g);
  else
    hipLaunchKernelGGL(attn_kernel<false>, dim3((uint32_t)total), dim3(kAttnThreads), 0, stream, g);
  return mx_host::launch_status();
}
