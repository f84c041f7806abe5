/*
 * mxfp8.h -- C ABI of libmxfp8: MXFP8 block-scaled quantization and the
 * block-scaled matrix product on AMD Instinct MI355X (gfx950).
 *
 * Sources (web pages, cited by title and section):
 *   [SM120]  "MXFP8 SM120 software support" (xuesongtap.github.io, 2026-09-22)
 *   [GLOSS]  "MXFP8 quantization" glossary (robocikowo.com)
 *   [FP8DS]  "FP8 训练为什么能稳：把缩放因子的粒度与累加精度算清楚" (magicnetworld.com)
 *   [NVFP4]  "NVFP4 如何用 4 bit 实现高精度" (theluyuan.com)
 *
 * Format. An MXFP8 block is 32 consecutive FP8 elements (E4M3 or E5M2) that
 * share one E8M0 scale 2^(e-127); decoded value x_hat_i = s_b * q_i
 * [SM120 §0.1]. Codes and scales live in separate arrays [SM120 §0.1]:
 * codes are one byte per element, scales one byte per block.
 *
 * Scale rule (the pages leave it to the implementation [SM120 §0.1]; this
 * library fixes it): X = 2^(floor(log2 amax) - emax_elem), emax_elem = 8 for
 * E4M3 and 15 for E5M2, code = clamp(floor(log2 amax) - emax_elem + 127, 0,
 * 254); amax == 0 gives code 0; a block holding NaN or Inf gets code 0xFF and
 * element codes 0x7F. Elements: q = RNE(x / X) with ties to even and
 * saturation at +-448 (E4M3) / +-57344 (E5M2); the sign of x is kept, so
 * negative values that round to zero give 0x80.
 *
 * Conventions shared by every entry point:
 *   - All data pointers are DEVICE pointers owned by the caller. The library
 *     allocates no memory and keeps no pointer after returning. Its only
 *     global state is a per-device cache of the architecture check and the
 *     device's compute-unit count (filled atomically on the first call on
 *     each device, never changed after), so calls from several threads and
 *     on different streams may run concurrently.
 *   - Work is enqueued on `stream` (asynchronous; no implicit sync). Argument
 *     errors are detected on the host before anything is launched and are
 *     returned synchronously; then nothing is written. A launch failure
 *     returns MX_ERR_HIP. Device-side faults surface at the caller's next
 *     synchronization.
 *   - Sizes and leading dimensions ("ld", row pitches) are in elements of the
 *     array they describe (bytes for codes and scales). Matrices are
 *     row-major: element (r, c) of an array with pitch ld is at r * ld + c.
 *   - An empty problem (a zero row, column, token or group count) writes
 *     nothing and returns MX_OK (MX_ERR_DEVICE off gfx950); its buffers,
 *     pitches and alignment are then not checked (NULL is accepted). Formats
 *     and negative sizes still are.
 *   - A blocked dimension must be a multiple of 32 (MX_ERR_SHAPE otherwise).
 *   - Alignment (MX_ERR_ALIGN otherwise): the base address and the byte pitch
 *     of every high-precision input, of the dequantize output and of every
 *     code array must be multiples of 16 bytes. Scale arrays have no
 *     alignment requirement; the mx_gemm output needs only the natural
 *     alignment of its element type.
 *   - Zero-sized problems are valid and launch nothing.
 */
#ifndef MXFP8_H
#define MXFP8_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t mx_status_t;
#define MX_OK          0
#define MX_ERR_NULL   -1 /* a required pointer is NULL */
#define MX_ERR_SHAPE  -2 /* negative size, pitch smaller than the row, blocked dim not a multiple of 32 */
#define MX_ERR_ALIGN  -3 /* base address or pitch breaks the 16-byte rule above */
#define MX_ERR_FORMAT -4 /* unknown element format or data type */
#define MX_ERR_DEVICE -5 /* current device is not gfx950 */
#define MX_ERR_HIP    -6 /* the HIP runtime reported an error at launch: read with
                             hipGetLastError() after the launch, so an error
                             left pending by an earlier HIP call on the same
                             thread is reported (and cleared) the same way */

/* Element encodings [SM120 §0.1 table; GLOSS]: E4M3 (448 max, used for
 * activations and weights), E5M2 (57344 max, used for gradients).
 * MX_E2M1 is the MXFP4 element [NVFP4 §2.4, §5.5]: values 0, +-0.5, +-1,
 * +-1.5, +-2, +-3, +-4, +-6, the same E8M0 scale per 32 (rule with
 * emax_elem = 2; a NaN/Inf block gets scale 0xFF and codes 0, E2M1 having no
 * NaN). Its codes are packed two per byte, element 2i in the low nibble, so
 * a row of `cols` elements holds cols/2 bytes and pitches stay in bytes.
 * E2M1 is accepted by mx_quantize, mx_quantize_colwise, mx_quantize_ex
 * (1-D blocks), mx_dequantize, mx_gemm and mx_grouped_gemm (see there); the
 * other entry points return MX_ERR_FORMAT for it. */
typedef enum { MX_E4M3 = 0, MX_E5M2 = 1, MX_E2M1 = 2 } mx_fmt_t;
/* High-precision data types of inputs and outputs. */
typedef enum { MX_F32 = 0, MX_BF16 = 1 } mx_dtype_t;

/*
 * mx_quantize -- rowwise (1 x 32) MXFP8 quantization.
 * [SM120 §0.1, §0.2; GLOSS]: per block of 32 consecutive values along a row,
 * find amax, choose a power-of-two E8M0 scale, round x / scale to FP8.
 *
 *   x    [rows x cols] input (xdt), pitch ldx >= cols
 *   q    [rows x cols] codes out, pitch ldq >= cols (E2M1: cols/2 bytes per row)
 *   s    [rows x cols/32] scales out, pitch lds >= cols/32
 * cols % 32 == 0.
 */
mx_status_t mx_quantize(const void* x, mx_dtype_t xdt, int64_t rows, int64_t cols, int64_t ldx, mx_fmt_t fmt,
                        uint8_t* q, int64_t ldq, uint8_t* s, int64_t lds, hipStream_t stream);

/*
 * mx_quantize_colwise -- columnwise (32 x 1) MX quantization, stored
 * transposed. Blocks are directional, so the second representation the
 * backward pass needs is quantized again from the high-precision input; a
 * transpose of the rowwise codes is not equivalent [SM120 §1.2, §1.3; GLOSS].
 *
 *   x    [rows x cols] input (xdt), pitch ldx >= cols
 *   qt   [cols x rows] codes out (qt[c][r] is element (r, c)), pitch ldq >= rows
 *        (E2M1: rows/2 bytes per row, element r in nibble r % 2 of byte r/2)
 *   st   [cols x rows/32] scales out (st[c][r/32]), pitch lds >= rows/32
 * rows % 32 == 0. The result equals mx_quantize applied to x^T, so it is
 * directly a K-contiguous operand of mx_gemm with K = rows.
 */
mx_status_t mx_quantize_colwise(const void* x, mx_dtype_t xdt, int64_t rows, int64_t cols, int64_t ldx,
                                mx_fmt_t fmt, uint8_t* qt, int64_t ldq, uint8_t* st, int64_t lds,
                                hipStream_t stream);

/*
 * mx_quantize_ex -- quantization with a choice of scale rule and block shape
 * [SM120 §1.3; GLOSS: how the E8M0 scale is chosen and rounded affects
 * accuracy].
 *
 *   rule    MX_SCALE_FLOOR: the rule of mx_quantize (X = 2^(floor(log2 amax)
 *           - emax_elem); the block maximum may saturate).
 *           MX_SCALE_CEIL: the smallest power of two X with amax / X <= the
 *           largest finite element, so no element saturates (one E8M0 step
 *           above the floor rule when amax's significand exceeds 1.75 (FP8)
 *           or 1.5 (E2M1), the same otherwise).
 *   blocks  MX_BLOCKS_1D: 1 x 32 blocks for the rowwise output and 32 x 1
 *           blocks for the colwise output, as mx_quantize / _colwise. With
 *           both outputs asked for, x is read once (rows % 32 == 0 and
 *           cols % 32 == 0; E4M3 / E5M2; E2M1 takes one pass per output).
 *           MX_BLOCKS_2D: one scale per 32 x 32 block (the 2-D weight
 *           quantization of [SM120 §1.3]), written in the MXFP8 layout: s
 *           repeats a block's scale on its 32 rows, st on its 32 columns, and
 *           the colwise codes are exactly the transpose of the rowwise codes.
 *           E4M3 / E5M2 only; rows % 32 == 0.
 *   q, s    rowwise output [rows x cols] / [rows x cols/32] (pitches ldq,
 *           lds), or both NULL;
 *   qt, st  colwise output stored transposed [cols x rows] / [cols x rows/32]
 *           (pitches ldqt, ldst), or both NULL. At least one pair is given.
 * Shapes, alignment and E2M1 packing follow mx_quantize / mx_quantize_colwise
 * (E2M1: 1-D blocks only).
 */
typedef enum { MX_SCALE_FLOOR = 0, MX_SCALE_CEIL = 1 } mx_scale_rule_t;
typedef enum { MX_BLOCKS_1D = 0, MX_BLOCKS_2D = 1 } mx_blocks_t;
typedef struct mx_quantize_desc {
    const void* x;  mx_dtype_t xdt;  int64_t rows, cols, ldx;
    mx_fmt_t fmt;   mx_scale_rule_t rule;  mx_blocks_t blocks;
    uint8_t* q;  int64_t ldq;  uint8_t* s;  int64_t lds;
    uint8_t* qt; int64_t ldqt; uint8_t* st; int64_t ldst;
} mx_quantize_desc_t;

mx_status_t mx_quantize_ex(const mx_quantize_desc_t* desc, hipStream_t stream);

/*
 * mx_scale_broadcast -- Float8BlockScaling scales to MXFP8 [SM120 §1.3]: a
 * power-of-two FP32 scale of a 128-element block becomes the E8M0 scale of
 * each of its four 32-element blocks, so the block's FP8 codes are used by
 * mx_gemm / mx_dequantize unchanged (nothing is re-quantized).
 *
 *   s_in    MX_BCAST_1X128: [rows x cols/128], s_in[r][c/128] scales row r's
 *           elements c; MX_BCAST_128X128: [ceil(rows/128) x cols/128], one
 *           scale per 128 x 128 block. Pitch ld_in (elements). s is the
 *           dequantizing factor: x_hat = q * s.
 *   out     E8M0 [rows x cols/32], pitch ld_out (bytes, a multiple of 4).
 * cols % 128 == 0; s_in and out 4-byte aligned. A scale that is not a positive
 * power of two 2^k with -127 <= k <= 127 gives code 0xFF, so its blocks
 * decode to NaN rather than to wrong values.
 */
typedef enum { MX_BCAST_1X128 = 0, MX_BCAST_128X128 = 1 } mx_bcast_layout_t;

mx_status_t mx_scale_broadcast(const float* s_in, int64_t ld_in, mx_bcast_layout_t layout, int64_t rows,
                               int64_t cols, uint8_t* out, int64_t ld_out, hipStream_t stream);

/*
 * mx_dequantize -- x_hat = s_b * q_i [SM120 §0.1], exact in f32, then
 * rounded to nearest-even for bf16 output. A scale code 0xFF (NaN) makes its
 * whole block NaN; NaN results are written as the canonical quiet NaN
 * (0x7FC00000 / 0x7FC0).
 *
 *   q    [rows x cols] codes, pitch ldq (E2M1: cols/2 bytes per row);
 *        s [rows x cols/32] scales, pitch lds
 *   y    [rows x cols] output (ydt), pitch ldy
 * cols % 32 == 0.
 */
mx_status_t mx_dequantize(const uint8_t* q, int64_t ldq, const uint8_t* s, int64_t lds, mx_fmt_t fmt, int64_t rows,
                          int64_t cols, void* y, mx_dtype_t ydt, int64_t ldy, hipStream_t stream);

/*
 * mx_kv_quant_write -- fused E4M3 quantization and paged KV-cache write
 * [SM120 §0.2]: for every token t and head h, the D values of K and of V are
 * quantized in blocks of 32 along the head dimension and written to cache
 * slot slot_mapping[t]: page = slot / page_size, offset = slot % page_size.
 *
 *   k, v           [T x H x D] inputs (dt); token t, head h starts at t*ld_token + h*D
 *   slot_mapping   [T] int64 (device); a negative slot marks a padding token
 *                  and is skipped; slots >= page_size * num_pages are ignored
 *   k_cache, v_cache [num_pages x page_size x H x D] codes out
 *   k_scale, v_scale [num_pages x page_size x H x D/32] scales out
 * D % 32 == 0, ld_token >= H*D. Slots not named by slot_mapping are left
 * untouched.
 */
mx_status_t mx_kv_quant_write(const void* k, const void* v, mx_dtype_t dt, int64_t T, int64_t H, int64_t D,
                              int64_t ld_token, const int64_t* slot_mapping, uint8_t* k_cache, uint8_t* k_scale,
                              uint8_t* v_cache, uint8_t* v_scale, int64_t page_size, int64_t num_pages,
                              hipStream_t stream);

/*
 * mx_gemm -- block-scaled matrix product [SM120 §0.3; NVFP4 §7.1, §7.4]:
 *
 *   y[m][n] = sum_b sa[m][b] * sb[n][b] * sum_{i<32} a[m][32b+i] * b[n][32b+i]
 *
 * with both operands K-contiguous (y = A * B^T; the "TN" call of a
 * column-major GEMM interface [SM120 §1.1, §1.2]). The per-block scale
 * products stay inside the sum over blocks; accumulation is in FP32. Other
 * transpositions are obtained by quantizing the operand colwise, which
 * yields a K-contiguous array directly.
 *
 * Batching: the problem is repeated for p = 0 .. batch_outer*batch_inner-1,
 * with o = p / batch_inner and i = p % batch_inner; operand X of problem
 * (o, i) starts at X + o*stride_X_outer + i*stride_X_inner (elements).
 * Zero batch sizes mean 1.
 *
 * Paged B: when b_page_table != NULL, row n of B in problem (o, i) is read
 * from page P = b_page_table[o * b_pages_per_seq + n / b_page_rows] at
 *   b  + P*b_page_stride   + (n % b_page_rows)*ldb  + i*stride_b_inner
 *   sb + P*b_page_stride_s + (n % b_page_rows)*ldsb + i*stride_sb_inner
 * (stride_b_outer and stride_sb_outer are then unused). The page table is a
 * device int32 array of batch_outer * b_pages_per_seq entries whose values
 * must index valid pages; the caller guarantees that.
 *
 * K % 32 == 0. Output y is f32 or bf16 (round to nearest even); y needs only
 * the natural alignment of its element type (wider stores are used when the
 * pitch allows them).
 *
 * Accumulation (field `accum`). The sum over blocks is FP32 in every mode;
 * the modes differ inside one matrix instruction:
 *   MX_ACCUM_FP32 -- codes decoded exactly to bf16 with the block scale
 *                    folded in, then bf16 MFMA with FP32-level accumulation;
 *                    half the peak rate of MX_ACCUM_FP8. Every output meets
 *                    |y - y_ref| <= 1e-5 * sum_k |a_k b_k| over the whole
 *                    E8M0 range, wherever that sum lies between 2^-100 and
 *                    2^120 (smaller sums fall under the f32 grid, larger ones
 *                    may overflow a partial sum). The fold is exact for scale
 *                    codes 10..246 (E4M3) / 17..239 (E5M2); a block with a
 *                    scale outside that window and a non-zero code is added
 *                    afterwards by an exact pass on the same kernel (slower;
 *                    all-zero blocks, e.g. code-0 padding, never start it).
 *                    E5M2 Inf codes under such a scale give NaN.
 * In every mode a block under the NaN scale code 0xFF is NaN, so every output
 * it enters is NaN, also when its element codes are all zero (the FP32 mode
 * routes such blocks through the exact pass; the FP8 instruction does so by
 * itself).
 *   MX_ACCUM_AUTO -- the same as MX_ACCUM_FP32 (E4M3 / E5M2 operands; for
 *                    E2M1 operands see below).
 *   MX_ACCUM_FP8  -- the scaled FP8 matrix instructions on the codes
 *                    (v_mfma_scale_f32_16x16x128_f8f6f4 / _32x32x64_), peak
 *                    rate, E8M0 scales applied by the instruction over the
 *                    whole range. On gfx950 these instructions add the
 *                    products of each group of 8 consecutive k with only about
 *                    14 significant bits, aligned to the group's largest
 *                    product (measured), so each group may lose up to ~2^-13
 *                    of that product: |err| <= ~2^-13 * sum|a b| in the worst
 *                    case, reached when a few products dominate an output.
 *                    Measured worst |err| / sum|a b| on every output: N(0,1)
 *                    E4M3 at 8192^3 1.6e-6, |N(0,1)| (same sign) at K = 2048
 *                    5.5e-6, Student-t (nu = 3) at K = 8192 8.4e-5 -- so the
 *                    1e-5 bound holds on data whose per-group errors cancel,
 *                    not on heavy-tailed data. [FP8DS §6.1-§6.3] discusses the
 *                    same kind of limited-precision accumulation in FP8 tensor
 *                    cores.
 *
 * E2M1 operands [NVFP4 §5.5; SM120 §0.3: the block-scaled instruction kind
 * names A's and B's element formats separately]: MXFP4 x MXFP4, or E2M1
 * against E4M3 / E5M2 on either side; codes packed two per byte, so the
 * E2M1 operand's pitch is in bytes >= K/2. Every shape mx_gemm takes
 * (K % 32 == 0, any M and N, paged B included) and every mode:
 *   MX_ACCUM_FP8  -- the scaled matrix instruction: MXFP4 x MXFP4 on the
 *                    large-tile kernel when it fits (K % 1024 == 0,
 *                    M >= 256, N >= 256, no page table, 16-byte aligned
 *                    scale rows), otherwise and for mixed products on the
 *                    general kernel. MXFP4 x MXFP4 is exact up to the FP32
 *                    sum over groups: a product of two E2M1 values has at
 *                    most 4 significant bits, so each group of 8 fits the
 *                    instruction's accumulator. A mixed product (up to 6
 *                    significant bits per product, exponents spread by the
 *                    FP8 operand) has the grouped accumulation above:
 *                    measured worst |err| / sum|a b| 1.3e-5 on N(0,1) at
 *                    K = 96, 2.5e-4 on codes drawn from every value.
 *   MX_ACCUM_FP32 -- the general kernel's FP32-accumulation mode, exact as
 *                    for FP8 operands; E2M1 codes fold exactly for scale
 *                    codes 2..252.
 *   MX_ACCUM_AUTO -- the instruction for MXFP4 x MXFP4 (exact there), the
 *                    FP32-accumulation mode for a mixed product.
 */
typedef enum { MX_ACCUM_AUTO = 0, MX_ACCUM_FP8 = 1, MX_ACCUM_FP32 = 2 } mx_accum_t;

typedef struct mx_gemm_desc {
    int64_t M, N, K;
    const uint8_t* a;  int64_t lda;  const uint8_t* sa; int64_t ldsa; mx_fmt_t a_fmt;
    const uint8_t* b;  int64_t ldb;  const uint8_t* sb; int64_t ldsb; mx_fmt_t b_fmt;
    void* y;           int64_t ldy;  mx_dtype_t y_dtype;
    int64_t batch_outer, batch_inner;
    int64_t stride_a_outer, stride_a_inner, stride_sa_outer, stride_sa_inner;
    int64_t stride_b_outer, stride_b_inner, stride_sb_outer, stride_sb_inner;
    int64_t stride_y_outer, stride_y_inner;
    const int32_t* b_page_table;
    int64_t b_pages_per_seq, b_page_rows, b_page_stride, b_page_stride_s;
    mx_accum_t accum;
} mx_gemm_desc_t;

mx_status_t mx_gemm(const mx_gemm_desc_t* desc, hipStream_t stream);

/*
 * mx_paged_attention -- attention of MXFP8 queries over the paged MXFP8 KV
 * cache that mx_kv_quant_write fills [SM120 §0.2]: the scores Q K^T are a
 * block-scaled FP8 product (query and key scales applied per 32-element block
 * of the head dimension), V is decoded to BF16 inside the kernel, and the
 * softmax-weighted sum P V is formed from it. For query row i of sequence s
 * (token t = s * q_len + i) and query head h, with L = kv_lens[s]:
 *
 *   key j is allowed  iff  j < L  and, when causal != 0, j <= L - q_len + i
 *                          (the queries are the last q_len positions);
 *   S_j  = sum_b sq[b] * sk_j[b] * sum_{e<32} q[32b+e] * k_j[32b+e]
 *   P_j  = exp(sm_scale * S_j - max) / sum over allowed keys
 *   O[d] = sum_j P_j * bf16(v_j[d] * sv_j[d/32])
 *   lse  = log sum_j exp(sm_scale * S_j)        (natural log)
 *
 * A row with no allowed key gets O = 0 and lse = -inf. Key j of sequence s
 * is read from cache slot page_table[s * pages_per_seq + j / page_size] *
 * page_size + j % page_size, kv head h / (num_q_heads / num_kv_heads).
 *
 * Layouts (device memory, caller-owned):
 *   q        [num_seqs * q_len][num_q_heads][head_dim] E4M3 codes, token pitch ld_q bytes
 *   q_scale  [num_seqs * q_len][num_q_heads][head_dim / 32] E8M0, token pitch ld_qs bytes
 *   k_cache, v_cache [pages][page_size][num_kv_heads][head_dim] E4M3 codes
 *   k_scale, v_scale [pages][page_size][num_kv_heads][head_dim / 32] E8M0
 *   page_table int32 [num_seqs][pages_per_seq]; kv_lens int32 [num_seqs]
 *   out      [num_seqs * q_len][num_q_heads][head_dim] (out_dtype), token pitch ld_o elements
 *   lse      f32 [num_seqs * q_len][num_q_heads], or NULL
 * The caller guarantees that every page_table entry a sequence's first
 * kv_lens[s] keys reach names a valid page; kv_lens values are clamped to
 * [0, pages_per_seq * page_size].
 *
 * Arithmetic: S in FP32 from the scaled FP8 matrix instruction (each group
 * of 8 products summed with about 14 significant bits, see mx_accum_t);
 * the softmax in f32 with exp2; P rounded to bf16 for the bf16 matrix
 * instruction, its normaliser summed in f32 from the unrounded values; O
 * accumulated in FP32, then divided by the normaliser; bf16 output rounds
 * to nearest even. Scales cover the whole E8M0 range: Q and K scales go to
 * the instruction; V is decoded with its scale clamped into 10..246 (exact
 * normal bf16) and a key whose scales leave that window has the rest of its
 * scale moved onto its weight P_j, which is exact unless one key's four V
 * scales span more than 236 codes (then its blocks 2^236 and more below its
 * largest are clamped). O is formed as the f32 sum of P_j * V_jd with the
 * weights taken relative to a running reference that lags the row maximum
 * by up to 2^8, before the division by the normaliser: an output whose
 * sum_j |V_jd| times 2^8 leaves the f32 range overflows even if O itself
 * would fit. Weights below bf16's normal range after that move (in the
 * worst case those under about 2^-116 of the row's normaliser) are flushed
 * or rounded coarsely: an output may then differ by up to the sum of
 * P_j |V_jd| over such keys beyond the relative bound, which matters only
 * where a tiny weight meets a huge V value. A NaN score (e.g. under a Q or K
 * scale code 0xFF) makes its row and its lse NaN; a V block under scale code
 * 0xFF makes NaN its 32 output columns in every row that sees the key, and
 * may do so in the rows of the same 128-query tile that the causal mask
 * hides it from.
 *
 * Requirements (MX_ERR_SHAPE / MX_ERR_ALIGN otherwise): head_dim == 128;
 * num_kv_heads divides num_q_heads; page_size a multiple of 128;
 * pages_per_seq >= 1 and pages_per_seq * page_size < 2^31; sm_scale finite
 * and > 0; ld_q >= num_q_heads * 128 and a multiple of 16; ld_qs >=
 * num_q_heads * 4 and a multiple of 4; ld_o >= num_q_heads * 128 and a
 * multiple of 4; q, k_cache, v_cache 16-byte aligned; the three scale arrays
 * and lse 4-byte aligned; out 16-byte (f32) or 8-byte (bf16) aligned.
 * num_seqs == 0 or q_len == 0 launches nothing.
 */
typedef struct mx_attention_desc {
    int64_t num_seqs, q_len, num_q_heads, num_kv_heads, head_dim;
    const uint8_t* q;       int64_t ld_q;
    const uint8_t* q_scale; int64_t ld_qs;
    const uint8_t* k_cache; const uint8_t* k_scale;
    const uint8_t* v_cache; const uint8_t* v_scale;
    int64_t page_size;
    const int32_t* page_table; int64_t pages_per_seq;
    const int32_t* kv_lens;
    float sm_scale;
    int32_t causal;
    void* out;              int64_t ld_o; mx_dtype_t out_dtype;
    float* lse;
} mx_attention_desc_t;

mx_status_t mx_paged_attention(const mx_attention_desc_t* desc, hipStream_t stream);

/*
 * mx_grouped_gemm -- one block-scaled product per group over a shared K, for
 * the many small GEMMs of a mixture-of-experts layer [SM120 §1.2: grouped
 * GEMM is its own entry point, beside the single GEMM]. Group q owns rows
 * [off[q], off[q+1]) of A and of y and its own B (the expert's weights):
 *
 *   y[r][n] = sum_b sa[r][b] * sb_q[n][b] * sum_{i<32} a[r][32b+i] * b_q[n][32b+i]
 *
 *   a, sa   [total_m x K] codes / [total_m x K/32] scales, pitches lda, ldsa
 *   b, sb   group q's [N x K] codes at b + q*stride_b, scales at sb + q*stride_sb
 *   group_offsets  DEVICE int64 [groups + 1] (typically a router's output, so
 *           the host never reads it); off[0] <= off[1] <= ... are row indices.
 *           Values are clamped to [0, total_m] and a decreasing step is an
 *           empty group, so any contents keep every access in bounds; with
 *           offsets that are not nondecreasing some rows may be left out.
 *   y       [total_m x N] out (y_dtype), pitch ldy; rows outside every group
 *           are left untouched.
 * Formats and accumulation modes are those of mx_gemm (E2M1 x E2M1 included).
 * Requirements (MX_ERR_SHAPE / MX_ERR_ALIGN otherwise): K % 512 == 0 (K %
 * 1024 for E2M1), N >= 256, groups < 2^20, 16-byte aligned code and scale
 * bases, pitches and group strides, 8-byte aligned group_offsets.
 */
typedef struct mx_grouped_gemm_desc {
    int64_t groups, total_m, N, K;
    const int64_t* group_offsets;
    const uint8_t* a;  int64_t lda;  const uint8_t* sa; int64_t ldsa; mx_fmt_t a_fmt;
    const uint8_t* b;  int64_t ldb;  const uint8_t* sb; int64_t ldsb; mx_fmt_t b_fmt;
    int64_t stride_b, stride_sb;
    void* y;           int64_t ldy;  mx_dtype_t y_dtype;
    mx_accum_t accum;
} mx_grouped_gemm_desc_t;

mx_status_t mx_grouped_gemm(const mx_grouped_gemm_desc_t* desc, hipStream_t stream);

/* Static description of a status code (never NULL). */
const char* mx_status_string(mx_status_t status);

/*
 * mx_query_support -- can this library run on `device`? Returns MX_OK, or an
 * error code with *reason (if reason != NULL) set to a static explanation:
 * the (bool, reason) shape of an availability check [SM120 §2].
 */
mx_status_t mx_query_support(int device, const char** reason);

#ifdef __cplusplus
}
#endif
#endif /* MXFP8_H */
