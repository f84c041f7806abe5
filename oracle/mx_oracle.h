/*
 * mx_oracle.h -- C interface of the CPU reference (test infrastructure only;
 * see mx_oracle.c). All pointers are host pointers owned by the caller.
 * Functions returning int give 0 on success and -2 for a shape the method
 * does not define (a blocked dimension that is not a multiple of 32, or a
 * negative size).
 */
#ifndef MX_ORACLE_H
#define MX_ORACLE_H
#include <stdint.h>

#define MXO_BLOCK 32

enum { MXO_E4M3 = 0, MXO_E5M2 = 1, MXO_E2M1 = 2 };
enum { MXO_F32 = 0, MXO_BF16 = 1 };
enum { MXO_RULE_FLOOR = 0, MXO_RULE_CEIL = 1 };

double mxo_decode_e4m3(unsigned code);
double mxo_decode_e5m2(unsigned code);
double mxo_decode_e2m1(unsigned code);
double mxo_decode(int fmt, unsigned code);
double mxo_decode_e8m0(unsigned e);
unsigned mxo_encode(int fmt, double y);
unsigned mxo_scale_code(int fmt, const double* x, int64_t n);
unsigned mxo_scale_code_rule(int fmt, const double* x, int64_t n, int rule);
uint16_t mxo_double_to_bf16(double v);
double mxo_dequant_value(int fmt, unsigned code, unsigned scale);

int mxo_quantize_rows(const void* x, int xdt, int64_t rows, int64_t cols, int64_t ldx, int fmt, uint8_t* q,
                      int64_t ldq, uint8_t* s, int64_t lds);
int mxo_quantize_cols(const void* x, int xdt, int64_t rows, int64_t cols, int64_t ldx, int fmt, uint8_t* qt,
                      int64_t ldq, uint8_t* st, int64_t lds);
int mxo_quantize_rows_rule(const void* x, int xdt, int64_t rows, int64_t cols, int64_t ldx, int fmt, int rule,
                           uint8_t* q, int64_t ldq, uint8_t* s, int64_t lds);
int mxo_quantize_cols_rule(const void* x, int xdt, int64_t rows, int64_t cols, int64_t ldx, int fmt, int rule,
                           uint8_t* qt, int64_t ldq, uint8_t* st, int64_t lds);
int mxo_quantize_2d(const void* x, int xdt, int64_t rows, int64_t cols, int64_t ldx, int fmt, int rule, uint8_t* q,
                    int64_t ldq, uint8_t* s, int64_t lds, uint8_t* qt, int64_t ldqt, uint8_t* st, int64_t ldst);
int mxo_scale_broadcast(const float* s_in, int64_t ld_in, int layout, int64_t rows, int64_t cols, uint8_t* out,
                        int64_t ld_out);
int mxo_kv_quant_write(const void* k, const void* v, int dt, int64_t T, int64_t H, int64_t D, int64_t ld_token,
                       const int64_t* slot_mapping, uint8_t* k_cache, uint8_t* k_scale, uint8_t* v_cache,
                       uint8_t* v_scale, int64_t page_size, int64_t num_pages);
int mxo_dequantize(const uint8_t* q, int64_t ldq, const uint8_t* s, int64_t lds, int fmt, int64_t rows, int64_t cols,
                   void* y, int ydt, int64_t ldy);
int mxo_gemm(int64_t M, int64_t N, int64_t K, const uint8_t* a, int64_t lda, const uint8_t* sa, int64_t ldsa,
             int afmt, const uint8_t* b, int64_t ldb, const uint8_t* sb, int64_t ldsb, int bfmt, double* y,
             int64_t ldy, double* t, int64_t ldt);
int mxo_gemm_at(int64_t K, const uint8_t* a, int64_t lda, const uint8_t* sa, int64_t ldsa, int afmt, const uint8_t* b,
                int64_t ldb, const uint8_t* sb, int64_t ldsb, int bfmt, const int64_t* mi, const int64_t* ni,
                int64_t count, double* y, double* t);
int mxo_paged_attention(const uint8_t* q, const uint8_t* qs, int64_t ld_q, int64_t ld_qs, const uint8_t* kc,
                        const uint8_t* ks, const uint8_t* vc, const uint8_t* vs, const int32_t* page_table,
                        int64_t pages_per_seq, const int32_t* kv_lens, int64_t num_seqs, int64_t q_len, int64_t hq,
                        int64_t hkv, int64_t D, int64_t page_size, double sm_scale, int causal, const int64_t* rows,
                        int64_t count, double* o, double* w, double* lse, double* tmax);
int mxo_num_threads(void);
void mxo_set_num_threads(int n);

#endif
