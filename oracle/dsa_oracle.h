/*
 * dsa_oracle.h -- C interface of the CPU reference (test infrastructure only).
 * Private to oracle/: the GPU library has its own, unrelated header.
 *
 * Layouts are dense row-major host arrays:
 *   q_i     [B,T,H_I,D_I] u8 e4m3fn     q_scale, w [B,T,H_I] f32
 *   k_i     [B,Lmax,D_I]  u8 e4m3fn     k_scale    [B,Lmax]  f32      len [B] i32
 *   scores  [B,T,Lmax] f32              idx        [B,T,k]   i32 (-1 = unused slot)
 *   latent form:  q [B,T,H,Dv+Dr], latent [B,Lmax,Dv+Dr], out [B,T,H,Dv] f64, lse [B,T,H] f64
 *   MHA form:     q, k [B,T,H,Dqk], v [B,T,H,Dv], out [B,T,H,Dv] f64, lse [B,T,H] f64
 * m (compress rate): 1 = every position is a cache row; m > 1 = the key and latent caches
 * hold compressed entries and row (b,t) sees entries e < (len[b] - T + t + 1) / m.
 * Attention inputs are read as ORC_F32, ORC_BF16 (raw 16-bit words) or ORC_F64.
 * ORC_FP8_LATENT (latent form only): bf16 queries and 656-byte FP8 latent rows
 *   [512 e4m3fn codes][4 fp32 scales, one per 128 columns][64 bf16 rope values],
 *   latent [B,Lmax,656] u8, Dv = 512, Dr = 64.
 */
#ifndef DSA_ORACLE_H
#define DSA_ORACLE_H
#include <stdint.h>

enum { ORC_OK = 0, ORC_ERR_SHAPE = 1, ORC_ERR_INDEX = 2 };
enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_F64 = 2, ORC_FP8_LATENT = 3 };
enum { ORC_FP8_LATENT_DV = 512, ORC_FP8_LATENT_DR = 64, ORC_FP8_LATENT_BLOCK = 128,
       ORC_FP8_LATENT_ROW_BYTES = 656 };

double orc_e4m3fn_value(uint8_t code);
double orc_bf16_value(uint16_t bits);
double orc_latent_fp8_value(const uint8_t* row, int d);
uint8_t orc_e4m3fn_encode(double y);

int orc_indexer_prep(const void* q, const void* k, int dtype, const float* cosT, const float* sinT,
                     int P, const int32_t* start, int B, int T, int H, int D, int R, int Lmax,
                     uint8_t* q_fp8, double* q_scale64, uint8_t* k_cache, float* k_scale,
                     double* k_scale64, double* q_y, double* k_y);

int orc_index_scores(const uint8_t* q, const float* q_scale, const float* w,
                     const uint8_t* k, const float* k_scale, const int32_t* len,
                     int B, int T, int H, int D, int Lmax, double sm_scale, int m, float* scores);

int orc_topk(const float* scores, const int32_t* len, int B, int T, int Lmax, int k, int m,
             int32_t* idx);

int orc_sparse_mla_decode(const void* q, const void* latent, const int32_t* idx,
                          const int32_t* len, int dtype, int B, int T, int H, int Dv, int Dr,
                          int Lmax, int k, double sm_scale, int m, double* out, double* lse);

int orc_sparse_mha_prefill(const void* q, const void* kk, const void* v, const int32_t* idx,
                           int dtype, int B, int T, int H, int Dqk, int Dv, int k,
                           double sm_scale, double* out, double* lse);

int orc_sparse_mha_prefill_rows(const void* q, const void* kk, const void* v, const int32_t* idx,
                                int dtype, int B, int T, int H, int Dqk, int Dv, int k,
                                double sm_scale, const int32_t* rows_b, const int32_t* rows_t,
                                int n_rows, double* out, double* lse);

int orc_sparse_mha_prefill_dense(const void* q, const void* kk, const void* v,
                                 const int32_t* idx, int dtype, int B, int T, int H, int Dqk,
                                 int Dv, int k, double sm_scale, double* out, double* lse);

int orc_layer_step_latent(const uint8_t* q_i, const float* q_scale, const float* w,
                          const uint8_t* k_i, const float* k_scale, const int32_t* len,
                          int B, int T, int H_I, int D_I, int Lmax, double sm_scale_i, int k,
                          const void* q, const void* latent, int dtype, int H, int Dv, int Dr,
                          double sm_scale, int m, double* out, double* lse, float* scores_out,
                          int32_t* idx_out);

int orc_layer_step_mha(const uint8_t* q_i, const float* q_scale, const float* w,
                       const uint8_t* k_i, const float* k_scale, int B, int T, int H_I, int D_I,
                       double sm_scale_i, int k, const void* q, const void* kk, const void* v,
                       int dtype, int H, int Dqk, int Dv, double sm_scale, double* out,
                       double* lse, float* scores_out, int32_t* idx_out);

int orc_max_threads(void);
void orc_set_threads(int n);

#endif
