// dsa_internal.h -- host-side launch interface between the C ABI (dsa_abi.cpp) and the
// kernel translation units.  Arguments are validated by the caller.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dsa {

// Phases of one layer step, for the optional kernel timing of dsa_profile_begin/_end.
enum Phase { kPhaseIndex = 0, kPhaseTopk = 1, kPhaseAttention = 2, kPhaseCombine = 3,
             kPhaseCount = 4, kPhaseNone = -1 };
// While profiling is on: a fresh start/stop event pair for the next kernel of `phase`
// (false when profiling is off or the pool is used up).
bool prof_kernel_events(int phase, hipEvent_t* start, hipEvent_t* stop);

// Launch of a kernel that belongs to `phase`.  While profiling is on, the start and stop
// events are part of the dispatch itself (hipExtLaunchKernelGGL), so they time the
// kernel's own execution, without the gaps between kernels.
template <typename... KArgs, typename... Args>
hipError_t launch_kernel(int phase, void (*kernel)(KArgs...), dim3 grid, dim3 block, uint32_t shmem,
                         hipStream_t stream, Args... args) {
    hipEvent_t e0, e1;
    if (phase != kPhaseNone && prof_kernel_events(phase, &e0, &e1))
        hipExtLaunchKernelGGL(kernel, grid, block, shmem, stream, e0, e1, 0u, static_cast<KArgs>(args)...);
    else
        hipLaunchKernelGGL(kernel, grid, block, shmem, stream, static_cast<KArgs>(args)...);
    return hipGetLastError();
}

struct IndexScoresArgs {
    const uint8_t* q;
    const float* q_scale;
    const float* w;
    const uint8_t* k;
    const float* k_scale;
    const int32_t* len;
    int B, T, H, D, Lmax;
    float sm_scale;
    float* scores;
    int fill_invisible;   // write -inf into every invisible position (else only near pos)
    int m;                // compress rate (1: every position is a cache row; see n_visible)
};
hipError_t launch_index_scores(const IndexScoresArgs& a, hipStream_t stream);

// Indexer preparation of the T new tokens of each sequence (rope, rotation, FP8
// quantisation, key-cache append); token t of sequence b sits at position start[b] + t.
struct IndexerPrepArgs {
    const void* q;          // [B,T,H,D] bf16 or f32
    const void* k;          // [B,T,D]
    int bf16;
    const float* cos;       // [P, R/2]
    const float* sin;       // [P, R/2]
    int P;
    const int32_t* start;   // [B]
    int B, T, H, D, R, Lmax;
    uint8_t* q_fp8;         // [B,T,H,D]
    float* q_scale;         // [B,T,H]
    uint8_t* k_cache;       // [B,Lmax,D]
    float* k_scale;         // [B,Lmax]
};
hipError_t launch_indexer_prep(const IndexerPrepArgs& a, hipStream_t stream);

struct TopkArgs {
    const float* scores;
    const int32_t* len;
    int B, T, Lmax, k;
    int32_t* idx;
    int m;                // compress rate (see n_visible)
};
size_t topk_workspace_bytes(int B, int T, int Lmax, int k);
hipError_t launch_topk(const TopkArgs& a, void* ws, hipStream_t stream);

// Element types of the latent form (the values of the ABI's dsa_dtype).  kLatFp8: bf16
// queries and outputs, cache rows of 656 bytes -- 512 e4m3fn codes, four fp32 scales (one
// per 128 columns), 64 bf16 rope values.
enum LatentType { kLatF32 = 0, kLatBf16 = 1, kLatFp8 = 2 };
constexpr int kFp8RowBytes = 656;
constexpr int kFp8Dv = 512;
constexpr int kFp8Dr = 64;

// Sparse attention over gathered rows.  Keys of row (b,t) for head h are read at
//   kbase + (b * kv_rows + s) * row_stride + h * head_stride   (Dk values)
// and values at
//   vbase + (b * kv_rows + s) * row_stride_v + h * head_stride_v (Dv values).
struct SparseAttnArgs {
    const void* q;          // [B,T,H,Dk]
    const void* kbase;
    const void* vbase;
    const int32_t* idx;     // [B,T,k]
    const int32_t* len;     // [B] (latent form) or NULL (MHA chunk from 0: pos = t)
    int B, T, H, Dk, Dv, k, kv_rows;
    size_t row_stride, head_stride, row_stride_v, head_stride_v;   // in elements
    float sm_scale;
    int bf16;               // element type: 1 bf16, 0 f32
    int fp8_latent;         // keys and values are 656-byte FP8 latent rows at kbase
                            // (row = b * kv_rows + s; strides unused); q, out bf16
    void* out;              // [B,T,H,Dv]
    float* lse;             // [B,T,H] or NULL
    int m;                  // compress rate (latent form; see n_visible)
};
hipError_t launch_sparse_attn_generic(const SparseAttnArgs& a, hipStream_t stream);

// Matrix-core path of the absorbed latent form (bf16 or FP8 rows, Dv = 512, Dr = 64,
// H = 64 or 128).  `type` is a LatentType.
bool mla_decode_mfma_supported(int H, int Dv, int Dr, int k, int type);
size_t mla_decode_workspace_bytes(int B, int T, int H, int Dv, int k, int type);
hipError_t launch_mla_decode_mfma(const void* q, const void* latent, const int32_t* idx,
                                  const int32_t* len, int B, int T, int H, int Lmax, int k,
                                  float sm_scale, int type, int m, void* out, float* lse, void* ws,
                                  hipStream_t stream);

// The 32x32x16 matrix-core kernel of the bf16 latent form (sparse_mla_decode32.hip): 64
// heads per workgroup (H = 64 or 128), at most mla_decode32_max_tiles() tiles of 32 slots
// per split.  Launches rows * n_splits * (H / 64) workgroups; with n_splits > 1 each split
// writes its normalised bf16 rows to part_o [rows][n_splits][H][512] and its log2-sum-exp
// to part_lse [rows][n_splits][H], which mla_combine_kernel merges.
bool mla_decode32_supported(int H, int k);
int mla_decode32_max_tiles();
hipError_t launch_mla_decode32(const void* q, const void* latent, const int32_t* idx,
                               const int32_t* len, int rows, int T, int H, int Lmax, int k, int m,
                               int tiles_per_split, int n_splits, float scale_log2, void* out,
                               float* lse, void* part_o, float* part_lse, hipStream_t stream);

// The same for latent rows in the 656-byte FP8 form (sparse_mla_decode32_fp8.hip): tiles of
// mla_decode32_fp8_tile_rows() slots, at most mla_decode32_fp8_max_tiles() per split;
// partials and the combine as above.
int mla_decode32_fp8_max_tiles();
int mla_decode32_fp8_tile_rows();
hipError_t launch_mla_decode32_fp8(const void* q, const void* latent, const int32_t* idx,
                                   const int32_t* len, int rows, int T, int H, int Lmax, int k, int m,
                                   int tiles_per_split, int n_splits, float scale_log2, void* out,
                                   float* lse, void* part_o, float* part_lse, hipStream_t stream);

// Matrix-core path of the MHA prefill form (bf16, Dqk = 192, Dv = 128).
bool mha_prefill_mfma_supported(int Dqk, int Dv, int bf16);
// the matrix-core prefill path: a supported shape and a finite, positive softmax scale
bool mha_prefill_mfma_path(int Dqk, int Dv, int bf16, float sm_scale);
size_t mha_prefill_workspace_bytes(int B, int T);
// Diagnostic: n (a multiple of 16) dot products of 128 FP8 codes, row p of a with row p
// of b, on the FP8 and on the bf16 matrix-core forms.
hipError_t launch_diag_fp8_dots(const uint8_t* a, const uint8_t* b, int n, float* out_fp8,
                                float* out_bf16, hipStream_t stream);
hipError_t launch_mha_prefill_mfma(const void* q, const void* k, const void* v, const int32_t* idx,
                                   int B, int T, int H, int topk, float sm_scale, void* out,
                                   float* lse, void* ws, hipStream_t stream);

}  // namespace dsa
