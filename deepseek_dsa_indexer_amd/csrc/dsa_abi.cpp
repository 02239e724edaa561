// dsa_abi.cpp -- the extern "C" entry points of libdsa_amd: argument validation,
// workspace carving and kernel launches on the caller's stream.  See include/dsa.h for
// the contract of each call.
#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/dsa.h"
#include "dsa_internal.h"

namespace {

thread_local std::string g_last_error;

dsa_status fail(dsa_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t round_up(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

dsa_status hip_status(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(DSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return DSA_OK;
}

constexpr size_t kProfPairsPerStep = 6;   // kernels per layer step, at most

#define DSA_REQUIRE(cond, st, ...) \
    do {                           \
        if (!(cond)) return fail(st, __VA_ARGS__); \
    } while (0)

constexpr long long kMaxRows = 1LL << 30;

dsa_status check_index_args(const uint8_t* q_fp8, const float* q_scale, const float* w,
                            const uint8_t* k_fp8, const float* k_scale, const int32_t* len,
                            int B, int T, int H_I, int d_I, int Lmax, int m = 1) {
    DSA_REQUIRE(q_fp8 && q_scale && w && k_fp8 && k_scale && len, DSA_ERR_NULL,
                "index scores: NULL input pointer");
    // with compressed entries (m > 1) the T rows are positions, the Lmax rows entries
    DSA_REQUIRE(B >= 1 && T >= 1 && Lmax >= 1 && (T <= Lmax || m > 1), DSA_ERR_SHAPE,
                "index scores: need B >= 1 and 1 <= T <= Lmax (B=%d T=%d Lmax=%d)", B, T, Lmax);
    DSA_REQUIRE(static_cast<long long>(B) * T <= kMaxRows, DSA_ERR_SHAPE, "index scores: B*T too large");
    DSA_REQUIRE(H_I >= 1 && H_I <= 64, DSA_ERR_SHAPE, "index scores: H_I=%d not in [1, 64]", H_I);
    DSA_REQUIRE(d_I == 32 || d_I == 64 || d_I == 128, DSA_ERR_SHAPE,
                "index scores: d_I=%d not in {32, 64, 128}", d_I);
    DSA_REQUIRE(aligned16(q_fp8) && aligned16(q_scale) && aligned16(w) && aligned16(k_fp8) &&
                    aligned16(k_scale) && aligned16(len),
                DSA_ERR_ALIGN, "index scores: inputs must be 16-byte aligned");
    return DSA_OK;
}

dsa_status check_topk_args(const float* scores, const int32_t* len, int B, int T, int Lmax, int k,
                           const int32_t* idx) {
    DSA_REQUIRE(scores && len && idx, DSA_ERR_NULL, "topk: NULL pointer");
    DSA_REQUIRE(B >= 1 && T >= 1 && Lmax >= 1 && T <= Lmax && k >= 1, DSA_ERR_SHAPE,
                "topk: need B, T, k >= 1 and T <= Lmax (B=%d T=%d Lmax=%d k=%d)", B, T, Lmax, k);
    DSA_REQUIRE(static_cast<long long>(B) * T <= kMaxRows, DSA_ERR_SHAPE, "topk: B*T too large");
    DSA_REQUIRE(aligned16(scores) && aligned16(len) && aligned16(idx), DSA_ERR_ALIGN,
                "topk: pointers must be 16-byte aligned");
    return DSA_OK;
}

constexpr size_t kGenericLdsLimit = 64 * 1024;
static_assert(static_cast<int>(DSA_F32) == dsa::kLatF32 && static_cast<int>(DSA_BF16) == dsa::kLatBf16 &&
                  static_cast<int>(DSA_FP8_LATENT) == dsa::kLatFp8,
              "dsa_dtype values are the kernels' latent types");

dsa_status check_latent_args(const void* q, const void* latent, const int32_t* idx,
                             const int32_t* len, int B, int T, int H, int Dv, int Dr, int Lmax,
                             int k, dsa_dtype dt, const void* out, int m = 1) {
    DSA_REQUIRE(q && latent && idx && len && out, DSA_ERR_NULL, "sparse_mla_decode: NULL pointer");
    DSA_REQUIRE(dt == DSA_F32 || dt == DSA_BF16 || dt == DSA_FP8_LATENT, DSA_ERR_DTYPE,
                "sparse_mla_decode: bad dtype %d", static_cast<int>(dt));
    DSA_REQUIRE(dt != DSA_FP8_LATENT || (Dv == dsa::kFp8Dv && Dr == dsa::kFp8Dr), DSA_ERR_DTYPE,
                "sparse_mla_decode: FP8 latent rows need Dv=512, Dr=64 (got Dv=%d Dr=%d)", Dv, Dr);
    DSA_REQUIRE(B >= 1 && T >= 1 && Lmax >= 1 && (T <= Lmax || m > 1) && H >= 1 && Dv >= 1 &&
                    Dr >= 0 && Dv + Dr <= 1024 && k >= 1,
                DSA_ERR_SHAPE, "sparse_mla_decode: bad shape (B=%d T=%d H=%d Dv=%d Dr=%d Lmax=%d k=%d)",
                B, T, H, Dv, Dr, Lmax, k);
    DSA_REQUIRE(static_cast<long long>(B) * T * H <= kMaxRows, DSA_ERR_SHAPE,
                "sparse_mla_decode: B*T*H too large");
    DSA_REQUIRE(aligned16(q) && aligned16(latent) && aligned16(idx) && aligned16(len) && aligned16(out),
                DSA_ERR_ALIGN, "sparse_mla_decode: pointers must be 16-byte aligned");
    if (!dsa::mla_decode_mfma_supported(H, Dv, Dr, k, dt))
        DSA_REQUIRE(sizeof(float) * (static_cast<size_t>(Dv + Dr) + k) <= kGenericLdsLimit, DSA_ERR_SHAPE,
                    "sparse_mla_decode: k=%d too large for this shape", k);
    return DSA_OK;
}

dsa_status launch_latent(const void* q, const void* latent, const int32_t* idx, const int32_t* len,
                         int B, int T, int H, int Dv, int Dr, int Lmax, int k, float sm_scale,
                         dsa_dtype dt, void* out, float* lse, void* ws, hipStream_t stream, int m) {
    if (dsa::mla_decode_mfma_supported(H, Dv, Dr, k, dt))
        return hip_status(dsa::launch_mla_decode_mfma(q, latent, idx, len, B, T, H, Lmax, k, sm_scale,
                                                      dt, m, out, lse, ws, stream),
                          "sparse_mla_decode");
    dsa::SparseAttnArgs a{};
    a.q = q;
    a.kbase = latent;
    a.vbase = latent;
    a.idx = idx;
    a.len = len;
    a.B = B; a.T = T; a.H = H; a.Dk = Dv + Dr; a.Dv = Dv; a.k = k; a.kv_rows = Lmax;
    a.row_stride = static_cast<size_t>(Dv + Dr);
    a.head_stride = 0;
    a.row_stride_v = static_cast<size_t>(Dv + Dr);
    a.head_stride_v = 0;
    a.sm_scale = sm_scale;
    a.bf16 = dt != DSA_F32;
    a.fp8_latent = dt == DSA_FP8_LATENT;
    a.out = out;
    a.lse = lse;
    a.m = m;
    return hip_status(dsa::launch_sparse_attn_generic(a, stream), "sparse_mla_decode");
}

size_t latent_ws(int B, int T, int H, int Dv, int Dr, int k, dsa_dtype dt) {
    if (dsa::mla_decode_mfma_supported(H, Dv, Dr, k, dt))
        return dsa::mla_decode_workspace_bytes(B, T, H, Dv, k, dt);
    return 0;
}

dsa_status check_mha_args(const void* q, const void* k, const void* v, const int32_t* idx, int B,
                          int T, int H, int Dqk, int Dv, int topk, float sm_scale, dsa_dtype dt,
                          const void* out) {
    DSA_REQUIRE(q && k && v && idx && out, DSA_ERR_NULL, "sparse_mla_prefill: NULL pointer");
    DSA_REQUIRE(dt == DSA_F32 || dt == DSA_BF16, DSA_ERR_DTYPE, "sparse_mla_prefill: bad dtype %d",
                static_cast<int>(dt));
    DSA_REQUIRE(B >= 1 && T >= 1 && H >= 1 && Dqk >= 1 && Dqk <= 1024 && Dv >= 1 && Dv <= 1024 &&
                    topk >= 1,
                DSA_ERR_SHAPE, "sparse_mla_prefill: bad shape (B=%d T=%d H=%d Dqk=%d Dv=%d k=%d)", B, T,
                H, Dqk, Dv, topk);
    DSA_REQUIRE(static_cast<long long>(B) * T * H <= kMaxRows, DSA_ERR_SHAPE,
                "sparse_mla_prefill: B*T*H too large");
    DSA_REQUIRE(aligned16(q) && aligned16(k) && aligned16(v) && aligned16(idx) && aligned16(out),
                DSA_ERR_ALIGN, "sparse_mla_prefill: pointers must be 16-byte aligned");
    if (!dsa::mha_prefill_mfma_path(Dqk, Dv, dt == DSA_BF16, sm_scale))
        DSA_REQUIRE(sizeof(float) * (static_cast<size_t>(Dqk) + topk) <= kGenericLdsLimit, DSA_ERR_SHAPE,
                    "sparse_mla_prefill: k=%d too large for this shape", topk);
    return DSA_OK;
}

dsa_status launch_mha(const void* q, const void* k, const void* v, const int32_t* idx, int B, int T,
                      int H, int Dqk, int Dv, int topk, float sm_scale, dsa_dtype dt, void* out,
                      float* lse, void* ws, hipStream_t stream) {
    if (dsa::mha_prefill_mfma_path(Dqk, Dv, dt == DSA_BF16, sm_scale))
        return hip_status(dsa::launch_mha_prefill_mfma(q, k, v, idx, B, T, H, topk, sm_scale, out, lse,
                                                       ws, stream),
                          "sparse_mla_prefill");
    dsa::SparseAttnArgs a{};
    a.q = q;
    a.kbase = k;
    a.vbase = v;
    a.idx = idx;
    a.len = nullptr;
    a.B = B; a.T = T; a.H = H; a.Dk = Dqk; a.Dv = Dv; a.k = topk; a.kv_rows = T;
    a.row_stride = static_cast<size_t>(H) * Dqk;
    a.head_stride = static_cast<size_t>(Dqk);
    a.row_stride_v = static_cast<size_t>(H) * Dv;
    a.head_stride_v = static_cast<size_t>(Dv);
    a.sm_scale = sm_scale;
    a.bf16 = dt == DSA_BF16;
    a.out = out;
    a.lse = lse;
    a.m = 1;
    return hip_status(dsa::launch_sparse_attn_generic(a, stream), "sparse_mla_prefill");
}

size_t mha_ws(int B, int T, int, int Dqk, int Dv, int, dsa_dtype dt) {
    if (dsa::mha_prefill_mfma_supported(Dqk, Dv, dt == DSA_BF16)) return dsa::mha_prefill_workspace_bytes(B, T);
    return 0;
}

// Kernel timing of dsa_layer_step phases (dsa_profile_begin / dsa_profile_end): one
// start/stop event pair per kernel, recorded by the dispatch itself.
struct Profiler {
    bool on = false;
    std::vector<hipEvent_t> pool;     // pairs: 2 i (start), 2 i + 1 (stop)
    std::vector<int> label;           // phase of pair i
    size_t used = 0;                  // pairs handed out
};
Profiler g_prof;

// Library-owned scratch of dsa_layer_step_noalloc: one array per GPU, in the code object's
// device memory (the loader places it when the library's code is loaded on a device and
// keeps it until the process ends).  Host code never uses the array's own name as an
// address: each device's copy is looked up once with hipGetSymbolAddress, with that
// device current, and only that pointer is passed to kernels.
constexpr size_t kStaticScratchBytes = static_cast<size_t>(DSA_NOALLOC_SCRATCH_BYTES);
__device__ __attribute__((aligned(256))) uint8_t scratch[kStaticScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// This device's copy of `scratch` (looked up on the first call on the device).
dsa_status device_scratch(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(DSA_ERR_HIP, "layer step (no alloc): hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return fail(DSA_ERR_HIP, "layer step (no alloc): device %d beyond %d", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr)
            return fail(DSA_ERR_HIP, "layer step (no alloc): hipGetSymbolAddress: %s", hipGetErrorString(e));
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return DSA_OK;
}

}  // namespace

bool dsa::prof_kernel_events(int phase, hipEvent_t* start, hipEvent_t* stop) {
    if (!g_prof.on || 2 * (g_prof.used + 1) > g_prof.pool.size()) return false;
    *start = g_prof.pool[2 * g_prof.used];
    *stop = g_prof.pool[2 * g_prof.used + 1];
    g_prof.label[g_prof.used] = phase;
    ++g_prof.used;
    return true;
}

extern "C" {

dsa_status dsa_profile_begin(int max_steps) {
    DSA_REQUIRE(max_steps >= 1 && max_steps <= (1 << 20), DSA_ERR_SHAPE,
                "profile: max_steps=%d out of range", max_steps);
    DSA_REQUIRE(!g_prof.on, DSA_ERR_SHAPE, "profile: already running");
    const size_t pairs = static_cast<size_t>(max_steps) * kProfPairsPerStep;
    const size_t n = 2 * pairs;
    g_prof.pool.resize(n);
    g_prof.label.assign(pairs, dsa::kPhaseNone);
    for (size_t i = 0; i < n; ++i) {
        hipError_t e = hipEventCreate(&g_prof.pool[i]);
        if (e != hipSuccess) {
            for (size_t j = 0; j < i; ++j) (void)hipEventDestroy(g_prof.pool[j]);
            g_prof.pool.clear();
            return hip_status(e, "profile: hipEventCreate");
        }
    }
    g_prof.used = 0;
    g_prof.on = true;
    return DSA_OK;
}

dsa_status dsa_profile_end(double* ms_total, int* counts) {
    DSA_REQUIRE(ms_total && counts, DSA_ERR_NULL, "profile: NULL output");
    DSA_REQUIRE(g_prof.on, DSA_ERR_SHAPE, "profile: not running");
    for (int p = 0; p < dsa::kPhaseCount; ++p) { ms_total[p] = 0.0; counts[p] = 0; }
    dsa_status st = DSA_OK;
    if (g_prof.used > 0) {
        st = hip_status(hipEventSynchronize(g_prof.pool[2 * g_prof.used - 1]), "profile: sync");
        for (size_t i = 0; st == DSA_OK && i < g_prof.used; ++i) {
            const int p = g_prof.label[i];
            if (p < 0) continue;
            float ms = 0.f;
            st = hip_status(hipEventElapsedTime(&ms, g_prof.pool[2 * i], g_prof.pool[2 * i + 1]),
                            "profile: elapsed time");
            ms_total[p] += ms;
            counts[p] += 1;
        }
    }
    for (hipEvent_t e : g_prof.pool) (void)hipEventDestroy(e);
    g_prof.pool.clear();
    g_prof.label.clear();
    g_prof.used = 0;
    g_prof.on = false;
    return st;
}

const char* dsa_last_error(void) { return g_last_error.c_str(); }

int dsa_version(void) { return 100; }

dsa_status dsa_indexer_prep(const void* q, const void* k, dsa_dtype dt, const float* rope_cos,
                            const float* rope_sin, int P, const int32_t* start, int B, int T,
                            int H_I, int d_I, int rope_dim, int Lmax, uint8_t* q_fp8,
                            float* q_scale, uint8_t* k_cache, float* k_scale, hipStream_t stream) {
    DSA_REQUIRE(q && k && start && q_fp8 && q_scale && k_cache && k_scale, DSA_ERR_NULL,
                "indexer prep: NULL pointer");
    DSA_REQUIRE(rope_dim == 0 || (rope_cos && rope_sin), DSA_ERR_NULL, "indexer prep: NULL rope table");
    DSA_REQUIRE(dt == DSA_F32 || dt == DSA_BF16, DSA_ERR_DTYPE, "indexer prep: bad dtype %d",
                static_cast<int>(dt));
    DSA_REQUIRE(B >= 1 && T >= 1 && Lmax >= 1 && T <= Lmax && P >= 1, DSA_ERR_SHAPE,
                "indexer prep: need B, T, P >= 1 and T <= Lmax (B=%d T=%d P=%d Lmax=%d)", B, T, P, Lmax);
    DSA_REQUIRE(static_cast<long long>(B) * T <= (1LL << 26), DSA_ERR_SHAPE,
                "indexer prep: B*T too large (one wave per row, at most 2^26 tokens)");
    DSA_REQUIRE(H_I >= 1 && H_I <= 64, DSA_ERR_SHAPE, "indexer prep: H_I=%d not in [1, 64]", H_I);
    DSA_REQUIRE(d_I == 32 || d_I == 64 || d_I == 128, DSA_ERR_SHAPE,
                "indexer prep: d_I=%d not in {32, 64, 128}", d_I);
    DSA_REQUIRE(rope_dim == 0 || (rope_dim >= 4 && rope_dim <= d_I && (rope_dim & (rope_dim - 1)) == 0),
                DSA_ERR_SHAPE, "indexer prep: rope_dim=%d must be 0 or a power of two in [4, d_I]",
                rope_dim);
    DSA_REQUIRE(aligned16(q) && aligned16(k) && aligned16(start) && aligned16(q_fp8) &&
                    aligned16(q_scale) && aligned16(k_cache) && aligned16(k_scale) &&
                    (rope_dim == 0 || (aligned16(rope_cos) && aligned16(rope_sin))),
                DSA_ERR_ALIGN, "indexer prep: pointers must be 16-byte aligned");
    dsa::IndexerPrepArgs a{q, k, dt == DSA_BF16, rope_cos, rope_sin, P, start, B, T, H_I, d_I,
                           rope_dim, Lmax, q_fp8, q_scale, k_cache, k_scale};
    return hip_status(dsa::launch_indexer_prep(a, stream), "indexer prep");
}

dsa_status dsa_index_scores(const uint8_t* q_fp8, const float* q_scale, const float* w,
                            const uint8_t* k_fp8, const float* k_scale, const int32_t* len, int B,
                            int T, int H_I, int d_I, int Lmax, float sm_scale_I, float* scores,
                            hipStream_t stream) {
    dsa_status st = check_index_args(q_fp8, q_scale, w, k_fp8, k_scale, len, B, T, H_I, d_I, Lmax);
    if (st != DSA_OK) return st;
    DSA_REQUIRE(scores, DSA_ERR_NULL, "index scores: NULL output");
    DSA_REQUIRE(aligned16(scores), DSA_ERR_ALIGN, "index scores: output must be 16-byte aligned");
    dsa::IndexScoresArgs a{q_fp8, q_scale, w, k_fp8, k_scale, len, B, T, H_I, d_I, Lmax, sm_scale_I,
                           scores, 1, 1};
    return hip_status(dsa::launch_index_scores(a, stream), "index scores");
}

size_t dsa_topk_workspace_bytes(int B, int T, int Lmax, int k) {
    return dsa::topk_workspace_bytes(B, T, Lmax, k);
}

dsa_status dsa_topk(const float* scores, const int32_t* len, int B, int T, int Lmax, int k,
                    int32_t* idx, void* ws, size_t ws_bytes, hipStream_t stream) {
    dsa_status st = check_topk_args(scores, len, B, T, Lmax, k, idx);
    if (st != DSA_OK) return st;
    const size_t need = dsa::topk_workspace_bytes(B, T, Lmax, k);
    DSA_REQUIRE(need == 0 || (ws && ws_bytes >= need), DSA_ERR_WORKSPACE,
                "topk: workspace of %zu bytes required", need);
    dsa::TopkArgs a{scores, len, B, T, Lmax, k, idx, 1};
    return hip_status(dsa::launch_topk(a, ws, stream), "topk");
}

size_t dsa_sparse_mla_decode_workspace_bytes(int B, int T, int H, int Dv, int Dr, int k, dsa_dtype dt) {
    if (B < 1 || T < 1 || H < 1 || Dv < 1 || Dr < 0 || k < 1) return 0;
    return latent_ws(B, T, H, Dv, Dr, k, dt);
}

dsa_status dsa_sparse_mla_decode(const void* q, const void* latent, const int32_t* idx,
                                 const int32_t* len, int B, int T, int H, int Dv, int Dr, int Lmax,
                                 int k, float sm_scale, dsa_dtype dt, void* out, float* lse, void* ws,
                                 size_t ws_bytes, hipStream_t stream) {
    dsa_status st = check_latent_args(q, latent, idx, len, B, T, H, Dv, Dr, Lmax, k, dt, out);
    if (st != DSA_OK) return st;
    DSA_REQUIRE(lse == nullptr || aligned16(lse), DSA_ERR_ALIGN, "sparse_mla_decode: lse alignment");
    const size_t need = latent_ws(B, T, H, Dv, Dr, k, dt);
    DSA_REQUIRE(need == 0 || (ws && ws_bytes >= need && aligned16(ws)), DSA_ERR_WORKSPACE,
                "sparse_mla_decode: workspace of %zu bytes required (got %zu)", need, ws_bytes);
    return launch_latent(q, latent, idx, len, B, T, H, Dv, Dr, Lmax, k, sm_scale, dt, out, lse, ws,
                         stream, 1);
}

size_t dsa_sparse_mla_prefill_workspace_bytes(int B, int T, int H, int Dqk, int Dv, int topk,
                                              dsa_dtype dt) {
    return mha_ws(B, T, H, Dqk, Dv, topk, dt);
}

dsa_status dsa_sparse_mla_prefill(const void* q, const void* k, const void* v, const int32_t* idx,
                                  int B, int T, int H, int Dqk, int Dv, int topk, float sm_scale,
                                  dsa_dtype dt, void* out, float* lse, void* ws, size_t ws_bytes,
                                  hipStream_t stream) {
    dsa_status st = check_mha_args(q, k, v, idx, B, T, H, Dqk, Dv, topk, sm_scale, dt, out);
    if (st != DSA_OK) return st;
    DSA_REQUIRE(lse == nullptr || aligned16(lse), DSA_ERR_ALIGN, "sparse_mla_prefill: lse alignment");
    const size_t need = mha_ws(B, T, H, Dqk, Dv, topk, dt);
    DSA_REQUIRE(need == 0 || (ws && ws_bytes >= need && aligned16(ws)), DSA_ERR_WORKSPACE,
                "sparse_mla_prefill: workspace of %zu bytes required (got %zu)", need, ws_bytes);
    return launch_mha(q, k, v, idx, B, T, H, Dqk, Dv, topk, sm_scale, dt, out, lse, ws, stream);
}

// Workspace layout of the layer step: [scores][idx][scratch], 256-byte aligned.  The
// scratch part serves the top-k candidates first and the attention partials after (the
// two never overlap in time on the stream).
static void layer_ws_parts(const dsa_layer_args* a, size_t* s_bytes, size_t* i_bytes, size_t* att) {
    const size_t rows = static_cast<size_t>(a->B) * a->T;
    *s_bytes = a->scores_out ? 0 : round_up(rows * a->Lmax * sizeof(float));
    *i_bytes = a->idx_out ? 0 : round_up(rows * a->topk * sizeof(int32_t));
    const size_t tk = dsa::topk_workspace_bytes(a->B, a->T, a->Lmax, a->topk);
    if (a->form == DSA_ATTN_LATENT)
        *att = round_up(std::max(tk, latent_ws(a->B, a->T, a->H, a->Dv, a->Dr, a->topk, a->dtype)));
    else
        *att = round_up(std::max(tk, mha_ws(a->B, a->T, a->H, a->Dqk, a->Dv, a->topk, a->dtype)));
}

size_t dsa_layer_step_workspace_bytes(const dsa_layer_args* a) {
    if (!a || a->B < 1 || a->T < 1 || a->Lmax < 1 || a->topk < 1) return 0;
    size_t s, i, t;
    layer_ws_parts(a, &s, &i, &t);
    return s + i + t;
}

dsa_status dsa_layer_step(const dsa_layer_args* a, void* ws, size_t ws_bytes, hipStream_t stream) {
    DSA_REQUIRE(a, DSA_ERR_NULL, "layer step: NULL args");
    DSA_REQUIRE(a->compress_rate >= 0, DSA_ERR_SHAPE, "layer step: compress_rate=%d", a->compress_rate);
    const int m = a->compress_rate > 1 ? a->compress_rate : 1;
    DSA_REQUIRE(m == 1 || a->form == DSA_ATTN_LATENT, DSA_ERR_SHAPE,
                "layer step: compressed entries (compress_rate > 1) need the latent form");
    dsa_status st = check_index_args(a->q_fp8, a->q_scale, a->w, a->k_fp8, a->k_scale, a->len, a->B,
                                     a->T, a->H_I, a->d_I, a->Lmax, m);
    if (st != DSA_OK) return st;
    DSA_REQUIRE(a->topk >= 1, DSA_ERR_SHAPE, "layer step: topk=%d", a->topk);
    DSA_REQUIRE(a->form == DSA_ATTN_LATENT || a->form == DSA_ATTN_MHA, DSA_ERR_DTYPE,
                "layer step: bad attention form %d", static_cast<int>(a->form));
    if (a->form == DSA_ATTN_LATENT) {
        st = check_latent_args(a->q, a->latent, a->len, a->len, a->B, a->T, a->H, a->Dv, a->Dr,
                               a->Lmax, a->topk, a->dtype, a->out, m);
    } else {
        DSA_REQUIRE(a->Lmax == a->T, DSA_ERR_SHAPE,
                    "layer step (MHA form): the chunk starts at 0, so Lmax must equal T");
        st = check_mha_args(a->q, a->k, a->v, a->len, a->B, a->T, a->H, a->Dqk, a->Dv, a->topk,
                            a->sm_scale, a->dtype, a->out);
    }
    if (st != DSA_OK) return st;
    DSA_REQUIRE(a->lse == nullptr || aligned16(a->lse), DSA_ERR_ALIGN, "layer step: lse alignment");
    DSA_REQUIRE(!a->idx_out || aligned16(a->idx_out), DSA_ERR_ALIGN, "layer step: idx_out alignment");
    DSA_REQUIRE(!a->scores_out || aligned16(a->scores_out), DSA_ERR_ALIGN,
                "layer step: scores_out alignment");
    size_t s_bytes, i_bytes, att_bytes;
    layer_ws_parts(a, &s_bytes, &i_bytes, &att_bytes);
    const size_t need = s_bytes + i_bytes + att_bytes;
    DSA_REQUIRE(need == 0 || (ws && ws_bytes >= need), DSA_ERR_WORKSPACE,
                "layer step: workspace of %zu bytes required (got %zu)", need, ws_bytes);
    DSA_REQUIRE(need == 0 || (reinterpret_cast<uintptr_t>(ws) & 255u) == 0, DSA_ERR_ALIGN,
                "layer step: workspace must be 256-byte aligned");
    uint8_t* p = static_cast<uint8_t*>(ws);
    float* scores = a->scores_out ? a->scores_out : reinterpret_cast<float*>(p);
    p += s_bytes;
    int32_t* idx = a->idx_out ? a->idx_out : reinterpret_cast<int32_t*>(p);
    p += i_bytes;
    void* att_ws = att_bytes ? p : nullptr;

    dsa::IndexScoresArgs ia{a->q_fp8, a->q_scale, a->w, a->k_fp8, a->k_scale, a->len, a->B, a->T,
                            a->H_I, a->d_I, a->Lmax, a->sm_scale_I, scores, a->scores_out ? 1 : 0, m};
    st = hip_status(dsa::launch_index_scores(ia, stream), "layer step: index scores");
    if (st != DSA_OK) return st;
    dsa::TopkArgs ta{scores, a->len, a->B, a->T, a->Lmax, a->topk, idx, m};
    st = hip_status(dsa::launch_topk(ta, att_ws, stream), "layer step: topk");
    if (st != DSA_OK) return st;
    if (a->form == DSA_ATTN_LATENT)
        st = launch_latent(a->q, a->latent, idx, a->len, a->B, a->T, a->H, a->Dv, a->Dr, a->Lmax,
                           a->topk, a->sm_scale, a->dtype, a->out, a->lse, att_ws, stream, m);
    else
        st = launch_mha(a->q, a->k, a->v, idx, a->B, a->T, a->H, a->Dqk, a->Dv, a->topk,
                        a->sm_scale, a->dtype, a->out, a->lse, att_ws, stream);
    return st;
}

dsa_status dsa_layer_step_noalloc(const dsa_layer_args* a, hipStream_t stream) {
    DSA_REQUIRE(a, DSA_ERR_NULL, "layer step (no alloc): NULL args");
    const size_t need = dsa_layer_step_workspace_bytes(a);
    DSA_REQUIRE(need <= kStaticScratchBytes, DSA_ERR_WORKSPACE,
                "layer step (no alloc): this shape needs %zu bytes of scratch, above the library's "
                "fixed %zu (use dsa_layer_step with a workspace)", need, kStaticScratchBytes);
    void* ws = nullptr;
    dsa_status st = device_scratch(&ws);
    if (st != DSA_OK) return st;
    return dsa_layer_step(a, ws, kStaticScratchBytes, stream);
}

dsa_status dsa_diag_fp8_mfma_dots(const uint8_t* a, const uint8_t* b, int n, float* out_fp8,
                                  float* out_bf16, hipStream_t stream) {
    DSA_REQUIRE(a && b && out_fp8 && out_bf16, DSA_ERR_NULL, "diag fp8 dots: NULL pointer");
    DSA_REQUIRE(n >= 16 && n % 16 == 0 && n <= (1 << 24), DSA_ERR_SHAPE,
                "diag fp8 dots: n=%d must be a positive multiple of 16 up to 2^24", n);
    DSA_REQUIRE(aligned16(a) && aligned16(b) && aligned16(out_fp8) && aligned16(out_bf16), DSA_ERR_ALIGN,
                "diag fp8 dots: pointers must be 16-byte aligned");
    const hipError_t e = dsa::launch_diag_fp8_dots(a, b, n, out_fp8, out_bf16, stream);
    DSA_REQUIRE(e == hipSuccess, DSA_ERR_HIP, "diag fp8 dots: %s", hipGetErrorString(e));
    return DSA_OK;
}

}  // extern "C"
