/*
 * dsa.h -- C ABI of the MI355X (gfx950) DeepSeek Sparse Attention layer-step library
 * (libdsa_amd.so).
 *
 * One DSA layer step, as the pages describe it:
 *   1. lightning-indexer scores      ("DeepSeek-V3.2-Exp - Split indexer heads": the
 *                                      Indexer.forward excerpt folds the query scales into
 *                                      the head weights and scores FP8 queries against the
 *                                      FP8 key cache; "dsa-indexer.excalidraw", score box:
 *                                      per-head ReLU of q.k, weighted sum over heads);
 *   2. causal mask                    ("DeepSeek-V3.2-Exp - Causal mask": -inf strictly
 *                                      above the diagonal);
 *   3. per-row top-k                  (Indexer.forward excerpt: the index_topk best
 *                                      positions, never more than are visible; the
 *                                      excalidraw top-k selector keeps 2048);
 *   4. sparse attention over the k selected positions, either in the absorbed latent
 *      (MQA) form of the excalidraw diagram, where all query heads share the selected
 *      latent rows and each row serves as key and value, or in the MHA prefill form of
 *      the MLA prefill excerpt ("Causal mask" page, Multi-head latent attention).
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers to dense row-major arrays, 16-byte aligned.
 *   - len[b] is the number of valid cache positions of sequence b.  The T query rows of
 *     a call are the LAST T positions: pos(b,t) = len[b] - T + t.  Cache position s is
 *     visible to row (b,t) iff 0 <= s <= pos(b,t).  Preconditions checked on the device
 *     side only by construction (the host cannot read device memory without a sync):
 *     T <= len[b] <= Lmax.
 *   - Every call only enqueues work on `stream` and returns; outputs are valid once the
 *     caller synchronises the stream.  The library never allocates, frees or
 *     synchronises; scratch memory comes from the caller as (ws, ws_bytes), sized by
 *     the matching *_workspace_bytes() query (dsa_layer_step_noalloc instead uses a
 *     fixed scratch array that the library's device code holds on each GPU).  Inputs must stay alive until the stream
 *     reaches the call; outputs must not alias inputs or the workspace.
 *   - Errors are reported by the returned status; nothing aborts.  dsa_last_error()
 *     returns a thread-local description of the last non-OK status.  Arguments are
 *     validated before anything is enqueued; DSA_ERR_HIP means a launch failed.
 *   - FP8 is OCP e4m3fn (max 448), one fp32 scale per row of d_I values (128-wide
 *     blocks at the V3.2 sizes).  bf16 is IEEE binary32 truncated to 16 bits.
 */
#ifndef DSA_H
#define DSA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    DSA_OK = 0,
    DSA_ERR_NULL = 1,       /* a required pointer is NULL                          */
    DSA_ERR_SHAPE = 2,      /* a size is out of the supported range                */
    DSA_ERR_DTYPE = 3,      /* dtype / form / shape combination not supported      */
    DSA_ERR_ALIGN = 4,      /* a pointer is not 16-byte aligned                    */
    DSA_ERR_WORKSPACE = 5,  /* ws is NULL or ws_bytes is below the queried size    */
    DSA_ERR_HIP = 6         /* a HIP launch or runtime call failed                 */
} dsa_status;

/* Attention element type.  DSA_FP8_LATENT (latent form only: dsa_sparse_mla_decode and
 * dsa_layer_step with DSA_ATTN_LATENT): q and out are bf16, and each latent cache row is
 * the 656-byte FP8 storage form of the excalidraw diagram's latent cache box and its
 * per-token byte figure -- 512 e4m3fn codes, then four fp32 scales (scale j multiplies
 * columns 128j .. 128j+127), then the 64 rope values as bf16 -- so latent is
 * [B,Lmax,656] bytes and the shape is fixed at Dv = 512, Dr = 64.  Column d < 512 of a
 * row is code[d] * scale[d / 128]; column 512 + r is rope value r. */
typedef enum { DSA_F32 = 0, DSA_BF16 = 1, DSA_FP8_LATENT = 2 } dsa_dtype;
typedef enum { DSA_ATTN_LATENT = 0, DSA_ATTN_MHA = 1 } dsa_attn_form;

/* Thread-local text for the last non-OK status of this thread ("" if none). */
const char* dsa_last_error(void);
/* Library version, major * 10000 + minor * 100 + patch. */
int dsa_version(void);

/*
 * dsa_indexer_prep -- the indexer's preparation of T new tokens per sequence, between the
 * projections and the scores ("Split indexer heads": Indexer.forward applies rope to the
 * leading rope columns without interleaving, then rotate_activation, then act_quant to
 * FP8 with one scale per block, and writes the keys into the key cache; the bodies of
 * those steps are not on the pages, so they are read as follows):
 *   rope      column j < rope_dim/2 of a row pairs with column j + rope_dim/2 and the pair
 *             (a, b) becomes (a c - b s, a s + b c), c/s = rope_cos/rope_sin[pos][j];
 *   rotation  the orthonormal Walsh-Hadamard transform of the d_I-wide row (Sylvester
 *             order: out_i = d_I^-1/2 sum_j (-1)^popcount(i & j) in_j);
 *   act_quant scale = max(amax, 1e-12) / 448 per row (fp32), code = e4m3fn nearest to
 *             clamp(x / scale, +-448), ties to even, sign from x.
 * All arithmetic is fp32; a value within fp32 rounding of a midpoint between two e4m3fn
 * values may take either neighbour.
 *   q        [B,T,H_I,d_I] (dtype F32 or BF16) projected indexer queries, rope columns first
 *   k        [B,T,d_I] normalised indexer keys of the new tokens, rope columns first
 *   rope_cos, rope_sin [P, rope_dim/2] f32 (may be NULL when rope_dim = 0)
 *   start    [B] i32: token t of sequence b sits at position start[b] + t
 *   q_fp8    [B,T,H_I,d_I] u8, q_scale [B,T,H_I] f32 (outputs: the inputs of dsa_index_scores)
 *   k_cache  [B,Lmax,d_I] u8, k_scale [B,Lmax] f32: rows start[b] .. start[b]+T-1 are
 *            written, every other row is left as it is.
 * Supported: 1 <= H_I <= 64, d_I in {32, 64, 128}, rope_dim 0 or a power of two in
 * [4, d_I].
 * A token whose position is outside [0, min(P, Lmax)) is skipped (device-side check).
 */
dsa_status dsa_indexer_prep(const void* q, const void* k, dsa_dtype dt, const float* rope_cos,
                            const float* rope_sin, int P, const int32_t* start, int B, int T,
                            int H_I, int d_I, int rope_dim, int Lmax, uint8_t* q_fp8,
                            float* q_scale, uint8_t* k_cache, float* k_scale, hipStream_t stream);

/*
 * dsa_index_scores -- lightning-indexer scores with the causal mask applied.
 *   scores[b,t,s] = k_scale[b,s] * sum_h (w[b,t,h] * q_scale[b,t,h] * sm_scale_I)
 *                                     * max(0, sum_d q[b,t,h,d] * k[b,s,d])
 *   for visible s, and -inf for every other s < Lmax.
 * ("Split indexer heads": the caller's `w` is the projected head weight, already scaled
 *  by the inverse square root of the head count; the library folds q_scale and the
 *  indexer softmax scale into it as the excerpt does; the ReLU is the one in the
 *  excalidraw score box.)
 *   q_fp8   [B,T,H_I,d_I] u8 e4m3fn     q_scale [B,T,H_I] f32     w [B,T,H_I] f32
 *   k_fp8   [B,Lmax,d_I]  u8 e4m3fn     k_scale [B,Lmax] f32      len [B] i32
 *   scores  [B,T,Lmax] f32 (output)
 * Supported: 1 <= H_I <= 64, d_I in {32, 64, 128}, 1 <= T <= Lmax.
 */
dsa_status dsa_index_scores(const uint8_t* q_fp8, const float* q_scale, const float* w,
                            const uint8_t* k_fp8, const float* k_scale, const int32_t* len,
                            int B, int T, int H_I, int d_I, int Lmax, float sm_scale_I,
                            float* scores, hipStream_t stream);

/*
 * dsa_topk -- per query row, the positions of the min(k, pos+1) largest visible scores.
 * (Indexer.forward excerpt: the index_topk best positions, capped at the number visible;
 *  unused slots hold -1, the warm-up sentinel of the DeepSeek-V4 mask visualiser.)
 *   scores [B,T,Lmax] f32 (only positions 0..pos(b,t) are read)   len [B] i32
 *   idx    [B,T,k] i32 (output): the selected positions in ascending order, then -1.
 * Equal scores at the threshold are resolved in favour of the smaller position, so the
 * result is deterministic.  Scores must not be NaN.  Supported: 1 <= k, T <= Lmax.
 * Rows longer than 16384 positions (Lmax > 16384 and k < 8192) use a workspace of
 * dsa_topk_workspace_bytes() for per-chunk candidates; otherwise it is 0 bytes.
 */
size_t dsa_topk_workspace_bytes(int B, int T, int Lmax, int k);
dsa_status dsa_topk(const float* scores, const int32_t* len, int B, int T, int Lmax, int k,
                    int32_t* idx, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * dsa_sparse_mla_decode -- absorbed (MQA) sparse attention over selected latent rows.
 * (excalidraw core-attention box: the 128 query heads share the 2048 selected latent
 *  rows, each of which serves as key and value; softmax and value mix as in the MLA
 *  prefill excerpt.)
 *   q      [B,T,H,Dv+Dr]   (absorbed query: Dv latent columns, then Dr rope columns)
 *   latent [B,Lmax,Dv+Dr]  (cache row: latent Dv, then rope Dr; with DSA_FP8_LATENT
 *                          [B,Lmax,656] bytes in the FP8 storage form, decoded as above)
 *   idx    [B,T,k] i32     (slots < 0 and positions > pos(b,t) are ignored)
 *   out    [B,T,H,Dv]      (same dtype as q), lse [B,T,H] f32 natural-log sum-exp of the
 *                          scaled logits, or NULL.
 *   logit_j = sm_scale * q[b,t,h,:] . latent[b,s_j,:]; out = softmax(logit) @ latent[.,:Dv]
 * A row with no usable slot gets out = 0 and lse = -inf.  Entries of idx must be unique
 * per row.  Any H, Dv, Dr with Dv+Dr <= 1024 and dtype F32 or BF16, and any H with
 * DSA_FP8_LATENT (the vector-ALU path keeps all k logits in LDS: 4 (Dv + Dr + k) <= 65536
 * bytes); the BF16 and FP8_LATENT shape H in {64, 128}, Dv = 512, Dr = 64, k <= 16384
 * runs on the matrix-core path, which splits each row's slots over up to 16 workgroups
 * (and the 128 heads of few rows over two) and needs a workspace for their partial
 * results (dsa_sparse_mla_decode_workspace_bytes(); 0 when the rows fill the GPU without
 * splitting the slots).  A DSA_FP8_LATENT dtype with other
 * widths is DSA_ERR_DTYPE.
 */
size_t dsa_sparse_mla_decode_workspace_bytes(int B, int T, int H, int Dv, int Dr, int k,
                                             dsa_dtype dt);
dsa_status dsa_sparse_mla_decode(const void* q, const void* latent, const int32_t* idx,
                                 const int32_t* len, int B, int T, int H, int Dv, int Dr,
                                 int Lmax, int k, float sm_scale, dsa_dtype dt, void* out,
                                 float* lse, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * dsa_sparse_mla_prefill -- MHA-form sparse attention over a chunk that starts at
 * position 0 (keys and values are the chunk's own T positions, per head).
 * (MLA prefill excerpt: query and key rows are the no-rope part followed by the rope
 *  part; the scaled scores get an index mask, 0 at the selected positions and -inf
 *  elsewhere, plus the causal mask, then a softmax mixes the value rows.)
 *   q, k [B,T,H,Dqk]   v [B,T,H,Dv]   idx [B,T,topk] i32 (slots < 0 or > t are ignored)
 *   out  [B,T,H,Dv] (same dtype), lse [B,T,H] f32 or NULL.
 * Supported: dtype F32 or BF16, Dqk <= 1024, Dv <= 1024 (the vector-ALU path keeps all
 * topk logits in LDS: 4 (Dqk + topk) <= 65536 bytes); the bf16 shape Dqk = 192, Dv = 128
 * with a finite sm_scale > 0 runs on the matrix-core path, which needs a workspace for the
 * per-row selection bit mask (B * T * ceil(T / 32) words;
 * dsa_sparse_mla_prefill_workspace_bytes(), sized for that path); any other scale takes
 * the vector-ALU path and its LDS bound on topk.
 */
size_t dsa_sparse_mla_prefill_workspace_bytes(int B, int T, int H, int Dqk, int Dv, int topk,
                                              dsa_dtype dt);
dsa_status dsa_sparse_mla_prefill(const void* q, const void* k, const void* v,
                                  const int32_t* idx, int B, int T, int H, int Dqk, int Dv,
                                  int topk, float sm_scale, dsa_dtype dt, void* out, float* lse,
                                  void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * dsa_layer_step -- the whole step: index scores -> causal mask -> top-k -> sparse
 * attention, in the latent form (len[] per sequence, T rows at the end) or the MHA
 * prefill form (len[b] = T for every b, Lmax = T).  The workspace
 * (dsa_layer_step_workspace_bytes(), 256-byte aligned) holds the scores and indices
 * that are not requested as outputs, then one scratch region shared by the top-k
 * candidates and the attention partials.  Errors as for the individual calls; nothing
 * is enqueued when validation fails.
 */
typedef struct dsa_layer_args {
    /* indexer */
    const uint8_t* q_fp8;     /* [B,T,H_I,d_I] e4m3fn                                */
    const float* q_scale;     /* [B,T,H_I]                                           */
    const float* w;           /* [B,T,H_I]                                           */
    const uint8_t* k_fp8;     /* [B,Lmax,d_I] e4m3fn                                 */
    const float* k_scale;     /* [B,Lmax]                                            */
    const int32_t* len;       /* [B]                                                 */
    int B, T, H_I, d_I, Lmax, topk;
    float sm_scale_I;
    /* attention */
    dsa_attn_form form;
    dsa_dtype dtype;          /* DSA_FP8_LATENT: latent form only                    */
    const void* q;            /* latent: [B,T,H,Dv+Dr]    MHA: [B,T,H,Dqk]           */
    const void* latent;       /* latent: [B,Lmax,Dv+Dr]   MHA: unused                */
    const void* k;            /* MHA: [B,T,H,Dqk]         latent: unused             */
    const void* v;            /* MHA: [B,T,H,Dv]          latent: unused             */
    int H, Dv, Dr, Dqk;
    float sm_scale;
    void* out;                /* [B,T,H,Dv]                                          */
    float* lse;               /* [B,T,H] or NULL                                     */
    /* optional intermediate outputs (NULL: kept in the workspace) */
    int32_t* idx_out;         /* [B,T,topk]                                          */
    float* scores_out;        /* [B,T,Lmax]; when NULL, scores of invisible positions
                                 are not materialised                               */
    /* Compressed entries (the DeepSeek-V4 mask visualiser's compressed-sparse layers):
     * 0 or 1 = every position is a cache row (the V3.2 step).  m > 1 = the key cache and
     * the latent cache hold compressed entries, each standing for m consecutive
     * positions; len[b] stays the sequence's position count, Lmax is the entry capacity,
     * and row (b,t) at position p = len[b] - T + t may select entry e iff e < (p + 1) / m
     * -- rows with no entry get all -1 slots, a zero output and lse = -inf.  Requires
     * the latent form and len[b] / m <= Lmax (T may then exceed Lmax).                */
    int compress_rate;
} dsa_layer_args;

size_t dsa_layer_step_workspace_bytes(const dsa_layer_args* a);
dsa_status dsa_layer_step(const dsa_layer_args* a, void* ws, size_t ws_bytes,
                          hipStream_t stream);

/*
 * dsa_layer_step_noalloc -- dsa_layer_step for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same step and results, with the workspace taken from a scratch array the library
 * holds in each GPU's memory (DSA_NOALLOC_SCRATCH_BYTES = 64 MiB per device, placed when
 * the library's device code is loaded and kept until the process ends) instead of a
 * caller buffer.  The caller still passes every input and output in `a`.
 *   - A shape whose dsa_layer_step_workspace_bytes() exceeds DSA_NOALLOC_SCRATCH_BYTES is
 *     rejected with DSA_ERR_WORKSPACE before anything is enqueued (the decode shapes up
 *     to B=64 x 65536 positions fit; a T=8192 prefill chunk's score matrix does not).
 *   - The call allocates and frees nothing (no hipMalloc, no torch allocation).  On its
 *     first use on a device it looks up that device's copy of the array once.
 *   - Every call on one GPU shares that GPU's array, which keeps the last call's
 *     contents: calls that overlap on one GPU (concurrent streams, or host threads
 *     enqueueing on different streams) race on it and must be serialised by the
 *     caller.  Nothing in the array needs to start at zero: each step writes every
 *     scratch value before reading it.
 * Other errors as for dsa_layer_step.
 */
#define DSA_NOALLOC_SCRATCH_BYTES (64u << 20)
dsa_status dsa_layer_step_noalloc(const dsa_layer_args* a, hipStream_t stream);

/*
 * Tracing aid: HIP-event timing of the kernels of dsa_layer_step.
 *   dsa_profile_begin(max_steps) creates (max_steps * 12) HIP events (host-side objects,
 *   no device memory) and makes every following layer-step call launch each of its
 *   kernels with a start/stop event pair that the dispatch itself records
 *   (hipExtLaunchKernel), so each pair spans one kernel's execution alone.  Phases:
 *   0 index scores, 1 top-k (one or two kernels; for the MHA form also the kernel
 *   that turns the selection into the attention's bit mask), 2 sparse attention (its
 *   main kernel), 3 split combine (only when the attention splits its k slots).  Kernels beyond the pool are not timed.
 *   dsa_profile_end(ms_total[4], counts[4]) waits for the last recorded event, returns
 *   the summed elapsed milliseconds and the number of timed kernels of each phase, and
 *   destroys the events.  Process-wide state: not for concurrent use from several
 *   threads or streams.
 */
dsa_status dsa_profile_begin(int max_steps);
dsa_status dsa_profile_end(double* ms_total, int* counts);

/*
 * Diagnostic: the precision of the two matrix-core forms of the indexer contraction.
 *   Row p of a and row p of b (n rows each, 128 FP8 e4m3fn codes per row, device
 *   memory, 16-byte aligned) give one dot product per row pair; out_fp8[p] is it as the
 *   gfx950 FP8 matrix-core instruction (v_mfma_f32_16x16x128_f8f6f4) computes it,
 *   out_bf16[p] as the bf16 form over the codes widened exactly (the form the index
 *   kernels use).  The pairs are those of the score box of "dsa-indexer.excalidraw"
 *   (q_j . k_s per head, before the ReLU and the scales).  n must be a positive
 *   multiple of 16 up to 2^24.  Enqueues one kernel; outputs valid after a sync.
 */
dsa_status dsa_diag_fp8_mfma_dots(const uint8_t* a, const uint8_t* b, int n, float* out_fp8,
                                  float* out_bf16, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* DSA_H */
