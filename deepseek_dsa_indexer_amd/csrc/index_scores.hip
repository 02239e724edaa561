// index_scores.hip -- lightning-indexer scores on gfx950 matrix cores.
//
// Computes, for every query row (b,t) and cache position s < Lmax,
//   I[b,t,s] = k_scale[b,s] * sum_h w'[b,t,h] * max(0, q[b,t,h,:] . k[b,s,:]),
//   w' = w * q_scale * sm_scale,
// with -inf where s > pos(b,t) = len[b] - T + t.  The weight fold follows the
// Indexer.forward excerpt ("DeepSeek-V3.2-Exp - Split indexer heads"); the per-head
// ReLU and weighted head sum follow the score box of "dsa-indexer.excalidraw"; the
// mask is the -inf-above-the-diagonal mask of the "Causal mask" page.
//
// Storage and arithmetic.  q and the key cache stay FP8 (e4m3fn) in memory, so the
// stream is 128 + 4 bytes per key.  In registers every FP8 byte is widened to bf16
// (exact: e4m3fn values are a subset of bf16) and the 128-wide products run on the
// bf16 MFMA, whose products and fp32 sums are exact to fp32 rounding.  The FP8 MFMA
// was measured on gfx950 to align its in-instruction products to about 13 significant
// bits (error up to 1.6e-4 of sum |q_d k_d|), which shows up as 1e-3-level relative
// errors on scores whose head terms cancel.
//
// Mapping.  One wave owns QR query rows and streams 64-key chunks of the key cache.
// The 64 heads of each query row stay in registers as A operands (4 head tiles x 4
// K-steps of 32).  A chunk is four 16-key B tiles read with 16-byte loads: lane l takes
// the bytes [16 g, 16 g + 16) and [64 + 16 g, 64 + 16 g + 16) of key (l % 16), g = l / 16,
// so each load instruction reads whole 64-byte halves of 16 key rows; K-steps 0 and 1
// use the first piece, 2 and 3 the second (q uses the same byte -> K-slot assignment, so
// the four K-steps cover each of the 128 dims once).  Each MFMA leaves lane l with 4
// heads x 1 key; ReLU and the head weights are applied in registers and three
// cross-lane exchanges finish the head sum, so lane l ends with the score of key
// (chunk + l): one coalesced 256-byte store per row and chunk.  Heads beyond H_I and
// columns beyond d_I are zero (weight 0), which covers the small test shapes.
//
// Blocks.  A block covers QR query rows and 256 * chunks consecutive keys.  With one
// query row per sequence (decode), only the key blocks that hold visible positions are
// launched work, numbered sequence after sequence (numbered_block), so a batch of
// unequal lengths loads the 8 XCDs evenly; a grid laid out as (sequence, key block)
// would give XCD j the sequences j, j + 8, ... and the longest of them would set the
// kernel's time.
#include <algorithm>

#include "dsa_device.h"
#include "dsa_internal.h"

namespace dsa {

namespace {

constexpr int kThreads = 256;       // 4 waves
constexpr int kChunk = 64;          // keys per wave iteration (4 MFMA column tiles)
constexpr int kMaxHeads = 64;       // indexer heads (4 MFMA row tiles)
constexpr int kMaxSeqPerThread = 16; // numbered decode launches: up to 4096 sequences

typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

// Two 16-byte pieces at p0 and p1, each zeroed when its flag is false.  The loads are
// issued unconditionally (callers pass clamped, in-bounds addresses): a load inside a
// divergent branch makes the compiler drain every outstanding load at the branch join.
__device__ __forceinline__ v8i load2x16(const uint8_t* p0, bool ok0, const uint8_t* p1, bool ok1) {
    const uint4 a = *reinterpret_cast<const uint4*>(p0);
    const uint4 b = *reinterpret_cast<const uint4*>(p1);
    const int m0 = ok0 ? -1 : 0;
    const int m1 = ok1 ? -1 : 0;
    return v8i{static_cast<int>(a.x) & m0, static_cast<int>(a.y) & m0, static_cast<int>(a.z) & m0,
               static_cast<int>(a.w) & m0, static_cast<int>(b.x) & m1, static_cast<int>(b.y) & m1,
               static_cast<int>(b.z) & m1, static_cast<int>(b.w) & m1};
}

// 8 FP8 bytes (two dwords) -> 8 bf16, exactly.
__device__ __forceinline__ v8bf fp8x8_to_bf16(int d0, int d1) {
    const v2bf a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, 1.0f, false);
    const v2bf b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, 1.0f, true);
    const v2bf c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, 1.0f, false);
    const v2bf d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, 1.0f, true);
    return v8bf{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// Lane (g, n) holds s[c] = partial score (heads of group g) of key 16c + n.  Returns,
// in every lane, the full head sum for key 16g + n, i.e. for chunk offset == lane.
__device__ __forceinline__ float head_sum_transpose(const float s[4], int g) {
    const bool lo = g < 2;
    float send0 = lo ? s[2] : s[0];
    float send1 = lo ? s[3] : s[1];
    const int lane = g << 4;                    // bits 4 and 5 of the lane index
    float r0 = from_xor32(send0, lane);
    float r1 = from_xor32(send1, lane);
    float a0 = (lo ? s[0] : s[2]) + r0;     // tile 0 (g < 2) or tile 2
    float a1 = (lo ? s[1] : s[3]) + r1;     // tile 1 (g < 2) or tile 3
    const bool odd = g & 1;
    float send = odd ? a0 : a1;
    float r = from_xor16(send, lane);
    return (odd ? a1 : a0) + r;
}

template <int D, int QR>
__global__ __launch_bounds__(kThreads)
void index_scores_kernel(const uint8_t* __restrict__ q, const float* __restrict__ q_scale,
                         const float* __restrict__ w, const uint8_t* __restrict__ k,
                         const float* __restrict__ k_scale, const int32_t* __restrict__ len,
                         int T, int H, int Lmax, float sm_scale, float* __restrict__ scores,
                         int fill_invisible, int chunks)
{
    __shared__ __attribute__((aligned(16))) uint8_t s_q[QR][kMaxHeads * 128];
    __shared__ __attribute__((aligned(16))) float s_wf[QR][kMaxHeads];
    const int keys_per_block = kThreads / kWave * kChunk * chunks;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int g = lane >> 4;
    const int n = lane & 15;

    const int row_groups = (T + QR - 1) / QR;
    int b, t0, yblk;
    if (T == 1 && gridDim.x <= kThreads * kMaxSeqPerThread) {
        // one query row per sequence: numbered blocks (sequences of unequal length
        // still spread evenly over the XCDs; no block past a sequence's end is run
        // unless its positions are to be filled with -inf)
        __shared__ int s_num[kThreads / kWave + 2];
        const int nblk = gridDim.y;
        auto count = [&](int s) {
            return fill_invisible ? nblk : (min(len[s], Lmax) + keys_per_block - 1) / keys_per_block;
        };
        if (!numbered_block<kThreads>(blockIdx.y * gridDim.x + blockIdx.x, gridDim.x, count, s_num, b, yblk))
            return;
        t0 = 0;
    } else {
        b = blockIdx.x / row_groups;
        t0 = (blockIdx.x - b * row_groups) * QR;
        yblk = blockIdx.y;
    }
    const int nrows = min(QR, T - t0);
    const int pos0 = min(len[b], Lmax) - T + t0;   // position of row t0
    const int pos_hi = pos0 + nrows - 1;

    const int key_blk = yblk * keys_per_block;
    float* out = scores + (static_cast<size_t>(b) * T + t0) * Lmax;

    if (key_blk > pos_hi) {                     // the whole block is masked
        if (fill_invisible) {
            for (int key = key_blk + threadIdx.x; key < min(key_blk + keys_per_block, Lmax); key += kThreads)
                for (int r = 0; r < nrows; ++r) out[static_cast<size_t>(r) * Lmax + key] = -INFINITY;
        }
        return;
    }

    const uint8_t* kb_ptr = k + static_cast<size_t>(b) * Lmax * D;
    const float* ks_ptr = k_scale + static_cast<size_t>(b) * Lmax;
    // chunk c of this wave starts at key_blk + (4 c + wave) * 64
    auto chunk_key = [&](int c) { return key_blk + (c * (kThreads / kWave) + wave) * kChunk; };
    auto load_chunk = [&](int c, v8i (&dst)[4], float& ks) {
        const int kb = chunk_key(c);
        const bool live = c < chunks && kb <= pos_hi;
#pragma unroll
        for (int tile = 0; tile < 4; ++tile) {
            const int key = kb + 16 * tile + n;
            const bool ok = live && key < Lmax;
            const int kc = min(key, Lmax - 1);
            const uint8_t* krow = kb_ptr + static_cast<size_t>(kc) * D;
            const int b0 = 16 * g, b1 = 64 + 16 * g;     // pieces past d_I read 0 (masked)
            dst[tile] = load2x16(krow + (b0 < D ? b0 : 0), ok && b0 < D,
                                 krow + (b1 < D ? b1 : 0), ok && b1 < D);
        }
        // positions at or beyond Lmax are never stored, so the clamped scale needs no mask
        ks = ks_ptr[min(kb + lane, Lmax - 1)];
    };

    // ---- the block's query rows and folded head weights go through LDS once: q as
    // [64 heads][128 bytes] (zero past H heads and D bytes), w * q_scale * sm_scale
    // (zero past H heads and for padded rows).  Their loads are issued before the first
    // two key chunks of every wave, so waiting for them leaves the chunks in flight, and
    // each chunk is waited for only when it is used.
    constexpr int kQLoads = QR * kMaxHeads * 8 / kThreads;     // 16-byte pieces per thread
    uint4 qv[kQLoads];
    bool qok[kQLoads];
#pragma unroll
    for (int u = 0; u < kQLoads; ++u) {
        const int i = threadIdx.x + u * kThreads;
        const int r = i / (kMaxHeads * 8);
        const int h = (i / 8) % kMaxHeads;
        const int c16 = i % 8;
        qok[u] = r < nrows && h < H && c16 * 16 < D;
        const size_t qrow = static_cast<size_t>(b) * T + t0 + min(r, nrows - 1);
        qv[u] = *reinterpret_cast<const uint4*>(
            q + (qrow * H + min(h, H - 1)) * D + (c16 * 16 < D ? c16 * 16 : 0));
    }
    float wv = 0.f, qsv = 0.f;
    const int wr = threadIdx.x / kMaxHeads;           // row of this thread's head weight
    const int wh = threadIdx.x % kMaxHeads;
    if (wr < QR) {
        const size_t qrow = static_cast<size_t>(b) * T + t0 + min(wr, nrows - 1);
        const int hc = min(wh, H - 1);
        wv = w[qrow * H + hc];
        qsv = q_scale[qrow * H + hc];
    }
    v8i cur[4], nxt[4];
    float ks_cur, ks_nxt;
    load_chunk(0, cur, ks_cur);
    load_chunk(1, nxt, ks_nxt);
#pragma unroll
    for (int u = 0; u < kQLoads; ++u) {
        const int i = threadIdx.x + u * kThreads;
        const int r = i / (kMaxHeads * 8);
        const int h = (i / 8) % kMaxHeads;
        const int c16 = i % 8;
        *reinterpret_cast<uint4*>(&s_q[r][h * 128 + c16 * 16]) = qok[u] ? qv[u] : uint4{0u, 0u, 0u, 0u};
    }
    if (wr < QR) s_wf[wr][wh] = (wr < nrows && wh < H) ? wv * qsv * sm_scale : 0.f;
    __syncthreads();
    v8bf qa[QR][4][4];
    float wf[QR][4][4];
#pragma unroll
    for (int r = 0; r < QR; ++r)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint4 lo = *reinterpret_cast<const uint4*>(&s_q[r][(16 * j + n) * 128 + 16 * g]);
            const uint4 hi = *reinterpret_cast<const uint4*>(&s_q[r][(16 * j + n) * 128 + 64 + 16 * g]);
            const int raw[8] = {static_cast<int>(lo.x), static_cast<int>(lo.y), static_cast<int>(lo.z),
                                static_cast<int>(lo.w), static_cast<int>(hi.x), static_cast<int>(hi.y),
                                static_cast<int>(hi.z), static_cast<int>(hi.w)};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) qa[r][j][kk] = fp8x8_to_bf16(raw[2 * kk], raw[2 * kk + 1]);
            const float4 wv = *reinterpret_cast<const float4*>(&s_wf[r][16 * j + 4 * g]);
            wf[r][j][0] = wv.x; wf[r][j][1] = wv.y; wf[r][j][2] = wv.z; wf[r][j][3] = wv.w;
        }

    for (int c = 0; c < chunks; ++c) {
        const int kb = chunk_key(c);
        const int key = kb + lane;
        if (kb > pos_hi) {
            if (fill_invisible && key < Lmax)
                for (int r = 0; r < nrows; ++r) out[static_cast<size_t>(r) * Lmax + key] = -INFINITY;
        } else {
            float s[QR][4];
#pragma unroll
            for (int tile = 0; tile < 4; ++tile) {
                v8bf kbf[4];
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) kbf[kk] = fp8x8_to_bf16(cur[tile][2 * kk], cur[tile][2 * kk + 1]);
#pragma unroll
                for (int r = 0; r < QR; ++r) {
                    // the four head tiles are independent accumulation chains: interleave them
                    v4f d[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) d[j] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
                        for (int j = 0; j < 4; ++j) d[j] = mfma_bf16_16x16x32(qa[r][j][kk], kbf[kk], d[j]);
                    float acc = 0.f;
#pragma unroll
                    for (int j = 0; j < 4; ++j)
#pragma unroll
                        for (int i = 0; i < 4; ++i) acc += wf[r][j][i] * fmaxf(d[j][i], 0.f);
                    s[r][tile] = acc;
                }
            }
#pragma unroll
            for (int r = 0; r < QR; ++r) {
                const float total = head_sum_transpose(s[r], g);
                if (r < nrows && key < Lmax)
                    out[static_cast<size_t>(r) * Lmax + key] = (key <= pos0 + r) ? total * ks_cur : -INFINITY;
            }
        }
#pragma unroll
        for (int tile = 0; tile < 4; ++tile) cur[tile] = nxt[tile];
        ks_cur = ks_nxt;
        if (c + 2 < chunks) load_chunk(c + 2, nxt, ks_nxt);
    }
}

// ---------------------------------------------------------------- decode form
//
// One query row per block (T = 1).  Each wave streams its chunks global -> LDS with direct
// loads (global_load_lds) into a ring of two 8.25 KB slots of its own, so two chunks per
// wave stay in flight without holding registers (the register-staged form above keeps
// one chunk per wave, 64 KB per CU, in flight).  The query row and the head weights
// arrive the same way.  Slot layout, in load order: 1 KB piece 2 t + p holds, at lane l,
// bytes [64 p + 16 (l / 16), + 16) of key 16 t + l % 16 of the chunk -- exactly what lane l
// reads as its MFMA operand piece, so each operand read is one contiguous 16-byte lane
// read -- and the 256 bytes after the keys hold their 64 scales.  The loads are inline
// assembly, invisible to the compiler's wait counting: every wait is an explicit vmcnt
// over this wave's own loads (they complete in issue order), and no other wave touches a
// wave's slots, so the ring needs no barrier.
constexpr int kRing = 2;
constexpr int kSlotBytes = kChunk * 128 + kChunk * 4;     // 8448
constexpr int kChunkLoads = 9;                            // 8 x 1 KB of keys + 256 B of scales
constexpr int kWaves = kThreads / kWave;

template <int N>
__device__ __forceinline__ void vm_wait() { asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory"); }

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
        (__attribute__((address_space(3))) const uint8_t*)(p)));
}
// Lane l's 16 bytes at src go to LDS byte lds + 16 l (M0 carries the wave-uniform base;
// no other instruction of these kernels uses M0).
__device__ __forceinline__ void dma16(uint32_t lds, const void* src) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
                 :: "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(src) : "memory");
}
// Lane l's 4 bytes at src go to LDS byte lds + 4 l.
__device__ __forceinline__ void dma4(uint32_t lds, const void* src) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, off"
                 :: "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(src) : "memory");
}

template <int D>
__global__ __launch_bounds__(kThreads)
void index_scores_decode_kernel(const uint8_t* __restrict__ q, const float* __restrict__ q_scale,
                                const float* __restrict__ w, const uint8_t* __restrict__ k,
                                const float* __restrict__ k_scale, const int32_t* __restrict__ len,
                                int H, int Lmax, float sm_scale, float* __restrict__ scores,
                                int fill_invisible, int chunks)
{
    __shared__ __attribute__((aligned(16))) uint8_t s_q[kMaxHeads * 128];
    __shared__ __attribute__((aligned(16))) float s_w[kMaxHeads];
    __shared__ __attribute__((aligned(16))) float s_qs[kMaxHeads];
    __shared__ __attribute__((aligned(16))) uint8_t s_ring[kWaves][kRing][kSlotBytes];
    __shared__ int s_num[kWaves + 2];
    const int keys_per_block = kWaves * kChunk * chunks;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int g = lane >> 4;
    const int n = lane & 15;

    // numbered blocks: sequences of unequal length still spread evenly over the XCDs, and
    // no block past a sequence's end is run unless its positions are to be filled
    int b, yblk;
    {
        const int nblk = gridDim.y;
        auto count = [&](int sq) {
            return fill_invisible ? nblk : (min(len[sq], Lmax) + keys_per_block - 1) / keys_per_block;
        };
        if (!numbered_block<kThreads>(blockIdx.y * gridDim.x + blockIdx.x, gridDim.x, count, s_num, b, yblk))
            return;
    }
    const int pos = min(len[b], Lmax) - 1;
    const int key_blk = yblk * keys_per_block;
    float* out = scores + static_cast<size_t>(b) * Lmax;
    if (key_blk > pos) {                        // the whole block is masked
        for (int key = key_blk + threadIdx.x; key < min(key_blk + keys_per_block, Lmax); key += kThreads)
            out[key] = -INFINITY;
        return;
    }

    const uint8_t* kb_ptr = k + static_cast<size_t>(b) * Lmax * D;
    const float* ks_ptr = k_scale + static_cast<size_t>(b) * Lmax;
    // chunk c of this wave starts at key_blk + (4 c + wave) * 64; the chunks holding a
    // visible position are c < n_live
    const int first = key_blk + wave * kChunk;
    const int n_live = pos < first ? 0 : min(chunks, (pos - first) / (kWaves * kChunk) + 1);
    auto issue = [&](int c) {
        uint8_t* slot = s_ring[wave][c & 1];
        const int kb = first + c * kWaves * kChunk;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const uint8_t* krow = kb_ptr + static_cast<size_t>(min(kb + 16 * t + n, Lmax - 1)) * D;
#pragma unroll
            for (int p = 0; p < 2; ++p) {
                const int byte = 64 * p + 16 * g;       // pieces past d_I are masked on read
                dma16(lds_addr(slot + (2 * t + p) * 1024), krow + (byte < D ? byte : 0));
            }
        }
        dma4(lds_addr(slot + kChunk * 128), ks_ptr + min(kb + lane, Lmax - 1));
    };

    // ---- the query row (wave w brings bytes [2048 w, 2048 w + 2048) of [64 heads][128]),
    // the head weights (wave 0) and q scales (wave 1), then the first two chunks
    const uint8_t* qrow = q + static_cast<size_t>(b) * H * D;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int o = 2048 * wave + 1024 * i + 16 * lane;
        const int h = min(o >> 7, H - 1), byte = o & 127;   // heads past H, bytes past D: masked on read
        dma16(lds_addr(s_q + 2048 * wave + 1024 * i), qrow + h * D + (byte < D ? byte : 0));
    }
    if (wave == 0) dma4(lds_addr(s_w), w + static_cast<size_t>(b) * H + min(lane, H - 1));
    if (wave == 1) dma4(lds_addr(s_qs), q_scale + static_cast<size_t>(b) * H + min(lane, H - 1));
    if (n_live > 0) issue(0);
    if (n_live > 1) issue(1);
    // this wave's query and weight loads are in when at most its chunk loads remain
    if (n_live > 1) vm_wait<2 * kChunkLoads>();
    else if (n_live > 0) vm_wait<kChunkLoads>();
    else vm_wait<0>();
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

    v8bf qa[4][4];
    float wf[4][4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int h = 16 * j + n;
        const uint4 lo = *reinterpret_cast<const uint4*>(&s_q[h * 128 + 16 * g]);
        const uint4 hi = *reinterpret_cast<const uint4*>(&s_q[h * 128 + 64 + 16 * g]);
        const int m0 = (h < H && 16 * g < D) ? -1 : 0;
        const int m1 = (h < H && 64 + 16 * g < D) ? -1 : 0;
        const int raw[8] = {static_cast<int>(lo.x) & m0, static_cast<int>(lo.y) & m0,
                            static_cast<int>(lo.z) & m0, static_cast<int>(lo.w) & m0,
                            static_cast<int>(hi.x) & m1, static_cast<int>(hi.y) & m1,
                            static_cast<int>(hi.z) & m1, static_cast<int>(hi.w) & m1};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) qa[j][kk] = fp8x8_to_bf16(raw[2 * kk], raw[2 * kk + 1]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int hh = 16 * j + 4 * g + i;
            wf[j][i] = hh < H ? s_w[hh] * s_qs[hh] * sm_scale : 0.f;
        }
    }

    for (int c = 0; c < n_live; ++c) {
        // chunk c is in when at most chunk c + 1's loads remain
        if (c + 1 < n_live) vm_wait<kChunkLoads>();
        else vm_wait<0>();
        const uint8_t* slot = s_ring[wave][c & 1];
        v8i cur[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const uint4 lo = *reinterpret_cast<const uint4*>(slot + (2 * t) * 1024 + 16 * lane);
            const uint4 hi = *reinterpret_cast<const uint4*>(slot + (2 * t + 1) * 1024 + 16 * lane);
            const int m0 = 16 * g < D ? -1 : 0;
            const int m1 = 64 + 16 * g < D ? -1 : 0;
            cur[t] = v8i{static_cast<int>(lo.x) & m0, static_cast<int>(lo.y) & m0,
                         static_cast<int>(lo.z) & m0, static_cast<int>(lo.w) & m0,
                         static_cast<int>(hi.x) & m1, static_cast<int>(hi.y) & m1,
                         static_cast<int>(hi.z) & m1, static_cast<int>(hi.w) & m1};
        }
        const float ks = *reinterpret_cast<const float*>(slot + kChunk * 128 + 4 * lane);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // slot read before it is refilled
        if (c + 2 < n_live) issue(c + 2);

        float sc[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            v8bf kbf[4];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) kbf[kk] = fp8x8_to_bf16(cur[t][2 * kk], cur[t][2 * kk + 1]);
            v4f d[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) d[j] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
#pragma unroll
                for (int j = 0; j < 4; ++j) d[j] = mfma_bf16_16x16x32(qa[j][kk], kbf[kk], d[j]);
            float acc = 0.f;
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i) acc += wf[j][i] * fmaxf(d[j][i], 0.f);
            sc[t] = acc;
        }
        const float total = head_sum_transpose(sc, g);
        const int key = first + c * kWaves * kChunk + lane;
        if (key < Lmax) out[key] = key <= pos ? total * ks : -INFINITY;
    }
    if (fill_invisible) {
        for (int c = n_live; c < chunks; ++c) {
            const int key = first + c * kWaves * kChunk + lane;
            if (key < Lmax) out[key] = -INFINITY;
        }
    }
}

template <int D, int QR>
hipError_t launch_d(const IndexScoresArgs& a, int chunks, hipStream_t stream) {
    const int keys_per_block = kThreads / kWave * kChunk * chunks;
    const int row_groups = (a.T + QR - 1) / QR;
    dim3 grid(a.B * row_groups, (a.Lmax + keys_per_block - 1) / keys_per_block);
    hipLaunchKernelGGL((index_scores_kernel<D, QR>), grid, dim3(kThreads), 0, stream,
                       a.q, a.q_scale, a.w, a.k, a.k_scale, a.len, a.T, a.H, a.Lmax, a.sm_scale,
                       a.scores, a.fill_invisible, chunks);
    return hipGetLastError();
}

// Key chunks per wave: enough waves to cover every SIMD twice (2048 waves), then longer
// streams per wave (up to 8 chunks) so the block's query and weight set-up is amortised.
template <int D>
hipError_t launch_rows(const IndexScoresArgs& a, hipStream_t stream) {
    if (a.T >= 2) return launch_d<D, 2>(a, 4, stream);
    const long long total_chunks = static_cast<long long>(a.B) * ((a.Lmax + kChunk - 1) / kChunk);
    const int chunks = static_cast<int>(std::min<long long>(8, std::max<long long>(2, total_chunks / 2048)));
    // short streams (two chunks per wave) gain nothing from the deeper LDS pipeline and
    // pay its longer issue sequence: measured 12.4 vs 10.9 us at B=32, L=8192; at
    // B=8, L=131072 (eight chunks per wave) the LDS form is ahead
    if (a.B > kThreads * kMaxSeqPerThread || chunks < 4) return launch_d<D, 1>(a, chunks, stream);
    const int keys_per_block = kWaves * kChunk * chunks;
    dim3 grid(a.B, (a.Lmax + keys_per_block - 1) / keys_per_block);
    hipLaunchKernelGGL((index_scores_decode_kernel<D>), grid, dim3(kThreads), 0, stream,
                       a.q, a.q_scale, a.w, a.k, a.k_scale, a.len, a.H, a.Lmax, a.sm_scale,
                       a.scores, a.fill_invisible, chunks);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_index_scores(const IndexScoresArgs& a, hipStream_t stream) {
    switch (a.D) {
    case 32: return launch_rows<32>(a, stream);
    case 64: return launch_rows<64>(a, stream);
    default: return launch_rows<128>(a, stream);
    }
}

}  // namespace dsa
