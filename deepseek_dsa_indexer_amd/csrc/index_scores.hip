// index_scores.hip -- lightning-indexer scores on gfx950 matrix cores.
//
// Computes, for every query row (b,t) and cache position s < Lmax,
//   I[b,t,s] = k_scale[b,s] * sum_h w'[b,t,h] * max(0, q[b,t,h,:] . k[b,s,:]),
//   w' = w * q_scale * sm_scale,
// with -inf where s > pos(b,t) = len[b] - T + t (with compressed entries, m > 1: where
// s >= (pos + 1) / m; see n_visible).  The weight fold follows the
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
// Mapping.  One wave owns QR query rows and streams 64-key chunks of the key cache, on
// the 32x32x16 matrix-core form (on gfx950 it issues in about the time of the 16x16x32
// form while doing twice the work): S = Q . K^T per (32-head group, 32-key group).  The
// 64 heads of each query row stay in registers as A operands (2 head groups x 8 K-steps
// of 16).  Lane l takes the 64 contiguous bytes [64 hf, 64 hf + 64) of key l % 32 of
// each key group, hf = l / 32, so K-step ks uses dims 64 hf + 8 ks .. + 7 (the queries
// use the same dim -> K-slot assignment, so the 8 K-steps cover each of the 128 dims
// once).  Each product leaves lane l with key l % 32 and heads 8 (r / 4) + 4 hf + r % 4;
// ReLU and the head weights are applied in registers, one exchange with lane l ^ 32
// finishes the head sum, and lane l ends with the score of key (chunk + l): one
// coalesced 256-byte store per row and chunk.  Heads beyond H_I and columns beyond d_I
// are zero (weight 0), which covers the small test shapes.
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

// LDS copy of a query row: [64 heads][128 bytes], the 16-byte chunk c of head h stored at
// chunk position c ^ qswz(h).  Head rows are 32 banks apart, so without the XOR a 16-lane
// read of one chunk over 16 heads would meet only two 4-bank groups (8-way conflicts);
// with it the heads of each parity take distinct groups.
__device__ __forceinline__ int qswz(int h) { return (h >> 1) & 7; }

// Query operands of one row from its LDS copy: lane l, head group hg takes head 32 hg +
// l % 32, dims 64 hf + 8 ks .. + 7; heads past H and bytes past D are zero.  Weights:
// element r of head group hg belongs to head 32 hg + 8 (r / 4) + 4 hf + r % 4.
template <int D>
__device__ __forceinline__ void load_queries(const uint8_t* sq, const float* swf, int H, int lane,
                                             v8bf (&qa)[2][8], float (&wf)[2][16]) {
    const int hf = lane >> 5;
#pragma unroll
    for (int hg = 0; hg < 2; ++hg) {
        const int h = 32 * hg + (lane & 31);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int byte = 64 * hf + 16 * j;
            const uint4 v = *reinterpret_cast<const uint4*>(sq + h * 128 + 16 * ((4 * hf + j) ^ qswz(h)));
            const int mk = (h < H && byte < D) ? -1 : 0;
            qa[hg][2 * j] = fp8x8_to_bf16(static_cast<int>(v.x) & mk, static_cast<int>(v.y) & mk);
            qa[hg][2 * j + 1] = fp8x8_to_bf16(static_cast<int>(v.z) & mk, static_cast<int>(v.w) & mk);
        }
#pragma unroll
        for (int b4 = 0; b4 < 4; ++b4) {
            const float4 w4 = *reinterpret_cast<const float4*>(swf + 32 * hg + 8 * b4 + 4 * hf);
            wf[hg][4 * b4 + 0] = w4.x; wf[hg][4 * b4 + 1] = w4.y;
            wf[hg][4 * b4 + 2] = w4.z; wf[hg][4 * b4 + 3] = w4.w;
        }
    }
}

// max(x, 0) as one instruction.  fmaxf(x, 0.f) compiles to two here: the compiler first
// quiets a possible signalling NaN (v_max_f32 x, x, x) because it cannot tell that the
// matrix-core result is canonical; the dot products of finite codes are never NaN.
__device__ __forceinline__ float relu(float x) {
    float y;
    asm("v_max_f32 %0, 0, %1" : "=v"(y) : "v"(x));
    return y;
}

// Head sum of one 64-key chunk for one query row: kr[kg][j] is lane l's 16-byte piece j
// of key 32 kg + l % 32 (bytes 64 hf + 16 j .. + 15).  Returns, in lane l, the score of
// key (chunk + l) before its key scale.
__device__ __forceinline__ float chunk_scores(const v8bf (&qa)[2][8], const float (&wf)[2][16],
                                              const uint4 (&kr)[2][4], int lane) {
    float tot[2];
#pragma unroll
    for (int kg = 0; kg < 2; ++kg) {
        v16f d[2];
#pragma unroll
        for (int hg = 0; hg < 2; ++hg)
#pragma unroll
            for (int r = 0; r < 16; ++r) d[hg][r] = 0.f;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            const uint4 pc = kr[kg][ks >> 1];
            const v8bf kb = (ks & 1) ? fp8x8_to_bf16(static_cast<int>(pc.z), static_cast<int>(pc.w))
                                     : fp8x8_to_bf16(static_cast<int>(pc.x), static_cast<int>(pc.y));
#pragma unroll
            for (int hg = 0; hg < 2; ++hg) d[hg] = mfma_bf16_32x32x16(qa[hg][ks], kb, d[hg]);
        }
        float acc = 0.f;
#pragma unroll
        for (int hg = 0; hg < 2; ++hg)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc += wf[hg][r] * relu(d[hg][r]);
        tot[kg] = sum_xor32(acc);
    }
    return (lane & 32) ? tot[1] : tot[0];
}

template <int D, int QR, int CHUNKS>
__global__ __launch_bounds__(kThreads)
void index_scores_kernel(const uint8_t* __restrict__ q, const float* __restrict__ q_scale,
                         const float* __restrict__ w, const uint8_t* __restrict__ k,
                         const float* __restrict__ k_scale, const int32_t* __restrict__ len,
                         int T, int H, int Lmax, float sm_scale, float* __restrict__ scores,
                         int fill_invisible, int m)
{
    // a compile-time chunk count: the chunk loop unrolls completely, so the compiler's own
    // waits for the loaded key registers count exactly the loads issued after them
    constexpr int chunks = CHUNKS;
    __shared__ __attribute__((aligned(16))) uint8_t s_q[QR][kMaxHeads * 128];
    __shared__ __attribute__((aligned(16))) float s_wf[QR][kMaxHeads];
    const int keys_per_block = kThreads / kWave * kChunk * chunks;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;

    const int row_groups = (T + QR - 1) / QR;
    int b, t0, yblk;
    if (T == 1 && gridDim.x <= kThreads * kMaxSeqPerThread) {
        // one query row per sequence: numbered blocks (sequences of unequal length
        // still spread evenly over the XCDs; no block past a sequence's end is run
        // unless its positions are to be filled with -inf)
        __shared__ int s_num[kThreads / kWave + 2];
        const int nblk = gridDim.y;
        auto count = [&](int s) {
            return fill_invisible ? nblk : (n_visible(len[s], 1, 0, Lmax, m) + keys_per_block - 1) / keys_per_block;
        };
        if (!number_block<kThreads>(blockIdx.y * gridDim.x + blockIdx.x, gridDim.x, count, s_num, b, yblk))
            return;
        t0 = 0;
    } else {
        b = blockIdx.x / row_groups;
        t0 = (blockIdx.x - b * row_groups) * QR;
        yblk = blockIdx.y;
    }
    const int nrows = min(QR, T - t0);
    // last visible row of each query row (non-decreasing in t)
    int last[QR];
#pragma unroll
    for (int r = 0; r < QR; ++r) last[r] = n_visible(len[b], T, t0 + min(r, nrows - 1), Lmax, m) - 1;
    const int pos_hi = last[QR - 1];

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
    // The raw bytes stay as loaded until the chunk is used (masking them here would make
    // the compiler wait for every load of both chunks before any work starts): okb bit kg
    // tells whether key group kg holds valid keys, and the pieces past d_I are zeroed at use.
    auto load_chunk = [&](int c, uint4 (&dst)[2][4], float& ks, uint32_t& okb) {
        const int kb = chunk_key(c);
        const bool live = c < chunks && kb <= pos_hi;
        okb = 0u;
#pragma unroll
        for (int kg = 0; kg < 2; ++kg) {
            const int key = kb + 32 * kg + (lane & 31);
            okb |= (live && key < Lmax) ? (1u << kg) : 0u;
            const uint8_t* krow = kb_ptr + static_cast<size_t>(min(key, Lmax - 1)) * D;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int byte = 64 * (lane >> 5) + 16 * j;      // pieces past d_I: masked at use
                dst[kg][j] = *reinterpret_cast<const uint4*>(krow + (byte < D ? byte : 0));
            }
        }
        // positions at or beyond Lmax are never stored, so the clamped scale needs no mask
        ks = ks_ptr[min(kb + lane, Lmax - 1)];
    };
    auto masked = [&](const uint4 (&raw)[2][4], uint32_t okb, uint4 (&dst)[2][4]) {
#pragma unroll
        for (int kg = 0; kg < 2; ++kg)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t mk = (((okb >> kg) & 1u) && 64 * (lane >> 5) + 16 * j < D) ? 0xffffffffu : 0u;
                dst[kg][j] = uint4{raw[kg][j].x & mk, raw[kg][j].y & mk, raw[kg][j].z & mk, raw[kg][j].w & mk};
            }
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
    // two register sets, used alternately: chunk c + 2 loads into the set chunk c has used
    uint4 ra[2][4], rb[2][4];
    float ks_a, ks_b;
    uint32_t ok_a, ok_b;
    load_chunk(0, ra, ks_a, ok_a);
    __builtin_amdgcn_sched_barrier(0);     // chunk 0's loads all go out before chunk 1's
    load_chunk(1, rb, ks_b, ok_b);
#pragma unroll
    for (int u = 0; u < kQLoads; ++u) {
        const int i = threadIdx.x + u * kThreads;
        const int r = i / (kMaxHeads * 8);
        const int h = (i / 8) % kMaxHeads;
        const int c16 = i % 8;
        *reinterpret_cast<uint4*>(&s_q[r][h * 128 + 16 * (c16 ^ qswz(h))]) = qok[u] ? qv[u] : uint4{0u, 0u, 0u, 0u};
    }
    if (wr < QR) s_wf[wr][wh] = (wr < nrows && wh < H) ? wv * qsv * sm_scale : 0.f;
    __syncthreads();
    v8bf qa[QR][2][8];
    float wf[QR][2][16];
#pragma unroll
    for (int r = 0; r < QR; ++r) load_queries<128>(s_q[r], s_wf[r], kMaxHeads, lane, qa[r], wf[r]);

    auto process = [&](int c, uint4 (&raw)[2][4], float ks, uint32_t okb) {
        const int kb = chunk_key(c);
        const int key = kb + lane;
        if (kb > pos_hi) {
            if (fill_invisible && key < Lmax)
                for (int r = 0; r < nrows; ++r) out[static_cast<size_t>(r) * Lmax + key] = -INFINITY;
        } else {
            uint4 kr[2][4];
            masked(raw, okb, kr);
#pragma unroll
            for (int r = 0; r < QR; ++r) {
                const float total = chunk_scores(qa[r], wf[r], kr, lane);
                if (r < nrows && key < Lmax)
                    out[static_cast<size_t>(r) * Lmax + key] = (key <= last[r]) ? total * ks : -INFINITY;
            }
        }
    };
    // (the scheduling barriers keep each chunk's work, and so its waits, ahead of the next
    // chunk's: otherwise the interleaved code waits for the later chunk's loads early)
#pragma unroll
    for (int c = 0; c < chunks; c += 2) {
        process(c, ra, ks_a, ok_a);
        __builtin_amdgcn_sched_barrier(0);
        if (c + 2 < chunks) load_chunk(c + 2, ra, ks_a, ok_a);
        if (c + 1 < chunks) {
            process(c + 1, rb, ks_b, ok_b);
            __builtin_amdgcn_sched_barrier(0);
            if (c + 3 < chunks) load_chunk(c + 3, rb, ks_b, ok_b);
        }
    }
}

// ---------------------------------------------------------------- decode form
//
// One query row per block (T = 1).  Each wave streams its chunks global -> LDS with direct
// loads (global_load_lds) into a ring of two 8.25 KB slots of its own, so two chunks per
// wave stay in flight without holding registers (the register-staged form above keeps
// one chunk per wave, 64 KB per CU, in flight).  The query row and the head weights
// arrive the same way.  Slot layout, in load order: 1 KB piece 4 kg + j holds, at lane l,
// bytes [64 hf + 16 j, + 16) of key 32 kg + l % 32 of the chunk -- exactly what lane l
// reads as its operand piece, so each read is one contiguous 16-byte lane read -- and
// the 256 bytes after the keys hold their 64 scales.  The loads are inline
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
                                int fill_invisible, int chunks, int m)
{
    __shared__ __attribute__((aligned(16))) uint8_t s_q[kMaxHeads * 128];
    __shared__ __attribute__((aligned(16))) float s_w[kMaxHeads];
    __shared__ __attribute__((aligned(16))) float s_qs[kMaxHeads];
    __shared__ __attribute__((aligned(16))) uint8_t s_ring[kWaves][kRing][kSlotBytes];
    __shared__ int s_num[kWaves + 2];
    const int keys_per_block = kWaves * kChunk * chunks;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);

    // numbered blocks: sequences of unequal length still spread evenly over the XCDs, and
    // no block past a sequence's end is run unless its positions are to be filled
    int b, yblk;
    {
        const int nblk = gridDim.y;
        auto count = [&](int sq) {
            return fill_invisible ? nblk : (n_visible(len[sq], 1, 0, Lmax, m) + keys_per_block - 1) / keys_per_block;
        };
        if (!number_block<kThreads>(blockIdx.y * gridDim.x + blockIdx.x, gridDim.x, count, s_num, b, yblk))
            return;
    }
    const int pos = n_visible(len[b], 1, 0, Lmax, m) - 1;
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
        for (int kg = 0; kg < 2; ++kg) {
            const uint8_t* krow = kb_ptr + static_cast<size_t>(min(kb + 32 * kg + (lane & 31), Lmax - 1)) * D;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int byte = 64 * (lane >> 5) + 16 * j;     // pieces past d_I are masked on read
                dma16(lds_addr(slot + (4 * kg + j) * 1024), krow + (byte < D ? byte : 0));
            }
        }
        dma4(lds_addr(slot + kChunk * 128), ks_ptr + min(kb + lane, Lmax - 1));
    };

    // ---- the query row (wave w brings LDS bytes [2048 w, 2048 w + 2048) of [64 heads][128]:
    // chunk position p of head h holds chunk p ^ qswz(h)), the head weights (wave 0) and q
    // scales (wave 1), then the first two chunks
    const uint8_t* qrow = q + static_cast<size_t>(b) * H * D;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int o = 2048 * wave + 1024 * i + 16 * lane;
        const int hq = o >> 7;
        const int h = min(hq, H - 1);                         // heads past H, bytes past D: masked on read
        const int byte = 16 * (((o & 127) >> 4) ^ qswz(hq));
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

    // folded weights into s_w (0 past H heads), then the operands
    if (threadIdx.x < kMaxHeads) {
        const int hh = threadIdx.x;
        const float wv = hh < H ? s_w[hh] * s_qs[hh] * sm_scale : 0.f;
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        s_w[hh] = wv;
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    v8bf qa[2][8];
    float wf[2][16];
    load_queries<D>(s_q, s_w, H, lane, qa, wf);

    for (int c = 0; c < n_live; ++c) {
        // chunk c is in when at most chunk c + 1's loads remain
        if (c + 1 < n_live) vm_wait<kChunkLoads>();
        else vm_wait<0>();
        const uint8_t* slot = s_ring[wave][c & 1];
        uint4 cur[2][4];
#pragma unroll
        for (int kg = 0; kg < 2; ++kg)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint4 v = *reinterpret_cast<const uint4*>(slot + (4 * kg + j) * 1024 + 16 * lane);
                const uint32_t mk = 64 * (lane >> 5) + 16 * j < D ? 0xffffffffu : 0u;
                cur[kg][j] = uint4{v.x & mk, v.y & mk, v.z & mk, v.w & mk};
            }
        const float ks = *reinterpret_cast<const float*>(slot + kChunk * 128 + 4 * lane);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // slot read before it is refilled
        if (c + 2 < n_live) issue(c + 2);

        const float total = chunk_scores(qa, wf, cur, lane);
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

template <int D, int QR, int CHUNKS>
hipError_t launch_d(const IndexScoresArgs& a, hipStream_t stream) {
    const int keys_per_block = kThreads / kWave * kChunk * CHUNKS;
    const int row_groups = (a.T + QR - 1) / QR;
    dim3 grid(a.B * row_groups, (a.Lmax + keys_per_block - 1) / keys_per_block);
    return launch_kernel(kPhaseIndex, index_scores_kernel<D, QR, CHUNKS>, grid, dim3(kThreads), 0, stream,
                         a.q, a.q_scale, a.w, a.k, a.k_scale, a.len, a.T, a.H, a.Lmax, a.sm_scale,
                         a.scores, a.fill_invisible, a.m);
}

// Key chunks per wave: enough waves to cover every SIMD twice (2048 waves), then longer
// streams per wave (up to 8 chunks) so the block's query and weight set-up is amortised --
// but at most 4 when full-length 8-chunk blocks would take more than one round of the
// 512 resident workgroups (two per CU): the blocks of many unequal sequences then do not
// fill the last round, and shorter blocks shorten that tail (64 sequences of 1024..65536
// positions: 67.2 -> 64.1 us; 8 sequences of 131072 fill exactly one round of 8-chunk
// blocks: 32.9 against 33.5 us with 4).
constexpr long long kResidentBlocks = 512;
template <int D>
hipError_t launch_rows(const IndexScoresArgs& a, hipStream_t stream) {
    // Several query rows (prefill): one row per wave and 8-chunk streams.  Two rows per wave
    // halve the key loads from L2 but need 419 registers (one wave per SIMD, accumulators
    // read back through AGPRs); one row fits two waves per SIMD (prefill chunk of 8192
    // rows: 837 -> 789 us).
    if (a.T >= 2) return launch_d<D, 1, 8>(a, stream);
    const long long total_chunks = static_cast<long long>(a.B) * ((a.Lmax + kChunk - 1) / kChunk);
    const long long blocks8 = static_cast<long long>(a.B) * ((a.Lmax + kWaves * kChunk * 8 - 1) / (kWaves * kChunk * 8));
    const long long cap = blocks8 > kResidentBlocks ? 4 : 8;
    const int chunks = static_cast<int>(std::min<long long>(cap, std::max<long long>(2, total_chunks / 2048)));
    // short streams (two chunks per wave) gain nothing from the deeper LDS pipeline and
    // pay its longer issue sequence: measured 12.4 vs 10.9 us at B=32, L=8192; at
    // B=8, L=131072 (eight chunks per wave) the LDS form is ahead
    if (a.B > kThreads * kMaxSeqPerThread || chunks < 4) {
        switch (chunks) {
        case 2: return launch_d<D, 1, 2>(a, stream);
        case 3: return launch_d<D, 1, 3>(a, stream);
        case 4: return launch_d<D, 1, 4>(a, stream);
        case 5: return launch_d<D, 1, 5>(a, stream);
        case 6: return launch_d<D, 1, 6>(a, stream);
        case 7: return launch_d<D, 1, 7>(a, stream);
        default: return launch_d<D, 1, 8>(a, stream);
        }
    }
    const int keys_per_block = kWaves * kChunk * chunks;
    dim3 grid(a.B, (a.Lmax + keys_per_block - 1) / keys_per_block);
    return launch_kernel(kPhaseIndex, index_scores_decode_kernel<D>, grid, dim3(kThreads), 0, stream,
                         a.q, a.q_scale, a.w, a.k, a.k_scale, a.len, a.H, a.Lmax, a.sm_scale,
                         a.scores, a.fill_invisible, chunks, a.m);
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
