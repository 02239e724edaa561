// sparse_attn.hip -- sparse attention over the top-k selected positions.
//
// Two paths:
//  * mla_decode_mfma_kernel: the absorbed (MQA) latent form of "dsa-indexer.excalidraw"
//    (core-attention box: all query heads share the selected latent rows, each row
//    serving as key and value) at the V3.2 shape: bf16, 576-wide rows (latent 512 then
//    rope 64), values = the first 512 columns, 64 or 128 heads, bf16 matrix cores.
//  * sparse_attn_generic_kernel: any shape and f32/bf16, both the latent form and the
//    MHA prefill form of the MLA prefill excerpt ("DeepSeek-V3.2-Exp - Causal mask",
//    Multi-head latent attention), on the vector ALUs.  Used for small or unusual shapes.
// Both compute softmax(sm_scale * q.K^T) over the selected and visible positions and mix
// the value rows; lse is the natural-log sum of exponentials of the scaled logits.
#include "dsa_device.h"
#include "dsa_internal.h"

namespace dsa {

namespace {

// ------------------------------------------------------------------ generic path

__device__ __forceinline__ float ld_elem(const void* p, size_t i, int bf16) {
    return bf16 ? bf16_to_f32(static_cast<const uint16_t*>(p)[i]) : static_cast<const float*>(p)[i];
}

// Column d of a 656-byte FP8 latent row: code * block scale for d < 512, else bf16 rope.
__device__ __forceinline__ float fp8_latent_elem(const uint8_t* row, int d) {
    if (d < kFp8Dv) return fp8_to_f32(row[d]) * reinterpret_cast<const float*>(row + kFp8Dv)[d >> 7];
    return bf16_to_f32(reinterpret_cast<const uint16_t*>(row + kFp8Dv + 16)[d - kFp8Dv]);
}

constexpr int kGenThreads = 256;

// One workgroup per (b, t, h).  Dynamic LDS: q row (Dk floats) + k logits.
__global__ __launch_bounds__(kGenThreads)
void sparse_attn_generic_kernel(SparseAttnArgs a)
{
    extern __shared__ float smem[];
    float* qs = smem;
    float* logit = smem + a.Dk;
    __shared__ float red[kGenThreads / kWave];
    __shared__ float bcast;

    const int H = a.H;
    const int row = blockIdx.x / H;
    const int h = blockIdx.x - row * H;
    const int b = row / a.T;
    const int t = row - b * a.T;
    const int pos = a.len ? n_visible(a.len[b], a.T, t, a.kv_rows, a.m) - 1 : t;   // last visible row
    const int32_t* sel = a.idx + static_cast<size_t>(row) * a.k;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;

    const size_t qoff = (static_cast<size_t>(row) * H + h) * a.Dk;
    for (int d = threadIdx.x; d < a.Dk; d += kGenThreads) qs[d] = ld_elem(a.q, qoff + d, a.bf16);
    __syncthreads();

    float mx = -INFINITY;
    for (int j = threadIdx.x; j < a.k; j += kGenThreads) {
        const int s = sel[j];
        float l = -INFINITY;
        if (s >= 0 && s <= pos) {
            float acc = 0.f;
            if (a.fp8_latent) {
                const uint8_t* row = static_cast<const uint8_t*>(a.kbase) +
                                     (static_cast<size_t>(b) * a.kv_rows + s) * kFp8RowBytes;
                for (int d = 0; d < a.Dk; ++d) acc += qs[d] * fp8_latent_elem(row, d);
            } else {
                const size_t koff = (static_cast<size_t>(b) * a.kv_rows + s) * a.row_stride +
                                    static_cast<size_t>(h) * a.head_stride;
                for (int d = 0; d < a.Dk; ++d) acc += qs[d] * ld_elem(a.kbase, koff + d, a.bf16);
            }
            l = acc * a.sm_scale;
        }
        logit[j] = l;
        mx = fmaxf(mx, l);
    }
    mx = wave_max(mx);
    if (lane == 0) red[wave] = mx;
    __syncthreads();
    if (threadIdx.x == 0) {
        float m = red[0];
        for (int i = 1; i < kGenThreads / kWave; ++i) m = fmaxf(m, red[i]);
        bcast = m;
    }
    __syncthreads();
    mx = bcast;
    __syncthreads();

    float sum = 0.f;
    for (int j = threadIdx.x; j < a.k; j += kGenThreads) {
        const float p = (logit[j] == -INFINITY) ? 0.f : expf(logit[j] - mx);
        logit[j] = p;
        sum += p;
    }
    sum = wave_sum(sum);
    if (lane == 0) red[wave] = sum;
    __syncthreads();
    if (threadIdx.x == 0) {
        float s = 0.f;
        for (int i = 0; i < kGenThreads / kWave; ++i) s += red[i];
        bcast = s;
    }
    __syncthreads();
    sum = bcast;
    const float inv = sum > 0.f ? 1.f / sum : 0.f;

    const size_t ooff = (static_cast<size_t>(row) * H + h) * a.Dv;
    for (int d = threadIdx.x; d < a.Dv; d += kGenThreads) {
        float acc = 0.f;
        for (int j = 0; j < a.k; ++j) {
            const float p = logit[j];
            if (p == 0.f) continue;
            const int s = sel[j];
            if (a.fp8_latent) {
                const uint8_t* row = static_cast<const uint8_t*>(a.vbase) +
                                     (static_cast<size_t>(b) * a.kv_rows + s) * kFp8RowBytes;
                acc += p * fp8_latent_elem(row, d);
                continue;
            }
            const size_t voff = (static_cast<size_t>(b) * a.kv_rows + s) * a.row_stride_v +
                                static_cast<size_t>(h) * a.head_stride_v;
            acc += p * ld_elem(a.vbase, voff + d, a.bf16);
        }
        acc *= inv;
        if (a.bf16) static_cast<uint16_t*>(a.out)[ooff + d] = f32_to_bf16(acc);
        else static_cast<float*>(a.out)[ooff + d] = acc;
    }
    if (a.lse && threadIdx.x == 0)
        a.lse[static_cast<size_t>(row) * H + h] = sum > 0.f ? mx + logf(sum) : -INFINITY;
}

// ------------------------------------------------------------------ matrix-core latent path
//
// One workgroup (8 waves, two per SIMD) owns one query row (b,t), one split of its k
// slots and 64 or 128 heads (128 heads of few rows go to two 64-head workgroups, which
// share each gathered tile through their XCD's L2), so every selected latent row is
// fetched from memory once per row and split.  Per tile of 32 selected positions:
//   gather   32 latent rows -> LDS with direct global->LDS 16-byte loads.  Four tile
//            buffers are distinct LDS objects; two tiles stay in flight while one is
//            multiplied against Q and the previous one against P.  The 16-byte chunks
//            of each row are XOR-swizzled inside 128-byte groups so the matrix-core
//            operand reads spread over the LDS banks;
//   QK       wave w computes S^T = K . Q^T for head tile w (16 heads) and all 32 keys of
//            the tile (keys as MFMA rows; the wave's queries stay in registers as 18 B
//            operands);
//   softmax  per head, entirely inside the owning wave, relative to a fixed reference
//            (below); the bf16 numerators go to LDS in MFMA operand layout;
//   PV       wave w owns output columns 64w..64w+63 for all heads: O += P . V with V read
//            from the same LDS tile by transpose reads (the value is the first 512
//            columns of the latent row).
// Software pipeline: step i runs PV of tile i-1 and QK + softmax of tile i between two
// workgroup barriers, then publishes P and the rescale factors of tile i, so a tile
// costs two barriers but the matrix-core work of both products sits in one phase.
// Waves 0-3 run at a raised issue priority over waves 4-7 (they pair up on the four
// SIMDs), so within a step the pair drifts apart and one wave's softmax overlaps the
// other's matrix-core work.  Splits of one row are merged by a log-sum-exp combine
// kernel.
//
// No running-maximum rescale of the output accumulators: each head's numerators are
// exp2(logit - m_ref) with m_ref the maximum of the first tile that has a usable slot,
// which is exact in floating point while nothing overflows, and keeps a conditional
// update of all accumulators (and the per-tile rescale factors) out of the loop.  A later
// logit more than 2^64 above the reference (log2 units) marks the split, and a marked
// split is recomputed from its first tile with the split's true maximum as the
// reference, so every numerator is then at most 1.
constexpr int kMlaThreads = 512;
constexpr int kMlaWaves = 8;
constexpr int kMaxHt = 8;                          // up to 128 heads per workgroup
constexpr int kDq = 576;
constexpr int kDv = 512;
constexpr int kRowBytes = kDq * 2;                 // 1152
constexpr int kRowChunks = kRowBytes / 16;         // 72
constexpr int kKt = 32;                            // selected positions per tile
constexpr int kTileBytes = kKt * kRowBytes;        // 36864
constexpr int kTileLoads = kTileBytes / (kWave * 16);   // 36 wave-wide 1 KB loads
constexpr int kMaxSlots = 1024;                    // slots per split held in LDS
constexpr int kDs = kDq / 32;                      // 18 K-steps of the QK product
constexpr int kDtW = kDv / kMlaWaves / 16;         // 4 output column tiles per wave
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRefSpan = 64.0f;                  // log2 units above the reference

constexpr int kBufs = 4;                          // tile ring
__shared__ __attribute__((aligned(16))) uint8_t g_kbuf[kBufs * kTileBytes];
__shared__ __attribute__((aligned(16))) uint8_t g_pbuf[kMaxHt][kWave][16];
__shared__ int32_t g_rescale[kMlaWaves];          // per-wave "recompute the split" flags
__shared__ float g_l[kMaxHt * 16];
__shared__ float g_m[kMaxHt * 16];
__shared__ int32_t g_keys[kMaxSlots];

__device__ __forceinline__ uint8_t* kbuf(int ti) { return g_kbuf + (ti & (kBufs - 1)) * kTileBytes; }

template <int N>
__device__ __forceinline__ void wait_vmcnt() { asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory"); }

__device__ __forceinline__ int swz_chunk(int key, int chunk) { return chunk ^ (key & 7); }

// Workgroup barrier for LDS data only: waits for this wave's LDS operations, not for
// its global loads, so tile prefetches stay in flight across it (__syncthreads() would
// also drain every outstanding global->LDS load).
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Wait until this wave's gathers of the current tile have landed, leaving the tile
// issued after it in flight (waves 0..3 issue 5 loads per tile, waves 4..7 four).
__device__ __forceinline__ void wait_tile(bool later, bool five) {
    if (!later) wait_vmcnt<0>();
    else if (five) wait_vmcnt<5>();
    else wait_vmcnt<4>();
}

// Issue the direct global->LDS loads of tile `ti` into `dst`: wave w issues the
// wave-wide 1 KB loads ci = w, w + 8, ... < 36 (five for waves 0..3, four for waves
// 4..7); lane l of load ci fetches the 16-byte chunk c = 64 ci + l of the tile, i.e.
// chunk c % 72 of selected row c / 72, stored at the swizzled chunk position of that row.
// The per-lane offsets are recomputed from an opaque copy of the lane id on every call
// (kept live across the loop they would cost registers, and spill reloads would drain
// the loads in flight).  The loads are written as inline assembly so that the compiler,
// which cannot tell the four tile buffers apart through a runtime tile index, does not
// drain them before every LDS read; completion is tracked explicitly with wait_tile()
// and made visible to the other waves by lds_barrier().  M0 carries the wave-uniform LDS
// destination; no other instruction of this kernel uses M0.
constexpr int kGatherMax = (kTileLoads + kMlaWaves - 1) / kMlaWaves;   // 5
__device__ __forceinline__ void gather_tile(const uint8_t* lat_b, int ti, uint8_t* dst, int wave,
                                            int lane) {
    asm volatile("" : "+v"(lane));
    const uint32_t lds_base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
        (__attribute__((address_space(3))) uint8_t*)(dst)));
    int s[kGatherMax], key[kGatherMax];
#pragma unroll
    for (int i = 0; i < kGatherMax; ++i) {
        const int c = (wave + kMlaWaves * i) * kWave + lane;
        key[i] = min(c / kRowChunks, kKt - 1);
        s[i] = g_keys[ti * kKt + key[i]];
    }
#pragma unroll
    for (int i = 0; i < kGatherMax; ++i) {
        const int ci = wave + kMlaWaves * i;
        if (ci < kTileLoads) {
            const int c = ci * kWave + lane;
            const int row = s[i] < 0 ? 0 : s[i];     // unused slots read row 0 (masked later)
            const uint32_t off = static_cast<uint32_t>(row) * kRowBytes +
                                 swz_chunk(key[i], c - key[i] * kRowChunks) * 16;
            const uint8_t* src = lat_b + off;
            const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds_base + ci * kWave * 16);
            asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
                         :: "s"(m0v), "v"(src) : "memory");
        }
    }
}

template <int NHT>
struct MlaState {
    v8bf qreg[kDs];
    v4f o[NHT][kDtW];
    float m_ref;                 // reference logit of this lane's head (log2 units)
    float m_max;                 // largest logit seen
    float l_run;
    bool over;                   // a logit exceeded m_ref + kRefSpan
};

typedef __bf16 v4bf_t __attribute__((ext_vector_type(4)));

// QK and softmax numerators of tile ti (buffer kb) for head tile `wave` (< NHT).  Returns
// the bf16 numerators in PV A-operand layout; they are published after the step's second
// barrier.  fixed: m_ref is final.
template <int NHT>
__device__ __forceinline__ void mla_qk_softmax(MlaState<NHT>& st, const uint8_t* kb, int ti,
                                               float scale_log2, int lane, v8s& pk, bool fixed) {
    // Per-lane LDS offsets are recomputed in every tile step from an opaque copy of the
    // lane id: hoisted out of the loop they would be kept live once per buffer copy.
    int lane_o = lane;
    asm volatile("" : "+v"(lane_o));
    const int go = lane_o >> 4;
    const int no = lane_o & 15;

    // ---- QK: 32 keys x 16 heads, two MFMA chains (key halves).
    // Logical chunk 4 ds + g of key row 16 kt + n sits at chunk (4 ds + g) ^ (n & 7)
    //   = 8 (ds / 2) + ((4 (ds & 1) + g) ^ (n & 7)),
    // so two base offsets per key half plus an immediate cover all 18 K-steps.
    v4f sacc[2] = {v4f{0.f, 0.f, 0.f, 0.f}, v4f{0.f, 0.f, 0.f, 0.f}};
    {
        const uint8_t* base[2][2];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
            const uint8_t* krow = kb + (16 * kt + no) * kRowBytes;
            base[kt][0] = krow + ((go) ^ (no & 7)) * 16;
            base[kt][1] = krow + ((4 + go) ^ (no & 7)) * 16;
        }
        constexpr int kPre = 2;               // K-steps of operand reads in flight
        v8bf a[kPre][2];
#pragma unroll
        for (int ds = 0; ds < kPre; ++ds)
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
                a[ds][kt] = *reinterpret_cast<const v8bf*>(base[kt][ds & 1] + (ds >> 1) * 128);
#pragma unroll
        for (int ds = 0; ds < kDs; ++ds) {
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
                sacc[kt] = mfma_bf16_16x16x32(a[ds % kPre][kt], st.qreg[ds], sacc[kt]);
            if (ds + kPre < kDs) {
                const int dn = ds + kPre;
#pragma unroll
                for (int kt = 0; kt < 2; ++kt)
                    a[ds % kPre][kt] = *reinterpret_cast<const v8bf*>(base[kt][dn & 1] + (dn >> 1) * 128);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    // ---- online softmax of the wave's 16 heads over the 32 keys of this tile.
    // Lane (g, n) holds head n, keys 16 kt + 4 g + i, which is exactly K-slot
    // j = 4 kt + i of the P operand of the PV product.
    float sv[8];
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bool valid = g_keys[ti * kKt + 16 * kt + 4 * go + i] >= 0;
            const float v = valid ? sacc[kt][i] * scale_log2 : -INFINITY;
            sv[4 * kt + i] = v;
            mx = fmaxf(mx, v);
        }
    mx = max_xor32(max_xor16(mx));
    if (!fixed) {
        if (st.m_ref == -INFINITY) st.m_ref = mx;       // first tile with a usable slot
        st.m_max = fmaxf(st.m_max, mx);
        st.over = st.over || mx > st.m_ref + kRefSpan;
    }
    // while no usable slot has been seen every logit is -inf: any finite reference gives 0
    const float mref = st.m_ref == -INFINITY ? 0.f : st.m_ref;
    float psum = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const float p = exp2_num(sv[j] - mref);
        psum += p;
        pk[j] = static_cast<short>(f32_to_bf16(p));
    }
    st.l_run += sum_xor32(sum_xor16(psum));
}

// PV of the previous tile (buffer kb, numerators in g_pbuf): output columns
// 64 wave .. + 63 for all heads.  V operands come
// from LDS transpose reads: for K-slots j = 4 kt + r the lane needs V[16 kt + 4 g + r][d],
// d = 64 wave + 16 dt + n; within each 16-lane group a transpose read hands lane n the
// element at (address of lane 4 r + n / 4) + n % 4, so lane m supplies row
// 16 kt + 4 g + m / 4, columns d0 + 4 (m % 4) .. + 3.
template <int NHT>
__device__ __forceinline__ void mla_pv(MlaState<NHT>& st, const uint8_t* kb, int wave, int lane) {
    int lane_o = lane;
    asm volatile("" : "+v"(lane_o));
    const int go = lane_o >> 4;
    const int no = lane_o & 15;
    v8bf vb[kDtW];
#pragma unroll
    for (int dt = 0; dt < kDtW; ++dt) {
        const int d0 = 64 * wave + 16 * dt;
        v4bf_t half[2];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
            const int key = 16 * kt + 4 * go + (no >> 2);
            const int chunk = (d0 >> 3) + ((no & 3) >> 1);
            const int off = key * kRowBytes + (chunk ^ (key & 7)) * 16 + (no & 1) * 8;
            half[kt] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                (__attribute__((address_space(3))) v4bf_t*)(kb + off));
        }
        vb[dt] = v8bf{half[0][0], half[0][1], half[0][2], half[0][3],
                      half[1][0], half[1][1], half[1][2], half[1][3]};
    }
#pragma unroll
    for (int h = 0; h < NHT; ++h) {
        __builtin_amdgcn_sched_barrier(0);
        const v8bf pa = *reinterpret_cast<const v8bf*>(&g_pbuf[h][lane][0]);
#pragma unroll
        for (int dt = 0; dt < kDtW; ++dt) st.o[h][dt] = mfma_bf16_16x16x32(pa, vb[dt], st.o[h][dt]);
    }
}

// Publish P of the wave's head tile (after the step's second barrier: every wave is then
// done reading the previous tile's).
__device__ __forceinline__ void mla_publish(const v8s& pk, int wave, int lane) {
    *reinterpret_cast<v8s*>(&g_pbuf[wave][lane][0]) = pk;
}

// ---- FP8 latent rows (656 bytes: 512 e4m3fn codes, four fp32 block scales, 64 bf16 rope
// values).  Same pipeline and roles as above; what changes:
//   tile     32 rows of 656 bytes, unswizzled, with a 128-byte gap between rows 15 and
//            16 (row r at 656 r, plus 128 from row 16 on) so that the transpose reads of
//            PV, which touch rows κ and κ + 16 together, fall in different LDS banks;
//            21 wave-wide 1 KB loads fill 1320 of the 1344 16-byte slots of a 21 KB
//            buffer (the gap and the tail slots get dummy copies);
//   QK       the code bytes are widened to bf16 exactly in registers, and each 128-column
//            block gets its own matrix-core chain, scaled per key afterwards in fp32
//            (logit = sum_j scale_j . (q_j . code_j) + q_rope . rope), so no product is
//            rounded beyond the fp32 accumulation;
//   PV       one 8-byte transpose read hands each lane the eight key codes of its
//            output column; wave w's columns lie in block w / 2, whose per-key scale is
//            folded into the wave's copy of P: every QK wave publishes four copies of
//            its bf16 numerators, p . scale_j for j = 0..3.
constexpr int kF8Row = kFp8RowBytes;                   // 656
constexpr int kF8Gap = 128;                            // LDS gap before row 16
constexpr int kF8Slots = (kKt * kF8Row + kF8Gap) / 16; // 1320 used 16-byte slots
constexpr int kF8Loads = (kF8Slots + kWave - 1) / kWave;   // 21
constexpr int kF8TileStride = kF8Loads * kWave * 16;   // 21504
constexpr int kF8Scale = kFp8Dv;                       // byte offset of the scales
constexpr int kF8Rope = kFp8Dv + 16;                   // byte offset of the rope values
constexpr int kF8PbufOff = kBufs * kF8TileStride;      // P copies: [block 4][ht 8][lane][16 B]
constexpr int kF8GatherMax = (kF8Loads + kMlaWaves - 1) / kMlaWaves;   // 3
static_assert(kF8PbufOff + 4 * kMaxHt * kWave * 16 <= kBufs * kTileBytes,
              "FP8 tiles and P copies fit in the tile ring's LDS");

__device__ __forceinline__ uint8_t* kbuf8(int ti) { return g_kbuf + (ti & (kBufs - 1)) * kF8TileStride; }
__device__ __forceinline__ int f8_row_off(int r) { return r * kF8Row + (r >= 16 ? kF8Gap : 0); }

// Wait for this wave's loads of the current tile (waves 0..4 issue 3 per tile, 5..7 two).
__device__ __forceinline__ void wait_tile8(bool later, bool three) {
    if (!later) wait_vmcnt<0>();
    else if (three) wait_vmcnt<3>();
    else wait_vmcnt<2>();
}

// Direct global->LDS loads of FP8 tile `ti`: lane l of wave load ci fills 16-byte slot
// p = 64 ci + l of the buffer.  Slots 0..655 are rows 0..15 (41 slots a row), 656..663
// the gap, 664..1319 rows 16..31, 1320..1343 slack; gap and slack lanes copy chunk 0 of
// the tile's first row (in bounds, never read back).
__device__ __forceinline__ void gather_tile8(const uint8_t* lat_b, int ti, uint8_t* dst, int wave,
                                             int lane) {
    asm volatile("" : "+v"(lane));
    const uint32_t lds_base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
        (__attribute__((address_space(3))) uint8_t*)(dst)));
    constexpr int kHalf = 16 * (kF8Row / 16);          // 656 slots per 16 rows
    constexpr int kHi = kHalf + kF8Gap / 16;           // 664: first slot of row 16
    int s[kF8GatherMax], chunk[kF8GatherMax];
#pragma unroll
    for (int i = 0; i < kF8GatherMax; ++i) {
        const int p = (wave + kMlaWaves * i) * kWave + lane;
        const bool lo = p < kHalf;
        const bool used = lo || (p >= kHi && p < kF8Slots);
        const int rel = lo ? p : p - kHi;
        const int r = used ? rel / (kF8Row / 16) : 0;
        chunk[i] = used ? rel - r * (kF8Row / 16) : 0;
        s[i] = g_keys[ti * kKt + (used && !lo ? 16 + r : r)];
    }
#pragma unroll
    for (int i = 0; i < kF8GatherMax; ++i) {
        const int ci = wave + kMlaWaves * i;
        if (ci < kF8Loads) {
            const int row = s[i] < 0 ? 0 : s[i];     // unused slots read row 0 (masked later)
            const uint8_t* src = lat_b + static_cast<uint32_t>(row) * kF8Row + chunk[i] * 16;
            const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds_base + ci * kWave * 16);
            asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
                         :: "s"(m0v), "v"(src) : "memory");
        }
    }
}

// QK and softmax numerators of FP8 tile ti for head tile `wave`; returns the four
// block-scaled bf16 copies of the numerators in PV A-operand layout.
template <int NHT>
__device__ __forceinline__ void mla_qk_softmax8(MlaState<NHT>& st, const uint8_t* kb, int ti,
                                                float scale_log2, int lane, v8s (&pk)[4],
                                                bool fixed) {
    int lane_o = lane;
    asm volatile("" : "+v"(lane_o));
    const int go = lane_o >> 4;
    const int no = lane_o & 15;
    // A operand: key row 16 kt + n, columns 32 ds + 8 g .. + 7
    const uint8_t* krow[2] = {kb + f8_row_off(no) + 8 * go, kb + f8_row_off(16 + no) + 8 * go};
    // scales of the keys this lane's results belong to: rows 16 kt + 4 g + i
    const uint8_t* srow = kb + f8_row_off(4 * go) + kF8Scale;
    auto scale_of = [&](int kt, int i, int blk) -> float {
        return *reinterpret_cast<const float*>(srow + kt * (16 * kF8Row + kF8Gap) + i * kF8Row + 4 * blk);
    };
    // Register budget: the queries and the output accumulators hold 200 of the wave's 256
    // registers, so the two key halves run one after the other (one chain each), the block
    // scales are read in the middle of their block and the rope operands only once the
    // last code bytes have been widened.
    v4f tot[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
        constexpr int kPre = 2;
        uint2 raw[kPre];
#pragma unroll
        for (int ds = 0; ds < kPre; ++ds) raw[ds] = *reinterpret_cast<const uint2*>(krow[kt] + 32 * ds);
        v8bf rope[2];
        tot[kt] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int blk = 0; blk < 4; ++blk) {
            v4f acc = v4f{0.f, 0.f, 0.f, 0.f};
            float sc[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int ds = 4 * blk + j;
                const v8bf a = fp8x8_to_bf16(static_cast<int>(raw[ds % kPre].x),
                                             static_cast<int>(raw[ds % kPre].y));
                if (ds + kPre < 16)
                    raw[ds % kPre] = *reinterpret_cast<const uint2*>(krow[kt] + 32 * (ds + kPre));
                if (ds == 15) {
#pragma unroll
                    for (int r = 0; r < 2; ++r)
                        rope[r] = *reinterpret_cast<const v8bf*>(krow[kt] - 8 * go + kF8Rope + 64 * r + 16 * go);
                }
                if (j == 1) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) sc[i] = scale_of(kt, i, blk);
                }
                acc = mfma_bf16_16x16x32(a, st.qreg[ds], acc);
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) tot[kt][i] += acc[i] * sc[i];
        }
        v4f acc = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int r = 0; r < 2; ++r) acc = mfma_bf16_16x16x32(rope[r], st.qreg[16 + r], acc);
        tot[kt] += acc;
    }
    // softmax numerators, as for bf16 rows
    float sv[8];
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bool valid = g_keys[ti * kKt + 16 * kt + 4 * go + i] >= 0;
            const float v = valid ? tot[kt][i] * scale_log2 : -INFINITY;
            sv[4 * kt + i] = v;
            mx = fmaxf(mx, v);
        }
    mx = max_xor32(max_xor16(mx));
    if (!fixed) {
        if (st.m_ref == -INFINITY) st.m_ref = mx;
        st.m_max = fmaxf(st.m_max, mx);
        st.over = st.over || mx > st.m_ref + kRefSpan;
    }
    const float mref = st.m_ref == -INFINITY ? 0.f : st.m_ref;
    float psum = 0.f;
    float p[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        p[j] = exp2_num(sv[j] - mref);
        psum += p[j];
    }
    st.l_run += sum_xor32(sum_xor16(psum));
    // value-block copies: numerator of key 16 kt + 4 g + i times that key's scale j
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float4 s4 = *reinterpret_cast<const float4*>(srow + kt * (16 * kF8Row + kF8Gap) + i * kF8Row);
            pk[0][4 * kt + i] = static_cast<short>(f32_to_bf16(p[4 * kt + i] * s4.x));
            pk[1][4 * kt + i] = static_cast<short>(f32_to_bf16(p[4 * kt + i] * s4.y));
            pk[2][4 * kt + i] = static_cast<short>(f32_to_bf16(p[4 * kt + i] * s4.z));
            pk[3][4 * kt + i] = static_cast<short>(f32_to_bf16(p[4 * kt + i] * s4.w));
        }
}

// PV of the previous FP8 tile: output columns 64 wave .. + 63 (block wave / 2) for all
// heads.  Within each 16-lane group an 8-byte transpose read hands lane n byte n % 8 of
// the address of lane 2 e + n / 8 as element e, so lane m supplies row
// κ = 16 (e / 4) + 4 g + e % 4 (e = m / 2), columns d0 + 8 (m % 2) .. + 7: lane n then
// holds column d0 + n of the eight keys of its P operand slots.
template <int NHT>
__device__ __forceinline__ void mla_pv8(MlaState<NHT>& st, const uint8_t* kb, int wave, int lane) {
    typedef int v2i_t __attribute__((ext_vector_type(2)));
    int lane_o = lane;
    asm volatile("" : "+v"(lane_o));
    const int go = lane_o >> 4;
    const int mo = lane_o & 15;
    const int e = mo >> 1;
    const uint8_t* src = kb + f8_row_off(16 * (e >> 2) + 4 * go + (e & 3)) + 8 * (mo & 1) + 64 * wave;
    v8bf vb[kDtW];
#pragma unroll
    for (int dt = 0; dt < kDtW; ++dt) {
        const v2i_t r = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
            (__attribute__((address_space(3))) v2i_t*)(src + 16 * dt));
        vb[dt] = fp8x8_to_bf16(r[0], r[1]);
    }
    const uint8_t* pb = g_kbuf + kF8PbufOff + ((wave >> 1) * kMaxHt * kWave + lane) * 16;
#pragma unroll
    for (int h = 0; h < NHT; ++h) {
        __builtin_amdgcn_sched_barrier(0);
        const v8bf pa = *reinterpret_cast<const v8bf*>(pb + h * kWave * 16);
#pragma unroll
        for (int dt = 0; dt < kDtW; ++dt) st.o[h][dt] = mfma_bf16_16x16x32(pa, vb[dt], st.o[h][dt]);
    }
}

__device__ __forceinline__ void mla_publish8(const v8s (&pk)[4], int wave, int lane) {
#pragma unroll
    for (int blk = 0; blk < 4; ++blk)
        *reinterpret_cast<v8s*>(g_kbuf + kF8PbufOff + ((blk * kMaxHt + wave) * kWave + lane) * 16) = pk[blk];
}

template <int NHT, bool F8>
__global__ __launch_bounds__(kMlaThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void mla_decode_mfma_kernel(const uint16_t* __restrict__ q, const uint8_t* __restrict__ latent,
                            const int32_t* __restrict__ idx, const int32_t* __restrict__ len,
                            int T, int Lmax, int k, int m, int tiles_per_split, int n_splits,
                            int H_total, float scale_log2, uint16_t* __restrict__ out,
                            float* __restrict__ lse, uint16_t* __restrict__ part_o,
                            float* __restrict__ part_lse)
{
    constexpr int H = NHT * 16;                        // heads of this workgroup
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);   // wave-uniform: SGPR
    const int g = lane >> 4;
    const int n = lane & 15;
    if (wave < 4) __builtin_amdgcn_s_setprio(1);

    // Workgroup (row, split, head part): H_total / H parts of H heads each.  Consecutive
    // workgroups go to different XCDs (round robin over 8), so block
    // (part * n_splits + split) * rows + row puts every workgroup of a row on the same
    // XCD whenever rows is a multiple of 8: the row's queries and selected latent rows
    // are then fetched into one L2 and shared.
    const int rows = gridDim.x / (n_splits * (H_total / H));
    const int row = blockIdx.x % rows;
    const int rest = blockIdx.x / rows;
    const int split = rest % n_splits;
    const int head0 = (rest / n_splits) * H;
    const int b = row / T;
    const int t = row - b * T;

    const int n_tiles_total = (k + kKt - 1) / kKt;
    const int tile0 = split * tiles_per_split;
    const int n_tiles = max(0, min(tiles_per_split, n_tiles_total - tile0));
    const int nslots = n_tiles * kKt;

    // The three independent start-up loads go out back to back, in the order they are
    // needed: this split's selected positions, the sequence length, the queries.  The
    // positions are checked against pos only when both have arrived (the queries stay
    // in flight), so the gathers wait for one memory latency instead of three.
    const int32_t* sel = idx + static_cast<size_t>(row) * k;
    constexpr int kSlotIters = kMaxSlots / kMlaThreads;
    int sraw[kSlotIters];
#pragma unroll
    for (int i = 0; i < kSlotIters; ++i) {
        const int j = threadIdx.x + i * kMlaThreads;
        const int slot = tile0 * kKt + j;
        sraw[i] = (j < nslots && slot < k) ? sel[slot] : -1;
    }
    const int seq_len = len[b];

    MlaState<NHT> st;
    {
        // queries of head tile `wave` as MFMA B operands: head 16 wave + n, dims 32 ds + 8 g
        // (only the QK waves hold them; with 64 heads the other four waves load nothing)
        if (wave < NHT) {
            const uint16_t* qrow = q + (static_cast<size_t>(row) * H_total + head0 + 16 * wave + n) * kDq + 8 * g;
#pragma unroll
            for (int ds = 0; ds < kDs; ++ds) st.qreg[ds] = *reinterpret_cast<const v8bf*>(qrow + 32 * ds);
        } else {
#pragma unroll
            for (int ds = 0; ds < kDs; ++ds) st.qreg[ds] = v8bf{};
        }
    }

    // selected positions of this split (-1: unused slot or not visible)
    const int pos = n_visible(seq_len, T, t, Lmax, m) - 1;   // last visible cache row
#pragma unroll
    for (int i = 0; i < kSlotIters; ++i) {
        const int j = threadIdx.x + i * kMlaThreads;
        const int s = sraw[i];
        if (j < nslots) g_keys[j] = (s >= 0 && s <= pos) ? s : -1;
    }
    st.m_ref = -INFINITY;
    st.m_max = -INFINITY;
    st.over = false;

    const uint8_t* lat_b = latent + static_cast<size_t>(b) * Lmax * (F8 ? kF8Row : kRowBytes);
    lds_barrier();        // g_keys ready (its stores waited for the idx loads)
    const bool qk_wave = wave < NHT;
    // One pass over the split's tiles; the queries and the selected positions stay in
    // place between passes.
    // Tile 0 goes out together with the queries; wait for both, then put tile 1 in
    // flight.  The compiler's own wait for the query registers (it does not see the
    // gathers) then falls here, where nothing else is outstanding.
    // Step 0: QK + softmax of tile 0.  Steps 1 .. n_tiles-1: PV of tile i-1 and QK +
    // softmax of tile i.  Last: PV of tile n_tiles-1.  Every step waits for its tile,
    // passes a barrier (tile i and P(i-1) visible; the buffer of tile i-2 released) and
    // prefetches tile i+2; a second barrier separates the reads of P(i-1) from the
    // publication of P(i).  The loop body has no data-dependent branch around the
    // accumulators, so they keep their registers across iterations.
    // The tile-format specific steps (bf16 rows or FP8 rows).
    auto gather = [&](int ti) {
        if constexpr (F8) gather_tile8(lat_b, ti, kbuf8(ti), wave, lane);
        else gather_tile(lat_b, ti, kbuf(ti), wave, lane);
    };
    auto wait_for = [&](bool later) {
        if constexpr (F8) wait_tile8(later, wave < 5);
        else wait_tile(later, wave < 4);
    };
    auto pv = [&](int ti) {
        if constexpr (F8) mla_pv8<NHT>(st, kbuf8(ti), wave, lane);
        else mla_pv<NHT>(st, kbuf(ti), wave, lane);
    };
    auto qk_publish = [&](int ti, bool fixed) {
        if constexpr (F8) {
            v8s pk[4];
            if (qk_wave) mla_qk_softmax8<NHT>(st, kbuf8(ti), ti, scale_log2, lane, pk, fixed);
            lds_barrier();
            if (qk_wave) mla_publish8(pk, wave, lane);
        } else {
            v8s pk;
            if (qk_wave) mla_qk_softmax<NHT>(st, kbuf(ti), ti, scale_log2, lane, pk, fixed);
            lds_barrier();
            if (qk_wave) mla_publish(pk, wave, lane);
        }
    };
    auto pass = [&](bool fixed) {
#pragma unroll
        for (int h = 0; h < NHT; ++h)
#pragma unroll
            for (int dt = 0; dt < kDtW; ++dt) st.o[h][dt] = v4f{0.f, 0.f, 0.f, 0.f};
        st.l_run = 0.f;
        if (n_tiles > 0) gather(0);
        wait_vmcnt<0>();
#pragma unroll
        for (int ds = 0; ds < kDs; ++ds) asm volatile("" :: "v"(st.qreg[ds]));
        if (n_tiles > 1) gather(1);
        if (n_tiles > 0) {
            wait_for(1 < n_tiles);
            lds_barrier();
            if (2 < n_tiles) gather(2);
            qk_publish(0, fixed);
        }
        for (int ti = 1; ti < n_tiles; ++ti) {
            wait_for(ti + 1 < n_tiles);
            lds_barrier();
            if (ti + 2 < n_tiles) gather(ti + 2);
            pv(ti - 1);
            __builtin_amdgcn_sched_barrier(0);
            qk_publish(ti, fixed);
        }
        if (n_tiles > 0) {
            lds_barrier();
            pv(n_tiles - 1);
        }
    };
    pass(false);
    // a head of the workgroup past its reference span: redo the split from the split's
    // maximum (a uniform decision: every wave reads the same flags)
    if (lane == 0) g_rescale[wave] = __ballot(st.over) != 0ull;
    __syncthreads();
    int redo = 0;
#pragma unroll
    for (int w = 0; w < kMlaWaves; ++w) redo |= g_rescale[w];
    if (redo) {
        st.m_ref = st.m_max;
        __syncthreads();  // every wave has read the flags
        pass(true);
    }

    // ---- epilogue: normalise, then write the final row or this split's partial
    if (wave < NHT && g == 0) {
        g_l[16 * wave + n] = st.l_run;
        g_m[16 * wave + n] = st.m_ref;
    }
    __syncthreads();      // every wave is past its last PV: the tile ring is free
    // Stage the normalised bf16 rows [head][512] in LDS (16-byte chunks XOR-swizzled by
    // head & 15 so the four head rows a store instruction touches use different banks),
    // then write them out as whole 1 KB head rows with 16-byte stores.
    uint16_t* stage = reinterpret_cast<uint16_t*>(g_kbuf);
#pragma unroll
    for (int h = 0; h < NHT; ++h) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int head = 16 * h + 4 * g + i;
            const float l = g_l[head];
            const float inv = l > 0.f ? recip(l) : 0.f;
#pragma unroll
            for (int dt = 0; dt < kDtW; ++dt) {
                const int d = 64 * wave + 16 * dt + n;
                const int pc = (d >> 3) ^ (head & 15);
                stage[head * kDv + pc * 8 + (d & 7)] = f32_to_bf16(st.o[h][dt][i] * inv);
            }
        }
    }
    __syncthreads();
    uint16_t* dst = n_splits == 1 ? out + (static_cast<size_t>(row) * H_total + head0) * kDv
                                  : part_o + ((static_cast<size_t>(row) * n_splits + split) * H_total + head0) * kDv;
    for (int c = threadIdx.x; c < H * (kDv / 8); c += kMlaThreads) {
        const int head = c / (kDv / 8);
        const int lc = c - head * (kDv / 8);
        const int pc = lc ^ (head & 15);
        *reinterpret_cast<uint4*>(dst + head * kDv + lc * 8) =
            *reinterpret_cast<const uint4*>(stage + head * kDv + pc * 8);
    }
    if (threadIdx.x < H) {
        const int head = threadIdx.x;
        const float l = g_l[head];
        const float lse2 = l > 0.f ? g_m[head] + log2f(l) : -INFINITY;
        if (n_splits == 1) {
            if (lse) lse[static_cast<size_t>(row) * H_total + head0 + head] = lse2 * kLn2;
        } else {
            part_lse[(static_cast<size_t>(row) * n_splits + split) * H_total + head0 + head] = lse2;
        }
    }
}

// Merge the splits of each (row, head): split s holds its own normalised output (bf16)
// and its log2-sum-exp; weights are 2^(lse_s - max).  One thread owns 8 columns.
constexpr int kCombCols = 8;
constexpr int kMaxSplits = 16;
__global__ __launch_bounds__(256)
void mla_combine_kernel(const uint16_t* __restrict__ part_o, const float* __restrict__ part_lse,
                        int rows, int H, int n_splits, uint16_t* __restrict__ out,
                        float* __restrict__ lse)
{
    // block = part * rows + row: a row's blocks share the XCD (block % 8) that ran its
    // splits, so the partials are read from that XCD's L2 when rows is a multiple of 8
    const size_t row = blockIdx.x % rows;
    const int gid = (blockIdx.x / rows) * blockDim.x + threadIdx.x;
    if (gid >= H * (kDv / kCombCols)) return;
    const int d8 = gid % (kDv / kCombCols);
    const int h = gid / (kDv / kCombCols);
    // every load goes out before the first wait (the split count is uniform, so the
    // guards do not diverge): one memory latency per thread instead of two
    float ls[kMaxSplits];
    uint4 v[kMaxSplits];
#pragma unroll
    for (int s = 0; s < kMaxSplits; ++s) {
        if (s < n_splits) {
            ls[s] = part_lse[(row * n_splits + s) * H + h];
            v[s] = *reinterpret_cast<const uint4*>(part_o + ((row * n_splits + s) * H + h) * kDv + kCombCols * d8);
        } else {
            ls[s] = -INFINITY;
            v[s] = uint4{0u, 0u, 0u, 0u};
        }
    }
    float M = -INFINITY;
#pragma unroll
    for (int s = 0; s < kMaxSplits; ++s) M = fmaxf(M, ls[s]);
    float W = 0.f;
    float acc[kCombCols] = {};
#pragma unroll
    for (int s = 0; s < kMaxSplits; ++s) {
        // a split with no usable slot (lse -inf) has weight 0 and a zero output
        const float wgt = ls[s] == -INFINITY ? 0.f : exp2f(ls[s] - M);
        W += wgt;
        const uint32_t wv[4] = {v[s].x, v[s].y, v[s].z, v[s].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            acc[2 * i] += wgt * bf16_to_f32(static_cast<uint16_t>(wv[i] & 0xffffu));
            acc[2 * i + 1] += wgt * bf16_to_f32(static_cast<uint16_t>(wv[i] >> 16));
        }
    }
    const float inv = W > 0.f ? recip(W) : 0.f;
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
        o[i] = f32_to_bf16(acc[2 * i] * inv) |
               (static_cast<uint32_t>(f32_to_bf16(acc[2 * i + 1] * inv)) << 16);
    *reinterpret_cast<uint4*>(out + (row * H + h) * kDv + kCombCols * d8) = uint4{o[0], o[1], o[2], o[3]};
    if (lse && d8 == 0) lse[row * H + h] = W > 0.f ? (M + log2f(W)) * kLn2 : -INFINITY;
}

int mla_splits(int rows, int k) {
    // enough (row, split) workgroups to give every CU one (a few rows of a long context
    // split up to 16 ways), within the LDS slot limit
    const int n_tiles = (k + kKt - 1) / kKt;
    int s = rows >= 256 ? 1 : (256 + rows - 1) / rows;
    s = min(s, kMaxSplits);
    const int min_s = (n_tiles * kKt + kMaxSlots - 1) / kMaxSlots;
    s = max(s, min_s);
    s = min(s, n_tiles);
    return max(s, 1);
}

}  // namespace

hipError_t launch_sparse_attn_generic(const SparseAttnArgs& a, hipStream_t stream) {
    const size_t shmem = sizeof(float) * (static_cast<size_t>(a.Dk) + a.k);
    return launch_kernel(kPhaseAttention, sparse_attn_generic_kernel, dim3(a.B * a.T * a.H),
                         dim3(kGenThreads), static_cast<uint32_t>(shmem), stream, a);
}

bool mla_decode_mfma_supported(int H, int Dv, int Dr, int k, int type) {
    // every split holds at most kMaxSlots selected positions in LDS
    return (type == kLatBf16 || type == kLatFp8) && Dv == kDv && Dv + Dr == kDq &&
           (H == 64 || H == 128) && k <= kMaxSplits * kMaxSlots;
}

// Launch shape of the matrix-core path.  128 heads go to two 64-head workgroups per
// (row, split) -- half the queries per workgroup, half the partial rows written, twice
// the workgroups for the same key splits -- when the key splits alone leave CUs idle
// (at most 16 splits: B = 8 decode ran 128 workgroups), and for bf16 rows when a row
// would need 8 or more splits (measured: decode B = 32 attention + combine 48.2 ->
// 45.8 us).  Otherwise not: at 64 rows (4 splits) and for FP8 rows, whose QK waves each
// widen the whole tile whatever their head count, the 64-head form measured slower.
struct MlaPlan {
    int nht;          // 16-head tiles per workgroup
    int parts;        // head parts per row
    int splits;       // key splits per row
    bool k32;         // the 32x32x16 kernel (sparse_mla_decode32.hip)
    bool k32f8;       // its FP8-row form (sparse_mla_decode32_fp8.hip)
    int tile_rows;    // slots per tile of the chosen kernel
};
MlaPlan mla_plan(int rows, int H, int k, int type) {
    MlaPlan p;
    p.k32 = false;
    p.k32f8 = false;
    p.tile_rows = kKt;
    if (type == kLatFp8 && (H == 64 || H == 128)) {
        // the 32x32x16 kernel over FP8 rows: 64-slot tiles, same split rule (one wave of at
        // most 256 workgroups, else the 16x16 kernel below)
        const int kt = mla_decode32_fp8_tile_rows();
        const int tmax = mla_decode32_fp8_max_tiles();
        const int n_tiles = (k + kt - 1) / kt;
        p.parts = H / 64;
        p.nht = 4;
        const int wg = rows * p.parts;
        int s = wg >= 256 ? 1 : (256 + wg - 1) / wg;
        s = min(s, kMaxSplits);
        s = max(s, (n_tiles + tmax - 1) / tmax);
        p.splits = max(1, min(s, n_tiles));
        if (static_cast<long long>(wg) * p.splits <= 256 && n_tiles <= tmax * kMaxSplits) {
            p.k32f8 = true;
            p.tile_rows = kt;
            return p;
        }
    }
    if (type == kLatBf16 && mla_decode32_supported(H, k)) {
        // the 32x32x16 kernel: 64 heads per workgroup, enough key splits to give every CU
        // a workgroup, at most mla_decode32_max_tiles() tiles per split -- when that fits
        // the 256 CUs in one wave of workgroups (decode batches up to 32 rows at k = 2048).
        // More rows run the 128-head kernel below, which gathers each selected row once
        // per (row, split) for all 128 heads (B = 64 decode: attention 72 us here against
        // 54 us; a 8192-row chunk: 7.4 ms against 4.9 ms).
        p.parts = H / 64;
        p.nht = 4;
        const int n_tiles = (k + kKt - 1) / kKt;
        const int wg = rows * p.parts;
        int s = wg >= 256 ? 1 : (256 + wg - 1) / wg;
        s = min(s, kMaxSplits);
        const int tmax = mla_decode32_max_tiles();
        s = max(s, (n_tiles + tmax - 1) / tmax);
        p.splits = max(1, min(s, n_tiles));
        if (static_cast<long long>(wg) * p.splits <= 256) {
            p.k32 = true;
            return p;
        }
    }
    const int s1 = mla_splits(rows, k);
    const bool idle = rows * s1 < 256;
    p.parts = (H == 128 && rows < 256 && (idle || (type == kLatBf16 && s1 >= 8))) ? 2 : 1;
    p.nht = H / 16 / p.parts;
    p.splits = p.parts == 1 ? s1 : mla_splits(rows * p.parts, k);
    return p;
}

size_t mla_decode_workspace_bytes(int B, int T, int H, int, int k, int type) {
    const int rows = B * T;
    const int s = mla_plan(rows, H, k, type).splits;
    if (s == 1) return 0;
    return static_cast<size_t>(rows) * s * H * (kDv * sizeof(uint16_t) + sizeof(float)) + 256;
}

hipError_t launch_mla_decode_mfma(const void* q, const void* latent, const int32_t* idx,
                                  const int32_t* len, int B, int T, int H, int Lmax, int k,
                                  float sm_scale, int type, int m, void* out, float* lse, void* ws,
                                  hipStream_t stream) {
    const int rows = B * T;
    const MlaPlan plan = mla_plan(rows, H, k, type);
    const int s = plan.splits;
    const int n_tiles = (k + plan.tile_rows - 1) / plan.tile_rows;
    const int tps = (n_tiles + s - 1) / s;
    uint16_t* part_o = static_cast<uint16_t*>(ws);
    float* part_lse = s > 1 ? reinterpret_cast<float*>(part_o + static_cast<size_t>(rows) * s * H * kDv)
                            : nullptr;
    const float scale_log2 = sm_scale * kLog2e;
    auto qp = static_cast<const uint16_t*>(q);
    auto lp = static_cast<const uint8_t*>(latent);
    auto op = static_cast<uint16_t*>(out);
    const bool f8 = type == kLatFp8;
    if (plan.k32 || plan.k32f8) {
        hipError_t e = plan.k32 ? launch_mla_decode32(q, latent, idx, len, rows, T, H, Lmax, k, m, tps, s,
                                                      scale_log2, out, lse, part_o, part_lse, stream)
                                : launch_mla_decode32_fp8(q, latent, idx, len, rows, T, H, Lmax, k, m, tps, s,
                                                          scale_log2, out, lse, part_o, part_lse, stream);
        if (e != hipSuccess || s == 1) return e;
        const int parts = (H * (kDv / kCombCols) + 255) / 256;
        return launch_kernel(kPhaseCombine, mla_combine_kernel, dim3(rows * parts), dim3(256), 0, stream,
                             part_o, part_lse, rows, H, s, op, lse);
    }
    auto kern = plan.nht == 8 ? (f8 ? mla_decode_mfma_kernel<8, true> : mla_decode_mfma_kernel<8, false>)
                              : (f8 ? mla_decode_mfma_kernel<4, true> : mla_decode_mfma_kernel<4, false>);
    hipError_t e = launch_kernel(kPhaseAttention, kern, dim3(rows * s * plan.parts), dim3(kMlaThreads), 0,
                                 stream, qp, lp, idx, len, T, Lmax, k, m, tps, s, H, scale_log2, op, lse,
                                 part_o, part_lse);
    if (e != hipSuccess || s == 1) return e;
    const int parts = (H * (kDv / kCombCols) + 255) / 256;
    return launch_kernel(kPhaseCombine, mla_combine_kernel, dim3(rows * parts), dim3(256), 0, stream,
                         part_o, part_lse, rows, H, s, op, lse);
}

}  // namespace dsa
