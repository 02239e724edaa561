// sparse_mla_decode32.hip -- absorbed (MQA) sparse attention over selected bf16 latent rows,
// on the gfx950 32x32x16 bf16 matrix-core form.
//
// The core-attention box of "dsa-indexer.excalidraw": all query heads share the selected
// latent rows, each row serving as key (all 576 columns: latent 512 then rope 64) and as
// value (the first 512 columns); the softmax and value mix follow the MLA prefill excerpt
// ("DeepSeek-V3.2-Exp - Causal mask", Multi-head latent attention).
//
// One workgroup (8 waves, two per SIMD) owns one query row (b,t), 64 of its heads and one
// split of its selected slots.  The roles of its waves are split so that both products run
// on the 32x32x16 form:
//   QK waves 0..3   wave w computes S = K . Q^T for head half hh = w & 1 (32 heads) over
//                   the column half dh = w >> 1 (288 of the 576 columns, 18 K-steps): its
//                   queries stay in registers (72 VGPRs).  The two column halves of a
//                   head half are summed through LDS: each wave sends the partner the
//                   16 keys the partner finishes (8 values per lane) and keeps its own;
//                   it forms the softmax numerators of its 16 keys one step later and
//                   publishes them in the P operand layout.  No wave holds output
//                   accumulators.
//   PV waves 4..7   wave 4 + c owns output columns 128 c .. 128 c + 127 of all 64 heads
//                   and accumulates O^T = V^T . P^T (output columns as MFMA rows, heads as
//                   MFMA columns: every lane ends with one head and runs of four adjacent
//                   columns, which go to LDS as 8-byte stores), V read by transpose reads
//                   straight from the gathered tile.
// Per tile of 32 selected rows the two waves of a SIMD issue 34 matrix-core instructions
// (18 QK + 16 PV).
//
// Pipeline: step i (two workgroup barriers) --
//   A(i)     tile i has landed for every wave.
//   phase 1  QK waves: QK(i), with the numerators of tile i-1 formed between its matrix-
//            core instructions and published as P(i-1); the partner's half of S(i) out.
//            PV waves: their share of the gathers of tile i+3, into tile i-1's buffer.
//   B(i)     P(i-1) and the halves of S(i) are published.
//   phase 2  QK waves: S(i) completed (the partner's half added); their share of the
//            gathers of tile i+3.
//            PV waves: PV(i-1) from P(i-1) and the V operands of tile i-1 held in
//            registers, then the V operands of tile i into the same registers.
// The softmax runs one tile behind QK so that its VALU work fills the matrix cores'
// issue gaps instead of a phase of its own, and the gathers of a tile are split between
// the two roles (5 and 4 of the 9 wave-wide loads per wave position) so that each role
// issues them while the other role's matrix-core chain runs.  Four buffers: tile i+3 goes
// into the buffer of tile i-1 while tiles i+1 and i+2 are in flight.  Step n_tiles forms
// the last tile's numerators and runs its PV.  The queries reach the QK waves through LDS
// (direct loads into buffers 2 and 3, read by each QK wave before A(0), so that the PV
// waves' share of tiles 2 and 3 goes out in phase 1 of step 0), so the compiler's own
// waits for register loads never drain the gathers.
// Softmax without a running rescale: each head's numerators are exp2(logit - m_ref), where
// m_ref is the largest logit of the split's first tile with a usable slot (posted by both
// column-half waves in phase 2 of that tile's step, read in the next step), so that tile's
// dominant key gets the numerator 1 exactly.  A key with a logit more than 2^64 above the
// reference (log2 units) marks the split, which is then recomputed with the split's
// maximum as reference; the normalised result is the same softmax.
#include "dsa_device.h"
#include "dsa_internal.h"

namespace dsa {

namespace {

constexpr int kThreads = 512;
constexpr int kWaves = 8;
constexpr int kHeads = 64;                          // heads per workgroup
constexpr int kDq = 576;
constexpr int kDv = 512;
constexpr int kRowBytes = kDq * 2;                  // 1152
constexpr int kRowChunks = kRowBytes / 16;          // 72
constexpr int kKt = 32;                             // selected rows per tile
constexpr int kTileBytes = kKt * kRowBytes;         // 36864
constexpr int kTileLoads = kTileBytes / (kWave * 16);   // 36 wave-wide 1 KB loads
constexpr int kGatherWaves = 4;                    // wave positions sharing a tile's loads
constexpr int kGatherLoads = kTileLoads / kGatherWaves;          // 9 per wave position and tile
constexpr int kPvLoads = 5;                         // of them issued by the PV wave (phase 1)
constexpr int kQkLoads = kGatherLoads - kPvLoads;   // and by the QK wave (phase 2)
constexpr int kBufs = 4;                            // tile ring
constexpr int kMaxTiles = 16;                       // tiles per split
constexpr int kMaxSlots = kMaxTiles * kKt;          // 512 slots per split
constexpr int kKs = kDq / 2 / 16;                   // 18 K-steps per column half
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRefSpan = 64.0f;                   // log2 units above the reference

// LDS: 147,456 (tiles) + 8,192 (S halves) + 512 (reference partials) + 4,096 (P) +
// 2,048 (slots) + small.
__shared__ __attribute__((aligned(16))) uint8_t s_tile[kBufs * kTileBytes];
__shared__ __attribute__((aligned(16))) float s_half[2][2][2][kWave][4];   // [hh][owner dh][j][lane][4]
__shared__ float s_ref[2][2][32];                   // [hh][dh][head]: reference exchange
__shared__ __attribute__((aligned(16))) uint8_t s_p[2][2][kWave][16];      // [hh][kk][lane][8 bf16]
__shared__ int32_t s_keys[kMaxSlots];
__shared__ uint32_t s_tmask[kMaxTiles];             // usable slots of each tile (bit = row)
__shared__ float s_l[2][2][32];                     // [hh][dh][head] numerator sums
__shared__ float s_m[2][2][32];                     // [hh][dh][head] reference / split maximum
__shared__ int32_t s_redo[kWaves];

template <int N> struct IntConst { static constexpr int value = N; };

__device__ __forceinline__ uint8_t* tile_buf(int ti) { return s_tile + (ti & (kBufs - 1)) * kTileBytes; }

template <int N>
__device__ __forceinline__ void wait_vmcnt() { asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory"); }

// Workgroup barrier for LDS data: waits for this wave's LDS operations only, so the tile
// gathers in flight stay in flight across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Waits for this wave's gathers of the tile used at step t (loads complete in issue
// order).  The PV waves issue all of tiles 0 and 1 (kGatherLoads each) and kPvLoads of
// every later tile; the QK waves issue the other kQkLoads of tiles 2 onwards.  Tiles in
// flight behind tile t: t + 1 and t + 2, except at step 0 (tile 1 only: tiles 2 and 3 go
// out after B(0)).
__device__ __forceinline__ void wait_tile_pv(int t, int n_tiles) {
    if (t >= n_tiles) return;
    if (t == 0) {
        if (n_tiles > 1) wait_vmcnt<kGatherLoads>();
        else wait_vmcnt<0>();
        return;
    }
    const int later = min(2, n_tiles - 1 - t);
    if (later == 2) wait_vmcnt<2 * kPvLoads>();
    else if (later == 1) wait_vmcnt<kPvLoads>();
    else wait_vmcnt<0>();
}
__device__ __forceinline__ void wait_tile_qk(int t, int n_tiles) {
    if (t < 2 || t >= n_tiles) return;
    const int later = min(2, n_tiles - 1 - t);
    if (later == 2) wait_vmcnt<2 * kQkLoads>();
    else if (later == 1) wait_vmcnt<kQkLoads>();
    else wait_vmcnt<0>();
}

// LDS layout of a tile: row r (1152 bytes = 72 chunks of 16 bytes) keeps its chunk c at
// chunk position c ^ swz(r), swz(r) = 4 ((r >> 1) & 1) + ((r >> 2) & 3), a bijection of
// (r >> 1) & 7.  Rows are 288 dwords apart, which is 32 banks, so rows of one parity share
// a half of the 64 banks; within it the XOR gives the 8 rows of each parity among any 16
// consecutive rows distinct 4-bank groups, so 16-lane reads of one chunk over 16
// consecutive rows (the QK operands) are free of bank conflicts.  The V transpose reads
// take, per 32-lane pass, one aligned group of 4 chunks from 4 consecutive rows 4 i ..
// 4 i + 3: bit 2 of swz, ((r >> 1) & 1), puts rows 4 i and 4 i + 2 (and 4 i + 1, 4 i + 3) in
// different bank quarters, so those reads are conflict-free as well.  (The XOR stays
// inside each aligned group of 8 chunks, so the rope chunks 64..71 stay in place.)
__device__ __forceinline__ int swz(int r) { return (((r >> 1) & 1) << 2) | ((r >> 2) & 3); }

// Direct global->LDS loads of a tile: 36 wave-wide 1 KB loads ci = c + 4 i (wave position
// c = 0..3, i = 0..8); lane l of load ci fetches 16-byte chunk q = 64 ci + l of the tile,
// i.e. chunk q % 72 of selected row q / 72, stored at its swizzled position.  PV wave c
// issues loads i < kPvLoads of position c in phase 1 (all nine for tiles 0 and 1), QK wave
// w the loads i >= kPvLoads of position w in phase 2, so each role's issue time overlaps
// the other role's matrix-core work.  Written as inline assembly so that the compiler,
// which cannot tell the ring's buffers apart, inserts no drain of these loads before later
// LDS reads; completion is tracked with wait_tile_*() and published by lds_barrier().  M0
// holds the wave-uniform LDS destination; nothing else in this kernel uses M0.  Unused
// slots fetch row 0 (masked).
template <int I0, int N>
struct GatherLane {
    int key[N];         // tile row of load I0 + i for this lane
    uint32_t off[N];    // byte offset of the lane's source chunk within that row
};
template <int I0, int N>
__device__ __forceinline__ GatherLane<I0, N> gather_lane(int c, int lane) {
    GatherLane<I0, N> gl;
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const int q = (c + kGatherWaves * (I0 + i)) * kWave + lane;
        const int key = q / kRowChunks;
        gl.key[i] = key;
        gl.off[i] = static_cast<uint32_t>(((q - key * kRowChunks) ^ swz(key)) * 16);
    }
    return gl;
}
// Loads I0 + J0 .. I0 + J0 + M - 1 of position c for tile ti.
template <int J0, int M, int I0, int N>
__device__ __forceinline__ void gather_tile(const uint8_t* lat_b, int ti, int c, const GatherLane<I0, N>& gl) {
    static_assert(J0 + M <= N, "loads outside the lane's part");
    const uint32_t lds_base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
        (__attribute__((address_space(3))) uint8_t*)(tile_buf(ti))));
    int s[M];
#pragma unroll
    for (int i = 0; i < M; ++i) s[i] = s_keys[ti * kKt + gl.key[J0 + i]];
#pragma unroll
    for (int i = 0; i < M; ++i) {
        const int ci = c + kGatherWaves * (I0 + J0 + i);
        const int row = max(s[i], 0);
        const uint8_t* src = lat_b + static_cast<size_t>(row) * kRowBytes + gl.off[J0 + i];
        const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds_base + ci * kWave * 16);
        asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
                     :: "s"(m0v), "v"(src) : "memory");
    }
}

typedef __bf16 v4bf_t __attribute__((ext_vector_type(4)));

// ---- QK waves

struct QkState {
    float m_ref;     // reference logit of this lane's head (log2 units), -inf until set
    float m_max;     // largest logit seen
    float l_run;     // sum of this lane's numerators
    bool over;       // a logit above m_ref + kRefSpan
};

// Phase 1 of a QK wave: the S partial of tile ti over column half DH for 32 heads, with the
// softmax numerators of the tile completed in the previous step formed between its
// matrix-core instructions and published as the P operand.
//   S: lane l supplies key l % 32 of the tile as A operand (columns 288 DH + 16 ks +
//   8 (l / 32) .. + 7 of its row) and holds the matching query columns of head l % 32 as B
//   operand; element r of the result is S[key 8 (r / 4) + 4 (l / 32) + r % 4][head l % 32].
//   The operand reads run nine K-steps ahead of the matrix cores (LDS latency), and the
//   order -- one instruction, the read nine steps ahead, one piece of the softmax -- is
//   pinned, so no instruction waits for a read issued just before it.
//   Numerators: exp2(logit - m_ref) as bf16.  Before any usable key every logit is -inf
//   and the numerators are 0 whatever the reference.
template <int DH>
__device__ __forceinline__ v16f qk_tile(const v8bf (&qreg)[kKs], const uint8_t* kb, int lane,
                                        const float (&v)[8], float mx, QkState& st, int hh, bool fixed) {
    int lo = lane;
    asm volatile("" : "+v"(lo));
    const int r = lo & 31;
    const int g = lo >> 5;
    const int x = swz(r);
    const uint8_t* row = kb + r * kRowBytes;
    // chunk 36 DH + 2 ks + g = 8 a + b sits at 16 (8 a + (b ^ x)); b = (C0 & 7) + g with
    // C0 = 36 DH + 2 ks even, so four per-lane offsets cover every K-step
    int off[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) off[e] = 16 * ((2 * e + g) ^ x);
    auto addr = [&](int ks) -> const v8bf* {
        const int c0 = 36 * DH + 2 * ks;
        return reinterpret_cast<const v8bf*>(row + 128 * (c0 >> 3) + off[(c0 & 7) >> 1]);
    };
    st.over = st.over || (!fixed && mx > st.m_ref + kRefSpan);
    const float mref = st.m_ref == -INFINITY ? 0.f : st.m_ref;
    v16f acc;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.f;
    constexpr int kPre = 9;               // K-steps of operand reads in flight (LDS latency)
    v8bf a[kPre];
#pragma unroll
    for (int ks = 0; ks < kPre; ++ks) a[ks] = *addr(ks);
    __builtin_amdgcn_sched_barrier(0);
    float p[8];
    float psum = 0.f;
#pragma unroll
    for (int ks = 0; ks < kKs; ++ks) {
        acc = mfma_bf16_32x32x16(a[ks % kPre], qreg[ks], acc);
        if (ks + kPre < kKs) a[ks % kPre] = *addr(ks + kPre);
        if (ks < 8) {
            p[ks] = exp2_num(v[ks] - mref);
            psum += p[ks];
        } else if (ks == 8) {
            v8s pk;
#pragma unroll
            for (int e = 0; e < 8; ++e) pk[e] = static_cast<short>(f32_to_bf16(p[e]));
            *reinterpret_cast<v8s*>(&s_p[hh][DH][lane][0]) = pk;
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    st.l_run += psum;
    return acc;
}

// Phase-1 tail: the partner's half of S (its 16 keys) to LDS.
template <int DH>
__device__ __forceinline__ void qk_send(const v16f& acc, int hh, int lane) {
    constexpr int kOther = 1 - DH;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        float4 v;
        v.x = acc[8 * kOther + 4 * j + 0];
        v.y = acc[8 * kOther + 4 * j + 1];
        v.z = acc[8 * kOther + 4 * j + 2];
        v.w = acc[8 * kOther + 4 * j + 3];
        *reinterpret_cast<float4*>(&s_half[hh][kOther][j][lane][0]) = v;
    }
}

// Phase 2: this wave's 16 keys of S complete (the partner's half added), in log2 units,
// -inf at unusable slots; returns the lane's maximum.  The lane holds keys
// 16 DH + 8 (s / 4) + 4 (l / 32) + s % 4, s = 0..7, of head l % 32 -- exactly K-slot s of
// the P operand for K-step DH of the PV product.
template <int DH>
__device__ __forceinline__ float qk_complete(const v16f& acc, int hh, int lane, uint32_t tmask,
                                             float scale_log2, float (&v)[8]) {
    const int g = lane >> 5;
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const float4 h = *reinterpret_cast<const float4*>(&s_half[hh][DH][j][lane][0]);
        const float hv[4] = {h.x, h.y, h.z, h.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int s = 4 * j + e;
            const int key = 16 * DH + 8 * j + 4 * g + e;
            const bool ok = (tmask >> key) & 1u;
            v[s] = ok ? (acc[8 * DH + s] + hv[e]) * scale_log2 : -INFINITY;
            mx = fmaxf(mx, v[s]);
        }
    }
    return mx;
}

// The numerators alone (the step after the last tile).
template <int DH>
__device__ __forceinline__ void qk_numerators(const float (&v)[8], float mx, QkState& st, int hh,
                                              int lane, bool fixed) {
    st.over = st.over || (!fixed && mx > st.m_ref + kRefSpan);
    const float mref = st.m_ref == -INFINITY ? 0.f : st.m_ref;
    float psum = 0.f;
    v8s pk;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
        const float p = exp2_num(v[s] - mref);
        psum += p;
        pk[s] = static_cast<short>(f32_to_bf16(p));
    }
    st.l_run += psum;
    *reinterpret_cast<v8s*>(&s_p[hh][DH][lane][0]) = pk;
}

// Query operands of QK wave (hh, dh) through LDS: 18 wave-wide direct loads of 1 KB into
// ring buffers 2 and 3 (wave w's at 18 KB * w), lane l of load ks fetching head
// 32 hh + l % 32, columns 288 dh + 16 ks + 8 (l / 32) .. + 7 -- the B-operand layout, so
// each lane later reads back its own 16 bytes.
__device__ __forceinline__ uint8_t* q_stage(int wave) { return s_tile + 2 * kTileBytes + wave * kKs * 1024; }
__device__ __forceinline__ void load_q(const uint16_t* qrow, int wave) {
    const uint32_t lds_base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
        (__attribute__((address_space(3))) uint8_t*)(q_stage(wave))));
#pragma unroll
    for (int ks = 0; ks < kKs; ++ks) {
        const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds_base + ks * 1024);
        asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
                     :: "s"(m0v), "v"(qrow + 16 * ks) : "memory");
    }
}

// ---- PV waves

// Output columns 128 c + 32 ct + ..., ct = 0..3, of all 64 heads, as O^T tiles:
// acc[hh][ct] element r of lane l is O[head 32 hh + l % 32][column 128 c + 32 ct +
// 8 (r / 4) + 4 (l / 32) + r % 4].
struct PvState {
    v16f acc[2][4];
};

// The A operand (V^T: output columns x keys) for K-step kk and column tile ct: lane l
// supplies column l % 32 of the tile and keys 16 kk + 8 q + 4 (l / 32) + e, e = 0..3,
// q = 0 (slots 0..3) and 1 (slots 4..7) -- the key order of the P operand.  Two 8-byte
// transpose reads per lane: inside a 16-lane group (lanes 16 G .. 16 G + 15, G = l / 16,
// K-slice g = G / 2, columns 16 (G % 2) + n), lane n receives element e from the address
// of lane 4 e + n / 4 plus n % 4, so lane m = 4 e + j points at row key0 + e, columns
// 4 j .. 4 j + 3 of the group's 16.
struct VAddr {
    int base;      // byte offset of (row 4 g + e, column group) for this lane, minus swizzle
    int t[2][2];   // swizzled 16-byte chunk offsets [key half q][ct & 1]
};
__device__ __forceinline__ VAddr v_addr(int c, int lane) {
    int lo = lane;
    asm volatile("" : "+v"(lo));
    const int G = lo >> 4;
    const int n = lo & 15;
    const int e = n >> 2;
    const int j = n & 3;
    const int g = G >> 1;
    const int low = 2 * (G & 1) + (j >> 1);   // column chunk bits below the tile's 4 ct
    VAddr va;
    va.base = (4 * g + e) * kRowBytes + 8 * (j & 1) + 16 * 16 * c;
#pragma unroll
    for (int qh = 0; qh < 2; ++qh) {
        // the lane's keys 16 kk + 8 qh + 4 g + e share swz (it depends on bits 1..3 of the row)
        const int x = swz(8 * qh + 4 * g + e);
        va.t[qh][0] = 16 * ((0 + low) ^ x);
        va.t[qh][1] = 16 * ((4 + low) ^ x);
    }
    return va;
}

__device__ __forceinline__ v8bf v_operand(const uint8_t* kb, const VAddr& va, int kk, int ct) {
    const uint8_t* p = kb + va.base + 16 * 8 * (ct >> 1) + 16 * kk * kRowBytes;
    const v4bf_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (__attribute__((address_space(3))) v4bf_t*)(p + va.t[0][ct & 1]));
    const v4bf_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (__attribute__((address_space(3))) v4bf_t*)(p + 8 * kRowBytes + va.t[1][ct & 1]));
    return v8bf{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// The V operands of one tile for this wave's four column tiles and both K-steps.
__device__ __forceinline__ void load_v(v8bf (&vop)[2][4], const uint8_t* kb, const VAddr& va) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) vop[kk][ct] = v_operand(kb, va, kk, ct);
}

// PV of one tile: 16 instructions (2 K-steps x 2 head halves x 4 column tiles).
__device__ __forceinline__ void pv_tile(PvState& st, const v8bf (&vop)[2][4], const v8bf (&pop)[2][2]) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int ct = 0; ct < 4; ++ct)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
                st.acc[hh][ct] = mfma_bf16_32x32x16(vop[kk][ct], pop[kk][hh], st.acc[hh][ct]);
}

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void mla_decode32_kernel(const uint16_t* __restrict__ q, const uint8_t* __restrict__ latent,
                         const int32_t* __restrict__ idx, const int32_t* __restrict__ len,
                         int T, int Lmax, int k, int m, int tiles_per_split, int n_splits,
                         int H_total, float scale_log2, uint16_t* __restrict__ out,
                         float* __restrict__ lse, uint16_t* __restrict__ part_o,
                         float* __restrict__ part_lse)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const bool qk_wave = wave < 4;
    const int hh = wave & 1;                  // QK waves: head half
    const int dh = (wave >> 1) & 1;           // QK waves: column half
    if (qk_wave) __builtin_amdgcn_s_setprio(1);

    // Workgroup (row, split, head part), block (part * n_splits + split) * rows + row: the
    // workgroups of a row share an XCD when rows is a multiple of 8 (round-robin dispatch
    // over the 8 XCDs), so the row's queries and gathered rows meet in one L2.
    const int parts = H_total / kHeads;
    const int rows = gridDim.x / (n_splits * parts);
    const int row = blockIdx.x % rows;
    const int rest = blockIdx.x / rows;
    const int split = rest % n_splits;
    const int head0 = (rest / n_splits) * kHeads;
    const int b = row / T;
    const int t = row - b * T;

    const int n_tiles_total = (k + kKt - 1) / kKt;
    const int tile0 = split * tiles_per_split;
    const int n_tiles = max(0, min(tiles_per_split, n_tiles_total - tile0));
    const int nslots = n_tiles * kKt;

    // start-up loads: this split's selected positions and the sequence length; the
    // positions are checked against pos once both are in
    const int32_t* sel = idx + static_cast<size_t>(row) * k;
    const int j0 = threadIdx.x;               // kMaxSlots == kThreads
    const int slot0 = tile0 * kKt + j0;
    const int sraw = (j0 < nslots && slot0 < k) ? sel[slot0] : -1;
    const int seq_len = len[b];
    const uint8_t* lat_b = latent + static_cast<size_t>(b) * Lmax * kRowBytes;

    {
        const int pos = n_visible(seq_len, T, t, Lmax, m) - 1;     // last visible cache row
        const int sv = (sraw >= 0 && sraw <= pos) ? sraw : -1;
        if (j0 < nslots) s_keys[j0] = sv;
        // usable-slot mask of each tile: wave w covers tiles 2 w and 2 w + 1
        const unsigned long long bal = __ballot(sv >= 0 && j0 < nslots);
        if (lane == 0) {
            s_tmask[2 * wave] = static_cast<uint32_t>(bal);
            s_tmask[2 * wave + 1] = static_cast<uint32_t>(bal >> 32);
        }
        lds_barrier();        // s_keys, s_tmask ready
    }
    auto redo_flags = [&](bool over) {
        if (lane == 0) s_redo[wave] = __ballot(over) != 0ull;
    };
    auto any_redo = [&]() {
        int redo = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) redo |= s_redo[w];
        return redo != 0;
    };
    // The softmax reference comes from the first tile with a usable slot (uniform).
    int ref_tile = -1;
    for (int i = n_tiles - 1; i >= 0; --i)
        if (s_tmask[i] != 0u) ref_tile = i;

    // The two roles run separate code with the same barrier sequence (the slot barrier,
    // A and B per step for n_tiles + 1 steps, the recompute decision, an optional second
    // pass, the staging barrier), so their registers -- queries and S for the QK waves,
    // output accumulators and V operands for the PV waves -- are never live at the same
    // time.  The PV waves issue and wait for every tile's gathers; the QK waves see the
    // tiles through barrier A.
    if (qk_wave) {
        v8bf qreg[kKs];
        const uint16_t* qrow = q + (static_cast<size_t>(row) * H_total + head0 + 32 * hh + (lane & 31)) * kDq +
                               288 * dh + 8 * (lane >> 5);
        const GatherLane<kPvLoads, kQkLoads> glq = gather_lane<kPvLoads, kQkLoads>(wave, lane);
        QkState qs;
        qs.m_ref = -INFINITY;
        qs.m_max = -INFINITY;
        qs.over = false;
        // Step ti: A(ti); QK(ti) with the numerators of tile ti-1 formed between its
        // matrix-core instructions, the partner's half of S(ti) out; B(ti); S(ti) completed.
        // Step n_tiles forms the last tile's numerators only.
        auto qk_pass = [&](auto dhc, bool fixed) {
            constexpr int DH = decltype(dhc)::value;
            bool ref_known = fixed;
            qs.l_run = 0.f;
            if (!fixed) load_q(qrow, wave);
            float v[8];                                               // S of the completed tile
#pragma unroll
            for (int s = 0; s < 8; ++s) v[s] = -INFINITY;
            float vmx = -INFINITY;
            for (int ti = 0; ti <= n_tiles; ++ti) {
                if (ti == 0) wait_vmcnt<0>();                         // this wave's queries
                else wait_tile_qk(ti, n_tiles);
                if (ti == 0 && !fixed) {
                    // this wave's queries, landed by its own loads (no barrier needed); read
                    // before A(0), so that A(0) frees buffers 2 and 3 for tiles 2 and 3
                    const uint8_t* qs_lds = q_stage(wave) + 16 * lane;
#pragma unroll
                    for (int ks = 0; ks < kKs; ++ks) qreg[ks] = *reinterpret_cast<const v8bf*>(qs_lds + ks * 1024);
                }
                lds_barrier();                                        // A(ti): LDS reads done first
                if (!ref_known && ref_tile >= 0 && ti == ref_tile + 1) {
                    qs.m_ref = fmaxf(s_ref[hh][0][lane & 31], s_ref[hh][1][lane & 31]);
                    ref_known = true;
                }
                if (ti < n_tiles) {
                    const v16f sacc = qk_tile<DH>(qreg, tile_buf(ti), lane, v, vmx, qs, hh, fixed);
                    qk_send<DH>(sacc, hh, lane);
                    lds_barrier();                                    // B(ti)
                    vmx = qk_complete<DH>(sacc, hh, lane, s_tmask[ti], scale_log2, v);
                    qs.m_max = fmaxf(qs.m_max, vmx);
                    if (!ref_known && ti == ref_tile) {
                        // the reference: the largest logit of this tile, over both halves
                        const float m2 = max_xor32(vmx);
                        if (lane < 32) s_ref[hh][DH][lane] = m2;
                    }
                    // this wave's share of a later tile, into a buffer released at A(ti)
                    if (ti == 0) {
                        for (int tj = 2; tj <= 3; ++tj)
                            if (tj < n_tiles) gather_tile<0, kQkLoads>(lat_b, tj, wave, glq);
                    } else if (ti + 3 < n_tiles) {
                        gather_tile<0, kQkLoads>(lat_b, ti + 3, wave, glq);
                    }
                } else {
                    qk_numerators<DH>(v, vmx, qs, hh, lane, fixed);
                    lds_barrier();                                    // B(ti)
                }
            }
        };
        if (dh == 0) qk_pass(IntConst<0>{}, false);
        else qk_pass(IntConst<1>{}, false);
        // a head past its reference span: redo the split with the split's maximum as the
        // reference (a uniform decision: every wave reads the same flags)
        redo_flags(qs.over);
        {
            const float mm = fmaxf(qs.m_max, from_xor32(qs.m_max, lane));
            if (lane < 32) s_m[hh][dh][lane] = mm;
        }
        __syncthreads();
        if (any_redo()) {
            qs.m_ref = fmaxf(s_m[hh][0][lane & 31], s_m[hh][1][lane & 31]);
            __syncthreads();      // every wave has read the flags and maxima
            if (dh == 0) qk_pass(IntConst<0>{}, true);
            else qk_pass(IntConst<1>{}, true);
        }
        // numerator sums and references per head for the normalisation and the lse
        const float l = qs.l_run + from_xor32(qs.l_run, lane);
        if (lane < 32) {
            s_l[hh][dh][lane] = l;
            if (dh == 0) s_m[hh][0][lane] = qs.m_ref;
        }
        __syncthreads();          // every wave is past its last PV: the tile ring is free
    } else {
        PvState pv;
        const int c = wave - 4;
        // Step ti: A(ti) (own loads of tile ti landed); the gathers of tile ti+3 into the
        // buffer of tile ti-1; B(ti); PV(ti-1) from the V operands held since step ti-1 and
        // P(ti-1), published at B(ti); then the V operands of tile ti into the same registers.
        auto pv_pass = [&](bool fixed) {
            const VAddr va = v_addr(c, lane);
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
                for (int ct = 0; ct < 4; ++ct)
#pragma unroll
                    for (int i = 0; i < 16; ++i) pv.acc[h2][ct][i] = 0.f;
            const GatherLane<0, kGatherLoads> gl = gather_lane<0, kGatherLoads>(c, lane);
            if (n_tiles > 0) gather_tile<0, kGatherLoads>(lat_b, 0, c, gl);
            if (n_tiles > 1) gather_tile<0, kGatherLoads>(lat_b, 1, c, gl);
            v8bf vop[2][4];                                           // V operands of the previous tile
            for (int ti = 0; ti <= n_tiles; ++ti) {
                wait_tile_pv(ti, n_tiles);
                lds_barrier();                                        // A(ti)
                if (ti >= 1 && ti + 3 < n_tiles) gather_tile<0, kPvLoads>(lat_b, ti + 3, c, gl);
                if (ti == 0) {
                    // buffers 2 and 3 held the queries until the QK waves' reads, done before A(0)
                    for (int tj = 2; tj <= 3; ++tj)
                        if (tj < n_tiles) gather_tile<0, kPvLoads>(lat_b, tj, c, gl);
                }
                lds_barrier();                                        // B(ti)
                if (ti > 0) {
                    v8bf pop[2][2];                                   // P(ti - 1) operands [kk][hh]
#pragma unroll
                    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                        for (int h2 = 0; h2 < 2; ++h2)
                            pop[kk][h2] = *reinterpret_cast<const v8bf*>(&s_p[h2][kk][lane][0]);
                    pv_tile(pv, vop, pop);
                }
                if (ti < n_tiles) load_v(vop, tile_buf(ti), va);
            }
        };
        pv_pass(false);
        redo_flags(false);
        __syncthreads();
        if (any_redo()) {
            __syncthreads();
            pv_pass(true);
        }
        __syncthreads();          // the sums are published; the tile ring is free
        // normalised bf16 rows staged in LDS as [64 heads][512] with the 16-byte chunk
        // index XOR-swizzled by the head, from 8-byte runs of four columns per lane
        uint16_t* stage = reinterpret_cast<uint16_t*>(s_tile);
        const int g = lane >> 5;
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
            const int head = 32 * h2 + (lane & 31);
            const float l = s_l[h2][0][lane & 31] + s_l[h2][1][lane & 31];
            const float inv = l > 0.f ? recip(l) : 0.f;
#pragma unroll
            for (int ct = 0; ct < 4; ++ct)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    // columns 128 c + 32 ct + 8 jj + 4 g .. + 3: 16-byte chunk 16 c + 4 ct + jj
                    const int pc = (16 * c + 4 * ct + jj) ^ (head & 63);
                    uint2 w2;
                    w2.x = static_cast<uint32_t>(f32_to_bf16(pv.acc[h2][ct][4 * jj + 0] * inv)) |
                           (static_cast<uint32_t>(f32_to_bf16(pv.acc[h2][ct][4 * jj + 1] * inv)) << 16);
                    w2.y = static_cast<uint32_t>(f32_to_bf16(pv.acc[h2][ct][4 * jj + 2] * inv)) |
                           (static_cast<uint32_t>(f32_to_bf16(pv.acc[h2][ct][4 * jj + 3] * inv)) << 16);
                    *reinterpret_cast<uint2*>(stage + head * kDv + pc * 8 + 4 * g) = w2;
                }
        }
    }
    __syncthreads();
    const uint16_t* stage = reinterpret_cast<const uint16_t*>(s_tile);
    uint16_t* dst = n_splits == 1 ? out + (static_cast<size_t>(row) * H_total + head0) * kDv
                                  : part_o + ((static_cast<size_t>(row) * n_splits + split) * H_total + head0) * kDv;
#pragma unroll
    for (int it = 0; it < kHeads * (kDv / 8) / kThreads; ++it) {
        const int cidx = threadIdx.x + it * kThreads;
        const int head = cidx / (kDv / 8);
        const int lc = cidx - head * (kDv / 8);
        const int pc = lc ^ (head & 63);
        *reinterpret_cast<uint4*>(dst + head * kDv + lc * 8) =
            *reinterpret_cast<const uint4*>(stage + head * kDv + pc * 8);
    }
    if (threadIdx.x < kHeads) {
        const int head = threadIdx.x;
        const int h2 = head >> 5;
        const float l = s_l[h2][0][head & 31] + s_l[h2][1][head & 31];
        const float lse2 = l > 0.f ? s_m[h2][0][head & 31] + log2f(l) : -INFINITY;
        if (n_splits == 1) {
            if (lse) lse[static_cast<size_t>(row) * H_total + head0 + head] = lse2 * kLn2;
        } else {
            part_lse[(static_cast<size_t>(row) * n_splits + split) * H_total + head0 + head] = lse2;
        }
    }
}

}  // namespace

bool mla_decode32_supported(int H, int k) {
    return (H == 64 || H == 128) && k <= 16 * kMaxSlots;
}

int mla_decode32_max_tiles() { return kMaxTiles; }

hipError_t launch_mla_decode32(const void* q, const void* latent, const int32_t* idx,
                               const int32_t* len, int rows, int T, int H, int Lmax, int k, int m,
                               int tiles_per_split, int n_splits, float scale_log2, void* out,
                               float* lse, void* part_o, float* part_lse, hipStream_t stream) {
    const int parts = H / kHeads;
    return launch_kernel(kPhaseAttention, mla_decode32_kernel, dim3(rows * n_splits * parts), dim3(kThreads),
                         0, stream, static_cast<const uint16_t*>(q), static_cast<const uint8_t*>(latent),
                         idx, len, T, Lmax, k, m, tiles_per_split, n_splits, H, scale_log2,
                         static_cast<uint16_t*>(out), lse, static_cast<uint16_t*>(part_o), part_lse);
}

}  // namespace dsa
