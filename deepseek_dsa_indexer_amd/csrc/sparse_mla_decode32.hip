// sparse_mla_decode32.hip -- absorbed (MQA) sparse attention over selected bf16 latent rows,
// on the gfx950 32x32x16 bf16 matrix-core form.
//
// The core-attention box of "dsa-indexer.excalidraw": all query heads share the selected
// latent rows, each row serving as key (all 576 columns: latent 512 then rope 64) and as
// value (the first 512 columns); the softmax and value mix follow the MLA prefill excerpt
// ("DeepSeek-V3.2-Exp - Causal mask", Multi-head latent attention).
//
// One workgroup (8 waves, two per SIMD) owns one query row (b,t), 64 of its heads and one
// split of its selected slots, as the 16x16 kernel of sparse_attn.hip, with the roles
// of its waves changed so that both products run on the 32x32x16 form (twice the work of
// 16x16x32 per instruction at about the same issue time):
//   QK waves 0..3   wave w computes S = K . Q^T for head half hh = w & 1 (32 heads) over
//                   the column half dh = w >> 1 (288 of the 576 columns, 18 K-steps): its
//                   queries stay in registers (72 VGPRs).  The two column halves of a
//                   head half are summed through LDS: each wave sends the partner the
//                   16 keys the partner finishes (8 values per lane) and keeps its own;
//                   it then forms the softmax numerators of its 16 keys and publishes
//                   them in the P operand layout.  No wave holds output accumulators.
//   PV waves 4..7   wave 4 + c owns output columns 128 c .. 128 c + 127 of all 64 heads
//                   and accumulates O^T = V^T . P^T (output columns as MFMA rows, heads as
//                   MFMA columns: every lane ends with one head and runs of four adjacent
//                   columns, which go to LDS as 8-byte stores), V read by transpose reads
//                   straight from the gathered tile.
// Per tile of 32 selected rows the four waves of a SIMD issue 34 matrix-core instructions
// (18 QK + 16 PV) against 68 of the 16x16x32 form.
//
// Pipeline.  A tile's buffer is released in its own step -- the QK waves read K in phase
// 1 and the PV waves copy their V operands into registers in the same phase -- so while
// tile i is in use, tiles i+1 and i+2 are in flight and tile i+3 goes out after step i's
// second barrier.  (A further tile in flight, which the ring would allow, measured no
// faster per step and slower overall.)  The PV waves issue all gathers, in phase 2, while
// the QK waves form the softmax numerators; issued between their PV instructions instead,
// the loads held back the matrix-core issue and the PV phase grew from 0.5 to 1.25 us.  The queries reach the QK waves through LDS (direct loads
// into buffers 2 and 3 before those tiles are issued), so the compiler's own waits for
// register loads never drain the gathers.
// Step i (two workgroup barriers):
//   A(i)     tile i has landed for every wave; P(i-1) is published.
//   phase 1  QK waves: QK(i), then the partner's half of S(i) to LDS.
//            PV waves: P(i-1) operands from LDS, PV(i-1) from the V operands held in
//            registers since step i-1, then the V operands of tile i into registers.
//   B(i)     tile i's buffer is free.
//   phase 2  QK waves: add the partner's half, softmax numerators, publish P(i).
//            PV waves: issue tile i+3 (at step 0: tiles 2 and 3).
// Softmax without a running rescale: each head's numerators are exp2(logit - m_ref), where
// m_ref is the largest logit of the split's first tile, so the tile's dominant key gets the
// numerator 1 exactly: at step 0 both waves of a head half post the maximum of their 16
// keys and read the partner's after one extra barrier.  A split whose first tile holds no
// usable slot takes instead the logit of the first usable key of its first usable tile
// (both column halves of that key's logit travel with S).  A key with a logit more than
// 2^64 above the reference (log2 units) marks the split, which is then recomputed with the
// split's maximum as reference; the normalised result is the same softmax.
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
constexpr int kGatherWaves = 4;                    // the PV waves issue every tile's loads
constexpr int kGatherLoads = kTileLoads / kGatherWaves;          // 9 per wave and tile
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

__device__ __forceinline__ uint8_t* tile_buf(int ti) { return s_tile + (ti & (kBufs - 1)) * kTileBytes; }

template <int N>
__device__ __forceinline__ void wait_vmcnt() { asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory"); }

// Workgroup barrier for LDS data: waits for this wave's LDS operations only, so the tile
// gathers in flight stay in flight across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Wait until this wave's gathers of the current tile have landed, leaving the `later`
// tiles issued after it (0..3) in flight: a PV wave issues kGatherLoads loads per tile,
// and loads complete in issue order.
__device__ __forceinline__ void wait_tile(int later) {
    if (later >= 3) wait_vmcnt<3 * kGatherLoads>();
    else if (later == 2) wait_vmcnt<2 * kGatherLoads>();
    else if (later == 1) wait_vmcnt<kGatherLoads>();
    else wait_vmcnt<0>();
}

// LDS layout of a tile: row r (1152 bytes = 72 chunks of 16 bytes) keeps its chunk c at
// chunk position c ^ swz(r), swz(r) = (r >> 1) & 7.  Rows are 288 dwords apart, which is 32
// banks, so rows of one parity share a half of the 64 banks; within it the XOR gives the 8
// rows of each parity among any 16 consecutive rows distinct 4-bank groups, and 16-lane
// reads of one chunk over 16 consecutive rows are free of bank conflicts.  (The XOR stays
// inside each aligned group of 8 chunks, so the rope chunks 64..71 stay in place.)
__device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }

// Direct global->LDS loads of tile `ti`, issued by the PV waves (the QK waves' time between
// their matrix-core chains goes to the softmax): PV wave c issues the wave-wide 1 KB loads
// ci = c, c + 4, ... < 36; lane l of load ci fetches 16-byte chunk q = 64 ci + l of the tile,
// i.e. chunk q % 72 of selected row q / 72, stored at its swizzled position.  Written as
// inline assembly so that the compiler, which cannot tell the ring's buffers apart, inserts
// no drain of these loads before later LDS reads; completion is tracked with wait_tile()
// and published by lds_barrier().  M0 holds the wave-uniform LDS destination; nothing else
// in this kernel uses M0.  Unused slots fetch row 0 (masked).
struct GatherLane {
    int key[kGatherLoads];       // tile row of load i for this lane
    uint32_t off[kGatherLoads];  // byte offset of the lane's source chunk within that row
};
__device__ __forceinline__ GatherLane gather_lane(int c, int lane) {
    GatherLane gl;
#pragma unroll
    for (int i = 0; i < kGatherLoads; ++i) {
        const int q = (c + kGatherWaves * i) * kWave + lane;
        const int key = q / kRowChunks;
        gl.key[i] = key;
        gl.off[i] = static_cast<uint32_t>(((q - key * kRowChunks) ^ swz(key)) * 16);
    }
    return gl;
}
__device__ __forceinline__ void gather_tile(const uint8_t* lat_b, int ti, int c, const GatherLane& gl) {
    const uint32_t lds_base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
        (__attribute__((address_space(3))) uint8_t*)(tile_buf(ti))));
    int s[kGatherLoads];
#pragma unroll
    for (int i = 0; i < kGatherLoads; ++i) s[i] = s_keys[ti * kKt + gl.key[i]];
#pragma unroll
    for (int i = 0; i < kGatherLoads; ++i) {
        const int ci = c + kGatherWaves * i;
        const int row = s[i] < 0 ? 0 : s[i];
        const uint8_t* src = lat_b + static_cast<size_t>(row) * kRowBytes + gl.off[i];
        const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds_base + ci * kWave * 16);
        asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
                     :: "s"(m0v), "v"(src) : "memory");
    }
}

typedef __bf16 v4bf_t __attribute__((ext_vector_type(4)));

// ---- QK waves

// S partial of one tile over column half DH for 32 heads: lane l supplies key l % 32 of
// the tile as A operand (columns 288 DH + 16 ks + 8 (l / 32) .. + 7 of its row) and
// holds the matching query columns of head l % 32 as B operand; element r of the result
// is S[key 8 (r / 4) + 4 (l / 32) + r % 4][head l % 32].
template <int DH>
__device__ __forceinline__ v16f qk_half(const v8bf (&qreg)[kKs], const uint8_t* kb, int lane) {
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
    v16f acc;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.f;
    constexpr int kPre = 9;               // K-steps of operand reads in flight (LDS latency)
    v8bf a[kPre];
#pragma unroll
    for (int ks = 0; ks < kPre; ++ks) a[ks] = *addr(ks);
#pragma unroll
    for (int ks = 0; ks < kKs; ++ks) {
        acc = mfma_bf16_32x32x16(a[ks % kPre], qreg[ks], acc);
        if (ks + kPre < kKs) a[ks % kPre] = *addr(ks + kPre);
    }
    return acc;
}

struct QkState {
    float m_ref;     // reference logit of this lane's head (log2 units), -inf until set
    float m_max;     // largest logit seen
    float l_run;     // sum of this lane's numerators
    bool over;       // a logit above m_ref + kRefSpan
};

// Phase-1 tail: the partner's half of S (its 16 keys) and, while no reference is set, the
// partial logit of the first usable key of the tile (for every head of the half).
template <int DH>
__device__ __forceinline__ void qk_send(const v16f& acc, int hh, int lane, bool want_ref, int ref_key) {
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
    if (want_ref) {
        // key ref_key is element r = 4 (key / 8) + key % 4 of the lanes with l / 32 = (key / 4) & 1
        const int rk = 4 * (ref_key >> 3) + (ref_key & 3);
        float v = acc[0];
#pragma unroll
        for (int i = 1; i < 16; ++i) v = (i == rk) ? acc[i] : v;
        if ((lane >> 5) == ((ref_key >> 2) & 1)) s_ref[hh][DH][lane & 31] = v;
    }
}

// Phase 2: this wave's 16 keys of S complete, softmax numerators, P published.  The lane
// holds keys 16 DH + 8 (s / 4) + 4 (l / 32) + s % 4, s = 0..7, of head l % 32 -- exactly
// K-slot s of the P operand for K-step DH of the PV product.
//   first_max  (step 0, tile 0 usable) the reference is the tile's largest logit: each
//              wave posts the maximum of its 16 keys, and after one extra barrier (which
//              the PV waves pass as well) takes the larger of the two;
//   want_ref   (a later first usable tile) the reference is the logit of the tile's first
//              usable key, the sum of the two halves' partials.
template <int DH>
__device__ __forceinline__ void qk_finish(v16f& acc, QkState& st, int hh, int lane, uint32_t tmask,
                                          bool first_max, bool want_ref, float scale_log2, bool fixed) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const float4 v = *reinterpret_cast<const float4*>(&s_half[hh][DH][j][lane][0]);
        acc[8 * DH + 4 * j + 0] += v.x;
        acc[8 * DH + 4 * j + 1] += v.y;
        acc[8 * DH + 4 * j + 2] += v.z;
        acc[8 * DH + 4 * j + 3] += v.w;
    }
    const int g = lane >> 5;
    float v[8];
    float mx = -INFINITY;
    if (tmask == 0xffffffffu) {                           // every slot usable (uniform)
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            v[s] = acc[8 * DH + s] * scale_log2;
            mx = fmaxf(mx, v[s]);
        }
    } else {
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const int key = 16 * DH + 8 * (s >> 2) + 4 * g + (s & 3);
            const bool ok = (tmask >> key) & 1u;
            v[s] = ok ? acc[8 * DH + s] * scale_log2 : -INFINITY;
            mx = fmaxf(mx, v[s]);
        }
    }
    if (first_max) {
        const float m2 = max_xor32(mx);
        if (lane < 32) s_ref[hh][DH][lane] = m2;
        lds_barrier();                                     // C: the extra step-0 barrier
        st.m_ref = fmaxf(s_ref[hh][0][lane & 31], s_ref[hh][1][lane & 31]);
    } else if (want_ref) {
        st.m_ref = (s_ref[hh][0][lane & 31] + s_ref[hh][1][lane & 31]) * scale_log2;
    }
    if (!fixed) {
        st.m_max = fmaxf(st.m_max, mx);
        st.over = st.over || mx > st.m_ref + kRefSpan;
    }
    // no usable key seen yet: every logit so far is -inf, any finite reference gives 0
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
        // the lane's keys 16 kk + 8 qh + 4 g + e share swz = (4 qh + 2 g + e / 2) & 7
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
    // Tiles in flight while tile ti is used: ti + 1 and ti + 2 (at step 0 only tile 1: tiles
    // 2 and 3 follow the queries through buffers 2 and 3 and go out after barrier B(0)).
    auto later_tiles = [&](int ti) { return ti == 0 ? min(1, n_tiles - 1) : min(2, n_tiles - 1 - ti); };
    // A(ti): the PV waves wait for their loads of tile ti (the QK waves load no tiles)
    auto step_begin = [&](int ti) {
        if (!qk_wave && ti < n_tiles) wait_tile(later_tiles(ti));
        lds_barrier();
    };
    auto step_gathers = [&](int ti, const GatherLane& gl) {   // PV waves, after B(ti): tile ti's buffer is free
        if (ti == 0) {
            for (int tj = 2; tj <= 3; ++tj)
                if (tj < n_tiles) gather_tile(lat_b, tj, wave - 4, gl);
        } else if (ti + 3 < n_tiles) {
            gather_tile(lat_b, ti + 3, wave - 4, gl);
        }
    };
    const bool tile0_usable = n_tiles > 0 && s_tmask[0] != 0u;

    // The two roles run separate code with the same barrier sequence (the slot barrier,
    // A and B per step for n_tiles + 1 steps plus C at step 0 of a first pass with a usable
    // first tile, the recompute decision, an optional second pass, the staging barrier),
    // so their registers -- queries and S for the QK waves, output accumulators and V
    // operands for the PV waves -- are never live at the same time.  The PV waves issue and
    // wait for every tile's gathers; the QK waves see the tiles through barrier A.
    if (qk_wave) {
        v8bf qreg[kKs];
        const uint16_t* qrow = q + (static_cast<size_t>(row) * H_total + head0 + 32 * hh + (lane & 31)) * kDq +
                               288 * dh + 8 * (lane >> 5);
        QkState qs;
        qs.m_ref = -INFINITY;
        qs.m_max = -INFINITY;
        qs.over = false;
        auto qk_pass = [&](bool fixed) {
            bool ref_set = fixed;
            qs.l_run = 0.f;
            if (!fixed) load_q(qrow, wave);
            for (int ti = 0; ti <= n_tiles; ++ti) {
                if (ti == 0) wait_vmcnt<0>();                         // this wave's queries
                step_begin(ti);
                if (ti == 0 && !fixed) {
                    // this wave's queries, landed with tile 0 (its own loads: no barrier needed)
                    const uint8_t* qs_lds = q_stage(wave) + 16 * lane;
#pragma unroll
                    for (int ks = 0; ks < kKs; ++ks) qreg[ks] = *reinterpret_cast<const v8bf*>(qs_lds + ks * 1024);
                }
                const uint32_t tmask = ti < n_tiles ? s_tmask[ti] : 0u;
                // reference still unset and this tile usable (uniform over the workgroup)
                const bool first_max = !ref_set && ti == 0 && tmask != 0u;
                const bool want_ref = !ref_set && ti > 0 && tmask != 0u;
                const int ref_key = want_ref ? __builtin_ctz(tmask) : 0;
                v16f sacc;
                if (ti < n_tiles) {
                    if (dh == 0) {
                        sacc = qk_half<0>(qreg, tile_buf(ti), lane);
                        qk_send<0>(sacc, hh, lane, want_ref, ref_key);
                    } else {
                        sacc = qk_half<1>(qreg, tile_buf(ti), lane);
                        qk_send<1>(sacc, hh, lane, want_ref, ref_key);
                    }
                }
                lds_barrier();                                        // B(ti)
                if (ti < n_tiles) {
                    if (dh == 0) qk_finish<0>(sacc, qs, hh, lane, tmask, first_max, want_ref, scale_log2, fixed);
                    else qk_finish<1>(sacc, qs, hh, lane, tmask, first_max, want_ref, scale_log2, fixed);
                }
                ref_set = ref_set || first_max || want_ref;
            }
        };
        qk_pass(false);
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
            qk_pass(true);
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
        auto pv_pass = [&](bool fixed) {
            const VAddr va = v_addr(c, lane);
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
                for (int ct = 0; ct < 4; ++ct)
#pragma unroll
                    for (int i = 0; i < 16; ++i) pv.acc[h2][ct][i] = 0.f;
            const GatherLane gl = gather_lane(c, lane);
            if (n_tiles > 0) gather_tile(lat_b, 0, c, gl);
            if (n_tiles > 1) gather_tile(lat_b, 1, c, gl);
            v8bf vop[2][4];                                           // V operands of the previous tile
            for (int ti = 0; ti <= n_tiles; ++ti) {
                step_begin(ti);
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
                lds_barrier();                                        // B(ti)
                step_gathers(ti, gl);
                if (!fixed && ti == 0 && tile0_usable) lds_barrier();  // C
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
