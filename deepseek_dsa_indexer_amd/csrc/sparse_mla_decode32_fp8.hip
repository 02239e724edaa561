// sparse_mla_decode32_fp8.hip -- absorbed (MQA) sparse attention over selected latent rows
// stored in the 656-byte FP8 form, on the gfx950 32x32x16 bf16 matrix-core form.
//
// The core-attention box of "dsa-indexer.excalidraw" over its latent cache drawn as FP8
// latents plus a bf16 rope part (656 B per token, its cost box): each selected row is the
// key (512 latent columns, then 64 rope columns) and the value (the 512 latent columns).
// Row layout: 512 e4m3fn codes, four fp32 scales (column d < 512 decodes to
// code[d] * scale[d / 128]), 64 bf16 rope values.  The softmax and value mix follow the MLA
// prefill excerpt ("DeepSeek-V3.2-Exp - Causal mask", Multi-head latent attention).
//
// The workgroup shape, the two wave roles and the fixed-reference softmax are those of
// sparse_mla_decode32.hip; what differs is the row form:
//   - tiles of 64 selected rows (the 656-byte rows let a 3-buffer ring of them fit in LDS,
//     halving the per-step latency cost per row against 32-row tiles), gathered as 42
//     wave-wide 16-byte-per-lane direct loads per tile plus four 4-byte-per-lane loads
//     that put the tile's block scales into a [block][row] table;
//   - QK waves: the column half of wave (hh, dh) is latent blocks 2 dh and 2 dh + 1 plus rope
//     columns 32 dh .. 32 dh + 31 (18 K-steps of 16), so each wave meets two scale blocks.
//     Codes are widened exactly to bf16 (every e4m3fn value is a bf16 value); each block
//     runs its own chain of eight matrix-core instructions, and its partial S is
//     multiplied by the row's block scale in fp32 (keys are the matrix rows, so a lane's
//     16 elements need the scales of 16 rows: four 16-byte reads of the scale table) and
//     added to the rope chain's result.  No dequantised value is rounded.
//   - PV waves: wave 4 + c owns output columns 128 c .. 128 c + 127, which is latent block c
//     exactly; its V operands are the codes, read by 8-byte transpose reads
//     (ds_read_b64_tr_b8: within a 16-lane group lane n receives byte n % 8 of the address
//     of lane 2 e + n / 8 as element e) and widened exactly, and the block scale of each key
//     is folded into that key's P operand value (bf16 numerator times the fp32 scale,
//     rounded to bf16 once more).
//
// Pipeline: step i (two workgroup barriers) --
//   A(i)     tile i has landed for every wave.
//   phase 1  QK waves: QK(i), with the numerators of tile i-1 formed between its matrix-
//            core instructions and published as P(i-1); the partner halves of S(i) out.
//            PV waves: their share of the gathers of tile i+2, into tile i-1's buffer.
//   B(i)
//   phase 2  QK waves: S(i) completed; their share (with the scale table) of tile i+2.
//            PV waves: PV(i-1) from P(i-1) and the codes of tile i-1 held in registers,
//            then the codes of tile i into the same registers.
// The scale tables live in a ring of four (tile i-1's is still read in phase 2 of step i
// while tile i+2's is loaded).  The queries go straight into the QK waves' registers.
#include "dsa_device.h"
#include "dsa_internal.h"

namespace dsa {

namespace {

constexpr int kThreads = 512;
constexpr int kWaves = 8;
constexpr int kHeads = 64;                          // heads per workgroup
constexpr int kDq = 576;
constexpr int kDv = 512;
constexpr int kRow = 656;                           // bytes per FP8 latent row
constexpr int kRowChunks = kRow / 16;               // 41
constexpr int kScaleOff = 512;                      // four fp32 block scales
constexpr int kRopeOff = 528;                       // 64 bf16 rope values
constexpr int kKt = 64;                             // selected rows per tile
constexpr int kGroupChunks = 16 * kRowChunks + 8;   // 16 rows, then 128 bytes of padding
constexpr int kTileChunks = 4 * kGroupChunks;       // 2656
constexpr int kTileBytes = kTileChunks * 16;        // 42,496
constexpr int kRowLoads = (kTileChunks + kWave - 1) / kWave;   // 42 (the last one half used)
constexpr int kLoads = kRowLoads + 4;               // + four block-scale loads
constexpr int kPositions = 4;                       // wave positions sharing a tile's loads
constexpr int kPerPos = (kLoads + kPositions - 1) / kPositions;  // 12
constexpr int kPvLoads = 6;                         // loads i < 6 of a position: its PV wave
constexpr int kQkLoads = kPerPos - kPvLoads;        // loads i >= 6: its QK wave
constexpr int kBufs = 3;                            // tile ring
constexpr int kScaleBufs = 4;                       // scale-table ring
constexpr int kMaxTiles = 8;                        // tiles per split
constexpr int kMaxSlots = kMaxTiles * kKt;          // 512 slots per split
constexpr int kKs = 18;                             // K-steps per column half
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRefSpan = 64.0f;                   // log2 units above the reference

static_assert(kMaxSlots == kThreads, "one slot per thread at start-up");

// LDS: 127,488 (tiles) + 4,096 (scale tables) + 16,384 (S halves) + 8,192 (P) + 2,048
// (slots) + small.
__shared__ __attribute__((aligned(16))) uint8_t s_tile[kBufs * kTileBytes];
__shared__ __attribute__((aligned(16))) float s_scale[kScaleBufs][4][kKt];          // [block][row]
__shared__ __attribute__((aligned(16))) float s_half[2][2][2][2][kWave][4];         // [hh][owner dh][kb][j][lane][4]
__shared__ __attribute__((aligned(16))) uint8_t s_p[2][4][kWave][16];               // [hh][kk][lane][8 bf16]
__shared__ int32_t s_keys[kMaxSlots];
__shared__ unsigned long long s_tmask[kMaxTiles];   // usable slots of each tile (bit = row)
__shared__ float s_ref[2][2][32];                   // [hh][dh][head]: reference exchange
__shared__ float s_l[2][2][32];                     // [hh][dh][head] numerator sums
__shared__ float s_m[2][2][32];                     // [hh][dh][head] reference / split maximum
__shared__ int32_t s_redo[kWaves];

template <int N> struct IntConst { static constexpr int value = N; };

__device__ __forceinline__ uint8_t* tile_buf(int ti) { return s_tile + (ti % kBufs) * kTileBytes; }
__device__ __forceinline__ float* scale_tab(int ti, int blk) { return &s_scale[ti & (kScaleBufs - 1)][blk][0]; }

// Tile layout: groups of 16 rows, each followed by 128 bytes of padding; within a group,
// row r sits at position kpos(r) = 8 (r / 8) + 2 (r % 4) + (r / 4) % 2, 656 bytes apart.
// With 64 banks of 4 bytes, position p starts 9 p (mod 16) 16-byte bank groups in, so the
// 16 rows of a group fill the 16 groups once: a 16-byte read of one column over 16 rows
// (QK operands, 16 lanes per pass) is free of conflicts.  The PV transpose reads take 32
// bytes of one column from rows {0, 1, 2, 3, 8, 9, 10, 11} (or the other eight) per 32-lane
// pass; those rows sit at even (odd) positions, whose 32-byte runs tile the 64 banks.
__device__ __forceinline__ int kpos(int r) { return 8 * (r >> 3) + 2 * (r & 3) + ((r >> 2) & 1); }
__device__ __forceinline__ int kslot(int p) { return 8 * (p >> 3) + 4 * (p & 1) + ((p & 7) >> 1); }
__device__ __forceinline__ int row_off(int r) { return ((r >> 4) * kGroupChunks + kpos(r & 15) * kRowChunks) * 16; }

template <int N>
__device__ __forceinline__ void wait_vmcnt() { asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory"); }

// Workgroup barrier for LDS data: waits for this wave's LDS operations only, so the tile
// gathers in flight stay in flight across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Gathers of tile t: wave-wide loads ci = c + 4 i of wave position c = 0..3, i = 0..11
// (ci >= kLoads repeats load ci - 4, so every position issues twelve).  ci < kRowLoads:
// lane l fetches 16-byte chunk p = 64 ci + l of the tile buffer -- row 16 (p / 664) +
// (p % 664) / 41, chunk (p % 664) % 41, or padding (p % 664 >= 656: a dummy fetch of the
// tile's first row), or nothing (p >= kTileChunks); ci >= kRowLoads: lane l fetches the
// 4-byte scale ci - kRowLoads of row l into the scale table.  PV wave c issues i < kPvLoads
// in phase 1 (all twelve for tiles 0 and 1), QK wave c the rest in phase 2.  Written as
// inline assembly so that the compiler, which cannot tell the ring's buffers apart,
// inserts no drain of these loads; completion is tracked with vmcnt and published by
// lds_barrier().  M0 holds the wave-uniform LDS destination; nothing else here uses M0.
// Unused slots fetch the sequence's row 0 (masked).
__device__ __forceinline__ int load_index(int c, int i) {
    const int ci = c + kPositions * i;
    return ci >= kLoads ? ci - kPositions : ci;
}
template <int I0, int N>
struct GatherLane {
    int key[N];         // tile row whose selected position this lane's load I0 + i fetches, -1: none
    int off[N];         // byte offset within that row
};
template <int I0, int N>
__device__ __forceinline__ GatherLane<I0, N> gather_lane(int c, int lane) {
    GatherLane<I0, N> gl;
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const int ci = load_index(c, I0 + i);
        if (ci < kRowLoads) {
            const int p = ci * kWave + lane;
            const int grp = p / kGroupChunks;
            const int w = p - grp * kGroupChunks;
            const bool data = w < 16 * kRowChunks;
            gl.key[i] = p >= kTileChunks ? -1 : data ? 16 * grp + kslot(w / kRowChunks) : 0;
            gl.off[i] = data ? (w % kRowChunks) * 16 : 0;
        } else {
            gl.key[i] = lane;
            gl.off[i] = kScaleOff + 4 * (ci - kRowLoads);
        }
    }
    return gl;
}
// Loads I0 + J0 .. I0 + J0 + M - 1 of position c for tile ti.
template <int J0, int M, int I0, int N>
__device__ __forceinline__ void gather_tile(const uint8_t* lat_b, int ti, int c, const GatherLane<I0, N>& gl) {
    static_assert(J0 + M <= N, "loads outside the lane's part");
    const uint32_t tile_lds = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
        (__attribute__((address_space(3))) uint8_t*)(tile_buf(ti))));
    int s[M];
#pragma unroll
    for (int i = 0; i < M; ++i) s[i] = s_keys[ti * kKt + max(gl.key[J0 + i], 0)];
#pragma unroll
    for (int i = 0; i < M; ++i) {
        const int ci = load_index(c, I0 + J0 + i);
        const uint8_t* src = lat_b + static_cast<size_t>(max(s[i], 0)) * kRow + gl.off[J0 + i];
        if (ci < kRowLoads) {
            const uint32_t m0v = __builtin_amdgcn_readfirstlane(tile_lds + ci * kWave * 16);
            if (gl.key[J0 + i] >= 0)
                asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
                             :: "s"(m0v), "v"(src) : "memory");
        } else {
            const uint32_t m0v = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
                (__attribute__((address_space(3))) float*)(scale_tab(ti, ci - kRowLoads)))));
            asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, off"
                         :: "s"(m0v), "v"(src) : "memory");
        }
    }
}

typedef int v2i_t __attribute__((ext_vector_type(2)));

// ---- QK waves

struct QkState {
    float m_ref;     // reference logit of this lane's head (log2 units), -inf until set
    float m_max;     // largest logit seen
    float l_run;     // sum of this lane's numerators
    bool over;       // a logit above m_ref + kRefSpan
};

// K-step order of a QK wave for one 32-row half kb of the tile: the two rope steps (into
// the total), then latent block 2 dh (steps 0..7) and block 2 dh + 1 (steps 8..15), each
// its own chain.  The lane supplies row 32 kb + l % 32 and eight columns of the step:
// codes at byte 256 dh + 32 (ks / 2) + 16 (l / 32) + 8 (ks % 2) (the two steps of a pair
// come from one 16-byte read; the block's columns are a permutation of its 128, the
// queries' K-steps use the same one), or rope values at byte 528 + 64 dh + 32 (ks - 16) +
// 16 (l / 32).
__device__ __forceinline__ constexpr int qk_order(int n) { return n < 2 ? 16 + n : n - 2; }

// Phase 1 of a QK wave: the numerators of the tile completed in the previous step,
// published as P, then the S partials of both 32-row halves of tile ti over its columns
// for 32 heads.  For half kb, element r of lane l is S[row 32 kb + 8 (r / 4) + 4 (l / 32)
// + r % 4][head l % 32]: as soon as a half is complete the 8 elements that the partner
// finishes go to LDS, and the wave keeps its own 8 (own[kb][s] = element 8 DH + s).
template <int DH>
__device__ __forceinline__ void qk_tile(float (&own)[2][8], const v8bf (&qreg)[kKs], const uint8_t* kb_lds,
                                        const float* sA, const float* sB, int lane,
                                        const float (&v)[2][8], float mx, QkState& st, int hh, bool fixed) {
    constexpr int kOther = 1 - DH;
    int lo = lane;
    asm volatile("" : "+v"(lo));
    const int r = lo & 31;
    const int g = lo >> 5;
    st.over = st.over || (!fixed && mx > st.m_ref + kRefSpan);
    const float mref = st.m_ref == -INFINITY ? 0.f : st.m_ref;
    // One 16-byte read per unit: units 0, 1 of a half are the two rope steps, units 2 + m the
    // code K-steps 2 m and 2 m + 1 (bytes 256 dh + 32 m + 16 g: codes 0..7 for step 2 m,
    // 8..15 for step 2 m + 1 -- the queries use the same column order).
    auto unit_of = [](int n) { const int m = n % kKs; return (kKs / 2 + 1) * (n / kKs) + (m < 2 ? m : 2 + (m - 2) / 2); };
    auto unit_read = [&](int u) -> int4 {
        const int kb = u / (kKs / 2 + 1);
        const int k = u % (kKs / 2 + 1);
        const uint8_t* row = kb_lds + row_off(32 * kb + r);
        if (k < 2) return *reinterpret_cast<const int4*>(row + kRopeOff + 64 * DH + 32 * k + 16 * g);
        return *reinterpret_cast<const int4*>(row + 256 * DH + 32 * (k - 2) + 16 * g);
    };
    auto op = [&](int ks, const int4& w) -> v8bf {
        if (ks < 16) return (ks & 1) ? fp8x8_to_bf16(w.z, w.w) : fp8x8_to_bf16(w.x, w.y);
        return __builtin_bit_cast(v8bf, w);
    };
    // acc += scale (of the lane's 16 rows: 32 kb + 8 j + 4 g + 0..3) * blk
    auto fold = [&](v16f& acc, const v16f& blk, const float* tab, int kb) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float4 s4 = *reinterpret_cast<const float4*>(tab + 32 * kb + 8 * j + 4 * g);
            acc[4 * j + 0] += s4.x * blk[4 * j + 0];
            acc[4 * j + 1] += s4.y * blk[4 * j + 1];
            acc[4 * j + 2] += s4.z * blk[4 * j + 2];
            acc[4 * j + 3] += s4.w * blk[4 * j + 3];
        }
    };
    constexpr int kN = 2 * kKs;           // K-steps of both halves
    constexpr int kUnits = 2 * (kKs / 2 + 1);   // 20 reads per tile
    constexpr int kPre = 4;               // read units in flight (LDS latency)
    int4 raw[kPre];
#pragma unroll
    for (int u = 0; u < kPre; ++u) raw[u] = unit_read(u);
    // numerators of the previous tile first, while the first operand reads are in flight
    // (the previous logits are then dead during the chains: registers are scarce here)
    float psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        v8s pk;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const float p = exp2_num(v[kb][s] - mref);
            psum += p;
            pk[s] = static_cast<short>(f32_to_bf16(p));
        }
        *reinterpret_cast<v8s*>(&s_p[hh][2 * kb + DH][lane][0]) = pk;
    }
    st.l_run += psum;
    v16f acc, accA, accB;
#pragma unroll
    for (int n = 0; n < kN; ++n) {
        const int kb = n / kKs;
        const int m = n % kKs;
        const int ks = qk_order(m);
        const int u = unit_of(n);
        const v8bf a = op(ks, raw[u % kPre]);
        // the unit's last step: its slot takes the read kPre units ahead
        if ((m < 2 || (ks & 1)) && u + kPre < kUnits) raw[u % kPre] = unit_read(u + kPre);
        if (m < 2) {
            acc = mfma_bf16_32x32x16(a, qreg[ks], m == 0 ? v16f{} : acc);
        } else if (m < 10) {
            accA = mfma_bf16_32x32x16(a, qreg[ks], m == 2 ? v16f{} : accA);
        } else {
            accB = mfma_bf16_32x32x16(a, qreg[ks], m == 10 ? v16f{} : accB);
        }
        // block 2 dh folded while block 2 dh + 1 runs; block 2 dh + 1 at the end of the half
        if (m == 12) fold(acc, accA, sA, kb);
        if (m == 17) {
            fold(acc, accB, sB, kb);
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                float4 w;
                w.x = acc[8 * kOther + 4 * j + 0];
                w.y = acc[8 * kOther + 4 * j + 1];
                w.z = acc[8 * kOther + 4 * j + 2];
                w.w = acc[8 * kOther + 4 * j + 3];
                *reinterpret_cast<float4*>(&s_half[hh][kOther][kb][j][lane][0]) = w;
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) own[kb][e] = acc[8 * DH + e];
        }
    }
}

// Phase 2: this wave's 16 rows of each half complete (the partner's part added), in log2
// units, -inf at unusable slots; returns the lane's maximum.  The lane holds rows
// 32 kb + 16 DH + 8 (s / 4) + 4 (l / 32) + s % 4 of head l % 32 -- K-slot s of the P operand
// for PV K-step 2 kb + DH.
template <int DH>
__device__ __forceinline__ float qk_complete(const float (&own)[2][8], int hh, int lane, unsigned long long tmask,
                                             float scale_log2, float (&v)[2][8]) {
    const int g = lane >> 5;
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const float4 h = *reinterpret_cast<const float4*>(&s_half[hh][DH][kb][j][lane][0]);
            const float hv[4] = {h.x, h.y, h.z, h.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int s = 4 * j + e;
                const int row = 32 * kb + 16 * DH + 8 * j + 4 * g + e;
                const bool ok = (tmask >> row) & 1ull;
                v[kb][s] = ok ? (own[kb][s] + hv[e]) * scale_log2 : -INFINITY;
                mx = fmaxf(mx, v[kb][s]);
            }
        }
    return mx;
}

// The numerators alone (the step after the last tile).
template <int DH>
__device__ __forceinline__ void qk_numerators(const float (&v)[2][8], float mx, QkState& st, int hh,
                                              int lane, bool fixed) {
    st.over = st.over || (!fixed && mx > st.m_ref + kRefSpan);
    const float mref = st.m_ref == -INFINITY ? 0.f : st.m_ref;
    float psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        v8s pk;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const float p = exp2_num(v[kb][s] - mref);
            psum += p;
            pk[s] = static_cast<short>(f32_to_bf16(p));
        }
        *reinterpret_cast<v8s*>(&s_p[hh][2 * kb + DH][lane][0]) = pk;
    }
    st.l_run += psum;
}

// ---- PV waves

// Output columns 128 c + 32 ct + ..., ct = 0..3, of all 64 heads, as O^T tiles:
// acc[hh][ct] element r of lane l is O[head 32 hh + l % 32][column 128 c + 32 ct +
// 8 (r / 4) + 4 (l / 32) + r % 4].
struct PvState {
    v16f acc[2][4];
};

// The codes of the A operand (V^T: output columns x rows) for K-step kk and column tile
// ct: lane l of 16-lane group G (n = l % 16, g = G / 2) needs column 32 ct + 16 (G % 2) + n
// and rows 16 kk + 8 (e / 4) + 4 g + e % 4, e = 0..7 (the P operand's K-slots); the
// transpose read hands it element e from the address of lane 2 e + n / 8, so lane m of the
// group points at row 16 kk + 8 (e / 4) + 4 g + e % 4 (e = m / 2), columns 32 ct + 16 (G % 2) +
// 8 (m % 2) .. + 7.
__device__ __forceinline__ int v_base(int c, int lane) {
    int lo = lane;
    asm volatile("" : "+v"(lo));
    const int G = lo >> 4;
    const int m = lo & 15;
    const int e = m >> 1;
    const int g = G >> 1;
    return (8 * (e >> 2) + 2 * (e & 3) + g) * kRow + 128 * c + 16 * (G & 1) + 8 * (m & 1);   // kpos of row 8 (e >> 2) + 4 g + (e & 3)
}
__device__ __forceinline__ void load_codes(v2i_t (&vc)[4][4], const uint8_t* kb_lds, int vb) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int ct = 0; ct < 4; ++ct)
            vc[kk][ct] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                (__attribute__((address_space(3))) v2i_t*)(kb_lds + kk * (kGroupChunks * 16) + 32 * ct + vb));
}

// PV of one tile: 32 instructions (4 K-steps x 2 head halves x 4 column tiles); the P
// operands of K-step kk scaled by the block-c scales of their rows 16 kk + 8 (s / 4) +
// 4 (l / 32) + s % 4.
__device__ __forceinline__ void pv_tile(PvState& st, const v2i_t (&vc)[4][4], const float* tab, int lane) {
    const int g = lane >> 5;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        const float4 s0 = *reinterpret_cast<const float4*>(tab + 16 * kk + 4 * g);
        const float4 s1 = *reinterpret_cast<const float4*>(tab + 16 * kk + 8 + 4 * g);
        const float sc[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
        v8bf pop[2];
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
            const v8s pr = *reinterpret_cast<const v8s*>(&s_p[h2][kk][lane][0]);
            v8s ps;
#pragma unroll
            for (int s = 0; s < 8; ++s)
                ps[s] = static_cast<short>(f32_to_bf16(bf16_to_f32(static_cast<uint16_t>(pr[s])) * sc[s]));
            pop[h2] = __builtin_bit_cast(v8bf, ps);
        }
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
            const v8bf va = fp8x8_to_bf16(vc[kk][ct][0], vc[kk][ct][1]);
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) st.acc[h2][ct] = mfma_bf16_32x32x16(va, pop[h2], st.acc[h2][ct]);
        }
    }
}

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void mla_decode32_fp8_kernel(const uint16_t* __restrict__ q, const uint8_t* __restrict__ latent,
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

    // Workgroup (row, split, head part), block (part * n_splits + split) * rows + row (the
    // workgroups of a row share an XCD when rows is a multiple of 8).
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

    const int32_t* sel = idx + static_cast<size_t>(row) * k;
    const int j0 = threadIdx.x;               // kMaxSlots == kThreads
    const int slot0 = tile0 * kKt + j0;
    const int sraw = (j0 < nslots && slot0 < k) ? sel[slot0] : -1;
    const int seq_len = len[b];
    // the sequence's rows, kept in scalar registers (wave-uniform)
    const uint8_t* lat_b;
    {
        const uint64_t a = reinterpret_cast<uint64_t>(latent + static_cast<size_t>(b) * Lmax * kRow);
        const uint32_t lo32 = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a));
        const uint32_t hi32 = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a >> 32));
        lat_b = reinterpret_cast<const uint8_t*>((static_cast<uint64_t>(hi32) << 32) | lo32);
    }

    {
        const int pos = n_visible(seq_len, T, t, Lmax, m) - 1;     // last visible cache row
        const int sv = (sraw >= 0 && sraw <= pos) ? sraw : -1;
        if (j0 < nslots) s_keys[j0] = sv;
        // usable-slot mask of each tile: wave w covers tile w
        const unsigned long long bal = __ballot(sv >= 0 && j0 < nslots);
        if (lane == 0) s_tmask[wave] = bal;
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
    int ref_tile = -1;
    for (int i = n_tiles - 1; i >= 0; --i)
        if (s_tmask[i] != 0ull) ref_tile = i;

    if (qk_wave) {
        // queries of head 32 hh + l % 32, in the column order of the code reads: K-step ks < 16
        // holds columns 256 dh + 32 (ks / 2) + 16 (l / 32) + 8 (ks % 2) .. + 7, ks >= 16 rope
        // columns 512 + 32 dh + 16 (ks - 16) + 8 (l / 32) .. + 7
        v8bf qreg[kKs];
        const uint16_t* qrow = q + (static_cast<size_t>(row) * H_total + head0 + 32 * hh + (lane & 31)) * kDq;
        const int gq = lane >> 5;
#pragma unroll
        for (int ks = 0; ks < kKs; ++ks)
            qreg[ks] = *reinterpret_cast<const v8bf*>(
                qrow + (ks < 16 ? 256 * dh + 32 * (ks >> 1) + 16 * gq + 8 * (ks & 1) : 512 + 32 * dh + 16 * (ks - 16) + 8 * gq));
        // wait for them here, with the wait instruction the compiler tracks (vmcnt(0)), so
        // that it places no wait for them inside the tile loop, where it would also drain
        // this wave's gathers
        __builtin_amdgcn_s_waitcnt(0x0f70);
        QkState qs;
        qs.m_ref = -INFINITY;
        qs.m_max = -INFINITY;
        qs.over = false;
        auto qk_pass = [&](auto dhc, bool fixed) {
            constexpr int DH = decltype(dhc)::value;
            bool ref_known = fixed;
            qs.l_run = 0.f;
            float v[2][8];                                            // S of the completed tile
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int s = 0; s < 8; ++s) v[kb][s] = -INFINITY;
            float vmx = -INFINITY;
            for (int ti = 0; ti <= n_tiles; ++ti) {
                if (ti >= 2 && ti < n_tiles) {
                    if (ti + 1 < n_tiles) wait_vmcnt<kQkLoads>();     // own loads of tile ti
                    else wait_vmcnt<0>();
                }
                lds_barrier();                                        // A(ti)
                if (!ref_known && ref_tile >= 0 && ti == ref_tile + 1) {
                    qs.m_ref = fmaxf(s_ref[hh][0][lane & 31], s_ref[hh][1][lane & 31]);
                    ref_known = true;
                }
                if (ti < n_tiles) {
                    float own[2][8];
                    qk_tile<DH>(own, qreg, tile_buf(ti), scale_tab(ti, 2 * DH), scale_tab(ti, 2 * DH + 1),
                                lane, v, vmx, qs, hh, fixed);
                    lds_barrier();                                    // B(ti)
                    vmx = qk_complete<DH>(own, hh, lane, s_tmask[ti], scale_log2, v);
                    qs.m_max = fmaxf(qs.m_max, vmx);
                    if (!ref_known && ti == ref_tile) {
                        const float m2 = max_xor32(vmx);
                        if (lane < 32) s_ref[hh][DH][lane] = m2;
                    }
                    // this wave's share of tile ti+2, into tile ti-1's buffer (the lane's
                    // load addresses recomputed here: registers are scarce in this role)
                    if (ti + 2 < n_tiles) {
                        int ln = lane;
                        asm volatile("" : "+v"(ln));                  // not hoisted out of the loop
                        const GatherLane<kPvLoads, kQkLoads> glq = gather_lane<kPvLoads, kQkLoads>(wave, ln);
                        gather_tile<0, kQkLoads>(lat_b, ti + 2, wave, glq);
                    }
                } else {
                    qk_numerators<DH>(v, vmx, qs, hh, lane, fixed);
                    lds_barrier();                                    // B(ti)
                }
            }
        };
        if (dh == 0) qk_pass(IntConst<0>{}, false);
        else qk_pass(IntConst<1>{}, false);
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
            const int vb = v_base(c, lane);
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
                for (int ct = 0; ct < 4; ++ct)
#pragma unroll
                    for (int i = 0; i < 16; ++i) pv.acc[h2][ct][i] = 0.f;
            const GatherLane<0, kPvLoads> gl = gather_lane<0, kPvLoads>(c, lane);
            {
                const GatherLane<kPvLoads, kQkLoads> gl2 = gather_lane<kPvLoads, kQkLoads>(c, lane);
                for (int tj = 0; tj < 2; ++tj)
                    if (tj < n_tiles) {
                        gather_tile<0, kPvLoads>(lat_b, tj, c, gl);
                        gather_tile<0, kQkLoads>(lat_b, tj, c, gl2);
                    }
            }
            v2i_t vc[4][4];                                           // codes of the previous tile
            for (int ti = 0; ti <= n_tiles; ++ti) {
                if (ti == 0) {
                    if (n_tiles > 1) wait_vmcnt<kPerPos>();           // tile 0 of the prologue
                    else wait_vmcnt<0>();
                } else if (ti < n_tiles) {
                    if (ti + 1 < n_tiles) wait_vmcnt<kPvLoads>();     // own loads of tile ti
                    else wait_vmcnt<0>();
                }
                lds_barrier();                                        // A(ti)
                if (ti + 2 < n_tiles) gather_tile<0, kPvLoads>(lat_b, ti + 2, c, gl);
                lds_barrier();                                        // B(ti)
                if (ti > 0) pv_tile(pv, vc, scale_tab(ti - 1, c), lane);
                if (ti < n_tiles) load_codes(vc, tile_buf(ti), vb);
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

int mla_decode32_fp8_max_tiles() { return kMaxTiles; }
int mla_decode32_fp8_tile_rows() { return kKt; }

hipError_t launch_mla_decode32_fp8(const void* q, const void* latent, const int32_t* idx,
                                   const int32_t* len, int rows, int T, int H, int Lmax, int k, int m,
                                   int tiles_per_split, int n_splits, float scale_log2, void* out,
                                   float* lse, void* part_o, float* part_lse, hipStream_t stream) {
    const int parts = H / kHeads;
    return launch_kernel(kPhaseAttention, mla_decode32_fp8_kernel, dim3(rows * n_splits * parts),
                         dim3(kThreads), 0, stream, static_cast<const uint16_t*>(q),
                         static_cast<const uint8_t*>(latent), idx, len, T, Lmax, k, m, tiles_per_split,
                         n_splits, H, scale_log2, static_cast<uint16_t*>(out), lse,
                         static_cast<uint16_t*>(part_o), part_lse);
}

}  // namespace dsa
