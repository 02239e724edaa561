// sparse_mha_prefill.hip -- MHA-form sparse attention of a prefill chunk on bf16 matrix
// cores (qk width 192 = nope 128 + rope 64, value width 128).
//
// The MLA prefill excerpt ("DeepSeek-V3.2-Exp - Causal mask" page, Multi-head latent
// attention, prefill) forms dense scores, adds an index mask that is 0 at the top-k
// positions and -inf elsewhere plus the causal mask, and takes a softmax.  Per head the
// selected keys of neighbouring query rows are unrelated (2048 of up to 8192 each), so
// a tile of query rows touches nearly every key block anyway; the kernel therefore
// runs a causal flash-attention sweep over key blocks and applies the selection as a
// bit mask built from idx by select_mask_kernel (bit s of row t set iff s is selected
// and s <= t).  Masked-dense work is about 2.3x the selected pairs at T = 8192, k = 2048.
//
// Mapping.  One workgroup (8 waves, two per SIMD) owns one head and 256 query rows; wave
// w owns rows 32w..32w+31, one 32-row tile of the 32x32x16 matrix-core form (on gfx950 it
// issues in about the time of the 16x16x32 form while doing twice the work).  Per key
// block of 64 positions:
//   load  K [64 x 192] and V [64 x 128] bf16 rows and the block's selection-mask words
//         of the 256 rows into LDS with direct global->LDS loads, in a three-stage
//         ring (two blocks in flight while one is computed), 16-byte chunks
//         XOR-swizzled per row (swz_k, swz_v);
//   QK    S^T = K . Q^T per 32-key group (keys as MFMA rows, the wave's 32 queries as 12
//         B operands in registers), so lane l holds query row l % 32 and keys
//         32 kg + 8 (r / 4) + 4 (l / 32) + r % 4;
//   mask  selection bits of the row and the causal bound;
//   softmax per row over its 32 + 32 keys in lanes l and l ^ 32, relative to a fixed
//         reference (below); the numerators stay in registers as the PV A operands:
//         K-slot e of lane half hf in K-step ks of key group kg is key
//         32 kg + 8 (2 ks + e / 4) + 4 hf + e % 4, exactly element 8 ks + e of the lane;
//   PV    O [32 x 128] += P . V in four 32-column groups, V operands by LDS transpose
//         reads.
// No running-maximum rescale: each row's numerators are exp2(logit - m_ref), m_ref the
// maximum of its first key block with a usable key, which is exact in floating point
// while nothing overflows; a logit more than 2^64 above it (log2 units) marks the
// workgroup, which then recomputes its rows with their true maxima as references.
// Heaviest query blocks go first and all query blocks of a head share an XCD, so the
// head's K and V blocks are fetched into one L2.
#include "dsa_device.h"
#include "dsa_internal.h"

namespace dsa {

namespace {

constexpr int kMhaThreads = 512;
constexpr int kMhaWaves = 8;
constexpr int kQB = 32 * kMhaWaves;     // query rows per workgroup (256)
constexpr int kKB = 64;                 // keys per block
constexpr int kDqk = 192;
constexpr int kDvM = 128;
constexpr int kKRow = kDqk * 2;         // 384 bytes
constexpr int kVRow = kDvM * 2;         // 256 bytes
constexpr int kKChunks = kKRow / 16;    // 24
constexpr int kVChunks = kVRow / 16;    // 16
constexpr int kKBytes = kKB * kKRow;    // 24576
constexpr int kVBytes = kKB * kVRow;    // 16384
constexpr int kKLoads = kKBytes / 1024; // 24 wave-wide 1 KB loads
constexpr int kVLoads = kVBytes / 1024; // 16
constexpr int kLoadsPerWave = (kKLoads + kVLoads) / kMhaWaves;   // 5
constexpr int kMaskBytes = kQB * 2 * 4;                          // 2 mask words per row
constexpr int kStageBytes = kKBytes + kVBytes + kMaskBytes;      // 43008
constexpr int kStages = 3;                                       // blocks i, i+1, i+2
constexpr int kDmaPerBlock = kLoadsPerWave + 1;                  // per wave, with the mask
static_assert((kKLoads + kVLoads) % kMhaWaves == 0, "block loads split evenly over the waves");
static_assert(kMaskBytes == kMhaWaves * kWave * 4, "one mask dword per lane");
constexpr float kLog2eM = 1.4426950408889634f;
constexpr float kLn2M = 0.6931471805599453f;
constexpr float kRefSpan = 64.0f;                   // log2 units above the reference

// Stage s: K block [64 x 384 B], V block [64 x 256 B], mask words [256 rows][2].
__shared__ __attribute__((aligned(16))) uint8_t m_stage[kStages * kStageBytes];

typedef __bf16 v4bf_m __attribute__((ext_vector_type(4)));

// LDS swizzles, chosen so that the operand reads are free of bank conflicts (64 banks of
// 4 bytes; a 16-byte read serves 16 lanes per pass, an 8-byte read 32 lanes):
//   K rows (384 B = 24 chunks of 16 bytes): chunk c of key row r sits at c ^ ((r >> 1) & 7),
//     inside its aligned group of 8.  A QK operand read takes one chunk of 16 consecutive
//     rows; rows are 96 dwords apart, so rows of one parity share bank alignment and the
//     XOR gives the 8 rows of each parity distinct 16-byte bank groups.
//   V rows (256 B = 16 chunks = 4 groups of 4): group g of row r sits at g ^ (r & 3).  A
//     transpose read takes one group (32 columns) of 4 consecutive rows per 16 lanes, and
//     rows are 64 dwords apart (all bank-aligned): the XOR puts the 4 rows in distinct
//     quarters of the banks.
__device__ __forceinline__ int swz_k(int row, int chunk) { return chunk ^ ((row >> 1) & 7); }
__device__ __forceinline__ int swz_v(int row, int chunk) { return chunk ^ ((row & 3) << 2); }

__device__ __forceinline__ void dma16(const uint8_t* src, uint32_t lds_addr) {
    const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds_addr);
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" :: "s"(m0v), "v"(src) : "memory");
}

__device__ __forceinline__ void dma4(const uint32_t* src, uint32_t lds_addr) {
    const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds_addr);
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, off" :: "s"(m0v), "v"(src) : "memory");
}

// A wave-uniform pointer, in scalar registers (the scalar-base loads below need it there).
__device__ __forceinline__ const uint8_t* sgpr_ptr(const void* p) {
    const uint64_t a = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a >> 32));
    return reinterpret_cast<const uint8_t*>((static_cast<uint64_t>(hi) << 32) | lo);
}

// The same with a wave-uniform 64-bit base in scalar registers and a 32-bit per-lane offset.
__device__ __forceinline__ void dma16_s(const uint8_t* sbase, uint32_t voff, uint32_t lds_addr) {
    const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds_addr);
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" :: "s"(m0v), "v"(voff), "s"(sbase) : "memory");
}

__device__ __forceinline__ void dma4_s(const uint8_t* sbase, uint32_t voff, uint32_t lds_addr) {
    const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds_addr);
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, %2" :: "s"(m0v), "v"(voff), "s"(sbase) : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const uint8_t*)(p)));
}

// Loads key block [s0, s0 + 64) of head h and the selection-mask words of the block's
// 256 query rows into stage `st`: 5 wave-wide 1 KB loads and one mask dword per lane.
// Rows past the chunk end read the last row (their scores are masked by causality).
__device__ __forceinline__ void load_block(const uint8_t* kbase, const uint8_t* vbase,
                                           const uint32_t* mask_b, int words, int t0, int T,
                                           int H, int h, int s0, uint8_t* st, int wave, int lane) {
    asm volatile("" : "+v"(lane));
    const uint32_t kl = lds_addr(st), vl = kl + kKBytes;
    {
        const int local = 32 * wave + (lane >> 1);
        const int row = min(t0 + local, T - 1);
        const int word = min((s0 >> 5) + (lane & 1), words - 1);
        dma4(mask_b + static_cast<size_t>(row) * words + word, vl + kVBytes + wave * kWave * 4);
    }
    for (int i = 0; i < kLoadsPerWave; ++i) {
        const int ci = wave + kMhaWaves * i;                 // 0..39
        if (ci < kKLoads) {
            const int c = ci * kWave + lane;
            const int key = c / kKChunks;
            const int phys = c - key * kKChunks;
            const int s = min(s0 + key, T - 1);
            const uint8_t* src = kbase + (static_cast<size_t>(s) * H + h) * kKRow + swz_k(key, phys) * 16;
            dma16(src, kl + ci * 1024);
        } else {
            const int cv = ci - kKLoads;
            const int c = cv * kWave + lane;
            const int key = c / kVChunks;
            const int phys = c - key * kVChunks;
            const int s = min(s0 + key, T - 1);
            const uint8_t* src = vbase + (static_cast<size_t>(s) * H + h) * kVRow + swz_v(key, phys) * 16;
            dma16(src, vl + cv * 1024);
        }
    }
}

// Per-lane byte offsets of a wave's block loads relative to the block's first key row,
// the same for every block (wave w issues loads w, w + 8, w + 16 of K and w, w + 8 of V,
// each lane one 16-byte chunk, and one mask dword).  Blocks wholly inside the chunk
// (s0 + 64 <= T) need no clamp and use them with a scalar base; the last, partial block
// takes the clamped loads above.
constexpr int kKPerWave = kKLoads / kMhaWaves;       // 3
constexpr int kVPerWave = kVLoads / kMhaWaves;       // 2
static_assert(kKLoads % kMhaWaves == 0 && kVLoads % kMhaWaves == 0, "K and V loads split evenly");
struct MhaDma {
    uint32_t k[kKPerWave];
    uint32_t v[kVPerWave];
    uint32_t m;
};

__device__ __forceinline__ MhaDma mha_dma(int t0, int T, int H, int words, int wave, int lane) {
    MhaDma d;
#pragma unroll
    for (int i = 0; i < kKPerWave; ++i) {
        const int c = (wave + kMhaWaves * i) * kWave + lane;
        const int key = c / kKChunks;
        const int phys = c - key * kKChunks;
        d.k[i] = static_cast<uint32_t>(key * H * kKRow + swz_k(key, phys) * 16);
        asm volatile("" : "+v"(d.k[i]));
    }
#pragma unroll
    for (int i = 0; i < kVPerWave; ++i) {
        const int c = (wave + kMhaWaves * i) * kWave + lane;
        const int key = c / kVChunks;
        const int phys = c - key * kVChunks;
        d.v[i] = static_cast<uint32_t>(key * H * kVRow + swz_v(key, phys) * 16);
        asm volatile("" : "+v"(d.v[i]));
    }
    const int row = min(t0 + 32 * wave + (lane >> 1), T - 1);
    d.m = static_cast<uint32_t>((row * words + (lane & 1)) * 4);
    asm volatile("" : "+v"(d.m));
    return d;
}

// load_block for a block with s0 + 64 <= T.
__device__ __forceinline__ void load_block_full(const uint8_t* kbase, const uint8_t* vbase,
                                                const uint32_t* mask_b, int H, int h, int s0,
                                                uint8_t* st, int wave, const MhaDma& d) {
    const uint32_t kl = lds_addr(st), vl = kl + kKBytes;
    dma4_s(sgpr_ptr(mask_b + (s0 >> 5)), d.m, vl + kVBytes + wave * kWave * 4);
    const uint8_t* kb = sgpr_ptr(kbase + (static_cast<size_t>(s0) * H + h) * kKRow);
    const uint8_t* vb = sgpr_ptr(vbase + (static_cast<size_t>(s0) * H + h) * kVRow);
#pragma unroll
    for (int i = 0; i < kKPerWave; ++i) dma16_s(kb, d.k[i], kl + (wave + kMhaWaves * i) * 1024);
#pragma unroll
    for (int i = 0; i < kVPerWave; ++i) dma16_s(vb, d.v[i], vl + (wave + kMhaWaves * i) * 1024);
}

__device__ __forceinline__ void lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

struct MhaState {
    v8bf qreg[kDqk / 16];       // 12 K-steps of 16 dims: row l % 32, dims 16 ks + 8 (l / 32)
    v16f o[kDvM / 32];          // four 32-column groups
    float m_ref, m_max, l_run;  // of row l % 32 (log2 units)
    bool over;
};

// Lane-invariant LDS byte offsets within a stage, computed once per workgroup (each block
// then adds only its stage base; the rest of a K read's address is an instruction
// immediate).
//   K: key 32 kg + r32, 16-byte chunk 2 ks + hf at position (2 ks + hf) ^ z, z = (r32 >> 1)
//      & 7 (= (key >> 1) & 7); for ks = 4 j + i that is 8 j + ((2 i + hf) ^ z), so koff[i] =
//      384 r32 + 16 ((2 i + hf) ^ z) and the read of (ks, kg) is koff[ks % 4] + 12288 kg +
//      128 (ks / 4).
//   V: key 32 kg + 16 ks + 8 e4 + sv, sv = 4 hf + m / 4 (key & 3 = m / 4), chunk 4 dg + c0,
//      c0 = 2 ch + (m % 4) / 2, at position 4 (dg ^ m / 4) + c0, so voff[dg] = 256 sv +
//      64 (dg ^ m / 4) + 16 c0 + 8 (m % 2) and the read of (dg, kg, ks, e4) is voff[dg] +
//      256 (32 kg + 16 ks + 8 e4).
//   mask: the two words of row 32 wave + r32.
struct MhaLane {
    uint32_t koff[4];
    uint32_t voff[4];
    uint32_t moff;
    int hf, r32;
};

__device__ __forceinline__ MhaLane mha_lane(int wave, int lane) {
    MhaLane ml;
    ml.hf = lane >> 5;
    ml.r32 = lane & 31;
    const int s = (ml.r32 >> 1) & 7;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        ml.koff[i] = static_cast<uint32_t>(kKRow * ml.r32 + 16 * ((2 * i + ml.hf) ^ s));
        asm volatile("" : "+v"(ml.koff[i]));      // kept, not recomputed per block
    }
    const int m = lane & 15;
    const int ch = (lane >> 4) & 1;
    const int sv = 4 * ml.hf + (m >> 2);
    const int c0 = 2 * ch + ((m & 3) >> 1);
#pragma unroll
    for (int dg = 0; dg < 4; ++dg) {
        ml.voff[dg] = static_cast<uint32_t>(kKBytes + kVRow * sv + 64 * (dg ^ (m >> 2)) + 16 * c0 + 8 * (m & 1));
        asm volatile("" : "+v"(ml.voff[dg]));
    }
    ml.moff = static_cast<uint32_t>(kKBytes + kVBytes + 8 * (32 * wave + ml.r32));
    asm volatile("" : "+v"(ml.moff));
    return ml;
}

__device__ __forceinline__ void mha_block(MhaState& st, const uint8_t* stage, const MhaLane& ml, int t_row,
                                          int s0, float scale_log2, bool fixed) {
    const int hf = ml.hf;
    const uint2 mw = *reinterpret_cast<const uint2*>(stage + ml.moff);

    // ---- S^T = K . Q^T for the two 32-key groups: independent accumulation chains
    v16f sacc[2];
#pragma unroll
    for (int kg = 0; kg < 2; ++kg)
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[kg][r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < kDqk / 16; ++ks) {
#pragma unroll
        for (int kg = 0; kg < 2; ++kg) {
            const v8bf a = *reinterpret_cast<const v8bf*>(stage + ml.koff[ks & 3] + 32 * kKRow * kg + 128 * (ks >> 2));
            sacc[kg] = mfma_bf16_32x32x16(a, st.qreg[ks], sacc[kg]);
        }
    }
    // ---- mask + softmax numerators; keys s0 + 32 kg + 8 (r / 4) + 4 hf + r % 4.  The
    // selection word of each key group is cut to the causal bound once, then shifted so
    // that the lane's keys sit at the fixed bits 8 (r / 4) + r % 4.
    float mx = -INFINITY;
#pragma unroll
    for (int kg = 0; kg < 2; ++kg) {
        const int lim = t_row - s0 - 32 * kg;                    // last visible key of the group
        const uint32_t vis = lim >= 31 ? 0xffffffffu : (lim < 0 ? 0u : (2u << lim) - 1u);
        const uint32_t word = ((kg ? mw.y : mw.x) & vis) >> (4 * hf);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            // all ones where the key is usable, else zero (a sign-extended one-bit field),
            // then one bitwise select between the (unscaled) logit and -inf
            const int bit = 8 * (r >> 2) + (r & 3);
            const uint32_t keep = static_cast<uint32_t>(static_cast<int32_t>(word << (31 - bit)) >> 31);
            const float v = __uint_as_float((__float_as_uint(sacc[kg][r]) & keep) | (0xff800000u & ~keep));
            sacc[kg][r] = v;
            mx = fmaxf(mx, v);
        }
    }
    // the logits stay unscaled: the maximum is scaled once (the scale is positive, so it
    // commutes with the maximum) and each numerator takes one fma before its exp2
    mx = max_xor32(mx) * scale_log2;
    if (!fixed) {
        if (st.m_ref == -INFINITY) st.m_ref = mx;       // first block with a usable key
        st.m_max = fmaxf(st.m_max, mx);
        st.over = st.over || mx > st.m_ref + kRefSpan;
    }
    // while no usable key has been seen every logit is -inf: any finite reference gives 0
    const float mref = st.m_ref == -INFINITY ? 0.f : st.m_ref;
    v8s pk[2][2];
    float psum = 0.f;
#pragma unroll
    for (int kg = 0; kg < 2; ++kg)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float p = exp2_num(fmaf(sacc[kg][r], scale_log2, -mref));
            psum += p;
            pk[kg][r >> 3][r & 7] = static_cast<short>(f32_to_bf16(p));
        }
    st.l_run += sum_xor32(psum);

    // ---- O += P . V.  V operand of (kg, ks), lane l: column 32 dg + l % 32, keys
    // 32 kg + 16 ks + 8 e4 + 4 hf + 0..3 (e4 = 0, 1), two transpose reads: lane m of a
    // 16-lane group supplies row key0 + m / 4, columns d0 + 4 (m % 4) .. + 3.
#pragma unroll
    for (int dg = 0; dg < kDvM / 32; ++dg) {
#pragma unroll
        for (int kg = 0; kg < 2; ++kg)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                v4bf_m half[2];
#pragma unroll
                for (int e4 = 0; e4 < 2; ++e4) {
                    const uint8_t* src = stage + ml.voff[dg] + kVRow * (32 * kg + 16 * ks + 8 * e4);
                    half[e4] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                        (__attribute__((address_space(3))) v4bf_m*)(src));
                }
                const v8bf vop = v8bf{half[0][0], half[0][1], half[0][2], half[0][3],
                                      half[1][0], half[1][1], half[1][2], half[1][3]};
                st.o[dg] = mfma_bf16_32x32x16(__builtin_bit_cast(v8bf, pk[kg][ks]), vop, st.o[dg]);
            }
    }
}

// per-wave row statistics for the epilogue and the recompute flags
__shared__ float m_rowl[kMhaWaves][32];
__shared__ float m_rowm[kMhaWaves][32];
__shared__ int32_t m_redo[kMhaWaves];

__global__ __launch_bounds__(kMhaThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void mha_prefill_mfma_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                             const uint16_t* __restrict__ v, const uint32_t* __restrict__ mask,
                             int B, int T, int H, float scale_log2, uint16_t* __restrict__ out,
                             float* __restrict__ lse)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int qblocks = (T + kQB - 1) / kQB;
    // Block j * (B H) + bh: heaviest query blocks (most key blocks under the causal
    // bound) first, and all query blocks of a head on one XCD (workgroups go round robin
    // over the 8 XCDs, B H being a multiple of 8 at the model's head counts), so the
    // head's K and V blocks are fetched into one L2 and shared there.
    const int qb = qblocks - 1 - static_cast<int>(blockIdx.x / (B * H));
    const int bh = static_cast<int>(blockIdx.x % (B * H));
    const int h = bh % H;
    const int b = bh / H;
    const int t0 = qb * kQB;
    const int words = (T + 31) / 32;

    const int t_row = min(t0 + 32 * wave + (lane & 31), T - 1);   // query row of this lane
    MhaState st;
    {
        const uint16_t* qrow = q + ((static_cast<size_t>(b) * T + t_row) * H + h) * kDqk + 8 * (lane >> 5);
#pragma unroll
        for (int ks = 0; ks < kDqk / 16; ++ks) st.qreg[ks] = *reinterpret_cast<const v8bf*>(qrow + 16 * ks);
    }
    st.m_ref = -INFINITY;
    st.m_max = -INFINITY;
    st.over = false;

    const uint8_t* kbase = reinterpret_cast<const uint8_t*>(k) + static_cast<size_t>(b) * T * H * kKRow;
    const uint8_t* vbase = reinterpret_cast<const uint8_t*>(v) + static_cast<size_t>(b) * T * H * kVRow;
    const uint32_t* mask_b = mask + static_cast<size_t>(b) * T * words;
    const int t_last = min(t0 + kQB, T) - 1;
    const int nblocks = t_last / kKB + 1;                    // causal: key blocks up to t_last

    // Three-stage ring: step j waits for block j (block j + 1 stays in flight), passes
    // one barrier (block j visible; stage of block j - 1 free), puts block j + 2 in
    // flight and computes block j.  The queries' own loads were issued first, so the
    // compiler's wait for them (it cannot see the direct-to-LDS loads) is the only
    // full drain, at the first block.
    auto stage = [&](int j) { return m_stage + (j % kStages) * kStageBytes; };
    const MhaLane ml = mha_lane(wave, lane);
    const MhaDma dma = mha_dma(t0, T, H, words, wave, lane);
    // the per-lane offsets are 32-bit: key rows up to 64 H apart, mask rows up to T words
    const bool offsets32 = static_cast<long long>(kKB) * H * kKRow < (1ll << 31) &&
                           static_cast<long long>(T) * words * 4 < (1ll << 31);
    auto sweep = [&](bool fixed) {
#pragma unroll
        for (int dg = 0; dg < kDvM / 32; ++dg)
#pragma unroll
            for (int r = 0; r < 16; ++r) st.o[dg][r] = 0.f;
        st.l_run = 0.f;
        auto issue = [&](int j) {
            const int s0 = j * kKB;
            if (s0 + kKB <= T && offsets32) load_block_full(kbase, vbase, mask_b, H, h, s0, stage(j), wave, dma);
            else load_block(kbase, vbase, mask_b, words, t0, T, H, h, s0, stage(j), wave, lane);
        };
        issue(0);
        if (nblocks > 1) issue(1);
        for (int j = 0; j < nblocks; ++j) {
            if (j + 1 < nblocks) asm volatile("s_waitcnt vmcnt(%0)" :: "n"(kDmaPerBlock) : "memory");
            else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            lds_sync();
            if (j + 2 < nblocks) issue(j + 2);
            mha_block(st, stage(j), ml, t_row, j * kKB, scale_log2, fixed);
        }
    };
    sweep(false);
    // a row of the workgroup past its reference span: recompute the workgroup's rows
    // from their true maxima (a uniform decision: every wave reads the same flags)
    if (lane == 0) m_redo[wave] = __ballot(st.over) != 0ull;
    __syncthreads();
    int redo = 0;
#pragma unroll
    for (int w = 0; w < kMhaWaves; ++w) redo |= m_redo[w];
    if (redo) {
        st.m_ref = st.m_max;
        __syncthreads();      // every wave has read the flags and left the ring
        sweep(true);
    }

    // ---- epilogue: element r of lane l in column group dg is row 8 (r / 4) + 4 (l / 32)
    // + r % 4 of the wave's 32, column 32 dg + l % 32; the rows' sums come from the lanes
    // that own them through this wave's own LDS slots (no other wave reads them)
    if (lane < 32) {
        m_rowl[wave][lane] = st.l_run;
        m_rowm[wave][lane] = st.m_ref;
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int rr = 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int t = t0 + 32 * wave + rr;
        const float l = m_rowl[wave][rr];
        const float inv = l > 0.f ? recip(l) : 0.f;
        if (t < T) {
            uint16_t* orow = out + ((static_cast<size_t>(b) * T + t) * H + h) * kDvM;
#pragma unroll
            for (int dg = 0; dg < kDvM / 32; ++dg) orow[32 * dg + (lane & 31)] = f32_to_bf16(st.o[dg][r] * inv);
        }
    }
    if (lse && lane < 32) {
        const int t = t0 + 32 * wave + lane;
        const float l = st.l_run;
        if (t < T) lse[(static_cast<size_t>(b) * T + t) * H + h] = l > 0.f ? (st.m_ref + log2f(l)) * kLn2M : -INFINITY;
    }
}

// Bit s of row (b,t) <- s is among idx[b,t,:] and s <= t.  One workgroup per row.
__global__ __launch_bounds__(256)
void select_mask_kernel(const int32_t* __restrict__ idx, int T, int k, uint32_t* __restrict__ mask)
{
    extern __shared__ uint32_t bits[];
    const int row = blockIdx.x;
    const int t = row % T;
    const int words = (T + 31) / 32;
    for (int i = threadIdx.x; i < words; i += blockDim.x) bits[i] = 0u;
    __syncthreads();
    const int32_t* sel = idx + static_cast<size_t>(row) * k;
    for (int j = threadIdx.x; j < k; j += blockDim.x) {
        const int s = sel[j];
        if (s >= 0 && s <= t) atomicOr(&bits[s >> 5], 1u << (s & 31));
    }
    __syncthreads();
    for (int i = threadIdx.x; i < words; i += blockDim.x) mask[static_cast<size_t>(row) * words + i] = bits[i];
}

}  // namespace

bool mha_prefill_mfma_supported(int Dqk, int Dv, int bf16) { return bf16 && Dqk == kDqk && Dv == kDvM; }
// The kernel takes each block's maximum over the unscaled logits and scales it once, which
// needs a positive scale (NaN fails both comparisons).
bool mha_prefill_mfma_path(int Dqk, int Dv, int bf16, float sm_scale) {
    return mha_prefill_mfma_supported(Dqk, Dv, bf16) && sm_scale > 0.f && sm_scale < INFINITY;
}

size_t mha_prefill_workspace_bytes(int B, int T) {
    return static_cast<size_t>(B) * T * ((T + 31) / 32) * sizeof(uint32_t) + 256;
}

hipError_t launch_mha_prefill_mfma(const void* q, const void* k, const void* v, const int32_t* idx,
                                   int B, int T, int H, int topk, float sm_scale, void* out,
                                   float* lse, void* ws, hipStream_t stream) {
    uint32_t* mask = static_cast<uint32_t*>(ws);
    const int words = (T + 31) / 32;
    // the selection's bit mask is timed with the top-k (it turns the selection into the
    // attention's operand form)
    hipError_t e = launch_kernel(kPhaseTopk, select_mask_kernel, dim3(B * T), dim3(256),
                                 static_cast<uint32_t>(words * sizeof(uint32_t)), stream, idx, T, topk, mask);
    if (e != hipSuccess) return e;
    const int qblocks = (T + kQB - 1) / kQB;
    return launch_kernel(kPhaseAttention, mha_prefill_mfma_kernel, dim3(B * H * qblocks), dim3(kMhaThreads), 0,
                         stream, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                         static_cast<const uint16_t*>(v), mask, B, T, H, sm_scale * kLog2eM,
                         static_cast<uint16_t*>(out), lse);
}

}  // namespace dsa
