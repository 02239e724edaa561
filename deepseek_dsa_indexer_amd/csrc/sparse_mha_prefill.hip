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
// w owns rows 32w..32w+31 as two 16-row query tiles, so every K and V operand read from
// LDS feeds two matrix-core products.  Per key block of 64 positions:
//   load  K [64 x 192] and V [64 x 128] bf16 rows and the block's selection-mask words
//         of the 256 rows into LDS with direct global->LDS loads, in a three-stage
//         ring (two blocks in flight while one is computed), 16-byte chunks
//         XOR-swizzled per row;
//   QK    S^T = K . Q^T (keys as MFMA rows, each query tile's 16 queries as 6 B
//         operands in registers), so lane (g, n) holds query row n of the tile and keys
//         16 kt + 4 g + i;
//   mask  selection bits of the row and the causal bound;
//   softmax online per row, entirely in the wave; the probabilities stay in registers
//         in the A-operand layout of the PV product;
//   PV    O [32 x 128] += P . V, V operands by LDS transpose reads.
// Heaviest query blocks go first and all query blocks of a head share an XCD, so the
// head's K and V blocks are fetched into one L2.
#include "dsa_device.h"
#include "dsa_internal.h"

namespace dsa {

namespace {

constexpr int kMhaThreads = 512;
constexpr int kMhaWaves = 8;
constexpr int kQT = 2;                  // 16-row query tiles per wave
constexpr int kQB = 16 * kQT * kMhaWaves;   // query rows per workgroup (256)
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
constexpr float kLazy = 8.0f;

// Stage s: K block [64 x 384 B], V block [64 x 256 B], mask words [256 rows][2].
__shared__ __attribute__((aligned(16))) uint8_t m_stage[kStages * kStageBytes];

typedef __bf16 v4bf_m __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int swz8(int row, int chunk) { return chunk ^ (row & 7); }

__device__ __forceinline__ void dma16(const uint8_t* src, uint32_t lds_addr) {
    const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds_addr);
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" :: "s"(m0v), "v"(src) : "memory");
}

__device__ __forceinline__ void dma4(const uint32_t* src, uint32_t lds_addr) {
    const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds_addr);
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, off" :: "s"(m0v), "v"(src) : "memory");
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
            const uint8_t* src = kbase + (static_cast<size_t>(s) * H + h) * kKRow + swz8(key, phys) * 16;
            dma16(src, kl + ci * 1024);
        } else {
            const int cv = ci - kKLoads;
            const int c = cv * kWave + lane;
            const int key = c / kVChunks;
            const int phys = c - key * kVChunks;
            const int s = min(s0 + key, T - 1);
            const uint8_t* src = vbase + (static_cast<size_t>(s) * H + h) * kVRow + swz8(key, phys) * 16;
            dma16(src, vl + cv * 1024);
        }
    }
}

__device__ __forceinline__ void lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

struct MhaState {
    v8bf qreg[kQT][kDqk / 32];  // 6 K-steps per query tile
    v4f o[kQT][kDvM / 16];      // 8 column tiles per query tile
    float m_run[kQT], l_run[kQT];
};

__device__ __forceinline__ void mha_block(MhaState& st, const uint8_t* stage, const int (&t_row)[kQT],
                                          int s0, float scale_log2, int wave, int lane) {
    const uint8_t* kb = stage;
    const uint8_t* vb = stage + kKBytes;
    const uint32_t* mk = reinterpret_cast<const uint32_t*>(stage + kKBytes + kVBytes);
    int lo = lane;
    asm volatile("" : "+v"(lo));
    const int g = lo >> 4;
    const int n = lo & 15;
    uint32_t mw[kQT][2];
#pragma unroll
    for (int qt = 0; qt < kQT; ++qt) {
        const uint2 m2 = *reinterpret_cast<const uint2*>(mk + 2 * (32 * wave + 16 * qt + n));
        mw[qt][0] = m2.x;
        mw[qt][1] = m2.y;
    }

    // ---- S^T = K . Q^T: 4 key tiles x 6 K-steps, each K operand used by both query tiles
    v4f sacc[kQT][4];
#pragma unroll
    for (int qt = 0; qt < kQT; ++qt)
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) sacc[qt][kt] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ds = 0; ds < kDqk / 32; ++ds) {
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
            const int key = 16 * kt + n;
            const v8bf a = *reinterpret_cast<const v8bf*>(kb + key * kKRow + swz8(key, ds * 4 + g) * 16);
#pragma unroll
            for (int qt = 0; qt < kQT; ++qt) sacc[qt][kt] = mfma_bf16_16x16x32(a, st.qreg[qt][ds], sacc[qt][kt]);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    // ---- mask + online softmax per query tile; keys s0 + 16 kt + 4 g + i
    v8s pk[kQT][2];
#pragma unroll
    for (int qt = 0; qt < kQT; ++qt) {
        float sv[16];
        float mx = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int kk = 16 * kt + 4 * g + i;              // 0..63
                const uint32_t word = kk < 32 ? mw[qt][0] : mw[qt][1];
                const bool sel = (word >> (kk & 31)) & 1u;
                const bool vis = s0 + kk <= t_row[qt];
                const float v = (sel && vis) ? sacc[qt][kt][i] * scale_log2 : -INFINITY;
                sv[4 * kt + i] = v;
                mx = fmaxf(mx, v);
            }
        mx = max_xor32(max_xor16(mx));
        float alpha = 1.f;
        if (mx > st.m_run[qt] + kLazy) {
            // nothing accumulated yet (O = 0, l = 0): no rescale needed
            alpha = (st.m_run[qt] == -INFINITY) ? 1.f : exp2f(st.m_run[qt] - mx);
            st.m_run[qt] = mx;
        }
        float psum = 0.f;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const float p = (sv[j] == -INFINITY) ? 0.f : exp2f(sv[j] - st.m_run[qt]);
            psum += p;
            pk[qt][j >> 3][j & 7] = static_cast<short>(f32_to_bf16(p));
        }
        psum = sum_xor32(sum_xor16(psum));
        st.l_run[qt] = st.l_run[qt] * alpha + psum;
        // alpha is per query row n: the O rows of this lane are rows 4 g + i, held by
        // lanes n' = 4 g + i; fetch their alphas
        if (__ballot(alpha != 1.f)) {
            float a4[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) a4[i] = __shfl(alpha, 4 * g + i, kWave);
#pragma unroll
            for (int dt = 0; dt < kDvM / 16; ++dt)
#pragma unroll
                for (int i = 0; i < 4; ++i) st.o[qt][dt][i] *= a4[i];
        }
    }
    // ---- O += P . V: K-step 0 covers keys of tiles 0, 1 (slots j = 4 kt + i), K-step 1
    // tiles 2, 3.  V operand of K-step ks: rows 32 ks + 16 kk + 4 g + r (kk = 0, 1).
#pragma unroll
    for (int dt = 0; dt < kDvM / 16; ++dt) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            v4bf_m half[2];
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const int key = 32 * ks + 16 * kk + 4 * g + (n >> 2);
                const int chunk = 2 * dt + ((n & 3) >> 1);
                const int off = key * kVRow + swz8(key, chunk) * 16 + (n & 1) * 8;
                half[kk] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) v4bf_m*)(vb + off));
            }
            const v8bf vop = v8bf{half[0][0], half[0][1], half[0][2], half[0][3],
                                  half[1][0], half[1][1], half[1][2], half[1][3]};
#pragma unroll
            for (int qt = 0; qt < kQT; ++qt)
                st.o[qt][dt] = mfma_bf16_16x16x32(__builtin_bit_cast(v8bf, pk[qt][ks]), vop, st.o[qt][dt]);
        }
    }
}

__global__ __launch_bounds__(kMhaThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void mha_prefill_mfma_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                             const uint16_t* __restrict__ v, const uint32_t* __restrict__ mask,
                             int B, int T, int H, float scale_log2, uint16_t* __restrict__ out,
                             float* __restrict__ lse)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int g = lane >> 4;
    const int n = lane & 15;
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

    int t_row[kQT];                         // query row of this lane in each tile
    MhaState st;
#pragma unroll
    for (int qt = 0; qt < kQT; ++qt) {
        t_row[qt] = min(t0 + 32 * wave + 16 * qt + n, T - 1);
        const uint16_t* qrow = q + ((static_cast<size_t>(b) * T + t_row[qt]) * H + h) * kDqk + 8 * g;
#pragma unroll
        for (int ds = 0; ds < kDqk / 32; ++ds) st.qreg[qt][ds] = *reinterpret_cast<const v8bf*>(qrow + 32 * ds);
#pragma unroll
        for (int dt = 0; dt < kDvM / 16; ++dt) st.o[qt][dt] = v4f{0.f, 0.f, 0.f, 0.f};
        st.m_run[qt] = -INFINITY;
        st.l_run[qt] = 0.f;
    }

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
    load_block(kbase, vbase, mask_b, words, t0, T, H, h, 0, stage(0), wave, lane);
    if (nblocks > 1) load_block(kbase, vbase, mask_b, words, t0, T, H, h, kKB, stage(1), wave, lane);
    for (int j = 0; j < nblocks; ++j) {
        if (j + 1 < nblocks) asm volatile("s_waitcnt vmcnt(%0)" :: "n"(kDmaPerBlock) : "memory");
        else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        lds_sync();
        if (j + 2 < nblocks)
            load_block(kbase, vbase, mask_b, words, t0, T, H, h, (j + 2) * kKB, stage(j + 2), wave, lane);
        mha_block(st, stage(j), t_row, j * kKB, scale_log2, wave, lane);
    }

    // ---- epilogue: rows 4 g + i of each query tile; l and m of row r sit in lane r
#pragma unroll
    for (int qt = 0; qt < kQT; ++qt) {
        float inv4[4], lse4[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float l = __shfl(st.l_run[qt], 4 * g + i, kWave);
            const float m = __shfl(st.m_run[qt], 4 * g + i, kWave);
            inv4[i] = l > 0.f ? recip(l) : 0.f;
            lse4[i] = l > 0.f ? (m + log2f(l)) * kLn2M : -INFINITY;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = t0 + 32 * wave + 16 * qt + 4 * g + i;
            if (t >= T) continue;
            uint16_t* orow = out + ((static_cast<size_t>(b) * T + t) * H + h) * kDvM;
#pragma unroll
            for (int dt = 0; dt < kDvM / 16; ++dt) orow[16 * dt + n] = f32_to_bf16(st.o[qt][dt][i] * inv4[i]);
            if (lse && n == 0) lse[(static_cast<size_t>(b) * T + t) * H + h] = lse4[i];
        }
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

size_t mha_prefill_workspace_bytes(int B, int T) {
    return static_cast<size_t>(B) * T * ((T + 31) / 32) * sizeof(uint32_t) + 256;
}

hipError_t launch_mha_prefill_mfma(const void* q, const void* k, const void* v, const int32_t* idx,
                                   int B, int T, int H, int topk, float sm_scale, void* out,
                                   float* lse, void* ws, hipStream_t stream) {
    uint32_t* mask = static_cast<uint32_t*>(ws);
    const int words = (T + 31) / 32;
    hipLaunchKernelGGL(select_mask_kernel, dim3(B * T), dim3(256), words * sizeof(uint32_t), stream,
                       idx, T, topk, mask);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int qblocks = (T + kQB - 1) / kQB;
    hipLaunchKernelGGL(mha_prefill_mfma_kernel, dim3(B * H * qblocks), dim3(kMhaThreads), 0, stream,
                       static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                       static_cast<const uint16_t*>(v), mask, B, T, H, sm_scale * kLog2eM,
                       static_cast<uint16_t*>(out), lse);
    return hipGetLastError();
}

}  // namespace dsa
