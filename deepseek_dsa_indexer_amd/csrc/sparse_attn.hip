// sparse_attn.hip -- sparse attention over the top-k selected positions.
//
// Two paths:
//  * mla_decode_mfma_kernel: the absorbed (MQA) latent form of "dsa-indexer.excalidraw"
//    ("core attention, MQA mode: q (128 heads) over the 2048 selected latents, each
//    latent is key and value") at the V3.2 shape: bf16, 576-wide rows (latent 512 then
//    rope 64), values = the first 512 columns, up to 128 heads, bf16 matrix cores.
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
    const int pos = a.len ? min(a.len[b], a.kv_rows) - a.T + t : t;
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
            const size_t koff = (static_cast<size_t>(b) * a.kv_rows + s) * a.row_stride +
                                static_cast<size_t>(h) * a.head_stride;
            float acc = 0.f;
            for (int d = 0; d < a.Dk; ++d) acc += qs[d] * ld_elem(a.kbase, koff + d, a.bf16);
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
// One workgroup (4 waves, one wave per SIMD) owns one query row (b,t), one split of its
// k slots and one group of 64 heads.  Per tile of 32 selected positions:
//   gather   32 rows -> LDS with direct global->LDS 16-byte loads, double buffered; the
//            16-byte chunks of each row are XOR-swizzled inside 128-byte groups so the
//            matrix-core operand reads spread over the LDS banks;
//   QK       wave w computes S^T = K . Q^T for heads 16w..16w+15 of the group (keys as
//            MFMA rows; the wave's queries stay in registers as 18 B operands);
//   softmax  online, per head, with lazy rescaling: the running maximum only moves when
//            a tile exceeds it by more than 2^8, so the accumulators are rarely touched;
//            bf16 probabilities go to LDS already in MFMA operand layout;
//   PV       wave w owns output columns 128w..128w+127 for the group's 64 heads:
//            O += P . V with V read from the same LDS tile (the value is the first 512
//            columns of the latent row).
// The two head groups of a (row, split) are given block ids 8 apart, which the
// dispatcher places on the same XCD, so the second gather of each latent row is
// served by that XCD's L2.  Splits of one row are merged by a log-sum-exp combine.
constexpr int kMlaThreads = 256;
constexpr int kMlaWaves = 4;
constexpr int kHeadsPerGroup = 64;
constexpr int kNht = kHeadsPerGroup / 16;          // head tiles per workgroup
constexpr int kDq = 576;
constexpr int kDv = 512;
constexpr int kRowBytes = kDq * 2;                 // 1152
constexpr int kRowChunks = kRowBytes / 16;         // 72
constexpr int kKt = 32;                            // selected positions per tile
constexpr int kTileBytes = kKt * kRowBytes;        // 36864
constexpr int kTileLoads = kTileBytes / (kWave * 16);   // 36 wave-wide 1 KB loads
constexpr int kMaxSlots = 2048;                    // slots per split held in LDS
constexpr int kDs = kDq / 32;                      // 18 K-steps of the QK product
constexpr int kDt = kDv / kMlaWaves / 16;          // 8 output column tiles per wave
constexpr int kXcds = 8;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLazyRescale = 8.0f;               // log2 units

__device__ __forceinline__ int swz_chunk(int key, int chunk) { return chunk ^ (key & 7); }

__global__ __launch_bounds__(kMlaThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void mla_decode_mfma_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ latent,
                            const int32_t* __restrict__ idx, const int32_t* __restrict__ len,
                            int T, int H, int Lmax, int k, int tiles_per_split, int n_splits,
                            int n_units, float scale_log2, uint16_t* __restrict__ out,
                            float* __restrict__ lse, float* __restrict__ part_o,
                            float* __restrict__ part_lse)
{
    __shared__ __attribute__((aligned(16))) uint8_t kbuf[2 * kTileBytes];
    __shared__ __attribute__((aligned(16))) uint8_t pbuf[kNht][kWave][16];
    __shared__ __attribute__((aligned(16))) float alpha_s[kHeadsPerGroup];
    __shared__ int32_t rescale_s[kNht];
    __shared__ float m_s[kHeadsPerGroup];
    __shared__ float l_s[kHeadsPerGroup];
    __shared__ int32_t keys_s[kMaxSlots];

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int g = lane >> 4;
    const int n = lane & 15;

    // block id -> (unit = row * n_splits + split, head group); groups of a unit share an XCD
    const int n_groups = H / kHeadsPerGroup;
    int unit, hg;
    {
        const int x = blockIdx.x;
        const int xcd = x % kXcds;
        const int local = x / kXcds;
        hg = local % n_groups;
        unit = (local / n_groups) * kXcds + xcd;
    }
    if (unit >= n_units) return;
    const int row = unit / n_splits;
    const int split = unit - row * n_splits;
    const int b = row / T;
    const int t = row - b * T;
    const int pos = min(len[b], Lmax) - T + t;
    const int head0 = hg * kHeadsPerGroup;

    const int n_tiles_total = (k + kKt - 1) / kKt;
    const int tile0 = split * tiles_per_split;
    const int n_tiles = max(0, min(tiles_per_split, n_tiles_total - tile0));
    const int nslots = n_tiles * kKt;

    // selected positions of this split (-1: unused slot or not visible)
    const int32_t* sel = idx + static_cast<size_t>(row) * k;
    for (int j = threadIdx.x; j < nslots; j += kMlaThreads) {
        const int slot = tile0 * kKt + j;
        const int s = slot < k ? sel[slot] : -1;
        keys_s[j] = (s >= 0 && s <= pos) ? s : -1;
    }

    // this wave's queries as MFMA B operands: head head0 + 16*wave + n, dims 32*ds + 8*g ..
    v8bf qreg[kDs];
    {
        const uint16_t* qrow = q + (static_cast<size_t>(row) * H + head0 + 16 * wave + n) * kDq + 8 * g;
#pragma unroll
        for (int ds = 0; ds < kDs; ++ds) qreg[ds] = *reinterpret_cast<const v8bf*>(qrow + 32 * ds);
    }

    v4f o[kNht][kDt];
#pragma unroll
    for (int ht = 0; ht < kNht; ++ht)
#pragma unroll
        for (int dt = 0; dt < kDt; ++dt) o[ht][dt] = v4f{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;

    const uint8_t* lat_b = reinterpret_cast<const uint8_t*>(latent) +
                           static_cast<size_t>(b) * Lmax * kRowBytes;
    __syncthreads();     // keys_s ready

    auto gather = [&](int ti, uint8_t* dst) {
        for (int ci = wave; ci < kTileLoads; ci += kMlaWaves) {
            const int c = ci * kWave + lane;
            const int key = c / kRowChunks;
            const int phys = c - key * kRowChunks;
            int s = keys_s[ti * kKt + key];
            s = s < 0 ? 0 : s;                       // unused slots read row 0 (masked later)
            const uint8_t* src = lat_b + static_cast<size_t>(s) * kRowBytes +
                                 swz_chunk(key, phys) * 16;
            __builtin_amdgcn_global_load_lds(
                (const __attribute__((address_space(1))) void*)(src),
                (__attribute__((address_space(3))) void*)(dst + ci * kWave * 16),
                16, 0, 0);
        }
    };

    if (n_tiles > 0) gather(0, kbuf);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();

    for (int ti = 0; ti < n_tiles; ++ti) {
        const uint8_t* kb = kbuf + (ti & 1) * kTileBytes;
        if (ti + 1 < n_tiles) gather(ti + 1, kbuf + ((ti + 1) & 1) * kTileBytes);

        // ---- QK for this wave's 16 heads (keys as rows) + online softmax
        {
            v4f sacc[2] = {v4f{0.f, 0.f, 0.f, 0.f}, v4f{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
            for (int ds = 0; ds < kDs; ++ds) {
#pragma unroll
                for (int kt = 0; kt < 2; ++kt) {
                    const int key = kt * 16 + n;
                    const v8bf a = *reinterpret_cast<const v8bf*>(
                        kb + key * kRowBytes + swz_chunk(key, ds * 4 + g) * 16);
                    sacc[kt] = mfma_bf16_16x16x32(a, qreg[ds], sacc[kt]);
                }
            }
            float sv[8];
            float mx = -INFINITY;
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const bool valid = keys_s[ti * kKt + kt * 16 + 4 * g + i] >= 0;
                    const float v = valid ? sacc[kt][i] * scale_log2 : -INFINITY;
                    sv[kt * 4 + i] = v;
                    mx = fmaxf(mx, v);
                }
            mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
            mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
            // move the running maximum only when this tile exceeds it by > 2^8
            float alpha = 1.f;
            if (mx > m_run + kLazyRescale) {
                alpha = (m_run == -INFINITY) ? 0.f : exp2f(m_run - mx);
                m_run = mx;
            }
            float psum = 0.f;
            v8s pk;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float p = (sv[j] == -INFINITY) ? 0.f : exp2f(sv[j] - m_run);
                psum += p;
                pk[j] = static_cast<short>(f32_to_bf16(p));
            }
            psum += __shfl_xor(psum, 16, kWave);
            psum += __shfl_xor(psum, 32, kWave);
            l_run = l_run * alpha + psum;
            *reinterpret_cast<v8s*>(&pbuf[wave][lane][0]) = pk;
            if (g == 0) alpha_s[16 * wave + n] = alpha;
            // the head tile's accumulators need rescaling when any alpha != 1
            const unsigned long long any = __ballot(alpha != 1.f);
            if (lane == 0) rescale_s[wave] = any != 0ull;
        }
        __syncthreads();

        // ---- PV: this wave's 128 output columns for the group's heads
        {
#pragma unroll
            for (int ht = 0; ht < kNht; ++ht) {
                if (rescale_s[ht]) {
                    const float4 al = *reinterpret_cast<const float4*>(&alpha_s[16 * ht + 4 * g]);
#pragma unroll
                    for (int dt = 0; dt < kDt; ++dt) {
                        o[ht][dt][0] *= al.x; o[ht][dt][1] *= al.y;
                        o[ht][dt][2] *= al.z; o[ht][dt][3] *= al.w;
                    }
                }
            }
            v8bf pa[kNht];
#pragma unroll
            for (int ht = 0; ht < kNht; ++ht) pa[ht] = *reinterpret_cast<const v8bf*>(&pbuf[ht][lane][0]);
#pragma unroll
            for (int dt = 0; dt < kDt; ++dt) {
                const int d = 128 * wave + 16 * dt + n;
                const int chunk = d >> 3;
                const int sub = (d & 7) * 2;
                v8s tmp;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int key = (j >> 2) * 16 + 4 * g + (j & 3);
                    tmp[j] = *reinterpret_cast<const short*>(
                        kb + key * kRowBytes + swz_chunk(key, chunk) * 16 + sub);
                }
                const v8bf vb = __builtin_bit_cast(v8bf, tmp);
#pragma unroll
                for (int ht = 0; ht < kNht; ++ht) o[ht][dt] = mfma_bf16_16x16x32(pa[ht], vb, o[ht][dt]);
            }
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
    }

    // ---- epilogue: normalise, then write the final row or this split's partial
    if (g == 0) {
        m_s[16 * wave + n] = m_run;
        l_s[16 * wave + n] = l_run;
    }
    __syncthreads();
#pragma unroll
    for (int ht = 0; ht < kNht; ++ht) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int hl = 16 * ht + 4 * g + i;
            const int head = head0 + hl;
            const float l = l_s[hl];
            const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
            for (int dt = 0; dt < kDt; ++dt) {
                const int d = 128 * wave + 16 * dt + n;
                const float v = o[ht][dt][i] * inv;
                if (n_splits == 1)
                    out[(static_cast<size_t>(row) * H + head) * kDv + d] = f32_to_bf16(v);
                else
                    part_o[((static_cast<size_t>(row) * n_splits + split) * H + head) * kDv + d] = v;
            }
        }
    }
    if (threadIdx.x < kHeadsPerGroup) {
        const int hl = threadIdx.x;
        const int head = head0 + hl;
        const float l = l_s[hl];
        const float lse2 = l > 0.f ? m_s[hl] + log2f(l) : -INFINITY;
        if (n_splits == 1) {
            if (lse) lse[static_cast<size_t>(row) * H + head] = lse2 * kLn2;
        } else {
            part_lse[(static_cast<size_t>(row) * n_splits + split) * H + head] = lse2;
        }
    }
}

// Merge the splits of each (row, head): weights 2^(lse_s - max), output in bf16.
__global__ __launch_bounds__(256)
void mla_combine_kernel(const float* __restrict__ part_o, const float* __restrict__ part_lse,
                        int rows, int H, int n_splits, uint16_t* __restrict__ out,
                        float* __restrict__ lse)
{
    const size_t gid = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    const size_t total = static_cast<size_t>(rows) * H * (kDv / 4);
    if (gid >= total) return;
    const int d4 = static_cast<int>(gid % (kDv / 4));
    const size_t rh = gid / (kDv / 4);
    const int h = static_cast<int>(rh % H);
    const size_t row = rh / H;
    float M = -INFINITY;
    for (int s = 0; s < n_splits; ++s) M = fmaxf(M, part_lse[(row * n_splits + s) * H + h]);
    float W = 0.f;
    float4 acc = {0.f, 0.f, 0.f, 0.f};
    if (M != -INFINITY) {
        for (int s = 0; s < n_splits; ++s) {
            const float ls = part_lse[(row * n_splits + s) * H + h];
            if (ls == -INFINITY) continue;
            const float wgt = exp2f(ls - M);
            W += wgt;
            const float4 v = *reinterpret_cast<const float4*>(
                part_o + ((row * n_splits + s) * H + h) * kDv + 4 * d4);
            acc.x += wgt * v.x; acc.y += wgt * v.y; acc.z += wgt * v.z; acc.w += wgt * v.w;
        }
    }
    const float inv = W > 0.f ? 1.f / W : 0.f;
    uint16_t* o = out + (row * H + h) * kDv + 4 * d4;
    o[0] = f32_to_bf16(acc.x * inv);
    o[1] = f32_to_bf16(acc.y * inv);
    o[2] = f32_to_bf16(acc.z * inv);
    o[3] = f32_to_bf16(acc.w * inv);
    if (lse && d4 == 0) lse[row * H + h] = W > 0.f ? (M + log2f(W)) * kLn2 : -INFINITY;
}

int mla_splits(int rows, int H, int k) {
    // enough (row, split, head group) blocks to give every CU one workgroup
    const int n_tiles = (k + kKt - 1) / kKt;
    const int per_split = rows * (H / kHeadsPerGroup);
    int s = per_split >= 256 ? 1 : (256 + per_split - 1) / per_split;
    s = min(s, 8);
    const int min_s = (n_tiles * kKt + kMaxSlots - 1) / kMaxSlots;   // slots per split fit LDS
    s = max(s, min_s);
    s = min(s, n_tiles);
    return max(s, 1);
}

}  // namespace

hipError_t launch_sparse_attn_generic(const SparseAttnArgs& a, hipStream_t stream) {
    const size_t shmem = sizeof(float) * (static_cast<size_t>(a.Dk) + a.k);
    hipLaunchKernelGGL(sparse_attn_generic_kernel, dim3(a.B * a.T * a.H), dim3(kGenThreads),
                       shmem, stream, a);
    return hipGetLastError();
}

bool mla_decode_mfma_supported(int H, int Dv, int Dr, int bf16) {
    return bf16 && Dv == kDv && Dv + Dr == kDq && H >= kHeadsPerGroup && H % kHeadsPerGroup == 0;
}

size_t mla_decode_workspace_bytes(int B, int T, int H, int, int k) {
    const int rows = B * T;
    const int s = mla_splits(rows, H, k);
    if (s == 1) return 0;
    return static_cast<size_t>(rows) * s * H * (kDv + 1) * sizeof(float) + 256;
}

hipError_t launch_mla_decode_mfma(const void* q, const void* latent, const int32_t* idx,
                                  const int32_t* len, int B, int T, int H, int Lmax, int k,
                                  float sm_scale, void* out, float* lse, void* ws,
                                  hipStream_t stream) {
    const int rows = B * T;
    const int s = mla_splits(rows, H, k);
    const int n_tiles = (k + kKt - 1) / kKt;
    const int tps = (n_tiles + s - 1) / s;
    const int n_units = rows * s;
    const int n_groups = H / kHeadsPerGroup;
    // units are dealt to the 8 XCD slots; pad so every slot has the same block count
    const int units_per_xcd = (n_units + kXcds - 1) / kXcds;
    const int blocks = units_per_xcd * n_groups * kXcds;
    float* part_o = static_cast<float*>(ws);
    float* part_lse = s > 1 ? part_o + static_cast<size_t>(rows) * s * H * kDv : nullptr;
    const float scale_log2 = sm_scale * kLog2e;
    hipLaunchKernelGGL(mla_decode_mfma_kernel, dim3(blocks), dim3(kMlaThreads), 0, stream,
                       static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(latent), idx,
                       len, T, H, Lmax, k, tps, s, n_units, scale_log2,
                       static_cast<uint16_t*>(out), lse, part_o, part_lse);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || s == 1) return e;
    const size_t total = static_cast<size_t>(rows) * H * (kDv / 4);
    hipLaunchKernelGGL(mla_combine_kernel, dim3((total + 255) / 256), dim3(256), 0, stream,
                       part_o, part_lse, rows, H, s, static_cast<uint16_t*>(out), lse);
    return hipGetLastError();
}

}  // namespace dsa
