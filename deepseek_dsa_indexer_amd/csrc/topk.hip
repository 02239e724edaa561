// topk.hip -- per-row top-k of the index scores by radix select (no sort).
//
// For row (b,t) with n = pos(b,t) + 1 visible scores, the kernel returns the positions
// of the min(k, n) largest ones (Indexer.forward excerpt, topk(min(index_topk,
// end_pos)) on the "DeepSeek-V3.2-Exp - Split indexer heads" page), in ascending
// position order, followed by -1 in the unused slots (the warm-up sentinel of the
// DeepSeek-V4 mask visualiser).
//
// Method.  Scores are mapped to order-preserving 32-bit keys.  Up to three histogram
// passes (11 + 11 + 10 key bits, 2048 LDS bins, LDS atomics) narrow the k-th largest
// key down to an exact threshold tau; a pass stops early when its threshold bin holds
// exactly the number of elements still needed.  One final pass compacts, in position
// order, every key above tau plus the first `need` keys equal to tau (block-wide
// prefix sums built from wave scans), so equal scores are resolved towards the smaller
// position and the output is deterministic.  One 1024-thread workgroup owns one row.
#include "dsa_device.h"
#include "dsa_internal.h"

namespace dsa {

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;
constexpr int kBins = 2048;
constexpr int kPerThread = 4;
constexpr int kPerIter = kThreads * kPerThread;

struct TopkShared {
    uint32_t hist[kBins];
    uint32_t scan[kWaves + 1];
    uint32_t bin;
    uint32_t need;
    uint32_t bin_count;
};

__device__ __forceinline__ uint32_t score_key(float f) {
    uint32_t u = __float_as_uint(f);
    if (u == 0x80000000u) u = 0;            // -0 ranks with +0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive prefix sum of v over the block (in thread order); *total gets the sum.
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, TopkShared& sh,
                                                         uint32_t* total) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const uint32_t inc = wave_inclusive_scan(v, lane);
    if (lane == kWave - 1) sh.scan[wave] = inc;
    __syncthreads();
    if (wave == 0) {
        const uint32_t x = lane < kWaves ? sh.scan[lane] : 0u;
        const uint32_t xi = wave_inclusive_scan(x, lane);
        if (lane < kWaves) sh.scan[lane] = xi - x;
        if (lane == kWaves - 1) sh.scan[kWaves] = xi;
    }
    __syncthreads();
    const uint32_t r = sh.scan[wave] + inc - v;
    *total = sh.scan[kWaves];
    __syncthreads();
    return r;
}

// Keys of positions base + 4*tid + j (j < 4); positions >= n get valid = false.
__device__ __forceinline__ void load_keys(const float* sc, int base, int n, bool vec4,
                                          uint32_t key[kPerThread], bool valid[kPerThread]) {
    const int i0 = base + threadIdx.x * kPerThread;
    if (vec4 && i0 + kPerThread <= n) {
        const float4 v = *reinterpret_cast<const float4*>(sc + i0);
        key[0] = score_key(v.x); key[1] = score_key(v.y);
        key[2] = score_key(v.z); key[3] = score_key(v.w);
#pragma unroll
        for (int j = 0; j < kPerThread; ++j) valid[j] = true;
    } else {
#pragma unroll
        for (int j = 0; j < kPerThread; ++j) {
            valid[j] = i0 + j < n;
            key[j] = valid[j] ? score_key(sc[i0 + j]) : 0u;
        }
    }
}

__global__ __launch_bounds__(kThreads)
void topk_radix_kernel(const float* __restrict__ scores, const int32_t* __restrict__ len,
                       int T, int Lmax, int k, int32_t* __restrict__ idx)
{
    __shared__ TopkShared sh;
    const int row = blockIdx.x;
    const int b = row / T;
    const int t = row - b * T;
    const int n = min(len[b], Lmax) - T + t + 1;   // clamped: never read past Lmax
    int32_t* out = idx + static_cast<size_t>(row) * k;

    if (n <= k) {                               // every visible position is kept
        for (int j = threadIdx.x; j < k; j += kThreads) out[j] = j < n ? j : -1;
        return;
    }

    const float* sc = scores + static_cast<size_t>(row) * Lmax;
    const bool vec4 = (Lmax & 3) == 0;
    uint32_t prefix = 0;       // fixed high key bits
    int shift = 32;            // keys with (key >> shift) == prefix are still candidates
    uint32_t need = static_cast<uint32_t>(k);

    const int level_bits[3] = {11, 11, 10};
    for (int level = 0; level < 3; ++level) {
        const int bits = level_bits[level];
        const int new_shift = shift - bits;
        const uint32_t mask = (1u << bits) - 1u;
        for (int i = threadIdx.x; i < kBins; i += kThreads) sh.hist[i] = 0;
        __syncthreads();
        for (int base = 0; base < n; base += kPerIter) {
            uint32_t key[kPerThread];
            bool valid[kPerThread];
            load_keys(sc, base, n, vec4, key, valid);
#pragma unroll
            for (int j = 0; j < kPerThread; ++j) {
                const bool cand = valid[j] && (shift == 32 || (key[j] >> shift) == prefix);
                if (cand) atomicAdd(&sh.hist[(key[j] >> new_shift) & mask], 1u);
            }
        }
        __syncthreads();
        // thread i looks at bins hi = 2047 - 2i and lo = hi - 1; counts above come from
        // an exclusive scan in thread order (= descending bin order)
        const int hi = kBins - 1 - 2 * static_cast<int>(threadIdx.x);
        const int lo = hi - 1;
        const uint32_t ch = sh.hist[hi], cl = sh.hist[lo];
        uint32_t total;
        const uint32_t above = block_exclusive_scan(ch + cl, sh, &total);
        if (above < need && need <= above + ch) {
            sh.bin = hi; sh.need = need - above; sh.bin_count = ch;
        } else if (above + ch < need && need <= above + ch + cl) {
            sh.bin = lo; sh.need = need - above - ch; sh.bin_count = cl;
        }
        __syncthreads();
        prefix = (shift == 32 ? 0u : (prefix << bits)) | sh.bin;
        need = sh.need;
        shift = new_shift;
        const bool exact = sh.bin_count == need;
        __syncthreads();
        if (exact) break;
    }

    // ---- ordered compaction: keys above the threshold, then the first `need` equal ones
    uint32_t gt_run = 0, eq_run = 0;
    for (int base = 0; base < n; base += kPerIter) {
        uint32_t key[kPerThread];
        bool valid[kPerThread];
        load_keys(sc, base, n, vec4, key, valid);
        uint32_t gt = 0, eq = 0;
        bool is_gt[kPerThread], is_eq[kPerThread];
#pragma unroll
        for (int j = 0; j < kPerThread; ++j) {
            const uint32_t top = key[j] >> shift;
            is_gt[j] = valid[j] && top > prefix;
            is_eq[j] = valid[j] && top == prefix;
            gt += is_gt[j];
            eq += is_eq[j];
        }
        uint32_t total;
        const uint32_t before = block_exclusive_scan(gt | (eq << 16), sh, &total);
        uint32_t G = gt_run + (before & 0xffffu);
        uint32_t E = eq_run + (before >> 16);
        const int i0 = base + threadIdx.x * kPerThread;
#pragma unroll
        for (int j = 0; j < kPerThread; ++j) {
            if (is_gt[j]) {
                const uint32_t slot = G + min(E, need);
                if (slot < static_cast<uint32_t>(k)) out[slot] = i0 + j;
                ++G;
            } else if (is_eq[j]) {
                if (E < need && G + E < static_cast<uint32_t>(k)) out[G + E] = i0 + j;
                ++E;
            }
        }
        gt_run += total & 0xffffu;
        eq_run += total >> 16;
    }
}

}  // namespace

size_t topk_workspace_bytes(int, int, int, int) { return 0; }

hipError_t launch_topk(const TopkArgs& a, void*, hipStream_t stream) {
    hipLaunchKernelGGL(topk_radix_kernel, dim3(a.B * a.T), dim3(kThreads), 0, stream, a.scores,
                       a.len, a.T, a.Lmax, a.k, a.idx);
    return hipGetLastError();
}

}  // namespace dsa
