// topk_select.h -- block-wide exact top-k selection over 32-bit order-preserving keys, for
// one workgroup of NT threads over up to 4 NT REG keys held in registers (or re-read when
// REG = 0).
//
// Method.  A block reduction finds the key range [lo, hi]; each histogram level splits
// the current range into at most 2048 equal bins (LDS atomics; two alternating
// histograms, so clearing costs no barrier), and a descending scan finds the bin holding
// the k-th largest key, which becomes the new range.  Bins follow the actual spread of
// the keys rather than fixed key bits (fixed top bits put scores that share an exponent
// into a handful of bins), so one or two levels usually isolate the threshold.  The loop
// ends when the range holds exactly the number of keys still needed or shrinks to one
// key value; when the bin of the k-th key holds at most kSelCand keys, they are instead
// gathered into LDS and one wave ranks them, which gives that key's exact value in place
// of further histogram levels.  A final compaction hands out, in index order, every key above the range
// plus the first `need` keys inside it, using one block-wide prefix sum; equal keys
// therefore resolve towards the smaller index.
#pragma once

#include "dsa_device.h"

namespace dsa {

constexpr int kSelBins = 2048;
constexpr int kSelBinBits = 11;
constexpr int kSelPerThread = 4;
constexpr int kSelMaxIters = 4;                      // register-held block iterations
constexpr uint32_t kNoKey = 0u;                      // no element (float bits of -NaN)
constexpr int kSelCand = 64;                         // bin sizes resolved by ranking

template <int NT>
struct SelectShared {
    uint32_t hist[2][kSelBins];
    uint32_t scan[NT / kWave + 1];
    uint32_t scan2[kSelMaxIters][NT / kWave + 1];
    uint32_t red[2][NT / kWave];
    uint32_t bin;
    uint32_t need;
    uint32_t bin_count;
    uint32_t cand[kSelCand];          // the keys of a small threshold bin
    uint32_t cand_n;
    uint32_t tau;                     // their need-th largest value
};

__device__ __forceinline__ uint32_t score_key(float f) {
    uint32_t u = __float_as_uint(f);
    if (u == 0x80000000u) u = 0;            // -0 ranks with +0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive prefix sums of N values per thread over the block (in thread order), with one
// set of barriers for all of them; tot[i] gets the block total of value i.
template <int NT, int N>
__device__ __forceinline__ void block_exclusive_scan_n(const uint32_t (&v)[N], SelectShared<NT>& sh,
                                                       uint32_t (&r)[N], uint32_t (&tot)[N]) {
    constexpr int kWaves = NT / kWave;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    uint32_t inc[N];
#pragma unroll
    for (int i = 0; i < N; ++i) {
        inc[i] = wave_inclusive_scan(v[i], lane);
        if (lane == kWave - 1) sh.scan2[i][wave] = inc[i];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < N; ++i) {
        uint32_t before = 0, all = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const uint32_t x = sh.scan2[i][w];
            before += w < wave ? x : 0u;
            all += x;
        }
        r[i] = before + inc[i] - v[i];
        tot[i] = all;
    }
    __syncthreads();
}

// Key sources: four consecutive keys at index i0; kNoKey marks an element that does not
// take part (a position past the visible range, an unused candidate slot).  No score
// maps to kNoKey except a negative NaN with every mantissa bit set.
struct ScoreSrc {                       // a row of scores, indices < n visible
    const float* sc;
    int n;
    bool vec4;
    __device__ __forceinline__ void load4(int i0, uint32_t (&key)[kSelPerThread]) const {
        if (vec4 && i0 + kSelPerThread <= n) {
            const float4 v = *reinterpret_cast<const float4*>(sc + i0);
            key[0] = score_key(v.x); key[1] = score_key(v.y);
            key[2] = score_key(v.z); key[3] = score_key(v.w);
        } else {
#pragma unroll
            for (int j = 0; j < kSelPerThread; ++j) key[j] = i0 + j < n ? score_key(sc[i0 + j]) : kNoKey;
        }
    }
};

struct CandSrc {                        // candidate keys of a row
    const uint32_t* key;
    int n;
    bool vec4;
    __device__ __forceinline__ void load4(int i0, uint32_t (&k4)[kSelPerThread]) const {
        if (vec4 && i0 + kSelPerThread <= n) {
            const uint4 v = *reinterpret_cast<const uint4*>(key + i0);
            k4[0] = v.x; k4[1] = v.y; k4[2] = v.z; k4[3] = v.w;
        } else {
#pragma unroll
            for (int j = 0; j < kSelPerThread; ++j) k4[j] = i0 + j < n ? key[i0 + j] : kNoKey;
        }
    }
};

// Keys of one selection, held in registers (REG block iterations) or re-read (REG = 0).
// Element index i0 + j of iteration `it` is it * 4 NT + 4 tid + j.
template <int NT, int REG, typename Src>
struct Keys {
    static constexpr int kPerIter = NT * kSelPerThread;
    uint32_t key[REG > 0 ? REG : 1][kSelPerThread];
    Src src;
    int iters;

    __device__ __forceinline__ void init(const Src& s, int n) {
        src = s;
        iters = (n + kPerIter - 1) / kPerIter;
        if constexpr (REG > 0) {
#pragma unroll
            for (int it = 0; it < REG; ++it) src.load4(it * kPerIter + threadIdx.x * kSelPerThread, key[it]);
        }
    }
    // f(key, index, live) for this thread's elements of block iteration `it`
    template <typename F>
    __device__ __forceinline__ void visit(int it, F&& f) {
        const int i0 = it * kPerIter + threadIdx.x * kSelPerThread;
        if constexpr (REG > 0) {
#pragma unroll
            for (int j = 0; j < kSelPerThread; ++j) f(key[it][j], i0 + j, key[it][j] != kNoKey);
        } else {
            uint32_t kk[kSelPerThread];
            src.load4(i0, kk);
#pragma unroll
            for (int j = 0; j < kSelPerThread; ++j) f(kk[j], i0 + j, kk[j] != kNoKey);
        }
    }
    // f for every element held by this thread; the re-reading form keeps four block
    // iterations of loads in flight.
    template <typename F>
    __device__ __forceinline__ void visit_all(F&& f) {
        if constexpr (REG > 0) {
#pragma unroll
            for (int it = 0; it < REG; ++it) visit(it, f);
        } else {
            constexpr int kBatch = 4;
            for (int it0 = 0; it0 < iters; it0 += kBatch) {
                uint32_t kk[kBatch][kSelPerThread];
#pragma unroll
                for (int u = 0; u < kBatch; ++u)
                    src.load4((it0 + u) * kPerIter + threadIdx.x * kSelPerThread, kk[u]);
#pragma unroll
                for (int u = 0; u < kBatch; ++u) {
                    const int i0 = (it0 + u) * kPerIter + threadIdx.x * kSelPerThread;
#pragma unroll
                    for (int j = 0; j < kSelPerThread; ++j) f(kk[u][j], i0 + j, kk[u][j] != kNoKey);
                }
            }
        }
    }
};

// Select the k largest live keys (k < number of live keys) of `ks`; store(slot, index,
// key) receives slots 0..k-1 in ascending index order.
template <int NT, int REG, typename Src, typename Store>
__device__ __forceinline__ void block_select(Keys<NT, REG, Src>& ks, int k, SelectShared<NT>& sh,
                                             Store&& store) {
    constexpr int kWaves = NT / kWave;
    constexpr int kBpt = kSelBins / NT;             // histogram bins per thread in the scan
    static_assert(kSelBins % NT == 0 && NT % kWave == 0, "bins must split evenly over the block");
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;

    // ---- key range
    uint32_t kmin = 0xffffffffu, kmax = 0u;
    ks.visit_all([&](uint32_t key, int, bool ok) {
        if (ok) { kmin = min(kmin, key); kmax = max(kmax, key); }
    });
    kmin = wave_min_u32(kmin);
    kmax = wave_max_u32(kmax);
    if (lane == 0) { sh.red[0][wave] = kmin; sh.red[1][wave] = kmax; }
    for (int i = threadIdx.x; i < kSelBins; i += NT) sh.hist[0][i] = 0;
    if (threadIdx.x == 0) sh.cand_n = 0;
    __syncthreads();
    uint32_t lo = sh.red[0][0], hi = sh.red[1][0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) { lo = min(lo, sh.red[0][w]); hi = max(hi, sh.red[1][w]); }

    // ---- narrow [lo, hi] to the class of the k-th largest key
    uint32_t need = static_cast<uint32_t>(k);
    int level = 0;
    // Each level shrinks the range by a factor of at least 2^10, so three levels reach a
    // single key value from any 32-bit range; the bound only guards the loop.
    for (int guard = 0; guard < 4 && hi != lo; ++guard) {
        uint32_t* hist = sh.hist[level & 1];
        const uint32_t span = hi - lo;
        const int shift = max(0, 32 - __clz(static_cast<int>(span)) - kSelBinBits);
        ks.visit_all([&](uint32_t key, int, bool ok) {
            if (ok && key >= lo && key <= hi) atomicAdd(&hist[(key - lo) >> shift], 1u);
        });
        // the other histogram was last read before the previous level's final barrier
        for (int i = threadIdx.x; i < kSelBins; i += NT) sh.hist[(level + 1) & 1][i] = 0;
        __syncthreads();
        // thread i looks at the kBpt bins 2047 - kBpt i - u, u = 0 .. kBpt - 1 (descending
        // bin order); wave totals go through LDS once, each wave forms its own prefix
        // from them, and exactly one thread finds the bin where the count above it first
        // reaches `need`
        uint32_t cb[kBpt];
        uint32_t csum = 0;
#pragma unroll
        for (int u = 0; u < kBpt; ++u) {
            cb[u] = hist[kSelBins - 1 - kBpt * static_cast<int>(threadIdx.x) - u];
            csum += cb[u];
        }
        const uint32_t inc = wave_inclusive_scan(csum, lane);
        if (lane == kWave - 1) sh.scan[wave] = inc;
        __syncthreads();
        uint32_t above = inc - csum;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) above += w < wave ? sh.scan[w] : 0u;
#pragma unroll
        for (int u = 0; u < kBpt; ++u) {
            if (above < need && need <= above + cb[u]) {
                sh.bin = kSelBins - 1 - kBpt * static_cast<int>(threadIdx.x) - u;
                sh.need = need - above;
                sh.bin_count = cb[u];
            }
            above += cb[u];
        }
        __syncthreads();
        const uint32_t bin = sh.bin;
        need = sh.need;
        const uint32_t count = sh.bin_count;
        const uint32_t new_lo = lo + (bin << shift);
        // the bin covers [new_lo, new_lo + 2^shift - 1] (in 64 bits: no wrap at the top)
        hi = static_cast<uint32_t>(min(static_cast<uint64_t>(hi),
                                       static_cast<uint64_t>(new_lo) + ((1ull << shift) - 1ull)));
        lo = new_lo;
        ++level;
        if (count == need) break;                       // the whole class is selected
        if (count <= static_cast<uint32_t>(kSelCand) && hi != lo) {
            // A small bin: gather its keys (order does not matter) and let wave 0 rank
            // them.  Key x is the need-th largest iff (keys > x) < need <= (keys >= x);
            // the range becomes [x, x] with need - (keys > x) of its copies still needed,
            // exactly what further levels would reach.  (cand_n was zeroed before the
            // level's first barrier; sh.tau / sh.need are read after the next barrier.)
            ks.visit_all([&](uint32_t key, int, bool ok) {
                if (ok && key >= lo && key <= hi) sh.cand[atomicAdd(&sh.cand_n, 1u)] = key;
            });
            __syncthreads();
            if (wave == 0) {
                const int m = static_cast<int>(count);
                const uint32_t x = lane < m ? sh.cand[lane] : 0u;
                uint32_t gt = 0, ge = 0;
                for (int j = 0; j < m; ++j) {
                    const uint32_t y = sh.cand[j];
                    gt += y > x;
                    ge += y >= x;
                }
                if (lane < m && gt < need && need <= ge) {   // lanes holding that value agree
                    sh.tau = x;
                    sh.need = need - gt;
                }
            }
            __syncthreads();
            lo = hi = sh.tau;
            need = sh.need;
            break;
        }
        // sh.bin / sh.need are rewritten only after the next level's two barriers
    }

    // ---- ordered compaction: keys above the class, then the first `need` inside it.
    // Slot of a selected key = selected keys at smaller indices: all block iterations
    // before its own, then threads before it, then its earlier elements.
    auto emit = [&](int it, uint32_t G, uint32_t E) {
        ks.visit(it, [&](uint32_t key, int i, bool ok) {
            const bool gt = ok && key > hi;
            const bool eq = ok && key >= lo && key <= hi;
            const uint32_t slot = gt ? G + min(E, need) : G + E;
            if (slot < static_cast<uint32_t>(k) && (gt || (eq && E < need))) store(slot, i, key);
            G += gt;
            E += eq;
        });
    };
    auto counts = [&](int it) {
        uint32_t gt = 0, eq = 0;
        ks.visit(it, [&](uint32_t key, int, bool ok) {
            gt += ok && key > hi;
            eq += ok && key >= lo && key <= hi;
        });
        return gt | (eq << 16);          // at most 4096 each per iteration
    };
    if constexpr (REG > 0) {
        uint32_t v[REG], r[REG], tot[REG];
#pragma unroll
        for (int it = 0; it < REG; ++it) v[it] = counts(it);
        block_exclusive_scan_n<NT, REG>(v, sh, r, tot);
        uint32_t gt_run = 0, eq_run = 0;
#pragma unroll
        for (int it = 0; it < REG; ++it) {
            emit(it, gt_run + (r[it] & 0xffffu), eq_run + (r[it] >> 16));
            gt_run += tot[it] & 0xffffu;
            eq_run += tot[it] >> 16;
        }
    } else {
        uint32_t gt_run = 0, eq_run = 0;
        for (int it = 0; it < ks.iters; ++it) {
            uint32_t v[1] = {counts(it)}, r[1], tot[1];
            block_exclusive_scan_n<NT, 1>(v, sh, r, tot);
            emit(it, gt_run + (r[0] & 0xffffu), eq_run + (r[0] >> 16));
            gt_run += tot[0] & 0xffffu;
            eq_run += tot[0] >> 16;
        }
    }
}

}  // namespace dsa
