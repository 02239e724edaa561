// topk.hip -- per-row top-k of the index scores by radix select (no sort).
//
// For row (b,t) with n = pos(b,t) + 1 visible scores, the kernels return the positions
// of the min(k, n) largest ones (the Indexer.forward excerpt on the "DeepSeek-V3.2-Exp -
// Split indexer heads" page keeps the index_topk best, capped at the visible count), in ascending
// position order, followed by -1 in the unused slots (the warm-up sentinel of the
// DeepSeek-V4 mask visualiser).  Equal scores resolve towards the smaller position, so
// the output is deterministic.
//
// Block select (one 1024-thread workgroup over up to 4096 * REG keys held in registers,
// or re-read when REG = 0).  Scores map to order-preserving 32-bit keys.  A block
// reduction finds the key range [lo, hi]; each histogram level splits the current range
// into at most 2048 equal bins (LDS atomics; two alternating histograms, so clearing
// costs no barrier), and a descending scan finds the bin holding the k-th largest key,
// which becomes the new range.  Bins follow the actual spread of the keys rather than
// fixed key bits (fixed top bits put scores that share an exponent into a handful of
// bins), so one or two levels usually isolate the threshold.  The loop ends when the
// range holds exactly the number of keys still needed or shrinks to one key value.  A
// final compaction writes, in index order, every key above the range plus the first
// `need` keys inside it, using one block-wide prefix sum.
//
// Rows up to 16384 positions: one workgroup per row.  Longer rows (a workgroup can keep
// only ~64 KB of loads in flight, far too little for one row of a long context) take
// two launches: every 8192- or 16384-position chunk of a row selects its own top-k
// candidates (key and position) in parallel, then one workgroup per row selects the
// top-k of the candidates.  The row's top-k is contained in the union of its chunks' top-k under
// the same (score, position) order, and candidates are stored chunk after chunk in
// position order, so candidate order is position order and ties still resolve towards
// the smaller position.
#include "dsa_device.h"
#include "dsa_internal.h"

namespace dsa {

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;
constexpr int kBins = 2048;
constexpr int kBinBits = 11;
constexpr int kPerThread = 4;
constexpr int kPerIter = kThreads * kPerThread;     // positions per block-wide iteration
constexpr int kMaxIters = 4;                         // register-held iterations
constexpr int kSingleMax = 4 * kPerIter;             // longest row for the one-launch form
constexpr uint32_t kNoKey = 0u;                      // unused candidate (float bits of -NaN)
constexpr int kStagedOut = 4096;                     // outputs staged in LDS up to this k

struct TopkShared {
    int32_t out[kStagedOut];          // selected positions, written out coalesced
    uint32_t hist[2][kBins];
    uint32_t scan[kWaves + 1];
    uint32_t scan2[kMaxIters][kWaves + 1];
    uint32_t red[2][kWaves];
    uint32_t bin;
    uint32_t need;
    uint32_t bin_count;
};

__device__ __forceinline__ uint32_t score_key(float f) {
    uint32_t u = __float_as_uint(f);
    if (u == 0x80000000u) u = 0;            // -0 ranks with +0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive prefix sums of N values per thread over the block (in thread order), with one
// set of barriers for all of them; tot[i] gets the block total of value i.
template <int N>
__device__ __forceinline__ void block_exclusive_scan_n(const uint32_t (&v)[N], TopkShared& sh,
                                                       uint32_t (&r)[N], uint32_t (&tot)[N]) {
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
    __device__ __forceinline__ void load4(int i0, uint32_t (&key)[kPerThread]) const {
        if (vec4 && i0 + kPerThread <= n) {
            const float4 v = *reinterpret_cast<const float4*>(sc + i0);
            key[0] = score_key(v.x); key[1] = score_key(v.y);
            key[2] = score_key(v.z); key[3] = score_key(v.w);
        } else {
#pragma unroll
            for (int j = 0; j < kPerThread; ++j) key[j] = i0 + j < n ? score_key(sc[i0 + j]) : kNoKey;
        }
    }
};

struct CandSrc {                        // candidate keys of a row
    const uint32_t* key;
    int n;
    bool vec4;
    __device__ __forceinline__ void load4(int i0, uint32_t (&k4)[kPerThread]) const {
        if (vec4 && i0 + kPerThread <= n) {
            const uint4 v = *reinterpret_cast<const uint4*>(key + i0);
            k4[0] = v.x; k4[1] = v.y; k4[2] = v.z; k4[3] = v.w;
        } else {
#pragma unroll
            for (int j = 0; j < kPerThread; ++j) k4[j] = i0 + j < n ? key[i0 + j] : kNoKey;
        }
    }
};

// Keys of one selection, held in registers (REG block iterations) or re-read (REG = 0).
// Element index i0 + j of iteration `it` is it * 4096 + 4 tid + j.
template <int REG, typename Src>
struct Keys {
    uint32_t key[REG > 0 ? REG : 1][kPerThread];
    Src src;
    int iters;

    __device__ __forceinline__ void init(const Src& s, int n) {
        src = s;
        iters = (n + kPerIter - 1) / kPerIter;
        if constexpr (REG > 0) {
#pragma unroll
            for (int it = 0; it < REG; ++it) src.load4(it * kPerIter + threadIdx.x * kPerThread, key[it]);
        }
    }
    // f(key, index, live) for this thread's elements of block iteration `it`
    template <typename F>
    __device__ __forceinline__ void visit(int it, F&& f) {
        const int i0 = it * kPerIter + threadIdx.x * kPerThread;
        if constexpr (REG > 0) {
#pragma unroll
            for (int j = 0; j < kPerThread; ++j) f(key[it][j], i0 + j, key[it][j] != kNoKey);
        } else {
            uint32_t kk[kPerThread];
            src.load4(i0, kk);
#pragma unroll
            for (int j = 0; j < kPerThread; ++j) f(kk[j], i0 + j, kk[j] != kNoKey);
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
                uint32_t kk[kBatch][kPerThread];
#pragma unroll
                for (int u = 0; u < kBatch; ++u)
                    src.load4((it0 + u) * kPerIter + threadIdx.x * kPerThread, kk[u]);
#pragma unroll
                for (int u = 0; u < kBatch; ++u) {
                    const int i0 = (it0 + u) * kPerIter + threadIdx.x * kPerThread;
#pragma unroll
                    for (int j = 0; j < kPerThread; ++j) f(kk[u][j], i0 + j, kk[u][j] != kNoKey);
                }
            }
        }
    }
};

// Select the k largest live keys (k < number of live keys) of `ks`; store(slot, index,
// key) receives slots 0..k-1 in ascending index order.
template <int REG, typename Src, typename Store>
__device__ __forceinline__ void block_select(Keys<REG, Src>& ks, int k, TopkShared& sh, Store&& store) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;

    // ---- key range
    uint32_t kmin = 0xffffffffu, kmax = 0u;
    ks.visit_all([&](uint32_t key, int, bool ok) {
        if (ok) { kmin = min(kmin, key); kmax = max(kmax, key); }
    });
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        kmin = min(kmin, static_cast<uint32_t>(__shfl_xor(static_cast<int>(kmin), o, kWave)));
        kmax = max(kmax, static_cast<uint32_t>(__shfl_xor(static_cast<int>(kmax), o, kWave)));
    }
    if (lane == 0) { sh.red[0][wave] = kmin; sh.red[1][wave] = kmax; }
    for (int i = threadIdx.x; i < kBins; i += kThreads) sh.hist[0][i] = 0;
    __syncthreads();
    uint32_t lo = sh.red[0][0], hi = sh.red[1][0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) { lo = min(lo, sh.red[0][w]); hi = max(hi, sh.red[1][w]); }

    // ---- narrow [lo, hi] to the class of the k-th largest key
    uint32_t need = static_cast<uint32_t>(k);
    int level = 0;
    while (hi != lo) {
        uint32_t* hist = sh.hist[level & 1];
        const uint32_t span = hi - lo;
        const int shift = max(0, 32 - __clz(static_cast<int>(span)) - kBinBits);
        ks.visit_all([&](uint32_t key, int, bool ok) {
            if (ok && key >= lo && key <= hi) atomicAdd(&hist[(key - lo) >> shift], 1u);
        });
        // the other histogram was last read before the previous level's final barrier
        for (int i = threadIdx.x; i < kBins; i += kThreads) sh.hist[(level + 1) & 1][i] = 0;
        __syncthreads();
        // thread i looks at bins hb = 2047 - 2i and lb = hb - 1 (descending bin order);
        // wave totals go through LDS once, each wave forms its own prefix from them
        const int hb = kBins - 1 - 2 * static_cast<int>(threadIdx.x);
        const int lb = hb - 1;
        const uint32_t ch = hist[hb], cl = hist[lb];
        const uint32_t inc = wave_inclusive_scan(ch + cl, lane);
        if (lane == kWave - 1) sh.scan[wave] = inc;
        __syncthreads();
        uint32_t above = inc - (ch + cl);
#pragma unroll
        for (int w = 0; w < kWaves; ++w) above += w < wave ? sh.scan[w] : 0u;
        if (above < need && need <= above + ch) {
            sh.bin = hb; sh.need = need - above; sh.bin_count = ch;
        } else if (above + ch < need && need <= above + ch + cl) {
            sh.bin = lb; sh.need = need - above - ch; sh.bin_count = cl;
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
        block_exclusive_scan_n<REG>(v, sh, r, tot);
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
            block_exclusive_scan_n<1>(v, sh, r, tot);
            emit(it, gt_run + (r[0] & 0xffffu), eq_run + (r[0] >> 16));
            gt_run += tot[0] & 0xffffu;
            eq_run += tot[0] >> 16;
        }
    }
}

__device__ __forceinline__ int visible(const int32_t* len, int row, int T, int Lmax) {
    const int b = row / T;
    const int t = row - b * T;
    return min(len[b], Lmax) - T + t + 1;       // clamped: never read past Lmax
}

// One workgroup per row (rows of at most 4096 * REG positions when REG > 0).
template <int REG>
__global__ __launch_bounds__(kThreads)
void topk_row_kernel(const float* __restrict__ scores, const int32_t* __restrict__ len,
                     int T, int Lmax, int k, int32_t* __restrict__ idx)
{
    __shared__ TopkShared sh;
    const int row = blockIdx.x;
    const int n = visible(len, row, T, Lmax);
    int32_t* out = idx + static_cast<size_t>(row) * k;
    if (n <= k) {                               // every visible position is kept
        for (int j = threadIdx.x; j < k; j += kThreads) out[j] = j < n ? j : -1;
        return;
    }
    Keys<REG, ScoreSrc> ks;
    ks.init(ScoreSrc{scores + static_cast<size_t>(row) * Lmax, n, (Lmax & 3) == 0}, n);
    if (k <= kStagedOut) {
        // slots arrive scattered; staging them in LDS turns k scattered 4-byte stores
        // into one coalesced pass
        block_select(ks, k, sh, [&](uint32_t slot, int i, uint32_t) { sh.out[slot] = i; });
        __syncthreads();
        for (int j = threadIdx.x; j < k; j += kThreads) out[j] = sh.out[j];
    } else {
        block_select(ks, k, sh, [&](uint32_t slot, int i, uint32_t) { out[slot] = i; });
    }
}

// Two-stage form, stage 1: chunk c of row r (its visible positions among [C c, C c + C),
// C = 4096 REG) writes its top-min(k, m) keys and positions, in position order, to
// candidate slots [c k, c k + k) of the row; the remaining slots get kNoKey / -1.
template <int REG>
__global__ __launch_bounds__(kThreads)
void topk_chunk_kernel(const float* __restrict__ scores, const int32_t* __restrict__ len,
                       int T, int Lmax, int k, int n_chunks, uint32_t* __restrict__ cand_key,
                       int32_t* __restrict__ cand_pos)
{
    __shared__ TopkShared sh;
    const int row = blockIdx.x / n_chunks;
    const int c = blockIdx.x - row * n_chunks;
    const int n = visible(len, row, T, Lmax);
    if (n <= k) return;                         // stage 2 fills such rows directly
    constexpr int kChunk = REG * kPerIter;
    const int base = c * kChunk;
    const int m = max(0, min(kChunk, n - base));
    const size_t slot0 = (static_cast<size_t>(row) * n_chunks + c) * k;
    uint32_t* ck = cand_key + slot0;
    int32_t* cp = cand_pos + slot0;
    const int kept = min(k, m);
    for (int j = kept + threadIdx.x; j < k; j += kThreads) { ck[j] = kNoKey; cp[j] = -1; }
    if (m <= k) {                               // the whole chunk is a candidate set
        const float* sc = scores + static_cast<size_t>(row) * Lmax + base;
        for (int j = threadIdx.x; j < m; j += kThreads) { ck[j] = score_key(sc[j]); cp[j] = base + j; }
        return;
    }
    Keys<REG, ScoreSrc> ks;
    ks.init(ScoreSrc{scores + static_cast<size_t>(row) * Lmax + base, m, ((Lmax | base) & 3) == 0}, m);
    block_select(ks, k, sh, [&](uint32_t slot, int i, uint32_t key) { ck[slot] = key; cp[slot] = base + i; });
}

// Two-stage form, stage 2: top-k of a row's candidates (REG = 0: re-read them).
template <int REG>
__global__ __launch_bounds__(kThreads)
void topk_merge_kernel(const uint32_t* __restrict__ cand_key, const int32_t* __restrict__ cand_pos,
                       const int32_t* __restrict__ len, int T, int Lmax, int k, int n_chunks,
                       int32_t* __restrict__ idx)
{
    __shared__ TopkShared sh;
    const int row = blockIdx.x;
    const int n = visible(len, row, T, Lmax);
    int32_t* out = idx + static_cast<size_t>(row) * k;
    if (n <= k) {
        for (int j = threadIdx.x; j < k; j += kThreads) out[j] = j < n ? j : -1;
        return;
    }
    const int nc = n_chunks * k;
    const size_t off = static_cast<size_t>(row) * nc;
    const int32_t* cp = cand_pos + off;
    Keys<REG, CandSrc> ks;
    ks.init(CandSrc{cand_key + off, nc, (nc & 3) == 0}, nc);
    if (k <= kStagedOut) {
        block_select(ks, k, sh, [&](uint32_t slot, int i, uint32_t) { sh.out[slot] = i; });
        __syncthreads();
        for (int j = threadIdx.x; j < k; j += kThreads) out[j] = cp[sh.out[j]];
    } else {
        block_select(ks, k, sh, [&](uint32_t slot, int i, uint32_t) { out[slot] = cp[i]; });
    }
}

// Chunk length of the two-stage form: 8192 positions while the candidates of a row fit
// the register-held merge (16384 keys), else 16384.
int chunk_for(int Lmax, int k) {
    const long long c8 = (Lmax + 2 * kPerIter - 1) / (2 * kPerIter);
    return c8 * k <= kSingleMax ? 2 * kPerIter : 4 * kPerIter;
}
int n_chunks_for(int Lmax, int k) { const int c = chunk_for(Lmax, k); return (Lmax + c - 1) / c; }
bool two_stage(int Lmax, int k) { return Lmax > kSingleMax && k < 2 * kPerIter; }

}  // namespace

size_t topk_workspace_bytes(int B, int T, int Lmax, int k) {
    if (!two_stage(Lmax, k)) return 0;
    return static_cast<size_t>(B) * T * n_chunks_for(Lmax, k) * k * (sizeof(uint32_t) + sizeof(int32_t)) + 256;
}

hipError_t launch_topk(const TopkArgs& a, void* ws, hipStream_t stream) {
    const int rows = a.B * a.T;
    const dim3 block(kThreads);
    if (!two_stage(a.Lmax, a.k)) {
        if (a.Lmax <= 2 * kPerIter)
            hipLaunchKernelGGL(topk_row_kernel<2>, dim3(rows), block, 0, stream, a.scores, a.len, a.T, a.Lmax, a.k, a.idx);
        else if (a.Lmax <= kSingleMax)
            hipLaunchKernelGGL(topk_row_kernel<4>, dim3(rows), block, 0, stream, a.scores, a.len, a.T, a.Lmax, a.k, a.idx);
        else
            hipLaunchKernelGGL(topk_row_kernel<0>, dim3(rows), block, 0, stream, a.scores, a.len, a.T, a.Lmax, a.k, a.idx);
        return hipGetLastError();
    }
    const int nch = n_chunks_for(a.Lmax, a.k);
    const size_t ncand = static_cast<size_t>(rows) * nch * a.k;
    uint32_t* ck = static_cast<uint32_t*>(ws);
    int32_t* cp = reinterpret_cast<int32_t*>(ck + ncand);
    if (chunk_for(a.Lmax, a.k) == 2 * kPerIter)
        hipLaunchKernelGGL(topk_chunk_kernel<2>, dim3(rows * nch), block, 0, stream, a.scores, a.len,
                           a.T, a.Lmax, a.k, nch, ck, cp);
    else
        hipLaunchKernelGGL(topk_chunk_kernel<4>, dim3(rows * nch), block, 0, stream, a.scores, a.len,
                           a.T, a.Lmax, a.k, nch, ck, cp);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const long long nc = static_cast<long long>(nch) * a.k;
    if (nc <= kSingleMax)
        hipLaunchKernelGGL(topk_merge_kernel<4>, dim3(rows), block, 0, stream, ck, cp, a.len, a.T, a.Lmax, a.k, nch, a.idx);
    else
        hipLaunchKernelGGL(topk_merge_kernel<0>, dim3(rows), block, 0, stream, ck, cp, a.len, a.T, a.Lmax, a.k, nch, a.idx);
    return hipGetLastError();
}

}  // namespace dsa
