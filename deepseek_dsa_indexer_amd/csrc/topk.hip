// topk.hip -- per-row top-k of the index scores by radix select (no sort).
//
// For row (b,t) with n = pos(b,t) + 1 visible scores (with compressed entries, m > 1:
// n = (pos + 1) / m; see n_visible), the kernels return the positions
// of the min(k, n) largest ones (the Indexer.forward excerpt on the "DeepSeek-V3.2-Exp -
// Split indexer heads" page keeps the index_topk best, capped at the visible count), in ascending
// position order, followed by -1 in the unused slots (the warm-up sentinel of the
// DeepSeek-V4 mask visualiser).  Equal scores resolve towards the smaller position, so
// the output is deterministic.
//
// Method (topk_select.h): scores map to order-preserving 32-bit keys; range-adaptive
// LDS histogram levels narrow the range that holds the k-th largest key; one ordered
// compaction writes the result.
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
#include "topk_select.h"

namespace dsa {

namespace {

constexpr int kThreads = 1024;
constexpr int kPerIter = kThreads * kSelPerThread;  // positions per block-wide iteration
constexpr int kSingleMax = 4 * kPerIter;             // longest row for the one-launch form
constexpr int kStagedOut = 4096;                     // outputs staged in LDS up to this k

constexpr int kMaxSeqPerThread = 16;                 // numbered chunk launches: 16384 rows

struct TopkShared {
    int32_t out[kStagedOut];          // selected positions, written out coalesced
    SelectShared<kThreads> sel;
    int num[kThreads / kWave + 2];    // block numbering
};

__device__ __forceinline__ int visible(const int32_t* len, int row, int T, int Lmax, int m) {
    const int b = row / T;
    const int t = row - b * T;
    return n_visible(len[b], T, t, Lmax, m);    // clamped: never read past Lmax
}

// One workgroup per row (rows of at most 4096 * REG positions when REG > 0).
template <int REG>
__global__ __launch_bounds__(kThreads)
void topk_row_kernel(const float* __restrict__ scores, const int32_t* __restrict__ len,
                     int T, int Lmax, int k, int m, int32_t* __restrict__ idx)
{
    __shared__ TopkShared sh;
    const int row = blockIdx.x;
    const int n = visible(len, row, T, Lmax, m);
    int32_t* out = idx + static_cast<size_t>(row) * k;
    if (n <= k) {                               // every visible position is kept
        for (int j = threadIdx.x; j < k; j += kThreads) out[j] = j < n ? j : -1;
        return;
    }
    Keys<kThreads, REG, ScoreSrc> ks;
    ks.init(ScoreSrc{scores + static_cast<size_t>(row) * Lmax, n, (Lmax & 3) == 0}, n);
    // Direct stores: the slots of neighbouring lanes lie close together, so a store
    // instruction touches few cache lines (staging the slots in LDS first measured
    // 9.9 us against 9.5 us for 32 rows of 8192 keys).
    block_select(ks, k, sh.sel, [&](uint32_t slot, int i, uint32_t) { out[slot] = i; });
}

// Two-stage form, stage 1: chunk c of row r (its visible positions among [C c, C c + C),
// C = 4096 REG) writes its top-min(k, m) keys and positions, in position order, to
// candidate slots [c k, c k + k) of the row; the remaining slots get kNoKey / -1.
// Chunks without a visible position write nothing: stage 2 reads only the candidates
// of the ceil(n / C) chunks that hold the row's n visible positions.
template <int REG>
__global__ __launch_bounds__(kThreads)
void topk_chunk_kernel(const float* __restrict__ scores, const int32_t* __restrict__ len,
                       int T, int Lmax, int k, int m, int n_chunks, uint32_t* __restrict__ cand_key,
                       int32_t* __restrict__ cand_pos)
{
    __shared__ TopkShared sh;
    constexpr int kChunk = REG * kPerIter;
    int row, c;
    if (T == 1 && gridDim.x <= kThreads * kMaxSeqPerThread * n_chunks) {
        // one query row per sequence: only the chunks of rows that need a selection,
        // numbered row after row, so unequal lengths still load the XCDs evenly
        auto count = [&](int r) {
            const int n = visible(len, r, 1, Lmax, m);
            return n > k ? (n + kChunk - 1) / kChunk : 0;
        };
        if (!number_block<kThreads>(blockIdx.x, gridDim.x / n_chunks, count, sh.num, row, c)) return;
    } else {
        // chunk c' of row r runs chunk (c' + r) % n_chunks: a block's XCD follows c', so
        // every XCD gets chunks from the whole length range of the rows
        row = blockIdx.x / n_chunks;
        c = (blockIdx.x - row * n_chunks + row) % n_chunks;
    }
    const int n = visible(len, row, T, Lmax, m);
    if (n <= k) return;                         // stage 2 fills such rows directly
    const int base = c * kChunk;
    if (base >= n) return;                      // not read by stage 2
    const int span = min(kChunk, n - base);
    const size_t slot0 = (static_cast<size_t>(row) * n_chunks + c) * k;
    uint32_t* ck = cand_key + slot0;
    int32_t* cp = cand_pos + slot0;
    const int kept = min(k, span);
    for (int j = kept + threadIdx.x; j < k; j += kThreads) { ck[j] = kNoKey; cp[j] = -1; }
    if (span <= k) {                               // the whole chunk is a candidate set
        const float* sc = scores + static_cast<size_t>(row) * Lmax + base;
        for (int j = threadIdx.x; j < span; j += kThreads) { ck[j] = score_key(sc[j]); cp[j] = base + j; }
        return;
    }
    Keys<kThreads, REG, ScoreSrc> ks;
    ks.init(ScoreSrc{scores + static_cast<size_t>(row) * Lmax + base, span, ((Lmax | base) & 3) == 0}, span);
    block_select(ks, k, sh.sel, [&](uint32_t slot, int i, uint32_t key) { ck[slot] = key; cp[slot] = base + i; });
}

// Two-stage form, stage 2: top-k of a row's candidates (REG = 0: re-read them), those
// of the chunks [0, ceil(n / chunk)) that hold visible positions.
template <int REG>
__global__ __launch_bounds__(kThreads)
void topk_merge_kernel(const uint32_t* __restrict__ cand_key, const int32_t* __restrict__ cand_pos,
                       const int32_t* __restrict__ len, int T, int Lmax, int k, int m, int n_chunks,
                       int chunk, int32_t* __restrict__ idx)
{
    __shared__ TopkShared sh;
    const int row = blockIdx.x;
    const int n = visible(len, row, T, Lmax, m);
    int32_t* out = idx + static_cast<size_t>(row) * k;
    if (n <= k) {
        for (int j = threadIdx.x; j < k; j += kThreads) out[j] = j < n ? j : -1;
        return;
    }
    const int nc = (n + chunk - 1) / chunk * k;
    const size_t off = static_cast<size_t>(row) * n_chunks * k;
    const int32_t* cp = cand_pos + off;
    Keys<kThreads, REG, CandSrc> ks;
    ks.init(CandSrc{cand_key + off, nc, ((n_chunks * k) & 3) == 0}, nc);   // 16-byte aligned rows
    if (k <= kStagedOut) {
        block_select(ks, k, sh.sel, [&](uint32_t slot, int i, uint32_t) { sh.out[slot] = i; });
        __syncthreads();
        for (int j = threadIdx.x; j < k; j += kThreads) out[j] = cp[sh.out[j]];
    } else {
        block_select(ks, k, sh.sel, [&](uint32_t slot, int i, uint32_t) { out[slot] = cp[i]; });
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
        auto kern = a.Lmax <= 2 * kPerIter ? topk_row_kernel<2>
                  : a.Lmax <= kSingleMax   ? topk_row_kernel<4>
                                           : topk_row_kernel<0>;
        return launch_kernel(kPhaseTopk, kern, dim3(rows), block, 0, stream, a.scores, a.len, a.T,
                             a.Lmax, a.k, a.m, a.idx);
    }
    const int nch = n_chunks_for(a.Lmax, a.k);
    const size_t ncand = static_cast<size_t>(rows) * nch * a.k;
    uint32_t* ck = static_cast<uint32_t*>(ws);
    int32_t* cp = reinterpret_cast<int32_t*>(ck + ncand);
    auto chunk_kern = chunk_for(a.Lmax, a.k) == 2 * kPerIter ? topk_chunk_kernel<2> : topk_chunk_kernel<4>;
    hipError_t e = launch_kernel(kPhaseTopk, chunk_kern, dim3(rows * nch), block, 0, stream, a.scores,
                                 a.len, a.T, a.Lmax, a.k, a.m, nch, ck, cp);
    if (e != hipSuccess) return e;
    const long long nc = static_cast<long long>(nch) * a.k;
    const int chunk = chunk_for(a.Lmax, a.k);
    auto merge_kern = nc <= kSingleMax ? topk_merge_kernel<4> : topk_merge_kernel<0>;
    return launch_kernel(kPhaseTopk, merge_kern, dim3(rows), block, 0, stream, ck, cp, a.len, a.T,
                         a.Lmax, a.k, a.m, nch, chunk, a.idx);
}

}  // namespace dsa
