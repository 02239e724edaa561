// indexer_prep.hip -- the indexer's per-token preparation, between the projections and
// the scores ("DeepSeek-V3.2-Exp - Split indexer heads", Indexer.forward excerpt): each
// query head row and the key row of a new token get rope on their leading rope columns
// ("not interleaved": column j pairs with column j + R/2), the rotation of the whole row
// (read as the orthonormal Walsh-Hadamard transform, Sylvester order), and blockwise FP8
// quantisation with one fp32 scale per row (scale = max(amax, 1e-12) / 448, codes rounded
// to the nearest e4m3fn value, ties to even); the key codes and scale are written into
// the key cache at the token's position.
//
// One wave per row (64 query heads + the key per token at the V3.2 sizes), fp32.  A
// lane holds EPL = max(1, D / 64) neighbouring columns, so the Walsh-Hadamard butterflies
// of distance < EPL stay in the lane and the others pair lane l with lane l ^ (dist /
// EPL).  HBM-bound and tiny: per token 16 KB of bf16 queries read, 8 KB of codes written.
#include "dsa_device.h"
#include "dsa_internal.h"

namespace dsa {

namespace {

constexpr int kPrepThreads = 256;
constexpr int kPrepWaves = kPrepThreads / kWave;

// OCP e4m3fn code of y, |y| <= 448: nearest magnitude, ties to the even code, the sign
// bit taken from y.  Integer rounding of the fp32 mantissa to 3 bits for normal results,
// y * 2^9 rounded to an integer in the subnormal range (step 2^-9; 8 is the smallest
// normal, 2^-6, whose code is also 8).
__device__ __forceinline__ uint32_t e4m3fn_code(float y) {
    const uint32_t u = __float_as_uint(y);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t a = u & 0x7fffffffu;
    uint32_t mag;
    if (a < 0x3c800000u) {                            // |y| < 2^-6
        mag = static_cast<uint32_t>(__builtin_rintf(__uint_as_float(a) * 512.0f));
    } else {
        const uint32_t e = (a >> 23) - 127u + 7u;     // e4m3 exponent field (1 .. 15)
        const uint32_t m = a & 0x7fffffu;
        const uint32_t keep = m >> 20;
        const uint32_t rem = m & 0xfffffu;
        const uint32_t up = (rem > 0x80000u || (rem == 0x80000u && (keep & 1u))) ? 1u : 0u;
        mag = (e << 3) + keep + up;                   // a carry moves into the exponent
    }
    return sign | mag;
}

__device__ __forceinline__ float ld_in(const void* p, size_t i, int bf16) {
    return bf16 ? bf16_to_f32(static_cast<const uint16_t*>(p)[i]) : static_cast<const float*>(p)[i];
}

// One row: rope, rotation, quantisation.  src: D input values (bf16 or f32); codes: D
// bytes out; returns the scale (every lane).
template <int D>
__device__ __forceinline__ float prep_row(const void* src, size_t off, int bf16, const float* cs,
                                          const float* sn, int R, int lane, uint8_t* codes) {
    constexpr int EPL = D >= 64 ? D / 64 : 1;
    constexpr int kLanes = D / EPL;                   // lanes that hold columns
    const bool holds = lane < kLanes;
    float v[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i)
        v[i] = holds ? ld_in(src, off + EPL * lane + i, bf16) : 0.f;
    // rope: column e < R/2 pairs with e + R/2 (same slot i in lane (e + R/2) / EPL)
    const int half = R / 2;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int e = EPL * lane + i;
        const bool lo = e < half;
        const int pe = lo ? e + half : e - half;
        const float p = __shfl(v[i], (e < R ? pe : e) / EPL);
        if (holds && e < R) {
            const int j = lo ? e : pe;
            const float c = cs[j], s = sn[j];
            v[i] = lo ? v[i] * c - p * s : p * s + v[i] * c;
        }
    }
    // Walsh-Hadamard butterflies: the lower column of each pair gets a + b, the upper a - b
#pragma unroll
    for (int dist = 1; dist < D; dist <<= 1) {
        if (dist < EPL) {
#pragma unroll
            for (int i = 0; i < EPL; ++i) {
                if (i & dist) continue;
                const float a = v[i], b = v[i + dist];
                v[i] = a + b;
                v[i + dist] = a - b;
            }
        } else {
            const int ld = dist / EPL;
            const bool upper = (lane & ld) != 0;
#pragma unroll
            for (int i = 0; i < EPL; ++i) {
                const float p = __shfl_xor(v[i], ld);
                v[i] = upper ? p - v[i] : v[i] + p;
            }
        }
    }
    const float norm = 1.0f / __builtin_sqrtf(static_cast<float>(D));
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        v[i] *= norm;
        amax = fmaxf(amax, fabsf(v[i]));
    }
    amax = wave_max(amax);
    const float scale = __fdiv_rn(fmaxf(amax, 1e-12f), 448.0f);
    uint32_t packed = 0;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const float y = fminf(fmaxf(__fdiv_rn(v[i], scale), -448.0f), 448.0f);
        packed |= e4m3fn_code(y) << (8 * i);
    }
    if (holds) {
        if constexpr (EPL == 2) reinterpret_cast<uint16_t*>(codes)[lane] = static_cast<uint16_t>(packed);
        else codes[lane] = static_cast<uint8_t>(packed);
    }
    return scale;
}

// One wave per row: the H query rows of token (b, t) and then its key row, so that every
// row's loads are in flight at once (a row is one memory latency plus a few hundred
// cycles of shuffles; walking rows one after another per wave made the step latency-bound).
template <int D>
__global__ __launch_bounds__(kPrepThreads)
void indexer_prep_kernel(IndexerPrepArgs a) {
    const int lane = threadIdx.x & (kWave - 1);
    const long long gr = static_cast<long long>(blockIdx.x) * kPrepWaves + threadIdx.x / kWave;
    const int rows_per_token = a.H + 1;
    if (gr >= static_cast<long long>(a.B) * a.T * rows_per_token) return;
    const int token = static_cast<int>(gr / rows_per_token);   // b * T + t
    const int r = static_cast<int>(gr - static_cast<long long>(token) * rows_per_token);
    const int b = token / a.T;
    const int t = token - b * a.T;
    const int pos = a.start[b] + t;
    if (pos < 0 || pos >= a.P || pos >= a.Lmax) return;   // outside the tables or the cache
    const float* cs = a.cos + static_cast<size_t>(pos) * (a.R / 2);
    const float* sn = a.sin + static_cast<size_t>(pos) * (a.R / 2);
    if (r < a.H) {
        const size_t qr = static_cast<size_t>(token) * a.H + r;
        const float sc = prep_row<D>(a.q, qr * D, a.bf16, cs, sn, a.R, lane, a.q_fp8 + qr * D);
        if (lane == 0) a.q_scale[qr] = sc;
    } else {
        const size_t kr = static_cast<size_t>(b) * a.Lmax + pos;
        const float sc = prep_row<D>(a.k, static_cast<size_t>(token) * D, a.bf16, cs, sn, a.R, lane,
                                     a.k_cache + kr * D);
        if (lane == 0) a.k_scale[kr] = sc;
    }
}

}  // namespace

hipError_t launch_indexer_prep(const IndexerPrepArgs& a, hipStream_t stream) {
    const long long rows = static_cast<long long>(a.B) * a.T * (a.H + 1);
    const dim3 grid(static_cast<unsigned>((rows + kPrepWaves - 1) / kPrepWaves)), block(kPrepThreads);
    switch (a.D) {
    case 32: hipLaunchKernelGGL(indexer_prep_kernel<32>, grid, block, 0, stream, a); break;
    case 64: hipLaunchKernelGGL(indexer_prep_kernel<64>, grid, block, 0, stream, a); break;
    default: hipLaunchKernelGGL(indexer_prep_kernel<128>, grid, block, 0, stream, a); break;
    }
    return hipGetLastError();
}

}  // namespace dsa
