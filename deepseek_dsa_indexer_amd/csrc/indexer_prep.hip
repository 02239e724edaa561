// indexer_prep.hip -- the indexer's per-token preparation, between the projections and
// the scores ("DeepSeek-V3.2-Exp - Split indexer heads", Indexer.forward excerpt): each
// query head row and the key row of a new token get rope on their leading rope columns
// ("not interleaved": column j pairs with column j + R/2), the rotation of the whole row
// (read as the orthonormal Walsh-Hadamard transform, Sylvester order), and blockwise FP8
// quantisation with one fp32 scale per row (scale = max(amax, 1e-12) / 448, codes rounded
// to the nearest e4m3fn value, ties to even); the key codes and scale are written into
// the key cache at the token's position.
//
// Rows (64 query heads + the key per token at the V3.2 sizes) go to groups of D / 8 lanes,
// fp32 throughout; cross-lane steps are DPP moves inside 16-lane rows.  HBM-bound: per
// token 16 KB of bf16 queries read, 8 KB of codes written.
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

// Value of lane l ^ M within its row of 16 lanes (M = 1, 2, 4, 8), by DPP moves: quad
// permutations for 1 and 2; a half-row mirror (l ^ 7) then a quad reversal (l ^ 3) for 4;
// a row mirror (l ^ 15) then a half-row mirror for 8.
template <int M>
__device__ __forceinline__ float xor_lane(float v) {
    const int x = __float_as_int(v);
    if constexpr (M == 1) return __int_as_float(__builtin_amdgcn_mov_dpp(x, 0xB1, 0xf, 0xf, false));
    else if constexpr (M == 2) return __int_as_float(__builtin_amdgcn_mov_dpp(x, 0x4E, 0xf, 0xf, false));
    else if constexpr (M == 4)
        return __int_as_float(__builtin_amdgcn_mov_dpp(__builtin_amdgcn_mov_dpp(x, 0x141, 0xf, 0xf, false),
                                                       0x1B, 0xf, 0xf, false));
    else
        return __int_as_float(__builtin_amdgcn_mov_dpp(__builtin_amdgcn_mov_dpp(x, 0x140, 0xf, 0xf, false),
                                                       0x141, 0xf, 0xf, false));
}

__device__ __forceinline__ float xor_lane_rt(float v, int m) {
    switch (m) {
    case 1: return xor_lane<1>(v);
    case 2: return xor_lane<2>(v);
    case 4: return xor_lane<4>(v);
    default: return xor_lane<8>(v);
    }
}

// Rows of D values are handled by groups of D / 8 lanes, lane n of a group holding
// columns 8n .. 8n+7, so a wave prepares 64 / (D / 8) rows at once: butterflies of
// distance 1, 2, 4 stay in the lane, distance 8m pairs lane n with lane n ^ m.
template <int D>
__global__ __launch_bounds__(kPrepThreads)
void indexer_prep_kernel(IndexerPrepArgs a) {
    constexpr int LPR = D / 8;                        // lanes per row
    constexpr int RPW = kWave / LPR;                  // rows per wave
    const int lane = threadIdx.x & (kWave - 1);
    const int n = lane % LPR;
    const long long gr = (static_cast<long long>(blockIdx.x) * kPrepWaves + threadIdx.x / kWave) * RPW +
                         lane / LPR;
    const int rows_per_token = a.H + 1;
    const long long n_rows = static_cast<long long>(a.B) * a.T * rows_per_token;
    bool live = gr < n_rows;
    const int token = live ? static_cast<int>(gr / rows_per_token) : 0;   // b * T + t
    const int r = live ? static_cast<int>(gr - static_cast<long long>(token) * rows_per_token) : 0;
    const int b = token / a.T;
    const int t = token - b * a.T;
    const int pos = a.start[b] + t;
    live = live && pos >= 0 && pos < a.P && pos < a.Lmax;   // outside the tables or the cache: skip
    const bool is_key = r == a.H;
    const void* src = is_key ? a.k : a.q;
    const size_t off = (is_key ? static_cast<size_t>(token) : static_cast<size_t>(token) * a.H + r) * D + 8 * n;

    float v[8];
    if (live) {
        if (a.bf16) {
            const uint4 w = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(src) + off);
            const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                v[2 * i] = __uint_as_float(ws[i] << 16);
                v[2 * i + 1] = __uint_as_float(ws[i] & 0xffff0000u);
            }
        } else {
            const float4 lo = *reinterpret_cast<const float4*>(static_cast<const float*>(src) + off);
            const float4 hi = *reinterpret_cast<const float4*>(static_cast<const float*>(src) + off + 4);
            v[0] = lo.x; v[1] = lo.y; v[2] = lo.z; v[3] = lo.w;
            v[4] = hi.x; v[5] = hi.y; v[6] = hi.z; v[7] = hi.w;
        }
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = 0.f;
    }

    // rope: column e < R/2 pairs with e + R/2
    const int R = a.R;
    const float* cs = a.cos + static_cast<size_t>(pos) * (R / 2);
    const float* sn = a.sin + static_cast<size_t>(pos) * (R / 2);
    if (R >= 16) {
        const int m = R / 16;                         // partner lane distance (power of two)
        float p[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) p[i] = xor_lane_rt(v[i], m);
        if (live && 8 * n < R) {
            const bool lo = 8 * n < R / 2;
            const int j0 = lo ? 8 * n : 8 * n - R / 2;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float c = cs[j0 + i], s = sn[j0 + i];
                v[i] = lo ? v[i] * c - p[i] * s : p[i] * s + v[i] * c;
            }
        }
    } else if (R > 0 && live && n == 0) {             // R = 4 or 8: the pairs sit in lane 0
        const int h = R / 2;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (i < h) {
                const float c = cs[i], s = sn[i];
                const float x0 = v[i], x1 = v[i + h];
                v[i] = x0 * c - x1 * s;
                v[i + h] = x0 * s + x1 * c;
            }
        }
    }

    // Walsh-Hadamard butterflies: the lower column of each pair gets a + b, the upper a - b
#pragma unroll
    for (int dist = 1; dist < 8; dist <<= 1)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if (i & dist) continue;
            const float x0 = v[i], x1 = v[i + dist];
            v[i] = x0 + x1;
            v[i + dist] = x0 - x1;
        }
#pragma unroll
    for (int m = 1; m < LPR; m <<= 1) {
        const bool upper = (n & m) != 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float p = xor_lane_rt(v[i], m);
            v[i] = upper ? p - v[i] : v[i] + p;
        }
    }
    const float norm = 1.0f / __builtin_sqrtf(static_cast<float>(D));
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        v[i] *= norm;
        amax = fmaxf(amax, fabsf(v[i]));
    }
#pragma unroll
    for (int m = 1; m < LPR; m <<= 1) amax = fmaxf(amax, xor_lane_rt(amax, m));
    const float scale = __fdiv_rn(fmaxf(amax, 1e-12f), 448.0f);
    uint32_t c0 = 0, c1 = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float y = fminf(fmaxf(__fdiv_rn(v[i], scale), -448.0f), 448.0f);
        if (i < 4) c0 |= e4m3fn_code(y) << (8 * i);
        else c1 |= e4m3fn_code(y) << (8 * (i - 4));
    }
    if (!live) return;
    uint8_t* codes;
    float* scale_out;
    if (is_key) {
        const size_t kr = static_cast<size_t>(b) * a.Lmax + pos;
        codes = a.k_cache + kr * D;
        scale_out = a.k_scale + kr;
    } else {
        const size_t qr = static_cast<size_t>(token) * a.H + r;
        codes = a.q_fp8 + qr * D;
        scale_out = a.q_scale + qr;
    }
    *reinterpret_cast<uint2*>(codes + 8 * n) = uint2{c0, c1};
    if (n == 0) *scale_out = scale;
}

}  // namespace

hipError_t launch_indexer_prep(const IndexerPrepArgs& a, hipStream_t stream) {
    const long long rows = static_cast<long long>(a.B) * a.T * (a.H + 1);
    const long long rows_per_block = static_cast<long long>(kPrepWaves) * (kWave / (a.D / 8));
    const dim3 grid(static_cast<unsigned>((rows + rows_per_block - 1) / rows_per_block)), block(kPrepThreads);
    switch (a.D) {
    case 32: hipLaunchKernelGGL(indexer_prep_kernel<32>, grid, block, 0, stream, a); break;
    case 64: hipLaunchKernelGGL(indexer_prep_kernel<64>, grid, block, 0, stream, a); break;
    default: hipLaunchKernelGGL(indexer_prep_kernel<128>, grid, block, 0, stream, a); break;
    }
    return hipGetLastError();
}

}  // namespace dsa
