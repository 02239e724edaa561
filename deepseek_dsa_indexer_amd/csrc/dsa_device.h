// dsa_device.h -- device-side helpers shared by the gfx950 kernels of libdsa_amd.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef short v8s __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
    return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// Round to nearest even (NaN stays NaN): the gfx950 conversion instruction
// (v_cvt_pk_bf16_f32), one VALU operation per pair and no branches.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

// 8 FP8 (OCP e4m3fn) bytes, two dwords, -> 8 bf16, byte order kept.  Exact: every
// e4m3fn value is a bf16 value (the scale operand of the conversion is 1).
__device__ __forceinline__ v8bf fp8x8_to_bf16(int d0, int d1) {
    const v2bf a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, 1.0f, false);
    const v2bf b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, 1.0f, true);
    const v2bf c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, 1.0f, false);
    const v2bf d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, 1.0f, true);
    return v8bf{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// One FP8 (OCP e4m3fn) byte -> float, exactly.
__device__ __forceinline__ float fp8_to_f32(uint8_t c) {
    return static_cast<float>(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(static_cast<int>(c), 1.0f, false)[0]);
}

// 1 / x for a normalising sum (x > 0): the hardware reciprocal (about 1 ulp), which is
// far inside the bf16 rounding the results get.
__device__ __forceinline__ float recip(float x) { return __builtin_amdgcn_rcpf(x); }

// 2^x for softmax numerators: the transcendental unit's v_exp_f32 (about 1 ulp), with no
// range reduction for subnormal results -- those flush to zero, which a numerator never
// needs, since each softmax row also holds a numerator of at least 1.  2^-inf = 0.
__device__ __forceinline__ float exp2_num(float x) { return __builtin_amdgcn_exp2f(x); }

// Cache rows visible to query row t of a call with T rows over a sequence of len
// positions, in a cache of Lmax rows.  m = 1: every position is a cache row and row t
// sits at position min(len, Lmax) - T + t, so that many rows plus one are visible.  m > 1:
// the cache holds compressed entries, each standing for m consecutive positions, and
// entry e is available to the query at position p = len - T + t iff e < (p + 1) / m.
__device__ __forceinline__ int n_visible(int len, int T, int t, int Lmax, int m) {
    return m == 1 ? min(len, Lmax) - T + t + 1 : min((len - T + t + 1) / m, Lmax);
}

// 16x16x128 FP8 (OCP e4m3fn) matrix-core product, fp32 accumulate.
// Lane l supplies row (l % 16) of A and column (l % 16) of B, 32 bytes each; the four
// lane groups (l / 16) cover disjoint quarters of K.  Output lane l holds rows
// 4 * (l / 16) + i, i = 0..3, of column l % 16.
__device__ __forceinline__ v4f mfma_fp8_16x16x128(const v8i& a, const v8i& b, const v4f& c) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// 16x16x32 bf16 matrix-core product: lane l supplies 8 K-values of row/column l % 16
// (lane group l / 16 selects the K slice); output layout as above.
__device__ __forceinline__ v4f mfma_bf16_16x16x32(const v8bf& a, const v8bf& b, const v4f& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 32x32x16 bf16 matrix-core product (twice the work of the 16x16x32 form in about the
// same issue time on gfx950): lane l supplies 8 K-values of row/column l % 32, lane
// half l / 32 selecting the K slice; output element r of lane l is
// D[8 (r / 4) + 4 (l / 32) + r % 4][l % 32].
typedef float v16f __attribute__((ext_vector_type(16)));
__device__ __forceinline__ v16f mfma_bf16_32x32x16(const v8bf& a, const v8bf& b, const v16f& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
    return v;
}

// ---- cross-lane steps on the VALU (DPP and the gfx950 lane-swap instructions) rather
// than through the LDS crossbar (ds_bpermute, about a hundred cycles per step).
// DPP controls: row_shr:n = 0x110 + n, row_ror:n = 0x120 + n, row_bcast:15 = 0x142,
// row_bcast:31 = 0x143 (rows are 16 lanes).
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
    // lanes without a source, and rows outside ROW_MASK, read 0
    return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), CTRL, ROW_MASK, 0xf, false));
}

// v_permlane16_swap / v_permlane32_swap with the same register on both sides: the pair
// holds, in some order, this lane's value and that of lane l ^ 16 (l ^ 32), so a
// commutative operation on the pair gives the same result in both lanes.
__device__ __forceinline__ void pair16(uint32_t v, uint32_t& a, uint32_t& b) {
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    a = r[0]; b = r[1];
}
__device__ __forceinline__ void pair32(uint32_t v, uint32_t& a, uint32_t& b) {
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    a = r[0]; b = r[1];
}
__device__ __forceinline__ float max_xor16(float v) {
    uint32_t a, b; pair16(__float_as_uint(v), a, b); return fmaxf(__uint_as_float(a), __uint_as_float(b));
}
__device__ __forceinline__ float max_xor32(float v) {
    uint32_t a, b; pair32(__float_as_uint(v), a, b); return fmaxf(__uint_as_float(a), __uint_as_float(b));
}
__device__ __forceinline__ float sum_xor16(float v) {
    uint32_t a, b; pair16(__float_as_uint(v), a, b); return __uint_as_float(a) + __uint_as_float(b);
}
__device__ __forceinline__ float sum_xor32(float v) {
    uint32_t a, b; pair32(__float_as_uint(v), a, b); return __uint_as_float(a) + __uint_as_float(b);
}
// The value of lane l ^ 32; `lane` is this lane's index in the wave.
__device__ __forceinline__ float from_xor32(float v, int lane) {
    uint32_t a, b; pair32(__float_as_uint(v), a, b); return __uint_as_float((lane & 32) ? a : b);
}

// Inclusive prefix sum over the 64 lanes of a wave: Hillis-Steele within each 16-lane
// row, then the row totals carried across rows by broadcasts.
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t v, int) {
    v += dpp<0x111>(v);
    v += dpp<0x112>(v);
    v += dpp<0x114>(v);
    v += dpp<0x118>(v);
    v += dpp<0x142, 0xa>(v);
    v += dpp<0x143, 0xc>(v);
    return v;
}

// Minimum / maximum over the wave, in every lane.
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
    v = min(v, dpp<0x128>(v)); v = min(v, dpp<0x124>(v));
    v = min(v, dpp<0x122>(v)); v = min(v, dpp<0x121>(v));
    uint32_t a, b;
    pair16(v, a, b); v = min(a, b);
    pair32(v, a, b); return min(a, b);
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = max(v, dpp<0x128>(v)); v = max(v, dpp<0x124>(v));
    v = max(v, dpp<0x122>(v)); v = max(v, dpp<0x121>(v));
    uint32_t a, b;
    pair16(v, a, b); v = max(a, b);
    pair32(v, a, b); return max(a, b);
}

// Work numbering for launches over the sequences of a batch whose sequences need
// unequal numbers of blocks (count(b) >= 0 for b < n_seq).  The blocks of sequence b
// take ids P(b) .. P(b) + count(b) - 1, P the exclusive prefix sum, so consecutive ids
// walk through one sequence after another.  The dispatcher hands consecutive
// workgroups to the 8 XCDs in turn, so every XCD gets an equal share of the work
// however unequal the sequences are, and no workgroup is spent on a block past a
// sequence's end: ids beyond the total return false (the same in every thread).
// Every thread of the NT-thread block must call it; thread t counts sequences
// [t * per, t * per + per), per = ceil(n_seq / NT).  sh: NT / 64 + 2 ints of LDS.
template <int NT, typename Count>
__device__ __forceinline__ bool numbered_block(int id, int n_seq, Count count, int* sh, int& seq,
                                               int& blk) {
    constexpr int kWaves = NT / kWave;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int per = (n_seq + NT - 1) / NT;
    const int s0 = threadIdx.x * per;
    int mine = 0;
    for (int i = 0; i < per; ++i) mine += s0 + i < n_seq ? count(s0 + i) : 0;
    const int inc = static_cast<int>(wave_inclusive_scan(static_cast<uint32_t>(mine), lane));
    if (lane == kWave - 1) sh[wave] = inc;
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        const int x = sh[w];
        before += w < wave ? x : 0;
        total += x;
    }
    int base = before + inc - mine;
    if (id >= base && id < base + mine) {
        for (int i = 0; i < per; ++i) {
            const int c = s0 + i < n_seq ? count(s0 + i) : 0;
            if (id < base + c) {
                sh[kWaves] = s0 + i;
                sh[kWaves + 1] = id - base;
                break;
            }
            base += c;
        }
    }
    __syncthreads();
    if (id >= total) return false;
    seq = sh[kWaves];
    blk = sh[kWaves + 1];
    return true;
}

// The same numbering for n_seq <= 64, worked out by every wave on its own: lane l
// counts sequence l, a wave scan gives each sequence's first id, and the lane whose
// range holds `id` names the sequence.  No LDS and no block barrier.
template <typename Count>
__device__ __forceinline__ bool numbered_block_wave(int id, int n_seq, Count count, int& seq, int& blk) {
    const int lane = threadIdx.x & (kWave - 1);
    const int mine = lane < n_seq ? count(lane) : 0;
    const int inc = static_cast<int>(wave_inclusive_scan(static_cast<uint32_t>(mine), lane));
    const int total = __builtin_amdgcn_readlane(inc, kWave - 1);
    if (id >= total) return false;
    const int first = inc - mine;
    const unsigned long long own = __ballot(id >= first && id < inc);   // exactly one lane
    const int s = __builtin_amdgcn_readfirstlane(__ffsll(static_cast<long long>(own)) - 1);
    seq = s;
    blk = id - __builtin_amdgcn_readlane(first, s);
    return true;
}

// Either form, by batch size (uniform over the block).
template <int NT, typename Count>
__device__ __forceinline__ bool number_block(int id, int n_seq, Count count, int* sh, int& seq, int& blk) {
    if (n_seq <= kWave) return numbered_block_wave(id, n_seq, count, seq, blk);
    return numbered_block<NT>(id, n_seq, count, sh, seq, blk);
}

}  // namespace dsa
