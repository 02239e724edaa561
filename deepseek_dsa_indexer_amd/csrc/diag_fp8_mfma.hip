// diag_fp8_mfma.hip -- diagnostic: the same dot products of 128 FP8 (OCP e4m3fn) codes on
// the two gfx950 matrix-core forms the indexer contraction could use.
//
// The score box of "dsa-indexer.excalidraw" forms, per head, the dot product of a 128-wide
// FP8 query row with a 128-wide FP8 key row.  gfx950 offers two ways to run it on the
// matrix cores: the FP8 form (v_mfma_f32_16x16x128_f8f6f4, one instruction per 128 codes)
// and the bf16 form over codes widened exactly to bf16 (four 16x16x32 instructions,
// products exact in fp32, fp32 accumulation).  This kernel runs both over the same pairs
// so that their errors can be measured against exact sums; the index kernels use the bf16
// form because of what that measurement shows (the FP8 form aligns the products of one
// instruction to a few more bits than fp32 keeps after the largest of them).
#include "dsa_device.h"
#include "dsa_internal.h"

namespace dsa {

namespace {

// One wave per 16 pairs: A holds the 16 first rows, B the 16 second rows, and the
// diagonal of the 16x16 product is the 16 pair dots.  Both forms give lane l row (or
// column) l % 16 and a quarter of K by lane group l / 16 -- the same K assignment for both
// operands, which is all a dot product needs.  Output lane l holds rows 4 (l / 16) + i of
// column l % 16, so element (j, j) sits in lane j + 16 (j / 4), element j % 4.
__global__ __launch_bounds__(kWave)
void diag_fp8_dots_kernel(const uint8_t* __restrict__ a, const uint8_t* __restrict__ b,
                          float* __restrict__ out_fp8, float* __restrict__ out_bf16)
{
    const int lane = threadIdx.x;
    const int r = lane & 15;
    const int g = lane >> 4;
    const size_t p = static_cast<size_t>(blockIdx.x) * 16 + r;
    const uint8_t* ar = a + p * 128;
    const uint8_t* br = b + p * 128;

    const v8i av = *reinterpret_cast<const v8i*>(ar + 32 * g);
    const v8i bv = *reinterpret_cast<const v8i*>(br + 32 * g);
    const v4f c8 = mfma_fp8_16x16x128(av, bv, v4f{0.f, 0.f, 0.f, 0.f});

    v4f cb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        const int2 x = *reinterpret_cast<const int2*>(ar + 32 * ks + 8 * g);
        const int2 y = *reinterpret_cast<const int2*>(br + 32 * ks + 8 * g);
        cb = mfma_bf16_16x16x32(fp8x8_to_bf16(x.x, x.y), fp8x8_to_bf16(y.x, y.y), cb);
    }
    if (g == (r >> 2)) {
        const size_t q = static_cast<size_t>(blockIdx.x) * 16 + r;
        const int e = r & 3;
        out_fp8[q] = e == 0 ? c8[0] : e == 1 ? c8[1] : e == 2 ? c8[2] : c8[3];
        out_bf16[q] = e == 0 ? cb[0] : e == 1 ? cb[1] : e == 2 ? cb[2] : cb[3];
    }
}

}  // namespace

hipError_t launch_diag_fp8_dots(const uint8_t* a, const uint8_t* b, int n, float* out_fp8,
                                float* out_bf16, hipStream_t stream) {
    return launch_kernel(kPhaseNone, diag_fp8_dots_kernel, dim3(n / 16), dim3(kWave), 0, stream, a, b,
                         out_fp8, out_bf16);
}

}  // namespace dsa
