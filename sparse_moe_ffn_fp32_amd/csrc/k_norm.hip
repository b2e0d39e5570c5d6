// RMS normalisation of the residual stream on the way into the FFN.
//
// qwen35moe Forward-Pass Design, "Block scaffold": each layer is a pre-norm
// sandwich, the shared-MoE FFN reads the post-attention RMS-normalised
// stream and its output is added to the un-normalised input.  ds4.c study
// notes Part 3, section 3, trace 1 (RMS normalisation):
//   out[i] = x[i] / sqrt(mean(x^2) + eps) * weight[i],
// with the squares accumulated in double.  Here one wave normalises one
// token row of 2048 bf16 values entirely in double: each lane takes 32
// consecutive values, sums their squares in a fixed order, the wave sums the
// 64 partials in a fixed order, and each product x * scale * weight is
// rounded once, correctly, to bf16 (the FFN's input type).  A double
// computation rounds to the same bf16 as any other accurate one except when
// a product lies within a few double ulps of a halfway point between two
// bf16 values, so the normalised rows match an fp64 reference bit for bit
// in practice; an fp32 computation would flip a few elements per hundred
// thousand.  The work is tiny (a few fp64 operations per element).
#include "moe_common.h"
#include "moe_kernels.h"

namespace moe {

// Nearest bf16 of a double, ties to even: round to fp32 by truncation with a
// sticky last bit (round to odd: 24 bits keep the information the second
// rounding needs), then to bf16 to nearest even.  Finite values only.
__device__ __forceinline__ uint16_t f64_to_bf16_rne(double d) {
    const float f = (float)d;
    uint32_t u = __float_as_uint(f);
    const double back = (double)f;
    if (back != d) {
        if (__builtin_fabs(back) > __builtin_fabs(d)) u -= 1;  // one fp32 ulp toward zero
        u |= 1u;
    }
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ double wave_sum_f64(double v) {
    // fixed xor butterfly: every lane ends with the same, order-fixed value
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
    return v;
}

__global__ void __launch_bounds__(256) k_rmsnorm(const uint16_t* __restrict__ h, const float* __restrict__ w, float eps,
                                                uint16_t* __restrict__ xn, int T) {
    const int lane = threadIdx.x & 63;
    const int t = 4 * blockIdx.x + (threadIdx.x >> 6);
    if (t >= T) return;  // the whole wave
    const uint16_t* row = h + (size_t)t * D + 32 * lane;
    u32x4 v[4];
#pragma unroll
    for (int i = 0; i < 4; i++) v[i] = *(const u32x4*)(row + 8 * i);
    f32x4 wv[8];
#pragma unroll
    for (int i = 0; i < 8; i++) wv[i] = *(const f32x4*)(w + 32 * lane + 4 * i);
    double ss = 0.0;
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const uint32_t d = v[i][j];
            const double lo = (double)bf16_to_f32(d & 0xffffu), hi = (double)bf16_to_f32(d >> 16);
            ss += lo * lo;
            ss += hi * hi;
        }
    ss = wave_sum_f64(ss);
    const double scale = 1.0 / __builtin_sqrt(ss / (double)D + (double)eps);
    u32x4 o[4];
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const uint32_t d = v[i][j];
            const int k = 8 * i + 2 * j;  // element index within the lane's 32
            const double lo = (double)bf16_to_f32(d & 0xffffu) * scale * (double)wv[k >> 2][k & 3];
            const double hi = (double)bf16_to_f32(d >> 16) * scale * (double)wv[(k + 1) >> 2][(k + 1) & 3];
            o[i][j] = (uint32_t)f64_to_bf16_rne(lo) | ((uint32_t)f64_to_bf16_rne(hi) << 16);
        }
    uint16_t* orow = xn + (size_t)t * D + 32 * lane;
#pragma unroll
    for (int i = 0; i < 4; i++) *(u32x4*)(orow + 8 * i) = o[i];
}

hipError_t launch_rmsnorm(const uint16_t* h, const float* w, float eps, uint16_t* xn, int T, hipStream_t s) {
    if (T <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_rmsnorm, dim3((T + 3) / 4), dim3(256), 0, s, h, w, eps, xn, T);
    return hipGetLastError();
}

}  // namespace moe
