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
