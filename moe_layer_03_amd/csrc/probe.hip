// Measurement helper, not part of the layer: a dense bf16 MFMA issue-rate
// probe, so that throughput can be reported against the rate this chip
// reaches under the same clocks, next to the published peak.
//
// Each wave keeps eight independent 32x32x16 accumulators busy (no memory
// traffic inside the loop); 8 waves per workgroup, two per SIMD.
#include "common.hpp"

namespace moe {
namespace {

constexpr int kProbeWaves = 8;
constexpr int kProbeAcc = 8;

__global__ __launch_bounds__(kProbeWaves * 64) void mfma_rate_kernel(int iters, float* __restrict__ sink) {
    u32x4 a, b;
    const uint32_t t = threadIdx.x;
    a[0] = 0x3F803F80u ^ t;   // bf16 pairs near 1.0, varied per lane
    a[1] = 0x3F003F00u;
    a[2] = 0x3E803E80u;
    a[3] = 0x3F403F40u;
    b = a;
    floatx16 acc[kProbeAcc];
#pragma unroll
    for (int j = 0; j < kProbeAcc; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[j][v] = 0.0f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < kProbeAcc; ++j)
            acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                             __builtin_bit_cast(bf16x8_t, b), acc[j], 0, 0, 0);
    }
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < kProbeAcc; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) s += acc[j][v];
    sink[static_cast<int64_t>(blockIdx.x) * blockDim.x + t] = s;
}

}  // namespace
}  // namespace moe

extern "C" {

int64_t moe_probe_mfma_bf16_flops(int blocks, int iters) {
    if (blocks <= 0 || iters <= 0) return 0;
    return static_cast<int64_t>(blocks) * moe::kProbeWaves * iters * moe::kProbeAcc * (2 * 32 * 32 * 16);
}

int moe_probe_mfma_bf16(int blocks, int iters, float* sink, void* stream) {
    if (blocks <= 0 || iters <= 0 || sink == nullptr) return MOE_ERR_INVALID_ARG;
    hipLaunchKernelGGL(moe::mfma_rate_kernel, dim3(blocks), dim3(moe::kProbeWaves * 64), 0,
                       static_cast<hipStream_t>(stream), iters, sink);
    MOE_CHECK_LAUNCH();
    return MOE_OK;
}

}  // extern "C"
