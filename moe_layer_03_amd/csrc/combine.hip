// Combine: weighted local accumulation back into token order.
//
// "Hosting Qwen on Blackwell" (Perplexity), sections "MoE Dispatch - Combine"
// and "Expert Parallel": combine accumulates, with the routing weights, the
// outputs of the experts held by the current rank for every token (the
// cross-rank all-reduce that follows is outside this library).
//
// Gather form: the workgroup that owns token t reads its slot_row/topk_w
// entries (at most K rows), adds w * y_row in ascending slot order in float32
// and writes the whole output row once -- no atomics, deterministic.  Each
// thread handles 8 consecutive features: one 16-byte bf16/fp16 load (or two
// 16-byte float32 loads) per slot, all slots' loads issued before the first
// is summed (K <= 8), then two 16-byte float32 stores.  Small batches
// give each workgroup one token and half of its features, so a few hundred
// tokens still spread over the chip.
#include "common.hpp"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kTokensPerBlock = 2;
constexpr int kMaxSlots = 8;        // local slots held in registers at once (K <= 8)

// 8 consecutive features of one y row (16-bit or float32) as float32.
template <typename YT, bool F16>
struct RowChunk {
    static constexpr int kWords = sizeof(YT) == 2 ? 4 : 8;
    uint32_t v[kWords];
    __device__ __forceinline__ void load(const YT* p) {
        if constexpr (sizeof(YT) == 2) {
            const u32x4 a = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
            for (int d = 0; d < 4; ++d) v[d] = a[d];
        } else {
            const u32x4 a = *reinterpret_cast<const u32x4*>(p);
            const u32x4 b = *reinterpret_cast<const u32x4*>(p + 4);
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                v[d] = a[d];
                v[4 + d] = b[d];
            }
        }
    }
    // acc[i] = fma(w, feature i, acc[i])
    __device__ __forceinline__ void accumulate(float w, float (&acc)[8]) const {
        if constexpr (sizeof(YT) == 2) {
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                float lo, hi;
                if constexpr (F16) {
                    lo = f16_to_f32(static_cast<uint16_t>(v[d] & 0xFFFFu));
                    hi = f16_to_f32(static_cast<uint16_t>(v[d] >> 16));
                } else {
                    lo = __uint_as_float(v[d] << 16);
                    hi = __uint_as_float(v[d] & 0xFFFF0000u);
                }
                acc[2 * d] = fmaf(w, lo, acc[2 * d]);
                acc[2 * d + 1] = fmaf(w, hi, acc[2 * d + 1]);
            }
        } else {
#pragma unroll
            for (int d = 0; d < 8; ++d) acc[d] = fmaf(w, __uint_as_float(v[d]), acc[d]);
        }
    }
};

template <typename YT, bool F16, int TPB>
__global__ __launch_bounds__(kThreads) void combine_kernel(const YT* __restrict__ y, int T, int H, int K,
                                                           const int32_t* __restrict__ slot_row,
                                                           const float* __restrict__ topk_w,
                                                           float* __restrict__ out) {
    // workgroup (x, y): tokens x*TPB .. +TPB-1, features y*CW .. +CW-1
    const int cw = (H + gridDim.y - 1) / gridDim.y;
    const int k_end = min(H, (static_cast<int>(blockIdx.y) + 1) * cw);
    for (int q = 0; q < TPB; ++q) {
        const int t = blockIdx.x * TPB + q;
        if (t >= T) return;
        // the token's local slots in ascending slot order (uniform over the workgroup)
        int rows[kMaxSlots];
        float ws[kMaxSlots];
        int nl = 0;
        if (K <= kMaxSlots) {
            for (int j = 0; j < K; ++j) {
                const int r = slot_row[static_cast<int64_t>(t) * K + j];
                if (r >= 0) {
                    rows[nl] = r;
                    ws[nl] = topk_w[static_cast<int64_t>(t) * K + j];
                    ++nl;
                }
            }
        }
        for (int k = blockIdx.y * cw + threadIdx.x * 8; k < k_end; k += kThreads * 8) {
            float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
            if (K <= kMaxSlots) {
                // every slot's row load in flight before the first is summed; the
                // sum still runs in ascending slot order
                RowChunk<YT, F16> c[kMaxSlots];
#pragma unroll
                for (int i = 0; i < kMaxSlots; ++i)
                    if (i < nl) c[i].load(y + static_cast<int64_t>(rows[i]) * H + k);
#pragma unroll
                for (int i = 0; i < kMaxSlots; ++i)
                    if (i < nl) c[i].accumulate(ws[i], acc);
            } else {
                for (int j = 0; j < K; ++j) {
                    const int r = slot_row[static_cast<int64_t>(t) * K + j];
                    if (r < 0) continue;
                    RowChunk<YT, F16> c;
                    c.load(y + static_cast<int64_t>(r) * H + k);
                    c.accumulate(topk_w[static_cast<int64_t>(t) * K + j], acc);
                }
            }
            float* o = out + static_cast<int64_t>(t) * H + k;
            *reinterpret_cast<floatx4*>(o) = floatx4{acc[0], acc[1], acc[2], acc[3]};
            *reinterpret_cast<floatx4*>(o + 4) = floatx4{acc[4], acc[5], acc[6], acc[7]};
        }
    }
}

}  // namespace

int launch_combine(const moe_shape& s, const void* y_packed, int y_dtype, const int32_t* slot_row,
                   const float* topk_w, float* out, hipStream_t st) {
    // small batches: one token per workgroup and the features split in two, so
    // that even a few hundred tokens spread over the chip; large batches: two
    // tokens per workgroup, whole rows
    const bool small = s.T < 2048;
    const int tpb = small ? 1 : kTokensPerBlock;
    const int ysplit = (small && s.H % (2 * kThreads * 8) == 0) ? 2 : 1;   // each half a whole number of passes
    const dim3 grid((s.T + tpb - 1) / tpb, ysplit);
    if (y_dtype == MOE_BF16) {
        if (small)
            hipLaunchKernelGGL((combine_kernel<uint16_t, false, 1>), grid, dim3(kThreads), 0, st,
                               static_cast<const uint16_t*>(y_packed), s.T, s.H, s.K, slot_row, topk_w, out);
        else
            hipLaunchKernelGGL((combine_kernel<uint16_t, false, kTokensPerBlock>), grid, dim3(kThreads), 0, st,
                               static_cast<const uint16_t*>(y_packed), s.T, s.H, s.K, slot_row, topk_w, out);
    } else if (y_dtype == MOE_F16) {
        if (small)
            hipLaunchKernelGGL((combine_kernel<uint16_t, true, 1>), grid, dim3(kThreads), 0, st,
                               static_cast<const uint16_t*>(y_packed), s.T, s.H, s.K, slot_row, topk_w, out);
        else
            hipLaunchKernelGGL((combine_kernel<uint16_t, true, kTokensPerBlock>), grid, dim3(kThreads), 0, st,
                               static_cast<const uint16_t*>(y_packed), s.T, s.H, s.K, slot_row, topk_w, out);
    } else {
        if (small)
            hipLaunchKernelGGL((combine_kernel<float, false, 1>), grid, dim3(kThreads), 0, st,
                               static_cast<const float*>(y_packed), s.T, s.H, s.K, slot_row, topk_w, out);
        else
            hipLaunchKernelGGL((combine_kernel<float, false, kTokensPerBlock>), grid, dim3(kThreads), 0, st,
                               static_cast<const float*>(y_packed), s.T, s.H, s.K, slot_row, topk_w, out);
    }
    MOE_CHECK_LAUNCH();
    return MOE_OK;
}

}  // namespace moe
