// Router launch that lets spare CUs warm the last-level cache for the kernel
// that follows it (the fused layer's small-batch path).
#pragma once

#include "common.hpp"

namespace moe {

// A device region that the kernel after the router streams: routing kernels
// with spare CUs read it meanwhile, so it is in the last-level cache by then.
struct CachePrefetch {
    const void* region = nullptr;
    size_t bytes = 0;   // whole KiB are read
};

// MI355X's last-level (Infinity) cache: regions larger than this are not prefetched.
constexpr size_t kLastLevelCacheBytes = static_cast<size_t>(256) << 20;

// launch_route, with the small-batch router's spare CUs reading pf meanwhile
// (other router kernels ignore pf).
int launch_route_prefetch(const moe_shape& s, const void* x, int x_dtype, const void* w, const float* bias,
                          int32_t* topk_idx, float* topk_w, float* logits, void* ws, size_t ws_bytes,
                          hipStream_t st, CachePrefetch pf);

}  // namespace moe
