// Helpers shared by the grouped-GEMM translation units (bf16/fp16 and MXFP8):
// epilogue modes and stores, SwiGLU, the per-expert tile prefix scan and the
// raw buffer resource used to read activation rows.
#pragma once

#include "common.hpp"

namespace moe {
namespace {

constexpr int kMaxExperts = 1024;

enum Mode { kPlain = 0, kGateUpPlain = 1, kSwiGLU = 2 };
enum Out { kOutF32 = 0, kOutBF16 = 1, kOutF16 = 2 };

// silu(g) = g / (1 + exp(-g)) with the hardware exp2 and reciprocal (about one
// ulp each, far below the 16-bit rounding of the stored result).
__device__ __forceinline__ float silu(float g) {
    const float e = __builtin_amdgcn_exp2f(-g * 1.4426950408889634f);
    return g * __builtin_amdgcn_rcpf(1.0f + e);
}

template <int OUT> struct OutType { typedef uint16_t type; };
template <> struct OutType<kOutF32> { typedef float type; };

template <int OUT> __device__ __forceinline__ void store_out(typename OutType<OUT>::type* p, float v) {
    if constexpr (OUT == kOutF32) *p = v;
    else if constexpr (OUT == kOutBF16) *p = f32_to_bf16(v);
    else *p = f32_to_f16_sat(v);
}

// Exclusive scan of per-expert row-unit counts (UNIT rows each) into s_mt[0..E_loc].
template <int NTHREADS, int UNIT>
__device__ void build_tile_prefix(const int32_t* __restrict__ offsets, int E_loc, int* s_mt, int* s_tmp) {
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1), wave = tid >> 6;
    constexpr int PER = kMaxExperts / NTHREADS;   // experts per thread
    int local[PER];
    int sum = 0;
#pragma unroll
    for (int q = 0; q < PER; ++q) {
        const int e = tid * PER + q;
        int v = 0;
        if (e < E_loc) v = (offsets[e + 1] - offsets[e] + UNIT - 1) / UNIT;
        local[q] = v;
        sum += v;
    }
    int inc = sum;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const int o = __shfl_up(inc, off, kWave);
        if (lane >= off) inc += o;
    }
    if (lane == kWave - 1) s_tmp[wave] = inc;
    __syncthreads();
    int wbase = 0;
    for (int w = 0; w < wave; ++w) wbase += s_tmp[w];
    int run = wbase + inc - sum;
#pragma unroll
    for (int q = 0; q < PER; ++q) {
        const int e = tid * PER + q;
        if (e <= E_loc) s_mt[e] = run;
        run += local[q];
    }
    if (tid == NTHREADS - 1) s_mt[E_loc] = run;   // total (experts past E_loc add 0)
    __syncthreads();
}

template <int N> struct IntC { static constexpr int value = N; };

// Raw buffer resource over the activation matrix (stride 0, byte-addressed):
// offsets at or past kBufferRange load zeros.  The launcher keeps every valid
// offset below kBufferRange.
constexpr int kBufferRange = 0x7FFFFFFF;
constexpr uint32_t kOutOfRange = 0x80000000u;
constexpr int kBufferFlags = 0x00020000;              // 32-bit data format, the usual gfx9 word 3

// Sum of v over the 256 threads of the workgroup (uniform result).
__device__ __forceinline__ int block_sum256(int v, int* s_w4) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
    __syncthreads();                                   // s_w4 free
    if ((threadIdx.x & (kWave - 1)) == 0) s_w4[threadIdx.x >> 6] = v;
    __syncthreads();
    return s_w4[0] + s_w4[1] + s_w4[2] + s_w4[3];
}

}  // namespace
}  // namespace moe
