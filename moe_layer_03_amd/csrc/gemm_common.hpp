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


constexpr int kDeriveMaxT = 1024;      // tokens of a derived dispatch (one expert's row list in LDS)
constexpr int kDeriveMaxE = 1024;

// The dispatch of expert e derived in the workgroup from the routing: the
// histogram of local experts gives the expert's first row (the exclusive sum
// over the experts before it) and row count, and an order-keeping compaction of
// the (token, slot) entries routed to e lists its rows by ascending token (a
// token lists an expert once), the stable order of the dispatch.  The first
// column block of every expert writes that expert's part of the dispatch
// outputs; expert 0's also writes the total and -1 for non-local slots.
// Args carries topk_idx, e_begin, T, K, E_loc and the d_* outputs; 256 threads.
// Routing entries 256 * q + tid for q < kDerivePrefetch, loaded before the
// weight ring so that the waits for them do not also wait for the ring (vector
// loads complete in order).  Entries past T * K read e_begin - 1 (not local).
constexpr int kDerivePrefetch = 8;
template <typename Args>
__device__ __forceinline__ void derive_prefetch(const Args& p, int (&pre)[kDerivePrefetch]) {
    const int n = p.T * p.K;
#pragma unroll
    for (int q = 0; q < kDerivePrefetch; ++q) {
        const int i = q * 256 + static_cast<int>(threadIdx.x);
        pre[q] = i < n ? p.topk_idx[i] : p.e_begin - 1;
    }
}

template <typename Args>
__device__ void derive_dispatch(const Args& p, int e, int nb, int* s_cnt, int* s_list, int* s_w4, int& seg0,
                                int& rows, const int (&pre)[kDerivePrefetch]) {
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1), wave = tid >> 6;
    for (int i = tid; i < p.E_loc; i += 256) s_cnt[i] = 0;
    __syncthreads();
    const int n = p.T * p.K;
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    int run = 0;                                       // entries of e listed so far (uniform)
    auto batch = [&](int base, int raw) {
        const int i = base + tid;
        const int v = raw - p.e_begin;                 // entries past n read e_begin - 1: v = -1
        if (v >= 0 && v < p.E_loc) atomicAdd(&s_cnt[v], 1);
        const bool mine = v == e;
        const uint64_t m = __ballot(mine);
        if (lane == 0) s_w4[wave] = __popcll(m);
        __syncthreads();
        int wb = 0;
        for (int w = 0; w < wave; ++w) wb += s_w4[w];
        const int tot = s_w4[0] + s_w4[1] + s_w4[2] + s_w4[3];
        if (mine) s_list[run + wb + __popcll(m & below)] = i;
        run += tot;
        __syncthreads();                               // s_w4 reuse
    };
#pragma unroll
    for (int q = 0; q < kDerivePrefetch; ++q)
        if (q * 256 < n) batch(q * 256, pre[q]);
    for (int base = kDerivePrefetch * 256; base < n; base += 256) {
        const int i = base + tid;
        batch(base, i < n ? p.topk_idx[i] : p.e_begin - 1);
    }
    rows = s_cnt[e];
    int part = 0;
    for (int k = tid; k < e; k += 256) part += s_cnt[k];
    seg0 = block_sum256(part, s_w4);
    if (nb != 0) return;
    if (tid == 0) {
        p.d_counts[e] = rows;
        p.d_offsets[e] = seg0;
    }
    for (int r = tid; r < rows; r += 256) {
        const int i = s_list[r];
        const int t = i / p.K;
        p.d_row_token[seg0 + r] = t;
        p.d_row_slot[seg0 + r] = i - t * p.K;
        p.d_slot_row[i] = seg0 + r;
    }
    if (e == 0) {
        int all = 0;
        for (int k = tid; k < p.E_loc; k += 256) all += s_cnt[k];
        all = block_sum256(all, s_w4);
        if (tid == 0) p.d_offsets[p.E_loc] = all;
        for (int i = tid; i < n; i += 256) {
            const int v = p.topk_idx[i] - p.e_begin;
            if (v < 0 || v >= p.E_loc) p.d_slot_row[i] = -1;
        }
    }
}

}  // namespace
}  // namespace moe
