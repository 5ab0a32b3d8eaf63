// Dispatch: select the (token, slot) pairs routed to local experts, give each
// a packed row (experts ascending, tokens ascending within an expert) and
// copy the tokens into the per-expert contiguous GEMM input buffer.
//
// "Hosting Qwen on Blackwell" (Perplexity), section "Expert Parallel": the
// expert-parallel inputs are replicated on every rank, so dispatch only has to
// select the tokens routed to the rank's experts, aggregate the routing
// information and prepare the tokens in the buffers the MoE GEMM reads.
//
// Four kernels, no host synchronisation (batches of at most 16 chunks run
// count, scan and scatter as one single-workgroup kernel):
//   count   one wave per chunk of 64 tokens; for every local expert a wave
//           ballot gives the bit mask of chunk tokens routed to it (a token
//           picks an expert at most once) and its population count;
//   scan    one workgroup: per-expert exclusive scan over chunks, exclusive
//           scan over experts -> counts, offsets and each chunk's base row;
//   scatter row = chunk base + number of earlier lanes in the chunk's mask,
//           which keeps token order (stable) without atomics;
//   pack    persistent row copy x[row_token[r]] -> x_packed[r], 16-byte
//           vector loads and stores (bf16 is copied; float32 input is
//           rounded to fp16, the GEMM operand type for float32 layers).
#include "common.hpp"

namespace moe {
namespace {

constexpr int kChunk = 64;          // tokens per chunk (one wave)
constexpr int kScanThreads = 1024;

struct Scratch {
    int32_t* chunk_count;    // [C][E_loc]
    uint64_t* chunk_mask;    // [C][E_loc]
    int32_t* chunk_base;     // [C][E_loc]
};

inline size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

Scratch carve(const moe_shape& s, void* base) {
    const size_t C = (static_cast<size_t>(s.T) + kChunk - 1) / kChunk;
    const size_t n = C * static_cast<size_t>(s.e_end - s.e_begin);
    char* p = static_cast<char*>(base);
    Scratch sc;
    sc.chunk_mask = reinterpret_cast<uint64_t*>(p);
    p += align256(n * sizeof(uint64_t));
    sc.chunk_count = reinterpret_cast<int32_t*>(p);
    p += align256(n * sizeof(int32_t));
    sc.chunk_base = reinterpret_cast<int32_t*>(p);
    return sc;
}

__global__ __launch_bounds__(256) void count_kernel(const int32_t* __restrict__ topk_idx, int T, int K,
                                                    int e_begin, int E_loc, int32_t* __restrict__ chunk_count,
                                                    uint64_t* __restrict__ chunk_mask, int C) {
    const int lane = threadIdx.x & (kWave - 1);
    const int c = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (c >= C) return;   // whole wave
    const int t = c * kChunk + lane;
    const bool valid = t < T;
    const int words = (E_loc + kWave - 1) / kWave;
    for (int wd = 0; wd < words; ++wd) {
        uint64_t bits = 0;
        if (valid) {
            for (int j = 0; j < K; ++j) {
                const int i = topk_idx[static_cast<int64_t>(t) * K + j] - e_begin;
                if (i >= 0 && i < E_loc && (i >> 6) == wd) bits |= 1ull << (i & 63);
            }
        }
        uint64_t mine = 0;
        const int nb = min(kWave, E_loc - wd * kWave);
        for (int b = 0; b < nb; ++b) {
            const uint64_t m = __ballot((bits >> b) & 1ull);
            if (lane == b) mine = m;
        }
        if (lane < nb) {
            const int64_t o = static_cast<int64_t>(c) * E_loc + wd * kWave + lane;
            chunk_mask[o] = mine;
            chunk_count[o] = __popcll(mine);
        }
    }
}

// Exclusive scan of one value per thread over a 1024-thread block; returns the
// prefix, total in *total.
__device__ int block_exclusive_scan_1024(int v, int* s_tmp /*[16]*/, int* total) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x >> 6;
    int inc = v;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const int o = __shfl_up(inc, off, kWave);
        if (lane >= off) inc += o;
    }
    if (lane == kWave - 1) s_tmp[wave] = inc;
    __syncthreads();
    if (wave == 0) {
        int wv = lane < 16 ? s_tmp[lane] : 0;
        int winc = wv;
#pragma unroll
        for (int off = 1; off < 16; off <<= 1) {
            const int o = __shfl_up(winc, off, kWave);
            if (lane >= off) winc += o;
        }
        if (lane < 16) s_tmp[lane] = winc - wv;   // exclusive wave prefix
        if (lane == 15) s_tmp[16] = winc;
    }
    __syncthreads();
    const int res = s_tmp[wave] + inc - v;
    *total = s_tmp[16];
    __syncthreads();
    return res;
}

__global__ __launch_bounds__(kScanThreads) void scan_kernel(const int32_t* __restrict__ chunk_count,
                                                            int32_t* __restrict__ chunk_base, int C, int E_loc,
                                                            int32_t* __restrict__ counts,
                                                            int32_t* __restrict__ offsets) {
    __shared__ int s_part[kScanThreads];   // [P][E_loc] partial sums, then their exclusive prefixes
    __shared__ int s_off[kScanThreads + 1];
    __shared__ int s_tmp[17];
    const int tid = threadIdx.x;
    const int P = max(1, kScanThreads / E_loc);
    const int per = (C + P - 1) / P;
    // phase 1: partial sums of chunk counts per (part, expert)
    for (int idx = tid; idx < P * E_loc; idx += kScanThreads) {
        const int p = idx / E_loc, i = idx % E_loc;
        int sum = 0;
        const int c1 = min(C, (p + 1) * per);
        for (int c = p * per; c < c1; ++c) sum += chunk_count[static_cast<int64_t>(c) * E_loc + i];
        s_part[idx] = sum;
    }
    __syncthreads();
    // phase 2: per expert, exclusive scan over parts; totals
    int total_i = 0;
    if (tid < E_loc) {
        int run = 0;
        for (int p = 0; p < P; ++p) {
            const int v = s_part[p * E_loc + tid];
            s_part[p * E_loc + tid] = run;
            run += v;
        }
        total_i = run;
        counts[tid] = run;
    }
    __syncthreads();
    // phase 3: exclusive scan over experts
    int all = 0;
    const int pre = block_exclusive_scan_1024(tid < E_loc ? total_i : 0, s_tmp, &all);
    if (tid < E_loc) {
        s_off[tid] = pre;
        offsets[tid] = pre;
    }
    if (tid == 0) offsets[E_loc] = all;
    __syncthreads();
    // phase 4: base row of every (chunk, expert)
    for (int idx = tid; idx < P * E_loc; idx += kScanThreads) {
        const int p = idx / E_loc, i = idx % E_loc;
        int run = s_off[i] + s_part[idx];
        const int c1 = min(C, (p + 1) * per);
        for (int c = p * per; c < c1; ++c) {
            const int64_t o = static_cast<int64_t>(c) * E_loc + i;
            chunk_base[o] = run;
            run += chunk_count[o];
        }
    }
}

__global__ __launch_bounds__(256) void scatter_kernel(const int32_t* __restrict__ topk_idx, int T, int K,
                                                      int e_begin, int E_loc,
                                                      const uint64_t* __restrict__ chunk_mask,
                                                      const int32_t* __restrict__ chunk_base, int C,
                                                      int32_t* __restrict__ row_token,
                                                      int32_t* __restrict__ row_slot,
                                                      int32_t* __restrict__ slot_row) {
    const int lane = threadIdx.x & (kWave - 1);
    const int c = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int t = c * kChunk + lane;
    if (c >= C || t >= T) return;
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int j = 0; j < K; ++j) {
        const int64_t o = static_cast<int64_t>(t) * K + j;
        const int i = topk_idx[o] - e_begin;
        int row = -1;
        if (i >= 0 && i < E_loc) {
            const int64_t co = static_cast<int64_t>(c) * E_loc + i;
            row = chunk_base[co] + __popcll(chunk_mask[co] & below);
            row_token[row] = t;
            row_slot[row] = j;
        }
        slot_row[o] = row;
    }
}

// Small batches (at most 16 chunks, C * E_loc <= 4096): count, scan and
// scatter in one workgroup with the chunk masks in LDS -- the same ballots,
// prefix sums and stable ranks as the three kernels above, one launch.
constexpr int kSmallChunks = kScanThreads / kWave;   // 16
constexpr int kSmallCells = 4096;                    // C * E_loc

__global__ __launch_bounds__(kScanThreads) void dispatch_small_kernel(const int32_t* __restrict__ topk_idx, int T,
                                                                      int K, int e_begin, int E_loc, int C,
                                                                      int32_t* __restrict__ counts,
                                                                      int32_t* __restrict__ offsets,
                                                                      int32_t* __restrict__ row_token,
                                                                      int32_t* __restrict__ row_slot,
                                                                      int32_t* __restrict__ slot_row) {
    __shared__ uint64_t s_mask[kSmallCells];
    __shared__ int s_base[kSmallCells];
    __shared__ int s_tmp[17];
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int c = tid >> 6;                            // chunk of this wave
    const int t = c * kChunk + lane;
    const bool valid = c < C && t < T;
    // count: for every local expert, the mask of this chunk's tokens routed to it
    if (c < C) {
        const int words = (E_loc + kWave - 1) / kWave;
        for (int wd = 0; wd < words; ++wd) {
            uint64_t bits = 0;
            if (valid) {
                for (int j = 0; j < K; ++j) {
                    const int i = topk_idx[static_cast<int64_t>(t) * K + j] - e_begin;
                    if (i >= 0 && i < E_loc && (i >> 6) == wd) bits |= 1ull << (i & 63);
                }
            }
            uint64_t mine = 0;
            const int nb = min(kWave, E_loc - wd * kWave);
            for (int b = 0; b < nb; ++b) {
                const uint64_t m = __ballot((bits >> b) & 1ull);
                if (lane == b) mine = m;
            }
            if (lane < nb) s_mask[c * E_loc + wd * kWave + lane] = mine;
        }
    }
    __syncthreads();
    // scan: per expert over chunks, then over experts
    int total_i = 0;
    for (int i = tid; i < E_loc; i += kScanThreads) {
        int run = 0;
        for (int cc = 0; cc < C; ++cc) {
            s_base[cc * E_loc + i] = run;
            run += __popcll(s_mask[cc * E_loc + i]);
        }
        counts[i] = run;
        if (i == tid) total_i = run;
    }
    int all = 0;
    const int pre = block_exclusive_scan_1024(tid < E_loc ? total_i : 0, s_tmp, &all);
    if (tid < E_loc) {
        offsets[tid] = pre;
        for (int cc = 0; cc < C; ++cc) s_base[cc * E_loc + tid] += pre;
    }
    if (tid == 0) offsets[E_loc] = all;
    __syncthreads();
    // scatter: stable rank within the chunk from the mask
    if (valid) {
        const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
        for (int j = 0; j < K; ++j) {
            const int64_t o = static_cast<int64_t>(t) * K + j;
            const int i = topk_idx[o] - e_begin;
            int row = -1;
            if (i >= 0 && i < E_loc) {
                const int cell = c * E_loc + i;
                row = s_base[cell] + __popcll(s_mask[cell] & below);
                row_token[row] = t;
                row_slot[row] = j;
            }
            slot_row[o] = row;
        }
    }
}

template <typename XT>
__global__ __launch_bounds__(256) void pack_kernel(const XT* __restrict__ x, int H,
                                                   const int32_t* __restrict__ row_token,
                                                   const int32_t* __restrict__ n_rows,
                                                   uint16_t* __restrict__ x_packed) {
    const int N = *n_rows;
    for (int r = blockIdx.x; r < N; r += gridDim.x) {
        const int64_t src = static_cast<int64_t>(row_token[r]) * H;
        const int64_t dst = static_cast<int64_t>(r) * H;
        for (int k = threadIdx.x * 8; k < H; k += 256 * 8) {
            u32x4 v;
            if constexpr (sizeof(XT) == 2) {
                v = *reinterpret_cast<const u32x4*>(x + src + k);
            } else {
                const floatx4 a = *reinterpret_cast<const floatx4*>(x + src + k);
                const floatx4 b = *reinterpret_cast<const floatx4*>(x + src + k + 4);
                v[0] = pack_f16x2(a[0], a[1]);
                v[1] = pack_f16x2(a[2], a[3]);
                v[2] = pack_f16x2(b[0], b[1]);
                v[3] = pack_f16x2(b[2], b[3]);
            }
            *reinterpret_cast<u32x4*>(x_packed + dst + k) = v;
        }
    }
}

}  // namespace

size_t dispatch_scratch_bytes(const moe_shape& s) {
    const size_t C = (static_cast<size_t>(s.T) + kChunk - 1) / kChunk;
    const size_t n = C * static_cast<size_t>(s.e_end - s.e_begin);
    return align256(n * sizeof(uint64_t)) + 2 * align256(n * sizeof(int32_t));
}

int launch_dispatch(const moe_shape& s, const int32_t* topk_idx, const void* x, int x_dtype,
                    int32_t* counts, int32_t* offsets, int32_t* row_token, int32_t* row_slot,
                    int32_t* slot_row, uint16_t* x_packed, void* scratch, hipStream_t st) {
    const int E_loc = s.e_end - s.e_begin;
    const int C = (s.T + kChunk - 1) / kChunk;
    Scratch sc = carve(s, scratch);
    const int g4 = (C + 3) / 4;
    if (C > 0 && C <= kSmallChunks && static_cast<int64_t>(C) * E_loc <= kSmallCells) {
        hipLaunchKernelGGL(dispatch_small_kernel, dim3(1), dim3(kScanThreads), 0, st, topk_idx, s.T, s.K, s.e_begin,
                           E_loc, C, counts, offsets, row_token, row_slot, slot_row);
    } else {
        if (C > 0)
            hipLaunchKernelGGL(count_kernel, dim3(g4), dim3(256), 0, st, topk_idx, s.T, s.K, s.e_begin, E_loc,
                               sc.chunk_count, sc.chunk_mask, C);
        // with no tokens the scan still runs and writes zero counts and offsets
        hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(kScanThreads), 0, st, sc.chunk_count, sc.chunk_base, C, E_loc,
                           counts, offsets);
        if (C > 0)
            hipLaunchKernelGGL(scatter_kernel, dim3(g4), dim3(256), 0, st, topk_idx, s.T, s.K, s.e_begin, E_loc,
                               sc.chunk_mask, sc.chunk_base, C, row_token, row_slot, slot_row);
    }
    if (x_packed != nullptr && C > 0) {
        const int64_t cap = static_cast<int64_t>(s.T) * min(s.K, E_loc);
        const int grid = static_cast<int>(cap < 4096 ? cap : 4096);
        if (x_dtype == MOE_BF16)
            hipLaunchKernelGGL(pack_kernel<uint16_t>, dim3(grid), dim3(256), 0, st,
                               static_cast<const uint16_t*>(x), s.H, row_token, offsets + E_loc, x_packed);
        else
            hipLaunchKernelGGL(pack_kernel<float>, dim3(grid), dim3(256), 0, st, static_cast<const float*>(x),
                               s.H, row_token, offsets + E_loc, x_packed);
    }
    MOE_CHECK_LAUNCH();
    return MOE_OK;
}

}  // namespace moe
