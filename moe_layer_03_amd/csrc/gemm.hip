// Grouped expert GEMMs on bf16 MFMA, plus the static weight packing they read.
//
// "Hosting Qwen on Blackwell" (Perplexity), section "MoE GEMM": the dispatched
// tokens of each expert form one matrix-multiply problem; with about 375
// tokens per expert at a 6000-token prefill ("Pre-remplisseurs") the problem
// is dense and compute-bound, while decode is bound by streaming the weights
// from HBM ("Decodeurs").
//
// Kernel shape (gfx950):
//   * persistent workgroups of 256 threads (4 waves in a 2x2 grid) walk a
//     tile list laid out per expert as [n-tile][m-tile], so workgroups that
//     run together share the same weight tile; tile ids are split into one
//     contiguous range per XCD (workgroup b runs on XCD b % 8), keeping those
//     sharers inside one L2;
//   * m-tiles per expert come from the device-side offsets (no host sync);
//   * both operands are K-contiguous bf16 rows staged through LDS in 16-byte
//     granules, XOR-swizzled by row so that the MFMA fragment reads are
//     bank-conflict free; double-buffered with register prefetch;
//   * v_mfma_f32_32x32x16_bf16 (bf16 operands) or v_mfma_f32_32x32x16_f16
//     (fp16 operands), float32 accumulators;
//   * epilogues: plain store (float32, bf16 or fp16), or SwiGLU for the
//     gate/up problem, whose weights are packed so that each 64-column block
//     holds 32 gate columns then the same 32 up columns: a lane owns g and u
//     of the same output element and applies silu(g) * u in registers.
//
// Operand types: the gate/up problem multiplies in the weights' own type
// (bf16), or in fp16 for float32 weights; the down problem multiplies the
// SwiGLU activations in fp16 (eight times finer rounding than bf16) with the
// down weights converted to fp16 once at packing time.
#include "common.hpp"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int BK = 64;                 // k per LDS stage (128 bytes of bf16 per row)
constexpr int kMaxExperts = 1024;

enum Mode { kPlain = 0, kGateUpPlain = 1, kSwiGLU = 2 };

struct GemmArgs {
    const uint16_t* a;         // [rows][Kd] bf16
    const uint16_t* b;         // [E_loc][N][Kd] bf16
    const int32_t* offsets;    // [E_loc + 1]
    void* c;                   // output rows
    int E_loc;
    int N;                     // packed output columns of B (2I for gate/up, H for down)
    int Kd;                    // reduction length
    int ldc;                   // output row stride (elements)
    int I;                     // intermediate size (gate/up column remap)
};

__device__ __forceinline__ int lds_off(int row, int kg) {
    // element offset of 16-byte granule kg (0..7) of a 64-element row
    return row * BK + ((kg ^ (row & 7)) << 3);
}

__device__ __forceinline__ float silu(float g) { return g / (1.0f + expf(-g)); }

enum Out { kOutF32 = 0, kOutBF16 = 1, kOutF16 = 2 };

template <int OUT> struct OutType { typedef uint16_t type; };
template <> struct OutType<kOutF32> { typedef float type; };

template <int OUT> __device__ __forceinline__ void store_out(typename OutType<OUT>::type* p, float v) {
    if constexpr (OUT == kOutF32) *p = v;
    else if constexpr (OUT == kOutBF16) *p = f32_to_bf16(v);
    else *p = f32_to_f16_sat(v);
}

template <bool F16>
__device__ __forceinline__ floatx16 mfma32(const uint16_t* a, const uint16_t* b, floatx16 c) {
    if constexpr (F16)
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(*reinterpret_cast<const halfx8_t*>(a),
                                                      *reinterpret_cast<const halfx8_t*>(b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8_t*>(a),
                                                       *reinterpret_cast<const bf16x8_t*>(b), c, 0, 0, 0);
}

// Exclusive scan of per-expert m-tile counts into s_mt[0..E_loc], 256 threads.
template <int BM>
__device__ void build_tile_prefix(const int32_t* __restrict__ offsets, int E_loc, int* s_mt, int* s_tmp) {
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1), wave = tid >> 6;
    constexpr int PER = kMaxExperts / kThreads;   // experts per thread
    int local[PER];
    int sum = 0;
#pragma unroll
    for (int q = 0; q < PER; ++q) {
        const int e = tid * PER + q;
        int v = 0;
        if (e < E_loc) v = (offsets[e + 1] - offsets[e] + BM - 1) / BM;
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
    if (tid == kThreads - 1) s_mt[E_loc] = run;   // total (experts past E_loc add 0)
    __syncthreads();
}

template <int BM, int BN, int MODE, bool F16, int OUT>
__global__ __launch_bounds__(kThreads, 2) void grouped_gemm_kernel(GemmArgs p) {
    typedef typename OutType<OUT>::type OutT;
    constexpr int WM = BM / 2, WN = BN / 2;      // wave tile (2x2 waves)
    constexpr int TM = WM / 32, TN = WN / 32;    // 32x32 MFMA tiles per wave
    constexpr int A_LOADS = BM * 8 / kThreads;   // 16-byte granules per thread per stage
    constexpr int B_LOADS = BN * 8 / kThreads;
    static_assert(A_LOADS >= 1 && B_LOADS >= 1, "tile too small");
    static_assert(MODE != kSwiGLU || (WN % 64) == 0, "SwiGLU pairs need 64-column wave tiles");

    __shared__ __attribute__((aligned(16))) uint16_t s_a[2][BM * BK];
    __shared__ __attribute__((aligned(16))) uint16_t s_b[2][BN * BK];
    __shared__ int s_mt[kMaxExperts + 1];
    __shared__ int s_tmp[kThreads / kWave];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid >> 6;
    const int wm0 = (wave >> 1) * WM;
    const int wn0 = (wave & 1) * WN;

    build_tile_prefix<BM>(p.offsets, p.E_loc, s_mt, s_tmp);
    const int NT = p.N / BN;
    const int total = s_mt[p.E_loc] * NT;

    // contiguous tile range per XCD
    const int G = gridDim.x;
    const int b = blockIdx.x;
    const int lid = (G % 8 == 0) ? (b % 8) * (G / 8) + (b / 8) : b;

    for (int tile = lid; tile < total; tile += G) {
        // locate the expert: largest e with s_mt[e] * NT <= tile
        int lo = 0, hi = p.E_loc - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (s_mt[mid] * NT <= tile) lo = mid; else hi = mid - 1;
        }
        const int e = lo;
        const int mt_e = s_mt[e + 1] - s_mt[e];
        const int local = tile - s_mt[e] * NT;
        const int n_tile = local / mt_e;
        const int m_tile = local - n_tile * mt_e;
        const int seg0 = p.offsets[e], seg1 = p.offsets[e + 1];
        const int row0 = seg0 + m_tile * BM;
        const int rows_valid = min(BM, seg1 - row0);

        const uint16_t* __restrict__ A = p.a + static_cast<int64_t>(row0) * p.Kd;
        const uint16_t* __restrict__ B = p.b + (static_cast<int64_t>(e) * p.N + n_tile * BN) * p.Kd;

        // per-thread granule coordinates (rows past the segment read row 0 and are never stored)
        int a_row[A_LOADS], a_kg[A_LOADS], b_row[B_LOADS], b_kg[B_LOADS];
#pragma unroll
        for (int s = 0; s < A_LOADS; ++s) {
            const int g = tid + s * kThreads;
            a_row[s] = g >> 3;
            a_kg[s] = g & 7;
        }
#pragma unroll
        for (int s = 0; s < B_LOADS; ++s) {
            const int g = tid + s * kThreads;
            b_row[s] = g >> 3;
            b_kg[s] = g & 7;
        }

        u32x4 ra[A_LOADS], rb[B_LOADS];
        auto gload = [&](int k0) {
#pragma unroll
            for (int s = 0; s < A_LOADS; ++s) {
                const int r = a_row[s] < rows_valid ? a_row[s] : 0;
                ra[s] = *reinterpret_cast<const u32x4*>(A + static_cast<int64_t>(r) * p.Kd + k0 + a_kg[s] * 8);
            }
#pragma unroll
            for (int s = 0; s < B_LOADS; ++s)
                rb[s] = *reinterpret_cast<const u32x4*>(B + static_cast<int64_t>(b_row[s]) * p.Kd + k0 + b_kg[s] * 8);
        };
        auto lstore = [&](int buf) {
#pragma unroll
            for (int s = 0; s < A_LOADS; ++s)
                *reinterpret_cast<u32x4*>(&s_a[buf][lds_off(a_row[s], a_kg[s])]) = ra[s];
#pragma unroll
            for (int s = 0; s < B_LOADS; ++s)
                *reinterpret_cast<u32x4*>(&s_b[buf][lds_off(b_row[s], b_kg[s])]) = rb[s];
        };

        floatx16 acc[TM][TN];
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

        const int nk = p.Kd / BK;
        gload(0);
        lstore(0);
        __syncthreads();
        for (int kt = 0; kt < nk; ++kt) {
            const int buf = kt & 1;
            if (kt + 1 < nk) gload((kt + 1) * BK);
#pragma unroll
            for (int ks = 0; ks < BK / 16; ++ks) {
                const int kg = ks * 2 + (lane >> 5);
                u32x4 fa[TM], fb[TN];
#pragma unroll
                for (int i = 0; i < TM; ++i) {
                    const int r = wm0 + i * 32 + (lane & 31);
                    fa[i] = *reinterpret_cast<const u32x4*>(&s_a[buf][lds_off(r, kg)]);
                }
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    const int n = wn0 + j * 32 + (lane & 31);
                    fb[j] = *reinterpret_cast<const u32x4*>(&s_b[buf][lds_off(n, kg)]);
                }
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j)
                        acc[i][j] = mfma32<F16>(reinterpret_cast<const uint16_t*>(&fa[i]),
                                                reinterpret_cast<const uint16_t*>(&fb[j]), acc[i][j]);
            }
            if (kt + 1 < nk) lstore(buf ^ 1);
            __syncthreads();
        }

        // epilogue: lane holds column (lane & 31) and rows 8*(v/4) + 4*(lane/32) + v%4 of each 32x32 tile
        OutT* __restrict__ C = static_cast<OutT*>(p.c);
#pragma unroll
        for (int i = 0; i < TM; ++i) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int r = wm0 + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                if (r >= rows_valid) continue;
                OutT* crow = C + static_cast<int64_t>(row0 + r) * p.ldc;
                if constexpr (MODE == kSwiGLU) {
#pragma unroll
                    for (int j = 0; j < TN; j += 2) {
                        const int pc = n_tile * BN + wn0 + j * 32;   // multiple of 64: gate block start
                        const int col = (pc >> 1) + (lane & 31);
                        store_out<OUT>(crow + col, silu(acc[i][j][v]) * acc[i][j + 1][v]);
                    }
                } else if constexpr (MODE == kGateUpPlain) {
#pragma unroll
                    for (int j = 0; j < TN; ++j) {
                        const int pc = n_tile * BN + wn0 + j * 32 + (lane & 31);
                        const int q = pc >> 6, w = pc & 63;
                        const int col = w < 32 ? q * 32 + w : p.I + q * 32 + (w - 32);
                        store_out<OUT>(crow + col, acc[i][j][v]);
                    }
                } else {
#pragma unroll
                    for (int j = 0; j < TN; ++j) {
                        const int col = n_tile * BN + wn0 + j * 32 + (lane & 31);
                        store_out<OUT>(crow + col, acc[i][j][v]);
                    }
                }
            }
        }
        __syncthreads();   // LDS reuse by the next tile
    }
}

// ---------------------------------------------------------------------------
// weight packing: [E_loc][R][Cs] (row-major, y = x W) -> [E_loc][Cs'][R] 16-bit,
// rows of the output are the GEMM's N index, K-contiguous.
// gate/up: output row p of 2I, 64-blocks of (32 gate | 32 up) columns.
// ---------------------------------------------------------------------------
template <typename ST, bool GATE_UP, bool F16OUT>
__global__ __launch_bounds__(256) void pack_kernel(const ST* __restrict__ src, int R, int Cs, int I,
                                                   bool is_up, uint16_t* __restrict__ dst, int dst_rows) {
    __shared__ float tile[64][65];
    const int e = blockIdx.z;
    const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
    const ST* s = src + static_cast<int64_t>(e) * R * Cs;
    for (int i = threadIdx.x; i < 64 * 64; i += 256) {
        const int rr = i / 64, cc = i % 64;
        float v;
        if constexpr (sizeof(ST) == 2) v = bf16_to_f32(s[static_cast<int64_t>(r0 + rr) * Cs + c0 + cc]);
        else v = s[static_cast<int64_t>(r0 + rr) * Cs + c0 + cc];
        tile[rr][cc] = v;
    }
    __syncthreads();
    uint16_t* d = dst + static_cast<int64_t>(e) * dst_rows * R;
    for (int i = threadIdx.x; i < 64 * 64; i += 256) {
        const int cc = i / 64, rr = i % 64;
        const int c = c0 + cc;
        int prow = c;
        if constexpr (GATE_UP) prow = (c >> 5) * 64 + (is_up ? 32 : 0) + (c & 31);
        const float v = tile[rr][cc];
        d[static_cast<int64_t>(prow) * R + r0 + rr] = F16OUT ? f32_to_f16_sat(v) : f32_to_bf16(v);
    }
}

template <int BM, int BN, int MODE, bool F16, int OUT>
int launch_gemm_t(const GemmArgs& args, int max_rows, hipStream_t st) {
    // upper bound of tiles: each expert adds at most one partial m-tile
    const int64_t mt_bound = (static_cast<int64_t>(max_rows) + BM - 1) / BM + args.E_loc;
    const int64_t tiles = mt_bound * (args.N / BN);
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess) {
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0) cus = v;
    }
    int64_t grid = 2LL * cus;
    if (tiles < grid) grid = tiles;
    if (grid < 1) grid = 1;
    hipLaunchKernelGGL((grouped_gemm_kernel<BM, BN, MODE, F16, OUT>), dim3(static_cast<unsigned>(grid)),
                       dim3(kThreads), 0, st, args);
    MOE_CHECK_LAUNCH();
    return MOE_OK;
}

}  // namespace

size_t packed_gate_up_elems(const moe_shape& s) {
    return static_cast<size_t>(s.e_end - s.e_begin) * 2 * s.I * s.H;
}
size_t packed_down_elems(const moe_shape& s) {
    return static_cast<size_t>(s.e_end - s.e_begin) * s.H * s.I;
}

int launch_pack_weights(const moe_shape& s, const void* w_gate, const void* w_up, const void* w_down, int dtype,
                        uint16_t* packed, hipStream_t st) {
    const int E_loc = s.e_end - s.e_begin;
    uint16_t* gu = packed;
    uint16_t* dn = packed + packed_gate_up_elems(s);
    const dim3 g_gu(s.I / 64, s.H / 64, E_loc), g_dn(s.H / 64, s.I / 64, E_loc);
    if (dtype == MOE_BF16) {
        auto g = static_cast<const uint16_t*>(w_gate);
        auto u = static_cast<const uint16_t*>(w_up);
        auto d = static_cast<const uint16_t*>(w_down);
        hipLaunchKernelGGL((pack_kernel<uint16_t, true, false>), g_gu, dim3(256), 0, st, g, s.H, s.I, s.I, false, gu,
                           2 * s.I);
        hipLaunchKernelGGL((pack_kernel<uint16_t, true, false>), g_gu, dim3(256), 0, st, u, s.H, s.I, s.I, true, gu,
                           2 * s.I);
        hipLaunchKernelGGL((pack_kernel<uint16_t, false, true>), g_dn, dim3(256), 0, st, d, s.I, s.H, s.I, false, dn,
                           s.H);
    } else {
        auto g = static_cast<const float*>(w_gate);
        auto u = static_cast<const float*>(w_up);
        auto d = static_cast<const float*>(w_down);
        hipLaunchKernelGGL((pack_kernel<float, true, true>), g_gu, dim3(256), 0, st, g, s.H, s.I, s.I, false, gu,
                           2 * s.I);
        hipLaunchKernelGGL((pack_kernel<float, true, true>), g_gu, dim3(256), 0, st, u, s.H, s.I, s.I, true, gu,
                           2 * s.I);
        hipLaunchKernelGGL((pack_kernel<float, false, true>), g_dn, dim3(256), 0, st, d, s.I, s.H, s.I, false, dn,
                           s.H);
    }
    MOE_CHECK_LAUNCH();
    return MOE_OK;
}

namespace {

template <int BM, int BN, int MODE, bool F16>
int launch_out(const GemmArgs& args, int max_rows, int c_dtype, hipStream_t st) {
    if (c_dtype == MOE_F32) return launch_gemm_t<BM, BN, MODE, F16, kOutF32>(args, max_rows, st);
    if (c_dtype == MOE_BF16) return launch_gemm_t<BM, BN, MODE, F16, kOutBF16>(args, max_rows, st);
    return launch_gemm_t<BM, BN, MODE, F16, kOutF16>(args, max_rows, st);
}

}  // namespace

int launch_grouped_gemm(const moe_shape& s, const uint16_t* a, int a_dtype, const int32_t* offsets,
                        const uint16_t* packed, int which, int epilogue, void* c, int c_dtype, hipStream_t st) {
    const int E_loc = s.e_end - s.e_begin;
    const int max_rows = s.T * (s.K < E_loc ? s.K : E_loc);
    GemmArgs args;
    args.a = a;
    args.offsets = offsets;
    args.c = c;
    args.E_loc = E_loc;
    args.I = s.I;
    if (which == MOE_GEMM_GATE_UP) {
        args.b = packed;
        args.N = 2 * s.I;
        args.Kd = s.H;
        args.ldc = epilogue == MOE_EPI_SWIGLU ? s.I : 2 * s.I;
        const bool f16 = a_dtype == MOE_F16;
        if (epilogue == MOE_EPI_SWIGLU)
            return f16 ? launch_out<128, 128, kSwiGLU, true>(args, max_rows, c_dtype, st)
                       : launch_out<128, 128, kSwiGLU, false>(args, max_rows, c_dtype, st);
        return f16 ? launch_out<128, 128, kGateUpPlain, true>(args, max_rows, c_dtype, st)
                   : launch_out<128, 128, kGateUpPlain, false>(args, max_rows, c_dtype, st);
    }
    args.b = packed + packed_gate_up_elems(s);
    args.N = s.H;
    args.Kd = s.I;
    args.ldc = s.H;
    if (s.H % 128 == 0) return launch_out<128, 128, kPlain, true>(args, max_rows, c_dtype, st);
    return launch_out<128, 64, kPlain, true>(args, max_rows, c_dtype, st);
}

}  // namespace moe
