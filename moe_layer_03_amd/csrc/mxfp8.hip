// MXFP8 expert GEMMs on gfx950's scaled MFMA, the activation quantiser and
// the static weight conversion.
//
// "Hosting Qwen on Blackwell" (Perplexity), section "Quantification": the
// model is deployed with the MXFP8 microscaling scheme, its weights converted
// statically once; microscaling is what the hardware needs for its best
// prefill and decode throughput.  The format is the Open Compute Project
// Microscaling (MX) MXFP8: blocks of 32 consecutive elements along the
// reduction dimension K share one E8M0 scale 2^(e - 127); elements are FP8
// E4M3 (bias 7, largest finite 448, no infinities).  A block converts with
// shared exponent floor(log2(max |v|)) - 8 (clamped to [-127, 127]; -127 for an
// all-zero block) and elements v / 2^shared rounded to the nearest E4M3 value,
// ties to the even code, saturating at +-448.
//
// Both GEMM operands are MXFP8 (the scaled MFMA takes no 16-bit operand):
// expert weights per output column along K, converted once at packing; token
// rows x per token along H (moe_quantize_mxfp8); SwiGLU activations h per row
// along I, converted in the gate/up epilogue (a wave's 32 h columns of a row
// are exactly one block).
//
// v_mfma_scale_f32_32x32x64_f8f6f4 (E4M3 x E4M3, float32 accumulate), as
// measured on this chip: lane l holds row (A) or column (B) l % 32; of its 32
// bytes, the first 16 are elements h*16 .. h*16+15 of the step's first
// 32-block and the last 16 the same elements of the second block (h = l / 32);
// the scale of (row or column r, block b of the step) comes from lane
// r + 32 b, byte 0 of its scale register.
//
// Layouts
//   activation codes [rows][K] bytes, scales [rows][K/32] bytes (E8M0);
//   packed weights: codes of every 64-k step as 2 KiB tiles per 32 columns,
//     [E_loc][N/64][K/64][2][2 parts][64 lanes][16 bytes] (part p = bytes
//     16p .. 16p+15 of each lane's operand, so every read is one contiguous
//     KiB per wave), gate/up columns interleaved per 64 as 32 gate | 32 up;
//     then the scales [E_loc][N][K/32] bytes in packed-column order;
//     gate/up codes, down codes, gate/up scales, down scales, in that order.
#include "gemm_common.hpp"

namespace moe {
namespace {

constexpr int kMxStepK = 64;          // k per scaled MFMA: two blocks
constexpr int kMxTile = 2048;         // bytes of one 32-column x 64-k operand tile

// ---- conversions (the rule in the header comment), bit for bit -------------

// floor(log2(amax)) - 8 clamped to [-127, 127]; zero and subnormal amax give -127.
__device__ __forceinline__ int mx_shared_exp(float amax) {
    const int e = static_cast<int>((__float_as_uint(amax) >> 23) & 0xFFu);
    return min(max(e - 127 - 8, -127), 127);
}

// 2^-se as a float32 (exact: se = 127 gives the subnormal 2^-127).
__device__ __forceinline__ float mx_inv_scale(int se) {
    return se == 127 ? __uint_as_float(0x00400000u) : __uint_as_float(static_cast<uint32_t>(127 - se) << 23);
}

// Nearest E4M3 code of a float32, ties to even, saturating at 448; the sign
// bit follows the input's.
__device__ __forceinline__ uint32_t e4m3_rne_sat(float a) {
    const uint32_t u = __float_as_uint(a);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t m = u & 0x7FFFFFFFu;
    uint32_t code;
    if (m >= 0x43E00000u) {                               // |a| >= 448
        code = 0x7Eu;
    } else if (m >= 0x3C800000u) {                        // 2^-6 <= |a| < 448: keep 3 mantissa bits
        code = ((m + 0x7FFFFu + ((m >> 20) & 1u)) >> 20) - (120u << 3);
    } else {                                              // subnormal: multiples of 2^-9
        code = static_cast<uint32_t>(__builtin_rintf(__uint_as_float(m) * 512.0f));
    }
    return sign | code;
}

// ---- activation quantiser: 8 elements per thread, 4 threads per block -------
template <typename XT>
__global__ __launch_bounds__(256) void mx_quantize_kernel(const XT* __restrict__ x, int64_t groups, int K,
                                                          uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
    const int64_t g = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;   // group of 8 elements
    if (g >= groups) return;            // groups is a multiple of 4: a block's four threads leave together
    const int64_t e0 = g * 8;
    float v[8];
    if constexpr (sizeof(XT) == 2) {
        const u32x4 w = *reinterpret_cast<const u32x4*>(x + e0);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            v[2 * j] = __uint_as_float(w[j] << 16);
            v[2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
        }
    } else {
        const floatx4 a = *reinterpret_cast<const floatx4*>(x + e0);
        const floatx4 b = *reinterpret_cast<const floatx4*>(x + e0 + 4);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            v[j] = a[j];
            v[4 + j] = b[j];
        }
    }
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(v[j]));
    amax = fmaxf(amax, __shfl_xor(amax, 1, 4));
    amax = fmaxf(amax, __shfl_xor(amax, 2, 4));
    const int se = mx_shared_exp(amax);
    const float inv = mx_inv_scale(se);
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        lo |= e4m3_rne_sat(v[j] * inv) << (8 * j);
        hi |= e4m3_rne_sat(v[4 + j] * inv) << (8 * j);
    }
    *reinterpret_cast<uint2*>(codes + e0) = make_uint2(lo, hi);
    if ((g & 3) == 0) scales[e0 / 32] = static_cast<uint8_t>(se + 127);   // [rows][K/32] is flat in e0 / 32
}

// ---- static weight conversion ------------------------------------------------
// Source [E_loc][Kd][Cs] (y = x W); one thread per (expert, source column, 32-k block).
template <typename ST>
__global__ __launch_bounds__(256) void mx_pack_weights_kernel(const ST* __restrict__ src, int Kd, int Cs, int N,
                                                              int gate_up, int is_up, uint8_t* __restrict__ codes,
                                                              uint8_t* __restrict__ scales) {
    const int e = blockIdx.z;
    const int b = blockIdx.y;                          // 32-k block
    const int c = blockIdx.x * 256 + threadIdx.x;      // source column
    if (c >= Cs) return;
    const ST* s = src + (static_cast<int64_t>(e) * Kd + b * 32) * Cs + c;
    float v[32];
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
        if constexpr (sizeof(ST) == 2) v[j] = bf16_to_f32(s[static_cast<int64_t>(j) * Cs]);
        else v[j] = s[static_cast<int64_t>(j) * Cs];
        amax = fmaxf(amax, fabsf(v[j]));
    }
    const int se = mx_shared_exp(amax);
    const float inv = mx_inv_scale(se);
    uint32_t w[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        w[q] = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) w[q] |= e4m3_rne_sat(v[4 * q + j] * inv) << (8 * j);
    }
    const int pc = gate_up ? (c >> 5) * 64 + (is_up ? 32 : 0) + (c & 31) : c;   // packed column
    const int n32 = pc >> 5, col = pc & 31;
    const int ks = b >> 1, part = b & 1;
    const int64_t tile = ((static_cast<int64_t>(e) * (N >> 6) + (n32 >> 1)) * (Kd / kMxStepK) + ks) * 2 + (n32 & 1);
    uint8_t* t = codes + tile * kMxTile + part * 1024;
    *reinterpret_cast<u32x4*>(t + col * 16) = u32x4{w[0], w[1], w[2], w[3]};          // elements 0..15: lane col
    *reinterpret_cast<u32x4*>(t + (col + 32) * 16) = u32x4{w[4], w[5], w[6], w[7]};   // 16..31: lane col + 32
    scales[(static_cast<int64_t>(e) * N + pc) * (Kd / 32) + b] = static_cast<uint8_t>(se + 127);
}

// ---- scaled MFMA ---------------------------------------------------------------
typedef int i32x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ floatx16 mfma_mx(const u32x4& a0, const u32x4& a1, uint32_t sa, const u32x4& b0,
                                            const u32x4& b1, uint32_t sb, floatx16 c) {
    const i32x8 a = {static_cast<int>(a0[0]), static_cast<int>(a0[1]), static_cast<int>(a0[2]),
                     static_cast<int>(a0[3]), static_cast<int>(a1[0]), static_cast<int>(a1[1]),
                     static_cast<int>(a1[2]), static_cast<int>(a1[3])};
    const i32x8 b = {static_cast<int>(b0[0]), static_cast<int>(b0[1]), static_cast<int>(b0[2]),
                     static_cast<int>(b0[3]), static_cast<int>(b1[0]), static_cast<int>(b1[1]),
                     static_cast<int>(b1[2]), static_cast<int>(b1[3])};
    // formats 0, 0: E4M3 x E4M3; scale bytes 0 of sa and sb
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, static_cast<int>(sa), 0,
                                                           static_cast<int>(sb));
}

enum MxOut { kMxOutF32 = 0, kMxOutBF16 = 1, kMxOutF16 = 2, kMxOutMX = 3 };

struct MxArgs {
    const uint8_t* a;          // activation codes [rows][Kd]
    const uint8_t* a_scales;   // [rows][Kd/32]
    const int32_t* a_rows;     // NULL, or: packed row r reads row a_rows[r] of a
    int a_rows_bound;          // rows of a
    const uint8_t* b;          // weight code tiles of this problem
    const uint8_t* b_scales;   // [E_loc][N][Kd/32]
    const int32_t* offsets;    // [E_loc + 1]
    void* c;                   // output rows (codes for kMxOutMX)
    uint8_t* c_scales;         // kMxOutMX: [rows][ldc/32]
    int E_loc, N, Kd, ldc, I;
    // weight-streaming gate/up only, optional: derive the dispatch from the
    // routing instead of reading offsets / a_rows (a holds the T token rows)
    const int32_t* topk_idx;   // [T][K] expert ids, NULL: not derived
    int e_begin, T, K;
    int32_t* d_counts;         // dispatch outputs, written by each expert's first column block
    int32_t* d_offsets;
    int32_t* d_row_token;
    int32_t* d_row_slot;
    int32_t* d_slot_row;
};

// One 16-byte-per-lane buffer -> LDS copy (lane l lands at base + 16 l).
__device__ __forceinline__ void copy16_to_lds(__amdgpu_buffer_rsrc_t rsrc, void* lds_wave_base, uint32_t voff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rsrc, reinterpret_cast<__attribute__((address_space(3))) void*>(reinterpret_cast<uintptr_t>(lds_wave_base)),
        16, static_cast<int>(voff), 0, 0, 0);
}

// SwiGLU value v of a lane's column, for its row: the 32 lanes of each half of
// the wave hold one row's 32 columns, one MX block.  Writes the code at *code
// and, from the half's first lane, the block's scale at *scale (when live).
__device__ __forceinline__ void store_mx_block(float v, bool live, uint8_t* code, uint8_t* scale) {
    float amax = fabsf(v);
#pragma unroll
    for (int off = 1; off < 32; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 32));
    const int se = mx_shared_exp(amax);
    if (live) {
        *code = static_cast<uint8_t>(e4m3_rne_sat(v * mx_inv_scale(se)));
        if ((threadIdx.x & 31) == 0) *scale = static_cast<uint8_t>(se + 127);
    }
}

template <int OUT> struct MxOutType { typedef uint16_t type; };
template <> struct MxOutType<kMxOutF32> { typedef float type; };
template <> struct MxOutType<kMxOutMX> { typedef uint8_t type; };

// ---------------------------------------------------------------------------
// Tiled form (many rows per expert): the structure of the bf16 tiled GEMM --
// persistent workgroups of 8 waves over a tile list laid out per expert as
// [n-tile][m-tile], contiguous per XCD; a tile of two 128-row slabs x 256
// columns; each wave 128 rows x 64 columns (4 x 2 MFMA tiles of 32 x 32, 128
// float32 accumulators per lane) -- with one 64-k step per LDS stage: 64-byte
// code rows of A (XOR-swizzled granules) and 2 KiB code tiles of B, by direct
// buffer -> LDS copies into a ring of NB stages; rows past the segment read
// zeros (no memory traffic).  Scales travel apart from the codes, 16 bytes
// (16 blocks: 8 k-steps) per A row and per B column in one copy per thread
// every 8 k-steps, into two alternating scale buffers: the scales are spread
// one row or column per lane, so fewer, wider copies cut the cache lines each
// copy touches 8-fold.  A K that is not a multiple of 512 ends in a half group,
// whose copy starts 8 blocks early so it never reads past a row; K >= 512.
// ---------------------------------------------------------------------------
template <int MODE, int OUT, int NB>
__global__ __launch_bounds__(512, 1) void grouped_gemm_mx_kernel(MxArgs p) {
    static_assert(NB % 2 == 0, "k-step parity follows the stage index");
    typedef typename MxOutType<OUT>::type OutT;
    constexpr int NWAVES = 8, NTHREADS = 512, WN = 4, BM = 128, UM = 256, BN = 256, TM = 4;
    constexpr int A_STAGE = UM * 64;                  // bytes
    constexpr int B_STAGE = BN * 64;
    constexpr int A_BLKS = BM / 16;                   // 16-row (1 KiB) copy blocks of one row half
    constexpr int A_DMA = A_BLKS / WN;                // A copies per thread per stage, at most: 2
    constexpr int B_DMA = B_STAGE / 16 / NTHREADS;    // 2
    constexpr int SG = 8;                             // k-steps per scale group
    constexpr int S_GROUP = (UM + BN) * 16;           // scale bytes of a group: 16 per A row and per B column
    static_assert(NB == 4 && A_DMA == 2 && B_DMA == 2 && A_STAGE == 2 * A_BLKS * 1024 && UM + BN == NTHREADS,
                  "stage split");
    static_assert(SG % NB == 0, "a scale group spans whole turns of the ring");
    __shared__ __attribute__((aligned(1024))) uint8_t s_a[NB][A_STAGE];
    __shared__ __attribute__((aligned(1024))) uint8_t s_b[NB][B_STAGE];
    __shared__ __attribute__((aligned(16))) uint8_t s_sc[2][S_GROUP];
    __shared__ int s_mt[kMaxExperts + 1];
    __shared__ int s_tmp[NWAVES];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int mh = wave / WN;
    const int nq = wave % WN;
    const int h = lane >> 5;

    build_tile_prefix<NTHREADS, UM>(p.offsets, p.E_loc, s_mt, s_tmp);
    const int NT = p.N / BN;
    const int total = s_mt[p.E_loc] * NT;
    const int nk = p.Kd / kMxStepK;
    const int kb32 = p.Kd / 32;
    const __amdgpu_buffer_rsrc_t a_rsrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p.a), 0, kBufferRange, kBufferFlags);
    const __amdgpu_buffer_rsrc_t as_rsrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p.a_scales), 0, kBufferRange, kBufferFlags);
    const __amdgpu_buffer_rsrc_t b_rsrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p.b), 0, kBufferRange, kBufferFlags);
    const __amdgpu_buffer_rsrc_t bs_rsrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p.b_scales), 0, kBufferRange, kBufferFlags);

    const int G = gridDim.x;
    const int bid = blockIdx.x;
    const int lid = (G % 8 == 0) ? (bid % 8) * (G / 8) + (bid / 8) : bid;

    for (int tile = lid; tile < total; tile += G) {
        int lo = 0, hi = p.E_loc - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (s_mt[mid] * NT <= tile) lo = mid; else hi = mid - 1;
        }
        const int e = lo;
        const int mt_e = s_mt[e + 1] - s_mt[e];
        const int local = tile - s_mt[e] * NT;
        const int n_tile = local / mt_e;
        const int m_unit = local - n_tile * mt_e;
        const int seg0 = p.offsets[e], seg1 = p.offsets[e + 1];
        const int um = min(UM, ((seg1 - seg0 + mt_e - 1) / mt_e + 31) & ~31);
        const int row0 = seg0 + m_unit * um;
        const int rows_valid = min(um, seg1 - row0);
        if (rows_valid <= 0) continue;
        const int my_rows = rows_valid - mh * BM;
        const bool active = my_rows > 0;
        const int na = min(TM, (my_rows + 31) >> 5);

        // A code copies: the waves of a row half copy that half's rows (only its waves
        // read them), copy i of column quarter nq moving 16-row block
        // blk = mh * A_BLKS + i * WN + nq; LDS granule slot blk * 64 + lane = (row, physical granule)
        uint32_t a_off[A_DMA];
#pragma unroll
        for (int i = 0; i < A_DMA; ++i) {
            const int slot = (mh * A_BLKS + i * WN + nq) * 64 + lane;
            const int row = slot >> 2;
            const int kg = (slot & 3) ^ ((row >> 2) & 3);
            uint32_t off = kOutOfRange;
            if (row < rows_valid) {
                const int r = row0 + row;
                const int64_t src = p.a_rows != nullptr ? p.a_rows[r] : r;
                off = static_cast<uint32_t>(src * p.Kd + kg * 16);
            }
            a_off[i] = off;
        }
        // B code copies: the stage's 16 KiB are [nq][tile][part][1 KiB]; wave w copies KiB 2w, 2w + 1
        uint32_t b_off[B_DMA];
#pragma unroll
        for (int d = 0; d < B_DMA; ++d) {
            const int j = wave * B_DMA + d;
            const int q = j >> 2, t = (j >> 1) & 1, part = j & 1;
            const int64_t tl = (static_cast<int64_t>(e) * (p.N >> 6) + n_tile * WN + q) * nk * 2 + t;   // k-step 0
            b_off[d] = static_cast<uint32_t>(tl * kMxTile + part * 1024 + lane * 16);
        }
        // scale copies: threads 0..255 the A rows of the tile, 256..511 its B columns (thread t's
        // 16 bytes land at record t of the group buffer); the split falls on a wave boundary and is
        // taken on the wave index, so the descriptor stays in scalar registers
        const bool a_side = wave < UM / kWave;
        const __amdgpu_buffer_rsrc_t s_rsrc = a_side ? as_rsrc : bs_rsrc;
        uint32_t s_off;
        if (a_side) {
            s_off = kOutOfRange;
            if (tid < rows_valid) {
                const int r = row0 + tid;
                const int64_t src = p.a_rows != nullptr ? p.a_rows[r] : r;
                s_off = static_cast<uint32_t>(src * kb32);
            }
        } else {
            s_off = static_cast<uint32_t>((static_cast<int64_t>(e) * p.N + n_tile * BN + (tid - UM)) * kb32);
        }
        // the copies of k-tile kt into ring stage st: AC code copies of activations (the
        // blocks that hold the half's active row groups) and the weight copies
        auto issue = [&](auto ac, int kt, int st) {
            constexpr int AC = decltype(ac)::value;
#pragma unroll
            for (int i = 0; i < AC; ++i)
                copy16_to_lds(a_rsrc, &s_a[st][(mh * A_BLKS + i * WN + nq) * 64 * 16], a_off[i] + kt * kMxStepK);
#pragma unroll
            for (int d = 0; d < B_DMA; ++d)
                copy16_to_lds(b_rsrc, &s_b[st][(wave * B_DMA + d) * 1024], b_off[d] + kt * 2 * kMxTile);
        };
        // scale group g covers k-steps 8g .. 8g+7, blocks 16g .. 16g+15; its copy starts at block
        // b0(g) = min(16 g, Kd/32 - 16), so a k-step's byte in a record is 2 kt + h - b0(g)
        const int ng = (nk + SG - 1) / SG;
        auto group_b0 = [&](int g) { return min(16 * g, kb32 - 16); };
        auto issue_scales = [&](int buf, int g) {
            copy16_to_lds(s_rsrc, &s_sc[buf][wave * 1024], s_off + static_cast<uint32_t>(group_b0(g)));
        };

        floatx16 acc[TM][2];
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

        // The k-loop for NA active 32-row groups.  A wave copies the activation blocks of
        // its half's first NA row groups, so its copies per stage (LOADS) are fixed per
        // instantiation; each wave waits for its own copies before the barrier.
        auto kloop = [&](auto nac) {
            constexpr int NA = decltype(nac)::value;
            constexpr int AC = (2 * NA + WN - 1) / WN < A_DMA ? (2 * NA + WN - 1) / WN : A_DMA;
            constexpr int LOADS = AC + B_DMA;          // copies per thread per stage
            issue_scales(0, 0);
#pragma unroll
            for (int q = 0; q + 1 < NB; ++q) issue(IntC<AC>{}, min(q, nk - 1), q);
            // fragments of one k-step: A 2 x 16 bytes per row tile, B 2 x 16 bytes per column tile,
            // and the lane's scale bytes (row / column lane & 31, block h of the step).  B fragments
            // are double-buffered: the next stage's are read first, while this stage's MFMAs run; A
            // fragments are single: each row tile's are refilled right after its two MFMAs issue.
            // The k-loop is unrolled over a scale group (8 k-steps, two turns of the ring), so ring
            // stage, register buffer and the step's place in its group are compile-time.
            u32x4 fa[TM][2], fb[2][2][2];
            uint32_t sa[TM], sb[2][2];
            const int a_rec = (mh * BM + (lane & 31)) * 16 + h;          // + i * 512: row tile i
            const int b_rec = (UM + nq * 64 + (lane & 31)) * 16 + h;     // + t * 512: column tile t
            auto sc_off = [&](int kt) {                                  // uniform part of a scale address
                kt = min(kt, nk - 1);                                    // (the last step reads ahead of the end)
                const int g = kt / SG;
                return (g & 1) * S_GROUP + 2 * kt - group_b0(g);
            };
            auto read_a = [&](int i, int st, int so) {
                const int row = mh * BM + i * 32 + (lane & 31);
                const int sw = (row >> 2) & 3;
                fa[i][0] = *reinterpret_cast<const u32x4*>(&s_a[st][row * 64 + ((h ^ sw) << 4)]);
                fa[i][1] = *reinterpret_cast<const u32x4*>(&s_a[st][row * 64 + (((2 + h) ^ sw) << 4)]);
                sa[i] = (&s_sc[0][0])[so + a_rec + i * 512];
            };
            auto read_b = [&](int buf, int st, int so) {
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    fb[buf][t][0] =
                        *reinterpret_cast<const u32x4*>(&s_b[st][((nq * 2 + t) * 2 + 0) * 1024 + lane * 16]);
                    fb[buf][t][1] =
                        *reinterpret_cast<const u32x4*>(&s_b[st][((nq * 2 + t) * 2 + 1) * 1024 + lane * 16]);
                    sb[buf][t] = (&s_sc[0][0])[so + b_rec + t * 512];
                }
            };
            // k-step kt, at place q of its scale group (compile-time)
            auto step = [&](int kt, auto qc) {
                constexpr int q = decltype(qc)::value;
                constexpr int st = q % NB, buf = q & 1, nbuf = buf ^ 1, nst = (q + 1) % NB;
                // this thread's copies of stage kt + 1 have landed (after the group copy issued at the
                // group's first step, one more copy may still be in flight at its second)
                wait_vmcnt<q == 1 ? LOADS + 1 : LOADS>();
                __builtin_amdgcn_s_barrier();          // ... everyone's; nobody reads stage kt - 1 any more
                if constexpr (q == 0) issue_scales((kt / SG + 1) & 1, min(kt / SG + 1, ng - 1));
                issue(IntC<AC>{}, min(kt + NB - 1, nk - 1), (st + NB - 1) % NB);
                if constexpr (NA > 0) {
                    const int so = sc_off(kt + 1);
                    read_b(nbuf, nst, so);
                    __builtin_amdgcn_sched_barrier(0);
                    asm volatile("" ::: "memory");
#pragma unroll
                    for (int i = 0; i < NA; ++i) {
                        acc[i][0] = mfma_mx(fa[i][0], fa[i][1], sa[i], fb[buf][0][0], fb[buf][0][1], sb[buf][0],
                                            acc[i][0]);
                        acc[i][1] = mfma_mx(fa[i][0], fa[i][1], sa[i], fb[buf][1][0], fb[buf][1][1], sb[buf][1],
                                            acc[i][1]);
                        read_a(i, nst, so);
                        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);   // the two MFMAs ...
                        __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);   // ... then the row tile's reads
                    }
                }
            };
            wait_vmcnt<LOADS * (NB - 2)>();            // scale group 0 and stage 0 have landed
            __builtin_amdgcn_s_barrier();
            if constexpr (NA > 0) {
                const int so = sc_off(0);
                read_b(0, 0, so);
#pragma unroll
                for (int i = 0; i < NA; ++i) read_a(i, 0, so);
            }
            int kt0 = 0;
            for (; kt0 + SG <= nk; kt0 += SG) {
                step(kt0 + 0, IntC<0>{});
                step(kt0 + 1, IntC<1>{});
                step(kt0 + 2, IntC<2>{});
                step(kt0 + 3, IntC<3>{});
                step(kt0 + 4, IntC<4>{});
                step(kt0 + 5, IntC<5>{});
                step(kt0 + 6, IntC<6>{});
                step(kt0 + 7, IntC<7>{});
            }
            if (kt0 < nk) {                            // nk % 8 == 4: the half group
                step(kt0 + 0, IntC<0>{});
                step(kt0 + 1, IntC<1>{});
                step(kt0 + 2, IntC<2>{});
                step(kt0 + 3, IntC<3>{});
            }
        };
        switch (active ? na : 0) {
            case 4: kloop(IntC<4>{}); break;
            case 3: kloop(IntC<3>{}); break;
            case 2: kloop(IntC<2>{}); break;
            case 1: kloop(IntC<1>{}); break;
            default: kloop(IntC<0>{}); break;
        }

        // epilogue: lane holds column (lane & 31) and rows 8*(v/4) + 4*(lane/32) + v%4 of each 32x32 tile
        if (active) {
            OutT* __restrict__ C = static_cast<OutT*>(p.c);
            const int pc0 = n_tile * BN + nq * 64;
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                if (i >= na) break;
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int r = i * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
                    const bool live = r < my_rows;
                    const int64_t row = row0 + mh * BM + r;
                    if constexpr (MODE == kSwiGLU && OUT == kMxOutMX) {
                        const float hv = silu(acc[i][0][v]) * acc[i][1][v];
                        store_mx_block(hv, live, &C[row * p.ldc + (pc0 >> 1) + (lane & 31)],
                                       &p.c_scales[row * (p.ldc / 32) + (pc0 >> 6)]);
                        continue;
                    }
                    if (!live) continue;
                    OutT* crow = C + row * p.ldc;
                    if constexpr (OUT != kMxOutMX) {
                        if constexpr (MODE == kSwiGLU) {
                            store_out<OUT>(crow + (pc0 >> 1) + (lane & 31), silu(acc[i][0][v]) * acc[i][1][v]);
                        } else if constexpr (MODE == kGateUpPlain) {
                            const int q = pc0 >> 6, w = lane & 31;
                            store_out<OUT>(crow + q * 32 + w, acc[i][0][v]);
                            store_out<OUT>(crow + p.I + q * 32 + w, acc[i][1][v]);
                        } else {
                            store_out<OUT>(crow + pc0 + (lane & 31), acc[i][0][v]);
                            store_out<OUT>(crow + pc0 + 32 + (lane & 31), acc[i][1][v]);
                        }
                    }
                }
            }
        }
        __syncthreads();   // LDS reuse by the next tile; drains this tile's copies
    }
}

// ---------------------------------------------------------------------------
// Weight-streaming form (few rows per expert, decode): one workgroup per
// (expert, 64-column block); the four waves take every fourth k-step and
// stream their weight tiles and scale bytes straight into a register ring BD
// steps deep, with the matching activation codes and scales of up to 64 rows
// (rows past the segment load zeros through the buffer range); the four
// partial tiles are added in wave order through LDS.
// ---------------------------------------------------------------------------
template <int MODE, int OUT, int BD>
__global__ __launch_bounds__(256, 2) void grouped_gemm_mx_skinny_kernel(MxArgs p) {
    typedef typename MxOutType<OUT>::type OutT;
    constexpr int MTMAX = 2;
    __shared__ __attribute__((aligned(16))) float s_red[4][MTMAX][2][16][64];

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int h = lane >> 5;
    const int nblk = p.N >> 6;
    const int e = blockIdx.x / nblk;
    const int nb = blockIdx.x - e * nblk;
    const int nk = p.Kd / kMxStepK;                    // a multiple of 4 (Kd % 256 == 0)
    const int kq = nk >> 2;                            // k-steps of this wave: wave, wave + 4, ...
    const int kb32 = p.Kd / 32;

    const __amdgpu_buffer_rsrc_t b_rsrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p.b), 0, kBufferRange, kBufferFlags);
    const __amdgpu_buffer_rsrc_t bs_rsrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p.b_scales), 0, kBufferRange, kBufferFlags);
    const __amdgpu_buffer_rsrc_t a_rsrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p.a), 0, kBufferRange, kBufferFlags);
    const __amdgpu_buffer_rsrc_t as_rsrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p.a_scales), 0, kBufferRange, kBufferFlags);

    // this wave's k-step kk (0 .. kq-1) is global step wave + 4 kk
    const uint32_t b_base = static_cast<uint32_t>(((static_cast<int64_t>(e) * nblk + nb) * nk) * 2 * kMxTile) +
                            lane * 16;
    const uint32_t bs_base[2] = {
        static_cast<uint32_t>((static_cast<int64_t>(e) * p.N + nb * 64 + (lane & 31)) * kb32 + h),
        static_cast<uint32_t>((static_cast<int64_t>(e) * p.N + nb * 64 + 32 + (lane & 31)) * kb32 + h)};
    u32x4 fb[BD][2][2];
    uint32_t sb[BD][2];
    auto load_b = [&](int slot, int kk) {
        const int ks = wave + 4 * min(kk, kq - 1);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const uint32_t o = b_base + static_cast<uint32_t>((ks * 2 + t) * kMxTile);
            fb[slot][t][0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(b_rsrc, o, 0, 0));
            fb[slot][t][1] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(b_rsrc, o + 1024, 0, 0));
            sb[slot][t] = __builtin_amdgcn_raw_buffer_load_b8(bs_rsrc, bs_base[t] + 2 * ks, 0, 0);
        }
    };
    // routing entries first (a derived dispatch), then the first ring of weight
    // loads, which needs no routing data: it is in flight while the expert's
    // row range and row indices are read or derived
    const bool derived = p.topk_idx != nullptr;        // uniform
    int pre[kDerivePrefetch];
    if (derived) derive_prefetch(p, pre);
#pragma unroll
    for (int j = 0; j < BD; ++j) load_b(j, j);

    __shared__ int s_cnt[kDeriveMaxE];
    __shared__ int s_list[kDeriveMaxT];
    __shared__ int s_w4[4];
    int seg0, rows;
    if (derived) {
        derive_dispatch(p, e, nb, s_cnt, s_list, s_w4, seg0, rows, pre);
    } else {
        seg0 = p.offsets[e];
        rows = p.offsets[e + 1] - seg0;
    }
    if (rows <= 0) {
#pragma unroll
        for (int j = 0; j < BD; ++j)
            asm volatile("" ::"v"(fb[j][0][0]), "v"(fb[j][0][1]), "v"(fb[j][1][0]), "v"(fb[j][1][1]), "v"(sb[j][0]),
                         "v"(sb[j][1]));
        return;
    }

    auto group = [&](auto mt_tag, int g0) {
        constexpr int MT = decltype(mt_tag)::value;
        if (g0 != 0) {
#pragma unroll
            for (int j = 0; j < BD; ++j) load_b(j, j);
        }
        uint32_t a_off[MT], as_off[MT];
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            const int rr = g0 + t * 32 + (lane & 31);
            const bool ok = rr < rows;
            const int64_t src = !ok ? 0
                                : derived ? s_list[rr] / p.K
                                : (p.a_rows != nullptr ? p.a_rows[seg0 + rr] : seg0 + rr);
            a_off[t] = ok ? static_cast<uint32_t>(src * p.Kd + h * 16) : kOutOfRange;
            as_off[t] = ok ? static_cast<uint32_t>(src * kb32 + h) : kOutOfRange;
        }
        floatx16 acc[MT][2];
#pragma unroll
        for (int t = 0; t < MT; ++t)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[t][j][v] = 0.0f;
        u32x4 fa[BD][MT][2];
        uint32_t sa[BD][MT];
        auto load_a = [&](int slot, int kk) {
            const int ks = wave + 4 * min(kk, kq - 1);
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                const uint32_t o = a_off[t] + static_cast<uint32_t>(ks * kMxStepK);
                fa[slot][t][0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(a_rsrc, o, 0, 0));
                fa[slot][t][1] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(a_rsrc, o + 32, 0, 0));
                sa[slot][t] = __builtin_amdgcn_raw_buffer_load_b8(as_rsrc, as_off[t] + 2 * ks, 0, 0);
            }
        };
        auto step = [&](int j) {
#pragma unroll
            for (int t = 0; t < MT; ++t)
#pragma unroll
                for (int c = 0; c < 2; ++c)
                    acc[t][c] = mfma_mx(fa[j][t][0], fa[j][t][1], sa[j][t], fb[j][c][0], fb[j][c][1], sb[j][c],
                                        acc[t][c]);
        };
#pragma unroll
        for (int j = 0; j < BD; ++j) load_a(j, j);
        int kb = 0;
        for (; kb + BD <= kq; kb += BD) {
#pragma unroll
            for (int j = 0; j < BD; ++j) {
                step(j);
                load_b(j, kb + j + BD);
                load_a(j, kb + j + BD);
            }
        }
#pragma unroll
        for (int j = 0; j < BD; ++j)
            if (kb + j < kq) step(j);

#pragma unroll
        for (int t = 0; t < MT; ++t)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) s_red[wave][t][j][v][lane] = acc[t][j][v];
        __syncthreads();
        {
            OutT* __restrict__ C = static_cast<OutT*>(p.c);
            const int pc0 = nb * 64;
#pragma unroll 2
            for (int i = 0; i < MT * 16 * 64 / 256; ++i) {
                const int idx = static_cast<int>(threadIdx.x) + i * 256;
                const int ln = idx & 63, v = (idx >> 6) & 15, t = idx >> 10;
                const int r = g0 + t * 32 + 8 * (v >> 2) + 4 * (ln >> 5) + (v & 3);
                float g = s_red[0][t][0][v][ln], u = s_red[0][t][1][v][ln];
#pragma unroll
                for (int w = 1; w < 4; ++w) {
                    g += s_red[w][t][0][v][ln];
                    u += s_red[w][t][1][v][ln];
                }
                const bool live = r < rows;
                const int64_t row = seg0 + r;
                if constexpr (MODE == kSwiGLU && OUT == kMxOutMX) {
                    store_mx_block(silu(g) * u, live, &C[row * p.ldc + (pc0 >> 1) + (ln & 31)],
                                   &p.c_scales[row * (p.ldc / 32) + (pc0 >> 6)]);
                } else if constexpr (OUT != kMxOutMX) {
                    if (live) {
                        OutT* crow = C + row * p.ldc;
                        if constexpr (MODE == kSwiGLU) {
                            store_out<OUT>(crow + (pc0 >> 1) + (ln & 31), silu(g) * u);
                        } else if constexpr (MODE == kGateUpPlain) {
                            const int q = pc0 >> 6, wc = ln & 31;
                            store_out<OUT>(crow + q * 32 + wc, g);
                            store_out<OUT>(crow + p.I + q * 32 + wc, u);
                        } else {
                            store_out<OUT>(crow + pc0 + (ln & 31), g);
                            store_out<OUT>(crow + pc0 + 32 + (ln & 31), u);
                        }
                    }
                }
            }
        }
        __syncthreads();
    };
    for (int g0 = 0; g0 < rows;) {
        if (rows - g0 <= 32) {
            group(IntC<1>{}, g0);
            g0 += 32;
        } else {
            group(IntC<2>{}, g0);
            g0 += 64;
        }
    }
}

template <int MODE, int OUT>
int launch_mx(const MxArgs& args, int max_rows, bool skinny, hipStream_t st) {
    if (skinny) {
        const int64_t grid = static_cast<int64_t>(args.E_loc) * (args.N / 64);
        hipLaunchKernelGGL((grouped_gemm_mx_skinny_kernel<MODE, OUT, 2>), dim3(static_cast<unsigned>(grid)),
                           dim3(256), 0, st, args);
    } else {
        const int64_t units = (static_cast<int64_t>(max_rows) + 255) / 256 + args.E_loc;
        const int64_t tiles = units * (args.N / 256);
        int dev = 0, cus = 256;
        if (hipGetDevice(&dev) == hipSuccess) {
            int v = 0;
            if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0) cus = v;
        }
        int64_t grid = cus;
        if (tiles < grid) grid = tiles;
        if (grid < 1) grid = 1;
        hipLaunchKernelGGL((grouped_gemm_mx_kernel<MODE, OUT, 4>), dim3(static_cast<unsigned>(grid)), dim3(512), 0,
                           st, args);
    }
    MOE_CHECK_LAUNCH();
    return MOE_OK;
}

template <int MODE>
int launch_mx_out(const MxArgs& args, int max_rows, bool skinny, int c_dtype, hipStream_t st) {
    switch (c_dtype) {
        case MOE_F32: return launch_mx<MODE, kMxOutF32>(args, max_rows, skinny, st);
        case MOE_BF16: return launch_mx<MODE, kMxOutBF16>(args, max_rows, skinny, st);
        case MOE_F16: return launch_mx<MODE, kMxOutF16>(args, max_rows, skinny, st);
        default:
            if constexpr (MODE == kSwiGLU) return launch_mx<MODE, kMxOutMX>(args, max_rows, skinny, st);
            return MOE_ERR_UNSUPPORTED;
    }
}

}  // namespace

size_t mx_packed_gate_up_code_bytes(const moe_shape& s) {
    return static_cast<size_t>(s.e_end - s.e_begin) * 2 * s.I * s.H;
}
size_t mx_packed_down_code_bytes(const moe_shape& s) { return static_cast<size_t>(s.e_end - s.e_begin) * s.H * s.I; }
size_t mx_packed_weight_bytes(const moe_shape& s) {
    const size_t codes = mx_packed_gate_up_code_bytes(s) + mx_packed_down_code_bytes(s);
    return codes + codes / 32;
}

int launch_mx_pack_weights(const moe_shape& s, const void* w_gate, const void* w_up, const void* w_down, int dtype,
                           uint8_t* packed, hipStream_t st) {
    const int E_loc = s.e_end - s.e_begin;
    uint8_t* gu = packed;
    uint8_t* dn = gu + mx_packed_gate_up_code_bytes(s);
    uint8_t* gus = dn + mx_packed_down_code_bytes(s);
    uint8_t* dns = gus + mx_packed_gate_up_code_bytes(s) / 32;
    const dim3 g_gu((s.I + 255) / 256, s.H / 32, E_loc), g_dn((s.H + 255) / 256, s.I / 32, E_loc);
    if (dtype == MOE_BF16) {
        auto g = static_cast<const uint16_t*>(w_gate);
        auto u = static_cast<const uint16_t*>(w_up);
        auto d = static_cast<const uint16_t*>(w_down);
        hipLaunchKernelGGL(mx_pack_weights_kernel<uint16_t>, g_gu, dim3(256), 0, st, g, s.H, s.I, 2 * s.I, 1, 0, gu, gus);
        hipLaunchKernelGGL(mx_pack_weights_kernel<uint16_t>, g_gu, dim3(256), 0, st, u, s.H, s.I, 2 * s.I, 1, 1, gu, gus);
        hipLaunchKernelGGL(mx_pack_weights_kernel<uint16_t>, g_dn, dim3(256), 0, st, d, s.I, s.H, s.H, 0, 0, dn, dns);
    } else {
        auto g = static_cast<const float*>(w_gate);
        auto u = static_cast<const float*>(w_up);
        auto d = static_cast<const float*>(w_down);
        hipLaunchKernelGGL(mx_pack_weights_kernel<float>, g_gu, dim3(256), 0, st, g, s.H, s.I, 2 * s.I, 1, 0, gu, gus);
        hipLaunchKernelGGL(mx_pack_weights_kernel<float>, g_gu, dim3(256), 0, st, u, s.H, s.I, 2 * s.I, 1, 1, gu, gus);
        hipLaunchKernelGGL(mx_pack_weights_kernel<float>, g_dn, dim3(256), 0, st, d, s.I, s.H, s.H, 0, 0, dn, dns);
    }
    MOE_CHECK_LAUNCH();
    return MOE_OK;
}

int launch_mx_quantize(int64_t rows, int K, const void* x, int x_dtype, uint8_t* codes, uint8_t* scales,
                       hipStream_t st) {
    const int64_t groups = rows * (K / 8);
    if (groups == 0) return MOE_OK;
    const dim3 grid(static_cast<unsigned>((groups + 255) / 256));
    if (x_dtype == MOE_BF16)
        hipLaunchKernelGGL(mx_quantize_kernel<uint16_t>, grid, dim3(256), 0, st, static_cast<const uint16_t*>(x),
                           groups, K, codes, scales);
    else
        hipLaunchKernelGGL(mx_quantize_kernel<float>, grid, dim3(256), 0, st, static_cast<const float*>(x), groups, K,
                           codes, scales);
    MOE_CHECK_LAUNCH();
    return MOE_OK;
}

bool mx_gemm_streams_weights(const moe_shape& s) {
    return static_cast<int64_t>(s.T) * s.K <= static_cast<int64_t>(64) * s.E;
}

bool mx_gemm_can_derive_dispatch(const moe_shape& s) {
    return mx_gemm_streams_weights(s) && s.H % 256 == 0 && s.T <= kDeriveMaxT && s.e_end - s.e_begin <= kDeriveMaxE &&
           static_cast<int64_t>(s.T) * s.H + 64 <= kBufferRange &&
           static_cast<int64_t>(s.e_end - s.e_begin) * 2 * s.I * s.H + 4096 <= kBufferRange;
}

int launch_mx_gate_up_deriving_dispatch(const moe_shape& s, const uint8_t* x_codes, const uint8_t* x_scales,
                                        const int32_t* topk_idx, const uint8_t* packed, uint8_t* h_codes,
                                        uint8_t* h_scales, int32_t* counts, int32_t* offsets, int32_t* row_token,
                                        int32_t* row_slot, int32_t* slot_row, hipStream_t st) {
    if (!mx_gemm_can_derive_dispatch(s)) return MOE_ERR_UNSUPPORTED;
    MxArgs args{};
    args.a = x_codes;
    args.a_scales = x_scales;
    args.a_rows_bound = s.T;
    args.c = h_codes;
    args.c_scales = h_scales;
    args.E_loc = s.e_end - s.e_begin;
    args.I = s.I;
    args.b = packed;
    args.b_scales = packed + mx_packed_gate_up_code_bytes(s) + mx_packed_down_code_bytes(s);
    args.N = 2 * s.I;
    args.Kd = s.H;
    args.ldc = s.I;
    args.topk_idx = topk_idx;
    args.e_begin = s.e_begin;
    args.T = s.T;
    args.K = s.K;
    args.d_counts = counts;
    args.d_offsets = offsets;
    args.d_row_token = row_token;
    args.d_row_slot = row_slot;
    args.d_slot_row = slot_row;
    const int64_t grid = static_cast<int64_t>(args.E_loc) * (args.N / 64);
    hipLaunchKernelGGL((grouped_gemm_mx_skinny_kernel<kSwiGLU, kMxOutMX, 2>), dim3(static_cast<unsigned>(grid)),
                       dim3(256), 0, st, args);
    MOE_CHECK_LAUNCH();
    return MOE_OK;
}

int launch_mx_grouped_gemm(const moe_shape& s, const uint8_t* a, const uint8_t* a_scales, const int32_t* a_rows,
                           const int32_t* offsets, const uint8_t* packed, int which, int epilogue, void* c,
                           int c_dtype, uint8_t* c_scales, hipStream_t st) {
    const int E_loc = s.e_end - s.e_begin;
    const int max_rows = s.T * (s.K < E_loc ? s.K : E_loc);
    MxArgs args{};
    args.a = a;
    args.a_scales = a_scales;
    args.a_rows = a_rows;
    args.a_rows_bound = a_rows != nullptr ? s.T : max_rows;
    args.offsets = offsets;
    args.c = c;
    args.c_scales = c_scales;
    args.E_loc = E_loc;
    args.I = s.I;
    const uint8_t* gu = packed;
    const uint8_t* dn = gu + mx_packed_gate_up_code_bytes(s);
    const uint8_t* gus = dn + mx_packed_down_code_bytes(s);
    const uint8_t* dns = gus + mx_packed_gate_up_code_bytes(s) / 32;
    // every buffer offset stays below 2^31 (the resources' range)
    const int64_t kd = which == MOE_GEMM_GATE_UP ? s.H : s.I;
    const int64_t nn = which == MOE_GEMM_GATE_UP ? 2 * s.I : s.H;
    if (static_cast<int64_t>(args.a_rows_bound) * kd + 64 > kBufferRange || E_loc * nn * kd + 4096 > kBufferRange)
        return MOE_ERR_UNSUPPORTED;
    // the tiled form stages scales 16 blocks at a time and needs K >= 512; below that every launch
    // takes the weight-streaming form, whatever the row count
    const bool skinny = (mx_gemm_streams_weights(s) && kd % 256 == 0) || kd < 512;
    if (which == MOE_GEMM_GATE_UP) {
        args.b = gu;
        args.b_scales = gus;
        args.N = 2 * s.I;
        args.Kd = s.H;
        args.ldc = epilogue == MOE_EPI_SWIGLU ? s.I : 2 * s.I;
        if (epilogue == MOE_EPI_SWIGLU) return launch_mx_out<kSwiGLU>(args, max_rows, skinny, c_dtype, st);
        return launch_mx_out<kGateUpPlain>(args, max_rows, skinny, c_dtype, st);
    }
    args.b = dn;
    args.b_scales = dns;
    args.N = s.H;
    args.Kd = s.I;
    args.ldc = s.H;
    return launch_mx_out<kPlain>(args, max_rows, skinny, c_dtype, st);
}

}  // namespace moe
