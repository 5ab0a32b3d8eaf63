// Grouped expert GEMMs on MFMA, plus the static weight packing they stream.
//
// "Hosting Qwen on Blackwell" (Perplexity), section "MoE GEMM": the dispatched
// tokens of each expert form one matrix-multiply problem; with about 375
// tokens per expert at a 6000-token prefill ("Pre-remplisseurs") the problem
// is dense and compute-bound, while decode is bound by streaming the weights
// from HBM ("Decodeurs").
//
// Kernel shape (gfx950):
//   * workgroup tile = two 128-row slabs of one expert x (64 * WN) columns, with
//     2 x WN waves (WN = 4 for the prefill shapes: 8 waves, two per SIMD, so
//     one wave's MFMAs run while the other waits on memory); every wave owns
//     128 rows x 64 columns: 4 x 2 tiles of v_mfma_f32_32x32x16_{bf16,f16},
//     128 float32 accumulators per lane.  The two slabs share every weight
//     copy; an expert's odd last slab leaves one half idle at no time cost, so
//     rows are padded only to 128;
//   * activation rows can be gathered straight from the unpacked input
//     through the dispatch's row-to-token map (no packed copy);
//   * both operands reach LDS through direct global->LDS copies (no register
//     staging) into a ring of NB = 4 stages: while one stage is read, the next
//     has landed and the two after it are in flight; the kernel waits on its
//     own copy counter (s_waitcnt vmcnt) and a raw barrier, since copies
//     retire in order;
//   * activations (A): 16-byte granules of 64-byte stage rows, XOR-swizzled by
//     row group so fragment reads are bank-conflict free (16 lanes of a 128-bit
//     read per pass over 64 banks); all NW waves read all 128 rows;
//   * a stage is 32 k: 16 KiB of activations (256 rows x 64 bytes) and 16 KiB
//     of weights (256 columns), 128 KiB for the ring; at the prefill shapes
//     this copy path, not the MFMAs, sets the kernel's pace;
//   * the waves of a row half copy that half's activation rows, and only the
//     16-row blocks that hold its active 32-row groups (a 183-row tile copies
//     192 rows per stage, not 256); the count is fixed per k-loop instance, so
//     every copy wait stays a compile-time constant;
//   * weights (B) are packed once in MFMA fragment order (one 1 KiB block per
//     32 columns x 16 k, lane-major), the two 32-column halves of each
//     64-column block side by side per 16 k: every copy and every fragment
//     read is one contiguous, conflict-free 1 KiB per wave, each wave reads
//     only its own columns, and a 64-column block's weights are one
//     contiguous run;
//   * fragments are read from LDS one k-step ahead of the MFMAs that use them,
//     and the once-per-stage barrier sits between a stage's two k-steps, so it
//     waits while MFMAs are still executing and every stage starts with its
//     operands already in registers;
//   * the k-loop is instantiated per count of active 32-row groups (0 .. 4)
//     and chosen once per tile, so a k-step has no branch: its six fragment
//     reads issue back to back, with no wait between them, and a scheduling
//     barrier keeps them ahead of the MFMAs they overlap;
//   * persistent workgroups walk a tile list laid out per expert as
//     [n-tile][m-tile], so workgroups that run together share one weight
//     tile; tile ids are split into one contiguous range per XCD (workgroup b
//     runs on XCD b % 8), keeping those sharers inside one L2; an expert's
//     rows are split into m-tiles of equal height, so the sharers do equal
//     work and stay in step, and MFMAs of 32-row groups past the segment are
//     skipped;
//   * m-tiles per expert come from the device-side offsets (no host sync);
//   * epilogues: plain store (float32, bf16 or fp16), or SwiGLU for the
//     gate/up problem, whose weights are packed so that each 64-column block
//     holds 32 gate columns then the same 32 up columns: a lane owns g and u
//     of the same output element and applies silu(g) * u in registers.
//
// Operand types: the gate/up problem multiplies in the weights' own type
// (bf16), or in fp16 for float32 weights; the down problem multiplies the
// SwiGLU activations in fp16 (eight times finer rounding than bf16) with the
// down weights converted to fp16 once at packing time.
#include "gemm_common.hpp"

namespace moe {
namespace {

constexpr int BM = 128;                // rows per workgroup tile
constexpr int BK = 32;                 // k per LDS stage (64 bytes of 16-bit data per row)
constexpr int KG = BK / 8;             // 16-byte granules per row of a stage
constexpr int kFragElems = 512;        // one 32-column x 16-k fragment block (64 lanes x 8)

// Packed weights: fragment block of expert e, 32-column tile n32 and 16-k block
// kb, in [E_loc][N/64][Kd/16][2] order (the pair of 32-column tiles of a
// 64-column block sits side by side at every kb).
__device__ __forceinline__ int64_t frag_block(int e, int n32, int kb, int N, int kblocks) {
    return ((static_cast<int64_t>(e) * (N >> 6) + (n32 >> 1)) * kblocks + kb) * 2 + (n32 & 1);
}


struct GemmArgs {
    const uint16_t* a;         // [rows][Kd] 16-bit
    const int32_t* a_rows;     // NULL, or: packed row r reads row a_rows[r] of a (gather)
    const uint16_t* b;         // [E_loc][N/64][Kd/16][2] fragment blocks
    const int32_t* offsets;    // [E_loc + 1]
    void* c;                   // output rows
    int E_loc;
    int N;                     // packed output columns of B (2I for gate/up, H for down)
    int Kd;                    // reduction length
    int ldc;                   // output row stride (elements)
    int I;                     // intermediate size (gate/up column remap)
    int skinny;                // few rows per expert expected: weight-streaming kernel
    // weight-streaming gate/up only, optional: derive the dispatch from the
    // routing instead of reading offsets / a_rows (a holds the unpacked rows)
    const int32_t* topk_idx;   // [T][K] expert ids, NULL: not derived
    int e_begin, T, K;
    int32_t* d_counts;         // dispatch outputs, written by each expert's first column block
    int32_t* d_offsets;
    int32_t* d_row_token;
    int32_t* d_row_slot;
    int32_t* d_slot_row;
};


__device__ __forceinline__ int swz(int row, int kg) {
    // Swizzled granule position of logical granule kg (0..3) of a 64-byte row.
    // Four rows share one 256-byte bank line; XOR with (row / 4) % 4 puts the
    // same granule of 16 consecutive rows (one ds_read_b128 pass: 16 lanes over
    // 64 banks) in 16 distinct 4-bank groups.
    return kg ^ ((row >> 2) & (KG - 1));
}

__device__ __forceinline__ int lds_off(int row, int kg) {
    // element offset of logical granule kg of a row
    return row * BK + (swz(row, kg) << 3);
}


template <bool F16>
__device__ __forceinline__ floatx16 mfma32(const u32x4& a, const u32x4& b, floatx16 c) {
    if constexpr (F16)
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(halfx8_t, a),
                                                      __builtin_bit_cast(halfx8_t, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                       __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}


template <int WN, int MODE, bool F16, int OUT, int NB>
__global__ __launch_bounds__(WN * 128, 1) void grouped_gemm_kernel(GemmArgs p) {
    typedef typename OutType<OUT>::type OutT;
    constexpr int NWAVES = 2 * WN;                     // 2 row halves x WN column quarters
    constexpr int NTHREADS = NWAVES * 64;
    constexpr int BN = WN * 64;
    constexpr int UM = 2 * BM;                         // rows per tile: two 128-row slabs
    constexpr int TM = BM / 32;                        // 32-row MFMA tiles per wave
    constexpr int KS = BK / 16;                        // MFMA k-steps per stage
    constexpr int A_BLKS = BM / 16;                    // 16-row copy blocks of one row half
    constexpr int A_DMA = A_BLKS / WN;                 // A copies per thread per stage, at most
    constexpr int B_BLK = 2 * KS;                      // B blocks per wave column per stage
    constexpr int B_DMA = B_BLK * WN / NWAVES;         // B copies per thread per stage
    static_assert(A_BLKS % WN == 0 && (B_BLK * WN) % NWAVES == 0, "stage must split evenly");

    __shared__ __attribute__((aligned(16))) uint16_t s_a[NB][UM * BK];
    __shared__ __attribute__((aligned(16))) uint16_t s_b[NB][WN][B_BLK][kFragElems];
    __shared__ int s_mt[kMaxExperts + 1];
    __shared__ int s_tmp[NWAVES];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int mh = wave / WN;                          // row half of this wave
    const int nq = wave % WN;                          // column quarter of this wave

    build_tile_prefix<NTHREADS, UM>(p.offsets, p.E_loc, s_mt, s_tmp);
    const int NT = p.N / BN;
    const int total = s_mt[p.E_loc] * NT;
    const int nk = p.Kd / BK;
    const int kblocks = p.Kd / 16;                     // fragment blocks per 32-column stream

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
        const int m_unit = local - n_tile * mt_e;
        const int seg0 = p.offsets[e], seg1 = p.offsets[e + 1];
        // the expert's rows are split into mt_e tiles of equal height (a multiple
        // of 32, at most UM), so the tiles that share one weight tile do equal
        // work and stream it through L2 together
        const int um = min(UM, ((seg1 - seg0 + mt_e - 1) / mt_e + 31) & ~31);
        const int row0 = seg0 + m_unit * um;
        const int rows_valid = min(um, seg1 - row0);
        if (rows_valid <= 0) continue;                  // uniform: the whole workgroup skips
        const int my_rows = rows_valid - mh * BM;      // rows of this wave's half (<= 0: idle half)
        const bool active = my_rows > 0;
        const int na = min(TM, (my_rows + 31) >> 5);   // 32-row MFMA tiles holding valid rows

        // A copies of this thread: the waves of a row half copy that half's rows (only
        // its waves read them), copy i of column quarter nq moving 16-row block
        // blk = mh * A_BLKS + i * WN + nq.  LDS granule slot blk * 64 + lane holds
        // swizzled position (row, g'); the swizzle is an involution, so the logical
        // granule is swz(row, g').  Rows past the segment copy the tile's first row
        // (never stored).  With a_rows the row is gathered from the unpacked input.
        const uint16_t* a_src[A_DMA];
#pragma unroll
        for (int i = 0; i < A_DMA; ++i) {
            const int slot = (mh * A_BLKS + i * WN + nq) * 64 + lane;
            const int row = slot / KG;
            const int kg = swz(row, slot % KG);
            const int r = row0 + (row < rows_valid ? row : 0);
            const int64_t src = p.a_rows != nullptr ? p.a_rows[r] : r;
            a_src[i] = p.a + src * p.Kd + kg * 8;
        }
        // B copies of this thread: blocks j = jb .. jb+B_DMA-1 of column quarter bq
        // (block j: stream j % 2, k-step j / 2)
        const int bq = (wave * B_DMA) / B_BLK;
        const int jb = (wave * B_DMA) % B_BLK;
        const uint16_t* b_src[2];
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
            b_src[s2] = p.b + frag_block(e, ((n_tile * BN + bq * 64) >> 5) + s2, 0, p.N, kblocks) * kFragElems +
                        lane * 8;
        // issue the copies of k-tile kt into ring stage st: AC activation copies (the
        // blocks that hold the half's active row groups) and the weight copies
        auto issue = [&](auto ac, int kt, int st) {
            constexpr int AC = decltype(ac)::value;
#pragma unroll
            for (int i = 0; i < AC; ++i) dma16(a_src[i] + kt * BK, &s_a[st][((mh * A_BLKS + i * WN + nq) * 64) * 8]);
#pragma unroll
            for (int d = 0; d < B_DMA; ++d) {
                const int j = jb + d;
                dma16(b_src[j & 1] + static_cast<int64_t>(kt * KS + (j >> 1)) * 2 * kFragElems, &s_b[st][bq][j][0]);
            }
        };
        floatx16 acc[TM][2];
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

        // The k-loop for NA active 32-row groups (0: an idle half that copies only
        // weights and synchronises).  NA is fixed per tile, so a k-step is one basic
        // block: its fragment reads and MFMAs interleave with no wait between reads.
        // A wave copies the activation blocks of its half's first NA row groups, so
        // its copies per stage (LOADS) are fixed per instantiation too; each wave
        // waits for its own copies before the barrier.
        auto kloop = [&](auto nac) {
            constexpr int NA = decltype(nac)::value;
            constexpr int AC = (2 * NA + WN - 1) / WN < A_DMA ? (2 * NA + WN - 1) / WN : A_DMA;
            constexpr int LOADS = AC + B_DMA;          // vector-memory operations per thread per stage
            // prologue: k-tiles 0 .. NB-2 in flight (indices past the end are clamped:
            // harmless copies keep the per-stage operation count constant)
#pragma unroll
            for (int q = 0; q + 1 < NB; ++q) issue(IntC<AC>{}, min(q, nk - 1), q);
            u32x4 fa_cur[TM], fb_cur[2], fa_nxt[TM], fb_nxt[2];
            auto read_frags = [&](u32x4 (&fa)[TM], u32x4 (&fb)[2], int st, int ks) {
                const int kg = ks * 2 + (lane >> 5);
#pragma unroll
                for (int i = 0; i < NA; ++i)
                    fa[i] = *reinterpret_cast<const u32x4*>(&s_a[st][lds_off(mh * BM + i * 32 + (lane & 31), kg)]);
                fb[0] = *reinterpret_cast<const u32x4*>(&s_b[st][nq][2 * ks][lane * 8]);
                fb[1] = *reinterpret_cast<const u32x4*>(&s_b[st][nq][2 * ks + 1][lane * 8]);
            };
            auto mfmas = [&](const u32x4 (&fa)[TM], const u32x4 (&fb)[2]) {
#pragma unroll
                for (int i = 0; i < NA; ++i) {
                    acc[i][0] = mfma32<F16>(fa[i], fb[0], acc[i][0]);
                    acc[i][1] = mfma32<F16>(fa[i], fb[1], acc[i][1]);
                }
            };
            static_assert(KS == 2, "the stage schedule below is written for two k-steps");
            // One k-tile from ring stage st, entered with its first k-step's fragments
            // in fa_cur/fb_cur.  k-step 0: read k-step 1's fragments while the MFMAs
            // run.  Then wait for this thread's copies of the next stage and meet the
            // other waves (the next stage has landed everywhere, and nobody still reads
            // the stage about to be refilled) while those MFMAs drain; refill that stage
            // with k-tile kt+NB-1.  k-step 1: read the next stage's first fragments
            // while its MFMAs run.  After each batch of reads, a scheduling barrier
            // and an empty asm statement with a memory clobber keep the reads ahead
            // of the MFMAs (left alone, the compiler sinks each read next to its use
            // and waits for it there); with both, the compiler places the rest in
            // the order that measured fastest.
            auto step = [&](int kt, int st) {
                if constexpr (NA > 0) {
                    read_frags(fa_nxt, fb_nxt, st, 1);
                    __builtin_amdgcn_sched_barrier(0);
                    asm volatile("" ::: "memory");
                    mfmas(fa_cur, fb_cur);
                }
                wait_vmcnt<LOADS * (NB - 3)>();
                __builtin_amdgcn_s_barrier();
                issue(IntC<AC>{}, min(kt + NB - 1, nk - 1), (st + NB - 1) % NB);
                if constexpr (NA > 0) {
                    read_frags(fa_cur, fb_cur, (st + 1) % NB, 0);
                    __builtin_amdgcn_sched_barrier(0);
                    asm volatile("" ::: "memory");
                    mfmas(fa_nxt, fb_nxt);
                }
            };
            // stage 0 must have landed before its first fragments are read
            wait_vmcnt<LOADS * (NB - 2)>();
            __builtin_amdgcn_s_barrier();
            if constexpr (NA > 0) read_frags(fa_cur, fb_cur, 0, 0);
            int kt0 = 0;
            for (; kt0 + NB <= nk; kt0 += NB) {
#pragma unroll
                for (int q = 0; q < NB; ++q) step(kt0 + q, q);
            }
#pragma unroll
            for (int q = 0; q + 1 < NB; ++q)
                if (kt0 + q < nk) step(kt0 + q, q);
        };
        static_assert(TM == 4, "the dispatch below covers 0 .. 4 active row groups");
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
            const int pc0 = n_tile * BN + nq * 64;   // packed column of acc[.][0] (multiple of 64)
#pragma unroll
            for (int i = 0; i < TM; ++i) {
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int r = i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                    if (r >= my_rows) continue;
                    OutT* crow = C + static_cast<int64_t>(row0 + mh * BM + r) * p.ldc;
                    if constexpr (MODE == kSwiGLU) {
                        const int col = (pc0 >> 1) + (lane & 31);
                        store_out<OUT>(crow + col, silu(acc[i][0][v]) * acc[i][1][v]);
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
        __syncthreads();   // LDS reuse by the next tile; drains this tile's copies
    }
}



// ---------------------------------------------------------------------------
// Few rows per expert (decode): the weights dominate the traffic, so each
// weight byte is read once and applied to all of the expert's rows.  A
// workgroup owns one (expert, 64-column block) unit; its four waves split the
// reduction into quarters and stream their weight fragments straight from the
// fragment-packed weights into a register ring BD k-steps deep, together with
// the matching fragments of up to 64 rows (one or two 32-row MFMA tiles; an
// expert with more rows is handled in further row groups).  The four partial
// tiles are added in wave order through LDS by all threads, which then apply
// the epilogue.
// ---------------------------------------------------------------------------
template <int MODE, bool F16, int OUT, int BD>
__global__ __launch_bounds__(256, 2) void grouped_gemm_skinny_kernel(GemmArgs p) {
    typedef typename OutType<OUT>::type OutT;
    constexpr int MTMAX = 2;                           // 32-row tiles per row group, at most
    __shared__ __attribute__((aligned(16))) float s_red[4][MTMAX][2][16][64];

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nblk = p.N >> 6;
    const int e = blockIdx.x / nblk;
    const int nb = blockIdx.x - e * nblk;

    const int nks = p.Kd >> 4;                         // k-steps (a multiple of 4)
    const int kq = nks >> 2;                           // k-steps of this wave: wave, wave + 4, ...
    const int k0 = wave;
    const int kblocks = nks;
    // the workgroup's weights are one contiguous run; the four waves take every
    // fourth k-step, so together they stream it front to back, 8 KiB per step
    const uint16_t* b_src = p.b + frag_block(e, nb * 2, k0, p.N, kblocks) * kFragElems + lane * 8;
    u32x4 fb[BD][2];
    auto load_b = [&](int slot, int kk) {              // k-step kk of this wave's range (clamped)
        // weights are read once: non-temporal loads keep them from displacing
        // the activation rows in the caches
        const uint16_t* bk = b_src + static_cast<int64_t>(min(kk, kq - 1)) * 8 * kFragElems;
        fb[slot][0] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(bk));
        fb[slot][1] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(bk + kFragElems));
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
    const __amdgpu_buffer_rsrc_t a_rsrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(p.a), 0, kBufferRange, kBufferFlags);
    if (rows <= 0) {                                   // uniform over the workgroup
        // consume the ring here too, so that its loads stay ahead of the branch
#pragma unroll
        for (int j = 0; j < BD; ++j) asm volatile("" ::"v"(fb[j][0]), "v"(fb[j][1]));
        return;
    }

    // one row group: MT 32-row tiles starting at row g0 of the segment (MT = 1
    // when at most 32 rows remain, which is the usual case in decode)
    auto group = [&](auto mt_tag, int g0) {
        constexpr int MT = decltype(mt_tag)::value;
        const bool first = g0 == 0;                    // its weight ring is already in flight
        // activation rows through a buffer resource: lanes of rows past the
        // segment get an offset past its range, so their loads return zeros
        // without touching memory (a decode expert fills few of the 32 rows)
        uint32_t a_off[MT];                            // bytes; step kc adds 128 kc
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            const int rr = g0 + t * 32 + (lane & 31);
            const int r = seg0 + (rr < rows ? rr : 0);
            const int64_t src = derived ? s_list[rr < rows ? rr : 0] / p.K : (p.a_rows != nullptr ? p.a_rows[r] : r);
            a_off[t] = rr < rows ? static_cast<uint32_t>((src * p.Kd + k0 * 16 + (lane >> 5) * 8) * 2) : kOutOfRange;
        }
        floatx16 acc[MT][2];
#pragma unroll
        for (int t = 0; t < MT; ++t)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[t][j][v] = 0.0f;

        u32x4 fa[BD][MT];
        auto load_a = [&](int slot, int kk) {
            const int kc = min(kk, kq - 1);
#pragma unroll
            for (int t = 0; t < MT; ++t)
                fa[slot][t] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                            a_rsrc, a_off[t] + static_cast<uint32_t>(kc) * 128, 0, 0));
        };
        auto step = [&](int j) {
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                acc[t][0] = mfma32<F16>(fa[j][t], fb[j][0], acc[t][0]);
                acc[t][1] = mfma32<F16>(fa[j][t], fb[j][1], acc[t][1]);
            }
        };
        if (!first) {
#pragma unroll
            for (int j = 0; j < BD; ++j) load_b(j, j);
        }
#pragma unroll
        for (int j = 0; j < BD; ++j) load_a(j, j);
        // whole turns of the ring with no branches inside, so that the wait before
        // each step lets the younger BD-1 steps' loads stay in flight (a guarded
        // step would make the compiler drain every load at the turn's start)
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
            if (kb + j < kq) step(j);                  // uniform

        // the four partial tiles go through LDS; each thread then adds the four
        // partials of 8 (row, column) pairs in wave order and applies the epilogue
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
                if (r < rows) {
                    OutT* crow = C + static_cast<int64_t>(seg0 + r) * p.ldc;
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
        __syncthreads();                               // s_red reuse by the next row group
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

// ---------------------------------------------------------------------------
// Weight packing into MFMA fragment order.
// Source [E_loc][Kd][Cs] row-major (y = x W: k is the row, the output column c
// the column).  Output column c maps to packed column pcol(c): identity for
// the down weights; 64-blocks of (32 gate | 32 up) columns for gate/up.
// Fragment block (n32, k16) holds, for lane l and j < 8, the element
// (k = k16*16 + (l/32)*8 + j, packed column n32*32 + l%32); blocks of one
// 32-column stream are contiguous along k.
// One thread gathers the 8 k-consecutive values of one source column.
// ---------------------------------------------------------------------------
template <typename ST, bool F16OUT>
__global__ __launch_bounds__(256) void pack_weights_kernel(const ST* __restrict__ src, int Kd, int Cs, int N,
                                                           int gate_up, int is_up, uint16_t* __restrict__ dst) {
    const int e = blockIdx.z;
    const int k8 = blockIdx.y;                         // group of 8 consecutive k
    const int c = blockIdx.x * 256 + threadIdx.x;      // source column
    if (c >= Cs) return;
    const ST* s = src + (static_cast<int64_t>(e) * Kd + k8 * 8) * Cs + c;
    uint16_t v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        float f;
        if constexpr (sizeof(ST) == 2) f = bf16_to_f32(s[static_cast<int64_t>(j) * Cs]);
        else f = s[static_cast<int64_t>(j) * Cs];
        v[j] = F16OUT ? f32_to_f16_sat(f) : f32_to_bf16(f);
    }
    const int pcol = gate_up ? (c >> 5) * 64 + (is_up ? 32 : 0) + (c & 31) : c;
    const int n32 = pcol >> 5;
    const int lanei = (pcol & 31) + 32 * (k8 & 1);
    const int k16 = k8 >> 1;
    uint16_t* d = dst + frag_block(e, n32, k16, N, Kd >> 4) * kFragElems + lanei * 8;
    u32x4 o;
    o[0] = v[0] | (static_cast<uint32_t>(v[1]) << 16);
    o[1] = v[2] | (static_cast<uint32_t>(v[3]) << 16);
    o[2] = v[4] | (static_cast<uint32_t>(v[5]) << 16);
    o[3] = v[6] | (static_cast<uint32_t>(v[7]) << 16);
    *reinterpret_cast<u32x4*>(d) = o;
}

template <int WN, int MODE, bool F16, int OUT>
int launch_gemm_t(const GemmArgs& args, int max_rows, hipStream_t st) {
    constexpr int NB = 4;
    constexpr int BN = WN * 64;
    // upper bound of tiles: each expert adds at most one partial row unit
    const int64_t units = (static_cast<int64_t>(max_rows) + 2 * BM - 1) / (2 * BM) + args.E_loc;
    const int64_t tiles = units * (args.N / BN);
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess) {
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0) cus = v;
    }
    int64_t grid = static_cast<int64_t>(cus) * (4 / WN);   // one workgroup per CU at WN = 4
    if (tiles < grid) grid = tiles;
    if (grid < 1) grid = 1;
    hipLaunchKernelGGL((grouped_gemm_kernel<WN, MODE, F16, OUT, NB>), dim3(static_cast<unsigned>(grid)),
                       dim3(WN * 128), 0, st, args);
    MOE_CHECK_LAUNCH();
    return MOE_OK;
}

template <int MODE, bool F16, int OUT>
int launch_skinny(const GemmArgs& args, hipStream_t st) {
    const int64_t grid = static_cast<int64_t>(args.E_loc) * (args.N / 64);
    hipLaunchKernelGGL((grouped_gemm_skinny_kernel<MODE, F16, OUT, 4>), dim3(static_cast<unsigned>(grid)), dim3(256),
                       0, st, args);
    MOE_CHECK_LAUNCH();
    return MOE_OK;
}

template <int MODE, bool F16, int OUT>
int launch_nw(const GemmArgs& args, int max_rows, hipStream_t st) {
    if (args.skinny) return launch_skinny<MODE, F16, OUT>(args, st);
    if (args.N % 256 == 0) return launch_gemm_t<4, MODE, F16, OUT>(args, max_rows, st);
    if (args.N % 128 == 0) return launch_gemm_t<2, MODE, F16, OUT>(args, max_rows, st);
    return launch_gemm_t<1, MODE, F16, OUT>(args, max_rows, st);
}

template <int MODE, bool F16>
int launch_out(const GemmArgs& args, int max_rows, int c_dtype, hipStream_t st) {
    if (c_dtype == MOE_F32) return launch_nw<MODE, F16, kOutF32>(args, max_rows, st);
    if (c_dtype == MOE_BF16) return launch_nw<MODE, F16, kOutBF16>(args, max_rows, st);
    return launch_nw<MODE, F16, kOutF16>(args, max_rows, st);
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
    const dim3 g_gu((s.I + 255) / 256, s.H / 8, E_loc), g_dn((s.H + 255) / 256, s.I / 8, E_loc);
    if (dtype == MOE_BF16) {
        auto g = static_cast<const uint16_t*>(w_gate);
        auto u = static_cast<const uint16_t*>(w_up);
        auto d = static_cast<const uint16_t*>(w_down);
        hipLaunchKernelGGL((pack_weights_kernel<uint16_t, false>), g_gu, dim3(256), 0, st, g, s.H, s.I, 2 * s.I, 1, 0,
                           gu);
        hipLaunchKernelGGL((pack_weights_kernel<uint16_t, false>), g_gu, dim3(256), 0, st, u, s.H, s.I, 2 * s.I, 1, 1,
                           gu);
        hipLaunchKernelGGL((pack_weights_kernel<uint16_t, true>), g_dn, dim3(256), 0, st, d, s.I, s.H, s.H, 0, 0, dn);
    } else {
        auto g = static_cast<const float*>(w_gate);
        auto u = static_cast<const float*>(w_up);
        auto d = static_cast<const float*>(w_down);
        hipLaunchKernelGGL((pack_weights_kernel<float, true>), g_gu, dim3(256), 0, st, g, s.H, s.I, 2 * s.I, 1, 0, gu);
        hipLaunchKernelGGL((pack_weights_kernel<float, true>), g_gu, dim3(256), 0, st, u, s.H, s.I, 2 * s.I, 1, 1, gu);
        hipLaunchKernelGGL((pack_weights_kernel<float, true>), g_dn, dim3(256), 0, st, d, s.I, s.H, s.H, 0, 0, dn);
    }
    MOE_CHECK_LAUNCH();
    return MOE_OK;
}

bool gemm_streams_weights(const moe_shape& s, int which, bool gather) {
    // routed evenly, an expert receives T*K/E rows; at most 64 expected -> the
    // weight-streaming kernel (it stays correct for any row count), provided its
    // byte offsets into the activation matrix fit its buffer range
    const int E_loc = s.e_end - s.e_begin;
    const int64_t max_rows = static_cast<int64_t>(s.T) * (s.K < E_loc ? s.K : E_loc);
    const int64_t a_rows_max = gather ? s.T : max_rows;
    const int64_t a_bytes = a_rows_max * (which == MOE_GEMM_GATE_UP ? s.H : s.I) * 2;
    return static_cast<int64_t>(s.T) * s.K <= static_cast<int64_t>(64) * s.E && a_bytes <= kBufferRange;
}

bool gemm_can_derive_dispatch(const moe_shape& s) {
    return gemm_streams_weights(s, MOE_GEMM_GATE_UP, true) && s.T <= kDeriveMaxT && s.e_end - s.e_begin <= kDeriveMaxE;
}

int launch_gate_up_deriving_dispatch(const moe_shape& s, const uint16_t* x, const int32_t* topk_idx,
                                     const uint16_t* packed, uint16_t* h, int32_t* counts, int32_t* offsets,
                                     int32_t* row_token, int32_t* row_slot, int32_t* slot_row, hipStream_t st) {
    GemmArgs args{};
    args.a = x;
    args.b = packed;
    args.c = h;
    args.E_loc = s.e_end - s.e_begin;
    args.I = s.I;
    args.N = 2 * s.I;
    args.Kd = s.H;
    args.ldc = s.I;
    args.skinny = 1;
    args.topk_idx = topk_idx;
    args.e_begin = s.e_begin;
    args.T = s.T;
    args.K = s.K;
    args.d_counts = counts;
    args.d_offsets = offsets;
    args.d_row_token = row_token;
    args.d_row_slot = row_slot;
    args.d_slot_row = slot_row;
    return launch_skinny<kSwiGLU, false, kOutF16>(args, st);
}

int launch_grouped_gemm(const moe_shape& s, const uint16_t* a, int a_dtype, const int32_t* a_rows,
                        const int32_t* offsets, const uint16_t* packed, int which, int epilogue, void* c, int c_dtype,
                        hipStream_t st) {
    const int E_loc = s.e_end - s.e_begin;
    const int max_rows = s.T * (s.K < E_loc ? s.K : E_loc);
    GemmArgs args{};
    args.a = a;
    args.a_rows = a_rows;
    args.offsets = offsets;
    args.c = c;
    args.E_loc = E_loc;
    args.I = s.I;
    // routed evenly, an expert receives T*K/E rows; at most 64 expected -> the
    // weight-streaming kernel (it stays correct for any row count), provided its
    // byte offsets into the activation matrix fit its buffer range
    args.skinny = gemm_streams_weights(s, which, a_rows != nullptr);
    if (which == MOE_GEMM_GATE_UP) {
        args.b = packed;
        args.N = 2 * s.I;
        args.Kd = s.H;
        args.ldc = epilogue == MOE_EPI_SWIGLU ? s.I : 2 * s.I;
        const bool f16 = a_dtype == MOE_F16;
        if (epilogue == MOE_EPI_SWIGLU)
            return f16 ? launch_out<kSwiGLU, true>(args, max_rows, c_dtype, st)
                       : launch_out<kSwiGLU, false>(args, max_rows, c_dtype, st);
        return f16 ? launch_out<kGateUpPlain, true>(args, max_rows, c_dtype, st)
                   : launch_out<kGateUpPlain, false>(args, max_rows, c_dtype, st);
    }
    args.b = packed + packed_gate_up_elems(s);
    args.N = s.H;
    args.Kd = s.I;
    args.ldc = s.H;
    return launch_out<kPlain, true>(args, max_rows, c_dtype, st);
}

}  // namespace moe
