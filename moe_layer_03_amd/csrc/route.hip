// Router: logits in the library's fixed float32 order, top-K selection and
// renormalised softmax weights.
//
// "Hosting Qwen on Blackwell" (Perplexity), section "Pre-remplisseurs": each
// token is routed to 8 of the 128 experts; the router function itself is not
// on the pages.  This library reads it as softmax over the experts, the K
// most probable kept, their probabilities renormalised.
//
// Every logit is one fused multiply-add chain over h in ascending order -- the
// order that decides near-ties -- so the logits come out identical to a
// sequential fmaf loop; that makes the router VALU work (T*E*H fma).
// For E <= 128 a lane owns (token, expert) chains; activations and router
// weights are staged per workgroup in LDS as float32 (double-buffered, global
// loads running several chunks ahead through registers), so the vector unit
// issues little besides v_fma.  Large bf16 batches with scratch screen the
// experts with MFMA estimates and run the chains of the candidates only; other
// large batches give each wave 3 tokens x all experts; small batches with
// scratch give each workgroup's chain wave a tile of 8 tokens x 8 experts, fed
// by a copy wave beside it (the chain length sets their time), without
// scratch each wave 1 token x 64 experts.  Larger E uses the generic kernel.
// Selection happens in registers over (orderable logit, ~expert) keys: the
// largest key of a wave or a 16-lane row by DPP row shifts, ties by ballot.
#include "common.hpp"
#include "route_prefetch.hpp"

#include <type_traits>
#include <utility>

namespace moe {
namespace {

constexpr int kRouteThreads = 256;
constexpr int kRouteWaves = kRouteThreads / kWave;
constexpr int kLdsFloatsW = 8192;   // 32 KiB of float32 router-weight staging
constexpr int kChainMaxT = 1024;     // batches up to this size use one workgroup per token

template <typename T> struct Widen;
template <> struct Widen<uint16_t> {
    static __device__ __forceinline__ float f(uint16_t v) { return bf16_to_f32(v); }
};
template <> struct Widen<float> {
    static __device__ __forceinline__ float f(float v) { return v; }
};

// Orderable 64-bit key: larger logit first, then smaller expert index.
// -0 is folded to +0 so that the two compare equal.
__device__ __forceinline__ uint64_t make_key(float v, int e) {
    uint32_t b = __float_as_uint(v);
    if (v == 0.0f) b = 0u;
    uint32_t ok = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
    return (static_cast<uint64_t>(ok) << 32) | static_cast<uint32_t>(~static_cast<uint32_t>(e));
}

__device__ __forceinline__ float key_logit(uint64_t k) {
    uint32_t ok = static_cast<uint32_t>(k >> 32);
    uint32_t b = (ok & 0x80000000u) ? (ok & 0x7FFFFFFFu) : ~ok;
    return __uint_as_float(b);
}

__device__ __forceinline__ int key_expert(uint64_t k) {
    return static_cast<int>(~static_cast<uint32_t>(k));
}

// Largest value over the wave: a running maximum within each row of 16 lanes
// by DPP row shifts (lanes shifted in from outside the row see 0, neutral for
// an unsigned maximum), then the four row maxima read out to scalars.  No LDS
// round trips.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x111, 0xf, 0xf, false)));
    v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x112, 0xf, 0xf, false)));
    v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x114, 0xf, 0xf, false)));
    v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x118, 0xf, 0xf, false)));
    const uint32_t r0 = __builtin_amdgcn_readlane(v, 15), r1 = __builtin_amdgcn_readlane(v, 31);
    const uint32_t r2 = __builtin_amdgcn_readlane(v, 47), r3 = __builtin_amdgcn_readlane(v, 63);
    return max(max(r0, r1), max(r2, r3));
}

// Select the top K of the wave's E logits (lane holds experts g*64 + lane) and
// write indices and renormalised weights of token t.  Uniform control flow.
// The order is that of make_key: larger logit first, then the smaller expert
// index.  Each round takes the largest upper key half (the ordered logit bits)
// over the experts still in play, then the lowest expert index holding it from
// a ballot.  A retired expert's key half becomes 0, below every finite logit;
// only a logit whose bits are all ones (a NaN) also maps to 0, so liveness is
// consulted when the round's maximum is 0.  The weights are exp(l - l_max)
// over their sum, added in rank order.
template <int NE>
__device__ __forceinline__ void select_and_write(const float (&l)[NE], int E, int K, int t,
                                                 int32_t* __restrict__ topk_idx, float* __restrict__ topk_w) {
    const int lane = threadIdx.x & (kWave - 1);
    uint32_t kv[NE];
    uint32_t dead = 0u;                              // bit g: expert g * 64 + lane is out of play
#pragma unroll
    for (int g = 0; g < NE; ++g) {
        const bool in = g * kWave + lane < E;
        kv[g] = in ? static_cast<uint32_t>(make_key(l[g], 0) >> 32) : 0u;
        dead |= in ? 0u : (1u << g);
    }
    int my_e = 0;
    uint32_t my_m = 0u;
    for (int k = 0; k < K; ++k) {
        uint32_t m = kv[0];
#pragma unroll
        for (int g = 1; g < NE; ++g) m = max(m, kv[g]);
        m = wave_max_u32(m);
        int best = -1;
#pragma unroll
        for (int g = 0; g < NE; ++g) {
            const uint64_t b = __ballot(kv[g] == m && (m != 0u || ((dead >> g) & 1u) == 0u));
            if (best < 0 && b != 0ull) best = g * kWave + __builtin_ctzll(b);
        }
#pragma unroll
        for (int g = 0; g < NE; ++g)
            if (g * kWave + lane == best) {
                kv[g] = 0u;
                dead |= 1u << g;
            }
        if (lane == k) {
            my_e = best;
            my_m = m;
        }
    }
    const float my_l = key_logit(static_cast<uint64_t>(my_m) << 32);
    const float l0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, my_l), 0));
    const float ex = lane < K ? expf(my_l - l0) : 0.0f;
    float sum = 0.0f;
    for (int k = 0; k < K; ++k) sum += __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, ex), k));
    if (lane < K) {
        topk_idx[static_cast<int64_t>(t) * K + lane] = my_e;
        topk_w[static_cast<int64_t>(t) * K + lane] = ex / sum;
    }
}

template <typename XT, int R, int NE>
__global__ __launch_bounds__(kRouteThreads) void route_kernel(
    const XT* __restrict__ x, const XT* __restrict__ w, const float* __restrict__ bias,
    int T, int H, int E, int K, int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
    float* __restrict__ logits) {
    constexpr int EW = NE * kWave;                          // experts covered by one wave
    constexpr int HC = (kLdsFloatsW / EW) < 64 ? (kLdsFloatsW / EW) : 64;   // h per chunk
    __shared__ float s_w[HC][EW];
    __shared__ float s_x[kRouteWaves][R][HC];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid >> 6;
    const int t0 = (blockIdx.x * kRouteWaves + wave) * R;   // first token of this wave

    float acc[R][NE];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int g = 0; g < NE; ++g) acc[r][g] = 0.0f;

    for (int h0 = 0; h0 < H; h0 += HC) {
        // stage router weights [HC][EW] (zero beyond E) as float32
        for (int i = tid; i < HC * EW; i += kRouteThreads) {
            const int hh = i / EW, e = i % EW;
            s_w[hh][e] = e < E ? Widen<XT>::f(w[static_cast<int64_t>(h0 + hh) * E + e]) : 0.0f;
        }
        // stage this wave's activations [R][HC]
        for (int i = lane; i < R * HC; i += kWave) {
            const int r = i / HC, hh = i % HC;
            const int t = t0 + r;
            s_x[wave][r][hh] = t < T ? Widen<XT>::f(x[static_cast<int64_t>(t) * H + h0 + hh]) : 0.0f;
        }
        __syncthreads();
#pragma unroll 8
        for (int hh = 0; hh < HC; ++hh) {
            float wv[NE];
#pragma unroll
            for (int g = 0; g < NE; ++g) wv[g] = s_w[hh][g * kWave + lane];
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const float xv = s_x[wave][r][hh];
#pragma unroll
                for (int g = 0; g < NE; ++g) acc[r][g] = fmaf(xv, wv[g], acc[r][g]);
            }
        }
        __syncthreads();
    }

#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int t = t0 + r;
        if (t >= T) break;   // uniform across the wave
        float l[NE];
#pragma unroll
        for (int g = 0; g < NE; ++g) {
            const int e = g * kWave + lane;
            float v = acc[r][g];
            if (bias != nullptr && e < E) v = v + bias[e];
            l[g] = v;
            if (logits != nullptr && e < E) logits[static_cast<int64_t>(t) * E + e] = v;
        }
        select_and_write<NE>(l, E, K, t, topk_idx, topk_w);
    }
}

// ---------------------------------------------------------------------------
// E <= 128 fast path.
// A workgroup of WAVES waves owns TOK = (WAVES / SPLIT) * R tokens and all
// experts.  Wave w runs R tokens against NE groups of 64 experts starting at
// group (w % SPLIT) * NE; SPLIT = 2 lets two waves share a token (shorter
// chains per lane for small batches).  Per HC-row chunk the workgroup stages
// the router-weight rows (one contiguous run of HC*E elements) and the TOK
// activation rows as float32 in LDS (double-buffered); global loads run P-1
// chunks ahead through a register ring so their latency is covered.
// ---------------------------------------------------------------------------
template <typename XT, int R, int NE, int SPLIT, int WAVES, int HC, int P>
__global__ __launch_bounds__(WAVES * 64) void route_fast_kernel(
    const XT* __restrict__ x, const XT* __restrict__ w, const float* __restrict__ bias,
    int T, int H, int E, int K, int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
    float* __restrict__ logits) {
    constexpr int NT = WAVES * 64;                 // threads
    constexpr int TOK = (WAVES / SPLIT) * R;       // tokens per workgroup
    constexpr int VEC = 16 / sizeof(XT);           // elements per 16-byte piece
    constexpr int WP_MAX = HC * 128 / VEC;         // router-weight pieces per chunk (E <= 128)
    constexpr int XP = TOK * HC / VEC;             // activation pieces per chunk
    constexpr int NPT = (WP_MAX + XP + NT - 1) / NT;   // pieces per thread per chunk
    static_assert(HC % VEC == 0, "chunk rows must split into 16-byte pieces");

    __shared__ __attribute__((aligned(16))) float s_w[2][HC * 128];
    __shared__ __attribute__((aligned(16))) float s_x[2][TOK][HC];
    __shared__ float s_l[SPLIT > 1 ? TOK : 1][128];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int tok0 = blockIdx.x * TOK;
    const int wtok = (wave / SPLIT) * R;           // first token of this wave (within the workgroup)
    const int g0 = (wave % SPLIT) * NE;            // first expert group of this wave
    const int WP = HC * E / VEC;                   // pieces of this E

    // piece p < WP: router weight run; WP <= p < WP + XP: activation (token, 16-byte column);
    // higher pieces reload piece 0.  Every thread issues the same loads with no
    // branches, so the wait counters stay exact and the ring keeps P-1 chunks
    // in flight.
    auto load = [&](u32x4 (&r)[NPT], int c) {
#pragma unroll
        for (int i = 0; i < NPT; ++i) {
            const int p = tid + i * NT;
            const int q = p - WP;
            const int tt = q / (HC / VEC), col = q % (HC / VEC);
            const int t = min(tok0 + tt, T - 1);
            const XT* src = (p < WP) ? w + static_cast<int64_t>(c) * HC * E + p * VEC
                          : (p < WP + XP) ? x + static_cast<int64_t>(t) * H + c * HC + col * VEC
                          : w;
            r[i] = *reinterpret_cast<const u32x4*>(src);
        }
    };
    auto store = [&](const u32x4 (&r)[NPT], int buf) {
#pragma unroll
        for (int i = 0; i < NPT; ++i) {
            const int p = tid + i * NT;
            float* dst;
            if (p < WP) {
                dst = &s_w[buf][p * VEC];
            } else if (p < WP + XP) {
                const int q = p - WP;
                dst = &s_x[buf][q / (HC / VEC)][(q % (HC / VEC)) * VEC];
            } else {
                continue;
            }
            if constexpr (sizeof(XT) == 2) {
                floatx4 a, b;
                a[0] = __uint_as_float(r[i][0] << 16); a[1] = __uint_as_float(r[i][0] & 0xFFFF0000u);
                a[2] = __uint_as_float(r[i][1] << 16); a[3] = __uint_as_float(r[i][1] & 0xFFFF0000u);
                b[0] = __uint_as_float(r[i][2] << 16); b[1] = __uint_as_float(r[i][2] & 0xFFFF0000u);
                b[2] = __uint_as_float(r[i][3] << 16); b[3] = __uint_as_float(r[i][3] & 0xFFFF0000u);
                *reinterpret_cast<floatx4*>(dst) = a;
                *reinterpret_cast<floatx4*>(dst + 4) = b;
            } else {
                *reinterpret_cast<u32x4*>(dst) = r[i];
            }
        }
    };

    float acc[R][NE];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int g = 0; g < NE; ++g) acc[r][g] = 0.0f;

    const int nc = H / HC;
    u32x4 ring[P][NPT];
    // prologue: chunks 0 .. P-1 in flight, chunk 0 in LDS, slot 0 refilled with chunk P
    // (chunk indices past the end are clamped: harmless reloads)
#pragma unroll
    for (int q = 0; q < P; ++q) load(ring[q], min(q, nc - 1));
    store(ring[0], 0);
    load(ring[0], min(P, nc - 1));
    __syncthreads();

    for (int c0 = 0; c0 < nc; c0 += P) {
#pragma unroll
        for (int q = 0; q < P; ++q) {
            const int c = c0 + q;
            if (c >= nc) break;                     // uniform
            const int buf = c & 1;
            // slot (q+1) % P holds chunk c+1: it goes to the other LDS buffer (the
            // last chunk writes an unused copy) and the slot is refilled with c+1+P
            const int nq = (q + 1) % P;
            store(ring[nq], buf ^ 1);
            load(ring[nq], min(c + 1 + P, nc - 1));
            const float* sw = s_w[buf];
#pragma unroll
            for (int h4 = 0; h4 < HC; h4 += 4) {
                floatx4 xv[R];
#pragma unroll
                for (int r = 0; r < R; ++r) xv[r] = *reinterpret_cast<const floatx4*>(&s_x[buf][wtok + r][h4]);
#pragma unroll
                for (int hh = 0; hh < 4; ++hh) {
                    float wv[NE];
#pragma unroll
                    for (int g = 0; g < NE; ++g) wv[g] = sw[(h4 + hh) * E + (g0 + g) * kWave + lane];
#pragma unroll
                    for (int r = 0; r < R; ++r)
#pragma unroll
                        for (int g = 0; g < NE; ++g) acc[r][g] = fmaf(xv[r][hh], wv[g], acc[r][g]);
                }
            }
            __syncthreads();
        }
    }

    if constexpr (SPLIT == 1) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int t = tok0 + wtok + r;
            if (t >= T) break;   // uniform across the wave
            float l[NE];
#pragma unroll
            for (int g = 0; g < NE; ++g) {
                const int e = g * kWave + lane;
                float v = acc[r][g];
                if (bias != nullptr && e < E) v = v + bias[e];
                l[g] = v;
                if (logits != nullptr && e < E) logits[static_cast<int64_t>(t) * E + e] = v;
            }
            select_and_write<NE>(l, E, K, t, topk_idx, topk_w);
        }
    } else {
        static_assert(SPLIT * NE == 2, "split path covers 128 experts");
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int t = tok0 + wtok + r;
#pragma unroll
            for (int g = 0; g < NE; ++g) {
                const int e = (g0 + g) * kWave + lane;
                float v = acc[r][g];
                if (bias != nullptr && e < E) v = v + bias[e];
                if (logits != nullptr && e < E && t < T) logits[static_cast<int64_t>(t) * E + e] = v;
                s_l[wtok + r][e] = v;
            }
        }
        __syncthreads();
        if (g0 == 0) {
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const int t = tok0 + wtok + r;
                if (t >= T) break;
                float l[2] = {s_l[wtok + r][lane], s_l[wtok + r][kWave + lane]};
                select_and_write<2>(l, E, K, t, topk_idx, topk_w);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Small batches without scratch for the logits, E <= 128: one chain per lane,
// one workgroup per TPW tokens, so that a batch of a hundred tokens still
// spreads over a hundred CUs.  (With scratch, or logits requested, the tiled
// kernel below streams far less and is used instead.)
//
// A workgroup has CW = TPW * WE chain waves (token ti, experts g*64 + lane)
// and DW copy waves.  The copy waves stream the router weight through an
// NB-deep ring of HC-row chunks straight into LDS (16-byte DMA; rows padded to
// EP = 64 * WE elements).  The token rows are widened to float32 in LDS once.
// A chain wave keeps four register slots of operands (8 rows each): while it
// runs the 8 dependent fmas of one group it reads the group two ahead, the
// compiler placing the waits and a scheduling pattern interleaving the reads
// with the fmas.  A bf16 weight widens exactly to float32 by a 16-bit shift.
// ---------------------------------------------------------------------------
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F& f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Operands of one group of 8 rows: the token row's 8 values (two 16-byte
// reads) and the chain's 8 weights (one column of the staged rows).  A bf16
// weight widens exactly to float32 by a 16-bit shift.
template <typename XT>
__device__ __forceinline__ void chain_fetch(floatx4& x0, floatx4& x1, float (&w)[8], const float* __restrict__ sx,
                                            const XT* __restrict__ sw, int rb) {
    x0 = *reinterpret_cast<const floatx4*>(sx);
    x1 = *reinterpret_cast<const floatx4*>(sx + 4);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        if constexpr (sizeof(XT) == 2)
            w[j] = __uint_as_float(static_cast<uint32_t>(sw[j * rb]) << 16);
        else
            w[j] = sw[j * rb];
    }
}

// The group's 8 dependent steps, rows in ascending order.
__device__ __forceinline__ void chain_steps(float& acc, const floatx4& x0, const floatx4& x1, const float (&w)[8]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) acc = __builtin_fmaf(x0[j], w[j], acc);
#pragma unroll
    for (int j = 0; j < 4; ++j) acc = __builtin_fmaf(x1[j], w[4 + j], acc);
}

// Reads units [b*n/B, (b+1)*n/B) of a region of n 1 KiB units (workgroup b of
// B) into a scratch KiB of LDS per wave, up to 32 copies in flight per wave,
// and discards them: the bytes pass through the last-level cache, where a
// kernel launched next finds them.  Every address stays inside the region
// (the last group repeats the last unit); all copies land before return.
constexpr int kCacheGroup = 16;   // copies issued per wave between waits
__device__ void cache_region(const uint16_t* __restrict__ region, int64_t units, int b, int B,
                             void* lds_scratch) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x >> 6;
    const int nw = blockDim.x >> 6;
    const int64_t u0 = units * b / B, u1 = units * (b + 1) / B;
    uint16_t* dst = static_cast<uint16_t*>(lds_scratch) + wave * 512;
    int64_t u = u0 + wave;
    const int64_t step = static_cast<int64_t>(nw) * kCacheGroup;
    bool first = true;
    for (; u < u1; u += step) {
#pragma unroll
        for (int j = 0; j < kCacheGroup; ++j) {
            const int64_t v = min(u + static_cast<int64_t>(j) * nw, u1 - 1);
            dma16(region + v * 512 + lane * 8, dst);
        }
        if (!first) wait_vmcnt<kCacheGroup>();   // the previous group has landed
        first = false;
    }
    wait_vmcnt<0>();
}

template <typename XT, int TPW, int WE, int DW, int HC, int NB, int XMAX>
__global__ __launch_bounds__((TPW * WE + DW) * 64) void route_chain_kernel(
    const XT* __restrict__ x, const XT* __restrict__ w, const float* __restrict__ bias,
    int T, int H, int E, int K, int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
    float* __restrict__ logits, int nroute, const uint16_t* __restrict__ pf, int64_t pf_units) {
    constexpr bool BF16 = sizeof(XT) == 2;
    constexpr int CW = TPW * WE;                              // chain waves
    constexpr int CT = CW * 64;                               // chain threads
    constexpr int DT = DW * 64;                               // copy threads
    constexpr int VEC = 16 / sizeof(XT);                      // elements per 16-byte piece
    constexpr int EP = WE * 64;                               // staged row stride (E padded)
    constexpr int RB = EP * static_cast<int>(sizeof(XT));     // bytes per staged row
    constexpr int RP = EP / VEC;                              // pieces per staged row
    constexpr int NPC = HC * RP / DT;                         // pieces per copy thread and chunk
    constexpr int NXP = TPW * XMAX / VEC / CT;                // token-row pieces per chain thread
    constexpr int GPC = HC / 8;                               // row groups per chunk
    static_assert(HC * RP % DT == 0 && NPC >= 1, "chunk staging");
    static_assert(NXP >= 1 && TPW * XMAX % (VEC * CT) == 0, "token staging");
    static_assert(NB >= 3 && (NB - 2) * NPC < 64, "one chunk of look-ahead; vmcnt range");
    static_assert(GPC % 4 == 0 && HC * RB < 65536, "register slots; LDS offsets");
    __shared__ __attribute__((aligned(16))) XT s_w[NB][HC * EP];
    __shared__ __attribute__((aligned(16))) float s_x[TPW][XMAX];
    __shared__ float s_l[WE > 1 ? TPW : 1][WE > 1 ? 128 : 1];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    if (static_cast<int>(blockIdx.x) >= nroute) {
        // workgroups past the routing ones read a region the next kernel streams
        // (the expert weights) so that it is in the last-level cache by then
        cache_region(pf, pf_units, blockIdx.x - nroute, gridDim.x - nroute, &s_w[0][0]);
        return;
    }
    const int tok0 = blockIdx.x * TPW;
    const int nc = H / HC;
    float acc = 0.0f;

    if (wave >= CW) {
        // ---- copy waves: chunk c lands in stage c % NB; chunk indices past the
        // end are clamped (harmless reloads into stages already consumed), so
        // every copy wave issues the same copies and the vmcnt waits stay exact
        const int dt = tid - CT;
        const int rp = E / VEC;                // pieces per row of this E
        int src_off[NPC];                      // pieces past a row's end copy its last piece into the padding
#pragma unroll
        for (int i = 0; i < NPC; ++i) {
            const int p = i * DT + dt;
            src_off[i] = (p / RP) * E + min(p % RP, rp - 1) * VEC;
        }
        auto issue = [&](int c, int stage) {
            const XT* src = w + static_cast<int64_t>(c) * HC * E;
#pragma unroll
            for (int i = 0; i < NPC; ++i)
                dma16(reinterpret_cast<const uint16_t*>(src + src_off[i]),
                      reinterpret_cast<uint16_t*>(&s_w[stage][(i * DT + (wave - CW) * kWave) * VEC]));
        };
#pragma unroll
        for (int q = 0; q < NB - 1; ++q) issue(min(q, nc - 1), q);
        wait_vmcnt<(NB - 2) * NPC>();          // chunk 0 has landed
        __builtin_amdgcn_s_barrier();
        for (int c = 0; c < nc; ++c) {
            wait_vmcnt<(NB - 3) * NPC>();      // chunk c+1 has landed
            __builtin_amdgcn_s_barrier();      // ... and every chain wave is done with stage c-1
            issue(min(c + NB - 1, nc - 1), (c + NB - 1) % NB);
        }
        wait_vmcnt<0>();                       // no copy may land after the workgroup's LDS is released
    } else {
        // ---- chain waves
        const int ti = wave / WE;
        const int ec = min((wave % WE) * kWave + lane, E - 1);   // lanes past E repeat the last column, unused
        // token rows -> float32 (rows past T are zero; columns past H land in unused staging)
        constexpr int XP = XMAX / VEC;
        u32x4 xr[NXP];
#pragma unroll
        for (int j = 0; j < NXP; ++j) {
            const int i = j * CT + tid;
            const int t = min(tok0 + i / XP, T - 1);
            const int col = min((i % XP) * VEC, H - VEC);
            xr[j] = *reinterpret_cast<const u32x4*>(x + static_cast<int64_t>(t) * H + col);
        }
#pragma unroll
        for (int j = 0; j < NXP; ++j) {
            const int i = j * CT + tid;
            const bool live = tok0 + i / XP < T;
            float* dst = &s_x[i / XP][(i % XP) * VEC];
            if constexpr (BF16) {
                floatx4 a, b;
                a[0] = __uint_as_float(xr[j][0] << 16); a[1] = __uint_as_float(xr[j][0] & 0xFFFF0000u);
                a[2] = __uint_as_float(xr[j][1] << 16); a[3] = __uint_as_float(xr[j][1] & 0xFFFF0000u);
                b[0] = __uint_as_float(xr[j][2] << 16); b[1] = __uint_as_float(xr[j][2] & 0xFFFF0000u);
                b[2] = __uint_as_float(xr[j][3] << 16); b[3] = __uint_as_float(xr[j][3] & 0xFFFF0000u);
                if (!live) a = b = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
                *reinterpret_cast<floatx4*>(dst) = a;
                *reinterpret_cast<floatx4*>(dst + 4) = b;
            } else {
                floatx4 a = __builtin_bit_cast(floatx4, xr[j]);
                if (!live) a = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
                *reinterpret_cast<floatx4*>(dst) = a;
            }
        }
        wait_lgkmcnt0();                       // the staged rows are written before the barrier

        // Four register slots: group Q computes from slot Q % 4 while the reads of
        // group Q + 2 fill slot (Q + 2) % 4; the compiler places the waits for
        // them, and a scheduling pattern interleaves the reads with the
        // dependent fmas (each fma leaves an issue slot that a read can fill).
        floatx4 xv[4][2];
        float wv[4][8];
        const float* sx0 = s_x[ti];
        const XT* sw0 = &s_w[0][ec];

        __builtin_amdgcn_s_barrier();          // chunk 0 and the token rows are in LDS
        chain_fetch<XT>(xv[0][0], xv[0][1], wv[0], sx0, sw0, EP);
        chain_fetch<XT>(xv[1][0], xv[1][1], wv[1], sx0 + 8, sw0 + 8 * EP, EP);
        for (int c = 0; c < nc; ++c) {
            __builtin_amdgcn_s_barrier();      // chunk c+1 is in LDS; stage c-1 may be refilled
            const float* sxc = sx0 + c * HC;
            const float* sxn = sx0 + min(c + 1, nc - 1) * HC;
            const XT* swc = sw0 + (c % NB) * (HC * EP);
            const XT* swn = sw0 + ((c + 1) % NB) * (HC * EP);
            static_for<GPC>([&](auto qc) {
                constexpr int Q = decltype(qc)::value;
                constexpr int S = Q % 4, NS = (Q + 2) % 4, QN = (Q + 2) % GPC;
                constexpr bool NEXT = Q + 2 >= GPC;
                chain_fetch<XT>(xv[NS][0], xv[NS][1], wv[NS], (NEXT ? sxn : sxc) + QN * 8,
                                (NEXT ? swn : swc) + QN * 8 * EP, EP);
                chain_steps(acc, xv[S][0], xv[S][1], wv[S]);
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);       // the two token-row reads
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    __builtin_amdgcn_sched_group_barrier(0x002, 1, 0);   // one fma (or widening) ...
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // ... one weight read
                }
            });
        }
    }

    if (wave < CW) {
        const int ti = wave / WE;
        const int e = (wave % WE) * kWave + lane;
        const int t = tok0 + ti;
        float v = acc;
        if (bias != nullptr && e < E) v = v + bias[e];
        if (logits != nullptr && e < E && t < T) logits[static_cast<int64_t>(t) * E + e] = v;
        if constexpr (WE == 1) {
            if (t < T) {
                float l[1] = {v};
                select_and_write<1>(l, E, K, t, topk_idx, topk_w);
            }
        } else {
            s_l[ti][e] = v;
        }
    }
    if constexpr (WE > 1) {
        static_assert(WE == 2, "E <= 128");
        __syncthreads();
        if (wave < CW && wave % WE == 0) {
            const int ti = wave / WE;
            const int t = tok0 + ti;
            if (t < T) {
                float l[2] = {s_l[ti][lane], s_l[ti][kWave + lane]};
                select_and_write<2>(l, E, K, t, topk_idx, topk_w);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Small batches with somewhere to put the logits.  A workgroup owns TT tokens
// and CH * TE experts: CH chain waves, each a TT x TE tile with one chain per
// lane (token lane / TE, expert lane % TE), and one copy wave.  The copy wave
// streams the TT token rows and the CH * TE weight columns through a ring of
// three LDS buffers of HC rows, widened to float32: token rows [TT][HC] and
// the weight columns transposed to [CH * TE][HC], rows padded by 4 floats.
// Its global loads run one chunk ahead in registers, and it fills chunk c + 2
// while the chains run over chunk c, so one barrier per chunk orders both.
// A chain step reads 4 h of its token and of its expert with two 16-byte
// reads (each row is read by TE or TT lanes at once) and runs 4 dependent
// fmas.  On one wave those reads and fmas serialise: the wave waits while an
// LDS read returns its 1 KiB, so the copies and the widening are kept out of
// the chain waves.  A selection pass over the written logits picks the top K.
// Workgroups past the tiles warm the last-level cache like the chain kernel's.
// ---------------------------------------------------------------------------
template <typename XT, int TT, int TE, int CH, int HC>
__global__ __launch_bounds__((CH + 1) * 64) void route_tile_kernel(
    const XT* __restrict__ x, const XT* __restrict__ w, const float* __restrict__ bias, int T, int H, int E,
    float* __restrict__ logits, int ntile, const uint16_t* __restrict__ pf, int64_t pf_units) {
    constexpr int NB = 3;                            // LDS ring: chains read c, copies fill c + 2
    constexpr int VEC = 16 / static_cast<int>(sizeof(XT));
    constexpr int HP = HC + 4;                       // padded LDS row (floats)
    constexpr int EW = CH * TE;                      // weight columns per workgroup
    constexpr int XPR = HC / VEC;                    // 16-byte pieces per token row of a chunk
    constexpr int WPR = EW / VEC;                    // 16-byte pieces per weight row (one h) of the workgroup
    constexpr int XL = TT * XPR / kWave;             // token pieces per copy lane and chunk
    constexpr int WG = HC / 4 * WPR / kWave;         // (4 rows, piece) groups per copy lane and chunk
    static_assert(TT * TE == kWave, "one chain per lane");
    static_assert(XL >= 1 && TT * XPR % kWave == 0 && WG >= 1 && HC / 4 * WPR % kWave == 0, "chunk split");
    static_assert(EW % VEC == 0 && HC % 4 == 0, "pieces");
    __shared__ __attribute__((aligned(16))) float s_x[NB][TT][HP];
    __shared__ __attribute__((aligned(16))) float s_w[NB][EW][HP];
    if (static_cast<int>(blockIdx.x) >= ntile) {
        cache_region(pf, pf_units, blockIdx.x - ntile, gridDim.x - ntile, &s_x[0][0][0]);
        return;
    }
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int net = (E + EW - 1) / EW;
    const int tok0 = (static_cast<int>(blockIdx.x) / net) * TT;
    const int e0 = (static_cast<int>(blockIdx.x) % net) * EW;
    const int nc = H / HC;

    if (wave == CH) {
        // ---- copy wave: chunk c sits in register slot c & 1 from one chunk before it is stored
        u32x4 xr[2][XL], wr[2][WG][4];
        // token rows past T repeat row T-1; weight pieces past E repeat the last piece (both unused)
        auto load = [&](int c, auto qc) {
            constexpr int q = decltype(qc)::value;
            const int h0 = c * HC;
#pragma unroll
            for (int j = 0; j < XL; ++j) {
                const int i = j * kWave + lane;
                const int t = min(tok0 + i / XPR, T - 1);
                xr[q][j] = *reinterpret_cast<const u32x4*>(x + static_cast<int64_t>(t) * H + h0 + (i % XPR) * VEC);
            }
#pragma unroll
            for (int j = 0; j < WG; ++j) {
                const int g = j * kWave + lane;          // rows 4 (g / WPR) .. +3, piece g % WPR
                const int ec = min(e0 + (g % WPR) * VEC, E - VEC);
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    wr[q][j][r] = *reinterpret_cast<const u32x4*>(
                        w + static_cast<int64_t>(h0 + 4 * (g / WPR) + r) * E + ec);
            }
        };
        auto widen = [](const u32x4& r, int v) -> float {
            if constexpr (sizeof(XT) == 2) {
                const uint32_t u = r[v >> 1];
                return __uint_as_float((v & 1) ? (u & 0xFFFF0000u) : (u << 16));
            } else {
                return __uint_as_float(r[v]);
            }
        };
        auto store = [&](int b, auto qc) {
            constexpr int q = decltype(qc)::value;
#pragma unroll
            for (int j = 0; j < XL; ++j) {
                const int i = j * kWave + lane;
                float* dst = &s_x[b][i / XPR][(i % XPR) * VEC];
#pragma unroll
                for (int v = 0; v < VEC; v += 4)
                    *reinterpret_cast<floatx4*>(dst + v) = floatx4{widen(xr[q][j], v), widen(xr[q][j], v + 1),
                                                                   widen(xr[q][j], v + 2), widen(xr[q][j], v + 3)};
            }
#pragma unroll
            for (int j = 0; j < WG; ++j) {
                const int g = j * kWave + lane;
                const int hr = 4 * (g / WPR), col = (g % WPR) * VEC;
#pragma unroll
                for (int v = 0; v < VEC; ++v)
                    *reinterpret_cast<floatx4*>(&s_w[b][col + v][hr]) =
                        floatx4{widen(wr[q][j][0], v), widen(wr[q][j][1], v), widen(wr[q][j][2], v),
                                widen(wr[q][j][3], v)};
            }
        };
        load(0, std::integral_constant<int, 0>());
        if (nc > 1) load(1, std::integral_constant<int, 1>());
        store(0, std::integral_constant<int, 0>());
        if (nc > 1) store(1, std::integral_constant<int, 1>());
        if (nc > 2) load(2, std::integral_constant<int, 0>());
        __syncthreads();                             // chunks 0 and 1 are in LDS
        // chunk c: store chunk c + 2 into the buffer chunk c - 1 used, load chunk c + 3 into the
        // register slot chunk c + 1 left
        for (int c0 = 0; c0 < nc; c0 += 2) {
            static_for<2>([&](auto qc) {
                constexpr int q = decltype(qc)::value;
                const int c = c0 + q;
                if (c < nc) {
                    if (c + 2 < nc) store((c + 2) % NB, std::integral_constant<int, q>());
                    if (c + 3 < nc) load(c + 3, std::integral_constant<int, 1 - q>());
                    __syncthreads();
                }
            });
        }
        return;
    }

    // ---- chain waves
    const int tl = lane / TE, el = wave * TE + lane % TE;
    float acc = 0.0f;
    __syncthreads();                                 // chunks 0 and 1 are in LDS
    for (int c = 0; c < nc; ++c) {
        const int b = c % NB;
        const float* px = s_x[b][tl];
        const float* pw = s_w[b][el];
#pragma unroll 8
        for (int h = 0; h < HC; h += 4) {
            const floatx4 xv = *reinterpret_cast<const floatx4*>(px + h);
            const floatx4 wv = *reinterpret_cast<const floatx4*>(pw + h);
            acc = __builtin_fmaf(xv[0], wv[0], acc);
            acc = __builtin_fmaf(xv[1], wv[1], acc);
            acc = __builtin_fmaf(xv[2], wv[2], acc);
            acc = __builtin_fmaf(xv[3], wv[3], acc);
        }
        __syncthreads();                             // chunk c + 1 is complete; buffer b may be refilled
    }
    const int t = tok0 + tl, e = e0 + el;
    if (t < T && e < E) {
        float v = acc;
        if (bias != nullptr) v = v + bias[e];
        logits[static_cast<int64_t>(t) * E + e] = v;
    }
}

template <int NE>
__global__ __launch_bounds__(kRouteThreads) void select_kernel(
    const float* __restrict__ logits, int T, int E, int K, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_w) {
    const int lane = threadIdx.x & (kWave - 1);
    const int t = blockIdx.x * kRouteWaves + (threadIdx.x >> 6);
    if (t >= T) return;   // whole wave
    float l[NE];
#pragma unroll
    for (int g = 0; g < NE; ++g) {
        const int e = g * kWave + lane;
        l[g] = e < E ? logits[static_cast<int64_t>(t) * E + e] : 0.0f;
    }
    select_and_write<NE>(l, E, K, t, topk_idx, topk_w);
}

template <typename XT, int R, int NE>
void launch_route_t(const moe_shape& s, const XT* x, const XT* w, const float* bias, int32_t* idx,
                    float* tw, float* logits, hipStream_t st) {
    const int tokens_per_block = kRouteWaves * R;
    const int grid = (s.T + tokens_per_block - 1) / tokens_per_block;
    hipLaunchKernelGGL((route_kernel<XT, R, NE>), dim3(grid), dim3(kRouteThreads), 0, st, x, w, bias, s.T,
                       s.H, s.E, s.K, idx, tw, logits);
}

template <typename XT, int R, int NE, int SPLIT, int WAVES, int HC, int P>
void launch_fast(const moe_shape& s, const XT* x, const XT* w, const float* bias, int32_t* idx, float* tw,
                 float* logits, hipStream_t st) {
    constexpr int TOK = (WAVES / SPLIT) * R;
    const int grid = (s.T + TOK - 1) / TOK;
    hipLaunchKernelGGL((route_fast_kernel<XT, R, NE, SPLIT, WAVES, HC, P>), dim3(grid), dim3(WAVES * 64), 0, st, x,
                       w, bias, s.T, s.H, s.E, s.K, idx, tw, logits);
}

// spare CUs past `grid` routing workgroups, to warm the last-level cache with pf
int prefetch_workgroups(int grid, const CachePrefetch& pf) {
    if (pf.region == nullptr || pf.bytes < 1024) return 0;
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess) {
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0) cus = v;
    }
    return grid < cus ? cus - grid : 0;
}

template <typename XT, int TPW, int WE, int DW, int HC, int NB, int XMAX>
void launch_chain(const moe_shape& s, const XT* x, const XT* w, const float* bias, int32_t* idx, float* tw,
                  float* logits, const CachePrefetch& pf, hipStream_t st) {
    const int grid = (s.T + TPW - 1) / TPW;
    // spare CUs read the prefetch region while the routing workgroups run
    const int extra = prefetch_workgroups(grid, pf);
    hipLaunchKernelGGL((route_chain_kernel<XT, TPW, WE, DW, HC, NB, XMAX>), dim3(grid + extra),
                       dim3((TPW * WE + DW) * 64), 0, st, x, w, bias, s.T, s.H, s.E, s.K, idx, tw, logits, grid,
                       static_cast<const uint16_t*>(pf.region), static_cast<int64_t>(pf.bytes / 1024));
}

constexpr int kTileTokens = 8;      // tiled router: tokens x experts per chain wave, h per chunk
constexpr int kTileExperts = 8;
constexpr int kTileChains = 1;      // chain waves per workgroup (beside one copy wave)
constexpr int kTileChunk = 256;
constexpr int kTileMaxT = 1024;

bool tile_eligible(const moe_shape& s, int x_dtype) {
    const int vec = x_dtype == MOE_BF16 ? 8 : 4;
    return s.T <= kTileMaxT && s.E % vec == 0 && s.H % kTileChunk == 0;
}

template <typename XT>
void launch_tile(const moe_shape& s, const XT* x, const XT* w, const float* bias, float* logits, int32_t* idx,
                 float* tw, const CachePrefetch& pf, hipStream_t st) {
    constexpr int EW = kTileChains * kTileExperts;
    const int ntile = ((s.T + kTileTokens - 1) / kTileTokens) * ((s.E + EW - 1) / EW);
    const int extra = prefetch_workgroups(ntile, pf);
    hipLaunchKernelGGL((route_tile_kernel<XT, kTileTokens, kTileExperts, kTileChains, kTileChunk>),
                       dim3(ntile + extra), dim3((kTileChains + 1) * kWave), 0, st, x, w, bias, s.T, s.H, s.E,
                       logits, ntile, static_cast<const uint16_t*>(pf.region), static_cast<int64_t>(pf.bytes / 1024));
    launch_route_from_logits(s, logits, idx, tw, st);
}

template <typename XT>
void launch_route_dt(const moe_shape& s, const XT* x, const XT* w, const float* bias, int32_t* idx,
                     float* tw, float* logits, const CachePrefetch& pf, hipStream_t st) {
    // rows of the router weight must split into 16-byte pieces (E a multiple of 8 for bf16, 4 for float32)
    if (s.E <= 128 && s.E % (16 / sizeof(XT)) == 0 && s.T <= kChainMaxT && s.H <= 4096) {
        // one token per workgroup: chains spread over as many CUs as there are tokens
        if (s.E <= 64) launch_chain<XT, 1, 1, 1, 64, 4, 4096>(s, x, w, bias, idx, tw, logits, pf, st);
        else launch_chain<XT, 1, 2, 2, 64, 4, 4096>(s, x, w, bias, idx, tw, logits, pf, st);
        return;
    }
    if (s.E <= 128) {
        if (s.T >= 2048) {
            // 8 waves x 3 tokens per workgroup: about two waves per SIMD at 6000 tokens
            if (s.E <= 64) launch_fast<XT, 3, 1, 1, 8, 32, 3>(s, x, w, bias, idx, tw, logits, st);
            else launch_fast<XT, 3, 2, 1, 8, 32, 3>(s, x, w, bias, idx, tw, logits, st);
        } else {
            // one chain per lane, 64-row chunks (fewer per-chunk barriers), four-chunk prefetch
            if (s.E <= 64) launch_fast<XT, 1, 1, 1, 8, 64, 4>(s, x, w, bias, idx, tw, logits, st);
            else launch_fast<XT, 1, 1, 2, 8, 64, 4>(s, x, w, bias, idx, tw, logits, st);
        }
        return;
    }
    if (s.E <= 256) {
        if (s.T >= 2048) launch_route_t<XT, 4, 4>(s, x, w, bias, idx, tw, logits, st);
        else launch_route_t<XT, 1, 4>(s, x, w, bias, idx, tw, logits, st);
    } else {
        launch_route_t<XT, 1, 16>(s, x, w, bias, idx, tw, logits, st);
    }
}

// ---------------------------------------------------------------------------
// Screened path: bf16 activations and router weights, E == 128, no logits
// output.  Two kernels:
//
//  1. route_screen_kernel -- estimates every logit with bf16 MFMA (any
//     summation order) over one H slice, together with the squared norms of
//     the token rows and of the router-weight columns, and writes a transposed
//     copy of the router weight ([E][H], so that one expert's weights are
//     contiguous);
//  2. route_exact_kernel -- per token, bounds the gap between estimate and
//     canonical logit, keeps the experts that the bound cannot exclude from
//     the top K, evaluates only their canonical fma chains, and selects among
//     them.
//
// Why the result is identical to evaluating every canonical logit.  For one
// token write p_h = x_h w_he (exact in float32: bf16 x bf16), B_e = sum |p_h|,
// u = 2^-24, L_e the canonical logit and A_e the estimate plus bias.
//   * The canonical chain rounds once per step: |L_e - (S_e + b_e)| <=
//     gamma_H B_e + u |L_e|, gamma_H = H u / (1 - H u) (recursive summation).
//   * One v_mfma adds 16 exact products to its accumulator.  Even an adder
//     that aligned all 17 terms to the largest one without guard bits would
//     err by at most 36 u times their absolute sum.  Every 64-h chunk starts
//     from a zero accumulator, so its four steps err by at most
//     36 u (4 B_1 + 3 B_2 + 2 B_3 + B_4) (1 + 150 u) <= 144.1 u B_c over the
//     chunk's products; the chunk sums, then the slice partials and the bias,
//     are added in float32, one after another: at most H/64 + 1 additions,
//     gamma_(H/64+1) times their absolute sum.  With the canonical chain's
//     gamma_H this stays below (1.0625 H + 192) u B_e + 2 u |A_e| for
//     H <= 65536 (gamma_n <= 1.004 n u there).
//   * Cauchy-Schwarz: B_e <= ||x|| ||w_e||.  The norms come from float32 sums
//     of squares, whose relative error (below 2 H u) is covered by the factor
//     (1 + 3 H u).
// Hence |A_e - L_e| <= D_e = (1.0625 H + 192) u ||x|| ||w_e|| (1 + 3 H u) +
// 2^-21 |A_e| + 1e-30, for H <= 65536.  If K experts f have A_f - D_f >= theta > A_e + D_e
// then L_f > L_e for each of them and e is outside the top K.  The
// candidates are the experts with A_e + D_e >= theta, theta = the K-th
// largest A_f - D_f: at least K of them (those defining theta), including
// every member of the top K.  Selecting the K best candidates by canonical
// logit, with the same key and tie rule, reproduces the full selection.
// ---------------------------------------------------------------------------
constexpr int kScreenE = 128;   // experts of the screened path
constexpr int kScrHC = 64;      // h per staged chunk: 128-byte rows of bf16
constexpr int kScrNB = 3;       // copy-ring stages (two chunks in flight; two workgroups fit a CU)

// Physical 16-byte slot of logical segment c of row r in a tile of 128-byte
// rows (XOR is its own inverse, so the same map gives the logical segment of a
// physical slot).  The 16 rows one ds_read_b128 pass reads at one segment land
// on 16 distinct 4-bank groups.
__device__ __forceinline__ int swz128(int r, int c) { return c ^ ((r >> 1) & 7); }
// 256-byte rows (one h of the router weight, 128 experts): rows h and h + 8,
// read together by one B fragment, put a 64-byte expert group on different banks.
__device__ __forceinline__ int swz256(int h, int c) { return c ^ (((h >> 3) & 3) << 2); }

__device__ __forceinline__ float bf_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

// Slices of H for the screening kernel: enough workgroups to cover the chip,
// and while there are fewer than 4 slices, enough for two per CU (two fit);
// every slice a whole number of chunks.
__host__ __device__ inline int screen_tokens_per_block(int T) { return T >= 2048 ? 64 : 32; }
inline int screen_slices(int T, int H) {
    const int nblk = (T + screen_tokens_per_block(T) - 1) / screen_tokens_per_block(T);
    const int chunks = H / kScrHC;
    int S = 1;
    while ((nblk * S < 256 || (nblk * S < 512 && S < 4)) && S < 16 && chunks % (2 * S) == 0) S *= 2;
    return S;
}

struct ScreenWs {
    uint16_t* wT;   // [E][H] bf16
    float* part;    // [S][T][E] estimate partial sums
    float* nx;      // [S][T] partial squared norms of token rows
    float* nw;      // [S][E] partial squared norms of router-weight columns
    size_t off_part, off_nx, off_nw;   // byte offsets of part, nx, nw from the base
    size_t bytes;
};

inline size_t align256(size_t n) { return (n + 255) & ~static_cast<size_t>(255); }

inline ScreenWs screen_layout(const moe_shape& s, void* base) {
    const int S = screen_slices(s.T, s.H);
    ScreenWs w{};
    char* p = static_cast<char*>(base);
    size_t off = 0;
    auto take = [&](size_t n) { char* q = p ? p + off : nullptr; off += align256(n); return q; };
    w.wT = reinterpret_cast<uint16_t*>(take(static_cast<size_t>(s.E) * s.H * 2));
    w.off_part = off;
    w.part = reinterpret_cast<float*>(take(static_cast<size_t>(S) * s.T * s.E * 4));
    w.off_nx = off;
    w.nx = reinterpret_cast<float*>(take(static_cast<size_t>(S) * s.T * 4));
    w.off_nw = off;
    w.nw = reinterpret_cast<float*>(take(static_cast<size_t>(S) * s.E * 4));
    w.bytes = off;
    return w;
}

template <int TM>   // 32-token MFMA tiles per workgroup
__global__ __launch_bounds__(256) void route_screen_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, int T, int H, int Hs, int nblk,
    uint16_t* __restrict__ wT, float* __restrict__ part, float* __restrict__ nx, float* __restrict__ nw) {
    constexpr int E = kScreenE;
    constexpr int BT = 32 * TM;
    constexpr int XSTAGE = BT * kScrHC;              // elements: BT rows of 64 h
    constexpr int WSTAGE = kScrHC * E;               // 64 rows of 128 experts
    constexpr int STAGE = XSTAGE + WSTAGE;
    constexpr int XI = XSTAGE / 512;                 // 1 KiB copies per stage (8 x rows each)
    constexpr int WI = WSTAGE / 512;                 // (4 weight rows each)
    constexpr int Q = (XI + WI) / 4;                 // copies per wave per stage
    static_assert((XI + WI) % 4 == 0, "copies must split evenly over the four waves");
    __shared__ __attribute__((aligned(1024))) uint16_t s_ring[kScrNB][STAGE];
    __shared__ float s_nx[4][BT];
    static_assert(kScrHC / 16 == 4, "one k-step of token norms per wave");

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int blk = blockIdx.x, sl = blockIdx.y;
    const int tok0 = blk * BT;
    const int hbeg = sl * Hs;
    const int nc = Hs / kScrHC;

    // this lane's source for chunk 0, the per-chunk stride, and the wave-uniform
    // LDS offset of each of the wave's copies
    const uint16_t* src[Q];
    int stride[Q], dst[Q];
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        const int ins = wave * Q + q;
        if (ins < XI) {
            const int r = ins * 8 + (lane >> 3);
            const int t = min(tok0 + r, T - 1);
            src[q] = x + static_cast<int64_t>(t) * H + hbeg + swz128(r, lane & 7) * 8;
            stride[q] = kScrHC;
            dst[q] = ins * 512;
        } else {
            const int j = ins - XI;
            const int h = j * 4 + (lane >> 4);
            src[q] = w + static_cast<int64_t>(hbeg + h) * E + swz256(h, lane & 15) * 8;
            stride[q] = kScrHC * E;
            dst[q] = XSTAGE + j * 512;
        }
    }
    auto issue = [&](int kc, int st) {
#pragma unroll
        for (int q = 0; q < Q; ++q) dma16(src[q] + static_cast<int64_t>(kc) * stride[q], &s_ring[st][dst[q]]);
    };

    floatx16 acc[TM];
#pragma unroll
    for (int m = 0; m < TM; ++m)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[m][v] = 0.0f;
    float nxp[TM];
#pragma unroll
    for (int m = 0; m < TM; ++m) nxp[m] = 0.0f;
    float nwp = 0.0f;

    const int col = lane & 31;            // B column / A row within a 32 tile
    const int kg = lane >> 5;             // which 8 of the 16 k of a step
    const int e = wave * 32 + col;        // this lane's expert (B operand)

    // one chunk: its four k-steps accumulate from zero, and the chunk sum is
    // then added to the running estimate in float32 (the bound counts on it)
    auto compute = [&](int st, int kc) {
        floatx16 cacc[TM];
#pragma unroll
        for (int m = 0; m < TM; ++m)
#pragma unroll
            for (int v = 0; v < 16; ++v) cacc[m][v] = 0.0f;
        const uint16_t* sx = s_ring[st];
        const uint16_t* sw = s_ring[st] + XSTAGE;
        const bool write_t = ((hbeg / kScrHC + kc) % nblk) == blk;   // this block stores this chunk of wT
#pragma unroll
        for (int ks = 0; ks < kScrHC / 16; ++ks) {
            // B fragment: 8 consecutive h of expert e
            uint32_t b32[4];
#pragma unroll
            for (int j2 = 0; j2 < 4; ++j2) {
                uint32_t pr = 0;
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    const int h = ks * 16 + kg * 8 + j2 * 2 + hf;
                    const uint32_t v = sw[h * E + swz256(h, e >> 3) * 8 + (e & 7)];
                    pr |= v << (16 * hf);
                }
                b32[j2] = pr;
            }
            u32x4 b = {b32[0], b32[1], b32[2], b32[3]};
#pragma unroll
            for (int j2 = 0; j2 < 4; ++j2) {
                const float lo = bf_lo(b32[j2]), hi = bf_hi(b32[j2]);
                nwp = fmaf(lo, lo, nwp);
                nwp = fmaf(hi, hi, nwp);
            }
            if (write_t)
                *reinterpret_cast<u32x4*>(wT + static_cast<int64_t>(e) * H + hbeg + kc * kScrHC + ks * 16 + kg * 8) = b;
#pragma unroll
            for (int m = 0; m < TM; ++m) {
                const int r = m * 32 + col;
                const u32x4 a = *reinterpret_cast<const u32x4*>(&sx[r * kScrHC + swz128(r, ks * 2 + kg) * 8]);
                if (wave == ks) {                        // token norms: wave w takes k-step w
#pragma unroll
                    for (int j2 = 0; j2 < 4; ++j2) {
                        const float lo = bf_lo(a[j2]), hi = bf_hi(a[j2]);
                        nxp[m] = fmaf(lo, lo, nxp[m]);
                        nxp[m] = fmaf(hi, hi, nxp[m]);
                    }
                }
                cacc[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                                  __builtin_bit_cast(bf16x8_t, b), cacc[m], 0, 0, 0);
            }
        }
#pragma unroll
        for (int m = 0; m < TM; ++m)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[m][v] += cacc[m][v];
    };

    // ring: chunk kc lives in stage kc % NB; NB-1 chunks in flight (indices past
    // the end are clamped: harmless reloads into stages already consumed)
#pragma unroll
    for (int q = 0; q < kScrNB - 1; ++q) issue(min(q, nc - 1), q);
    for (int kc = 0; kc < nc; ++kc) {
        wait_vmcnt<Q * (kScrNB - 2)>();     // this wave's copies of chunk kc have landed
        __builtin_amdgcn_s_barrier();       // ... everyone's, and stage (kc - 1) is free
        issue(min(kc + kScrNB - 1, nc - 1), (kc + kScrNB - 1) % kScrNB);
        compute(kc % kScrNB, kc);
    }
    wait_vmcnt<0>();   // no copy may land after the workgroup's LDS is released

    // estimates: lane holds column e and rows 8*(v/4) + 4*kg + v%4 of each 32-row tile
#pragma unroll
    for (int m = 0; m < TM; ++m)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int t = tok0 + m * 32 + 8 * (v >> 2) + 4 * kg + (v & 3);
            if (t < T) part[(static_cast<int64_t>(sl) * T + t) * E + e] = acc[m][v];
        }
    // token norms: the four waves' partials (k-steps 0..3 of every chunk), added in wave order
#pragma unroll
    for (int m = 0; m < TM; ++m) {
        const float n2 = nxp[m] + __shfl_xor(nxp[m], 32, kWave);
        if (kg == 0) s_nx[wave][m * 32 + col] = n2;
    }
    __syncthreads();
    if (wave == 0) {
#pragma unroll
        for (int m = 0; m < TM; ++m) {
            const int r = m * 32 + col;
            const float n2 = ((s_nx[0][r] + s_nx[1][r]) + s_nx[2][r]) + s_nx[3][r];
            const int t = tok0 + r;
            if (kg == 0 && t < T) nx[static_cast<int64_t>(sl) * T + t] = n2;
        }
    }
    if (blk == 0) {
        const float n2 = nwp + __shfl_xor(nwp, 32, kWave);
        if (kg == 0) nw[sl * E + e] = n2;
    }
}

// Largest value over each row of 16 lanes, in every lane of the row: a running
// maximum by DPP row shifts (lanes shifted in from outside the row see 0,
// neutral for an unsigned maximum), then lane 15's result broadcast to its row.
__device__ __forceinline__ uint32_t row16_max_u32(uint32_t v) {
    v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x111, 0xf, 0xf, false)));
    v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x112, 0xf, 0xf, false)));
    v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x114, 0xf, 0xf, false)));
    v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x118, 0xf, 0xf, false)));
    return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x15F, 0xf, 0xf, false));
}

// Largest 64-bit value over each row of 16 lanes: the largest upper half, then
// the largest lower half among the lanes holding it.
__device__ __forceinline__ uint64_t group16_max_u64(uint64_t v) {
    const uint32_t hi = row16_max_u32(static_cast<uint32_t>(v >> 32));
    const uint32_t lo = row16_max_u32(static_cast<uint32_t>(v >> 32) == hi ? static_cast<uint32_t>(v) : 0u);
    return (static_cast<uint64_t>(hi) << 32) | lo;
}

// 256-byte rows (128 bf16): the 16 rows one ds_read_b128 pass reads at one
// segment land on 16 distinct 4-bank groups.
__device__ __forceinline__ int swz256r(int r, int c) { return c ^ (r & 15); }

// Eight canonical chain steps of the exact kernel: acc = fma(x[j], w[j], acc)
// for j = 0..7 in order, w[j] the bf16 halves of w0..w3 (low half first)
// widened exactly.  Each widening runs one step ahead into its own temporary,
// so an fma waits only for the previous fma.  The _fetch form also issues the next segment's three LDS
// reads (weights at aw, token row at ax + OX) before the steps and waits for
// them at its end, so the reads overlap the steps and no load is in flight
// outside the block.
#define MOE_EXACT_STEPS                                                                                        \
    "v_lshlrev_b32 %[t0], 16, %[w0]\n\t"                                                                      \
    "v_and_b32 %[t1], 0xffff0000, %[w0]\n\t"                                                                  \
    "v_fmac_f32 %[acc], %[a0], %[t0]\n\t"                                                                     \
    "v_lshlrev_b32 %[t2], 16, %[w1]\n\t"                                                                      \
    "v_fmac_f32 %[acc], %[a1], %[t1]\n\t"                                                                     \
    "v_and_b32 %[t3], 0xffff0000, %[w1]\n\t"                                                                  \
    "v_fmac_f32 %[acc], %[a2], %[t2]\n\t"                                                                     \
    "v_lshlrev_b32 %[t0], 16, %[w2]\n\t"                                                                      \
    "v_fmac_f32 %[acc], %[a3], %[t3]\n\t"                                                                     \
    "v_and_b32 %[t1], 0xffff0000, %[w2]\n\t"                                                                  \
    "v_fmac_f32 %[acc], %[a4], %[t0]\n\t"                                                                     \
    "v_lshlrev_b32 %[t2], 16, %[w3]\n\t"                                                                      \
    "v_fmac_f32 %[acc], %[a5], %[t1]\n\t"                                                                     \
    "v_and_b32 %[t3], 0xffff0000, %[w3]\n\t"                                                                  \
    "v_fmac_f32 %[acc], %[a6], %[t2]\n\t"                                                                     \
    "v_fmac_f32 %[acc], %[a7], %[t3]\n\t"

template <int OX>
__device__ __forceinline__ void exact_steps_fetch(float& acc, const u32x4& w, const floatx4& x0, const floatx4& x1,
                                                  u32x4& nw, floatx4& nx0, floatx4& nx1, uint32_t aw, uint32_t ax) {
    float t0, t1, t2, t3;
    asm volatile("ds_read_b128 %[nw], %[aw]\n\t"
                 "ds_read_b128 %[nx0], %[ax] offset:%[ox0]\n\t"
                 "ds_read_b128 %[nx1], %[ax] offset:%[ox1]\n\t"
                 MOE_EXACT_STEPS
                 "s_waitcnt lgkmcnt(0)"
                 : [acc] "+v"(acc), [nw] "=&v"(nw), [nx0] "=&v"(nx0), [nx1] "=&v"(nx1), [t0] "=&v"(t0),
                   [t1] "=&v"(t1), [t2] "=&v"(t2), [t3] "=&v"(t3)
                 : [w0] "v"(w[0]), [w1] "v"(w[1]), [w2] "v"(w[2]), [w3] "v"(w[3]), [a0] "v"(x0[0]),
                   [a1] "v"(x0[1]), [a2] "v"(x0[2]), [a3] "v"(x0[3]), [a4] "v"(x1[0]), [a5] "v"(x1[1]),
                   [a6] "v"(x1[2]), [a7] "v"(x1[3]), [aw] "v"(aw), [ax] "v"(ax), [ox0] "i"(OX), [ox1] "i"(OX + 16)
                 : "memory");
}

__device__ __forceinline__ void exact_steps(float& acc, const u32x4& w, const floatx4& x0, const floatx4& x1) {
    float t0, t1, t2, t3;
    asm volatile(MOE_EXACT_STEPS
                 : [acc] "+v"(acc), [t0] "=&v"(t0), [t1] "=&v"(t1), [t2] "=&v"(t2), [t3] "=&v"(t3)
                 : [w0] "v"(w[0]), [w1] "v"(w[1]), [w2] "v"(w[2]), [w3] "v"(w[3]), [a0] "v"(x0[0]),
                   [a1] "v"(x0[1]), [a2] "v"(x0[2]), [a3] "v"(x0[3]), [a4] "v"(x1[0]), [a5] "v"(x1[1]),
                   [a6] "v"(x1[2]), [a7] "v"(x1[3]));
}
#undef MOE_EXACT_STEPS

// Segments C .. NSEG-1 of one 128-h chunk of a chain (segment C's operands
// already in registers); aw is the chain's weight row, ax its token row.
template <int C, int NSEG>
__device__ __forceinline__ void exact_chain_segments(float& a, u32x4 wv, floatx4 x0, floatx4 x1, uint32_t aw,
                                                     int u, uint32_t ax) {
    if constexpr (C + 1 < NSEG) {
        u32x4 wn;
        floatx4 y0, y1;
        exact_steps_fetch<(8 * C + 8) * 4>(a, wv, x0, x1, wn, y0, y1, aw + swz256r(u, C + 1) * 16, ax);
        exact_chain_segments<C + 1, NSEG>(a, wn, y0, y1, aw, u, ax);
    } else {
        exact_steps(a, wv, x0, x1);
    }
}

// A workgroup owns BT = 4 * WAVES tokens; 16 lanes per token.  Lane s of a
// token's group screens experts s, s+16, ..., s+112.  The candidate chains of
// a wave's four tokens are then laid out one after another and dealt over all
// 64 lanes (chain c to lane c % 64), so a token with more than 16 candidates
// borrows lanes its neighbours leave idle instead of running a second round.
// The canonical chains read 128-h chunks of the transposed router-weight rows
// of the union of the block's candidates and of the token rows, staged in LDS
// by a ring of direct-to-LDS copies (NB stages); each wave widens its four
// token rows to float32 once per chunk in a wave-private area, so a chain step
// costs one widening of the weight and one fma.  The finished logits go back
// through LDS to the 16 lanes of their token, which select its top K.
template <int WAVES, int NB, int SMAX>
__global__ __launch_bounds__(WAVES * 64) void route_exact_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wT, const float* __restrict__ bias,
    const float* __restrict__ part, const float* __restrict__ nx, const float* __restrict__ nw,
    int T, int H, int K, int S, int32_t* __restrict__ topk_idx, float* __restrict__ topk_w) {
    constexpr int E = kScreenE;
    constexpr int NT = WAVES * 64;
    constexpr int BT = 4 * WAVES;
    constexpr int HC = 128;                                 // h per chunk: 256-byte bf16 rows
    constexpr int RE = HC;                                  // elements per staged row
    constexpr int TROWS = BT < 4 ? 4 : BT;                  // token rows (a copy moves 4 rows)
    constexpr int XOFF = E * RE;                            // element offset of the token rows
    constexpr int SPARE = XOFF + TROWS * RE;                // 1 KiB target of padding copies
    constexpr int STAGE = SPARE + 512;                      // elements
    constexpr int QMAX = (E / 4 + TROWS / 4 + WAVES - 1) / WAVES;   // copies per wave per chunk, at most
    __shared__ __attribute__((aligned(1024))) uint16_t s_ring[NB][STAGE];
    __shared__ __attribute__((aligned(16))) float s_xf[WAVES][4][HC + 4];
    __shared__ uint16_t s_chain[WAVES][4 * E];             // expert | (token of the wave << 8)
    __shared__ uint16_t s_perm[WAVES][4 * E];              // chain dealt to slot j (lane j % 64)
    __shared__ int s_hist[WAVES][16];
    static_assert(STAGE * 2 >= WAVES * 4 * E * 4, "the first ring stage holds the finished chain sums");
    __shared__ int s_flag[E];
    __shared__ uint8_t s_map[E];
    __shared__ uint8_t s_list[E];
    __shared__ int s_nu;
    __shared__ float s_nw[E];
    __shared__ float s_bias[E];                            // the bias (0 without one), read from LDS below

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, s = lane & 15;
    const int tl = wave * 4 + g;                 // token within the block
    const int tok0 = blockIdx.x * BT;
    const int t = tok0 + tl;
    const bool valid = t < T;
    const float Hu = static_cast<float>(H) * 0x1p-24f;

    // all slice partials of this lane's 8 experts are loaded before any is
    // summed, and before the weight norms below: their latencies overlap.  The
    // loads are unconditional (a lane past T or a slice past S reads token 0 or
    // slice 0, then drops the value), so they issue back to back instead of
    // one branch and one wait each.
    float pv[SMAX][8];
    float nxv[SMAX];
    const int64_t tl_safe = valid ? t : 0;
#pragma unroll
    for (int sl = 0; sl < SMAX; ++sl) {
        const bool live = valid && sl < S;
        const int64_t row = static_cast<int64_t>(sl < S ? sl : 0) * T + tl_safe;
        const float nv = nx[row];
        nxv[sl] = live ? nv : 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float v = part[row * E + s + 16 * i];
            pv[sl][i] = live ? v : 0.0f;
        }
    }
    // squared norms of the router-weight columns (sum of the slice partials, once
    // per workgroup; loads unconditional, as above), and the bias
    for (int i = tid; i < E; i += NT) {
        s_flag[i] = 0;
        float w2[SMAX];
#pragma unroll
        for (int sl = 0; sl < SMAX; ++sl) w2[sl] = nw[(sl < S ? sl : 0) * E + i];
        float n2 = 0.0f;
#pragma unroll
        for (int sl = 0; sl < SMAX; ++sl)
            if (sl < S) n2 += w2[sl];
        s_nw[i] = n2;
        s_bias[i] = bias != nullptr ? bias[i] : 0.0f;
    }
    __syncthreads();

    // ---- screen: estimates, windows, theta, candidates ----
    float nxs = 0.0f;
#pragma unroll
    for (int sl = 0; sl < SMAX; ++sl) nxs += nxv[sl];
    const float sx = sqrtf(nxs) * (1.0f + 3.0f * Hu);
    const float dcoef = (1.0625f * static_cast<float>(H) + 192.0f) * 0x1p-24f;
    float hi[8];
    uint64_t klo[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int e = s + 16 * i;
        float a = 0.0f;
#pragma unroll
        for (int sl = 0; sl < SMAX; ++sl) a += pv[sl][i];
        const float la = bias != nullptr ? a + s_bias[e] : a;
        const float d = dcoef * (sx * sqrtf(s_nw[e])) + 0x1p-21f * fabsf(la) + 1e-30f;
        hi[i] = valid ? la + d : -INFINITY;
        klo[i] = make_key(valid ? la - d : -INFINITY, e);
    }
    uint64_t kth = 0ull;
    {
        uint32_t taken = 0u;
        for (int r = 0; r < K; ++r) {
            uint64_t best = 0ull;
#pragma unroll
            for (int i = 0; i < 8; ++i) best = (!((taken >> i) & 1u) && klo[i] > best) ? klo[i] : best;
            best = group16_max_u64(best);
#pragma unroll
            for (int i = 0; i < 8; ++i)
                if (klo[i] == best) taken |= 1u << i;
            kth = best;
        }
    }
    const float theta = key_logit(kth);
    uint32_t cm = 0u;
#pragma unroll
    for (int i = 0; i < 8; ++i)
        if (valid && hi[i] >= theta) cm |= 1u << i;
    const int mine = __builtin_popcount(cm);
    int incl = mine;
#pragma unroll
    for (int d = 1; d < 16; d <<= 1) {
        const int o = __shfl_up(incl, d, 16);
        if (s >= d) incl += o;
    }
    const int total = __shfl(incl, 15, 16);      // candidates of this token
    // the wave's chain list: token 0's candidates, then token 1's, ...
    const int tot0 = __shfl(incl, 15, kWave), tot1 = __shfl(incl, 31, kWave);
    const int tot2 = __shfl(incl, 47, kWave), tot3 = __shfl(incl, 63, kWave);
    const int nwc = tot0 + tot1 + tot2 + tot3;   // chains of this wave (wave-uniform)
    const int base = (g > 0 ? tot0 : 0) + (g > 1 ? tot1 : 0) + (g > 2 ? tot2 : 0);   // first chain of token g
    {
        int pos = base + incl - mine;
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if ((cm >> i) & 1u) {
                s_chain[wave][pos++] = static_cast<uint16_t>((s + 16 * i) | (g << 8));
                s_flag[s + 16 * i] = 1;
            }
    }
    __syncthreads();
    if (wave == 0) {
        const bool f0 = s_flag[lane] != 0, f1 = s_flag[lane + 64] != 0;
        const uint64_t m0 = __ballot(f0), m1 = __ballot(f1);
        const uint64_t below = (1ull << lane) - 1ull;
        const int r0 = __popcll(m0 & below);
        const int r1 = __popcll(m0) + __popcll(m1 & below);
        if (f0) { s_list[r0] = static_cast<uint8_t>(lane); s_map[lane] = static_cast<uint8_t>(r0); }
        if (f1) { s_list[r1] = static_cast<uint8_t>(lane + 64); s_map[lane + 64] = static_cast<uint8_t>(r1); }
        if (lane == 0) s_nu = __popcll(m0) + __popcll(m1);
    }
    __syncthreads();
    const int nu = s_nu;

    // ---- copy plan: ceil(nu/4) copies of union rows and TROWS/4 of token rows
    // (4 rows of 256 B each), spread evenly over the waves (padding copies go to
    // the spare KiB) ----
    const int nU = (nu + 3) >> 2;
    const int nI = nU + TROWS / 4;
    const int q = (nI + WAVES - 1) / WAVES;      // uniform over the workgroup
    const uint16_t* src[QMAX];
    int dst[QMAX];
#pragma unroll
    for (int j = 0; j < QMAX; ++j) {
        const int ins = wave * q + j;
        const int slot = lane & 15;
        if (ins < nU) {
            const int u = ins * 4 + (lane >> 4);
            const int ex = s_list[u < nu ? u : 0];
            src[j] = wT + static_cast<int64_t>(ex) * H + swz256r(u, slot) * 8;
            dst[j] = ins * 4 * RE;
        } else if (ins < nI) {
            const int rr = (ins - nU) * 4 + (lane >> 4);
            const int tt = min(tok0 + rr, T - 1);
            src[j] = x + static_cast<int64_t>(tt) * H + slot * 8;
            dst[j] = XOFF + (ins - nU) * 4 * RE;
        } else {
            src[j] = x + static_cast<int64_t>(tok0) * H + slot * 8;
            dst[j] = SPARE;
        }
    }
    auto issue = [&](int kc, int st) {
#pragma unroll
        for (int j = 0; j < QMAX; ++j)
            if (j < q) dma16(src[j] + static_cast<int64_t>(kc) * HC, &s_ring[st][dst[j]]);
    };

    // ---- deal the wave's chains to slots (slot j runs on lane j % 64, round
    // j / 64).  A chain reads its union row in bank group (row index mod 16)
    // (swz256r), and the 16 lanes of one LDS read pass conflict when two of them
    // read different rows of one group.  So the chains are ordered by (rank
    // within their group, group): any 16 consecutive slots then hold at most two
    // chains of one group, and a full rank holds each group once. ----
    constexpr int PMAX = 4 * E / kWave;
    if (lane < 16) s_hist[wave][lane] = 0;
    __syncthreads();
    int rk[PMAX], rg[PMAX];
#pragma unroll
    for (int p = 0; p < PMAX; ++p) {
        const int c = lane + kWave * p;
        rg[p] = c < nwc ? (s_map[s_chain[wave][c] & 0xFF] & 15) : 0;
        rk[p] = c < nwc ? atomicAdd(&s_hist[wave][rg[p]], 1) : 0;
    }
    __syncthreads();
    int cnt[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) cnt[r] = s_hist[wave][r];
#pragma unroll
    for (int p = 0; p < PMAX; ++p) {
        const int c = lane + kWave * p;
        if (c < nwc) {
            int pos = 0;
#pragma unroll
            for (int r = 0; r < 16; ++r) pos += min(cnt[r], rk[p]) + ((r < rg[p] && cnt[r] > rk[p]) ? 1 : 0);
            s_perm[wave][pos] = static_cast<uint16_t>(c);
        }
    }
    __syncthreads();

    // this lane's chains: slots lane + 64 p (tokens past T have no candidates,
    // so every slot below nwc is a real chain)
    int urow[PMAX];
    int xoff[PMAX];                               // float offset of the chain's token row in s_xf[wave]
    int orig[PMAX];                               // the chain's place in the wave's list
    const int np = (nwc - lane + kWave - 1) / kWave;   // chains of this lane
#pragma unroll
    for (int p = 0; p < PMAX; ++p) {
        const int j = lane + kWave * p;
        orig[p] = j < nwc ? s_perm[wave][j] : 0;
        const int ent = j < nwc ? s_chain[wave][orig[p]] : 0;
        urow[p] = j < nwc ? s_map[ent & 0xFF] : 0;
        xoff[p] = (ent >> 8) * (HC + 4);
    }
    float acc[PMAX];
#pragma unroll
    for (int p = 0; p < PMAX; ++p) acc[p] = 0.0f;
    const int nc = H / HC;
    const float* xw0 = &s_xf[wave][0][0];
    const int xrow = XOFF + (wave * 4 + g) * RE;

#pragma unroll
    for (int j = 0; j < NB - 1; ++j) issue(min(j, nc - 1), j);
    for (int kc = 0; kc < nc; ++kc) {
        // chunk kc's copies are followed by q * (NB - 2) younger ones (vmcnt holds
        // at most 63; waiting for fewer than needed is merely stricter)
        wait_vmcnt_bin<0, 64>(min(q * (NB - 2), 63));
        __builtin_amdgcn_s_barrier();
        issue(min(kc + NB - 1, nc - 1), (kc + NB - 1) % NB);
        const uint16_t* sr = s_ring[kc % NB];
        // widen this wave's four token rows: lane (g, s) converts elements 8s .. 8s+7
        {
            const u32x4 v = *reinterpret_cast<const u32x4*>(&sr[xrow + s * 8]);
            floatx4 lo4 = {bf_lo(v[0]), bf_hi(v[0]), bf_lo(v[1]), bf_hi(v[1])};
            floatx4 hi4 = {bf_lo(v[2]), bf_hi(v[2]), bf_lo(v[3]), bf_hi(v[3])};
            *reinterpret_cast<floatx4*>(&s_xf[wave][g][8 * s]) = lo4;
            *reinterpret_cast<floatx4*>(&s_xf[wave][g][8 * s + 4]) = hi4;
        }
#pragma unroll
        for (int p = 0; p < PMAX; ++p) {
            if (p < np) {
                // operands of segment c + 1 are read while segment c's fma chain runs
                float a = acc[p];
                const int u = urow[p];
                const float* xw = xw0 + xoff[p];
                const uint16_t* wr = sr + u * RE;
                const uint32_t aw = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(wr));
                const uint32_t ax = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(xw));
                u32x4 wv = *reinterpret_cast<const u32x4*>(&wr[swz256r(u, 0) * 8]);
                floatx4 x0 = *reinterpret_cast<const floatx4*>(&xw[0]);
                floatx4 x1 = *reinterpret_cast<const floatx4*>(&xw[4]);
                exact_chain_segments<0, HC / 8>(a, wv, x0, x1, aw, u, ax);
                acc[p] = a;
            }
        }
    }
    wait_vmcnt<0>();
    __syncthreads();   // every wave is done with the ring: it now holds the canonical chain sums

    // ---- select the top K of the candidates by canonical logit ----
    float* s_lg = reinterpret_cast<float*>(&s_ring[0][0]) + wave * 4 * E;
#pragma unroll
    for (int p = 0; p < PMAX; ++p)
        if (p < np) s_lg[orig[p]] = acc[p];
    wait_lgkmcnt0();   // the wave reads back only its own list
    constexpr int PTOK = E / 16;                  // candidates s + 16 q of the token, per lane
    uint64_t key[PTOK];
#pragma unroll
    for (int q = 0; q < PTOK; ++q) {
        const int c = s + 16 * q;
        if (valid && c < total) {
            const int e = s_chain[wave][base + c] & 0xFF;
            const float a = s_lg[base + c];
            key[q] = make_key(bias != nullptr ? a + s_bias[e] : a, e);
        } else {
            key[q] = 0ull;
        }
    }
    int my_e[4] = {0, 0, 0, 0};
    float my_l[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    float l0 = 0.0f, sum = 0.0f;
    for (int r = 0; r < K; ++r) {
        uint64_t best = 0ull;
#pragma unroll
        for (int q = 0; q < PTOK; ++q) best = key[q] > best ? key[q] : best;
        best = group16_max_u64(best);
#pragma unroll
        for (int q = 0; q < PTOK; ++q)
            if (key[q] == best) key[q] = 0ull;
        const float l = key_logit(best);
        if (r == 0) l0 = l;
        sum += expf(l - l0);
        if ((r & 15) == s) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if ((r >> 4) == j) {
                    my_e[j] = key_expert(best);
                    my_l[j] = l;
                }
        }
    }
    if (valid) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = s + 16 * j;
            if (r < K) {
                topk_idx[static_cast<int64_t>(t) * K + r] = my_e[j];
                topk_w[static_cast<int64_t>(t) * K + r] = expf(my_l[j] - l0) / sum;
            }
        }
    }
}

template <int TM>
void launch_screen(const moe_shape& s, const uint16_t* x, const uint16_t* w, const ScreenWs& ws, int S,
                   hipStream_t st) {
    const int nblk = (s.T + 32 * TM - 1) / (32 * TM);
    hipLaunchKernelGGL(route_screen_kernel<TM>, dim3(nblk, S), dim3(256), 0, st, x, w, s.T, s.H, s.H / S, nblk,
                       ws.wT, ws.part, ws.nx, ws.nw);
}

template <int WAVES, int NB, int SMAX>
void launch_exact(const moe_shape& s, const uint16_t* x, const float* bias, const ScreenWs& ws, int S,
                  int32_t* idx, float* tw, hipStream_t st) {
    const int grid = (s.T + 4 * WAVES - 1) / (4 * WAVES);
    hipLaunchKernelGGL((route_exact_kernel<WAVES, NB, SMAX>), dim3(grid), dim3(WAVES * 64), 0, st, x, ws.wT, bias,
                       ws.part, ws.nx, ws.nw, s.T, s.H, s.K, S, idx, tw);
}

void launch_route_screened(const moe_shape& s, const uint16_t* x, const uint16_t* w, const float* bias,
                           int32_t* idx, float* tw, void* ws_base, hipStream_t st) {
    const ScreenWs ws = screen_layout(s, ws_base);
    const int S = screen_slices(s.T, s.H);
    if (screen_tokens_per_block(s.T) == 64) launch_screen<2>(s, x, w, ws, S, st);
    else launch_screen<1>(s, x, w, ws, S, st);
    // the exact kernel sums SMAX >= S slice partials (screen_slices gives S <= 16)
    if (s.T >= 2048) {
        // One workgroup fits a CU (LDS) and the chain steps are bound by the CU's
        // LDS, so a launch costs about (rounds of workgroups over the CUs) x (waves
        // per workgroup): 6 waves (24 tokens) when that fills the chip in fewer
        // rounds -- 6000 tokens make 250 workgroups, one round -- else 8 waves
        // (16384 tokens: 512 workgroups, two rounds, against three at 6 waves).
        int dev = 0, cus = 256;
        if (hipGetDevice(&dev) == hipSuccess) {
            int v = 0;
            if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0) cus = v;
        }
        auto cost = [&](int waves) {
            const int64_t wgs = (static_cast<int64_t>(s.T) + 4 * waves - 1) / (4 * waves);
            return ((wgs + cus - 1) / cus) * waves;
        };
        if (cost(6) < cost(8)) {
            if (S <= 4) launch_exact<6, 3, 4>(s, x, bias, ws, S, idx, tw, st);
            else launch_exact<6, 3, 16>(s, x, bias, ws, S, idx, tw, st);
        } else {
            if (S <= 4) launch_exact<8, 3, 4>(s, x, bias, ws, S, idx, tw, st);
            else launch_exact<8, 3, 16>(s, x, bias, ws, S, idx, tw, st);
        }
    } else {
        launch_exact<4, 3, 16>(s, x, bias, ws, S, idx, tw, st);
    }
}

// The exact kernel walks H in whole 128-element chunks (H % 128 == 0); the
// error bound holds for H <= 65536.  Below 512 tokens there are too few
// candidate chains to fill the chip and each one is a dependent sequence of
// H fma, so evaluating every logit directly is as fast.
constexpr int kScreenMinTokens = 512;
bool screen_eligible(const moe_shape& s, int x_dtype, int w_dtype) {
    return x_dtype == MOE_BF16 && w_dtype == MOE_BF16 && s.E == kScreenE && s.T >= kScreenMinTokens &&
           s.H % 128 == 0 && s.H <= 65536;
}

}  // namespace

size_t route_screen_bytes(const moe_shape& s, int x_dtype, int w_dtype) {
    return screen_eligible(s, x_dtype, w_dtype) ? screen_layout(s, nullptr).bytes : 0;
}

size_t route_workspace_bytes(const moe_shape& s) {
    // the screened path (bf16 only) or the tiled path's logits (float32 eligibility includes bf16's)
    const size_t screen = route_screen_bytes(s, MOE_BF16, MOE_BF16);
    const size_t tile = tile_eligible(s, MOE_F32) ? static_cast<size_t>(s.T) * s.E * sizeof(float) : 0;
    return screen > tile ? screen : tile;
}

bool route_screen_layout(const moe_shape& s, int x_dtype, int w_dtype, moe_route_screen_info* info) {
    if (!screen_eligible(s, x_dtype, w_dtype)) return false;
    const ScreenWs w = screen_layout(s, nullptr);
    info->slices = screen_slices(s.T, s.H);
    info->part_offset = w.off_part;
    info->nx_offset = w.off_nx;
    info->nw_offset = w.off_nw;
    info->bytes = w.bytes;
    return true;
}

int launch_route(const moe_shape& s, const void* x, int x_dtype, const void* w, const float* bias,
                 int32_t* topk_idx, float* topk_w, float* logits, void* ws, size_t ws_bytes, hipStream_t st) {
    return launch_route_prefetch(s, x, x_dtype, w, bias, topk_idx, topk_w, logits, ws, ws_bytes, st,
                                 CachePrefetch());
}

int launch_route_prefetch(const moe_shape& s, const void* x, int x_dtype, const void* w, const float* bias,
                          int32_t* topk_idx, float* topk_w, float* logits, void* ws, size_t ws_bytes,
                          hipStream_t st, CachePrefetch pf) {
    const size_t need = route_screen_bytes(s, x_dtype, x_dtype);
    const size_t tile_need = static_cast<size_t>(s.T) * s.E * sizeof(float);
    if (logits == nullptr && ws != nullptr && need > 0 && ws_bytes >= need) {
        launch_route_screened(s, static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w), bias, topk_idx,
                              topk_w, ws, st);
    } else if (tile_eligible(s, x_dtype) && (logits != nullptr || (ws != nullptr && ws_bytes >= tile_need))) {
        // the logits go to the caller's array, else to the workspace
        float* l = logits != nullptr ? logits : static_cast<float*>(ws);
        if (x_dtype == MOE_BF16)
            launch_tile<uint16_t>(s, static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w), bias, l,
                                  topk_idx, topk_w, pf, st);
        else
            launch_tile<float>(s, static_cast<const float*>(x), static_cast<const float*>(w), bias, l, topk_idx,
                               topk_w, pf, st);
    } else if (x_dtype == MOE_BF16)
        launch_route_dt<uint16_t>(s, static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w), bias,
                                  topk_idx, topk_w, logits, pf, st);
    else
        launch_route_dt<float>(s, static_cast<const float*>(x), static_cast<const float*>(w), bias, topk_idx,
                               topk_w, logits, pf, st);
    MOE_CHECK_LAUNCH();
    return MOE_OK;
}

int launch_route_from_logits(const moe_shape& s, const float* logits, int32_t* topk_idx, float* topk_w,
                             hipStream_t st) {
    const int grid = (s.T + kRouteWaves - 1) / kRouteWaves;
    if (s.E <= 64)
        hipLaunchKernelGGL(select_kernel<1>, dim3(grid), dim3(kRouteThreads), 0, st, logits, s.T, s.E, s.K,
                           topk_idx, topk_w);
    else if (s.E <= 128)
        hipLaunchKernelGGL(select_kernel<2>, dim3(grid), dim3(kRouteThreads), 0, st, logits, s.T, s.E, s.K,
                           topk_idx, topk_w);
    else if (s.E <= 256)
        hipLaunchKernelGGL(select_kernel<4>, dim3(grid), dim3(kRouteThreads), 0, st, logits, s.T, s.E, s.K,
                           topk_idx, topk_w);
    else
        hipLaunchKernelGGL(select_kernel<16>, dim3(grid), dim3(kRouteThreads), 0, st, logits, s.T, s.E, s.K,
                           topk_idx, topk_w);
    MOE_CHECK_LAUNCH();
    return MOE_OK;
}

}  // namespace moe
