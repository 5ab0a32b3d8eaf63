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
// issues little besides v_fma.  Large batches give each wave 3 tokens x all
// experts; small batches give each wave 1 token x 64 experts, the shortest
// dependent chain, with a deeper prefetch.  Larger E uses the generic kernel.  Selection happens in registers with wave-wide
// 64-bit max reductions over (orderable logit, ~expert) keys.
#include "common.hpp"

namespace moe {
namespace {

constexpr int kRouteThreads = 256;
constexpr int kRouteWaves = kRouteThreads / kWave;
constexpr int kLdsFloatsW = 8192;   // 32 KiB of float32 router-weight staging

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

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        uint32_t lo = __shfl_xor(static_cast<uint32_t>(v), off, kWave);
        uint32_t hi = __shfl_xor(static_cast<uint32_t>(v >> 32), off, kWave);
        uint64_t o = (static_cast<uint64_t>(hi) << 32) | lo;
        v = o > v ? o : v;
    }
    return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
    return v;
}

// Select the top K of the wave's E logits (lane holds experts g*64 + lane) and
// write indices and renormalised weights of token t.  Uniform control flow.
template <int NE>
__device__ __forceinline__ void select_and_write(const float (&l)[NE], int E, int K, int t,
                                                 int32_t* __restrict__ topk_idx, float* __restrict__ topk_w) {
    const int lane = threadIdx.x & (kWave - 1);
    uint64_t key[NE];
#pragma unroll
    for (int g = 0; g < NE; ++g) {
        const int e = g * kWave + lane;
        key[g] = e < E ? make_key(l[g], e) : 0ull;
    }
    int my_e = 0;
    float my_l = 0.0f;
    for (int k = 0; k < K; ++k) {
        uint64_t best = 0ull;
#pragma unroll
        for (int g = 0; g < NE; ++g) best = key[g] > best ? key[g] : best;
        best = wave_max_u64(best);
#pragma unroll
        for (int g = 0; g < NE; ++g)
            if (key[g] == best) key[g] = 0ull;
        if (lane == k) {
            my_e = key_expert(best);
            my_l = key_logit(best);
        }
    }
    const float l0 = __shfl(my_l, 0, kWave);
    const float ex = lane < K ? expf(my_l - l0) : 0.0f;
    const float sum = wave_sum(ex);
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

template <typename XT>
void launch_route_dt(const moe_shape& s, const XT* x, const XT* w, const float* bias, int32_t* idx,
                     float* tw, float* logits, hipStream_t st) {
    if (s.E <= 128) {
        if (s.T >= 2048) {
            // 8 waves x 3 tokens per workgroup: about two waves per SIMD at 6000 tokens
            if (s.E <= 64) launch_fast<XT, 3, 1, 1, 8, 32, 3>(s, x, w, bias, idx, tw, logits, st);
            else launch_fast<XT, 3, 2, 1, 8, 32, 3>(s, x, w, bias, idx, tw, logits, st);
        } else {
            // one chain per lane, deep prefetch: latency-bound small batches
            if (s.E <= 64) launch_fast<XT, 1, 1, 1, 8, 32, 8>(s, x, w, bias, idx, tw, logits, st);
            else launch_fast<XT, 1, 1, 2, 8, 32, 8>(s, x, w, bias, idx, tw, logits, st);
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

}  // namespace

int launch_route(const moe_shape& s, const void* x, int x_dtype, const void* w, const float* bias,
                 int32_t* topk_idx, float* topk_w, float* logits, hipStream_t st) {
    if (x_dtype == MOE_BF16)
        launch_route_dt<uint16_t>(s, static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w), bias,
                                  topk_idx, topk_w, logits, st);
    else
        launch_route_dt<float>(s, static_cast<const float*>(x), static_cast<const float*>(w), bias, topk_idx,
                               topk_w, logits, st);
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
