// Internal helpers shared by the HIP translation units of the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_layer_03_amd.h"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest, ties to even (inputs are finite).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

typedef _Float16 halfx8_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ float f16_to_f32(uint16_t b) {
    return static_cast<float>(__builtin_bit_cast(_Float16, b));
}

// Round to nearest even; saturates to +-65504 instead of overflowing to Inf.
__device__ __forceinline__ uint16_t f32_to_f16_sat(float f) {
    const _Float16 h = static_cast<_Float16>(fminf(fmaxf(f, -65504.0f), 65504.0f));
    return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
    return static_cast<uint32_t>(f32_to_f16_sat(lo)) | (static_cast<uint32_t>(f32_to_f16_sat(hi)) << 16);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return static_cast<uint32_t>(f32_to_bf16(lo)) | (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
}

// Asynchronous global -> LDS copies ------------------------------------------
//
// The compiler does not track which LDS bytes a direct-to-LDS copy writes, so
// kernels that use dma16() order them by hand: wait_vmcnt<N>() (at most N of
// this wave's vector-memory operations still in flight; they retire in order)
// followed by a workgroup barrier before the staged data is read.

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    // gfx9 s_waitcnt encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] at [15:14]
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Same with a wave-uniform run-time bound n, LO <= n < HI (a binary search
// over the immediate encodings: log2(HI - LO) scalar branches).
// Wait until this wave's LDS and scalar-memory operations are done (vmcnt untouched).
__device__ __forceinline__ void wait_lgkmcnt0() {
    __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));
}

template <int LO, int HI>
__device__ __forceinline__ void wait_vmcnt_bin(int n) {
    if constexpr (HI - LO == 1) {
        wait_vmcnt<LO>();
    } else {
        constexpr int MID = (LO + HI) / 2;
        if (n < MID) wait_vmcnt_bin<LO, MID>(n);
        else wait_vmcnt_bin<MID, HI>(n);
    }
}

// One 16-byte-per-lane global -> LDS copy: lane l's 16 bytes from g land at
// LDS address (wave-uniform base) + 16 * l.
__device__ __forceinline__ void dma16(const uint16_t* g, uint16_t* lds_wave_base) {
    __builtin_amdgcn_global_load_lds(g, reinterpret_cast<__attribute__((address_space(3))) void*>(
                                            reinterpret_cast<uintptr_t>(lds_wave_base)),
                                     16, 0, 0);
}

// Kernel launch bookkeeping -------------------------------------------------

// Records the hipError_t of a failed launch for moe_last_hip_error().
void set_last_hip_error(hipError_t e);

#define MOE_CHECK_LAUNCH()                                  \
    do {                                                    \
        hipError_t moe_err_ = hipGetLastError();            \
        if (moe_err_ != hipSuccess) {                       \
            ::moe::set_last_hip_error(moe_err_);            \
            return MOE_ERR_HIP;                             \
        }                                                   \
    } while (0)

#define MOE_TRY(expr)                                       \
    do {                                                    \
        int moe_st_ = (expr);                               \
        if (moe_st_ != MOE_OK) return moe_st_;              \
    } while (0)

// Launchers (defined in the kernel translation units).  Arguments are
// validated by the entry points before these are called.
size_t route_screen_bytes(const moe_shape& s, int x_dtype, int w_dtype);
// Scratch bytes that let the router take its faster paths: the screened path
// (large bf16 batches), or the tiled path's logits (small batches).
size_t route_workspace_bytes(const moe_shape& s);
// Where the screened path leaves its estimates in the workspace; false when
// the shape and dtypes do not take that path.
bool route_screen_layout(const moe_shape& s, int x_dtype, int w_dtype, moe_route_screen_info* info);
int launch_route(const moe_shape& s, const void* x, int x_dtype, const void* w, const float* bias,
                 int32_t* topk_idx, float* topk_w, float* logits, void* ws, size_t ws_bytes, hipStream_t st);
int launch_route_from_logits(const moe_shape& s, const float* logits, int32_t* topk_idx, float* topk_w,
                             hipStream_t st);

size_t dispatch_scratch_bytes(const moe_shape& s);
int launch_dispatch(const moe_shape& s, const int32_t* topk_idx, const void* x, int x_dtype,
                    int32_t* counts, int32_t* offsets, int32_t* row_token, int32_t* row_slot,
                    int32_t* slot_row, uint16_t* x_packed, void* scratch, hipStream_t st);

size_t packed_gate_up_elems(const moe_shape& s);
size_t packed_down_elems(const moe_shape& s);
int launch_pack_weights(const moe_shape& s, const void* w_gate, const void* w_up, const void* w_down,
                        int dtype, uint16_t* packed, hipStream_t st);
// Operand type of the MFMA products: bf16 weights keep bf16, float32 weights
// are converted to fp16; the down projection always runs in fp16.
inline int gate_up_operand_dtype(int weight_dtype) { return weight_dtype == MOE_BF16 ? MOE_BF16 : MOE_F16; }
// a_rows: NULL, or the row of `a` that packed row r reads (gather from the unpacked input)
int launch_grouped_gemm(const moe_shape& s, const uint16_t* a, int a_dtype, const int32_t* a_rows,
                        const int32_t* offsets, const uint16_t* packed, int which, int epilogue, void* c,
                        int c_dtype, hipStream_t st);
// Whether launch_grouped_gemm takes its weight-streaming form (few rows per
// expert); gather: the rows are read through a row-to-token map.
bool gemm_streams_weights(const moe_shape& s, int which, bool gather);
// Whether the gate/up launch below applies (bf16 rows gathered from x, weight
// streaming, at most 1024 tokens and 1024 local experts).
bool gemm_can_derive_dispatch(const moe_shape& s);
// Weight-streaming gate/up GEMM with the SwiGLU epilogue (fp16 h) that derives
// the dispatch from topk_idx itself and writes the dispatch outputs (counts,
// offsets, row_token, row_slot, slot_row) on the way: dispatch and gate/up in
// one launch.
int launch_gate_up_deriving_dispatch(const moe_shape& s, const uint16_t* x, const int32_t* topk_idx,
                                     const uint16_t* packed, uint16_t* h, int32_t* counts, int32_t* offsets,
                                     int32_t* row_token, int32_t* row_slot, int32_t* slot_row, hipStream_t st);

int launch_combine(const moe_shape& s, const void* y_packed, int y_dtype, const int32_t* slot_row,
                   const float* topk_w, float* out, hipStream_t st);

// MXFP8 (mxfp8.hip)
size_t mx_packed_gate_up_code_bytes(const moe_shape& s);
size_t mx_packed_down_code_bytes(const moe_shape& s);
size_t mx_packed_weight_bytes(const moe_shape& s);
int launch_mx_pack_weights(const moe_shape& s, const void* w_gate, const void* w_up, const void* w_down, int dtype,
                           uint8_t* packed, hipStream_t st);
int launch_mx_quantize(int64_t rows, int K, const void* x, int x_dtype, uint8_t* codes, uint8_t* scales,
                       hipStream_t st);
// Whether launch_mx_grouped_gemm takes its weight-streaming form.
bool mx_gemm_streams_weights(const moe_shape& s);
// Whether the gate/up launch below applies (weight streaming, at most 1024
// tokens and 1024 local experts, offsets within the buffer range).
bool mx_gemm_can_derive_dispatch(const moe_shape& s);
// Weight-streaming MXFP8 gate/up GEMM with the SwiGLU epilogue (MXFP8 h) that
// reads the quantised token rows [T][H] directly, derives the dispatch from
// topk_idx itself and writes the dispatch outputs on the way: dispatch and
// gate/up in one launch.
int launch_mx_gate_up_deriving_dispatch(const moe_shape& s, const uint8_t* x_codes, const uint8_t* x_scales,
                                        const int32_t* topk_idx, const uint8_t* packed, uint8_t* h_codes,
                                        uint8_t* h_scales, int32_t* counts, int32_t* offsets, int32_t* row_token,
                                        int32_t* row_slot, int32_t* slot_row, hipStream_t st);
int launch_mx_grouped_gemm(const moe_shape& s, const uint8_t* a, const uint8_t* a_scales, const int32_t* a_rows,
                           const int32_t* offsets, const uint8_t* packed, int which, int epilogue, void* c,
                           int c_dtype, uint8_t* c_scales, hipStream_t st);

}  // namespace moe
