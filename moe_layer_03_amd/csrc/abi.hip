// C-ABI entry points: argument validation on the host (before any HIP call),
// workspace carving and kernel sequencing.  Every entry point returns a
// status; nothing throws across the boundary.
#include <stdint.h>

#include <cstddef>
#include <mutex>

#include "common.hpp"
#include "route_prefetch.hpp"

// Workspace of moe_layer_noalloc: one copy per GPU, held by that GPU from the
// moment the library's code is loaded on it until the process ends.  In host
// code this name is only a handle for hipGetSymbolAddress, never an address.
__device__ __attribute__((aligned(256))) unsigned char scratch[MOE_LAYER_NOALLOC_MAX_WS_BYTES];

namespace moe {

namespace {
thread_local int32_t g_last_hip_error = 0;

// Device address of `scratch` on each GPU, resolved once per device (with that
// device current) on the first moe_layer_noalloc call there.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int scratch_of_current_device(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        g_last_hip_error = static_cast<int32_t>(e);
        return MOE_ERR_HIP;
    }
    if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || p == nullptr) {
            g_last_hip_error = static_cast<int32_t>(e != hipSuccess ? e : hipErrorInvalidSymbol);
            return MOE_ERR_HIP;
        }
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return MOE_OK;
}

inline size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

inline bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// 16-byte aligned, non-null bulk tensor
inline bool ok16(const void* p) { return p != nullptr && aligned(p, 16); }
// 4-byte aligned, non-null small array
inline bool ok4(const void* p) { return p != nullptr && aligned(p, 4); }
// optional 4-byte aligned array
inline bool opt4(const void* p) { return p == nullptr || aligned(p, 4); }

int check_shape(const moe_shape* s) {
    if (s == nullptr) return MOE_ERR_INVALID_ARG;
    if (s->T < 0 || s->H <= 0 || s->I <= 0) return MOE_ERR_INVALID_ARG;
    if (s->K < 1 || s->E < s->K || s->E > 1024) return MOE_ERR_INVALID_ARG;
    if (s->e_begin < 0 || s->e_begin >= s->e_end || s->e_end > s->E) return MOE_ERR_INVALID_ARG;
    if (static_cast<int64_t>(s->T) * s->K >= (int64_t(1) << 31)) return MOE_ERR_INVALID_ARG;
    if (s->H % 64 != 0 || s->I % 64 != 0 || s->K > 64) return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

inline bool dtype_ok(int d) { return d == MOE_F32 || d == MOE_BF16; }
inline bool out_dtype_ok(int d) { return d == MOE_F32 || d == MOE_BF16 || d == MOE_F16; }

inline int64_t cap_rows(const moe_shape& s) {
    const int E_loc = s.e_end - s.e_begin;
    return static_cast<int64_t>(s.T) * (s.K < E_loc ? s.K : E_loc);
}

// Workspace of moe_layer, in carve order.
struct LayerWs {
    int32_t* topk_idx;
    float* topk_w;
    int32_t* counts;
    int32_t* offsets;
    int32_t* row_token;
    int32_t* row_slot;
    int32_t* slot_row;
    void* dispatch_scratch;
    void* route_scratch;  // screened router (bf16 layers with 128 experts)
    size_t route_bytes;
    uint16_t* x_packed;
    uint16_t* h;      // SwiGLU activations, fp16
    uint16_t* y;      // expert outputs, fp16
    size_t bytes;
};

LayerWs carve_layer(const moe_shape& s, void* base) {
    const size_t TK = static_cast<size_t>(s.T) * s.K;
    const size_t E_loc = static_cast<size_t>(s.e_end - s.e_begin);
    const size_t cap = static_cast<size_t>(cap_rows(s));
    char* p = static_cast<char*>(base);
    size_t off = 0;
    auto take = [&](size_t bytes) -> char* {
        char* r = p ? p + off : nullptr;
        off += align256(bytes);
        return r;
    };
    LayerWs w;
    w.topk_idx = reinterpret_cast<int32_t*>(take(TK * 4));
    w.topk_w = reinterpret_cast<float*>(take(TK * 4));
    w.counts = reinterpret_cast<int32_t*>(take(E_loc * 4));
    w.offsets = reinterpret_cast<int32_t*>(take((E_loc + 1) * 4));
    w.row_token = reinterpret_cast<int32_t*>(take(cap * 4));
    w.row_slot = reinterpret_cast<int32_t*>(take(cap * 4));
    w.slot_row = reinterpret_cast<int32_t*>(take(TK * 4));
    w.dispatch_scratch = take(dispatch_scratch_bytes(s));
    w.route_bytes = route_workspace_bytes(s);
    w.route_scratch = take(w.route_bytes);
    w.x_packed = reinterpret_cast<uint16_t*>(take(cap * s.H * 2));
    w.h = reinterpret_cast<uint16_t*>(take(cap * s.I * 2));
    w.y = reinterpret_cast<uint16_t*>(take(cap * s.H * 2));
    w.bytes = off;
    return w;
}

// Workspace of moe_layer_mxfp8, in carve order.
struct MxLayerWs {
    int32_t* topk_idx;
    float* topk_w;
    int32_t* counts;
    int32_t* offsets;
    int32_t* row_token;
    int32_t* row_slot;
    int32_t* slot_row;
    void* dispatch_scratch;
    void* route_scratch;
    size_t route_bytes;
    uint8_t* x_codes;   // [T][H]
    uint8_t* x_scales;  // [T][H/32]
    uint8_t* h_codes;   // [cap][I]
    uint8_t* h_scales;  // [cap][I/32]
    uint16_t* y;        // [cap][H] fp16
    size_t bytes;
};

MxLayerWs carve_layer_mx(const moe_shape& s, void* base) {
    const size_t TK = static_cast<size_t>(s.T) * s.K;
    const size_t E_loc = static_cast<size_t>(s.e_end - s.e_begin);
    const size_t cap = static_cast<size_t>(cap_rows(s));
    const size_t T = static_cast<size_t>(s.T);
    char* p = static_cast<char*>(base);
    size_t off = 0;
    auto take = [&](size_t bytes) -> char* {
        char* r = p ? p + off : nullptr;
        off += align256(bytes);
        return r;
    };
    MxLayerWs w;
    w.topk_idx = reinterpret_cast<int32_t*>(take(TK * 4));
    w.topk_w = reinterpret_cast<float*>(take(TK * 4));
    w.counts = reinterpret_cast<int32_t*>(take(E_loc * 4));
    w.offsets = reinterpret_cast<int32_t*>(take((E_loc + 1) * 4));
    w.row_token = reinterpret_cast<int32_t*>(take(cap * 4));
    w.row_slot = reinterpret_cast<int32_t*>(take(cap * 4));
    w.slot_row = reinterpret_cast<int32_t*>(take(TK * 4));
    w.dispatch_scratch = take(dispatch_scratch_bytes(s));
    w.route_bytes = route_workspace_bytes(s);
    w.route_scratch = take(w.route_bytes);
    w.x_codes = reinterpret_cast<uint8_t*>(take(T * s.H));
    w.x_scales = reinterpret_cast<uint8_t*>(take(T * s.H / 32));
    w.h_codes = reinterpret_cast<uint8_t*>(take(cap * s.I));
    w.h_scales = reinterpret_cast<uint8_t*>(take(cap * s.I / 32));
    w.y = reinterpret_cast<uint16_t*>(take(cap * s.H * 2));
    w.bytes = off;
    return w;
}

// MXFP8 calls: H and I multiples of 256 (whole 64-k steps in groups of four).
int check_mx_shape(const moe_shape* s) {
    MOE_TRY(check_shape(s));
    if (s->H % 256 != 0 || s->I % 256 != 0) return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

}  // namespace

void set_last_hip_error(hipError_t e) { g_last_hip_error = static_cast<int32_t>(e); }

}  // namespace moe

using namespace moe;

extern "C" {

size_t moe_dispatch_workspace_bytes(const moe_shape* s) {
    if (check_shape(s) != MOE_OK) return 0;
    return dispatch_scratch_bytes(*s);
}

size_t moe_route_workspace_bytes(const moe_shape* s) {
    if (check_shape(s) != MOE_OK) return 0;
    return route_workspace_bytes(*s);
}

int moe_route_screen_layout(const moe_shape* s, int x_dtype, int w_dtype, moe_route_screen_info* info) {
    MOE_TRY(check_shape(s));
    if (info == nullptr) return MOE_ERR_INVALID_ARG;
    if (!dtype_ok(x_dtype) || !dtype_ok(w_dtype)) return MOE_ERR_UNSUPPORTED;
    return route_screen_layout(*s, x_dtype, w_dtype, info) ? MOE_OK : MOE_ERR_UNSUPPORTED;
}

size_t moe_layer_workspace_bytes(const moe_shape* s) {
    if (check_shape(s) != MOE_OK) return 0;
    return carve_layer(*s, nullptr).bytes;
}

size_t moe_packed_weight_bytes(const moe_shape* s) {
    if (check_shape(s) != MOE_OK) return 0;
    return (packed_gate_up_elems(*s) + packed_down_elems(*s)) * sizeof(uint16_t);
}

int moe_pack_weights(const moe_shape* s, const void* w_gate, const void* w_up, const void* w_down, int dtype,
                     void* packed, void* stream) {
    MOE_TRY(check_shape(s));
    if (!dtype_ok(dtype)) return MOE_ERR_UNSUPPORTED;
    if (!ok16(w_gate) || !ok16(w_up) || !ok16(w_down) || !ok16(packed)) return MOE_ERR_INVALID_ARG;
    return launch_pack_weights(*s, w_gate, w_up, w_down, dtype, static_cast<uint16_t*>(packed),
                               static_cast<hipStream_t>(stream));
}

int moe_route(const moe_shape* s, const void* x, int x_dtype, const void* w_router, int w_dtype, const float* bias,
              int32_t* topk_idx, float* topk_w, float* logits, void* ws, size_t ws_bytes, void* stream) {
    MOE_TRY(check_shape(s));
    if (!dtype_ok(x_dtype) || !dtype_ok(w_dtype)) return MOE_ERR_UNSUPPORTED;
    if (x_dtype != w_dtype) return MOE_ERR_UNSUPPORTED;
    if (ws != nullptr) {
        if (!aligned(ws, 16)) return MOE_ERR_INVALID_ARG;
        if (ws_bytes < route_workspace_bytes(*s)) return MOE_ERR_WORKSPACE;
    }
    if (s->T == 0) return MOE_OK;   // nothing to route; empty tensors may have null pointers
    if (!ok16(x) || !ok16(w_router) || !ok4(topk_idx) || !ok4(topk_w) || !opt4(bias) || !opt4(logits))
        return MOE_ERR_INVALID_ARG;
    return launch_route(*s, x, x_dtype, w_router, bias, topk_idx, topk_w, logits, ws, ws_bytes,
                        static_cast<hipStream_t>(stream));
}

int moe_route_from_logits(const moe_shape* s, const float* logits, int32_t* topk_idx, float* topk_w,
                          void* stream) {
    MOE_TRY(check_shape(s));
    if (s->T == 0) return MOE_OK;
    if (!ok4(logits) || !ok4(topk_idx) || !ok4(topk_w)) return MOE_ERR_INVALID_ARG;
    return launch_route_from_logits(*s, logits, topk_idx, topk_w, static_cast<hipStream_t>(stream));
}

int moe_dispatch(const moe_shape* s, const int32_t* topk_idx, const void* x, int x_dtype, int32_t* counts,
                 int32_t* offsets, int32_t* row_token, int32_t* row_slot, int32_t* slot_row, uint16_t* x_packed,
                 void* ws, size_t ws_bytes, void* stream) {
    MOE_TRY(check_shape(s));
    if (!ok4(counts) || !ok4(offsets)) return MOE_ERR_INVALID_ARG;
    if ((x == nullptr) != (x_packed == nullptr)) return MOE_ERR_INVALID_ARG;
    if (s->T > 0 && (!ok4(topk_idx) || !ok4(row_token) || !ok4(row_slot) || !ok4(slot_row)))
        return MOE_ERR_INVALID_ARG;
    if (x != nullptr && s->T > 0) {
        if (!dtype_ok(x_dtype)) return MOE_ERR_UNSUPPORTED;
        if (!ok16(x) || !ok16(x_packed)) return MOE_ERR_INVALID_ARG;
    }
    const size_t need = dispatch_scratch_bytes(*s);
    if (ws_bytes < need) return MOE_ERR_WORKSPACE;
    if (need > 0 && !ok16(ws)) return MOE_ERR_INVALID_ARG;
    return launch_dispatch(*s, topk_idx, x, x_dtype, counts, offsets, row_token, row_slot, slot_row, x_packed, ws,
                           static_cast<hipStream_t>(stream));
}

int moe_grouped_gemm(const moe_shape* s, const uint16_t* a, int a_dtype, const int32_t* a_rows, const int32_t* offsets,
                     const void* packed, int which, int epilogue, void* c, int c_dtype, void* stream) {
    MOE_TRY(check_shape(s));
    if (which != MOE_GEMM_GATE_UP && which != MOE_GEMM_DOWN) return MOE_ERR_INVALID_ARG;
    if (epilogue != MOE_EPI_NONE && epilogue != MOE_EPI_SWIGLU) return MOE_ERR_INVALID_ARG;
    if (which == MOE_GEMM_DOWN && epilogue != MOE_EPI_NONE) return MOE_ERR_INVALID_ARG;
    if (!out_dtype_ok(c_dtype)) return MOE_ERR_UNSUPPORTED;
    if (which == MOE_GEMM_GATE_UP && a_dtype != MOE_BF16 && a_dtype != MOE_F16) return MOE_ERR_UNSUPPORTED;
    if (which == MOE_GEMM_DOWN && a_dtype != MOE_F16) return MOE_ERR_UNSUPPORTED;
    if (s->T == 0) return MOE_OK;
    if (!ok16(a) || !opt4(a_rows) || !ok4(offsets) || !ok16(packed) || !ok16(c)) return MOE_ERR_INVALID_ARG;
    return launch_grouped_gemm(*s, a, a_dtype, a_rows, offsets, static_cast<const uint16_t*>(packed), which,
                               epilogue, c, c_dtype, static_cast<hipStream_t>(stream));
}

int moe_combine(const moe_shape* s, const void* y_packed, int y_dtype, const int32_t* slot_row, const float* topk_w,
                float* out, void* stream) {
    MOE_TRY(check_shape(s));
    if (!out_dtype_ok(y_dtype)) return MOE_ERR_UNSUPPORTED;
    if (s->T == 0) return MOE_OK;
    if (!ok16(y_packed) || !ok4(slot_row) || !ok4(topk_w) || !ok16(out)) return MOE_ERR_INVALID_ARG;
    return launch_combine(*s, y_packed, y_dtype, slot_row, topk_w, out, static_cast<hipStream_t>(stream));
}

int moe_layer(const moe_shape* s, const void* x, int x_dtype, const void* w_router, int w_dtype, const float* bias,
              const void* packed, float* out, int32_t* topk_idx, float* topk_w, int32_t* counts, int32_t* offsets,
              int32_t* row_token, int32_t* row_slot, int32_t* slot_row, void* ws, size_t ws_bytes, void* stream) {
    MOE_TRY(check_shape(s));
    if (!dtype_ok(x_dtype) || !dtype_ok(w_dtype)) return MOE_ERR_UNSUPPORTED;
    if (x_dtype != w_dtype) return MOE_ERR_UNSUPPORTED;
    if (!opt4(topk_idx) || !opt4(topk_w) || !opt4(counts) || !opt4(offsets) || !opt4(row_token) ||
        !opt4(row_slot) || !opt4(slot_row))
        return MOE_ERR_INVALID_ARG;
    const size_t need = carve_layer(*s, nullptr).bytes;
    if (ws_bytes < need) return MOE_ERR_WORKSPACE;
    if (!ok16(ws)) return MOE_ERR_INVALID_ARG;
    if (s->T == 0) {
        // no tokens: only the per-expert counts and offsets (all zero) are produced
        if (counts == nullptr && offsets == nullptr) return MOE_OK;
        LayerWs w = carve_layer(*s, ws);
        return launch_dispatch(*s, nullptr, nullptr, x_dtype, counts ? counts : w.counts,
                               offsets ? offsets : w.offsets, nullptr, nullptr, nullptr, nullptr, w.dispatch_scratch,
                               static_cast<hipStream_t>(stream));
    }
    if (!ok16(x) || !ok16(w_router) || !ok16(packed) || !ok16(out) || !opt4(bias)) return MOE_ERR_INVALID_ARG;

    hipStream_t st = static_cast<hipStream_t>(stream);
    LayerWs w = carve_layer(*s, ws);
    int32_t* idx = topk_idx ? topk_idx : w.topk_idx;
    float* tw = topk_w ? topk_w : w.topk_w;
    int32_t* cnt = counts ? counts : w.counts;
    int32_t* off = offsets ? offsets : w.offsets;
    int32_t* rt = row_token ? row_token : w.row_token;
    int32_t* rs = row_slot ? row_slot : w.row_slot;
    int32_t* sr = slot_row ? slot_row : w.slot_row;

    const uint16_t* pk = static_cast<const uint16_t*>(packed);
    // Few rows per expert: the gate/up GEMM after routing streams its weights
    // from HBM and the router leaves most CUs idle, so those CUs read the
    // gate/up weights into the last-level cache meanwhile (when they fit).
    CachePrefetch pf;
    const size_t gu_bytes = packed_gate_up_elems(*s) * 2;
    if (gemm_streams_weights(*s, MOE_GEMM_GATE_UP, x_dtype == MOE_BF16) && gu_bytes <= kLastLevelCacheBytes) {
        pf.region = pk;
        pf.bytes = gu_bytes;
    }
    MOE_TRY(launch_route_prefetch(*s, x, x_dtype, w_router, bias, idx, tw, nullptr, w.route_scratch, w.route_bytes,
                                  st, pf));
    // bf16 layers multiply in bf16 (exact inputs) and the gate/up GEMM gathers
    // the token rows straight from x; float32 layers pack the rows as fp16
    // first.  The SwiGLU activations and expert outputs are fp16: rounding them
    // to bf16 instead would cost about 2% of the output RMS in the largest
    // elements.
    const int op = gate_up_operand_dtype(x_dtype);
    if (x_dtype == MOE_BF16 && gemm_can_derive_dispatch(*s)) {
        // few rows per expert: the weight-streaming gate/up GEMM derives the
        // dispatch itself (one launch fewer) and writes its outputs on the way
        MOE_TRY(launch_gate_up_deriving_dispatch(*s, static_cast<const uint16_t*>(x), idx, pk, w.h, cnt, off, rt, rs,
                                                 sr, st));
    } else if (x_dtype == MOE_BF16) {
        MOE_TRY(launch_dispatch(*s, idx, nullptr, x_dtype, cnt, off, rt, rs, sr, nullptr, w.dispatch_scratch, st));
        MOE_TRY(launch_grouped_gemm(*s, static_cast<const uint16_t*>(x), op, rt, off, pk, MOE_GEMM_GATE_UP,
                                    MOE_EPI_SWIGLU, w.h, MOE_F16, st));
    } else {
        MOE_TRY(launch_dispatch(*s, idx, x, x_dtype, cnt, off, rt, rs, sr, w.x_packed, w.dispatch_scratch, st));
        MOE_TRY(launch_grouped_gemm(*s, w.x_packed, op, nullptr, off, pk, MOE_GEMM_GATE_UP, MOE_EPI_SWIGLU, w.h,
                                    MOE_F16, st));
    }
    MOE_TRY(launch_grouped_gemm(*s, w.h, MOE_F16, nullptr, off, pk, MOE_GEMM_DOWN, MOE_EPI_NONE, w.y, MOE_F16, st));
    MOE_TRY(launch_combine(*s, w.y, MOE_F16, sr, tw, out, st));
    return MOE_OK;
}

size_t moe_packed_weight_bytes_mxfp8(const moe_shape* s) {
    if (check_mx_shape(s) != MOE_OK) return 0;
    return mx_packed_weight_bytes(*s);
}

int moe_pack_weights_mxfp8(const moe_shape* s, const void* w_gate, const void* w_up, const void* w_down, int dtype,
                           void* packed, void* stream) {
    MOE_TRY(check_mx_shape(s));
    if (!dtype_ok(dtype)) return MOE_ERR_UNSUPPORTED;
    if (!ok16(w_gate) || !ok16(w_up) || !ok16(w_down) || !ok16(packed)) return MOE_ERR_INVALID_ARG;
    return launch_mx_pack_weights(*s, w_gate, w_up, w_down, dtype, static_cast<uint8_t*>(packed),
                                  static_cast<hipStream_t>(stream));
}

int moe_quantize_mxfp8(int64_t rows, int32_t K, const void* x, int x_dtype, uint8_t* codes, uint8_t* scales,
                       void* stream) {
    if (rows < 0 || K <= 0 || K % 32 != 0) return MOE_ERR_INVALID_ARG;
    if (!dtype_ok(x_dtype)) return MOE_ERR_UNSUPPORTED;
    if (rows == 0) return MOE_OK;
    if (!ok16(x) || !ok16(codes) || scales == nullptr) return MOE_ERR_INVALID_ARG;
    return launch_mx_quantize(rows, K, x, x_dtype, codes, scales, static_cast<hipStream_t>(stream));
}

int moe_grouped_gemm_mxfp8(const moe_shape* s, const uint8_t* a, const uint8_t* a_scales, const int32_t* a_rows,
                           const int32_t* offsets, const void* packed, int which, int epilogue, void* c, int c_dtype,
                           uint8_t* c_scales, void* stream) {
    MOE_TRY(check_mx_shape(s));
    if (which != MOE_GEMM_GATE_UP && which != MOE_GEMM_DOWN) return MOE_ERR_INVALID_ARG;
    if (epilogue != MOE_EPI_NONE && epilogue != MOE_EPI_SWIGLU) return MOE_ERR_INVALID_ARG;
    if (which == MOE_GEMM_DOWN && epilogue != MOE_EPI_NONE) return MOE_ERR_INVALID_ARG;
    if (!out_dtype_ok(c_dtype) && !(c_dtype == MOE_MXFP8 && epilogue == MOE_EPI_SWIGLU)) return MOE_ERR_UNSUPPORTED;
    if (s->T == 0) return MOE_OK;
    if (!ok16(a) || a_scales == nullptr || !opt4(a_rows) || !ok4(offsets) || !ok16(packed) || !ok16(c))
        return MOE_ERR_INVALID_ARG;
    if (c_dtype == MOE_MXFP8 && c_scales == nullptr) return MOE_ERR_INVALID_ARG;
    return launch_mx_grouped_gemm(*s, a, a_scales, a_rows, offsets, static_cast<const uint8_t*>(packed), which,
                                  epilogue, c, c_dtype, c_scales, static_cast<hipStream_t>(stream));
}

size_t moe_layer_workspace_bytes_mxfp8(const moe_shape* s) {
    if (check_mx_shape(s) != MOE_OK) return 0;
    return carve_layer_mx(*s, nullptr).bytes;
}

int moe_layer_mxfp8(const moe_shape* s, const void* x, int x_dtype, const void* w_router, int w_dtype,
                    const float* bias, const void* packed, float* out, int32_t* topk_idx, float* topk_w,
                    int32_t* counts, int32_t* offsets, int32_t* row_token, int32_t* row_slot, int32_t* slot_row,
                    void* ws, size_t ws_bytes, void* stream) {
    MOE_TRY(check_mx_shape(s));
    if (!dtype_ok(x_dtype) || !dtype_ok(w_dtype)) return MOE_ERR_UNSUPPORTED;
    if (x_dtype != w_dtype) return MOE_ERR_UNSUPPORTED;
    if (!opt4(topk_idx) || !opt4(topk_w) || !opt4(counts) || !opt4(offsets) || !opt4(row_token) ||
        !opt4(row_slot) || !opt4(slot_row))
        return MOE_ERR_INVALID_ARG;
    if (ws_bytes < carve_layer_mx(*s, nullptr).bytes) return MOE_ERR_WORKSPACE;
    if (!ok16(ws)) return MOE_ERR_INVALID_ARG;
    hipStream_t st = static_cast<hipStream_t>(stream);
    MxLayerWs w = carve_layer_mx(*s, ws);
    int32_t* cnt = counts ? counts : w.counts;
    int32_t* off = offsets ? offsets : w.offsets;
    if (s->T == 0) {
        if (counts == nullptr && offsets == nullptr) return MOE_OK;
        return launch_dispatch(*s, nullptr, nullptr, x_dtype, cnt, off, nullptr, nullptr, nullptr, nullptr,
                               w.dispatch_scratch, st);
    }
    if (!ok16(x) || !ok16(w_router) || !ok16(packed) || !ok16(out) || !opt4(bias)) return MOE_ERR_INVALID_ARG;
    int32_t* idx = topk_idx ? topk_idx : w.topk_idx;
    float* tw = topk_w ? topk_w : w.topk_w;
    int32_t* rt = row_token ? row_token : w.row_token;
    int32_t* rs = row_slot ? row_slot : w.row_slot;
    int32_t* sr = slot_row ? slot_row : w.slot_row;
    const uint8_t* pk = static_cast<const uint8_t*>(packed);
    // few rows per expert: the router's idle CUs read the gate/up weight codes into the last-level cache
    CachePrefetch pf;
    const size_t gu_bytes = mx_packed_gate_up_code_bytes(*s);
    if (mx_gemm_streams_weights(*s) && gu_bytes <= kLastLevelCacheBytes) {
        pf.region = pk;
        pf.bytes = gu_bytes;
    }
    MOE_TRY(launch_route_prefetch(*s, x, x_dtype, w_router, bias, idx, tw, nullptr, w.route_scratch, w.route_bytes,
                                  st, pf));
    MOE_TRY(launch_mx_quantize(s->T, s->H, x, x_dtype, w.x_codes, w.x_scales, st));
    if (mx_gemm_can_derive_dispatch(*s)) {
        // few rows per expert: the weight-streaming gate/up GEMM derives the
        // dispatch itself (one launch fewer) and writes its outputs on the way
        MOE_TRY(launch_mx_gate_up_deriving_dispatch(*s, w.x_codes, w.x_scales, idx, pk, w.h_codes, w.h_scales, cnt,
                                                    off, rt, rs, sr, st));
    } else {
        MOE_TRY(launch_dispatch(*s, idx, nullptr, x_dtype, cnt, off, rt, rs, sr, nullptr, w.dispatch_scratch, st));
        MOE_TRY(launch_mx_grouped_gemm(*s, w.x_codes, w.x_scales, rt, off, pk, MOE_GEMM_GATE_UP, MOE_EPI_SWIGLU,
                                       w.h_codes, MOE_MXFP8, w.h_scales, st));
    }
    MOE_TRY(launch_mx_grouped_gemm(*s, w.h_codes, w.h_scales, nullptr, off, pk, MOE_GEMM_DOWN, MOE_EPI_NONE, w.y,
                                   MOE_F16, nullptr, st));
    MOE_TRY(launch_combine(*s, w.y, MOE_F16, sr, tw, out, st));
    return MOE_OK;
}

int moe_layer_noalloc(const moe_shape* s, const void* x, int x_dtype, const void* w_router, int w_dtype,
                      const float* bias, const void* packed, float* out, int32_t* topk_idx, float* topk_w,
                      int32_t* counts, int32_t* offsets, int32_t* row_token, int32_t* row_slot, int32_t* slot_row,
                      void* stream) {
    MOE_TRY(check_shape(s));
    if (carve_layer(*s, nullptr).bytes > MOE_LAYER_NOALLOC_MAX_WS_BYTES) return MOE_ERR_WORKSPACE;
    void* ws = nullptr;
    MOE_TRY(scratch_of_current_device(&ws));
    return moe_layer(s, x, x_dtype, w_router, w_dtype, bias, packed, out, topk_idx, topk_w, counts, offsets,
                     row_token, row_slot, slot_row, ws, MOE_LAYER_NOALLOC_MAX_WS_BYTES, stream);
}

const char* moe_status_string(int status) {
    switch (status) {
        case MOE_OK: return "MOE_OK";
        case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG: bad shape, range, null or misaligned pointer";
        case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: valid request outside what is implemented";
        case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace smaller than required";
        case MOE_ERR_HIP: return "MOE_ERR_HIP: a HIP call failed (see moe_last_hip_error)";
        default: return "unknown status";
    }
}

int32_t moe_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
