/*
 * moe_layer_03_amd -- one expert-parallel rank's share of a Mixture-of-Experts
 * layer on AMD Instinct MI355X (gfx950), as a C ABI.
 *
 * The operation is the one "Hosting Qwen on Blackwell" (Perplexity) states
 * for its prefill expert-parallel kernel (section "Expert Parallel") and its
 * dispatch/combine pair (section "MoE Dispatch - Combine"): every rank holds
 * all T tokens; the router sends each token to K of E experts (128 experts,
 * 8 per token in section "Pre-remplisseurs"); the rank selects the tokens
 * routed to its own experts [e_begin, e_end), packs them into per-expert
 * contiguous buffers, runs one GEMM problem per local expert (section
 * "MoE GEMM"), and accumulates the weighted expert outputs back in token
 * order.  That local sum is the rank's partial output; adding the partial
 * outputs of all ranks (an all-reduce) is outside this library.
 *
 * Readings of what the pages leave open (the router function, the expert
 * activation, orders, precision) are fixed here and stated per call.
 *
 * Conventions for every call
 *   - Tensor pointers are DEVICE pointers (HIP device memory), row-major,
 *     owned by the caller, 16-byte aligned.  The library never allocates
 *     or frees memory.  Its global state is a per-thread copy of the last
 *     HIP error code and, for moe_layer_noalloc, one static workspace array
 *     per GPU with its device address cached per device.
 *   - `stream` is a hipStream_t passed as void* (NULL: the null stream).
 *     A call only enqueues work on it and returns; outputs are valid once
 *     the stream has synchronised, and inputs must stay alive until then.
 *   - Arguments are validated on the host before any HIP call; an invalid
 *     call returns an error status and enqueues nothing.
 *   - Non-finite inputs (NaN, Inf) are outside the contract.
 *   - bf16 tensors are raw bfloat16 bit patterns in uint16_t storage.
 */
#ifndef MOE_LAYER_03_AMD_H
#define MOE_LAYER_03_AMD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define MOE_OK               0
#define MOE_ERR_INVALID_ARG (-1)   /* bad shape, range, null or misaligned pointer */
#define MOE_ERR_UNSUPPORTED (-2)   /* valid but not implemented (dtype mix, H or I not a multiple of 64, K > 64) */
#define MOE_ERR_WORKSPACE   (-3)   /* ws_bytes smaller than the matching *_workspace_bytes() */
#define MOE_ERR_HIP         (-4)   /* a HIP launch failed; see moe_last_hip_error() */

/* Element types.  MOE_F16 appears only for intermediates and GEMM outputs;
 * MOE_MXFP8 only for MXFP8 GEMM outputs (codes plus scales, see below). */
#define MOE_F32   0
#define MOE_BF16  1
#define MOE_F16   2
#define MOE_MXFP8 3

/* Grouped-GEMM operand selector and epilogues. */
#define MOE_GEMM_GATE_UP 0   /* A = packed tokens [*, H], B = gate and up weights of each expert  */
#define MOE_GEMM_DOWN    1   /* A = SwiGLU activations [*, I], B = down weights of each expert    */
#define MOE_EPI_NONE     0   /* C = A.B (gate/up: columns 0..I-1 gate, I..2I-1 up)                 */
#define MOE_EPI_SWIGLU   1   /* C = silu(A.Wg) * (A.Wu), silu(z) = z / (1 + exp(-z)); gate/up only */

/*
 * Problem shape of one rank.
 *   T tokens, H hidden size, E experts in the layer, K experts per token,
 *   I expert intermediate size, local experts [e_begin, e_end).
 * Limits: T >= 0 (T == 0 makes every call a no-op), 1 <= K <= E <= 1024,
 * K <= 64, 0 <= e_begin < e_end <= E, H >= 64 and I >= 64 and both
 * multiples of 64, T * K < 2^31.
 * E_loc = e_end - e_begin.  cap = T * min(K, E_loc) bounds the number of
 * (token, slot) pairs that can be routed to local experts; buffers indexed by
 * packed row are sized by cap, and only the first N_loc = offsets[E_loc]
 * rows are meaningful.
 */
typedef struct moe_shape {
    int32_t T, H, E, K, I, e_begin, e_end;
} moe_shape;

/* Bytes of scratch memory moe_dispatch() needs (host-only, no HIP call). */
size_t moe_dispatch_workspace_bytes(const moe_shape* s);

/*
 * Bytes of scratch memory that let moe_route() take its faster paths
 * (host-only, no HIP call), the larger of:
 *   the screened path: bf16 inputs, E == 128, T >= 512, H a multiple of 128
 *     and at most 65536, no logits output;
 *   the tiled small-batch path: T <= 1024, E a multiple of 8 (bf16) or 4
 *     (float32), H a multiple of 256: T * E * 4 bytes of logits (not needed
 *     when the caller asks for logits).
 * 0 when the shape takes neither.
 */
size_t moe_route_workspace_bytes(const moe_shape* s);

/*
 * Where the screened path of moe_route() leaves its estimates in the
 * workspace (host-only, no HIP call).  For callers that check the error bound
 * on which the screening's exactness rests.
 *
 * After moe_route() ran with ws != NULL on a shape that takes the screened
 * path, and its stream has synchronised, ws holds at these byte offsets
 * (S = slices; slice s covers h in [s*H/S, (s+1)*H/S)):
 *   part_offset: float32 [S][T][E], the bf16-MFMA estimate of slice s of
 *                sum_h x[t,h] * w_router[h,e] (each 64-h chunk summed by MFMA
 *                from zero, the chunk sums added in float32 in ascending h);
 *   nx_offset:   float32 [S][T], sum over slice s of x[t,h]^2;
 *   nw_offset:   float32 [S][E], sum over slice s of w_router[h,e]^2.
 * With u = 2^-24 and Hu = H*u, the router then forms, in float32 and in this
 * order:
 *   A[t,e] = ((part[0] + part[1]) + ...) + part[S-1], plus bias[e] if given;
 *   nX = sum_s nx[s][t], nW = sum_s nw[s][e] (ascending s);
 *   D[t,e] = ((1.0625 H + 192) u) (sqrt(nX) (1 + 3 Hu) sqrt(nW))
 *            + 2^-21 |A| + 1e-30;
 * and its selection is exact because |A[t,e] - L[t,e]| <= D[t,e] for the
 * canonical logit L of moe_route().  Returns MOE_ERR_UNSUPPORTED when
 * (s, x_dtype, w_dtype) does not take the screened path.
 */
typedef struct moe_route_screen_info {
    int32_t slices;
    size_t part_offset, nx_offset, nw_offset;
    size_t bytes;        /* == moe_route_workspace_bytes(s) */
} moe_route_screen_info;
int moe_route_screen_layout(const moe_shape* s, int x_dtype, int w_dtype, moe_route_screen_info* info);

/* Bytes of scratch memory moe_layer() needs (host-only, no HIP call). */
size_t moe_layer_workspace_bytes(const moe_shape* s);

/* Bytes of the packed expert weights of the E_loc local experts (host-only). */
size_t moe_packed_weight_bytes(const moe_shape* s);

/*
 * moe_pack_weights -- static conversion of the local experts' weights into
 * the layout the grouped GEMM streams (the pages convert their weights
 * statically once, section "Quantification").  Run once, outside any timed
 * region.
 *   w_gate [E_loc, H, I], w_up [E_loc, H, I], w_down [E_loc, I, H]: the
 *   expert FFN is y = (silu(x Wg) * (x Wu)) Wd; dtype MOE_BF16 or MOE_F32.
 *   Gate and up weights keep bf16 (bf16 input) or are rounded to fp16
 *   (float32 input); down weights are converted to fp16 (exact for bf16
 *   values of magnitude 2^-17 .. 65504; fp16 conversions saturate at 65504).
 *   packed: moe_packed_weight_bytes(s) bytes, written; opaque layout.
 */
int moe_pack_weights(const moe_shape* s, const void* w_gate, const void* w_up, const void* w_down,
                     int dtype, void* packed, void* stream);

/*
 * moe_route -- router logits, softmax over the E experts, top-K, renormalised
 * ("Pre-remplisseurs": each token is routed to 8 of the 128 experts; the pages
 * do not name the router function, this library takes softmax -> top-K ->
 * renormalise).
 *   x [T, H], w_router [H, E]: both MOE_F32 or both MOE_BF16.
 *   bias [E] float32 or NULL: added to each logit after the dot product.
 *   logits (output, optional) [T, E] float32:
 *       l[t,e] = fma-chain over h = 0..H-1 ascending, starting from +0.0f,
 *       acc = fmaf(x[t,h], w_router[h,e], acc); then acc + bias[e].
 *       This order is part of the definition: it decides near-ties.
 *   topk_idx (output) [T, K] int32: the K largest logits, slot 0 the largest,
 *       equal logits (-0 == +0) ordered by ascending expert index.
 *   topk_w (output) [T, K] float32: exp(l_j - l_0) / sum_i exp(l_i - l_0)
 *       over the chosen K, i.e. the softmax probabilities renormalised.
 *   ws, ws_bytes: scratch memory, or NULL.  With ws != NULL (16-byte aligned,
 *       ws_bytes >= moe_route_workspace_bytes(s), else MOE_ERR_WORKSPACE) and
 *       a large bf16 batch, logits are first estimated with bf16 MFMA and
 *       only the experts a rigorous error bound cannot exclude from the top K
 *       are evaluated in the fma chain above; a small batch writes its logits
 *       to ws (or to logits) and selects from them.  The outputs are
 *       identical on every path, which is what happens with ws == NULL.
 */
int moe_route(const moe_shape* s, const void* x, int x_dtype, const void* w_router, int w_dtype,
              const float* bias, int32_t* topk_idx, float* topk_w, float* logits, void* ws, size_t ws_bytes,
              void* stream);

/*
 * moe_route_from_logits -- the selection and weighting step of moe_route on
 * caller-supplied logits [T, E] float32 (same outputs, same rules).
 */
int moe_route_from_logits(const moe_shape* s, const float* logits, int32_t* topk_idx, float* topk_w,
                          void* stream);

/*
 * moe_dispatch -- select the (token, slot) pairs routed to local experts and
 * pack the tokens per expert ("Expert Parallel": the inputs are replicated on
 * every rank, so dispatch only selects the tokens routed to the rank's
 * experts, aggregates the routing information and prepares the GEMM input
 * buffers).
 *   topk_idx [T, K] int32 (from moe_route).  Precondition: a token lists an
 *       expert at most once (moe_route guarantees it); a row that repeats a
 *       local expert gives undefined counts and row maps.
 *   counts (output) [E_loc] int32: pairs routed to expert e_begin + i.
 *   offsets (output) [E_loc + 1] int32: exclusive prefix sum of counts.
 *   row_token, row_slot (output) [cap] int32: token and slot of packed row r;
 *       an expert's rows are in ascending token order, experts ascending.
 *   slot_row (output) [T, K] int32: packed row of (t, j), -1 if not local.
 *   x [T, H] (MOE_F32 or MOE_BF16) and x_packed (output) [cap, H]:
 *       x_packed[r] = x[row_token[r]] in the GEMM operand type -- a bf16 copy
 *       of bf16 x, fp16 (nearest-even, saturating) for float32 x; both NULL
 *       to skip the pack.
 *   ws: moe_dispatch_workspace_bytes(s) bytes of device scratch.
 */
int moe_dispatch(const moe_shape* s, const int32_t* topk_idx, const void* x, int x_dtype,
                 int32_t* counts, int32_t* offsets, int32_t* row_token, int32_t* row_slot,
                 int32_t* slot_row, uint16_t* x_packed, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_grouped_gemm -- one GEMM problem per local expert over its packed rows
 * ("MoE GEMM"); rows [offsets[i], offsets[i+1]) use expert e_begin + i.
 *   which = MOE_GEMM_GATE_UP: a_dtype MOE_BF16 for weights packed from bf16,
 *       MOE_F16 for weights packed from float32; epilogue MOE_EPI_SWIGLU ->
 *       c [cap, I], or MOE_EPI_NONE -> c [cap, 2I] (gate columns then up
 *       columns).
 *   which = MOE_GEMM_DOWN: a [cap, I] fp16 (a_dtype MOE_F16); epilogue
 *       MOE_EPI_NONE -> c [cap, H].
 *   a_rows: NULL, then a holds the packed rows ([cap, Kd]); or [cap] int32,
 *       then packed row r is row a_rows[r] of a, 0 <= a_rows[r] < T (for
 *       instance a = x [T, H] and a_rows = the row_token of moe_dispatch: no
 *       packed copy needed).
 *   c_dtype MOE_F32, MOE_BF16 or MOE_F16 (16-bit outputs round to nearest
 *   even; fp16 saturates at 65504); products accumulate in float32.  Rows
 *   >= N_loc are not written.
 *   packed: the buffer moe_pack_weights() wrote for the same shape.
 *   offsets [E_loc + 1] int32, on the device (counts never visit the host).
 */
int moe_grouped_gemm(const moe_shape* s, const uint16_t* a, int a_dtype, const int32_t* a_rows,
                     const int32_t* offsets, const void* packed, int which, int epilogue, void* c, int c_dtype,
                     void* stream);

/*
 * moe_combine -- weighted local accumulation back to token order
 * ("MoE Dispatch - Combine", "Expert Parallel": the combine kernel first
 * accumulates the contributions of the experts on the current rank).
 *   out[t, :] = sum over j = 0..K-1 ascending with slot_row[t,j] >= 0 of
 *               topk_w[t,j] * y_packed[slot_row[t,j], :], in float32.
 *   Rows of tokens with no local expert are written as zeros.
 *   y_packed [cap, H], y_dtype MOE_F16, MOE_BF16 or MOE_F32; slot_row [T, K] int32,
 *   topk_w [T, K] float32,
 *   out (output) [T, H] float32, fully overwritten.
 */
int moe_combine(const moe_shape* s, const void* y_packed, int y_dtype, const int32_t* slot_row, const float* topk_w,
                float* out, void* stream);

/*
 * moe_layer -- route, dispatch, grouped gate/up GEMM with the SwiGLU epilogue,
 * grouped down GEMM and combine, enqueued on one stream with no host
 * synchronisation (the pages split the prefill kernel into several kernels
 * and fuse the decode kernel into one, section "Expert Parallel").
 *   x [T, H], w_router [H, E] as in moe_route; bias [E] or NULL;
 *   packed: moe_pack_weights() output; out (output) [T, H] float32.
 *   topk_idx, topk_w, counts, offsets, row_token, row_slot, slot_row:
 *       optional outputs (NULL: kept in the workspace), as in moe_route and
 *       moe_dispatch.
 *   ws: moe_layer_workspace_bytes(s) bytes of device scratch.
 *   x and the packed weights must come from the same dtype.  Intermediates:
 *   bf16 layers read the token rows straight from x (no packed copy);
 *   float32 layers pack them as fp16 first; SwiGLU activations and expert
 *   outputs are fp16.
 *   Small batches (an evenly routed expert gets at most 64 rows): while the
 *   router runs, CUs it leaves idle read the gate/up weights into the
 *   last-level cache; for bf16 layers of at most 1024 tokens the gate/up GEMM
 *   also derives the dispatch itself (no separate dispatch launch).  Every
 *   output is the same, to the bit, as the staged calls moe_route,
 *   moe_dispatch, moe_grouped_gemm (gate/up, then down) and moe_combine.
 */
int moe_layer(const moe_shape* s, const void* x, int x_dtype, const void* w_router, int w_dtype,
              const float* bias, const void* packed, float* out,
              int32_t* topk_idx, float* topk_w, int32_t* counts, int32_t* offsets,
              int32_t* row_token, int32_t* row_slot, int32_t* slot_row,
              void* ws, size_t ws_bytes, void* stream);

/*
 * MXFP8 expert GEMMs ("Quantification": the deployment quantises the model
 * with the MXFP8 microscaling scheme, converting the weights statically).
 * The format is the Open Compute Project Microscaling MXFP8 with E4M3
 * elements: 32 consecutive elements along the reduction dimension K share one
 * E8M0 scale 2^(e - 127) (a byte e); an element is an FP8 E4M3 code (bias 7,
 * largest finite 448, no infinities).  A block converts with shared exponent
 * floor(log2(max |v|)) - 8, clamped to [-127, 127] (-127 for an all-zero
 * block), and elements v / 2^shared rounded to the nearest E4M3 value, ties to
 * the even code, saturating at +-448.  Both operands of every expert GEMM are
 * MXFP8, multiplied on gfx950's scaled MFMA with float32 accumulation:
 * weights quantised per output column along K (H for gate/up, I for down),
 * token rows x per token along H, SwiGLU activations h per row along I.
 * Activation data: codes [rows][K] (uint8), scales [rows][K/32] (uint8 E8M0).
 * Every MXFP8 call needs H and I multiples of 256 (else MOE_ERR_UNSUPPORTED).
 */

/* Bytes of the MXFP8-packed weights of the E_loc local experts (host-only):
 * 3*E_loc*H*I bytes of codes plus one scale byte per 32 of them. */
size_t moe_packed_weight_bytes_mxfp8(const moe_shape* s);

/*
 * moe_pack_weights_mxfp8 -- static conversion of the local experts' weights
 * (w_gate, w_up [E_loc, H, I], w_down [E_loc, I, H], MOE_BF16 or MOE_F32) to
 * MXFP8, per output column along K, into the layout the MXFP8 grouped GEMM
 * streams.  packed: moe_packed_weight_bytes_mxfp8(s) bytes, written; opaque.
 */
int moe_pack_weights_mxfp8(const moe_shape* s, const void* w_gate, const void* w_up, const void* w_down,
                           int dtype, void* packed, void* stream);

/*
 * moe_quantize_mxfp8 -- MXFP8 conversion of rows along their last axis:
 *   x [rows, K] (MOE_BF16 or MOE_F32), K a multiple of 32 ->
 *   codes [rows, K] uint8 and scales [rows, K/32] uint8.  rows >= 0.
 */
int moe_quantize_mxfp8(int64_t rows, int32_t K, const void* x, int x_dtype, uint8_t* codes, uint8_t* scales,
                       void* stream);

/*
 * moe_grouped_gemm_mxfp8 -- moe_grouped_gemm() on MXFP8 operands.
 *   a, a_scales: activation codes and scales (rows of K = H for gate/up, I
 *       for down); a_rows as in moe_grouped_gemm (NULL: a holds the packed
 *       rows; else packed row r reads row a_rows[r] of a and of a_scales,
 *       0 <= a_rows[r] < T).
 *   packed: moe_pack_weights_mxfp8() output for the same shape.
 *   which / epilogue as in moe_grouped_gemm.  c_dtype MOE_F32, MOE_BF16 or
 *   MOE_F16 (rows of the plain product, or of h for MOE_EPI_SWIGLU), or, with
 *   MOE_EPI_SWIGLU only, MOE_MXFP8: c receives the codes of h [cap, I] and
 *   c_scales its scales [cap, I/32] (c_scales is ignored otherwise).
 *   Rows >= N_loc are not written.
 */
int moe_grouped_gemm_mxfp8(const moe_shape* s, const uint8_t* a, const uint8_t* a_scales, const int32_t* a_rows,
                           const int32_t* offsets, const void* packed, int which, int epilogue, void* c,
                           int c_dtype, uint8_t* c_scales, void* stream);

/* Bytes of scratch memory moe_layer_mxfp8() needs (host-only, no HIP call). */
size_t moe_layer_workspace_bytes_mxfp8(const moe_shape* s);

/*
 * moe_layer_mxfp8 -- moe_layer() with MXFP8 expert GEMMs: routing and
 * dispatch from the unquantised x exactly as moe_layer; each token row
 * quantised once along H; gate/up on the scaled MFMA with the SwiGLU epilogue
 * writing h as MXFP8; down on the scaled MFMA writing fp16 expert outputs;
 * combine as moe_layer.  Same arguments as moe_layer(), with packed from
 * moe_pack_weights_mxfp8() and ws of moe_layer_workspace_bytes_mxfp8(s) bytes.
 */
int moe_layer_mxfp8(const moe_shape* s, const void* x, int x_dtype, const void* w_router, int w_dtype,
                    const float* bias, const void* packed, float* out,
                    int32_t* topk_idx, float* topk_w, int32_t* counts, int32_t* offsets,
                    int32_t* row_token, int32_t* row_slot, int32_t* slot_row,
                    void* ws, size_t ws_bytes, void* stream);

/*
 * moe_layer_noalloc -- moe_layer() for callers that cannot allocate device
 * memory: code under stream (graph) capture, tight serving loops, harnesses
 * that forbid hipMalloc.  Same arguments, outputs and bits as moe_layer()
 * without ws / ws_bytes: the workspace is a static device array of
 * MOE_LAYER_NOALLOC_MAX_WS_BYTES bytes inside the library, one per GPU, held
 * by that GPU until the process ends.  The call allocates nothing (no
 * hipMalloc, no library allocation).
 *   Limit: moe_layer_workspace_bytes(s) <= MOE_LAYER_NOALLOC_MAX_WS_BYTES
 *   (64 MiB: decode-sized batches, e.g. 128 tokens x top-8 over 8 local
 *   experts of hidden 4096 needs about 20 MiB), else MOE_ERR_WORKSPACE and
 *   nothing is enqueued.
 *   The first call on each GPU (with that GPU current) resolves the array's
 *   address with hipGetSymbolAddress; make it outside stream capture.
 *   Every call on one GPU uses that GPU's one array: calls that overlap on a
 *   GPU (different streams, or threads, without ordering between them) race
 *   and give undefined results.  No part of the array needs to start zeroed:
 *   every call writes each workspace byte it reads.
 */
#define MOE_LAYER_NOALLOC_MAX_WS_BYTES ((size_t)64 << 20)
int moe_layer_noalloc(const moe_shape* s, const void* x, int x_dtype, const void* w_router, int w_dtype,
                      const float* bias, const void* packed, float* out,
                      int32_t* topk_idx, float* topk_w, int32_t* counts, int32_t* offsets,
                      int32_t* row_token, int32_t* row_slot, int32_t* slot_row, void* stream);

/*
 * Measurement helpers (not part of the layer).  moe_probe_mfma_bf16 launches
 * `blocks` workgroups of 8 waves, each wave issuing `iters` rounds of eight
 * independent v_mfma_f32_32x32x16_bf16 with no memory traffic, and writes one
 * float per thread to sink [blocks * 512] (device memory, caller-owned);
 * moe_probe_mfma_bf16_flops gives the FLOPs of one such launch.  Timing the
 * launch gives the dense bf16 MFMA rate the chip reaches under the current
 * clocks, to set beside the published peak.
 */
int64_t moe_probe_mfma_bf16_flops(int blocks, int iters);
int moe_probe_mfma_bf16(int blocks, int iters, float* sink, void* stream);

/* Text of a status code (static storage). */
const char* moe_status_string(int status);

/* hipError_t value of the last MOE_ERR_HIP returned on the calling thread (0 if none). */
int32_t moe_last_hip_error(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_LAYER_03_AMD_H */
