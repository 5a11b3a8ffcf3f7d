/*
 * Sparse Mixture-of-Experts block forward on one MI355X (gfx950) - C ABI.
 *
 * The operation is the MoE MLP block of the "GPT-OSS on day 0" post
 * (Perplexity, 2025): section "GPT-OSS on Hopper" lists its parts (sparse
 * mixture of experts, SwiGLU activation, softmax after top-k for the expert
 * weights, experts with biases) and the serving format (FP8 with 128x128
 * block scaling); section "MoE" says the softmax runs over the selected
 * experts only, that the expert GEMMs carry their bias in the accumulator,
 * and that tokens are dispatched to their experts and combined by a weighted
 * accumulation.  For one token x (hidden size d):
 *
 *   l      = x . W_router + b_router                     (E logits, fp32)
 *   S      = the k largest logits (descending; ties -> lower expert index)
 *   w_j    = exp(l_j - max_S l) / sum_{i in S} exp(l_i - max_S l)
 *   xq,xs  = e4m3 codes and fp32 scales of x, one scale per 128 columns:
 *            s = amax/448 (1 if the group is all zero), q = e4m3_rne(x/s)
 *   per selected expert e:
 *     P    = deq(xq,xs) . deq(W_gateup[e],S_gateup[e]) + b_gateup[e]   (2f)
 *     h    = silu(P[0:f]) * P[f:2f]                     (gate half first)
 *     hq,hs= e4m3 codes / scales of h per 128 columns (same rule)
 *     Y_e  = deq(hq,hs) . deq(W_down[e],S_down[e]) + b_down[e]          (d)
 *   out    = bf16_rne( sum_j w_j * Y_{e_j} )
 *
 * deq(W,S) multiplies every e4m3 weight by the fp32 scale of its 128x128
 * block.  FP8 is OCP E4M3 ("fn": max 448, NaN 0x7F/0xFF, no infinities).
 *
 * Conventions for every entry point below:
 *  - Tensor pointers are DEVICE pointers, row-major, owned by the caller;
 *    the library allocates no device memory and keeps no pointer after the
 *    call returns.  Every pointer must be 16-byte aligned.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream)
 *    and the call returns without waiting for it; results are valid once
 *    the stream has reached that point.  There is no host-device sync and
 *    no device-to-host copy, so the sequence can be captured in a graph.
 *  - Argument errors are found on the host before anything is enqueued and
 *    return a negative status; nothing is written then.  A launch failure
 *    returns MOE_ERR_HIP.  Device faults surface at the caller's next sync.
 *  - T == 0 is a no-op returning MOE_OK (x and out may then be NULL).
 *  - Deterministic: the same inputs give the same output bits (no atomics
 *    on data paths; every reduction has a fixed order).
 *  - `out` must not alias any input or the workspace.
 *  - NaN inputs propagate to outputs; expert indices are always valid and
 *    distinct whatever the logits hold.
 *  - Calls that share a workspace must be ordered (same stream); calls on
 *    different workspaces may overlap.
 */
#ifndef SPARSE_MOE_MI355_H
#define SPARSE_MOE_MI355_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_NULL = -1,        /* a required pointer is NULL                         */
  MOE_ERR_SHAPE = -2,       /* T < 0, d or f not a positive multiple of 128, E < 1 */
  MOE_ERR_UNSUPPORTED = -3, /* k < 1, k > E, k > MOE_MAX_TOPK, E > MOE_MAX_EXPERTS,
                               d or f > MOE_MAX_HIDDEN, or tensors of 2^31 bytes
                               or more (T*d, T*k*f, d*2f, scales)                 */
  MOE_ERR_WORKSPACE = -4,   /* workspace NULL or smaller than moe_workspace_bytes */
  MOE_ERR_ALIGN = -5,       /* a pointer is not 16-byte aligned                   */
  MOE_ERR_HIP = -6,         /* a kernel launch failed (hipGetLastError)           */
  MOE_ERR_FLAGS = -7        /* unknown bits in `flags`, path 3, MOE_WEIGHTS_FP4 without
                               MOE_FORMAT_MX, or a bad stage range */
} moe_status;

#define MOE_MAX_EXPERTS 256
#define MOE_MAX_TOPK 8
#define MOE_BLOCK 128
#define MOE_MAX_HIDDEN 8192 /* d and f: at most 64 blocks of 128 */

/* Argument `flags`: bits 0-1 select the path of the expert GEMMs, */
#define MOE_PATH_AUTO 0u    /* pick by the mean rows per expert, T*k/E           */
#define MOE_PATH_PREFILL 1u /* large row tiles, MFMA-bound shape                  */
#define MOE_PATH_DECODE 2u  /* small row tiles streaming weights (memory-bound)   */
#define MOE_PATH_MASK 3u
/* and two bits change the gate weights (the expert selection never changes).
 * MOE_ROUTE_SOFTMAX_ALL: the softmax runs over all E logits before top-k and
 * each selected expert keeps its full-softmax probability (not renormalised
 * over the k): the routing rule that "GPT-OSS on day 0", section "MoE",
 * contrasts with gpt-oss's softmax over the selected logits (the default).
 * MOE_GATE_BF16: the gate weights are rounded to bf16 (nearest even) before
 * the combine (the same section keeps the expert weights in bf16; by default
 * they stay fp32). */
#define MOE_ROUTE_SOFTMAX_ALL 4u
#define MOE_GATE_BF16 8u
/* MOE_FORMAT_MX: the MXFP8 variant ("GPT-OSS on day 0", section
 * "Quantization": microscaling, the Blackwell format, with the weights
 * converted statically).  Every 32 consecutive elements along the
 * contraction share one E8M0 scale (a uint8 e; value 2^(e-127), 0xFF NaN):
 *   S_gateup   E8M0 [E, d/32, 2f]   scale of W_gateup[e, 32i..32i+31, c]
 *   S_down     E8M0 [E, f/32, d]    scale of W_down[e, 32i..32i+31, c]
 * passed through the `const float*` scale arguments (moe_forward_mx takes
 * them typed).  x and h are quantised per 32 columns: the scale 2^e of a
 * block is the smallest power of two with amax <= 448 * 2^e (2^-127 for an
 * all-zero block; no element saturates), q = e4m3_rne(v / 2^e).  The debug
 * copies xs / hs then hold E8M0 bytes [T, d/32] / [T*k, f/32]: the same
 * byte counts as the fp32 scales of the default format. */
#define MOE_FORMAT_MX 16u
/* MOE_WEIGHTS_FP4 (only together with MOE_FORMAT_MX; MOE_FORMAT_MXFP4 sets
 * both): MXFP4 weights, the format the gpt-oss checkpoints ship in ("GPT-OSS
 * on day 0", section "GPT-OSS on Hopper").  Elements are OCP E2M1 (sign,
 * 2 exponent bits with bias 1, 1 mantissa bit: +-{0, 0.5, 1, 1.5, 2, 3, 4, 6}),
 * two per byte along K, the even K in the low nibble:
 *   W_gateup   [E, d/2, 2f] bytes    W_down   [E, f/2, d] bytes
 * with the E8M0 scales of MOE_FORMAT_MX ([E, d/32, 2f], [E, f/32, d]).  x and
 * h stay MXFP8 (e4m3 per 32 columns), so every MFMA multiplies E2M1 weights
 * by e4m3 activations. */
#define MOE_WEIGHTS_FP4 32u
#define MOE_FORMAT_MXFP4 (MOE_FORMAT_MX | MOE_WEIGHTS_FP4)

/* Bytes of device workspace moe_forward needs for these sizes (0 if the sizes
 * are invalid).  The workspace holds the routing tables, the quantised
 * activations, h and the per-row expert outputs; its content between calls
 * is meaningless.  Size for C-ABI users: about T*(d + k*(f + 4*d + 8)) bytes. */
size_t moe_workspace_bytes(int32_t T, int32_t d, int32_t f, int32_t E, int32_t k);

/* The block forward for T tokens.
 *   x          bf16  [T, d]
 *   W_router   fp32  [d, E]
 *   b_router   fp32  [E]
 *   k          experts per token, 1 <= k <= min(E, 8)
 *   W_gateup   e4m3  [E, d, 2f]   column c < f is gate column c, f + c the up column c
 *   S_gateup   fp32  [E, d/128, 2f/128]   one scale per 128x128 block
 *   b_gateup   bf16  [E, 2f]
 *   W_down     e4m3  [E, f, d]
 *   S_down     fp32  [E, f/128, d/128]
 *   b_down     bf16  [E, d]
 *   out        bf16  [T, d]       written
 *   workspace  >= moe_workspace_bytes(T, d, f, E, k) bytes of device memory
 *   stream     hipStream_t
 */
moe_status moe_forward(const void* x, const float* W_router, const float* b_router, int32_t k,
                       const uint8_t* W_gateup, const float* S_gateup, const void* b_gateup,
                       const uint8_t* W_down, const float* S_down, const void* b_down, void* out,
                       int32_t T, int32_t d, int32_t f, int32_t E, void* workspace,
                       size_t workspace_bytes, void* stream);

/* moe_forward with `flags`: a GEMM path (MOE_PATH_*; the paths give the same
 * results to rounding of the fp32 accumulation order), the gate-weight
 * options MOE_ROUTE_SOFTMAX_ALL and MOE_GATE_BF16, and the weight format
 * MOE_FORMAT_MX. */
moe_status moe_forward_ex(const void* x, const float* W_router, const float* b_router, int32_t k,
                          const uint8_t* W_gateup, const float* S_gateup, const void* b_gateup,
                          const uint8_t* W_down, const float* S_down, const void* b_down,
                          void* out, int32_t T, int32_t d, int32_t f, int32_t E, void* workspace,
                          size_t workspace_bytes, uint32_t flags, void* stream);

/* moe_forward_ex with MXFP8 weights (flags | MOE_FORMAT_MX):
 *   X_gateup   E8M0 [E, d/32, 2f]
 *   X_down     E8M0 [E, f/32, d]
 * the other arguments and `flags` bits as for moe_forward_ex (MOE_WEIGHTS_FP4
 * selects MXFP4 weights). */
moe_status moe_forward_mx(const void* x, const float* W_router, const float* b_router, int32_t k,
                          const uint8_t* W_gateup, const uint8_t* X_gateup, const void* b_gateup,
                          const uint8_t* W_down, const uint8_t* X_down, const void* b_down,
                          void* out, int32_t T, int32_t d, int32_t f, int32_t E, void* workspace,
                          size_t workspace_bytes, uint32_t flags, void* stream);

/* The forward runs in six stages, in this order on the stream.  For a batch
 * of at most 64 tokens the router stage performs the whole routing (counts,
 * offsets, tile lists, placement) and the scan and place stages have no work. */
#define MOE_STAGE_ROUTER 0  /* router logits, top-k, softmax, x quantisation, tile histogram */
#define MOE_STAGE_SCAN 1    /* expert counts, offsets, per-tile row bases, GEMM tile offsets  */
#define MOE_STAGE_PLACE 2   /* permuted row of every (token, slot); both GEMMs' tile lists     */
#define MOE_STAGE_GATEUP 3  /* gate/up grouped GEMM + bias + SwiGLU + h quantisation           */
#define MOE_STAGE_DOWN 4    /* down grouped GEMM + bias                                        */
#define MOE_STAGE_COMBINE 5 /* weighted sum of each token's k rows -> bf16 out                */
#define MOE_NUM_STAGES 6

/* moe_forward_ex restricted to stages first_stage..last_stage (inclusive).
 * Running all stages in order, in one or several calls on the same stream
 * and workspace with the same arguments, equals moe_forward_ex.  A stage reads
 * the tables the earlier stages wrote into the workspace: running a stage
 * whose predecessors have not run on that workspace with the same arguments
 * is undefined behaviour (out-of-bounds device accesses).  Meant for timing
 * single kernels between events.  MOE_ERR_FLAGS for a bad stage range. */
moe_status moe_forward_stages(const void* x, const float* W_router, const float* b_router,
                              int32_t k, const uint8_t* W_gateup, const float* S_gateup,
                              const void* b_gateup, const uint8_t* W_down, const float* S_down,
                              const void* b_down, void* out, int32_t T, int32_t d, int32_t f,
                              int32_t E, void* workspace, size_t workspace_bytes, uint32_t flags,
                              int32_t first_stage, int32_t last_stage, void* stream);

/* moe_forward_ex, then copies of intermediates into the optional (nullable)
 * device buffers, for parity tests and debugging:
 *   topk_idx   int32 [T, k]   selected experts, descending logit
 *   topk_w     fp32  [T, k]   gate weights in the same order
 *   offsets    int32 [E+1]    first permuted row of every expert (exclusive scan)
 *   row_token  int32 [T*k]    token of every permuted row (expert-major, token-ascending)
 *   row_of     int32 [T, k]   permuted row of every (token, slot)
 *   xq         e4m3  [T, d]   quantised x;  xs fp32 [T, d/128] its scales
 *   hq         e4m3  [T*k, f] quantised h per permuted row;  hs fp32 [T*k, f/128]
 *   y          fp32  [T*k, d] expert output per permuted row, bias included
 */
moe_status moe_forward_debug(const void* x, const float* W_router, const float* b_router,
                             int32_t k, const uint8_t* W_gateup, const float* S_gateup,
                             const void* b_gateup, const uint8_t* W_down, const float* S_down,
                             const void* b_down, void* out, int32_t T, int32_t d, int32_t f,
                             int32_t E, void* workspace, size_t workspace_bytes, uint32_t flags,
                             void* stream, int32_t* topk_idx, float* topk_w, int32_t* offsets,
                             int32_t* row_token, int32_t* row_of, uint8_t* xq, float* xs,
                             uint8_t* hq, float* hs, float* y);

/* Static text for a status code. */
const char* moe_status_string(int32_t status);

#ifdef __cplusplus
}
#endif
#endif
