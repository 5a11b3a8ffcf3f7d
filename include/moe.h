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
 * Conventions for every entry point below.  The pages describe serving
 * engines rather than this interface; each convention names the passage it
 * serves.
 *  - Memory: tensor pointers are DEVICE pointers, row-major, owned by the
 *    caller; the library allocates no device memory and keeps no pointer
 *    after the call returns ("Fast embeddings on GPUs", section "CUDA graph
 *    management": buffers are set up once, in the eager warm-up before a
 *    graph is captured, and reused by every replay).  Every pointer must be
 *    16-byte aligned.
 *  - Ordering: work is enqueued on `stream` (a hipStream_t; NULL = the null
 *    stream) and the call returns without waiting for it; results are valid
 *    once the stream has reached that point.  There is no host-device sync
 *    and no device-to-host copy, so the launch sequence can be captured in a
 *    HIP graph and replayed ("GPT-OSS on day 0", the opening of section
 *    "Kernels for GPT-OSS": the decoders and their CUDA-graph framework were
 *    reused unchanged for the new model; "Fast
 *    embeddings on GPUs", sections "CUDA graph management" and "Lazy
 *    Tensors": the forward is launched asynchronously and its result is
 *    tracked through an event; the page "The GPU sat idle, and the CPU was to
 *    blame" on Moondream's Photon engine, section "Two slots and copying
 *    behind the GPU's back": reading a result back to the host forces a
 *    synchronisation, so none happens inside the step).
 *  - Errors: argument errors are found on the host before anything is
 *    enqueued and return a negative status; nothing is written then.  A
 *    launch failure returns MOE_ERR_HIP.  Device faults surface at the
 *    caller's next sync.  No C++ exception crosses the boundary.
 *  - T == 0 is a no-op returning MOE_OK (x and out may then be NULL).
 *  - Deterministic: the same inputs give the same output bits (every
 *    floating-point reduction has a fixed order; atomics only add integer
 *    counts, whose sums do not depend on the order), so a replayed graph
 *    reproduces the eager call bit for bit.
 *  - `out` must not alias any input or the workspace.
 *  - NaN: a NaN in x makes every output of its token NaN; a NaN weight code,
 *    weight scale or bias of an expert makes the outputs of the tokens routed
 *    to it NaN.  The expert indices are always valid and distinct: the logit
 *    bits order the selection, so a positive NaN logit ranks above every
 *    number and a negative NaN logit below every number.
 *  - Calls that share a workspace must be ordered (same stream); calls on
 *    different workspaces may overlap.
 *  - Thread safety: entry points may be called from several host threads;
 *    the only process-wide state is a per-device cache of the compute-unit
 *    count and kernel occupancy, filled once under a lock.
 */
#ifndef SPARSE_MOE_MI355_H
#define SPARSE_MOE_MI355_H

#include <hip/hip_runtime_api.h>
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
                               d or f > MOE_MAX_HIDDEN, or buffers of 2^31 bytes
                               or more: x codes (T*d), h codes (T*k*f), one
                               expert's gate/up weights (2*d*f), the activation
                               scales, or the fp32 expert outputs (4*T*k*d)   */
  MOE_ERR_WORKSPACE = -4,   /* workspace NULL or smaller than moe_workspace_bytes */
  MOE_ERR_ALIGN = -5,       /* a pointer is not 16-byte aligned                   */
  MOE_ERR_HIP = -6,         /* a kernel launch failed (hipGetLastError)           */
  MOE_ERR_FLAGS = -7,       /* unknown bits in `flags`, path 3, MOE_WEIGHTS_FP4 without
                               MOE_FORMAT_MX, or a bad stage range */
  MOE_ERR_SCRATCH = -8      /* moe_forward_noalloc: the sizes need more workspace
                               than MOE_SCRATCH_BYTES                             */
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
/* MOE_FORMAT_MX: the MXFP8 variant ("Hosting Qwen on Blackwell", section
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
 * are invalid).  The workspace holds the routing tables ("GPT-OSS on day 0",
 * section "MoE": the dispatcher selects the tokens of each expert; "Hosting
 * Qwen on Blackwell", section "Expert Parallel": dispatch aggregates the
 * routing information and stages the tokens in the MoE GEMM's input buffer),
 * the quantised activations, h and the per-row expert outputs; nothing in it
 * has to be initialised and its content between calls is meaningless.  The
 * caller allocates it once per batch shape, as "Fast embeddings on GPUs",
 * section "CUDA graph management", sets up buffers before capture.  Size for
 * C-ABI users: about T*(d + k*(f + 4*d + 8)) bytes. */
size_t moe_workspace_bytes(int32_t T, int32_t d, int32_t f, int32_t E, int32_t k);

/* The block forward for T tokens: the formula above ("GPT-OSS on day 0",
 * sections "GPT-OSS on Hopper" and "MoE").
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
                       size_t workspace_bytes, hipStream_t stream);

/* moe_forward with `flags`: a GEMM path (MOE_PATH_*; the paths give the same
 * results to rounding of the fp32 accumulation order; "Hosting Qwen on
 * Blackwell", sections "Prefiller" and "Decoder": prefill batches make the
 * MoE GEMM dense and compute-bound, decode batches are bound by loading the
 * weights; "Disaggregated prefill and decode", section "Prefill vs decode
 * performance"), the gate-weight options MOE_ROUTE_SOFTMAX_ALL and
 * MOE_GATE_BF16 ("GPT-OSS on day 0", section "MoE"), and the weight formats
 * MOE_FORMAT_MX / MOE_FORMAT_MXFP4 ("Hosting Qwen on Blackwell", section
 * "Quantization"; "GPT-OSS on day 0", section "GPT-OSS on Hopper"). */
moe_status moe_forward_ex(const void* x, const float* W_router, const float* b_router, int32_t k,
                          const uint8_t* W_gateup, const float* S_gateup, const void* b_gateup,
                          const uint8_t* W_down, const float* S_down, const void* b_down,
                          void* out, int32_t T, int32_t d, int32_t f, int32_t E, void* workspace,
                          size_t workspace_bytes, uint32_t flags, hipStream_t stream);

/* moe_forward_ex with MXFP8 weights (flags | MOE_FORMAT_MX; "Hosting Qwen on
 * Blackwell", section "Quantization"):
 *   X_gateup   E8M0 [E, d/32, 2f]
 *   X_down     E8M0 [E, f/32, d]
 * the other arguments and `flags` bits as for moe_forward_ex (MOE_WEIGHTS_FP4
 * selects MXFP4 weights). */
moe_status moe_forward_mx(const void* x, const float* W_router, const float* b_router, int32_t k,
                          const uint8_t* W_gateup, const uint8_t* X_gateup, const void* b_gateup,
                          const uint8_t* W_down, const uint8_t* X_down, const void* b_down,
                          void* out, int32_t T, int32_t d, int32_t f, int32_t E, void* workspace,
                          size_t workspace_bytes, uint32_t flags, hipStream_t stream);

/* The forward runs in six stages, in this order on the stream: routing,
 * dispatch, the two expert GEMMs and the weighted combine ("GPT-OSS on day
 * 0", section "MoE"; "Hosting Qwen on Blackwell", section "Expert
 * Parallel").  For a batch
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
 * single kernels between events, the way "Hosting Qwen on Blackwell",
 * section "MoE GEMM", benchmarks the grouped GEMM on its own.  MOE_ERR_FLAGS
 * for a bad stage range. */
moe_status moe_forward_stages(const void* x, const float* W_router, const float* b_router,
                              int32_t k, const uint8_t* W_gateup, const float* S_gateup,
                              const void* b_gateup, const uint8_t* W_down, const float* S_down,
                              const void* b_down, void* out, int32_t T, int32_t d, int32_t f,
                              int32_t E, void* workspace, size_t workspace_bytes, uint32_t flags,
                              int32_t first_stage, int32_t last_stage, hipStream_t stream);

/* moe_forward_ex, then copies of intermediates into the optional (nullable)
 * device buffers, for parity tests and debugging (each array is one step of
 * the formula above; the copies are device-to-device and stream-ordered, so
 * no synchronisation happens here either):
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
                             hipStream_t stream, int32_t* topk_idx, float* topk_w, int32_t* offsets,
                             int32_t* row_token, int32_t* row_of, uint8_t* xq, float* xs,
                             uint8_t* hq, float* hs, float* y);

/* moe_forward_ex for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * no workspace argument; the library's own static device array of
 * MOE_SCRATCH_BYTES per GPU serves as the workspace.  It is set up on the
 * first call on each device (its address is looked up with that device
 * current) and each GPU holds it until the process ends.  The call allocates
 * nothing.  Sizes whose moe_workspace_bytes exceeds MOE_SCRATCH_BYTES return
 * MOE_ERR_SCRATCH before anything is enqueued (64 MiB holds decode-sized
 * batches: a 2944-wide layer with k = 4 and 32 experts up to 1025 tokens,
 * with 128 experts up to 902).  Every
 * call on one GPU shares that GPU's array: calls that overlap on one GPU
 * (different streams, or host threads without ordering) race and give
 * undefined results; order them on one stream.  Nothing in the array has to
 * start at zero, so its leftover content from an earlier call is harmless. */
#define MOE_SCRATCH_BYTES (64u << 20)
moe_status moe_forward_noalloc(const void* x, const float* W_router, const float* b_router,
                               int32_t k, const uint8_t* W_gateup, const float* S_gateup,
                               const void* b_gateup, const uint8_t* W_down, const float* S_down,
                               const void* b_down, void* out, int32_t T, int32_t d, int32_t f,
                               int32_t E, uint32_t flags, hipStream_t stream);

/* Static text for a status code (never NULL; "unknown status" for other
 * values), so callers can report an error without a device call. */
const char* moe_status_string(int32_t status);

#ifdef __cplusplus
}
#endif
#endif
