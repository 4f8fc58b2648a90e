/*
 * moe.h -- C ABI of the MI355X (gfx950) routed mixture-of-experts layer library.
 *
 * The layer: a Qwen-family sparse MoE FFN block as the pages run it in
 * speculative-decoding verify passes and prefill chunks.
 *   - veloGB10 README, "The model": routed experts per layer, top-k per token,
 *     plus one always-on shared expert.
 *   - Qwen3.6-35B-A3B for NInfer, "Artifact": routed gate/up and down
 *     projections; shared experts of the same form.
 *   - Qwen3.8 Flash-Next . GB10 UltraFast, first bullet: a deterministic
 *     floor -- token-to-expert alignment independent of thread arrival order
 *     and a combine without float atomicAdd.
 *   - veloGB10 README, "Kernel work": router fold spread over the GPU,
 *     grouped expert kernels that stream weights without rebuilding them,
 *     routing folded into neighbouring kernels, shared expert overlapped with
 *     the routed step.
 *
 * Arithmetic (the pages name the steps but do not write them; these are the
 * readings the library implements):
 *   logits  l[t][e] = sum_h x[t][h] * Wr[e][h] + b[e]          (fp32)
 *   top-k   the k largest logits, ties to the lower expert index, -0 == +0,
 *           NaN ranked below every number; slot j = rank j
 *   gates   w[t][j] = exp(l_j - l_0) / sum_{j'<k} exp(l_j' - l_0)
 *           (softmax over all experts renormalised over the chosen k), or the
 *           plain softmax probability when renormalize == 0
 *   expert  h_r = bf16(silu(x.Wgu[r]) * x.Wgu[I+r]);  y_o = bf16(h . Wd[o])
 *   shared  gamma_t = sigmoid(x_t . w_sg); y_s as an expert with I_s
 *   combine out[t] = bf16(sum_{j<k} w[t][j] * y_{t,j} + gamma_t * y_s[t]),
 *           summed in slot order in fp32 registers; no float atomics anywhere
 *   fp8     W = code * row_scale (OCP E4M3FN codes, one fp32 scale per output
 *           row); the scale multiplies the finished row sum
 *
 * Conventions for every entry point:
 *   - Tensor pointers are DEVICE pointers unless stated; bf16 values are
 *     uint16_t bit patterns, fp8 values uint8_t E4M3FN codes; all arrays are
 *     dense row-major with the shapes given.
 *   - Structs (moe_bank, moe_layer) are HOST memory, read only during the call.
 *   - All work is enqueued on `stream` (a hipStream_t; NULL = the default
 *     stream); calls return without synchronising, allocate nothing and keep no
 *     pointer after returning.  The caller keeps buffers alive until the stream
 *     has run the work.  No call records a memset, so calls can be captured
 *     into a HIP graph.
 *   - Validation is synchronous and happens before anything is enqueued; on a
 *     non-OK status nothing has been written and moe_last_error() names the
 *     violated constraint.  Launch failures return MOE_ERR_DEVICE.
 *   - Results are bitwise reproducible run to run: reductions have a fixed
 *     order and the only atomics are integer LDS counters.
 *   - Calls on one stream are ordered; concurrent calls on different streams
 *     must not share output or workspace buffers.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1, /* a null pointer, a negative or out-of-range size */
  MOE_ERR_MISALIGNED = 2,  /* a tensor pointer not 16-byte aligned */
  MOE_ERR_WORKSPACE = 3,   /* workspace or capacity too small */
  MOE_ERR_UNSUPPORTED = 4, /* shape/dtype combination not implemented, or device not gfx950 */
  MOE_ERR_DEVICE = 5       /* a HIP call or kernel launch failed */
} moe_status;

/* Weight (and activation) types of a bank.
 *   MOE_W_BF16: bf16 weights and activations.
 *   MOE_W_FP8_E4M3: OCP E4M3FN weight codes with one fp32 scale per weight row
 *     (s_gate_up, s_down); bf16 activations.
 *   MOE_W_FP8_E4M3_A8: the same weight storage.  On the prefill path the activations
 *     entering each expert matrix are quantised too -- every token row, and every
 *     slot's bf16 h row, to E4M3FN codes with one scale per row (the least power of two
 *     s with amax <= 448 s; code = the nearest E4M3FN code of a / s, ties to an even
 *     mantissa) -- and the expert GEMMs run on the fp8
 *     matrix cores (Qwen3.8 Flash-Next . GB10 UltraFast and veloGB10 README, FP8
 *     layers; gfx950 fp8 MFMA).  The decode path (T <= 64) streams the same weights
 *     with bf16 activations, exactly as MOE_W_FP8_E4M3.
 *   MOE_W_MXFP4: OCP MX (Microscaling) FP4 -- E2M1 codes, two per byte with the
 *     even-indexed weight in the low nibble, w_gate_up [n][2I][H/2] and w_down
 *     [n][H][I/2] bytes, and one E8M0 scale byte (2^(X-127)) per block of 32 consecutive
 *     weights of a row in mx_gate_up [n][2I][H/32] and mx_down [n][H][I/32].  4-bit routed
 *     experts with 16-bit activations (Qwen3.8 Flash-Next . GB10 UltraFast, "Target
 *     precision"; Qwen3.6-35B-A3B for NInfer, "Artifact"; veloGB10 README, NVFP4 packs),
 *     in the format gfx950 converts natively.  Decode path only (T <= 64): a prefill
 *     chunk returns MOE_ERR_UNSUPPORTED. */
typedef enum { MOE_W_BF16 = 0, MOE_W_FP8_E4M3 = 1, MOE_W_FP8_E4M3_A8 = 2, MOE_W_MXFP4 = 3 } moe_wtype;

/* A bank of experts of one form (routed: n = E experts; shared: n = 1).
 * Qwen3.6-35B-A3B for NInfer, "Artifact" (gate/up and down per expert). */
typedef struct {
  int32_t wtype;              /* moe_wtype */
  int32_t num_experts;        /* n; a shared bank with n == 0 means "no shared expert" */
  int32_t hidden;             /* H, multiple of 64, at most 8192 */
  int32_t inter;              /* I, multiple of 64 */
  const void *w_gate_up;      /* [n][2I][H]: rows [0,I) gate, rows [I,2I) up (MXFP4: [n][2I][H/2] bytes) */
  const void *w_down;         /* [n][H][I] (MXFP4: [n][H][I/2] bytes) */
  const float *s_gate_up;     /* fp8 types: [n][2I] fp32 row scales, 4-byte aligned; ignored otherwise */
  const float *s_down;        /* fp8 types: [n][H] fp32 row scales, 4-byte aligned; ignored otherwise */
  const uint8_t *mx_gate_up;  /* MXFP4: [n][2I][H/32] E8M0 block-scale bytes; ignored otherwise */
  const uint8_t *mx_down;     /* MXFP4: [n][H][I/32] E8M0 block-scale bytes; ignored otherwise */
} moe_bank;

/* One MoE layer.  veloGB10 README, "The model". */
typedef struct {
  int32_t hidden;          /* H */
  int32_t num_experts;     /* E, 1..1024 */
  int32_t top_k;           /* k, 1..min(E, 32) */
  int32_t renormalize;     /* 1: renormalise the gates over the chosen k */
  const float *router_w;   /* [E][H] fp32 */
  const float *router_b;   /* [E] fp32, or NULL */
  moe_bank routed;         /* n = E */
  moe_bank shared;         /* n = 1, or n = 0 for no shared expert; same wtype and H */
  const float *shared_gate_w; /* [H] fp32; required when the shared expert is present */
} moe_layer;

/* Capacity (entries) of the padded slot list of moe_align:
 * roundup(T*k + min(E, T*k)*(BM-1), BM).  Pure host arithmetic; 0 on bad input. */
size_t moe_align_capacity(int32_t T, int32_t k, int32_t E, int32_t BM);

/* Workspace bytes moe_align needs for T tokens of k slots over E experts. */
size_t moe_align_workspace_size(int32_t T, int32_t k, int32_t E);

/* Top-k routing from fp32 logits.  veloGB10 README, "The model" (top-k per
 * token); Qwen3.8 Flash-Next . GB10 UltraFast, "How it works" (sort-free
 * verify-path top-k): k rounds of a wavefront-wide arg-max, no sort.
 *   logits [T][E] fp32 (in); topk_ids [T][k] int32 (out); topk_w [T][k] fp32 (out).
 * E <= 1024, 1 <= k <= min(E, 32).  T == 0 is a no-op. */
moe_status moe_route_topk(const float *logits, int32_t T, int32_t E, int32_t k, int32_t renormalize,
                          int32_t *topk_ids, float *topk_w, void *stream);

/* Token-to-expert alignment: histogram, padded exclusive scan, stable scatter.
 * Qwen3.8 Flash-Next . GB10 UltraFast, first bullet and "Configuration
 * reference" (moe_align_block_size with the arrival-order shim).
 *   topk_ids [T][k] int32 in [0, E) (in); slot i = t*k + j.
 *   expert_counts [E]: slots routed to each expert.
 *   expert_offsets [E+1]: exclusive scan of the counts rounded up to BM.
 *   num_padded [1]: expert_offsets[E].
 *   sorted_ids [cap]: expert e's slots in ascending order at
 *     [offsets[e], offsets[e] + counts[e]), then the sentinel T*k up to the next
 *     offset and from num_padded to cap.
 *   block_expert [cap/BM]: expert of each BM-block, -1 past num_padded.
 * BM in {16, 32, 64, 128}; cap >= moe_align_capacity(T, k, E, BM) and a
 * multiple of BM; ws >= moe_align_workspace_size(T, k, E) bytes (may be NULL
 * when that size is 0).  Ids outside [0, E) are an error of the caller (they
 * are not checked on the device). */
moe_status moe_align(const int32_t *topk_ids, int32_t T, int32_t k, int32_t E, int32_t BM, int64_t cap,
                     int32_t *sorted_ids, int32_t *block_expert, int32_t *expert_counts,
                     int32_t *expert_offsets, int32_t *num_padded, void *ws, size_t ws_bytes, void *stream);

/* Workspace bytes moe_experts_forward needs. */
size_t moe_experts_workspace_size(int32_t T, int32_t k, const moe_bank *routed, int32_t BM);

/* Routed experts and the weighted combine, given a routing and its alignment
 * (the outputs of moe_route_topk and moe_align).  veloGB10 README, "Kernel
 * work" (grouped MoE expert kernels for decode and prefill); Qwen3.8 Flash-Next
 * . GB10 UltraFast, first bullet (combine without float atomics).
 *   x [T][H] bf16; topk_w [T][k]; alignment arrays as moe_align wrote them;
 *   out [T][H] bf16 = bf16(sum_j w[t][j] * y_{t,j}) (no shared expert).
 * T <= 64 runs the weight-streaming GEMV path (each touched expert's rows are
 * read once); larger T runs the grouped MFMA GEMM path (bf16 weights, or fp8 codes
 * widened exactly to bf16 in LDS, with the row scales applied to the finished sums;
 * MOE_W_FP8_E4M3_A8 quantises the token and h rows and runs fp8 x fp8 MFMAs, and
 * then needs inter % 128 == 0). */
moe_status moe_experts_forward(const uint16_t *x, int32_t T, const moe_bank *routed, int32_t k,
                               const float *topk_w, const int32_t *sorted_ids, const int32_t *block_expert,
                               const int32_t *expert_counts, const int32_t *expert_offsets, int32_t BM,
                               int64_t cap, uint16_t *out, void *ws, size_t ws_bytes, void *stream);

/* Workspace bytes moe_layer_forward needs for T tokens.  The workspace is scratch for one
 * call at a time on one device; calls of any T may take turns on it.  Its first bytes hold
 * the synchronisation words of the fused decode kernel (an arrival count that carries over
 * from call to call, so no call needs a reset or a memset; a status word; per-entry
 * readiness counts), laid out the same in every plan: zero a new workspace once, before its
 * first call, and do not write into it between calls. */
size_t moe_layer_workspace_size(int32_t T, const moe_layer *L);

/* The whole layer: router, top-k, alignment, routed experts, shared expert and
 * combine -- the routed MoE FFN block of veloGB10 README, "The model" (top-k routed
 * experts plus one always-on shared expert), with the routing folded into the expert
 * kernels (same README, "Kernel work") and the deterministic alignment and combine of
 * Qwen3.8 Flash-Next . GB10 UltraFast, first bullet.
 *   x [T][H] bf16 (in); out [T][H] bf16 (out).
 *   logits_out [T][E] fp32, ids_out [T][k] int32, w_out [T][k] fp32: optional
 *   (NULL to skip) copies of the routing the layer used.
 * Decode/verify blocks (T <= 64) use BM = 16 and the GEMV path; prefill chunks
 * use BM = 64 and the MFMA path (bf16 or fp8 weights; fp8 activations as well
 * for MOE_W_FP8_E4M3_A8, which then needs inter % 128 == 0).
 * Residency: a decode block that fits the fused kernel runs one block per CU and needs
 * all of them resident together (its blocks wait for one another).  Kernels of other
 * streams or processes that hold CUs can delay some of its blocks; every wait is bounded,
 * and a wait that gives up adds one to the workspace's status word
 * (moe_workspace_status_offset) and makes the call write NaN for the output rows that
 * depended on it -- a wrong result is never silent and no call hangs.  Run the fused path
 * on a GPU it does not share, or read the status word after a batch of calls. */
moe_status moe_layer_forward(const uint16_t *x, int32_t T, const moe_layer *L, uint16_t *out, float *logits_out,
                             int32_t *ids_out, float *w_out, void *ws, size_t ws_bytes, void *stream);

/* moe_layer_forward for callers that cannot allocate -- code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc: the same computation with no workspace
 * argument.  Its scratch is a static 8 MiB array in device memory (one per device, held
 * until the process ends), so it serves calls whose plan needs at most that much
 * (moe_layer_workspace_size(T, L) <= 8 MiB: every decode/verify block of the Qwen-like
 * shapes; a larger call returns MOE_ERR_WORKSPACE and names the size).  It calls no
 * hipMalloc, hipFree or allocating library routine.  Every call on a device shares that
 * device's scratch, which keeps the last call's contents: calls that overlap on one device
 * (different streams, or different threads without ordering) race and must not be made.
 * On the first call on a device its synchronisation words are cleared by a small kernel on
 * `stream`.  Arguments, outputs and errors as moe_layer_forward. */
moe_status moe_layer_forward_noalloc(const uint16_t *x, int32_t T, const moe_layer *L, uint16_t *out,
                                     float *logits_out, int32_t *ids_out, float *w_out, void *stream);

/* Byte offset, inside every moe_layer_forward workspace, of a uint32 count of the fused
 * decode kernel's waits that gave up (0 in normal use; see moe_layer_forward).  The count
 * only grows; zeroing the workspace clears it.  Pure host function. */
size_t moe_workspace_status_offset(void);

/* Detail of the last non-OK status on the calling thread (empty if none). */
const char *moe_last_error(void);

/* The kernels moe_layer_forward would launch for T tokens, as text (thread-local
 * buffer, valid until the next call on the thread). */
const char *moe_describe_plan(int32_t T, const moe_layer *L);

/* Options of the calling thread (no environment variable is read).
 *   MOE_OPT_DECODE_FUSED: 1 (default) runs decode/verify blocks that fit the fused
 *   kernel (H <= 2048, I and I_s <= 512, tokens and intermediates within LDS) as one
 *   kernel -- router, top-k, alignment, experts and combine with one grid-wide barrier
 *   (one block per CU, all resident); 0 runs the same steps as four kernels (router,
 *   top-k + alignment, gate/up, down + combine).  Both give bitwise the same routing and
 *   output.  Other shapes always take the four-kernel path. */
enum { MOE_OPT_DECODE_FUSED = 1 };
moe_status moe_set_option(int32_t key, int32_t value);

/* Measurement hook.  events: n_events hipEvent_t handles (host array, created with
 * timing enabled), or NULL to turn the hook off; at most 64.  While set on a thread,
 * stage i of each moe_layer_forward call on that thread takes events[2i] and
 * events[2i+1] (only as many as n_events holds): they are handed to the stage's kernel
 * dispatches (hipExtLaunchKernel), events[2i] marking the start of its first kernel and
 * events[2i+1] the end of its last, so their elapsed time is the stage's kernel time.  A
 * stage is one kernel or a fixed group of kernels; moe_describe_plan names the stages in
 * launch order (fused decode: 1 stage; four-kernel decode: 4; prefill: 6, or 8 with a
 * shared expert -- its two GEMMs first, on a second stream -- or with fp8 activations). */
moe_status moe_set_stage_events(void *const *events, int32_t n_events);

/* Measurement aid, no part of the layer: enqueues one plain streaming read of `bytes`
 * bytes of device memory at buf (both multiples of 16), by `blocks` workgroups of 256
 * threads, each thread keeping `depth` (4, 8 or 16) non-temporal 16-byte loads in flight;
 * the blocks stride over the buffer in chunks of 256 * depth * 16 bytes.  sink (device,
 * `blocks` uint32) receives one checksum word per block, which keeps every load.  Timed by
 * the caller (events around the call), it gives the read rate the device attains -- the
 * context for the HBM fractions of the layer kernels, which stay against the nominal
 * peak.  The pages define no such call. */
moe_status moe_measure_stream_read(const void *buf, size_t bytes, int32_t blocks, int32_t depth, uint32_t *sink,
                                   void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
