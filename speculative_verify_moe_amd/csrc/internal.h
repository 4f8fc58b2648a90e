// internal.h -- host-side launchers shared between the translation units of the library.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// Measurement hook of moe_set_stage_events: while a stage runs, its start and stop events
// (or null).  Every kernel is launched through launch_k, which hands them to the kernel's
// own dispatch (hipExtLaunchKernel), so they time the kernel itself: the start event is
// consumed by the first launch of the stage, the stop event is given to every launch of
// it and the last one's end remains.
extern thread_local hipEvent_t g_kstart, g_kstop;
template <typename... KArgs, typename... Args>
inline hipError_t launch_k(void (*kern)(KArgs...), dim3 grid, dim3 block, size_t lds, hipStream_t s, Args... args) {
  hipExtLaunchKernelGGL(kern, grid, block, (uint32_t)lds, s, g_kstart, g_kstop, 0u, args...);
  g_kstart = nullptr;
  return hipGetLastError();
}

// Decode/verify blocks run the GEMV path when T <= kDecodeMaxT and T*k <= kSmallSlots.
constexpr int kDecodeMaxT = 64;
constexpr int kSmallSlots = 1024;
constexpr int kMaxExperts = 1024;
constexpr int kMaxTopK = 32;
// Slots per block of the multi-block alignment.
constexpr int kAlignChunk = 256;
// Blocks of the fused decode kernel at most (one per CU).
constexpr int kMaxBlocks = 1024;
// The fused kernel's synchronisation words, at offset 0 of every layer workspace (so no other
// buffer of any plan aliases them, whichever calls share the workspace), 32-bit words:
//   [0, kMaxBlocks)         arrival flag of each block at the grid barrier (the call's token)
//   [kBarRelease]           release word of the grid barrier: the last token, with bit 31 set
//                           when a wait of that barrier gave up
//   [kBarStatus]            count of waits that gave up (0 in normal use) -- read by the caller
//   [kBarReady]             gate/up entries every block has finished, published by block 0
//   [kBarProgress, +NB)     gate/up entries block b has finished and stored (a prefix count)
// Each group sits on its own 256-byte line.
constexpr int kBarRelease = kMaxBlocks;
constexpr int kBarStatus = kMaxBlocks + 64;
constexpr int kBarReady = kMaxBlocks + 128;
constexpr int kBarProgress = kMaxBlocks + 192;
constexpr int kBarrierWords = kBarProgress + kMaxBlocks;

struct AlignOut {
  int32_t *sorted;
  int32_t *block_expert;
  int32_t *counts;
  int32_t *offsets;
  int32_t *num_padded;
};

// Compact list of the touched experts for the decode kernels (all pointers may be null
// when not wanted): n[0] experts with at least one slot, their ids ascending in e[],
// their slots grouped by expert (ascending inside a group) in slots[start[i] ..
// start[i+1]).  Capacity: e[E], start[E+1], slots[T*k].
struct Touched {
  int32_t *n;
  int32_t *e;
  int32_t *start;
  int32_t *slots;
};
inline size_t touched_ints(int E, int64_t n_slots) { return (size_t)(1 + E + E + 1 + n_slots); }
inline Touched touched_at(int32_t *base, int E) {
  return Touched{base, base + 1, base + 1 + E, base + 2 + 2 * E};
}

// ---------------------------------------------------------------- route.hip
hipError_t launch_router_rows(const uint16_t *x, int T, int H, const float *w_r, const float *b_r, int E,
                              const float *w_sg, float *logits, float *gate_logit, hipStream_t s);
hipError_t launch_topk(const float *logits, int T, int E, int k, int renorm, int32_t *ids, float *w,
                       const float *gate_logit, float *gamma, hipStream_t s);
hipError_t launch_topk_align_small(const float *logits, const float *gate_logit, int T, int E, int k, int renorm,
                                   int BM, int64_t cap, int32_t *ids, float *w, float *gamma, AlignOut al,
                                   Touched tl, hipStream_t s);
hipError_t launch_compact_touched(const int32_t *counts, const int32_t *offsets, const int32_t *sorted, int E,
                                  Touched tl, hipStream_t s);
hipError_t launch_align_small(const int32_t *ids, int n, int E, int BM, int64_t cap, AlignOut al, hipStream_t s);
// hist: align_hist_ints(n, E) int32 of scratch.
size_t align_hist_ints(int64_t n, int E);
hipError_t launch_align_large(const int32_t *ids, int n, int E, int BM, int64_t cap, AlignOut al, int32_t *hist,
                              hipStream_t s);

// ---------------------------------------------------------------- gemv.hip
struct GemvArgs {
  const uint16_t *x;
  int T, H, k;
  int wtype;
  // routed bank
  int E, I;
  const void *w_gu;
  const float *s_gu;
  const void *w_d;
  const float *s_d;
  const uint8_t *x_gu;  // MXFP4: E8M0 block-scale bytes [E][2I][H/32]
  const uint8_t *x_d;   // MXFP4: [E][H][I/32]
  const int32_t *tl_n;
  const int32_t *tl_e;
  const int32_t *tl_start;
  const int32_t *tl_slots;
  const float *topk_w;
  // shared expert (has_shared == 0: absent)
  int has_shared, I_s;
  const void *ws_gu;
  const float *ss_gu;
  const void *ws_d;
  const float *ss_d;
  const uint8_t *xs_gu;  // MXFP4: the shared expert's block-scale bytes
  const uint8_t *xs_d;
  const float *gamma;
  // intermediates and output
  uint16_t *h;    // [T*k][I], row = slot
  uint16_t *h_s;  // [T][I_s]
  uint16_t *out;  // [T][H]
};
hipError_t launch_gemv_gate_up(const GemvArgs &a, hipStream_t s, char *desc, size_t desc_len);
hipError_t launch_gemv_down(const GemvArgs &a, hipStream_t s, char *desc, size_t desc_len);
// a plain streaming read of n16 16-byte words (measurement aid; depth 4, 8 or 16)
hipError_t launch_stream_read(const void *buf, size_t n16, int blocks, int depth, uint32_t *sink, hipStream_t s);

// ---------------------------------------------------------------- fused.hip
struct FusedArgs {
  const uint16_t *x;
  int T, H, E, k, I, I_s, renorm, has_shared, BM, cap, wtype;
  const float *w_r;
  const float *b_r;
  const float *w_sg;
  const void *w_gu;
  const float *s_gu;
  const void *w_d;
  const float *s_d;
  const void *ws_gu;
  const float *ss_gu;
  const void *ws_d;
  const float *ss_d;
  const uint8_t *x_gu, *x_d, *xs_gu, *xs_d;  // MXFP4 block-scale bytes (routed, shared)
  float *logits;      // [T][E]
  float *gate_logit;  // [T]
  int32_t *ids;       // [T][k]   (block 0 writes)
  float *topw;        // [T][k]   (block 0 writes)
  float *gamma;       // [T]      (block 0 writes)
  AlignOut al;        // padded alignment (block 0 writes)
  uint16_t *h;        // [T*k][I]
  uint16_t *h_s;      // [T][I_s]
  uint16_t *out;      // [T][H]
  unsigned *bar;      // synchronisation words (kBarrierWords, layout above)
  size_t lds_route;   // set by the launcher
  int h_ring;         // rows of the LDS ring of staged routed h rows (set by the launcher)
};
bool fused_decode_fits(int T, int H, int E, int k, int I, int I_s, int wtype);
hipError_t launch_fused_decode(FusedArgs a, hipStream_t s, char *desc, size_t desc_len);

// ---------------------------------------------------------------- gemm.hip
// Which segments an expert-GEMM launch covers: the routed experts' and the shared expert's
// (one launch), or one kind only (the shared expert then runs on a stream of its own).
constexpr int SEG_ALL = 0, SEG_ROUTED = 1, SEG_SHARED = 2;
struct GemmArgs {
  int seg_mode;  // SEG_ALL, SEG_ROUTED or SEG_SHARED
  const uint16_t *x;
  int T, H, k, E, I, BM;
  int64_t cap;
  const uint16_t *w_gu;
  const uint16_t *w_d;
  const int32_t *sorted;
  const int32_t *block_expert;
  const int32_t *offsets;  // [E+1] padded expert offsets of the alignment
  const int32_t *counts;   // [E] tokens of each expert (its rows past them are padding)
  int has_shared, I_s;
  const uint16_t *ws_gu;
  const uint16_t *ws_d;
  int wtype;            // 0 bf16, 1 fp8 e4m3 (the matrices are then byte codes with row scales),
                        // 2 fp8 e4m3 with fp8 activations (x8 / h8 / hs8 below)
  const float *s_gu;    // fp8: [E][2I] row scales of w_gu
  const float *s_d;     // fp8: [E][H] row scales of w_d
  const float *ss_gu;   // fp8: [2 I_s] of the shared expert
  const float *ss_d;    // fp8: [H]
  uint16_t *h;    // [cap][I], row = sorted position
  uint16_t *h_s;  // [T][I_s]
  uint16_t *y;    // [T*k][H], row = slot
  uint16_t *y_s;  // [T][H]
  // wtype 2: the activations as fp8 codes with one fp32 scale per row
  const uint8_t *x8;  // [T][H]
  const float *sx;    // [T]
  uint8_t *h8;        // [cap][I], row = sorted position (rows of real slots only)
  float *sh;          // [cap]
  uint8_t *hs8;       // [T][I_s]
  float *shs;         // [T]
};
hipError_t launch_router_gemm(const uint16_t *x, int T, int H, const float *w_r, const float *b_r, int E,
                              const float *w_sg, float *logits, float *gate_logit, hipStream_t s);
hipError_t launch_gemm_gate_up(const GemmArgs &a, hipStream_t s);
hipError_t launch_gemm_down(const GemmArgs &a, hipStream_t s);
// wtype 2: the tokens, and the h rows of the real slots plus the shared h rows, to fp8 codes
// with one scale per row
hipError_t launch_quant_tokens(const uint16_t *x, int T, int H, uint8_t *x8, float *sx, hipStream_t s);
hipError_t launch_quant_h(const GemmArgs &a, hipStream_t s);
hipError_t launch_combine(const uint16_t *y, const uint16_t *y_s, const float *topk_w, const float *gamma, int T,
                          int H, int k, uint16_t *out, hipStream_t s);

}  // namespace moe
