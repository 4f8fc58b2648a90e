// api.hip -- the C ABI of include/moe.h: validation, workspace plan, kernel dispatch.
//
// Everything here runs on the host.  Validation comes first and touches no HIP
// API, so a bad argument is reported without any device work; then the device is
// checked to be gfx950, the workspace is carved into buffers and the kernels of
// the chosen path are enqueued on the caller's stream.  Nothing is allocated.
//
// Bad configurations are refused before any work with the arithmetic that failed,
// as the veloGB10 README ("Concurrent requests on the EXL3 path") refuses a model
// that cannot fit; the library reads no environment variable (same README, "Still
// in force from v0.7.0": every option is an explicit argument).
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "../../include/moe.h"
#include "internal.h"

using namespace moe;

namespace moe {
thread_local hipEvent_t g_kstart = nullptr, g_kstop = nullptr;
}

namespace {

thread_local char g_err[512];
thread_local char g_plan[2048];
thread_local void *g_events[64];
thread_local int g_nevents = 0;
thread_local int g_opt_fused = 1;

moe_status fail(moe_status st, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void *p) { return ((uintptr_t)p & 3u) == 0; }

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

int64_t capacity(int64_t T, int64_t k, int64_t E, int64_t BM) {
  const int64_t n = T * k;
  const int64_t touched = n < E ? n : E;
  const int64_t c = n + touched * (BM - 1);
  return (c + BM - 1) / BM * BM;
}

bool valid_bm(int BM) { return BM == 16 || BM == 32 || BM == 64 || BM == 128; }

std::atomic<int> g_arch[64];

moe_status check_device() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MOE_ERR_DEVICE, "hipGetDevice failed: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= 64) return fail(MOE_ERR_UNSUPPORTED, "device index %d out of range", dev);
  int st = g_arch[dev].load(std::memory_order_relaxed);
  if (st == 0) {
    hipDeviceProp_t p;
    e = hipGetDeviceProperties(&p, dev);
    if (e != hipSuccess) return fail(MOE_ERR_DEVICE, "hipGetDeviceProperties failed: %s", hipGetErrorString(e));
    st = strncmp(p.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_arch[dev].store(st, std::memory_order_relaxed);
  }
  if (st != 1) return fail(MOE_ERR_UNSUPPORTED, "device %d is not gfx950 (MI355X); this library targets gfx950 only", dev);
  return MOE_OK;
}

// Stage i of a call takes events 2i (start of its first kernel) and 2i+1 (end of its last).
struct Stager {
  int i = 0;
  Stager() = default;
  ~Stager() { g_kstart = g_kstop = nullptr; }
  void begin() {
    g_kstart = 2 * i < g_nevents ? (hipEvent_t)g_events[2 * i] : nullptr;
    g_kstop = 2 * i + 1 < g_nevents ? (hipEvent_t)g_events[2 * i + 1] : nullptr;
  }
  void end() {
    g_kstart = g_kstop = nullptr;
    ++i;
  }
};

moe_status launched(hipError_t e, const char *what) {
  if (e != hipSuccess) return fail(MOE_ERR_DEVICE, "%s: launch failed: %s", what, hipGetErrorString(e));
  return MOE_OK;
}

// ---------------------------------------------------------------- bank validation
moe_status check_bank(const moe_bank *b, const char *name, int H, bool need_n, int n_expected) {
  if (b->wtype != MOE_W_BF16 && b->wtype != MOE_W_FP8_E4M3 && b->wtype != MOE_W_FP8_E4M3_A8 &&
      b->wtype != MOE_W_MXFP4)
    return fail(MOE_ERR_INVALID_ARG,
                "%s.wtype = %d: must be MOE_W_BF16 (0), MOE_W_FP8_E4M3 (1), MOE_W_FP8_E4M3_A8 (2) or MOE_W_MXFP4 (3)",
                name, b->wtype);
  if (need_n && b->num_experts != n_expected)
    return fail(MOE_ERR_INVALID_ARG, "%s.num_experts = %d: expected %d", name, b->num_experts, n_expected);
  if (b->hidden != H) return fail(MOE_ERR_INVALID_ARG, "%s.hidden = %d: expected H = %d", name, b->hidden, H);
  if (b->inter < 64 || b->inter % 64 != 0 || b->inter > 8192)
    return fail(MOE_ERR_INVALID_ARG, "%s.inter = %d: must be a multiple of 64 in [64, 8192]", name, b->inter);
  if (b->w_gate_up == nullptr || b->w_down == nullptr)
    return fail(MOE_ERR_INVALID_ARG, "%s: w_gate_up and w_down are required", name);
  if (!aligned16(b->w_gate_up) || !aligned16(b->w_down))
    return fail(MOE_ERR_MISALIGNED, "%s: weight pointers must be 16-byte aligned", name);
  if (b->wtype == MOE_W_MXFP4) {
    if (b->mx_gate_up == nullptr || b->mx_down == nullptr)
      return fail(MOE_ERR_INVALID_ARG, "%s: MXFP4 weights need the mx_gate_up and mx_down block scales", name);
  } else if (b->wtype != MOE_W_BF16) {
    if (b->s_gate_up == nullptr || b->s_down == nullptr)
      return fail(MOE_ERR_INVALID_ARG, "%s: fp8 weights need s_gate_up and s_down row scales", name);
    if (!aligned4(b->s_gate_up) || !aligned4(b->s_down))
      return fail(MOE_ERR_MISALIGNED, "%s: scale pointers must be 4-byte aligned", name);
  }
  return MOE_OK;
}

moe_status check_hidden(int H) {
  if (H < 64 || H % 64 != 0 || H > 8192)
    return fail(MOE_ERR_INVALID_ARG, "hidden = %d: must be a multiple of 64 in [64, 8192]", H);
  return MOE_OK;
}

moe_status check_ek(int E, int k) {
  if (E < 1 || E > kMaxExperts) return fail(MOE_ERR_INVALID_ARG, "num_experts = %d: must be in [1, %d]", E, kMaxExperts);
  const int kmax = E < kMaxTopK ? E : kMaxTopK;
  if (k < 1 || k > kmax) return fail(MOE_ERR_INVALID_ARG, "top_k = %d: must be in [1, min(E, %d)] = [1, %d]", k, kMaxTopK, kmax);
  return MOE_OK;
}

// ---------------------------------------------------------------- layer plan
enum Path { PATH_NONE = 0, PATH_DECODE = 1, PATH_PREFILL = 2 };

struct LayerPlan {
  Path path = PATH_NONE;
  int BM = 16;
  int64_t cap = 0;
  size_t off_logits, off_gate, off_ids, off_w, off_gamma, off_counts, off_offsets, off_np, off_sorted, off_bexp;
  size_t off_h, off_hs, off_hist, off_y, off_ys, off_tl, off_bar;
  size_t off_x8 = 0, off_sx = 0, off_h8 = 0, off_sh = 0, off_hs8 = 0, off_shs = 0;  // fp8 activations
  size_t total = 0;
};

bool is_decode(int T, int k) { return T <= kDecodeMaxT && (int64_t)T * k <= kSmallSlots; }

LayerPlan plan_layer(int T, const moe_layer *L) {
  LayerPlan p;
  if (T == 0) return p;
  const int H = L->hidden, E = L->num_experts, k = L->top_k, I = L->routed.inter;
  const bool shared = L->shared.num_experts > 0;
  const int I_s = shared ? L->shared.inter : 0;
  const int64_t n = (int64_t)T * k;
  p.path = is_decode(T, k) ? PATH_DECODE : PATH_PREFILL;
  p.BM = p.path == PATH_DECODE ? 16 : 64;
  p.cap = capacity(T, k, E, p.BM);
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t r = o;
    o = align_up(o + bytes, 256);
    return r;
  };
  // the fused kernel's synchronisation words first, in every plan: calls of any size may
  // share one workspace without another buffer overwriting them
  p.off_bar = take((size_t)kBarrierWords * 4);
  p.off_logits = take((size_t)T * E * 4);
  p.off_gate = take((size_t)T * 4);
  p.off_ids = take((size_t)n * 4);
  p.off_w = take((size_t)n * 4);
  p.off_gamma = take((size_t)T * 4);
  p.off_counts = take((size_t)E * 4);
  p.off_offsets = take((size_t)(E + 1) * 4);
  p.off_np = take(4);
  p.off_sorted = take((size_t)p.cap * 4);
  p.off_bexp = take((size_t)(p.cap / p.BM) * 4);
  if (p.path == PATH_DECODE) {
    p.off_h = take((size_t)n * I * 2);
    p.off_hs = take((size_t)T * I_s * 2);
    p.off_tl = take(touched_ints(E, n) * 4);
    p.off_hist = p.off_y = p.off_ys = 0;
  } else {
    p.off_hist = take(align_hist_ints(n, E) * 4);
    p.off_h = take((size_t)p.cap * I * 2);
    p.off_hs = take((size_t)T * I_s * 2);
    p.off_y = take((size_t)n * H * 2);
    p.off_ys = take((size_t)T * H * 2);
    p.off_tl = 0;
    if (L->routed.wtype == MOE_W_FP8_E4M3_A8) {
      p.off_x8 = take((size_t)T * H);
      p.off_sx = take((size_t)T * 4);
      p.off_h8 = take((size_t)p.cap * I);
      p.off_sh = take((size_t)p.cap * 4);
      p.off_hs8 = take((size_t)T * I_s);
      p.off_shs = take((size_t)T * 4);
    }
  }
  p.total = o;
  return p;
}

moe_status validate_layer(int T, const moe_layer *L) {
  if (L == nullptr) return fail(MOE_ERR_INVALID_ARG, "layer descriptor is NULL");
  if (T < 0) return fail(MOE_ERR_INVALID_ARG, "T = %d: must be >= 0", T);
  moe_status st;
  if ((st = check_hidden(L->hidden)) != MOE_OK) return st;
  if ((st = check_ek(L->num_experts, L->top_k)) != MOE_OK) return st;
  if (L->router_w == nullptr) return fail(MOE_ERR_INVALID_ARG, "router_w is required");
  if (!aligned16(L->router_w)) return fail(MOE_ERR_MISALIGNED, "router_w must be 16-byte aligned");
  if (L->router_b != nullptr && !aligned4(L->router_b)) return fail(MOE_ERR_MISALIGNED, "router_b must be 4-byte aligned");
  if ((st = check_bank(&L->routed, "routed", L->hidden, true, L->num_experts)) != MOE_OK) return st;
  if (L->shared.num_experts != 0) {
    if ((st = check_bank(&L->shared, "shared", L->hidden, true, 1)) != MOE_OK) return st;
    if (L->shared.wtype != L->routed.wtype)
      return fail(MOE_ERR_UNSUPPORTED, "shared.wtype = %d differs from routed.wtype = %d", L->shared.wtype, L->routed.wtype);
    if (L->shared_gate_w == nullptr) return fail(MOE_ERR_INVALID_ARG, "shared_gate_w is required with a shared expert");
    if (!aligned16(L->shared_gate_w)) return fail(MOE_ERR_MISALIGNED, "shared_gate_w must be 16-byte aligned");
  }
  if (T > 0 && !is_decode(T, L->top_k)) {
    if (L->routed.wtype == MOE_W_MXFP4)
      return fail(MOE_ERR_UNSUPPORTED, "MXFP4 experts run on the decode path only (T <= %d and T*k <= %d; T = %d)",
                  kDecodeMaxT, kSmallSlots, T);
    if (L->hidden % 128 != 0)
      return fail(MOE_ERR_UNSUPPORTED, "prefill path needs hidden %% 128 == 0 (hidden = %d)", L->hidden);
    // fp8 activations: 128 codes of K per stage in both expert GEMMs
    if (L->routed.wtype == MOE_W_FP8_E4M3_A8 &&
        (L->routed.inter % 128 != 0 || (L->shared.num_experts != 0 && L->shared.inter % 128 != 0)))
      return fail(MOE_ERR_UNSUPPORTED, "fp8 activations on the prefill path need inter %% 128 == 0 (inter = %d%s)",
                  L->routed.inter, L->shared.num_experts != 0 ? ", or the shared expert's" : "");
  }
  return MOE_OK;
}

// The decode kernels read fp8 banks of either fp8 type the same way: GEMVs stream the
// weights with bf16 activations (quantising the activations saves no bytes there).
int decode_wtype(int wtype) { return wtype == MOE_W_FP8_E4M3_A8 ? MOE_W_FP8_E4M3 : wtype; }

void fill_gemv(GemvArgs &g, const uint16_t *x, int T, int H, int k, const moe_bank *routed, int E) {
  memset(&g, 0, sizeof(g));
  g.x = x;
  g.T = T;
  g.H = H;
  g.k = k;
  g.wtype = decode_wtype(routed->wtype);
  g.E = E;
  g.I = routed->inter;
  g.w_gu = routed->w_gate_up;
  g.s_gu = routed->s_gate_up;
  g.w_d = routed->w_down;
  g.s_d = routed->s_down;
  g.x_gu = routed->mx_gate_up;
  g.x_d = routed->mx_down;
}

// ---------------------------------------------------------------- allocation-free entry point
// The scratch moe_layer_forward_noalloc uses in place of a caller's workspace: a file-scope
// device array; every device the library runs on holds its own copy until the process ends.
// In host code its name stands for a host-side shadow, not a device address: the device
// address of each device's copy comes from hipGetSymbolAddress (once per device, with that
// device current), and only that address is handed to kernels.
constexpr size_t kScratchBytes = (size_t)8 << 20;

}  // namespace

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

std::mutex g_scratch_mu;
void *g_scratch_ptr[64];

// Clears the first n words of the scratch (the fused kernel's synchronisation words) with a
// kernel, not a memset, so that the clear may also be captured into a HIP graph.
__global__ void clear_words_kernel(unsigned *p, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0u;
}

// The current device's scratch address; on the device's first use, its synchronisation words
// are cleared on the caller's stream (the array also starts zeroed when the code object loads).
moe_status scratch_for_current_device(void **out, hipStream_t s) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MOE_ERR_DEVICE, "hipGetDevice failed: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= 64) return fail(MOE_ERR_UNSUPPORTED, "device index %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(MOE_ERR_DEVICE, "hipGetSymbolAddress of the scratch failed: %s", hipGetErrorString(e));
    hipLaunchKernelGGL(clear_words_kernel, dim3(4), dim3(256), 0, s, (unsigned *)p, kBarrierWords);
    e = hipGetLastError();
    if (e != hipSuccess) return fail(MOE_ERR_DEVICE, "clearing the scratch failed: %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

// ---------------------------------------------------------------- the shared expert's stream
// At prefill the shared expert depends on the tokens only, so its two GEMMs run on a stream of
// their own while the router, the top-k and the alignment run on the caller's (veloGB10
// README, "Kernel work": shared-expert work overlapped with the MoE step).  One stream and two
// events per device, made on first use; a call holds the device's lock from the fork to the
// join so that concurrent calls from several host threads keep their own dependencies.
struct SideStream {
  std::mutex mu;
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};
SideStream g_side[64];

// The device's side stream, locked into `lock`, or null (then the shared expert runs in order
// on the caller's stream).  Nothing is created while the caller's stream is being captured
// into a graph: creating a stream there could invalidate the capture.
SideStream *side_stream(hipStream_t caller, std::unique_lock<std::mutex> &lock) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  SideStream &ss = g_side[dev];
  lock = std::unique_lock<std::mutex>(ss.mu);
  if (ss.s == nullptr) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(caller, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) return nullptr;
    hipStream_t st = nullptr;
    hipEvent_t ef = nullptr, ej = nullptr;
    if (hipStreamCreateWithFlags(&st, hipStreamNonBlocking) != hipSuccess) return nullptr;
    if (hipEventCreateWithFlags(&ef, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&ej, hipEventDisableTiming) != hipSuccess) {
      if (ef != nullptr) (void)hipEventDestroy(ef);
      (void)hipStreamDestroy(st);
      return nullptr;
    }
    ss.s = st;
    ss.fork = ef;
    ss.join = ej;
  }
  return &ss;
}

// Once the side stream has forked, every return -- also an early one on a failed launch --
// leaves the caller's stream waiting for the side stream's work, so that no kernel of the call
// still writes the workspace after the caller's stream has moved past it.
struct SideJoin {
  SideStream *side = nullptr;
  hipStream_t caller = nullptr;
  ~SideJoin() {
    if (side != nullptr) {
      (void)hipEventRecord(side->join, side->s);
      (void)hipStreamWaitEvent(caller, side->join, 0);
    }
  }
};

moe_status layer_forward(const uint16_t *x, int32_t T, const moe_layer *L, uint16_t *out, float *logits_out,
                         int32_t *ids_out, float *w_out, void *ws, size_t ws_bytes, void *stream, bool allow_side);

}  // namespace

// ======================================================================== exported
extern "C" {

size_t moe_align_capacity(int32_t T, int32_t k, int32_t E, int32_t BM) {
  if (T < 0 || k < 1 || E < 1 || !valid_bm(BM)) return 0;
  return (size_t)capacity(T, k, E, BM);
}

size_t moe_align_workspace_size(int32_t T, int32_t k, int32_t E) {
  if (T < 0 || k < 1 || E < 1) return 0;
  const int64_t n = (int64_t)T * k;
  if (n <= kSmallSlots) return 0;
  return align_hist_ints(n, E) * 4;
}

const char *moe_last_error(void) { return g_err; }

size_t moe_workspace_status_offset(void) { return (size_t)kBarStatus * 4; }

moe_status moe_set_option(int32_t key, int32_t value) {
  if (key == MOE_OPT_DECODE_FUSED) {
    if (value != 0 && value != 1) return fail(MOE_ERR_INVALID_ARG, "MOE_OPT_DECODE_FUSED takes 0 or 1 (got %d)", value);
    g_opt_fused = value;
    return MOE_OK;
  }
  return fail(MOE_ERR_INVALID_ARG, "unknown option key %d", key);
}

moe_status moe_set_stage_events(void *const *events, int32_t n_events) {
  if (events == nullptr || n_events <= 0) {
    g_nevents = 0;
    return MOE_OK;
  }
  if (n_events > 64) return fail(MOE_ERR_INVALID_ARG, "n_events = %d: at most 64", n_events);
  for (int i = 0; i < n_events; ++i) g_events[i] = events[i];
  g_nevents = n_events;
  return MOE_OK;
}

moe_status moe_measure_stream_read(const void *buf, size_t bytes, int32_t blocks, int32_t depth, uint32_t *sink,
                                   void *stream) {
  g_err[0] = 0;
  if (buf == nullptr || sink == nullptr) return fail(MOE_ERR_INVALID_ARG, "buf and sink are required");
  if (bytes == 0 || bytes % 16 != 0) return fail(MOE_ERR_INVALID_ARG, "bytes = %zu: a positive multiple of 16", bytes);
  if ((uintptr_t)buf % 16 != 0 || !aligned4(sink)) return fail(MOE_ERR_MISALIGNED, "buf must be 16-byte and sink 4-byte aligned");
  if (blocks < 1 || blocks > (1 << 20)) return fail(MOE_ERR_INVALID_ARG, "blocks = %d: 1 .. 2^20", blocks);
  if (depth != 4 && depth != 8 && depth != 16) return fail(MOE_ERR_INVALID_ARG, "depth = %d: 4, 8 or 16", depth);
  moe_status st = check_device();
  if (st != MOE_OK) return st;
  return launched(launch_stream_read(buf, bytes / 16, blocks, depth, sink, (hipStream_t)stream), "stream_read");
}

moe_status moe_route_topk(const float *logits, int32_t T, int32_t E, int32_t k, int32_t renormalize,
                          int32_t *topk_ids, float *topk_w, void *stream) {
  g_err[0] = 0;
  if (T < 0) return fail(MOE_ERR_INVALID_ARG, "T = %d: must be >= 0", T);
  moe_status st = check_ek(E, k);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  if (logits == nullptr || topk_ids == nullptr || topk_w == nullptr)
    return fail(MOE_ERR_INVALID_ARG, "logits, topk_ids and topk_w are required");
  if (!aligned4(logits) || !aligned4(topk_ids) || !aligned4(topk_w))
    return fail(MOE_ERR_MISALIGNED, "logits, topk_ids and topk_w must be 4-byte aligned");
  if ((st = check_device()) != MOE_OK) return st;
  return launched(launch_topk(logits, T, E, k, renormalize != 0, topk_ids, topk_w, nullptr, nullptr,
                              (hipStream_t)stream),
                  "moe_route_topk");
}

moe_status moe_align(const int32_t *topk_ids, int32_t T, int32_t k, int32_t E, int32_t BM, int64_t cap,
                     int32_t *sorted_ids, int32_t *block_expert, int32_t *expert_counts, int32_t *expert_offsets,
                     int32_t *num_padded, void *ws, size_t ws_bytes, void *stream) {
  g_err[0] = 0;
  if (T < 0) return fail(MOE_ERR_INVALID_ARG, "T = %d: must be >= 0", T);
  moe_status st = check_ek(E, k);
  if (st != MOE_OK) return st;
  if (!valid_bm(BM)) return fail(MOE_ERR_INVALID_ARG, "BM = %d: must be 16, 32, 64 or 128", BM);
  const int64_t need = capacity(T, k, E, BM);
  if (cap < need) return fail(MOE_ERR_WORKSPACE, "cap = %lld < moe_align_capacity(T=%d, k=%d, E=%d, BM=%d) = %lld",
                              (long long)cap, T, k, E, BM, (long long)need);
  if (cap % BM != 0) return fail(MOE_ERR_INVALID_ARG, "cap = %lld is not a multiple of BM = %d", (long long)cap, BM);
  if (cap > (int64_t)1 << 30) return fail(MOE_ERR_INVALID_ARG, "cap = %lld exceeds 2^30", (long long)cap);
  if (topk_ids == nullptr && T > 0) return fail(MOE_ERR_INVALID_ARG, "topk_ids is required");
  if (sorted_ids == nullptr || block_expert == nullptr || expert_counts == nullptr || expert_offsets == nullptr ||
      num_padded == nullptr)
    return fail(MOE_ERR_INVALID_ARG, "sorted_ids, block_expert, expert_counts, expert_offsets and num_padded are required");
  const int64_t n = (int64_t)T * k;
  const size_t wsz = moe_align_workspace_size(T, k, E);
  if (ws_bytes < wsz || (wsz > 0 && ws == nullptr))
    return fail(MOE_ERR_WORKSPACE, "workspace of %zu bytes < moe_align_workspace_size = %zu", ws_bytes, wsz);
  if ((st = check_device()) != MOE_OK) return st;
  AlignOut al{sorted_ids, block_expert, expert_counts, expert_offsets, num_padded};
  hipError_t e;
  if (n <= kSmallSlots) e = launch_align_small(topk_ids, (int)n, E, BM, cap, al, (hipStream_t)stream);
  else e = launch_align_large(topk_ids, (int)n, E, BM, cap, al, (int32_t *)ws, (hipStream_t)stream);
  return launched(e, "moe_align");
}

size_t moe_experts_workspace_size(int32_t T, int32_t k, const moe_bank *routed, int32_t BM) {
  if (routed == nullptr || T <= 0 || k < 1 || routed->num_experts < 1 || !valid_bm(BM)) return 0;
  const int64_t n = (int64_t)T * k;
  const size_t I = (size_t)routed->inter, H = (size_t)routed->hidden;
  if (is_decode(T, k)) return align_up((size_t)n * I * 2, 256) + align_up(touched_ints(routed->num_experts, n) * 4, 256);
  const int64_t cap = capacity(T, k, routed->num_experts, BM);
  size_t total = align_up((size_t)cap * I * 2, 256) + align_up((size_t)n * H * 2, 256);
  if (routed->wtype == MOE_W_FP8_E4M3_A8)  // tokens and h as fp8 codes with row scales
    total += align_up((size_t)T * H, 256) + align_up((size_t)T * 4, 256) + align_up((size_t)cap * I, 256) +
             align_up((size_t)cap * 4, 256);
  return total;
}

moe_status moe_experts_forward(const uint16_t *x, int32_t T, const moe_bank *routed, int32_t k, const float *topk_w,
                               const int32_t *sorted_ids, const int32_t *block_expert, const int32_t *expert_counts,
                               const int32_t *expert_offsets, int32_t BM, int64_t cap, uint16_t *out, void *ws,
                               size_t ws_bytes, void *stream) {
  g_err[0] = 0;
  if (routed == nullptr) return fail(MOE_ERR_INVALID_ARG, "routed bank is NULL");
  if (T < 0) return fail(MOE_ERR_INVALID_ARG, "T = %d: must be >= 0", T);
  moe_status st;
  if ((st = check_hidden(routed->hidden)) != MOE_OK) return st;
  const int E = routed->num_experts, H = routed->hidden;
  if ((st = check_ek(E, k)) != MOE_OK) return st;
  if ((st = check_bank(routed, "routed", H, false, 0)) != MOE_OK) return st;
  if (!valid_bm(BM)) return fail(MOE_ERR_INVALID_ARG, "BM = %d: must be 16, 32, 64 or 128", BM);
  if (T == 0) return MOE_OK;
  const int64_t need = capacity(T, k, E, BM);
  if (cap < need || cap % BM != 0)
    return fail(MOE_ERR_WORKSPACE, "cap = %lld must be a multiple of BM = %d and >= %lld", (long long)cap, BM,
                (long long)need);
  if (x == nullptr || out == nullptr || topk_w == nullptr || sorted_ids == nullptr || block_expert == nullptr ||
      expert_counts == nullptr || expert_offsets == nullptr)
    return fail(MOE_ERR_INVALID_ARG, "x, out, topk_w and the alignment arrays are required");
  if (!aligned16(x) || !aligned16(out)) return fail(MOE_ERR_MISALIGNED, "x and out must be 16-byte aligned");
  const bool decode = is_decode(T, k);
  if (!decode) {
    if (BM != 64 && BM != 128) return fail(MOE_ERR_UNSUPPORTED, "the prefill path needs BM = 64 or 128 (got %d)", BM);
    if (H % 128 != 0) return fail(MOE_ERR_UNSUPPORTED, "prefill path needs hidden %% 128 == 0 (hidden = %d)", H);
    if (routed->wtype == MOE_W_MXFP4)
      return fail(MOE_ERR_UNSUPPORTED, "MXFP4 experts run on the decode path only (T <= %d; T = %d)", kDecodeMaxT, T);
    if (routed->wtype == MOE_W_FP8_E4M3_A8 && routed->inter % 128 != 0)
      return fail(MOE_ERR_UNSUPPORTED, "fp8 activations on the prefill path need inter %% 128 == 0 (inter = %d)",
                  routed->inter);
  }
  const size_t wsz = moe_experts_workspace_size(T, k, routed, BM);
  if (ws == nullptr || ws_bytes < wsz)
    return fail(MOE_ERR_WORKSPACE, "workspace of %zu bytes < moe_experts_workspace_size = %zu", ws_bytes, wsz);
  if (!aligned16(ws)) return fail(MOE_ERR_MISALIGNED, "workspace must be 16-byte aligned");
  if ((st = check_device()) != MOE_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  if (decode) {
    const int64_t n = (int64_t)T * k;
    const Touched tl = touched_at((int32_t *)((char *)ws + align_up((size_t)n * routed->inter * 2, 256)), E);
    if ((st = launched(launch_compact_touched(expert_counts, expert_offsets, sorted_ids, E, tl, s),
                       "compact_touched")) != MOE_OK)
      return st;
    GemvArgs g;
    fill_gemv(g, x, T, H, k, routed, E);
    g.tl_n = tl.n;
    g.tl_e = tl.e;
    g.tl_start = tl.start;
    g.tl_slots = tl.slots;
    g.topk_w = topk_w;
    g.h = (uint16_t *)ws;
    g.out = out;
    if ((st = launched(launch_gemv_gate_up(g, s, nullptr, 0), "gemv_gate_up")) != MOE_OK) return st;
    return launched(launch_gemv_down(g, s, nullptr, 0), "gemv_down");
  }
  GemmArgs a{};
  a.x = x;
  a.T = T;
  a.H = H;
  a.k = k;
  a.E = E;
  a.I = routed->inter;
  a.BM = BM;
  a.cap = cap;
  a.w_gu = (const uint16_t *)routed->w_gate_up;
  a.w_d = (const uint16_t *)routed->w_down;
  a.sorted = sorted_ids;
  a.block_expert = block_expert;
  a.offsets = expert_offsets;
  a.counts = expert_counts;
  a.wtype = routed->wtype;
  a.s_gu = routed->s_gate_up;
  a.s_d = routed->s_down;
  a.h = (uint16_t *)ws;
  a.y = (uint16_t *)((char *)ws + align_up((size_t)cap * a.I * 2, 256));
  const bool act8 = routed->wtype == MOE_W_FP8_E4M3_A8;
  if (act8) {
    char *q = (char *)a.y + align_up((size_t)T * k * H * 2, 256);
    a.x8 = (const uint8_t *)q;
    q += align_up((size_t)T * H, 256);
    a.sx = (const float *)q;
    q += align_up((size_t)T * 4, 256);
    a.h8 = (uint8_t *)q;
    q += align_up((size_t)cap * a.I, 256);
    a.sh = (float *)q;
    if ((st = launched(launch_quant_tokens(x, T, H, (uint8_t *)a.x8, (float *)a.sx, s), "quant_tokens")) != MOE_OK)
      return st;
  }
  if ((st = launched(launch_gemm_gate_up(a, s), "gemm_gate_up")) != MOE_OK) return st;
  if (act8 && (st = launched(launch_quant_h(a, s), "quant_h")) != MOE_OK) return st;
  if ((st = launched(launch_gemm_down(a, s), "gemm_down")) != MOE_OK) return st;
  return launched(launch_combine(a.y, nullptr, topk_w, nullptr, T, H, k, out, s), "combine");
}

size_t moe_layer_workspace_size(int32_t T, const moe_layer *L) {
  if (L == nullptr || T <= 0) return 0;
  if (L->num_experts < 1 || L->num_experts > kMaxExperts || L->top_k < 1) return 0;
  return plan_layer(T, L).total;
}

const char *moe_describe_plan(int32_t T, const moe_layer *L) {
  g_plan[0] = 0;
  if (validate_layer(T, L) != MOE_OK) {
    snprintf(g_plan, sizeof(g_plan), "invalid: %s", g_err);
    return g_plan;
  }
  if (T == 0) {
    snprintf(g_plan, sizeof(g_plan), "T=0: no kernels");
    return g_plan;
  }
  const LayerPlan p = plan_layer(T, L);
  const int E = L->num_experts, k = L->top_k;
  const bool shared = L->shared.num_experts > 0;
  if (p.path == PATH_DECODE && g_opt_fused != 0 &&
      fused_decode_fits(T, L->hidden, E, k, L->routed.inter, shared ? L->shared.inter : 0,
                        decode_wtype(L->routed.wtype))) {
    snprintf(g_plan, sizeof(g_plan),
             "path=decode-fused T=%d E=%d k=%d BM=%d cap=%lld workspace=%zu stages: 0 moe_decode_fused "
             "(router, top-k, alignment, gate/up, down, combine; one kernel, one grid barrier)",
             T, E, k, p.BM, (long long)p.cap, p.total);
    return g_plan;
  }
  if (p.path == PATH_DECODE) {
    snprintf(g_plan, sizeof(g_plan),
             "path=decode T=%d E=%d k=%d BM=%d cap=%lld workspace=%zu stages: 0 router_rows grid=%d; "
             "1 topk_align_small grid=1x1024; 2 gemv_gate_up; 3 gemv_down_combine",
             T, E, k, p.BM, (long long)p.cap, p.total, (E + (L->shared.num_experts > 0 ? 1 : 0) + 3) / 4);
  } else if (L->routed.wtype == MOE_W_FP8_E4M3_A8) {
    snprintf(g_plan, sizeof(g_plan),
             "path=prefill T=%d E=%d k=%d BM=%d cap=%lld workspace=%zu fp8 activations; stages: 0 router_gemm_mfma; "
             "1 topk; 2 align (align_hist, align_colscan, align_offsets, align_scatter); 3 quant_tokens; "
             "4 gemm_gate_up_mfma (fp8 x fp8); 5 quant_h; 6 gemm_down_mfma (fp8 x fp8); 7 combine",
             T, E, k, p.BM, (long long)p.cap, p.total);
  } else if (shared) {
    snprintf(g_plan, sizeof(g_plan),
             "path=prefill T=%d E=%d k=%d BM=%d cap=%lld workspace=%zu stages: 0 shared_gate_up_mfma "
             "(second stream, beside stages 2-6); 1 shared_down_mfma (second stream); 2 router_gemm_mfma; "
             "3 topk; 4 align (align_hist, align_colscan, align_offsets, align_scatter); 5 gemm_gate_up_mfma "
             "(routed); 6 gemm_down_mfma (routed); 7 combine",
             T, E, k, p.BM, (long long)p.cap, p.total);
  } else {
    snprintf(g_plan, sizeof(g_plan),
             "path=prefill T=%d E=%d k=%d BM=%d cap=%lld workspace=%zu stages: 0 router_gemm_mfma; "
             "1 topk; 2 align (align_hist, align_colscan, align_offsets, align_scatter); 3 gemm_gate_up_mfma; "
             "4 gemm_down_mfma; 5 combine",
             T, E, k, p.BM, (long long)p.cap, p.total);
  }
  return g_plan;
}

moe_status moe_layer_forward(const uint16_t *x, int32_t T, const moe_layer *L, uint16_t *out, float *logits_out,
                             int32_t *ids_out, float *w_out, void *ws, size_t ws_bytes, void *stream) {
  return layer_forward(x, T, L, out, logits_out, ids_out, w_out, ws, ws_bytes, stream, true);
}

}  // extern "C"

namespace {

moe_status layer_forward(const uint16_t *x, int32_t T, const moe_layer *L, uint16_t *out, float *logits_out,
                         int32_t *ids_out, float *w_out, void *ws, size_t ws_bytes, void *stream, bool allow_side) {
  g_err[0] = 0;
  moe_status st = validate_layer(T, L);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  if (x == nullptr || out == nullptr) return fail(MOE_ERR_INVALID_ARG, "x and out are required");
  if (!aligned16(x) || !aligned16(out)) return fail(MOE_ERR_MISALIGNED, "x and out must be 16-byte aligned");
  if ((logits_out && !aligned4(logits_out)) || (ids_out && !aligned4(ids_out)) || (w_out && !aligned4(w_out)))
    return fail(MOE_ERR_MISALIGNED, "logits_out, ids_out and w_out must be 4-byte aligned");
  const LayerPlan p = plan_layer(T, L);
  if (ws == nullptr || ws_bytes < p.total)
    return fail(MOE_ERR_WORKSPACE, "workspace of %zu bytes < moe_layer_workspace_size(T=%d) = %zu", ws_bytes, T, p.total);
  if (!aligned16(ws)) return fail(MOE_ERR_MISALIGNED, "workspace must be 16-byte aligned");
  if ((st = check_device()) != MOE_OK) return st;

  hipStream_t s = (hipStream_t)stream;
  char *base = (char *)ws;
  const int H = L->hidden, E = L->num_experts, k = L->top_k;
  const bool shared = L->shared.num_experts > 0;
  const int64_t n = (int64_t)T * k;
  float *logits = logits_out ? logits_out : (float *)(base + p.off_logits);
  float *gate = (float *)(base + p.off_gate);
  int32_t *ids = ids_out ? ids_out : (int32_t *)(base + p.off_ids);
  float *w = w_out ? w_out : (float *)(base + p.off_w);
  float *gamma = (float *)(base + p.off_gamma);
  AlignOut al{(int32_t *)(base + p.off_sorted), (int32_t *)(base + p.off_bexp), (int32_t *)(base + p.off_counts),
              (int32_t *)(base + p.off_offsets), (int32_t *)(base + p.off_np)};
  Stager sg;

  const bool fused = p.path == PATH_DECODE && g_opt_fused != 0 &&
                     fused_decode_fits(T, H, E, k, L->routed.inter, shared ? L->shared.inter : 0,
                                       decode_wtype(L->routed.wtype));
  if (fused) {
    FusedArgs f{};
    f.x = x;
    f.T = T;
    f.H = H;
    f.E = E;
    f.k = k;
    f.I = L->routed.inter;
    f.I_s = shared ? L->shared.inter : 0;
    f.renorm = L->renormalize != 0;
    f.has_shared = shared ? 1 : 0;
    f.BM = p.BM;
    f.cap = (int)p.cap;
    f.wtype = decode_wtype(L->routed.wtype);
    f.w_r = L->router_w;
    f.b_r = L->router_b;
    f.w_sg = shared ? L->shared_gate_w : nullptr;
    f.w_gu = L->routed.w_gate_up;
    f.s_gu = L->routed.s_gate_up;
    f.w_d = L->routed.w_down;
    f.s_d = L->routed.s_down;
    f.x_gu = L->routed.mx_gate_up;
    f.x_d = L->routed.mx_down;
    if (shared) {
      f.ws_gu = L->shared.w_gate_up;
      f.ss_gu = L->shared.s_gate_up;
      f.ws_d = L->shared.w_down;
      f.ss_d = L->shared.s_down;
      f.xs_gu = L->shared.mx_gate_up;
      f.xs_d = L->shared.mx_down;
    }
    f.logits = logits;
    f.gate_logit = gate;
    f.ids = ids;
    f.topw = w;
    f.gamma = gamma;
    f.al = al;
    f.h = (uint16_t *)(base + p.off_h);
    f.h_s = (uint16_t *)(base + p.off_hs);
    f.out = out;
    f.bar = (unsigned *)(base + p.off_bar);
    sg.begin();
    if ((st = launched(launch_fused_decode(f, s, nullptr, 0), "moe_decode_fused")) != MOE_OK) return st;
    sg.end();
    return MOE_OK;
  }

  if (p.path == PATH_DECODE) {
    sg.begin();
    if ((st = launched(launch_router_rows(x, T, H, L->router_w, L->router_b, E, shared ? L->shared_gate_w : nullptr,
                                          logits, gate, s), "router_rows")) != MOE_OK)
      return st;
    sg.end();
    sg.begin();
    const Touched tl = touched_at((int32_t *)(base + p.off_tl), E);
    if ((st = launched(launch_topk_align_small(logits, shared ? gate : nullptr, T, E, k, L->renormalize != 0, p.BM,
                                               p.cap, ids, w, shared ? gamma : nullptr, al, tl, s),
                       "topk_align_small")) != MOE_OK)
      return st;
    GemvArgs g;
    fill_gemv(g, x, T, H, k, &L->routed, E);
    g.tl_n = tl.n;
    g.tl_e = tl.e;
    g.tl_start = tl.start;
    g.tl_slots = tl.slots;
    g.topk_w = w;
    g.has_shared = shared ? 1 : 0;
    if (shared) {
      g.I_s = L->shared.inter;
      g.ws_gu = L->shared.w_gate_up;
      g.ss_gu = L->shared.s_gate_up;
      g.ws_d = L->shared.w_down;
      g.ss_d = L->shared.s_down;
      g.xs_gu = L->shared.mx_gate_up;
      g.xs_d = L->shared.mx_down;
      g.gamma = gamma;
    }
    g.h = (uint16_t *)(base + p.off_h);
    g.h_s = (uint16_t *)(base + p.off_hs);
    g.out = out;
    sg.end();
    sg.begin();
    if ((st = launched(launch_gemv_gate_up(g, s, nullptr, 0), "gemv_gate_up")) != MOE_OK) return st;
    sg.end();
    sg.begin();
    if ((st = launched(launch_gemv_down(g, s, nullptr, 0), "gemv_down")) != MOE_OK) return st;
    sg.end();
    return MOE_OK;
  }

  // prefill chunk
  GemmArgs a{};
  a.x = x;
  a.T = T;
  a.H = H;
  a.k = k;
  a.E = E;
  a.I = L->routed.inter;
  a.BM = p.BM;
  a.cap = p.cap;
  a.w_gu = (const uint16_t *)L->routed.w_gate_up;
  a.w_d = (const uint16_t *)L->routed.w_down;
  a.sorted = al.sorted;
  a.block_expert = al.block_expert;
  a.offsets = al.offsets;
  a.counts = al.counts;
  a.has_shared = shared ? 1 : 0;
  a.I_s = shared ? L->shared.inter : 0;
  a.ws_gu = shared ? (const uint16_t *)L->shared.w_gate_up : nullptr;
  a.ws_d = shared ? (const uint16_t *)L->shared.w_down : nullptr;
  a.wtype = L->routed.wtype;
  a.s_gu = L->routed.s_gate_up;
  a.s_d = L->routed.s_down;
  a.ss_gu = shared ? L->shared.s_gate_up : nullptr;
  a.ss_d = shared ? L->shared.s_down : nullptr;
  a.h = (uint16_t *)(base + p.off_h);
  a.h_s = (uint16_t *)(base + p.off_hs);
  a.y = (uint16_t *)(base + p.off_y);
  a.y_s = (uint16_t *)(base + p.off_ys);
  const bool act8 = L->routed.wtype == MOE_W_FP8_E4M3_A8;
  if (act8) {
    a.x8 = (const uint8_t *)(base + p.off_x8);
    a.sx = (const float *)(base + p.off_sx);
    a.h8 = (uint8_t *)(base + p.off_h8);
    a.sh = (float *)(base + p.off_sh);
    a.hs8 = shared ? (uint8_t *)(base + p.off_hs8) : nullptr;
    a.shs = shared ? (float *)(base + p.off_shs) : nullptr;
  }
  // the shared expert's gate/up and down as stages of their own, first, on the side stream
  // from the fork (the tokens are ready) to the join before the combine -- or in order on the
  // caller's stream when there is no side stream.  Whole 192-token passes keep the shared
  // expert to about a third of the CUs, so the routing beside it keeps the rest (64-token
  // passes, which spread it over every CU, and its down projection moved after the routed one
  // both measured slower).  fp8 activations keep the one-launch order (their shared rows are
  // quantised with the routed ones).
  const bool split_shared = shared && !act8;
  std::unique_lock<std::mutex> side_lock;
  SideStream *side = split_shared && allow_side ? side_stream(s, side_lock) : nullptr;
  SideJoin side_join;  // (declared after the lock: it runs before the lock is released)
  if (split_shared) {
    hipStream_t ss = s;
    if (side != nullptr) {
      hipError_t e = hipEventRecord(side->fork, s);
      if (e == hipSuccess) e = hipStreamWaitEvent(side->s, side->fork, 0);
      if (e != hipSuccess)
        return fail(MOE_ERR_DEVICE, "forking the shared expert's stream failed: %s", hipGetErrorString(e));
      side_join.side = side;
      side_join.caller = s;
      ss = side->s;
    }
    GemmArgs as = a;
    as.seg_mode = SEG_SHARED;
    sg.begin();
    if ((st = launched(launch_gemm_gate_up(as, ss), "shared gemm_gate_up")) != MOE_OK) return st;
    sg.end();
    sg.begin();
    if ((st = launched(launch_gemm_down(as, ss), "shared gemm_down")) != MOE_OK) return st;
    sg.end();
    if (side != nullptr) {
      const hipError_t e = hipEventRecord(side->join, side->s);
      if (e != hipSuccess)
        return fail(MOE_ERR_DEVICE, "recording the shared expert's join failed: %s", hipGetErrorString(e));
    }
    a.seg_mode = SEG_ROUTED;
  }
  sg.begin();
  if ((st = launched(launch_router_gemm(x, T, H, L->router_w, L->router_b, E, shared ? L->shared_gate_w : nullptr,
                                        logits, gate, s),
                     "router_gemm")) != MOE_OK)
    return st;
  sg.end();
  sg.begin();
  if ((st = launched(launch_topk(logits, T, E, k, L->renormalize != 0, ids, w, shared ? gate : nullptr,
                                 shared ? gamma : nullptr, s), "topk")) != MOE_OK)
    return st;
  sg.end();
  sg.begin();
  if ((st = launched(launch_align_large(ids, (int)n, E, p.BM, p.cap, al, (int32_t *)(base + p.off_hist), s),
                     "align")) != MOE_OK)
    return st;
  sg.end();
  if (act8) {
    sg.begin();
    if ((st = launched(launch_quant_tokens(x, T, H, (uint8_t *)a.x8, (float *)a.sx, s), "quant_tokens")) != MOE_OK)
      return st;
    sg.end();
  }
  sg.begin();
  if ((st = launched(launch_gemm_gate_up(a, s), "gemm_gate_up")) != MOE_OK) return st;
  sg.end();
  if (act8) {
    sg.begin();
    if ((st = launched(launch_quant_h(a, s), "quant_h")) != MOE_OK) return st;
    sg.end();
  }
  sg.begin();
  if ((st = launched(launch_gemm_down(a, s), "gemm_down")) != MOE_OK) return st;
  sg.end();
  if (side != nullptr) {
    side_join.side = nullptr;  // joined here, with its status checked
    const hipError_t e = hipStreamWaitEvent(s, side->join, 0);
    if (e != hipSuccess) return fail(MOE_ERR_DEVICE, "joining the shared expert's stream failed: %s", hipGetErrorString(e));
  }
  sg.begin();
  if ((st = launched(launch_combine(a.y, shared ? a.y_s : nullptr, w, shared ? gamma : nullptr, T, H, k, out, s),
                     "combine")) != MOE_OK)
    return st;
  sg.end();
  return MOE_OK;
}

}  // namespace

extern "C" {

moe_status moe_layer_forward_noalloc(const uint16_t *x, int32_t T, const moe_layer *L, uint16_t *out,
                                     float *logits_out, int32_t *ids_out, float *w_out, void *stream) {
  g_err[0] = 0;
  moe_status st = validate_layer(T, L);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  const size_t need = plan_layer(T, L).total;
  if (need > kScratchBytes)
    return fail(MOE_ERR_WORKSPACE,
                "T = %d needs %zu bytes of scratch; the library's static scratch holds %zu (call "
                "moe_layer_forward with a workspace of moe_layer_workspace_size bytes)",
                T, need, kScratchBytes);
  if ((st = check_device()) != MOE_OK) return st;
  void *ws = nullptr;
  if ((st = scratch_for_current_device(&ws, (hipStream_t)stream)) != MOE_OK) return st;
  // no side stream here: its first use would create a stream and events
  return layer_forward(x, T, L, out, logits_out, ids_out, w_out, ws, kScratchBytes, stream, false);
}

}  // extern "C"
