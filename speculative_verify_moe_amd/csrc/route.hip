// route.hip -- router logits, top-k routing and token-to-expert alignment for gfx950.
//
// Router: veloGB10 README, "Kernel work" ("router fold spread across more of the
// GPU"): at decode the router is a 2-4 MiB fp32 read on the serial head of the
// layer, so every wavefront takes one router row for all tokens and the rows spread
// over all CUs.
// Top-k: Qwen3.8 Flash-Next . GB10 UltraFast, "How it works" (a sort-free
// verify-path top-k): one wavefront per token holds the token's E logits in
// registers as order-preserving 32-bit codes; each of the k rounds is a wavefront
// maximum with ties to the lower expert index, and the winner is retired (topk.h).
// Alignment: Qwen3.8 Flash-Next . GB10 UltraFast, first bullet (moe_align_block_size
// with an arrival-order shim): counts come from integer LDS atomics (their final
// value does not depend on arrival order) and each slot's place inside its expert's
// segment is its rank among earlier slots of the same expert, so the output is the
// stable order by slot index whatever the thread timing.
#include "device.h"
#include "internal.h"
#include "topk.h"

namespace moe {

// ============================================================ router (decode)
// One wavefront per router row n (n < E: expert rows, n == E: the shared gate row) and
// block row y per chunk of kRouterTB tokens, so that a 16-token block fills the chip
// (blockIdx.y splits the tokens; a router row is read once per chunk, from L2 after the
// first).  The wavefront's fp32 row is loaded into registers first (lane l owns float4
// groups g = l + 64c), the block stages its tokens into LDS while those loads are in
// flight (kStage loads per thread in flight together), then each token is one register
// dot product and one DPP reduction.
constexpr int kRouterLds = 64 * 1024;
constexpr int kRouterTB = 4;

template <int C>
__global__ __launch_bounds__(256) void router_rows_kernel(const uint16_t *__restrict__ x, int T, int H,
                                                          const float *__restrict__ w_r,
                                                          const float *__restrict__ b_r, int E,
                                                          const float *__restrict__ w_sg,
                                                          float *__restrict__ logits,
                                                          float *__restrict__ gate_logit) {
  extern __shared__ uint4 s_x[];
  const int lane = lane_id();
  const int n = blockIdx.x * 4 + wave_id();
  const int NR = E + (w_sg != nullptr ? 1 : 0);
  const bool active = n < NR;
  const int G4 = H / 4;
  float4 w[C];
  if (active) {
    const float4 *row = reinterpret_cast<const float4 *>(n < E ? w_r + (size_t)n * H : w_sg);
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const int g = lane + kWave * c;
      if (g < G4) {
        const uint4 u = ld_stream(reinterpret_cast<const uint4 *>(row + g));
        w[c] = make_float4(__uint_as_float(u.x), __uint_as_float(u.y), __uint_as_float(u.z), __uint_as_float(u.w));
      } else {
        w[c] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
  }
  const float bias = (active && n < E && b_r != nullptr) ? b_r[n] : 0.0f;
  const int TP = min(kRouterLds / (H * 2), kRouterTB);
  const int G8 = H / 8;
  const uint2 *sx2 = reinterpret_cast<const uint2 *>(s_x);
  const int tb0 = blockIdx.y * TP, tb1 = min(T, tb0 + TP);
  for (int t0 = tb0; t0 < tb1; t0 += TP) {
    const int nt = tb1 - t0;
    const uint4 *src = reinterpret_cast<const uint4 *>(x + (size_t)t0 * H);
    constexpr int kStage = 8;
    for (int i0 = threadIdx.x; i0 < nt * G8; i0 += 256 * kStage) {
      uint4 v[kStage];
#pragma unroll
      for (int j = 0; j < kStage; ++j)
        if (i0 + 256 * j < nt * G8) v[j] = src[i0 + 256 * j];
#pragma unroll
      for (int j = 0; j < kStage; ++j)
        if (i0 + 256 * j < nt * G8) s_x[i0 + 256 * j] = v[j];
    }
    __syncthreads();
    if (!active) continue;
    for (int i = 0; i < nt; i += 4) {
      float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < C; ++c) {
        const int g = lane + kWave * c;
        if (g < G4) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            if (i + j < nt) {
              const uint2 xv = sx2[(size_t)(i + j) * G4 + g];
              float a = acc[j];
              a = fmaf(w[c].x, bf16_lo(xv.x), a);
              a = fmaf(w[c].y, bf16_hi(xv.x), a);
              a = fmaf(w[c].z, bf16_lo(xv.y), a);
              a = fmaf(w[c].w, bf16_hi(xv.y), a);
              acc[j] = a;
            }
          }
        }
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (i + j < nt) {
          const float v = wave_sum(acc[j]);
          const int t = t0 + i + j;
          if (lane == 0) {
            if (n < E) logits[(size_t)t * E + n] = v + bias;
            else gate_logit[t] = v;
          }
        }
      }
    }
  }
}

hipError_t launch_router_rows(const uint16_t *x, int T, int H, const float *w_r, const float *b_r, int E,
                              const float *w_sg, float *logits, float *gate_logit, hipStream_t s) {
  const int NR = E + (w_sg != nullptr ? 1 : 0);
  const int TP = std::min(kRouterLds / (H * 2), kRouterTB);
  dim3 grid((NR + 3) / 4, (T + TP - 1) / TP), block(256);
  const size_t lds = (size_t)(T < TP ? T : TP) * H * 2;
  const int C = (H / 4 + kWave - 1) / kWave;
  if (C <= 2) return launch_k(router_rows_kernel<2>, grid, block, lds, s, x, T, H, w_r, b_r, E, w_sg, logits, gate_logit);
  else if (C <= 4) return launch_k(router_rows_kernel<4>, grid, block, lds, s, x, T, H, w_r, b_r, E, w_sg, logits, gate_logit);
  else if (C <= 8) return launch_k(router_rows_kernel<8>, grid, block, lds, s, x, T, H, w_r, b_r, E, w_sg, logits, gate_logit);
  else if (C <= 16) return launch_k(router_rows_kernel<16>, grid, block, lds, s, x, T, H, w_r, b_r, E, w_sg, logits, gate_logit);
  else return launch_k(router_rows_kernel<32>, grid, block, lds, s, x, T, H, w_r, b_r, E, w_sg, logits, gate_logit);
}

// ============================================================ top-k (one wavefront per token): topk.h
template <int EPL>
__global__ __launch_bounds__(256) void topk_kernel(const float *__restrict__ logits, int T, int E, int k,
                                                   int renorm, int32_t *__restrict__ ids, float *__restrict__ w,
                                                   const float *__restrict__ gate_logit,
                                                   float *__restrict__ gamma) {
  const int t = blockIdx.x * 4 + wave_id();
  if (t >= T) return;
  topk_wave<EPL>(logits + (size_t)t * E, E, k, renorm, ids + (size_t)t * k, w + (size_t)t * k, nullptr);
  if (gamma != nullptr && lane_id() == 0) gamma[t] = 1.0f / (1.0f + expf(-gate_logit[t]));
}

hipError_t launch_topk(const float *logits, int T, int E, int k, int renorm, int32_t *ids, float *w,
                       const float *gate_logit, float *gamma, hipStream_t s) {
  dim3 grid((T + 3) / 4), block(256);
  const int epl = (E + kWave - 1) / kWave;
  if (epl <= 1) return launch_k(topk_kernel<1>, grid, block, 0, s, logits, T, E, k, renorm, ids, w, gate_logit, gamma);
  else if (epl <= 2) return launch_k(topk_kernel<2>, grid, block, 0, s, logits, T, E, k, renorm, ids, w, gate_logit, gamma);
  else if (epl <= 4) return launch_k(topk_kernel<4>, grid, block, 0, s, logits, T, E, k, renorm, ids, w, gate_logit, gamma);
  else if (epl <= 8) return launch_k(topk_kernel<8>, grid, block, 0, s, logits, T, E, k, renorm, ids, w, gate_logit, gamma);
  else return launch_k(topk_kernel<16>, grid, block, 0, s, logits, T, E, k, renorm, ids, w, gate_logit, gamma);
}

// ============================================================ alignment, one block (n <= 1024, E <= 1024)
// s_ids: the n slot ids in LDS.  1024 threads.  Writes every output array and, when
// tl.n is not null, the compact touched-expert list of the decode kernels.
struct AlignLds {
  int32_t cnt[kMaxExperts];
  int32_t off[kMaxExperts + 1];
  int32_t cstart[kMaxExperts];
  int tmp[1024 / kWave + 1];
  // per wavefront of slots: how many of them chose each expert (<= 64), 4 to a word
  uint32_t whist[1024 / kWave][kMaxExperts / 4];
};

__device__ __forceinline__ void align_block(const int32_t *s_ids, int n, int E, int BM, int cap, AlignLds &L,
                                            AlignOut al, Touched tl) {
  constexpr int NT = 1024, NW = NT / kWave;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), w = tid / kWave;
  const int EW = (E + 3) / 4;  // words of one wavefront's counts
  // a slot's rank among the earlier slots of its expert: for a few slots, a count over the
  // earlier slots; for many, inside its wavefront one ballot per distinct expert, led by its
  // first lane (the leader stores the wavefront's count), plus the earlier wavefronts' counts
  const bool by_ballot = n > 256;
  if (tid < E) L.cnt[tid] = 0;
  if (by_ballot)
    for (int j = tid; j < NW * EW; j += NT) L.whist[j / EW][j % EW] = 0u;
  __syncthreads();
  if (tid < n) atomicAdd(&L.cnt[s_ids[tid]], 1);
  const int se = tid < n ? s_ids[tid] : -1;
  int r = 0;
  uint64_t todo = by_ballot ? __ballot(se >= 0) : 0ull;
  while (todo != 0) {
    const int leader = __builtin_ctzll(todo);
    const int v = __builtin_amdgcn_readlane(se, leader);
    const uint64_t m = __ballot(se == v);
    if (se == v) r = (int)__popcll(m & ((1ull << lane) - 1ull));
    if (lane == leader) L.whist[w][v >> 2] |= (uint32_t)__popcll(m) << (8 * (v & 3));
    todo &= ~m;
  }
  __syncthreads();
  const int c = tid < E ? L.cnt[tid] : 0;
  const int padded = (c + BM - 1) / BM * BM;
  int total;
  const int excl = block_excl_scan<NT>(padded, L.tmp, &total);
  if (tid < E) L.off[tid] = excl;
  if (tid == 0) L.off[E] = total;
  const bool want_tl = tl.n != nullptr;
  if (want_tl) {
    // touched flags (high half) and counts (low half, <= n <= 1024) in one scan
    int both;
    const int sc = block_excl_scan<NT>((c > 0 ? 1 << 16 : 0) | c, L.tmp, &both);
    const int idx = sc >> 16, cs = sc & 0xFFFF, n_touched = both >> 16, n_slots = both & 0xFFFF;
    if (tid < E) L.cstart[tid] = cs;
    if (c > 0) {
      tl.e[idx] = tid;
      tl.start[idx] = cs;
    }
    if (tid == 0) {
      tl.n[0] = n_touched;
      tl.start[n_touched] = n_slots;
    }
  }
  __syncthreads();
  // the stable order by slot index
  if (se >= 0) {
    if (by_ballot) {
      for (int w2 = 0; w2 < w; ++w2) r += (int)((L.whist[w2][se >> 2] >> (8 * (se & 3))) & 0xFFu);
    } else {
      for (int i = 0; i < tid; ++i) r += (s_ids[i] == se) ? 1 : 0;
    }
    al.sorted[L.off[se] + r] = tid;
    if (want_tl) tl.slots[L.cstart[se] + r] = tid;
  }
  // padding: every position that no slot takes holds the sentinel n (an expert's pad
  // positions follow its slots; past num_padded the tail up to cap); block_expert: the
  // expert of each BM-row block of the padded order, -1 past num_padded
  if (tid < E) {
    for (int p = L.off[tid] + c; p < L.off[tid + 1]; ++p) al.sorted[p] = n;
    for (int b = L.off[tid] / BM; b < L.off[tid + 1] / BM; ++b) al.block_expert[b] = tid;
  }
  for (int p = total + tid; p < cap; p += NT) al.sorted[p] = n;
  for (int b = total / BM + tid; b < cap / BM; b += NT) al.block_expert[b] = -1;
  if (tid < E) {
    al.counts[tid] = L.cnt[tid];
    al.offsets[tid] = L.off[tid];
  }
  if (tid == 0) {
    al.offsets[E] = total;
    al.num_padded[0] = total;
  }
}

__global__ __launch_bounds__(1024) void align_small_kernel(const int32_t *__restrict__ ids, int n, int E, int BM,
                                                           int cap, AlignOut al, Touched tl) {
  __shared__ int32_t s_ids[kSmallSlots];
  __shared__ AlignLds L;
  if (threadIdx.x < n) s_ids[threadIdx.x] = ids[threadIdx.x];
  __syncthreads();
  align_block(s_ids, n, E, BM, cap, L, al, tl);
}

hipError_t launch_align_small(const int32_t *ids, int n, int E, int BM, int64_t cap, AlignOut al, hipStream_t s) {
  return launch_k(align_small_kernel, dim3(1), dim3(1024), 0, s, ids, n, E, BM, (int)cap, al,
                  Touched{nullptr, nullptr, nullptr, nullptr});
}

// Decode head: top-k of all T tokens (16 wavefronts) then the alignment, one block.
template <int EPL>
__global__ __launch_bounds__(1024) void topk_align_small_kernel(const float *__restrict__ logits,
                                                                const float *__restrict__ gate_logit, int T, int E,
                                                                int k, int renorm, int BM, int cap,
                                                                int32_t *__restrict__ ids, float *__restrict__ w,
                                                                float *__restrict__ gamma, AlignOut al, Touched tl) {
  __shared__ int32_t s_ids[kSmallSlots];
  __shared__ AlignLds L;
  for (int t = wave_id(); t < T; t += 1024 / kWave)
    topk_wave<EPL>(logits + (size_t)t * E, E, k, renorm, ids + (size_t)t * k, w + (size_t)t * k,
                   s_ids + t * k);
  if (gamma != nullptr && threadIdx.x < T) gamma[threadIdx.x] = 1.0f / (1.0f + expf(-gate_logit[threadIdx.x]));
  __syncthreads();
  align_block(s_ids, T * k, E, BM, cap, L, al, tl);
}

hipError_t launch_topk_align_small(const float *logits, const float *gate_logit, int T, int E, int k, int renorm,
                                   int BM, int64_t cap, int32_t *ids, float *w, float *gamma, AlignOut al,
                                   Touched tl, hipStream_t s) {
  // more tokens than the block's 16 wavefronts: the top-k spread over the chip first (one
  // wavefront per token, the same arithmetic), then the alignment in one block
  if (T > 1024 / kWave) {
    hipError_t e = launch_topk(logits, T, E, k, renorm, ids, w, gate_logit, gamma, s);
    if (e != hipSuccess) return e;
    return launch_k(align_small_kernel, dim3(1), dim3(1024), 0, s, ids, T * k, E, BM, (int)cap, al, tl);
  }
  const int epl = (E + kWave - 1) / kWave;
  dim3 grid(1), block(1024);
  const int c = (int)cap;
  if (epl <= 1) return launch_k(topk_align_small_kernel<1>, grid, block, 0, s, logits, gate_logit, T, E, k, renorm, BM, c, ids, w, gamma, al, tl);
  else if (epl <= 2) return launch_k(topk_align_small_kernel<2>, grid, block, 0, s, logits, gate_logit, T, E, k, renorm, BM, c, ids, w, gamma, al, tl);
  else if (epl <= 4) return launch_k(topk_align_small_kernel<4>, grid, block, 0, s, logits, gate_logit, T, E, k, renorm, BM, c, ids, w, gamma, al, tl);
  else if (epl <= 8) return launch_k(topk_align_small_kernel<8>, grid, block, 0, s, logits, gate_logit, T, E, k, renorm, BM, c, ids, w, gamma, al, tl);
  else return launch_k(topk_align_small_kernel<16>, grid, block, 0, s, logits, gate_logit, T, E, k, renorm, BM, c, ids, w, gamma, al, tl);
}

// Compact touched-expert list from an existing alignment (counts, offsets, sorted ids).
__global__ __launch_bounds__(1024) void compact_touched_kernel(const int32_t *__restrict__ counts,
                                                               const int32_t *__restrict__ offsets,
                                                               const int32_t *__restrict__ sorted, int E,
                                                               Touched tl) {
  __shared__ int s_tmp[1024 / kWave + 1];
  const int tid = threadIdx.x;
  const int c = tid < E ? counts[tid] : 0;
  int n_touched, n_slots;
  const int idx = block_excl_scan<1024>(c > 0 ? 1 : 0, s_tmp, &n_touched);
  const int cs = block_excl_scan<1024>(c, s_tmp, &n_slots);
  if (c > 0) {
    tl.e[idx] = tid;
    tl.start[idx] = cs;
    const int off = offsets[tid];
    for (int r = 0; r < c; ++r) tl.slots[cs + r] = sorted[off + r];
  }
  if (tid == 0) {
    tl.n[0] = n_touched;
    tl.start[n_touched] = n_slots;
  }
}

hipError_t launch_compact_touched(const int32_t *counts, const int32_t *offsets, const int32_t *sorted, int E,
                                  Touched tl, hipStream_t s) {
  return launch_k(compact_touched_kernel, dim3(1), dim3(1024), 0, s, counts, offsets, sorted, E, tl);
}

// ============================================================ alignment, many blocks (any n)
// 1. per-chunk histograms  hist[c][e]  (chunks of kAlignChunk slots)
// 2. per-expert exclusive scan over chunks (in place) and the counts
// 3. scatter: every block scans the padded counts over the experts itself (the same
//    offsets in every block, with no kernel between); block 0 writes offsets and
//    num_padded, the blocks share block_expert; position = offsets[e] + hist[c][e] + rank
//    inside the chunk; sentinel fill
size_t align_hist_ints(int64_t n, int E) {
  const int64_t chunks = (n + kAlignChunk - 1) / kAlignChunk;
  return (size_t)(chunks * E);
}

__global__ __launch_bounds__(kAlignChunk) void align_hist_kernel(const int32_t *__restrict__ ids, int n, int E,
                                                                 int32_t *__restrict__ hist) {
  __shared__ int32_t s_cnt[kMaxExperts];
  for (int e = threadIdx.x; e < E; e += kAlignChunk) s_cnt[e] = 0;
  __syncthreads();
  const int i = blockIdx.x * kAlignChunk + threadIdx.x;
  if (i < n) atomicAdd(&s_cnt[ids[i]], 1);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kAlignChunk) hist[(size_t)blockIdx.x * E + e] = s_cnt[e];
}

// One block per expert: exclusive scan of hist[.][e] over the chunks.
__global__ __launch_bounds__(256) void align_colscan_kernel(int32_t *__restrict__ hist, int chunks, int E,
                                                            int32_t *__restrict__ counts) {
  __shared__ int s_tmp[256 / kWave + 1];
  const int e = blockIdx.x;
  int carry = 0;
  for (int c0 = 0; c0 < chunks; c0 += 256) {
    const int c = c0 + threadIdx.x;
    const int v = c < chunks ? hist[(size_t)c * E + e] : 0;
    int total;
    const int ex = block_excl_scan<256>(v, s_tmp, &total);
    if (c < chunks) hist[(size_t)c * E + e] = carry + ex;
    carry += total;
  }
  if (threadIdx.x == 0) counts[e] = carry;
}

__global__ __launch_bounds__(kAlignChunk) void align_scatter_kernel(const int32_t *__restrict__ ids, int n, int E,
                                                                    int BM, int cap, const int32_t *__restrict__ hist,
                                                                    AlignOut al) {
  constexpr int NW = kAlignChunk / kWave;
  // per wavefront of the chunk, how many of its slots chose each expert
  __shared__ int32_t s_whist[NW][kMaxExperts];
  // the counts and their padded exclusive scan, in LDS: the sentinel fill searches them per
  // position (a binary search over global memory would be a chain of dependent loads)
  __shared__ int32_t s_off[kMaxExperts + 1];
  __shared__ int32_t s_cnt[kMaxExperts];
  __shared__ int s_tmp[kAlignChunk / kWave + 1];
  constexpr int PER = (kMaxExperts + kAlignChunk - 1) / kAlignChunk;  // experts per thread in the scan
  const int lane = lane_id(), w = wave_id();
  const int i = blockIdx.x * kAlignChunk + threadIdx.x;
  const int e = i < n ? ids[i] : -1;
  for (int j = threadIdx.x; j < NW * E; j += kAlignChunk) s_whist[j / E][j % E] = 0;
  {
    // thread t scans experts PER t .. PER t + PER - 1 (consecutive, so the scan is in expert order)
    int pc[PER], sum = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int ex = PER * threadIdx.x + i;
      const int c = ex < E ? al.counts[ex] : 0;
      if (ex < E) s_cnt[ex] = c;
      pc[i] = (c + BM - 1) / BM * BM;
      sum += pc[i];
    }
    int total;
    int run = block_excl_scan<kAlignChunk>(sum, s_tmp, &total);
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int ex = PER * threadIdx.x + i;
      if (ex < E) s_off[ex] = run;
      run += pc[i];
    }
    if (threadIdx.x == 0) s_off[E] = total;
  }
  __syncthreads();
  if (blockIdx.x == 0) {
    for (int j = threadIdx.x; j <= E; j += kAlignChunk) al.offsets[j] = s_off[j];
    if (threadIdx.x == 0) al.num_padded[0] = s_off[E];
  }
  for (int bb = blockIdx.x * kAlignChunk + threadIdx.x; bb < cap / BM; bb += gridDim.x * kAlignChunk) {
    const int p = bb * BM;
    al.block_expert[bb] = p < s_off[E] ? segment_of(s_off, E, p) : -1;
  }
  // the slot's rank among the chunk's earlier slots of its expert (the chunk's slots in
  // order): inside the wavefront, one ballot per distinct expert, led by its first lane
  int r = 0;
  uint64_t todo = __ballot(e >= 0);
  while (todo != 0) {
    const int leader = __builtin_ctzll(todo);
    const int v = __builtin_amdgcn_readlane(e, leader);
    const uint64_t m = __ballot(e == v);
    if (e == v) r = (int)__popcll(m & ((1ull << lane) - 1ull));
    if (lane == leader) s_whist[w][v] = (int)__popcll(m);
    todo &= ~m;
  }
  __syncthreads();
  if (e >= 0) {
    for (int w2 = 0; w2 < w; ++w2) r += s_whist[w2][e];  // ... and in the earlier wavefronts
    al.sorted[s_off[e] + hist[(size_t)blockIdx.x * E + e] + r] = i;
  }
  const int total = s_off[E];  // num_padded
  for (int p = i; p < cap; p += gridDim.x * kAlignChunk) {
    bool pad = true;
    if (p < total) {
      const int ex = segment_of(s_off, E, p);
      pad = (p - s_off[ex]) >= s_cnt[ex];
    }
    if (pad) al.sorted[p] = n;
  }
}

hipError_t launch_align_large(const int32_t *ids, int n, int E, int BM, int64_t cap, AlignOut al, int32_t *hist,
                              hipStream_t s) {
  const int chunks = (n + kAlignChunk - 1) / kAlignChunk;
  // (each launch's own status: a later hipGetLastError would read it cleared)
  hipError_t e = launch_k(align_hist_kernel, dim3(chunks), dim3(kAlignChunk), 0, s, ids, n, E, hist);
  if (e == hipSuccess) e = launch_k(align_colscan_kernel, dim3(E), dim3(256), 0, s, hist, chunks, E, al.counts);
  if (e == hipSuccess)
    e = launch_k(align_scatter_kernel, dim3(chunks), dim3(kAlignChunk), 0, s, ids, n, E, BM, (int)cap, hist, al);
  return e;
}

}  // namespace moe
