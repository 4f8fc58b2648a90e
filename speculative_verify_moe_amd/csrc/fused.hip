// fused.hip -- the whole decode/verify-block MoE layer in one kernel (gfx950).
//
// veloGB10 README, "Kernel work": the router fold spread across the GPU, several small
// kernels (the expert routing among them) folded into their neighbours, grouped expert
// kernels that never rebuild weights, shared-expert work overlapped with the MoE step.
// Qwen3.8 Flash-Next . GB10 UltraFast, first bullet: a deterministic floor -- alignment
// in slot order and a combine without float atomics.
//
// One block per CU (8 wavefronts); the grid never exceeds what the device holds resident
// at once, so every block runs concurrently and the grid-wide barriers complete.  Four
// phases separated by two barriers:
//   0  tokens staged in LDS; router row n runs on block n % NB, its tokens spread over
//      the block's wavefronts.                                           -- grid sync
//   1  every block routes all T tokens itself from the logits (top-k per wavefront,
//      histogram, scans, stable slot lists in LDS): no launch, no second sync.  Block 0
//      also writes the routing and the padded alignment to global memory.
//   A  gate/up stream: block b owns gate/up row pair b (2b, 2b+1 and I+2b, I+2b+1) of
//      every touched expert and of the shared expert; h goes to global memory.
//                                                                        -- grid sync
//      Each wavefront then issues its first phase-B weight rows while h is staged.
//   B  down stream: h staged in LDS, block b owns output rows 8b..8b+7 of every touched
//      expert and the shared one, y kept in LDS, combine in slot order in fp32.
// Lane mapping as in gemv.hip: four 16-lane DPP rows per wavefront, one weight row each,
// 16-byte column groups per lane, one 4-step DPP sum per dot product set.
//
// Grid barrier: each block stores this call's token into its own flag word, one
// wavefront of block 0 polls all flags with one coalesced load per round and then
// stores the token into a release word that every block polls; spins are bounded, so a
// misuse can give wrong results but never a hang.  Wavefront 0 does the polling and never
// has weight prefetches in flight at a barrier: vector loads return in issue order, so a
// poll queued behind 16 KiB of prefetch would see the flags microseconds late.  Data that crosses a barrier (logits,
// gate logits, h) is written and read with agent-scope atomic accesses (sc1: coherent
// across the XCDs' L2s), so the barrier needs no cache write-back or invalidate --
// every wavefront waits for its own stores to complete before its block arrives.

#include <algorithm>
#include <atomic>
#include <cstdio>
#include <mutex>

#include "device.h"
#include "internal.h"
#include "mxfp4.h"
#include "topk.h"

namespace moe {

namespace {
constexpr int kNW = 8;
constexpr int kNT = kNW * kWave;
constexpr int kOct = 8;  // output rows per block in phase B
// Widths (elements) the lanes' column groups span: H <= kXW, I and I_s <= kHW.  The LDS
// rows of the tokens and of h end in two zero uint4; a lane's column index beyond the row
// is clamped onto them (its weights are zero too), so the dot-product loops have no
// bounds tests and no branch.
constexpr int kXW = 2048;
constexpr int kHW = 512;
}  // namespace

__host__ __device__ __forceinline__ size_t al16(size_t v) { return (v + 15) & ~(size_t)15; }

constexpr unsigned kSpinLimit = 1u << 20;

__device__ __forceinline__ unsigned ld_agent(const unsigned *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(unsigned *p, unsigned v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wait until this wavefront's stores have completed (vmcnt counts loads and stores in
// issue order, so this also waits for earlier loads); the clobber keeps the compiler from
// moving memory operations across it.
__device__ __forceinline__ void wait_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Mark a register buffer as consumed here: the compiler waits for its loads at this point,
// so no later reuse of those registers waits on the loads issued after them.
template <int N>
__device__ __forceinline__ void consume(const uint4 (&w)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) asm volatile("" ::"v"(w[i].x), "v"(w[i].y), "v"(w[i].z), "v"(w[i].w));
}

// Barrier words (kBarrierWords in the workspace): arrival flags [kMaxBlocks], the release
// word, the timeout count.

// flags[kMaxBlocks]: per-block arrival words, then the release word and a timeout count.
// Every wavefront that wrote data the other blocks will read calls wait_stores() first.
// The barrier is split in two: grid_arrive stores the block's arrival word once every
// wavefront got there; grid_wait polls for the release.  Work issued between the two
// (loads only) overlaps the wait without delaying the arrival.
__device__ __forceinline__ void grid_arrive(unsigned *flags, unsigned token) {
  __syncthreads();
  if (threadIdx.x == 0) st_agent(&flags[blockIdx.x], token);
}
__device__ __forceinline__ void grid_wait(unsigned *flags, unsigned token) {
  const unsigned nb = gridDim.x;
  unsigned *rel = flags + kMaxBlocks;
  if (blockIdx.x == 0 && threadIdx.x < kWave) {
    unsigned spins = 0;
    while (true) {
      // every flag of a round loaded at once (no short-circuit chain of loads)
      constexpr int kPer = kMaxBlocks / kWave;
      unsigned v[kPer];
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        const unsigned i = threadIdx.x + kWave * j;
        if (kWave * j < nb) v[j] = ld_agent(&flags[i < nb ? i : nb - 1]);
      }
      bool ok = true;
#pragma unroll
      for (int j = 0; j < kPer; ++j)
        if (kWave * j < nb) ok &= v[j] == token;
      if (__all(ok)) break;
      __builtin_amdgcn_s_sleep(1);
      if (++spins > kSpinLimit) {
        if (threadIdx.x == 0) atomicAdd(rel + 1, 1u);
        break;
      }
    }
    if (threadIdx.x == 0) st_agent(rel, token);
  }
  if (threadIdx.x == 0) {
    unsigned spins = 0;
    while (ld_agent(rel) != token) {
      __builtin_amdgcn_s_sleep(1);
      if (++spins > kSpinLimit) {
        atomicAdd(rel + 1, 1u);
        break;
      }
    }
  }
  asm volatile("" ::: "memory");
  __syncthreads();
}
__device__ __forceinline__ void grid_barrier(unsigned *flags, unsigned token) {
  grid_arrive(flags, token);
  grid_wait(flags, token);
}

// Block barrier for LDS data only: waits for this wavefront's LDS operations but not for
// its vector memory operations, so loads stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// VPG: weights per 16-byte column group -- 8 bf16, 16 fp8 codes, or 32 MXFP4 codes (which
// are also one scale block).  CGU / CGD: column groups per lane and weight row in phase A /
// phase B; CR: float4 router groups per lane.
template <int VPG, int CGU, int CGD, int CR>
__global__ __launch_bounds__(kNT) __attribute__((amdgpu_waves_per_eu(2, 2))) void moe_decode_fused_kernel(FusedArgs a) {
  static_assert(16 * CGU * VPG == kXW && 64 * 4 * CR == kXW, "lanes must span a token row");
  static_assert(16 * CGD * VPG == kHW, "lanes must span an h row");
  extern __shared__ __attribute__((aligned(16))) char smem[];
  constexpr bool kFp4 = VPG == 32;
  constexpr int NSU = kFp4 ? CGU : 1, NSD = kFp4 ? CGD : 1;  // MXFP4 scale bytes per lane and row
  // bytes of n weights (n even)
  auto nbytes = [](auto n) { return kFp4 ? n / 2 : n * (16 / VPG); };
  const int tid = threadIdx.x, lane = lane_id(), wave = wave_id(), rg = lane >> 4, l16 = lane & 15;
  const int NB = gridDim.x;
  const int T = a.T, H = a.H, E = a.E, k = a.k;
  const int n_slots = T * k;
  const int G8 = H / 8;
  const int xg = G8 + 2;                                                // uint4 per LDS token row
  const int hg = ((a.has_shared && a.I_s > a.I) ? a.I_s : a.I) / 8 + 2;  // uint4 per LDS h row

  // ---------------- LDS: routing region, then the data region (x, later h and y)
  int *s_ids = reinterpret_cast<int *>(smem);         // [T*k]
  float *s_topw = reinterpret_cast<float *>(s_ids + n_slots);
  int *s_slots = reinterpret_cast<int *>(s_topw + n_slots);      // [T*k] grouped by expert
  int *s_stok = s_slots + n_slots;                                // [T*k] their tokens
  float *s_gamma = reinterpret_cast<float *>(s_stok + n_slots);   // [64]
  int *s_cnt = reinterpret_cast<int *>(s_gamma + kDecodeMaxT);    // [E]
  int *s_qs = s_cnt + E;                                          // [E] first position of an expert's slots
  int *s_e = s_qs + E;                                            // [E]
  int *s_start = s_e + E;                                         // [E+1]
  int *s_off = s_start + E + 1;                                   // [E+1] padded offsets
  unsigned *s_mlo = reinterpret_cast<unsigned *>(s_off + E + 1);  // [E] tokens 0..31 per expert
  unsigned *s_mhi = s_mlo + E;                                    // [E] tokens 32..63
  __shared__ int s_nt;
  __shared__ int s_qa, s_qb;  // phase A / phase B entry counters
  __shared__ uint32_t s_wsum[2 * kNW];
  char *data = smem + a.lds_route;
  // this call's barrier tokens follow the workspace's last release word: block 0 rewrites it
  // only once every block has arrived, and a block's arrival depends on this load
  const unsigned tok0 = ld_agent(a.bar + kMaxBlocks);

  // ---------------- phase 0: router rows, tokens to LDS
  const int NR = E + (a.w_sg != nullptr ? 1 : 0);
  // Router row n runs on block n % NB; every wavefront of the block holds the row (the
  // block's 8 loads of it share the CU's caches) and takes the tokens wave, wave + 8, ...,
  // so each token's dot product is one short chain.  The block's first kRR rows and their
  // biases are loaded first of all.
  constexpr int kRR = 3;
  float4 wr[kRR][CR];
  float bias[kRR];
  auto load_router_row = [&](float4(&w)[CR], float &b, int n) {
    b = (n < E && a.b_r != nullptr) ? a.b_r[n] : 0.0f;
    const float4 *row = reinterpret_cast<const float4 *>(n < E ? a.w_r + (size_t)n * H : a.w_sg);
#pragma unroll
    for (int c = 0; c < CR; ++c) {
      const int g = lane + kWave * c;
      if (g < H / 4) {
        const uint4 u = ld_stream(reinterpret_cast<const uint4 *>(row + g));
        w[c] = make_float4(__uint_as_float(u.x), __uint_as_float(u.y), __uint_as_float(u.z), __uint_as_float(u.w));
      } else {
        w[c] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
  };

  // phase-A weight buffers; the prefetch wavefront's first entry is the shared expert
  const int NPair = (a.has_shared && a.I_s > a.I ? a.I_s : a.I) / 2;
  uint4 wa[CGU], wb[CGU];
  uint32_t xa[NSU], xb[NSU];  // MXFP4: the E8M0 scale byte of each of the lane's groups
  // Weight rows are streamed with raw buffer loads: the expert's matrix is the buffer (base
  // in scalar registers), the lane's row and column offset one VGPR, the column group a
  // uniform scalar offset.  Exactly CGU (CGD per row set) load instructions, all in range:
  // groups past the row (whole groups: H, I, I_s are multiples of 16 groups) reload the
  // last group and are zeroed where they are used, so nothing waits for a load here.
  typedef int i4_t __attribute__((ext_vector_type(4)));
  constexpr int kNt = 2;  // cache policy: non-temporal (weights are read once)
  auto as_u4 = [](i4_t v) { return make_uint4(v.x, v.y, v.z, v.w); };
  // the lane's byte offset in an expert's gate/up matrix for row pair p (gate rows 2p, 2p+1,
  // up rows Iw+2p, Iw+2p+1): fixed for the whole phase, computed once
  auto gu_row = [&](int Iw, int p) { return rg < 2 ? 2 * p + rg : Iw + 2 * p + (rg - 2); };
  auto gu_voff = [&](int Iw, int p) { return nbytes(gu_row(Iw, p) * H) + l16 * 16; };
  // MXFP4: the lane's byte offset in the matching scale matrix (one byte per group)
  auto gu_soff = [&](int Iw, int p) { return gu_row(Iw, p) * (H / VPG) + l16; };
  // valid == false: an empty descriptor, so the loads return zeros without reading memory
  // (they still issue, which keeps every wait count the same on all paths)
  auto gu_load = [&](uint4(&w)[CGU], uint32_t(&xs)[NSU], bool valid, bool shared, int e, int voff, int soff) {
    e = __builtin_amdgcn_readfirstlane(e);  // uniform (read from LDS): the descriptor stays scalar
    const int Iw = shared ? a.I_s : a.I;
    const uint8_t *bank = shared ? (const uint8_t *)a.ws_gu : (const uint8_t *)a.w_gu + nbytes((size_t)e * 2 * a.I * H);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(bank), 0,
                                                                        valid ? nbytes(2 * Iw * H) : 0, 0x00020000);
    const int last = H / VPG / 16 - 1;
#pragma unroll
    for (int c = 0; c < CGU; ++c) w[c] = as_u4(__builtin_amdgcn_raw_buffer_load_b128(rs, voff, 256 * min(c, last), kNt));
    if (kFp4) {
      const uint8_t *sbank = shared ? (const uint8_t *)a.ss_gu : (const uint8_t *)a.s_gu + (size_t)e * 2 * a.I * (H / VPG);
      const __amdgpu_buffer_rsrc_t rsc = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint8_t *>(sbank), 0, valid ? 2 * Iw * (H / VPG) : 0, 0x00020000);
#pragma unroll
      for (int c = 0; c < NSU; ++c) xs[c] = __builtin_amdgcn_raw_buffer_load_b8(rsc, soff, 16 * min(c, last), kNt);
    }
    // the offsets stay allocated past the loads, so no load lands in their registers (a
    // later write of those registers would have to wait for the load)
    if (kFp4) asm volatile("" ::"v"(voff), "v"(soff));
    else asm volatile("" ::"v"(voff));
  };

  // per lane: the column groups in order, four products each, one accumulation chain;
  // then the wavefront sum (the same order as the router kernel of the four-kernel path)
  auto router_dot = [&](const float4(&w)[CR], float b, int n, int t, const uint2(&xv)[CR]) {
    float acc = 0.0f;
#pragma unroll
    for (int c = 0; c < CR; ++c) {
      acc = fmaf(w[c].x, bf16_lo(xv[c].x), acc);
      acc = fmaf(w[c].y, bf16_hi(xv[c].x), acc);
      acc = fmaf(w[c].z, bf16_lo(xv[c].y), acc);
      acc = fmaf(w[c].w, bf16_hi(xv[c].y), acc);
    }
    const float v = wave_sum(acc);
    if (lane == 0) {
      float *dst = n < E ? a.logits + (size_t)t * E + n : a.gate_logit + t;
      __hip_atomic_store(dst, n < E ? v + b : v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  };
  // The router's critical path: the block's rows and each wavefront's first token (t = wave)
  // straight into registers, before the token staging's loads (loads return in issue
  // order); column groups past the row read the last group and are zeroed (zero weights).
#pragma unroll
  for (int r = 0; r < kRR; ++r)
    if (blockIdx.x + r * NB < NR) load_router_row(wr[r], bias[r], blockIdx.x + r * NB);
  uint2 xt[CR];
  {
    const uint2 *xrow = reinterpret_cast<const uint2 *>(a.x) + (size_t)min(wave, T - 1) * (H / 4);
#pragma unroll
    for (int c = 0; c < CR; ++c) {
      const int g = lane + kWave * c;
      xt[c] = xrow[min(g, H / 4 - 1)];
      if (g >= H / 4) xt[c] = make_uint2(0, 0);
    }
  }

  // tokens to LDS (for phase A and the router's later tokens), in rows of xg uint4 ending
  // in the zero pad; unguarded (clamped) loads, so they are in flight together
  uint4 *sx = reinterpret_cast<uint4 *>(data);
  {
    constexpr int kStep = kNT, kB = 8;
    const uint4 *gx = reinterpret_cast<const uint4 *>(a.x);
    const int n16 = T * xg, last = T * G8 - 1;
    uint4 v[kB];
    auto x_load = [&](int base) {
#pragma unroll
      for (int j = 0; j < kB; ++j) {
        const int i = base + j * kStep, t = i / xg, g = i - t * xg;
        v[j] = gx[min(t * G8 + g, last)];
        if (g >= G8) v[j] = make_uint4(0, 0, 0, 0);
      }
    };
    auto x_store = [&](int base) {
#pragma unroll
      for (int j = 0; j < kB; ++j)
        if (base + j * kStep < n16) sx[base + j * kStep] = v[j];
    };
    x_load(tid);
    if (wave < T) {
#pragma unroll
      for (int r = 0; r < kRR; ++r)
        if (blockIdx.x + r * NB < NR) router_dot(wr[r], bias[r], blockIdx.x + r * NB, wave, xt);
    }
    x_store(tid);
    for (int base = tid + kB * kStep; base < n16; base += kB * kStep) {
      x_load(base);
      x_store(base);
    }
  }
  const uint4 *xs = sx;
  for (int e = tid; e < E; e += kNT) {
    s_mlo[e] = 0u;
    s_mhi[e] = 0u;
  }
  __syncthreads();

  // the wavefront's further tokens and the rows past the first kRR, from the staged tokens
  auto lds_token = [&](uint2(&xv)[CR], int t) {
    const uint2 *x2 = reinterpret_cast<const uint2 *>(xs) + (size_t)t * (2 * xg);
#pragma unroll
    for (int c = 0; c < CR; ++c) xv[c] = x2[min(lane + kWave * c, H / 4)];  // H / 4: the zero pad
  };
  for (int t = wave + kNW; t < T; t += kNW) {
    uint2 xv[CR];
    lds_token(xv, t);
#pragma unroll
    for (int r = 0; r < kRR; ++r)
      if (blockIdx.x + r * NB < NR) router_dot(wr[r], bias[r], blockIdx.x + r * NB, t, xv);
  }
  for (int n = blockIdx.x + kRR * NB; n < NR; n += NB) {  // E + 1 > kRR * NB: the rest
    load_router_row(wr[0], bias[0], n);
    for (int t = wave; t < T; t += kNW) {
      uint2 xv[CR];
      lds_token(xv, t);
      router_dot(wr[0], bias[0], n, t, xv);
    }
  }
  wait_stores();  // the router rows' logit stores
  grid_barrier(a.bar, tok0 + 1u);

  // ---------------- phase 1: routing in every block
  {
    const int epl = (E + kWave - 1) / kWave;
    // per expert, the set of tokens that chose it (T <= 64: two 32-bit words, cleared in
    // phase 0); the k experts of one token are distinct, so a slot's rank inside its
    // expert's group (slot order) is the number of earlier tokens in that set
    for (int t = wave; t < T; t += kNW) {
      const float *lg = a.logits + (size_t)t * E;
      if (epl <= 1) topk_wave<1, true>(lg, E, k, a.renorm, s_ids + t * k, s_topw + t * k, nullptr);
      else if (epl <= 2) topk_wave<2, true>(lg, E, k, a.renorm, s_ids + t * k, s_topw + t * k, nullptr);
      else if (epl <= 4) topk_wave<4, true>(lg, E, k, a.renorm, s_ids + t * k, s_topw + t * k, nullptr);
      else if (epl <= 8) topk_wave<8, true>(lg, E, k, a.renorm, s_ids + t * k, s_topw + t * k, nullptr);
      else topk_wave<16, true>(lg, E, k, a.renorm, s_ids + t * k, s_topw + t * k, nullptr);
      if (lane < k) {
        const int e = s_ids[t * k + lane];
        atomicOr(t < 32 ? &s_mlo[e] : &s_mhi[e], 1u << (t & 31));
      }
    }
    if (a.has_shared && tid < T) {
      const float z = __hip_atomic_load(a.gate_logit + tid, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s_gamma[tid] = 1.0f / (1.0f + expf(-z));
    }
    __syncthreads();
    // The entries (touched experts) in order of first use: slot i = t*k + j opens one when
    // no earlier token chose its expert.  Entry q's slots, in token order, take positions
    // s_start[q] .. s_start[q+1] of s_slots / s_stok.  One wavefront, 64 slots a step:
    // ballots number the entries, a scan over the opening slots places them.  (The order
    // of entries changes no result: every h row and y row depends on its own slot only.)
    if (wave == 0) {
      int nq = 0, pos = 0;
      for (int c0 = 0; c0 < n_slots; c0 += kWave) {
        const int i = c0 + lane;
        const bool v = i < n_slots;
        const int e = v ? s_ids[i] : 0;
        const int t = min(i / k, kWave - 1);
        const uint64_t m = ((uint64_t)s_mhi[e] << 32) | s_mlo[e];
        const bool first = v && (m & ((1ull << t) - 1ull)) == 0;
        const uint64_t fb = __ballot(first);
        const uint32_t cf = first ? (uint32_t)__popcll(m) : 0u;
        const uint32_t incl = wave_incl_scan_u32(cf);
        if (first) {
          const int q = nq + (int)__popcll(fb & ((1ull << lane) - 1ull));
          const int st = pos + (int)(incl - cf);
          s_e[q] = e;
          s_start[q] = st;
          s_qs[e] = st;
        }
        nq += (int)__popcll(fb);
        pos += __builtin_amdgcn_readlane((int)incl, kWave - 1);
      }
      for (int c0 = 0; c0 < n_slots; c0 += kWave) {
        const int i = c0 + lane;
        if (i < n_slots) {
          const int e = s_ids[i], t = i / k;
          const uint64_t m = ((uint64_t)s_mhi[e] << 32) | s_mlo[e];
          const int p = s_qs[e] + (int)__popcll(m & ((1ull << t) - 1ull));
          s_slots[p] = i;
          s_stok[p] = t;
        }
      }
      if (lane == 0) {
        s_start[nq] = n_slots;
        s_nt = nq;
        s_qa = 0;
        s_qb = 0;
      }
    }
    __syncthreads();
  }
  const int nr = s_nt;

  // ---------------- phase A: gate/up of row pair p = b (2b, 2b+1 and I+2b, I+2b+1) for
  // every entry: entry 0 is the shared expert when this pair has one, then the touched
  // experts in order of first use.  The wavefronts take entries from an LDS counter, two in
  // flight each.
  const int pA = blockIdx.x;
  const bool shA = a.has_shared && 2 * pA < a.I_s;
  const int NEA = pA < NPair ? (2 * pA < a.I ? nr : 0) + (shA ? 1 : 0) : 0;
  {
    auto compute = [&](uint4(&w)[CGU], const uint32_t(&xsc)[NSU], int q) {
      consume(w);
      // column groups past the row (whole groups) hold a repeated load: zero them in place
#pragma unroll
      for (int c = 0; c < CGU; ++c)
        if (16 * c >= H / VPG) w[c] = make_uint4(0, 0, 0, 0);
      const bool shared = shA && q == 0;
      const int ri = q - (shA ? 1 : 0);
      const int e = shared ? 0 : s_e[ri];
      const int q0 = shared ? 0 : s_start[ri];
      const int q1 = shared ? T : s_start[ri + 1];
      const int p = pA;
      float bsc[NSU];  // MXFP4 block scales of the lane's groups
#pragma unroll
      for (int c = 0; c < NSU; ++c) bsc[c] = kFp4 ? e8m0_scale(xsc[c]) : 1.0f;
      float sg0 = 1.f, sg1 = 1.f, su0 = 1.f, su1 = 1.f;
      if (VPG == 16) {
        const float *sc = shared ? a.ss_gu : a.s_gu + (size_t)e * 2 * a.I;
        const int Iw = shared ? a.I_s : a.I;
        sg0 = sc[2 * p];
        sg1 = sc[2 * p + 1];
        su0 = sc[Iw + 2 * p];
        su1 = sc[Iw + 2 * p + 1];
      }
      for (int qq = q0; qq < q1; ++qq) {
        const int slot = shared ? qq : s_slots[qq];
        const int t = shared ? qq : s_stok[qq];
        const uint4 *xr = xs + (size_t)t * xg;
        float acc = 0.0f;
        // the token's LDS reads in groups of 4, the next group issued before the current one
        // is used (scheduling barriers keep at most two groups in registers); one
        // accumulation chain in lane-loop order
        constexpr int kGrp = 4, NG = CGU / kGrp, XPG = VPG / 8;  // uint4 of x per column group
        static_assert(CGU % kGrp == 0, "column groups come in fours");
        uint4 xv[2][kGrp * XPG];
        auto read_group = [&](uint4(&dst)[kGrp * XPG], int gi) {
#pragma unroll
          for (int u = 0; u < kGrp; ++u) {
            const int gu = min(l16 + 16 * (gi * kGrp + u), H / VPG);  // H / VPG: the zero pad
            if (VPG == 8) {
              dst[u] = xr[gu];
            } else if (kFp4) {  // four uint4 a group: a group past the row rereads the last one
              const int gv = min(gu, H / VPG - 1);
#pragma unroll
              for (int d = 0; d < 4; ++d) dst[4 * u + d] = xr[4 * gv + d];
            } else {
              dst[2 * u] = xr[2 * gu];
              dst[2 * u + 1] = xr[2 * gu + 1];
            }
          }
        };
        read_group(xv[0], 0);
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) {
          if (gi + 1 < NG) read_group(xv[(gi + 1) & 1], gi + 1);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int u = 0; u < kGrp; ++u) {
            const int c = gi * kGrp + u;
            const uint4 wc = w[c];
            if (VPG == 8) {
              acc = dot8_bf16(wc, xv[gi & 1][u], acc);
            } else if (kFp4) {
              acc = fmaf(dot32_fp4_bf16(wc, &xv[gi & 1][4 * u]), bsc[c], acc);
            } else {
              const uint4 x0 = xv[gi & 1][2 * u], x1 = xv[gi & 1][2 * u + 1];
              acc = dot2_bf16(fp8x2_to_bf16x2<false>(wc.x), x0.x, acc);
              acc = dot2_bf16(fp8x2_to_bf16x2<true>(wc.x), x0.y, acc);
              acc = dot2_bf16(fp8x2_to_bf16x2<false>(wc.y), x0.z, acc);
              acc = dot2_bf16(fp8x2_to_bf16x2<true>(wc.y), x0.w, acc);
              acc = dot2_bf16(fp8x2_to_bf16x2<false>(wc.z), x1.x, acc);
              acc = dot2_bf16(fp8x2_to_bf16x2<true>(wc.z), x1.y, acc);
              acc = dot2_bf16(fp8x2_to_bf16x2<false>(wc.w), x1.z, acc);
              acc = dot2_bf16(fp8x2_to_bf16x2<true>(wc.w), x1.w, acc);
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        acc = row16_sum(acc);
        const float g0 = lane_value(acc, 0) * sg0, g1 = lane_value(acc, 16) * sg1;
        const float u0 = lane_value(acc, 32) * su0, u1 = lane_value(acc, 48) * su1;
        if (lane == 0) {
          uint16_t *dst = shared ? a.h_s + (size_t)t * a.I_s + 2 * p : a.h + (size_t)slot * a.I + 2 * p;
          __hip_atomic_store(reinterpret_cast<uint32_t *>(dst),
                             pack_bf16x2(g0 / (1.0f + expf(-g0)) * u0, g1 / (1.0f + expf(-g1)) * u1),
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    };
    const int voff_r = gu_voff(a.I, pA), voff_s = gu_voff(a.I_s, pA);
    const int soff_r = gu_soff(a.I, pA), soff_s = gu_soff(a.I_s, pA);
    auto load = [&](uint4(&w)[CGU], uint32_t(&xs)[NSU], int q) {  // q >= NEA: an empty descriptor
      const bool valid = q < NEA, shared = shA && q == 0;
      gu_load(w, xs, valid, shared, (valid && !shared) ? s_e[q - (shA ? 1 : 0)] : 0, shared ? voff_s : voff_r,
              shared ? soff_s : soff_r);
    };
    auto grab = [&]() -> int {
      int v = 0;
      if (lane == 0) v = atomicAdd(&s_qa, 1);
      return __builtin_amdgcn_readfirstlane(v);
    };
    // every load is issued (past the last entry they read nothing), so the compiler's wait
    // counts are the same on every path and no prefetch is waited for early
    int q = grab();
    int q2 = grab();
    load(wa, xa, q);
    load(wb, xb, q2);
    while (q < NEA) {
      compute(wa, xa, q);
      const int q3 = grab();
      load(wa, xa, q3);
      if (q2 >= NEA) break;
      compute(wb, xb, q2);
      const int q4 = grab();
      load(wb, xb, q4);
      q = q3;
      q2 = q4;
    }
  }

  // ---------------- phase B: down + combine for output rows 8o .. 8o+7, o = b.  Entries:
  // 0 the shared expert (with one), then the touched experts, taken from an LDS counter.
  // Each wavefront except 0 takes its first two entries and starts their weight loads
  // before the second grid barrier (wavefront 0 polls the barrier and keeps its load queue
  // empty), so the barrier wait streams weights.
  const int NOct = H / kOct;
  const int oB = blockIdx.x;
  const int NEB = oB < NOct ? nr + (a.has_shared ? 1 : 0) : 0;
  uint4 da[2][CGD], db[2][CGD], dc[2][CGD], dd[2][CGD];
  uint32_t sa[2][NSD], sb[2][NSD], sc_[2][NSD], sd[2][NSD];  // MXFP4 scale bytes
  // the lane's byte offsets in a down matrix for output rows 8o+rg and 8o+4+rg (row length
  // I or I_s): fixed for the whole phase, computed once
  const int dv_r0 = nbytes((kOct * oB + rg) * a.I) + l16 * 16, dv_r1 = dv_r0 + nbytes(4 * a.I);
  const int dv_s0 = nbytes((kOct * oB + rg) * a.I_s) + l16 * 16, dv_s1 = dv_s0 + nbytes(4 * a.I_s);
  // MXFP4: the lane's offsets in the scale matrix (one byte per group)
  const int ds_r0 = (kOct * oB + rg) * (a.I / VPG) + l16, ds_r1 = ds_r0 + 4 * (a.I / VPG);
  const int ds_s0 = (kOct * oB + rg) * (a.I_s / VPG) + l16, ds_s1 = ds_s0 + 4 * (a.I_s / VPG);
  auto dn_load = [&](uint4(&w)[2][CGD], uint32_t(&xs)[2][NSD], int q) {  // q >= NEB: an empty descriptor
    const bool valid = q < NEB;
    const bool shared = a.has_shared && q == 0;
    const int ri = q - (a.has_shared ? 1 : 0);
    const int K = shared ? a.I_s : a.I;
    const int e = (shared || !valid) ? 0 : __builtin_amdgcn_readfirstlane(s_e[ri]);  // uniform: a scalar descriptor
    const uint8_t *bank = shared ? (const uint8_t *)a.ws_d : (const uint8_t *)a.w_d + nbytes((size_t)e * H * a.I);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(bank), 0,
                                                                        valid ? nbytes(H * K) : 0, 0x00020000);
    const int last = K / VPG / 16 - 1;
    const int v0 = shared ? dv_s0 : dv_r0, v1 = shared ? dv_s1 : dv_r1;
#pragma unroll
    for (int c = 0; c < CGD; ++c) {
      w[0][c] = as_u4(__builtin_amdgcn_raw_buffer_load_b128(rs, v0, 256 * min(c, last), kNt));  // zeroed at use
      w[1][c] = as_u4(__builtin_amdgcn_raw_buffer_load_b128(rs, v1, 256 * min(c, last), kNt));
    }
    const int s0 = shared ? ds_s0 : ds_r0, s1 = shared ? ds_s1 : ds_r1;
    if (kFp4) {
      const uint8_t *sbank = shared ? (const uint8_t *)a.ss_d : (const uint8_t *)a.s_d + (size_t)e * H * (a.I / VPG);
      const __amdgpu_buffer_rsrc_t rsc = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(sbank), 0,
                                                                           valid ? H * (K / VPG) : 0, 0x00020000);
#pragma unroll
      for (int c = 0; c < NSD; ++c) {
        xs[0][c] = __builtin_amdgcn_raw_buffer_load_b8(rsc, s0, 16 * min(c, last), kNt);
        xs[1][c] = __builtin_amdgcn_raw_buffer_load_b8(rsc, s1, 16 * min(c, last), kNt);
      }
    }
    if (kFp4) asm volatile("" ::"v"(v0), "v"(v1), "v"(s0), "v"(s1));  // as in gu_load
    else asm volatile("" ::"v"(v0), "v"(v1));
  };
  auto grab_b = [&]() -> int {
    int v = 0;
    if (lane == 0) v = atomicAdd(&s_qb, 1);
    return __builtin_amdgcn_readfirstlane(v);
  };
  wait_stores();  // this wavefront's h stores
  // Four entries in flight per wavefront.  Wavefronts 1..7 issue the first two between the
  // block's arrival and the wait for the release (wavefront 0 polls and keeps its load
  // queue empty), so the barrier wait streams weights and the arrival waits for none of
  // them.  After the barrier the h loads go first and the other two entries' weights
  // right behind them: loads return in issue order, so h is not held up by them, and the
  // weight stream continues while h is staged.
  int qb1 = 0, qb2 = 0, qb3 = 0, qb4 = 0;
  const bool early = wave != 0;
  grid_arrive(a.bar, tok0 + 2u);
  if (early) {
    qb1 = grab_b();
    qb2 = grab_b();
    dn_load(da, sa, qb1);
    dn_load(db, sb, qb2);
  }
  grid_wait(a.bar, tok0 + 2u);
  // (after the barrier the tokens are dead: y and h take the data region)
  float *s_y = reinterpret_cast<float *>(data);  // [T*k][8]
  float *s_ys = s_y + (size_t)n_slots * kOct;   // [T][8]
  // h rows in LDS, hg uint4 each ending in the zero pad: row r < T*k is position r of the
  // slots grouped by expert, row T*k + t the shared expert's token t.  h crosses the barrier:
  // 16-byte loads with the sc1 cache policy (coherent across the XCDs' L2s).  A block with
  // no rows in this phase reads from empty descriptors (zeros, no traffic), so every
  // wavefront issues the same loads.
  uint4 *hl = reinterpret_cast<uint4 *>(data + al16((size_t)(n_slots + T) * kOct * 4));
  {
    constexpr int kSc1 = 16;
    const int gr = a.I / 8, gs = a.I_s / 8;
    const bool any = NEB > 0;
    // one descriptor for h and h_s (h_s lies after h, checked by the launcher): a per-lane
    // choice between two descriptors would become a loop over them
    const int dsh = a.has_shared ? (int)((const char *)a.h_s - (const char *)a.h) : 0;
    const __amdgpu_buffer_rsrc_t rh = __builtin_amdgcn_make_buffer_rsrc(
        a.h, 0, any ? (a.has_shared ? dsh + T * gs * 16 : n_slots * gr * 16) : 0, 0x00020000);
    const int sh0 = a.has_shared ? T : 0;
    const int nrow = n_slots + sh0;
    constexpr int kB = 12;  // 72 rows of 66 uint4 (T = 8) in one round
    i4_t v[kB];
    // offsets first (every slot-list read in flight together), then the loads; a lane past
    // the rows reads past the buffer, which returns zeros
    auto stage_load = [&](int base) {
      int off[kB];
#pragma unroll
      for (int jj = 0; jj < kB; ++jj) {
        const int idx = base + jj * kNT, r = idx / hg, g = idx - r * hg;
        const bool shr = r >= n_slots;  // rows n_slots.. : the shared expert
        const int sl = s_slots[min(r, n_slots - 1)];
        const bool ok = idx < nrow * hg && g < (shr ? gs : gr);
        off[jj] = ok ? (shr ? dsh + ((r - n_slots) * gs + g) * 16 : (sl * gr + g) * 16) : 0x7FFFFFF0;
      }
#pragma unroll
      for (int jj = 0; jj < kB; ++jj) v[jj] = __builtin_amdgcn_raw_buffer_load_b128(rh, off[jj], 0, kSc1);
    };
    auto stage_store = [&](int base) {
#pragma unroll
      for (int jj = 0; jj < kB; ++jj) {
        const int idx = base + jj * kNT;
        if (idx < nrow * hg) hl[idx] = make_uint4(v[jj].x, v[jj].y, v[jj].z, v[jj].w);
      }
    };
    stage_load(tid);
    if (!early) {
      qb1 = grab_b();
      qb2 = grab_b();
      dn_load(da, sa, qb1);
      dn_load(db, sb, qb2);
    }
    qb3 = grab_b();
    qb4 = grab_b();
    dn_load(dc, sc_, qb3);
    dn_load(dd, sd, qb4);
    // while those loads are in flight: the padded counts and their block-wide scan for the
    // caller's alignment (LDS only, so bare barriers)
    {
      const int BM = a.BM;
      const int per = (E + kNT - 1) / kNT;
      const int e0 = tid * per;
      uint32_t vb = 0;
      for (int u = 0; u < per; ++u) {
        const int e = e0 + u;
        if (e < E) {
          const int c = __popc(s_mlo[e]) + __popc(s_mhi[e]);
          s_cnt[e] = c;
          vb += (uint32_t)((c + BM - 1) / BM * BM);
        }
      }
      const uint32_t ib = wave_incl_scan_u32(vb);
      if (lane == kWave - 1) s_wsum[wave] = ib;
      lds_barrier();
      uint32_t rb = ib - vb;
      for (int w = 0; w < wave; ++w) rb += s_wsum[w];
      for (int u = 0; u < per; ++u) {
        const int e = e0 + u;
        if (e < E) {
          s_off[e] = (int)rb;
          rb += (uint32_t)((s_cnt[e] + BM - 1) / BM * BM);
        }
      }
      if (tid == kNT - 1) s_off[E] = (int)rb;
    }
    stage_store(tid);
    for (int base = tid + kB * kNT; base < nrow * hg; base += kB * kNT) {  // larger blocks
      stage_load(base);
      stage_store(base);
    }
  }
  lds_barrier();  // h staged; the weight loads stay in flight
  {
    // ---- entries from the LDS counter, four in flight per wavefront
    auto compute = [&](uint4(&w)[2][CGD], const uint32_t(&xsc)[2][NSD], int q) {
      const bool shared = a.has_shared && q == 0;
      const int ri = q - (a.has_shared ? 1 : 0);
      const int e = shared ? 0 : s_e[ri];
      const int q0 = shared ? 0 : s_start[ri];
      const int q1 = shared ? T : s_start[ri + 1];
      const int Kv = (shared ? a.I_s : a.I) / VPG;
      consume(w[0]);
      consume(w[1]);
      // column groups past the row (whole groups) hold a repeated load: zero them in place
#pragma unroll
      for (int c = 0; c < CGD; ++c)
        if (16 * c >= Kv) w[0][c] = w[1][c] = make_uint4(0, 0, 0, 0);
      const int o = oB;
      float bsc[2][NSD];  // MXFP4 block scales
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int c = 0; c < NSD; ++c) bsc[s][c] = kFp4 ? e8m0_scale(xsc[s][c]) : 1.0f;
      float sc0 = 1.f, sc1 = 1.f;
      if (VPG == 16) {
        const float *sc = shared ? a.ss_d : a.s_d + (size_t)e * H;
        sc0 = sc[kOct * o + rg];
        sc1 = sc[kOct * o + 4 + rg];
      }
      for (int qq = q0; qq < q1; ++qq) {
        const int slot = shared ? qq : s_slots[qq];
        const uint4 *hr = hl + (size_t)(shared ? n_slots + qq : qq) * hg;
        float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
        for (int c = 0; c < CGD; ++c) {
          const int g = min(l16 + 16 * c, Kv);  // Kv: the zero pad
          const uint4 w0 = w[0][c], w1 = w[1][c];
          if (VPG == 8) {
            const uint4 hv = hr[g];
            acc0 = dot8_bf16(w0, hv, acc0);
            acc1 = dot8_bf16(w1, hv, acc1);
          } else if (kFp4) {  // four uint4 a group: a group past the row rereads the last one
            const uint4 *hg4 = hr + 4 * min(g, Kv - 1);
            acc0 = fmaf(dot32_fp4_bf16(w0, hg4), bsc[0][c], acc0);
            acc1 = fmaf(dot32_fp4_bf16(w1, hg4), bsc[1][c], acc1);
          } else {
            const uint4 h0 = hr[2 * g], h1 = hr[2 * g + 1];
#pragma unroll
            for (int s = 0; s < 2; ++s) {
              const uint4 ws = s == 0 ? w0 : w1;
              float acc = s == 0 ? acc0 : acc1;
              acc = dot2_bf16(fp8x2_to_bf16x2<false>(ws.x), h0.x, acc);
              acc = dot2_bf16(fp8x2_to_bf16x2<true>(ws.x), h0.y, acc);
              acc = dot2_bf16(fp8x2_to_bf16x2<false>(ws.y), h0.z, acc);
              acc = dot2_bf16(fp8x2_to_bf16x2<true>(ws.y), h0.w, acc);
              acc = dot2_bf16(fp8x2_to_bf16x2<false>(ws.z), h1.x, acc);
              acc = dot2_bf16(fp8x2_to_bf16x2<true>(ws.z), h1.y, acc);
              acc = dot2_bf16(fp8x2_to_bf16x2<false>(ws.w), h1.z, acc);
              acc = dot2_bf16(fp8x2_to_bf16x2<true>(ws.w), h1.w, acc);
              if (s == 0) acc0 = acc;
              else acc1 = acc;
            }
          }
        }
        acc0 = row16_sum(acc0);
        acc1 = row16_sum(acc1);
        if (l16 == 0) {
          float *dst = shared ? s_ys + (size_t)qq * kOct : s_y + (size_t)slot * kOct;
          dst[rg] = round_bf16(acc0 * sc0);
          dst[4 + rg] = round_bf16(acc1 * sc1);
        }
      }
    };
    // entries are grabbed in increasing order, so the first one past the end ends the loop
    int q1 = qb1, q2 = qb2, q3 = qb3, q4 = qb4;
    while (q1 < NEB) {
      compute(da, sa, q1);
      q1 = grab_b();
      dn_load(da, sa, q1);
      if (q2 >= NEB) break;
      compute(db, sb, q2);
      q2 = grab_b();
      dn_load(db, sb, q2);
      if (q3 >= NEB) break;
      compute(dc, sc_, q3);
      q3 = grab_b();
      dn_load(dc, sc_, q3);
      if (q4 >= NEB) break;
      compute(dd, sd, q4);
      q4 = grab_b();
      dn_load(dd, sd, q4);
    }
  }
  __syncthreads();
  if (oB < NOct) {
    for (int idx = tid; idx < T * kOct; idx += kNT) {
      const int t = idx / kOct, rr = idx % kOct;
      float acc = 0.0f;
      for (int j = 0; j < k; ++j) acc = fmaf(s_topw[t * k + j], s_y[(size_t)(t * k + j) * kOct + rr], acc);
      if (a.has_shared) acc = fmaf(s_gamma[t], s_ys[t * kOct + rr], acc);
      a.out[(size_t)t * H + kOct * oB + rr] = to_bf16(acc);
    }
  }
  // the routing and the padded alignment for the caller, spread over the blocks: any
  // position p of the padded list follows from the padded scan and the slot lists
  {
    const int NBk = gridDim.x, b = blockIdx.x, BM = a.BM;
    for (int i = b * kNT + tid; i < n_slots; i += NBk * kNT) {
      a.ids[i] = s_ids[i];
      a.topw[i] = s_topw[i];
    }
    if (a.has_shared && b == NBk - 1 && tid < T) a.gamma[tid] = s_gamma[tid];
    const int total = s_off[E];
    for (int e = b * kNT + tid; e <= E; e += NBk * kNT) {
      if (e < E) a.al.counts[e] = s_cnt[e];
      a.al.offsets[e] = s_off[e];
    }
    if (b == 0 && tid == 0) a.al.num_padded[0] = total;
    for (int p = b * kNT + tid; p < a.cap; p += NBk * kNT) {
      int v = n_slots;
      if (p < total) {
        const int e = segment_of(s_off, E, p);
        const int r = p - s_off[e];
        if (r < s_cnt[e]) v = s_slots[s_qs[e] + r];
      }
      a.al.sorted[p] = v;
    }
    for (int bb = b * kNT + tid; bb < a.cap / BM; bb += NBk * kNT) {
      const int p = bb * BM;
      a.al.block_expert[bb] = p < total ? segment_of(s_off, E, p) : -1;
    }
  }
}

// ============================================================ host side
namespace {
constexpr size_t kFusedLdsMax = 156 * 1024;

size_t route_bytes(int T, int k, int E) {
  const size_t n = (size_t)T * k;
  return al16((4 * n + kDecodeMaxT + 7 * (size_t)E + 3) * 4);
}
}  // namespace

// LDS of one block: the routing region, then the data region -- the tokens in phases 0
// and A, then the expert outputs y of the block's rows and the h rows in phase B.
size_t fused_lds_bytes(int T, int H, int E, int k, int I, int I_s, int has_shared) {
  const size_t rb = route_bytes(T, k, E);
  const size_t n = (size_t)T * k;
  const size_t xb = al16((size_t)T * (H / 8 + 2) * 16);
  const size_t yb = al16((n + T) * kOct * 4);
  const size_t hb = (n + (has_shared ? (size_t)T : 0)) * ((has_shared && I_s > I ? I_s : I) / 8 + 2) * 16;
  return rb + std::max(xb, yb + hb);
}

namespace {
// CU count of the current device (cached per device; 0 when it cannot be read).
int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int c = cache[dev].load(std::memory_order_relaxed);
  if (c == 0) {
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cache[dev].store(c, std::memory_order_relaxed);
  }
  return c;
}
}  // namespace

// The fused kernel's register tiles hold H <= 2048 and I, I_s <= 512; one block owns one
// gate/up row pair and one octet of output rows, so the grid (one block per CU) must cover
// max(I, I_s) / 2 pairs and H / 8 octets; the tokens, y and h must fit in LDS together.
bool fused_decode_fits(int T, int H, int E, int k, int I, int I_s, int wtype) {
  if (T < 1 || T > kDecodeMaxT || T * k > kSmallSlots || E > kMaxExperts) return false;
  if (H > kXW || I > kHW || I_s > kHW) return false;
  // elements in 16 column groups of 16 bytes (MXFP4: no partial lane groups at all)
  const int grp = 16 * (wtype == 0 ? 8 : wtype == 3 ? 32 : 16);
  if (H % grp != 0 || I % grp != 0 || I_s % grp != 0) return false;
  const int nb = std::min(device_cus(), kMaxBlocks);
  if ((I_s > I ? I_s : I) / 2 > nb || H / kOct > nb) return false;
  return fused_lds_bytes(T, H, E, k, I, I_s, I_s > 0) <= kFusedLdsMax;
}

// Per device: the LDS size the kernel was opened up to, the CU count and how many
// blocks of that LDS size fit on a CU (queried once per device and LDS size).
struct FusedLaunchInfo {
  size_t lds_allowed = 64 * 1024;
  size_t lds_queried = 0;
  int cus = 0, per_cu = 0;
};

template <int VPG, int CGU, int CGD, int CR>
static hipError_t launch_fused_t(FusedArgs &a, size_t lds, hipStream_t s, int *nb_out) {
  auto kern = moe_decode_fused_kernel<VPG, CGU, CGD, CR>;
  static std::mutex mu;
  static FusedLaunchInfo info[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  int cus = 0, per_cu = 0;
  {
    std::lock_guard<std::mutex> lock(mu);
    FusedLaunchInfo &d = info[dev];
    if (lds > d.lds_allowed) {
      e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)lds);
      if (e != hipSuccess) return e;
      d.lds_allowed = lds;
    }
    if (d.lds_queried != lds) {
      e = hipDeviceGetAttribute(&d.cus, hipDeviceAttributeMultiprocessorCount, dev);
      if (e != hipSuccess) return e;
      e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&d.per_cu, reinterpret_cast<const void *>(kern), kNT, lds);
      if (e != hipSuccess) return e;
      d.lds_queried = lds;
    }
    cus = d.cus;
    per_cu = d.per_cu;
  }
  // one block per CU; the whole grid must be resident at once for the barriers
  const int nb = std::min(cus, kMaxBlocks);
  if (per_cu < 1 || (long)per_cu * cus < nb) return hipErrorInvalidConfiguration;
  // one gate/up row pair and one output octet per block at most
  if ((a.has_shared && a.I_s > a.I ? a.I_s : a.I) / 2 > nb || a.H / kOct > nb) return hipErrorInvalidConfiguration;
  *nb_out = nb;
  return launch_k(kern, dim3(nb), dim3(kNT), lds, s, a);
}

hipError_t launch_fused_decode(FusedArgs a, hipStream_t s, char *desc, size_t desc_len) {
  const size_t lds = fused_lds_bytes(a.T, a.H, a.E, a.k, a.I, a.I_s, a.has_shared);
  if (lds > kFusedLdsMax) return hipErrorInvalidValue;
  // phase B reads h and h_s through one buffer descriptor based at h
  if (a.has_shared) {
    const ptrdiff_t d = (const char *)a.h_s - (const char *)a.h;
    if (d < (ptrdiff_t)a.T * a.k * a.I * 2 || d + (ptrdiff_t)a.T * a.I_s * 2 >= ((ptrdiff_t)1 << 31))
      return hipErrorInvalidValue;
  }
  a.lds_route = route_bytes(a.T, a.k, a.E);
  int nb = 0;
  hipError_t e;
  if (a.wtype == 0) e = launch_fused_t<8, 16, 4, 8>(a, lds, s, &nb);
  else if (a.wtype == 3) e = launch_fused_t<32, 4, 1, 8>(a, lds, s, &nb);
  else e = launch_fused_t<16, 8, 2, 8>(a, lds, s, &nb);
  if (desc)
    snprintf(desc, desc_len, "moe_decode_fused<%s> grid=%d block=%d lds=%zu",
             a.wtype == 0 ? "bf16" : a.wtype == 3 ? "mxfp4" : "fp8", nb, kNT, lds);
  return e;
}

}  // namespace moe
