// fused.hip -- the whole decode/verify-block MoE layer in one kernel (gfx950).
//
// veloGB10 README, "Kernel work": the router fold spread across the GPU, several small
// kernels (the expert routing among them) folded into their neighbours, grouped expert
// kernels that never rebuild weights, shared-expert work overlapped with the MoE step.
// Qwen3.8 Flash-Next . GB10 UltraFast, first bullet: a deterministic floor -- alignment
// in slot order and a combine without float atomics.
//
// One block per CU (8 wavefronts); the grid never exceeds what the device holds resident
// at once.  Phases:
//   0  router row n on block n % NB, tokens staged in LDS; wavefront 0 also loads the
//      shared expert's gate/up rows of its block's row pair (they do not depend on the
//      routing, so they stream while the head of the kernel is latency-bound).
//                                                                  -- grid barrier
//   1  every block routes all T tokens itself from the logits (top-k per wavefront, token
//      masks per expert, entry lists): no exchange, no second launch.
//   A  wavefronts 0..6: gate/up row pair b (2b, 2b+1 and I+2b, I+2b+1) of the shared expert
//      (entry 0, taken by wavefront 0, its rows already in registers) and of every touched
//      expert; each entry's
//      h values go to an LDS outbox.  Wavefront 7, the stager, stores the outbox to global
//      memory entry by entry and publishes how many entries the block has finished; one
//      wavefront of block 0 publishes the minimum over the blocks; the stagers copy the h
//      rows of every entry that all blocks have finished into LDS with direct-to-LDS
//      loads, while the gate/up stream goes on.
//   B  wavefronts 0..6, each as soon as it runs out of gate/up entries: down rows
//      8b..8b+7 of the shared expert and of every touched expert, weights prefetched four
//      entries deep; an entry is computed once the stager has staged its h rows.  y stays
//      in LDS, the combine sums in slot order in fp32.
// There is no grid barrier between the two expert phases: an entry's down projection waits
// only for that entry's h, so the down stream starts while slower blocks finish gate/up.
// The compute wavefronts never wait for a store: all stores that other blocks read come
// from the stager, whose memory queue holds nothing else.
//
// Lane mapping: four 16-lane DPP rows per wavefront, one weight row each, 16-byte column
// groups per lane, one 4-step DPP sum per dot product.
//
// Synchronisation through global memory uses agent-scope atomic loads and stores (sc1:
// coherent across the XCDs' L2s) for every word that crosses blocks (logits, gate logits,
// h, flags, progress counts), and each word has one writer -- no read-modify-write on a
// shared word, which the memory side would serialise.  A flag or count is stored only after
// the data it announces has completed (vmcnt), so no cache write-back or invalidate is
// needed.  Every wait is bounded: a wait that gives up adds one to the workspace's status
// word and the affected blocks write NaN for their output rows, so a misuse (a block that
// never became resident) is visible and never hangs.

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
constexpr int kStager = kNW - 1;  // the wavefront that publishes and stages h
constexpr int kAggr = kNW - 2;    // in block 0: the wavefront that publishes the blocks' minimum
constexpr unsigned kTokMask = 0x7FFFFFFFu, kBarErr = 0x80000000u, kNoFlag = 0xFFFFFFFFu;
constexpr int kOct = 8;           // output rows per block in phase B
// Widths (elements) the lanes' column groups span: H <= kXW, I and I_s <= kHW.  The LDS
// rows of the tokens and of h end in two zero uint4; a lane's column index beyond the row
// is clamped onto them (its weights are zero too), so the dot-product loops have no
// bounds tests and no branch.
constexpr int kXW = 2048;
constexpr int kHW = 512;
typedef __attribute__((address_space(3))) void lds_void;
}  // namespace

__host__ __device__ __forceinline__ size_t al16(size_t v) { return (v + 15) & ~(size_t)15; }

constexpr unsigned kSpinLimit = 1u << 20;

__device__ __forceinline__ unsigned ld_agent(const unsigned *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(unsigned *p, unsigned v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void add_agent(unsigned *p, unsigned v) {
  __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wait until this wavefront's earlier vector memory operations have completed (vmcnt
// counts loads and stores in issue order); the clobber keeps the compiler from moving
// memory operations across it.
__device__ __forceinline__ void wait_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Mark a register buffer as consumed here: the compiler waits for its loads at this point,
// so no later reuse of those registers waits on the loads issued after them.
template <int N>
__device__ __forceinline__ void consume(const uint4 (&w)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) asm volatile("" ::"v"(w[i].x), "v"(w[i].y), "v"(w[i].z), "v"(w[i].w));
}

// A wait that gave up: count it in the workspace (the caller reads the count; the only
// read-modify-write on a global word, and only on this path) and mark the block, which then
// writes NaN for its output rows.
__device__ __forceinline__ void note_timeout(unsigned *bar, int *s_err) {
  add_agent(bar + kBarStatus, 1u);
  __hip_atomic_store(s_err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// VPG: weights per 16-byte column group -- 8 bf16, 16 fp8 codes, or 32 MXFP4 codes (which
// are also one scale block).  CGU / CGD: column groups per lane and weight row in phase A /
// phase B; CR: float4 router groups per lane.
// RING: the staged h rows of the routed slots wrap around an LDS ring smaller than T*k rows.
// RAMP: each compute wavefront starts phase A with one entry in flight instead of two.
template <int VPG, int CGU, int CGD, int CR, bool RING, bool RAMP>
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

  // ---------------- LDS: routing region, tokens, expert outputs y, h rows
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
  __shared__ int s_hready;    // phase-B entries whose h rows are staged (shared expert first)
  __shared__ int s_err;       // a wait of this block gave up
  __shared__ unsigned s_tok;  // this call's barrier token
  // entries whose gate/up rows of this block are in the outbox (or that have none here)
  __shared__ unsigned long long s_done[(kMaxExperts + 1 + 63) / 64];
  // phase-B entries whose down rows this block has computed (their h rows may be overwritten)
  __shared__ unsigned long long s_bdone[(kMaxExperts + 1 + 63) / 64];
  uint4 *sx = reinterpret_cast<uint4 *>(smem + a.lds_route);            // [T][xg]
  float *s_y = reinterpret_cast<float *>(sx + (size_t)T * xg);          // [T*k][8]
  float *s_ys = s_y + (size_t)n_slots * kOct;                           // [T][8]
  // h values of this block's row pair, one packed pair per slot position (then T shared)
  uint32_t *s_out = reinterpret_cast<uint32_t *>(s_ys + (size_t)T * kOct);  // [T*k + T]
  // staged h rows: a ring of HR rows for the routed slot positions (position r in row r % HR;
  // HR = T*k, no wrap, wherever every position fits), then the shared expert's T rows
  const int HR = RING ? a.h_ring : n_slots;
  uint4 *hl = reinterpret_cast<uint4 *>(smem + a.lds_route + al16((size_t)T * xg * 16) +
                                        al16((size_t)(n_slots + T) * (kOct + 1) * 4));  // [HR + T][hg]
  // this call's barrier token follows the release word the previous call left: block 0
  // rewrites that word only after every block has arrived, so every block reads the same
  // value here (the token lives in bits 0..30, never 0, so it differs from a cleared flag)
  unsigned rel0 = 0;
  if (tid == 0) rel0 = ld_agent(a.bar + kBarRelease);

  // ---------------- phase 0: router rows, tokens to LDS, the shared expert's gate/up
  const int NR = E + (a.w_sg != nullptr ? 1 : 0);
  // Router row n runs on block n % NB; every wavefront of the block holds the row (the
  // block's 8 loads of it share the CU's caches) and takes the tokens wave, wave + 8, ...,
  // so each token's dot product is one short chain.  The block's first kRR rows and their
  // biases are loaded first of all.
  constexpr int kRR = 2;
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

  uint4 wa[CGU], wb[CGU];
  uint32_t xa[NSU], xb[NSU];  // MXFP4: the E8M0 scale byte of each of the lane's groups
  // Weight rows are streamed with raw buffer loads: the expert's matrix is the buffer (base
  // in scalar registers), the lane's row and column offset one VGPR, the column group a
  // uniform scalar offset.  Exactly kGuLoads load instructions, all in range: groups past
  // the row (whole groups: H, I, I_s are multiples of 16 groups) reload the last group and
  // are zeroed where they are used, so nothing waits for a load here.
  typedef int i4_t __attribute__((ext_vector_type(4)));
  constexpr int kNt = 2;    // cache policy: non-temporal (weights are read once)
  constexpr int kSc1 = 16;  // cache policy: coherent across the XCDs (data other blocks wrote)
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
      const uint8_t *sbank = shared ? a.xs_gu : a.x_gu + (size_t)e * 2 * a.I * (H / VPG);
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
  // One token's gate/up partial sums for the wavefront's four rows (lane row group rg): the
  // token's LDS reads in groups of 4, the next group issued before the current one is used
  // (scheduling barriers keep at most two groups in registers); one accumulation chain in
  // lane-loop order.  Column groups of w past the row must be zero.
  auto gu_token = [&](const uint4(&w)[CGU], const float(&bsc)[NSU], int t) {
    const uint4 *xr = sx + (size_t)t * xg;
    float acc = 0.0f;
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
    return row16_sum(acc);
  };
  // Prepare a gate/up weight buffer for use: wait for it, zero the column groups past the row
  // (whole groups, holding a repeated load), decode the MXFP4 block scales.
  auto gu_ready = [&](uint4(&w)[CGU], const uint32_t(&xsc)[NSU], float(&bsc)[NSU]) {
    consume(w);
#pragma unroll
    for (int c = 0; c < CGU; ++c)
      if (16 * c >= H / VPG) w[c] = make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int c = 0; c < NSU; ++c) bsc[c] = kFp4 ? e8m0_scale(xsc[c]) : 1.0f;
  };
  // h values of one token for row pair pA: lane 0 puts silu(g) * u of rows 2pA and 2pA+1 (the
  // row sums sit in lanes 0, 16 | 32, 48, scaled by the fp8 row scales) into outbox slot p
  auto gu_out = [&](float acc, int p, float sg0, float sg1, float su0, float su1) {
    const float g0 = lane_value(acc, 0) * sg0, g1 = lane_value(acc, 16) * sg1;
    const float u0 = lane_value(acc, 32) * su0, u1 = lane_value(acc, 48) * su1;
    if (lane == 0) s_out[p] = pack_bf16x2(g0 / (1.0f + expf(-g0)) * u0, g1 / (1.0f + expf(-g1)) * u1);
  };

  // The router's critical path: the block's rows and each wavefront's first token (t = wave)
  // straight into registers, before the other loads (loads return in issue order); column
  // groups past the row read the last group and are zeroed (zero weights).
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
  // the shared expert's gate/up rows of this block's row pair, in wavefront 0, which takes
  // entry 0 in phase A: the bytes stream during the head (the other wavefronts' loads are
  // empty)
  const int pA = blockIdx.x;
  const bool shA = a.has_shared && 2 * pA < a.I_s;
  gu_load(wa, xa, shA && wave == 0, true, 0, gu_voff(a.I_s, pA), gu_soff(a.I_s, pA));

  // tokens to LDS (for phase A and the router's later tokens), in rows of xg uint4 ending
  // in the zero pad; unguarded (clamped) loads, so they are in flight together
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
  // LDS set-up: the token masks, the h rows (zero, so that the pads and any row tail no
  // copy fills read as zeros), the counters; this call's readiness counts start at zero
  for (int e = tid; e < E; e += kNT) {
    s_mlo[e] = 0u;
    s_mhi[e] = 0u;
  }
  for (int i = tid; i < (HR + T) * hg; i += kNT) hl[i] = make_uint4(0, 0, 0, 0);
  for (int i = tid; i < (kMaxExperts + 1 + 63) / 64; i += kNT) {
    s_done[i] = 0ull;
    s_bdone[i] = 0ull;
  }
  if (tid == 0) {
    s_err = 0;
    s_hready = 0;
    const unsigned t = ((rel0 & kTokMask) + 1u) & kTokMask;
    s_tok = t == 0 ? 1u : t;
    // this call's progress counts start at zero (published before the barrier)
    st_agent(a.bar + kBarProgress + blockIdx.x, 0u);
    if (blockIdx.x == 0) st_agent(a.bar + kBarReady, 0u);
  }
  __syncthreads();

  // the wavefront's further tokens and the rows past the first kRR, from the staged tokens
  auto lds_token = [&](uint2(&xv)[CR], int t) {
    const uint2 *x2 = reinterpret_cast<const uint2 *>(sx) + (size_t)t * (2 * xg);
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
  // grid barrier: every wavefront's logit and count stores have completed before the block
  // stores its arrival flag; wavefront 0 of block 0 polls all flags (one batched load per
  // lane and round) and stores the release word, which every block polls.  A wait that
  // gives up sets bit 31 of the release word, so every block of the call knows; a block
  // whose own wait gave up (it started after the release: its token is off by one) clears
  // its flag, so that no later call takes the stale token for an arrival.
  wait_stores();
  __syncthreads();
  {
    const unsigned tok = s_tok;
    unsigned *flags = a.bar, *rel = a.bar + kBarRelease;
    if (tid == 0) st_agent(flags + blockIdx.x, tok);
    if (blockIdx.x == 0 && wave == 0) {
      constexpr int kPer = kMaxBlocks / kWave;
      unsigned spins = 0;
      bool gave_up = false;
      while (true) {
        unsigned v[kPer];
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
          const int i = lane + kWave * j;
          if (kWave * j < NB) v[j] = ld_agent(flags + (i < NB ? i : NB - 1));
        }
        bool ok = true;
#pragma unroll
        for (int j = 0; j < kPer; ++j)
          if (kWave * j < NB) ok &= v[j] == tok;
        if (__all(ok)) break;
        __builtin_amdgcn_s_sleep(1);
        if (++spins > kSpinLimit) {
          gave_up = true;
          break;
        }
      }
      if (lane == 0) {
        if (gave_up) note_timeout(a.bar, &s_err);
        st_agent(rel, tok | (gave_up ? kBarErr : 0u));
      }
    }
    if (tid == 0) {
      unsigned spins = 0;
      unsigned r;
      while (((r = ld_agent(rel)) & kTokMask) != tok) {
        __builtin_amdgcn_s_sleep(1);
        if (++spins > kSpinLimit) {
          note_timeout(a.bar, &s_err);
          st_agent(flags + blockIdx.x, kNoFlag);
          r = 0;
          break;
        }
      }
      if (r & kBarErr) __hip_atomic_store(&s_err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
  }
  asm volatile("" ::: "memory");
  __syncthreads();

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
        s_qa = a.has_shared ? 1 : 0;  // entry 0, the shared expert, belongs to wavefront 0
        s_qb = 0;
      }
    }
    __syncthreads();
  }
  const int nr = s_nt;
  const int sh = a.has_shared ? 1 : 0;  // phase-B entry 0 is the shared expert
  const int NOct = H / kOct;
  const int oB = blockIdx.x;
  const int NEB = oB < NOct ? nr + sh : 0;

  const int total = nr + sh;                     // phase-B entries (and gate/up entries)
  const bool ownR = 2 * pA < a.I;                // this block has a gate/up row pair of the routed experts
  if (wave == kStager) {
    // ---------------- the stager.  (1) Stores the outbox of every entry the compute
    // wavefronts have finished, in entry order, then -- once the stores have completed --
    // publishes the count in the block's progress word.  (2) Copies the h rows of every
    // entry all blocks have finished (block 0's published minimum) into LDS, in phase-B entry
    // order: row r < T*k of hl is position r of the slots grouped by entry, row T*k + t the
    // shared expert's token t; one direct-to-LDS load per row (64 lanes x 16 bytes = 1 KiB,
    // the row of I = 512); consecutive entries have consecutive rows.  Coherent (sc1) loads:
    // h was written by other blocks.
    // entries with no gate/up rows in this block are done from the start
    if (lane == 0) {
      if (sh && !shA) s_done[0] |= 1ull;
      if (!ownR)
        for (int q = sh; q < total; ++q) s_done[q >> 6] |= 1ull << (q & 63);
    }
    const int rbytes = a.I * 2, srbytes = a.I_s * 2;
    const __amdgpu_buffer_rsrc_t rh =
        __builtin_amdgcn_make_buffer_rsrc(a.h, 0, NEB > 0 ? n_slots * rbytes : 0, 0x00020000);
    const __amdgpu_buffer_rsrc_t rhs =
        __builtin_amdgcn_make_buffer_rsrc(a.h_s, 0, (NEB > 0 && sh) ? T * srbytes : 0, 0x00020000);
    // the first entry at or after q whose bit in mask is clear
    auto done_upto = [&](const unsigned long long *mask, int q) {
      while (q < total) {
        const unsigned long long m =
            __hip_atomic_load(&mask[q >> 6], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) >> (q & 63);
        const int run = m == ~0ull >> (q & 63) ? 64 - (q & 63) : (int)__builtin_ctzll(~m);
        q += run;
        if (run < 64 - ((q - run) & 63)) break;
      }
      return min(q, total);
    };
    int pub = 0, staged = 0, cons = 0;
    unsigned spins = 0;
    while (pub < total || (NEB > 0 && staged < total)) {
      bool moved = false;
      const int m = done_upto(s_done, pub);
      asm volatile("" ::: "memory");
      if (m > pub) {
        // (1) the outbox of entries [pub, m), then the progress word
        if (sh && pub == 0 && shA)
          for (int t = lane; t < T; t += kWave)
            st_agent(reinterpret_cast<unsigned *>(a.h_s + (size_t)t * a.I_s + 2 * pA), s_out[n_slots + t]);
        if (ownR) {
          const int p0 = s_start[max(pub - sh, 0)], p1 = s_start[m - sh];
          for (int p = p0 + lane; p < p1; p += kWave)
            st_agent(reinterpret_cast<unsigned *>(a.h + (size_t)s_slots[p] * a.I + 2 * pA), s_out[p]);
        }
        wait_stores();
        if (lane == 0) st_agent(a.bar + kBarProgress + blockIdx.x, (unsigned)m);
        pub = m;
        moved = true;
      }
      if (NEB > 0 && staged < total) {
        // (2) entries every block has finished: h rows into LDS
        const unsigned g = __builtin_amdgcn_readfirstlane(ld_agent(a.bar + kBarReady));
        const int gr = min((int)(g & kTokMask), total);
        if (g & kBarErr) {  // block 0 gave up waiting for some block: stage what there is
          if (lane == 0) __hip_atomic_store(&s_err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        }
        int upto = (g & kBarErr) ? total : gr;
        if (RING && upto > staged) {
          // the ring: the rows of entries [staged, upto) may only replace rows of positions
          // whose entries this block's phase B has computed
          cons = done_upto(s_bdone, cons);
          const int cpos = s_start[max(cons - sh, 0)];
          while (upto > max(staged, sh) && s_start[upto - sh] > cpos + HR) --upto;
        }
        if (upto > staged) {
          if (sh && staged == 0)
            for (int t = 0; t < T; ++t)
              if (lane * 16 < srbytes)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rhs, (lds_void *)(hl + (size_t)(HR + t) * hg), 16,
                                                         lane * 16, t * srbytes, 0, kSc1);
          if (upto > sh) {
            const int r0 = s_start[max(staged - sh, 0)], r1 = s_start[upto - sh];
            int row = RING ? r0 % HR : r0;  // LDS row of position r
            for (int r = r0; r < r1; ++r) {
              if (lane * 16 < rbytes)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rh, (lds_void *)(hl + (size_t)row * hg), 16, lane * 16,
                                                         s_slots[r] * rbytes, 0, kSc1);
              row = RING && row + 1 == HR ? 0 : row + 1;
            }
          }
          wait_stores();  // the copies have landed in LDS
          staged = upto;
          if (lane == 0) __hip_atomic_store(&s_hready, staged, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
          moved = true;
        }
      }
      if (moved) {
        spins = 0;
      } else {
        __builtin_amdgcn_s_sleep(1);
        if (++spins > kSpinLimit) {  // let the compute wavefronts finish (their rows become NaN)
          if (lane == 0) {
            note_timeout(a.bar, &s_err);
            __hip_atomic_store(&s_hready, total, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
          }
          break;
        }
      }
    }
    // the padded counts and their scan for the caller's alignment (one wavefront, 64 experts
    // a step)
    {
      const int BM = a.BM;
      int run = 0;
      for (int e0 = 0; e0 < E; e0 += kWave) {
        const int e = e0 + lane;
        const int c = e < E ? __popc(s_mlo[e]) + __popc(s_mhi[e]) : 0;
        const uint32_t pc = (uint32_t)((c + BM - 1) / BM * BM);
        const uint32_t incl = wave_incl_scan_u32(pc);
        if (e < E) {
          s_cnt[e] = c;
          s_off[e] = run + (int)(incl - pc);
        }
        run += __builtin_amdgcn_readlane((int)incl, kWave - 1);
      }
      if (lane == 0) s_off[E] = run;
    }
  } else if (blockIdx.x == 0 && wave == kAggr) {
    // ---------------- block 0's aggregator: the minimum of all blocks' progress counts into the
    // ready word the stagers poll (one batched load per lane and round)
    constexpr int kPer = kMaxBlocks / kWave;
    unsigned last = 0, spins = 0;
    while ((int)last < total) {
      unsigned v[kPer];
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        const int i = lane + kWave * j;
        if (kWave * j < NB) v[j] = ld_agent(a.bar + kBarProgress + (i < NB ? i : NB - 1));
      }
      unsigned mn = ~0u;
#pragma unroll
      for (int j = 0; j < kPer; ++j)
        if (kWave * j < NB) mn = min(mn, v[j]);
      mn = wave_min_u32(mn);
      if (mn > last) {
        last = mn;
        if (lane == 0) st_agent(a.bar + kBarReady, last);
        spins = 0;
      } else {
        __builtin_amdgcn_s_sleep(1);
        if (++spins > kSpinLimit) {  // some block never finished: release the stagers, flagged
          if (lane == 0) {
            note_timeout(a.bar, &s_err);
            st_agent(a.bar + kBarReady, (unsigned)total | kBarErr);
          }
          break;
        }
      }
    }
  } else {
    // ---------------- phase A: gate/up of row pair pA for the shared expert (entry 0, with one)
    // and every touched expert, taken from an LDS counter by the compute wavefronts, two
    // entries in flight each; the h values go to the outbox
    auto owned = [&](int q) { return (sh && q == 0) ? shA : ownR; };
    auto compute_a = [&](uint4(&w)[CGU], const uint32_t(&xsc)[NSU], int q) {
      float bsc[NSU];
      gu_ready(w, xsc, bsc);
      const bool shared = sh && q == 0;
      if (owned(q)) {
        const int ri = q - sh;
        const int e = shared ? 0 : s_e[ri];
        const int Iw = shared ? a.I_s : a.I;
        const int q0 = shared ? 0 : s_start[ri], q1 = shared ? T : s_start[ri + 1];
        float sg0 = 1.f, sg1 = 1.f, su0 = 1.f, su1 = 1.f;
        if (VPG == 16) {
          const float *sc = shared ? a.ss_gu : a.s_gu + (size_t)e * 2 * a.I;
          sg0 = sc[2 * pA];
          sg1 = sc[2 * pA + 1];
          su0 = sc[Iw + 2 * pA];
          su1 = sc[Iw + 2 * pA + 1];
        }
        for (int qq = q0; qq < q1; ++qq)
          gu_out(gu_token(w, bsc, shared ? qq : s_stok[qq]), shared ? n_slots + qq : qq, sg0, sg1, su0, su1);
      }
      // the outbox writes of this wavefront precede the done bit (LDS operations of one
      // wavefront complete in order)
      asm volatile("" ::: "memory");
      if (lane == 0)
        __hip_atomic_fetch_or(&s_done[q >> 6], 1ull << (q & 63), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    };
    const int voff_r = gu_voff(a.I, pA), soff_r = gu_soff(a.I, pA);
    auto load_a = [&](uint4(&w)[CGU], uint32_t(&xs)[NSU], int q) {  // q >= total or not owned: an empty descriptor
      const bool shared = sh && q == 0;
      const bool valid = q < total && owned(q);
      gu_load(w, xs, valid, shared, (valid && !shared) ? s_e[q - sh] : 0, shared ? gu_voff(a.I_s, pA) : voff_r,
              shared ? gu_soff(a.I_s, pA) : soff_r);
    };
    auto grab = [&]() -> int {
      int v = 0;
      if (lane == 0) v = atomicAdd(&s_qa, 1);
      return __builtin_amdgcn_readfirstlane(v);
    };
    // every load is issued (past the last entry they read nothing), so the compiler's wait
    // counts are the same on every path and no prefetch is waited for early; entry 0 (the
    // shared expert) is wavefront 0's first, its rows from phase 0 already in wa
    if constexpr (!RAMP) {
      int q = (sh && wave == 0) ? 0 : grab();
      int q2 = grab();
      if (!(sh && q == 0)) load_a(wa, xa, q);
      load_a(wb, xb, q2);
      while (q < total) {
        compute_a(wa, xa, q);
        const int q3 = grab();
        load_a(wa, xa, q3);
        if (q2 >= total) break;
        compute_a(wb, xb, q2);
        const int q4 = grab();
        load_a(wb, xb, q4);
        q = q3;
        q2 = q4;
      }
    } else {
      // the first entry alone in flight: computed before the second is issued, so the
      // blocks' first h rows (which every phase B waits for) arrive sooner; two after that
      int q = (sh && wave == 0) ? 0 : grab();
      if (!(sh && q == 0)) load_a(wa, xa, q);
      if (q < total) compute_a(wa, xa, q);
      int q2 = grab();
      load_a(wb, xb, q2);
      int q3 = grab();
      load_a(wa, xa, q3);
      while (q2 < total) {
        compute_a(wb, xb, q2);
        const int q4 = grab();
        load_a(wb, xb, q4);
        if (q3 >= total) break;
        compute_a(wa, xa, q3);
        const int q5 = grab();
        load_a(wa, xa, q5);
        q2 = q4;
        q3 = q5;
      }
    }

    // ---------------- phase B: down rows 8o .. 8o+7, o = b, for entry 0 (the shared expert,
    // with one) and the touched experts, taken from an LDS counter; four entries in flight
    // per wavefront; an entry waits only for its staged h rows
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
      const bool shared = sh && q == 0;
      const int ri = q - sh;
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
        const uint8_t *sbank = shared ? a.xs_d : a.x_d + (size_t)e * H * (a.I / VPG);
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
    // entry q's h rows are in LDS once the stager has published a count above q
    auto wait_staged = [&](int q) {
      while (__hip_atomic_load(&s_hready, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) <= q)
        __builtin_amdgcn_s_sleep(1);
    };
    auto compute = [&](uint4(&w)[2][CGD], const uint32_t(&xsc)[2][NSD], int q) {
      const bool shared = sh && q == 0;
      const int ri = q - sh;
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
      float bsc[2][NSD];  // MXFP4 block scales
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int c = 0; c < NSD; ++c) bsc[s][c] = kFp4 ? e8m0_scale(xsc[s][c]) : 1.0f;
      float sc0 = 1.f, sc1 = 1.f;
      if (VPG == 16) {
        const float *sc = shared ? a.ss_d : a.s_d + (size_t)e * H;
        sc0 = sc[kOct * oB + rg];
        sc1 = sc[kOct * oB + 4 + rg];
      }
      wait_staged(q);
      int row = shared ? HR + q0 : RING ? q0 % HR : q0;  // LDS row of position qq
      for (int qq = q0; qq < q1; ++qq) {
        const int slot = shared ? qq : s_slots[qq];
        const uint4 *hr = hl + (size_t)row * hg;
        row = RING && !shared && row + 1 == HR ? 0 : row + 1;
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
      // the entry's h rows have been read (their values are used above): the stager may
      // reuse them (LDS operations of one wavefront complete in order)
      asm volatile("" ::: "memory");
      if (RING && lane == 0)
        __hip_atomic_fetch_or(&s_bdone[q >> 6], 1ull << (q & 63), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    };
    int q1 = grab_b(), q2b = grab_b(), q3 = grab_b(), q4 = grab_b();
    dn_load(da, sa, q1);
    dn_load(db, sb, q2b);
    dn_load(dc, sc_, q3);
    dn_load(dd, sd, q4);
    // entries are grabbed in increasing order, so the first one past the end ends the loop
    while (q1 < NEB) {
      compute(da, sa, q1);
      q1 = grab_b();
      dn_load(da, sa, q1);
      if (q2b >= NEB) break;
      compute(db, sb, q2b);
      q2b = grab_b();
      dn_load(db, sb, q2b);
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
  const bool err = __hip_atomic_load(&s_err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) != 0;
  if (oB < NOct) {
    for (int idx = tid; idx < T * kOct; idx += kNT) {
      const int t = idx / kOct, rr = idx % kOct;
      float acc = 0.0f;
      for (int j = 0; j < k; ++j) acc = fmaf(s_topw[t * k + j], s_y[(size_t)(t * k + j) * kOct + rr], acc);
      if (a.has_shared) acc = fmaf(s_gamma[t], s_ys[t * kOct + rr], acc);
      a.out[(size_t)t * H + kOct * oB + rr] = err ? (uint16_t)0x7FC0u : to_bf16(acc);
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
constexpr int kFusedRingMaxT = 16;  // the largest block that takes the fused kernel with a wrapping ring

size_t route_bytes(int T, int k, int E) {
  const size_t n = (size_t)T * k;
  return al16((4 * n + kDecodeMaxT + 7 * (size_t)E + 3) * 4);
}
}  // namespace

// LDS of one block: the routing region, the tokens, the expert outputs y of the block's rows
// and the outbox of its h values, and the h rows (all live together: the stager fills h while
// the tokens are still in use).  The h rows of the routed slots form a ring: all T*k of them
// where they fit, else as many as fit (at least T, one entry's slots).
namespace {
size_t fused_fixed_bytes(int T, int H, int E, int k) {
  const size_t n = (size_t)T * k;
  return route_bytes(T, k, E) + al16((size_t)T * (H / 8 + 2) * 16) + al16((n + T) * (kOct + 1) * 4);
}
size_t fused_hrow_bytes(int I, int I_s, int has_shared) { return (size_t)((has_shared && I_s > I ? I_s : I) / 8 + 2) * 16; }
}  // namespace

int fused_h_ring(int T, int H, int E, int k, int I, int I_s, int has_shared) {
  const size_t fixed = fused_fixed_bytes(T, H, E, k), row = fused_hrow_bytes(I, I_s, has_shared);
  if (fixed + (size_t)T * row >= kFusedLdsMax) return 0;
  const size_t rows = (kFusedLdsMax - fixed) / row - T;
  return (int)std::min((size_t)T * k, rows);
}

size_t fused_lds_bytes(int T, int H, int E, int k, int I, int I_s, int has_shared) {
  const int hr = fused_h_ring(T, H, E, k, I, I_s, has_shared);
  return fused_fixed_bytes(T, H, E, k) + (size_t)(hr + T) * fused_hrow_bytes(I, I_s, has_shared);
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
  // a ring smaller than the T*k slots stalls the staging on phase B: past 16 tokens the
  // four kernels are faster (T = 20 at H = 2048: 143 against 137 us; T = 16: 110 against 118)
  const int hr = fused_h_ring(T, H, E, k, I, I_s, I_s > 0);
  return hr >= T && (T <= kFusedRingMaxT || hr == T * k) && fused_lds_bytes(T, H, E, k, I, I_s, I_s > 0) <= kFusedLdsMax;
}

// Per device: the LDS size the kernel was opened up to, the CU count and how many
// blocks of that LDS size fit on a CU (queried once per device and LDS size).
struct FusedLaunchInfo {
  size_t lds_allowed = 64 * 1024;
  size_t lds_queried = 0;
  int cus = 0, per_cu = 0;
};

template <int VPG, int CGU, int CGD, int CR, bool RING, bool RAMP>
static hipError_t launch_fused_t(FusedArgs &a, size_t lds, hipStream_t s, int *nb_out) {
  auto kern = moe_decode_fused_kernel<VPG, CGU, CGD, CR, RING, RAMP>;
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
  // one block per CU; the whole grid must be resident at once for the barrier and the
  // readiness waits
  const int nb = std::min(cus, kMaxBlocks);
  if (per_cu < 1 || (long)per_cu * cus < nb) return hipErrorInvalidConfiguration;
  // one gate/up row pair and one output octet per block at most
  if ((a.has_shared && a.I_s > a.I ? a.I_s : a.I) / 2 > nb || a.H / kOct > nb) return hipErrorInvalidConfiguration;
  *nb_out = nb;
  return launch_k(kern, dim3(nb), dim3(kNT), lds, s, a);
}

hipError_t launch_fused_decode(FusedArgs a, hipStream_t s, char *desc, size_t desc_len) {
  const size_t lds = fused_lds_bytes(a.T, a.H, a.E, a.k, a.I, a.I_s, a.has_shared);
  a.h_ring = fused_h_ring(a.T, a.H, a.E, a.k, a.I, a.I_s, a.has_shared);
  if (lds > kFusedLdsMax || a.h_ring < a.T) return hipErrorInvalidValue;
  a.lds_route = route_bytes(a.T, a.k, a.E);
  int nb = 0;
  hipError_t e;
  const bool ring = a.h_ring < a.T * a.k;
  // bf16 and MXFP4 start phase A with one entry in flight per wavefront (measured faster at
  // T = 1 and 16 and no slower elsewhere); fp8 with two (one was slower at T = 6)
  if (a.wtype == 0) e = ring ? launch_fused_t<8, 16, 4, 8, true, true>(a, lds, s, &nb) : launch_fused_t<8, 16, 4, 8, false, true>(a, lds, s, &nb);
  else if (a.wtype == 3) e = ring ? launch_fused_t<32, 4, 1, 8, true, true>(a, lds, s, &nb) : launch_fused_t<32, 4, 1, 8, false, true>(a, lds, s, &nb);
  else e = ring ? launch_fused_t<16, 8, 2, 8, true, false>(a, lds, s, &nb) : launch_fused_t<16, 8, 2, 8, false, false>(a, lds, s, &nb);
  if (desc)
    snprintf(desc, desc_len, "moe_decode_fused<%s> grid=%d block=%d lds=%zu h_ring=%d",
             a.wtype == 0 ? "bf16" : a.wtype == 3 ? "mxfp4" : "fp8", nb, kNT, lds, a.h_ring);
  return e;
}

}  // namespace moe
