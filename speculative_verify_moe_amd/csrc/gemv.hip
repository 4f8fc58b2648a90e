// gemv.hip -- decode/verify-block expert kernels for gfx950 (T <= 64 tokens).
//
// veloGB10 README, "Kernel work": grouped MoE expert kernels that never rebuild full
// weights; the shared expert overlapped with the MoE step.  Qwen3.8 Flash-Next .
// GB10 UltraFast, first bullet: a combine without a float-atomicAdd epilogue.
//
// At these token counts every touched expert sees 1..T tokens, so the work is a
// weight stream: ~4 MiB (bf16) of gate/up rows and ~2 MiB of down rows per touched
// expert, each read exactly once from HBM, with a handful of dot products per weight
// row.  Both kernels are "row owners": a block owns a fixed slice of output rows and
// walks every touched expert (plus the shared expert) for that slice, so every block
// streams the same number of bytes whatever the routing, and the grid does not depend
// on the routing.  Inside a block, wavefront w takes entries w, w+NW, ... of the
// touched list; the next entry's weight rows are loaded while the current one is
// reduced.  A lane owns 16-byte column groups g = lane + 64*c of a row, so each
// wavefront-wide load is a contiguous 1 KiB of one weight row.
//
//   gate/up: block b owns gate rows [b*RT, b*RT+RT) and the matching up rows
//            (I + the same); h[slot][r] = bf16(silu(g) * u).
//   down:    block b owns output rows [b*RO, b*RO+RO); y = bf16(h . W_d[row]) for
//            every slot of every touched expert into LDS, then the block combines
//            out[t][row] = bf16(sum_j w[t][j] * y[t*k+j][row] + gamma_t * y_s[t][row])
//            in slot order.  No float atomics; each output is written once.
#include <cstdio>

#include "device.h"
#include "internal.h"

namespace moe {

// Touched experts (counts > 0) in ascending order, computed by wavefront 0.
__device__ __forceinline__ void touched_list(const int32_t *__restrict__ counts, int E, int32_t *s_e, int *s_n) {
  if (wave_id() != 0) return;
  const int lane = lane_id();
  int n = 0;
  for (int base = 0; base < E; base += kWave) {
    const int e = base + lane;
    const int c = e < E ? counts[e] : 0;
    const uint64_t m = __ballot(c > 0);
    if (c > 0) s_e[n + __popcll(m & ((1ull << lane) - 1ull))] = e;
    n += __popcll(m);
  }
  if (lane == 0) *s_n = n;
}

struct Entry {
  const uint8_t *w;   // this expert's weight bank (bytes)
  const float *scale; // fp8 row scales of the bank, or nullptr
  int rows_half;      // I of the bank (gate/up) or its contraction length (down)
  int off, cnt;       // slot list [off, off + cnt) of sorted (routed) / tokens 0..cnt-1 (shared)
  bool routed;
};

__device__ __forceinline__ Entry gate_up_entry(const GemvArgs &a, const int32_t *s_e, int nr, int ent, int esz) {
  Entry en;
  if (ent < nr) {
    const int e = s_e[ent];
    en.w = (const uint8_t *)a.w_gu + (size_t)e * 2 * a.I * a.H * esz;
    en.scale = a.s_gu != nullptr ? a.s_gu + (size_t)e * 2 * a.I : nullptr;
    en.rows_half = a.I;
    en.off = a.offsets[e];
    en.cnt = a.counts[e];
    en.routed = true;
  } else {
    en.w = (const uint8_t *)a.ws_gu;
    en.scale = a.ss_gu;
    en.rows_half = a.I_s;
    en.off = 0;
    en.cnt = a.T;
    en.routed = false;
  }
  return en;
}

// ============================================================ gate/up, bf16 weights
// RT gate rows per block, NW wavefronts, CH = ceil(H / 512) column groups per lane.
template <int RT, int NW, int CH, bool XLDS>
__global__ __launch_bounds__(NW * kWave) void gemv_gate_up_bf16_kernel(GemvArgs a) {
  extern __shared__ uint4 s_x[];  // x [T][H/8] when XLDS
  __shared__ int32_t s_e[kMaxExperts];
  __shared__ int s_n;
  const int lane = lane_id(), wave = wave_id();
  const int r0 = blockIdx.x * RT;
  const bool do_routed = r0 < a.I;
  const bool do_shared = a.has_shared != 0 && r0 < a.I_s;
  const int G8 = a.H / 8;
  if (do_routed) touched_list(a.counts, a.E, s_e, &s_n);
  else if (threadIdx.x == 0) s_n = 0;
  if (XLDS) {
    const uint4 *xs = reinterpret_cast<const uint4 *>(a.x);
    for (int i = threadIdx.x; i < a.T * G8; i += NW * kWave) s_x[i] = xs[i];
  }
  __syncthreads();
  const int nr = s_n;
  const int NE = nr + (do_shared ? 1 : 0);

  uint4 wa[2 * RT][CH], wb[2 * RT][CH];
  auto load = [&](uint4(&w)[2 * RT][CH], int ent) {
    const Entry en = gate_up_entry(a, s_e, nr, ent, 2);
    const uint16_t *base = reinterpret_cast<const uint16_t *>(en.w);
#pragma unroll
    for (int rr = 0; rr < RT; ++rr) {
      const uint4 *g_row = reinterpret_cast<const uint4 *>(base + (size_t)(r0 + rr) * a.H);
      const uint4 *u_row = reinterpret_cast<const uint4 *>(base + (size_t)(en.rows_half + r0 + rr) * a.H);
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        const int g = lane + kWave * c;
        if (g < G8) {
          w[rr][c] = ld_stream(g_row + g);
          w[RT + rr][c] = ld_stream(u_row + g);
        } else {
          w[rr][c] = make_uint4(0, 0, 0, 0);
          w[RT + rr][c] = make_uint4(0, 0, 0, 0);
        }
      }
    }
  };
  auto compute = [&](const uint4(&w)[2 * RT][CH], int ent) {
    const Entry en = gate_up_entry(a, s_e, nr, ent, 2);
    for (int q = 0; q < en.cnt; ++q) {
      const int slot = en.routed ? a.sorted[en.off + q] : q;
      const int t = en.routed ? slot / a.k : q;
      float acc[2 * RT];
#pragma unroll
      for (int r = 0; r < 2 * RT; ++r) acc[r] = 0.0f;
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        const int g = lane + kWave * c;
        if (g < G8) {
          const uint4 xv = XLDS ? s_x[t * G8 + g] : reinterpret_cast<const uint4 *>(a.x + (size_t)t * a.H)[g];
#pragma unroll
          for (int r = 0; r < 2 * RT; ++r) acc[r] = dot8_bf16(w[r][c], xv, acc[r]);
        }
      }
#pragma unroll
      for (int r = 0; r < 2 * RT; ++r) acc[r] = wave_sum(acc[r]);
      if (lane == 0) {
        uint16_t *dst = en.routed ? a.h + (size_t)slot * a.I + r0 : a.h_s + (size_t)t * a.I_s + r0;
#pragma unroll
        for (int rr = 0; rr < RT; ++rr) {
          const float gg = acc[rr], uu = acc[RT + rr];
          dst[rr] = to_bf16(gg / (1.0f + expf(-gg)) * uu);
        }
      }
    }
  };

  int ent = wave;
  if (ent < NE) load(wa, ent);
  while (ent < NE) {
    const int e2 = ent + NW;
    if (e2 < NE) load(wb, e2);
    compute(wa, ent);
    if (e2 >= NE) break;
    const int e3 = e2 + NW;
    if (e3 < NE) load(wa, e3);
    compute(wb, e2);
    ent = e3;
  }
}

// ============================================================ gate/up, fp8 weights
// Lane column group g covers 16 codes (16 columns); CH = ceil(H / 1024).
template <int RT, int NW, int CH, bool XLDS>
__global__ __launch_bounds__(NW * kWave) void gemv_gate_up_fp8_kernel(GemvArgs a) {
  extern __shared__ uint4 s_x[];
  __shared__ int32_t s_e[kMaxExperts];
  __shared__ int s_n;
  const int lane = lane_id(), wave = wave_id();
  const int r0 = blockIdx.x * RT;
  const bool do_routed = r0 < a.I;
  const bool do_shared = a.has_shared != 0 && r0 < a.I_s;
  const int G16 = a.H / 16;
  const int G8 = a.H / 8;
  if (do_routed) touched_list(a.counts, a.E, s_e, &s_n);
  else if (threadIdx.x == 0) s_n = 0;
  if (XLDS) {
    const uint4 *xs = reinterpret_cast<const uint4 *>(a.x);
    for (int i = threadIdx.x; i < a.T * G8; i += NW * kWave) s_x[i] = xs[i];
  }
  __syncthreads();
  const int nr = s_n;
  const int NE = nr + (do_shared ? 1 : 0);

  uint4 wa[2 * RT][CH], wb[2 * RT][CH];
  auto load = [&](uint4(&w)[2 * RT][CH], int ent) {
    const Entry en = gate_up_entry(a, s_e, nr, ent, 1);
#pragma unroll
    for (int rr = 0; rr < RT; ++rr) {
      const uint4 *g_row = reinterpret_cast<const uint4 *>(en.w + (size_t)(r0 + rr) * a.H);
      const uint4 *u_row = reinterpret_cast<const uint4 *>(en.w + (size_t)(en.rows_half + r0 + rr) * a.H);
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        const int g = lane + kWave * c;
        if (g < G16) {
          w[rr][c] = ld_stream(g_row + g);
          w[RT + rr][c] = ld_stream(u_row + g);
        } else {
          w[rr][c] = make_uint4(0, 0, 0, 0);
          w[RT + rr][c] = make_uint4(0, 0, 0, 0);
        }
      }
    }
  };
  auto compute = [&](const uint4(&w)[2 * RT][CH], int ent) {
    const Entry en = gate_up_entry(a, s_e, nr, ent, 1);
    // codes -> bf16 pairs once per entry
    uint32_t wv[2 * RT][CH][8];
#pragma unroll
    for (int r = 0; r < 2 * RT; ++r)
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        wv[r][c][0] = fp8x2_to_bf16x2<false>(w[r][c].x);
        wv[r][c][1] = fp8x2_to_bf16x2<true>(w[r][c].x);
        wv[r][c][2] = fp8x2_to_bf16x2<false>(w[r][c].y);
        wv[r][c][3] = fp8x2_to_bf16x2<true>(w[r][c].y);
        wv[r][c][4] = fp8x2_to_bf16x2<false>(w[r][c].z);
        wv[r][c][5] = fp8x2_to_bf16x2<true>(w[r][c].z);
        wv[r][c][6] = fp8x2_to_bf16x2<false>(w[r][c].w);
        wv[r][c][7] = fp8x2_to_bf16x2<true>(w[r][c].w);
      }
    float sg[RT], su[RT];
#pragma unroll
    for (int rr = 0; rr < RT; ++rr) {
      sg[rr] = en.scale[r0 + rr];
      su[rr] = en.scale[en.rows_half + r0 + rr];
    }
    for (int q = 0; q < en.cnt; ++q) {
      const int slot = en.routed ? a.sorted[en.off + q] : q;
      const int t = en.routed ? slot / a.k : q;
      float acc[2 * RT];
#pragma unroll
      for (int r = 0; r < 2 * RT; ++r) acc[r] = 0.0f;
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        const int g = lane + kWave * c;
        if (g < G16) {
          uint4 x0, x1;
          if (XLDS) {
            x0 = s_x[t * G8 + 2 * g];
            x1 = s_x[t * G8 + 2 * g + 1];
          } else {
            const uint4 *xr = reinterpret_cast<const uint4 *>(a.x + (size_t)t * a.H);
            x0 = xr[2 * g];
            x1 = xr[2 * g + 1];
          }
#pragma unroll
          for (int r = 0; r < 2 * RT; ++r) {
            float s = acc[r];
            s = dot2_bf16(wv[r][c][0], x0.x, s);
            s = dot2_bf16(wv[r][c][1], x0.y, s);
            s = dot2_bf16(wv[r][c][2], x0.z, s);
            s = dot2_bf16(wv[r][c][3], x0.w, s);
            s = dot2_bf16(wv[r][c][4], x1.x, s);
            s = dot2_bf16(wv[r][c][5], x1.y, s);
            s = dot2_bf16(wv[r][c][6], x1.z, s);
            s = dot2_bf16(wv[r][c][7], x1.w, s);
            acc[r] = s;
          }
        }
      }
#pragma unroll
      for (int r = 0; r < 2 * RT; ++r) acc[r] = wave_sum(acc[r]);
      if (lane == 0) {
        uint16_t *dst = en.routed ? a.h + (size_t)slot * a.I + r0 : a.h_s + (size_t)t * a.I_s + r0;
#pragma unroll
        for (int rr = 0; rr < RT; ++rr) {
          const float gg = acc[rr] * sg[rr], uu = acc[RT + rr] * su[rr];
          dst[rr] = to_bf16(gg / (1.0f + expf(-gg)) * uu);
        }
      }
    }
  };

  int ent = wave;
  if (ent < NE) load(wa, ent);
  while (ent < NE) {
    const int e2 = ent + NW;
    if (e2 < NE) load(wb, e2);
    compute(wa, ent);
    if (e2 >= NE) break;
    const int e3 = e2 + NW;
    if (e3 < NE) load(wa, e3);
    compute(wb, e2);
    ent = e3;
  }
}

// ============================================================ down + combine
// RO output rows per block; a lane's column group covers 8 bf16 of h (bf16 weights)
// or 16 of them (fp8 weights, ESZ = 1).  CI = groups per lane.
template <int RO, int NW, int CI, int ESZ>
__global__ __launch_bounds__(NW * kWave) void gemv_down_kernel(GemvArgs a) {
  extern __shared__ float s_y[];  // [T*k][RO] then [T][RO] for the shared expert
  __shared__ int32_t s_e[kMaxExperts];
  __shared__ int s_n;
  const int lane = lane_id(), wave = wave_id();
  const int o0 = blockIdx.x * RO;
  float *s_ys = s_y + (size_t)a.T * a.k * RO;
  touched_list(a.counts, a.E, s_e, &s_n);
  __syncthreads();
  const int nr = s_n;
  const int NE = nr + (a.has_shared ? 1 : 0);
  constexpr int VPG = ESZ == 2 ? 8 : 16;  // weights per 16-byte group

  auto entry = [&](int ent) {
    Entry en;
    if (ent < nr) {
      const int e = s_e[ent];
      en.w = (const uint8_t *)a.w_d + (size_t)e * a.H * a.I * ESZ;
      en.scale = a.s_d != nullptr ? a.s_d + (size_t)e * a.H : nullptr;
      en.rows_half = a.I;
      en.off = a.offsets[e];
      en.cnt = a.counts[e];
      en.routed = true;
    } else {
      en.w = (const uint8_t *)a.ws_d;
      en.scale = a.ss_d;
      en.rows_half = a.I_s;
      en.off = 0;
      en.cnt = a.T;
      en.routed = false;
    }
    return en;
  };
  uint4 wa[RO][CI], wb[RO][CI];
  auto load = [&](uint4(&w)[RO][CI], int ent) {
    const Entry en = entry(ent);
    const int G = en.rows_half / VPG;
#pragma unroll
    for (int rr = 0; rr < RO; ++rr) {
      const uint4 *row = reinterpret_cast<const uint4 *>(en.w + (size_t)(o0 + rr) * en.rows_half * ESZ);
#pragma unroll
      for (int c = 0; c < CI; ++c) {
        const int g = lane + kWave * c;
        w[rr][c] = g < G ? ld_stream(row + g) : make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto compute = [&](const uint4(&w)[RO][CI], int ent) {
    const Entry en = entry(ent);
    const int G = en.rows_half / VPG;
    float sc[RO];
#pragma unroll
    for (int rr = 0; rr < RO; ++rr) sc[rr] = en.scale != nullptr ? en.scale[o0 + rr] : 1.0f;
    for (int q = 0; q < en.cnt; ++q) {
      const int slot = en.routed ? a.sorted[en.off + q] : q;
      const uint16_t *hrow = en.routed ? a.h + (size_t)slot * a.I : a.h_s + (size_t)q * a.I_s;
      float acc[RO];
#pragma unroll
      for (int rr = 0; rr < RO; ++rr) acc[rr] = 0.0f;
#pragma unroll
      for (int c = 0; c < CI; ++c) {
        const int g = lane + kWave * c;
        if (g < G) {
          if (ESZ == 2) {
            const uint4 hv = reinterpret_cast<const uint4 *>(hrow)[g];
#pragma unroll
            for (int rr = 0; rr < RO; ++rr) acc[rr] = dot8_bf16(w[rr][c], hv, acc[rr]);
          } else {
            const uint4 h0 = reinterpret_cast<const uint4 *>(hrow)[2 * g];
            const uint4 h1 = reinterpret_cast<const uint4 *>(hrow)[2 * g + 1];
#pragma unroll
            for (int rr = 0; rr < RO; ++rr) {
              float s = acc[rr];
              s = dot2_bf16(fp8x2_to_bf16x2<false>(w[rr][c].x), h0.x, s);
              s = dot2_bf16(fp8x2_to_bf16x2<true>(w[rr][c].x), h0.y, s);
              s = dot2_bf16(fp8x2_to_bf16x2<false>(w[rr][c].y), h0.z, s);
              s = dot2_bf16(fp8x2_to_bf16x2<true>(w[rr][c].y), h0.w, s);
              s = dot2_bf16(fp8x2_to_bf16x2<false>(w[rr][c].z), h1.x, s);
              s = dot2_bf16(fp8x2_to_bf16x2<true>(w[rr][c].z), h1.y, s);
              s = dot2_bf16(fp8x2_to_bf16x2<false>(w[rr][c].w), h1.z, s);
              s = dot2_bf16(fp8x2_to_bf16x2<true>(w[rr][c].w), h1.w, s);
              acc[rr] = s;
            }
          }
        }
      }
#pragma unroll
      for (int rr = 0; rr < RO; ++rr) acc[rr] = wave_sum(acc[rr]);
      if (lane == 0) {
        float *dst = en.routed ? s_y + (size_t)slot * RO : s_ys + (size_t)q * RO;
#pragma unroll
        for (int rr = 0; rr < RO; ++rr) dst[rr] = round_bf16(acc[rr] * sc[rr]);
      }
    }
  };

  int ent = wave;
  if (ent < NE) load(wa, ent);
  while (ent < NE) {
    const int e2 = ent + NW;
    if (e2 < NE) load(wb, e2);
    compute(wa, ent);
    if (e2 >= NE) break;
    const int e3 = e2 + NW;
    if (e3 < NE) load(wa, e3);
    compute(wb, e2);
    ent = e3;
  }
  __syncthreads();
  // combine in slot order, fp32, one write per output element
  for (int idx = threadIdx.x; idx < a.T * RO; idx += NW * kWave) {
    const int t = idx / RO, rr = idx % RO;
    float acc = 0.0f;
    for (int j = 0; j < a.k; ++j) acc = fmaf(a.topk_w[t * a.k + j], s_y[(size_t)(t * a.k + j) * RO + rr], acc);
    if (a.has_shared) acc = fmaf(a.gamma[t], s_ys[t * RO + rr], acc);
    a.out[(size_t)t * a.H + o0 + rr] = to_bf16(acc);
  }
}

// ============================================================ launchers
namespace {
constexpr int kGuRT = 2, kGuNW = 4;
constexpr int kDnRO = 8, kDnNW = 4;
constexpr size_t kLdsBudget = 60 * 1024;
}  // namespace

template <int CH, bool XLDS>
static void launch_gu(const GemvArgs &a, hipStream_t s, dim3 grid, size_t lds) {
  if (a.wtype == 0)
    hipLaunchKernelGGL((gemv_gate_up_bf16_kernel<kGuRT, kGuNW, CH, XLDS>), grid, dim3(kGuNW * kWave), lds, s, a);
  else
    hipLaunchKernelGGL((gemv_gate_up_fp8_kernel<kGuRT, kGuNW, CH, XLDS>), grid, dim3(kGuNW * kWave), lds, s, a);
}

hipError_t launch_gemv_gate_up(const GemvArgs &a, hipStream_t s, char *desc, size_t desc_len) {
  const int rows = a.I > (a.has_shared ? a.I_s : 0) ? a.I : a.I_s;
  dim3 grid((rows + kGuRT - 1) / kGuRT);
  const size_t xbytes = (size_t)a.T * a.H * 2;
  const bool xlds = xbytes + kMaxExperts * 4 + 64 <= kLdsBudget;
  const int per_group = a.wtype == 0 ? 512 : 1024;  // columns per lane group sweep
  const int ch = (a.H + per_group - 1) / per_group;
  const size_t lds = xlds ? xbytes : 0;
  if (desc) snprintf(desc, desc_len, "gemv_gate_up_%s<RT=%d,NW=%d,CH=%d,XLDS=%d> grid=%u block=%d", a.wtype == 0 ? "bf16" : "fp8", kGuRT, kGuNW, ch, (int)xlds, grid.x, kGuNW * kWave);
  if (ch <= 1) { if (xlds) launch_gu<1, true>(a, s, grid, lds); else launch_gu<1, false>(a, s, grid, lds); }
  else if (ch <= 2) { if (xlds) launch_gu<2, true>(a, s, grid, lds); else launch_gu<2, false>(a, s, grid, lds); }
  else if (ch <= 4) { if (xlds) launch_gu<4, true>(a, s, grid, lds); else launch_gu<4, false>(a, s, grid, lds); }
  else if (ch <= 8) { if (xlds) launch_gu<8, true>(a, s, grid, lds); else launch_gu<8, false>(a, s, grid, lds); }
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

template <int CI>
static void launch_dn(const GemvArgs &a, hipStream_t s, dim3 grid, size_t lds) {
  if (a.wtype == 0)
    hipLaunchKernelGGL((gemv_down_kernel<kDnRO, kDnNW, CI, 2>), grid, dim3(kDnNW * kWave), lds, s, a);
  else
    hipLaunchKernelGGL((gemv_down_kernel<kDnRO, kDnNW, CI, 1>), grid, dim3(kDnNW * kWave), lds, s, a);
}

hipError_t launch_gemv_down(const GemvArgs &a, hipStream_t s, char *desc, size_t desc_len) {
  dim3 grid(a.H / kDnRO);
  const size_t lds = ((size_t)a.T * a.k + (a.has_shared ? a.T : 0)) * kDnRO * sizeof(float);
  const int kmax = a.I > (a.has_shared ? a.I_s : 0) ? a.I : a.I_s;
  const int per_group = a.wtype == 0 ? 512 : 1024;
  const int ci = (kmax + per_group - 1) / per_group;
  if (desc) snprintf(desc, desc_len, "gemv_down_combine_%s<RO=%d,NW=%d,CI=%d> grid=%u block=%d", a.wtype == 0 ? "bf16" : "fp8", kDnRO, kDnNW, ci, grid.x, kDnNW * kWave);
  if (ci <= 1) launch_dn<1>(a, s, grid, lds);
  else if (ci <= 2) launch_dn<2>(a, s, grid, lds);
  else if (ci <= 4) launch_dn<4>(a, s, grid, lds);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace moe
