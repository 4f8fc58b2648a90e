// gemv.hip -- decode/verify-block expert kernels for gfx950 (T <= 64 tokens).
//
// veloGB10 README, "Kernel work": grouped MoE expert kernels that never rebuild full
// weights; the shared expert overlapped with the MoE step.  Qwen3.8 Flash-Next .
// GB10 UltraFast, first bullet: a combine without a float-atomicAdd epilogue.
//
// At these token counts every touched expert sees 1..T tokens, so the work is a weight
// stream: ~4 MiB (bf16) of gate/up rows and ~2 MiB of down rows per touched expert,
// each read exactly once from HBM, with a few dot products per row.  Both kernels are
// "row owners": a block owns a fixed slice of output rows and walks every touched
// expert (plus the shared expert) for that slice, so every block streams the same bytes
// whatever the routing and the grid does not depend on the routing.
//
// Lane mapping: a wavefront is four 16-lane rows; DPP row r of the wavefront holds one
// weight row, each lane 16-byte column groups g = lane%16 + 16c, so one load
// instruction fetches 256 contiguous bytes from each of four weight rows and the four
// dot products finish with one 4-step DPP sum inside the rows.  Wavefront w of a block
// takes entries w, w+NW, ... of the touched list; the next entry's rows are in flight
// (non-temporal loads) while the current entry is reduced.  Tokens (gate/up) and the
// intermediate h (down) are staged in LDS once per block, so the loop reads only LDS
// and registers besides the weight stream.
//
//   gate/up: block b owns gate rows 2b, 2b+1 and the matching up rows I+2b, I+2b+1
//            (DPP rows 0..3); h[slot][r] = bf16(silu(g) * u).
//   down:    block b owns output rows 8b..8b+7 (DPP rows 0..3 hold 8b+r and 8b+4+r);
//            y = bf16(h . W_d[row]) for every slot of every touched expert goes to LDS,
//            then the block combines out[t][row] = bf16(sum_j w[t][j] * y[t*k+j][row]
//            + gamma_t * y_s[t][row]) in slot order.  No float atomics.
#include <cstdio>
#include <mutex>

#include "device.h"
#include "internal.h"
#include "mxfp4.h"

namespace moe {

namespace {
constexpr int kGuNW = 8;      // wavefronts per gate/up block
constexpr int kDnNW = 8;      // wavefronts per down block
constexpr int kDnRows = 8;    // output rows per down block
constexpr size_t kLdsMax = 150 * 1024;
}  // namespace

__device__ __forceinline__ size_t align16(size_t v) { return (v + 15) & ~(size_t)15; }

// LDS image of the touched list: e[nr], start[nr+1], slots[T*k]
struct ListLds {
  const int32_t *e;
  const int32_t *start;
  const int32_t *slots;
};

__device__ __forceinline__ ListLds stage_list(const GemvArgs &a, int nr, int32_t *base, int nthreads) {
  int32_t *e = base, *start = base + nr, *slots = base + 2 * nr + 1;
  const int n_slots = a.T * a.k;
  for (int i = threadIdx.x; i < nr; i += nthreads) e[i] = a.tl_e[i];
  for (int i = threadIdx.x; i <= nr; i += nthreads) start[i] = a.tl_start[i];
  for (int i = threadIdx.x; i < n_slots; i += nthreads) slots[i] = a.tl_slots[i];
  return ListLds{e, start, slots};
}

__device__ __forceinline__ void copy_to_lds(uint4 *dst, const uint4 *src, int n, int nthreads) {
  for (int i = threadIdx.x; i < n; i += nthreads) dst[i] = src[i];
}

// ============================================================ gate/up
// VPG: weights per 16-byte group (8 bf16, 16 fp8 codes, 32 MXFP4 codes, which are also one
// scale block).  CG: 16-byte groups per lane per row.
template <int VPG, int CG, bool XLDS>
__global__ __launch_bounds__(kGuNW * kWave) void gemv_gate_up_kernel(GemvArgs a) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  constexpr int NT = kGuNW * kWave;
  const int lane = lane_id(), wave = wave_id(), rg = lane >> 4, l16 = lane & 15;
  const int r0 = blockIdx.x * 2;
  const bool do_routed = r0 < a.I;
  const bool do_shared = a.has_shared != 0 && r0 < a.I_s;
  const int nr = do_routed ? a.tl_n[0] : 0;
  const int NE = nr + (do_shared ? 1 : 0);
  const int H = a.H;
  const int G = H / VPG;       // groups per weight row
  const int G8 = H / 8;        // 16-byte groups per token row

  // weight row of this lane for entry `ent` (expert id known), and its MXFP4 block scales
  auto row_of = [&](int ent, int e, const uint8_t *&srow) -> const uint4 * {
    const uint8_t *bank, *sbank;
    int Iw;
    if (ent < nr) {
      bank = (const uint8_t *)a.w_gu + (size_t)e * 2 * a.I * G * 16;
      sbank = a.x_gu + (size_t)e * 2 * a.I * G;
      Iw = a.I;
    } else {
      bank = (const uint8_t *)a.ws_gu;
      sbank = a.xs_gu;
      Iw = a.I_s;
    }
    const int row = rg < 2 ? r0 + rg : Iw + r0 + (rg - 2);
    srow = VPG == 32 ? sbank + (size_t)row * G : nullptr;
    return reinterpret_cast<const uint4 *>(bank + (size_t)row * G * 16);
  };
  uint4 wa[CG], wb[CG];
  uint32_t xa[VPG == 32 ? CG : 1], xb[VPG == 32 ? CG : 1];  // MXFP4: scale byte of each group
  auto load = [&](uint4(&w)[CG], uint32_t(&xs)[VPG == 32 ? CG : 1], int ent, int e) {
    const uint8_t *srow;
    const uint4 *p = row_of(ent, e, srow);
#pragma unroll
    for (int c = 0; c < CG; ++c) {
      const int g = l16 + 16 * c;
      w[c] = g < G ? ld_stream(p + g) : make_uint4(0, 0, 0, 0);
      if (VPG == 32) xs[c] = g < G ? srow[g] : 127u;
    }
  };

  // blocks (b, y) for y < gridDim.y share row pair b and split the entries: wavefront w of
  // block y takes entries y*NW + w, then every NW*gridDim.y-th (more of a small weight
  // format in flight per row pair)
  const int NWS = kGuNW * gridDim.y;
  // token chunk z of gridDim.z: tokens [t_lo, t_hi), whose rows fit the LDS together.  A
  // block computes the slots of its chunk's tokens only (each slot once, with the same
  // arithmetic as without chunks) and walks only the entries that have such slots.
  const bool chunked = gridDim.z > 1;
  const int TCH = (a.T + gridDim.z - 1) / gridDim.z;
  const int t_lo = blockIdx.z * TCH, t_hi = min(a.T, t_lo + TCH);
  // first entry's rows go out before the staging below (with chunks, the entries are known
  // only after it)
  int ent = blockIdx.y * kGuNW + wave;
  if (!chunked && ent < NE) load(wa, xa, ent, ent < nr ? a.tl_e[ent] : 0);

  int32_t *lbase = reinterpret_cast<int32_t *>(smem);
  const ListLds lst = stage_list(a, nr, lbase, NT);
  // chunked: the entries with slots in the chunk, in order, and each one's slot range
  int32_t *c_ent = lbase + 2 * nr + 1 + a.T * a.k, *c_q0 = c_ent + NE, *c_q1 = c_q0 + NE;
  int32_t *c_tmp = c_q1 + NE;  // block scan scratch (kGuNW + 1 ints)
  const size_t xoff = align16((size_t)(2 * nr + 1 + a.T * a.k + (chunked ? 3 * NE + kGuNW + 1 : 0)) * 4);
  const uint4 *xs;
  int x_t0 = 0;  // first token row held in xs
  if (XLDS) {
    uint4 *s_x = reinterpret_cast<uint4 *>(smem + xoff);
    copy_to_lds(s_x, reinterpret_cast<const uint4 *>(a.x) + (size_t)t_lo * G8, (t_hi - t_lo) * G8, NT);
    xs = s_x;
    x_t0 = t_lo;
  } else {
    xs = reinterpret_cast<const uint4 *>(a.x);
  }
  __syncthreads();
  int NCE = NE;  // entries this block walks
  if (chunked) {
    // an entry's slots are in slot order, i.e. in token order: its chunk slots are one run
    int run = 0;
    for (int i0 = 0; i0 < NE; i0 += NT) {
      const int i = i0 + threadIdx.x;
      int q0 = 0, q1 = 0;
      if (i < nr) {
        const int s1 = lst.start[i + 1];
        q0 = lst.start[i];
        while (q0 < s1 && lst.slots[q0] / a.k < t_lo) ++q0;
        q1 = q0;
        while (q1 < s1 && lst.slots[q1] / a.k < t_hi) ++q1;
      } else if (i < NE) {  // the shared expert: every token of the chunk
        q0 = t_lo;
        q1 = t_hi;
      }
      const int keep = q1 > q0 ? 1 : 0;
      int cnt;
      const int idx = run + block_excl_scan<NT>(keep, c_tmp, &cnt);
      if (keep) {
        c_ent[idx] = i;
        c_q0[idx] = q0;
        c_q1[idx] = q1;
      }
      run += cnt;
    }
    __syncthreads();
    NCE = run;
    if (ent < NCE) load(wa, xa, ent, c_ent[ent] < nr ? lst.e[c_ent[ent]] : 0);
  }
  // the walked entry ci: its index in the list (nr: the shared expert) and slot range
  auto entry_of = [&](int ci) { return chunked ? c_ent[ci] : ci; };

  auto compute = [&](const uint4(&w)[CG], const uint32_t(&ws)[VPG == 32 ? CG : 1], int ci) {
    const int ent = entry_of(ci);
    const bool routed = ent < nr;
    const int e = routed ? lst.e[ent] : 0;
    const int q0 = chunked ? c_q0[ci] : routed ? lst.start[ent] : 0;
    const int q1 = chunked ? c_q1[ci] : routed ? lst.start[ent + 1] : a.T;
    float bsc[VPG == 32 ? CG : 1];  // MXFP4 block scales of the lane's groups
#pragma unroll
    for (int c = 0; c < (VPG == 32 ? CG : 1); ++c) bsc[c] = VPG == 32 ? e8m0_scale(ws[c]) : 1.0f;
    float sg0 = 1.f, sg1 = 1.f, su0 = 1.f, su1 = 1.f;
    if (VPG == 16) {
      const float *sc = routed ? a.s_gu + (size_t)e * 2 * a.I : a.ss_gu;
      const int Iw = routed ? a.I : a.I_s;
      sg0 = sc[r0];
      sg1 = sc[r0 + 1];
      su0 = sc[Iw + r0];
      su1 = sc[Iw + r0 + 1];
    }
    for (int q = q0; q < q1; ++q) {
      const int slot = routed ? lst.slots[q] : q;
      const int t = routed ? slot / a.k : q;
      const uint4 *xr = xs + (size_t)(t - x_t0) * G8;
      float acc = 0.0f;
#pragma unroll
      for (int c = 0; c < CG; ++c) {
        const int g = l16 + 16 * c;
        if (g < G) {
          if (VPG == 8) {
            acc = dot8_bf16(w[c], xr[g], acc);
          } else if (VPG == 32) {
            acc = fmaf(dot32_fp4_bf16(w[c], xr + 4 * g), bsc[c], acc);
          } else {
            const uint4 x0 = xr[2 * g], x1 = xr[2 * g + 1];
            acc = dot2_bf16(fp8x2_to_bf16x2<false>(w[c].x), x0.x, acc);
            acc = dot2_bf16(fp8x2_to_bf16x2<true>(w[c].x), x0.y, acc);
            acc = dot2_bf16(fp8x2_to_bf16x2<false>(w[c].y), x0.z, acc);
            acc = dot2_bf16(fp8x2_to_bf16x2<true>(w[c].y), x0.w, acc);
            acc = dot2_bf16(fp8x2_to_bf16x2<false>(w[c].z), x1.x, acc);
            acc = dot2_bf16(fp8x2_to_bf16x2<true>(w[c].z), x1.y, acc);
            acc = dot2_bf16(fp8x2_to_bf16x2<false>(w[c].w), x1.z, acc);
            acc = dot2_bf16(fp8x2_to_bf16x2<true>(w[c].w), x1.w, acc);
          }
        }
      }
      acc = row16_sum(acc);
      const float g0 = lane_value(acc, 0) * sg0, g1 = lane_value(acc, 16) * sg1;
      const float u0 = lane_value(acc, 32) * su0, u1 = lane_value(acc, 48) * su1;
      if (lane == 0) {
        uint16_t *dst = routed ? a.h + (size_t)slot * a.I + r0 : a.h_s + (size_t)t * a.I_s + r0;
        *reinterpret_cast<uint32_t *>(dst) =
            pack_bf16x2(g0 / (1.0f + expf(-g0)) * u0, g1 / (1.0f + expf(-g1)) * u1);
      }
    }
  };

  auto load_ci = [&](uint4(&w)[CG], uint32_t(&xs_)[VPG == 32 ? CG : 1], int ci) {
    const int en = entry_of(ci);
    load(w, xs_, en, en < nr ? lst.e[en] : 0);
  };
  while (ent < NCE) {
    const int e2 = ent + NWS;
    if (e2 < NCE) load_ci(wb, xb, e2);
    compute(wa, xa, ent);
    if (e2 >= NCE) break;
    const int e3 = e2 + NWS;
    if (e3 < NCE) load_ci(wa, xa, e3);
    compute(wb, xb, e2);
    ent = e3;
  }
}

// ============================================================ down + combine
// CG: 16-byte groups per lane per weight row; each lane holds two rows (o0 + rg and
// o0 + 4 + rg).
template <int VPG, int CG, bool HLDS>
__global__ __launch_bounds__(kDnNW * kWave) void gemv_down_kernel(GemvArgs a) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  constexpr int NT = kDnNW * kWave;
  constexpr int NS = VPG == 32 ? CG : 1;  // MXFP4 scale bytes per lane and row
  const int lane = lane_id(), wave = wave_id(), rg = lane >> 4, l16 = lane & 15;
  const int o0 = blockIdx.x * kDnRows;
  const int nr = a.tl_n[0];
  const int NE = nr + (a.has_shared ? 1 : 0);
  const int n_slots = a.T * a.k;

  uint4 wa[2][CG], wb[2][CG];
  uint32_t xa[2][NS], xb[2][NS];  // MXFP4: scale byte of each group
  auto load = [&](uint4(&w)[2][CG], uint32_t(&xs)[2][NS], int ent, int e) {
    const int K = ent < nr ? a.I : a.I_s;
    const int G = K / VPG;
    const uint8_t *bank = ent < nr ? (const uint8_t *)a.w_d + (size_t)e * a.H * G * 16 : (const uint8_t *)a.ws_d;
    const uint8_t *sbank = ent < nr ? a.x_d + (size_t)e * a.H * G : a.xs_d;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int row = o0 + 4 * s + rg;
      const uint4 *p = reinterpret_cast<const uint4 *>(bank + (size_t)row * G * 16);
#pragma unroll
      for (int c = 0; c < CG; ++c) {
        const int g = l16 + 16 * c;
        w[s][c] = g < G ? ld_stream(p + g) : make_uint4(0, 0, 0, 0);
        if (VPG == 32) xs[s][c] = g < G ? sbank[(size_t)row * G + g] : 127u;
      }
    }
  };

  int ent = wave;
  if (ent < NE) load(wa, xa, ent, ent < nr ? a.tl_e[ent] : 0);

  // LDS: list, y [T*k][8] fp32, y_s [T][8] fp32, then h [T*k][I] and h_s [T][I_s] bf16
  int32_t *lbase = reinterpret_cast<int32_t *>(smem);
  const ListLds lst = stage_list(a, nr, lbase, NT);
  float *s_y = reinterpret_cast<float *>(smem + align16((size_t)(2 * nr + 1 + n_slots) * 4));
  float *s_ys = s_y + (size_t)n_slots * kDnRows;
  const uint4 *hs, *hss;
  if (HLDS) {
    uint4 *h_l = reinterpret_cast<uint4 *>(reinterpret_cast<char *>(s_ys) +
                                           align16((size_t)(a.has_shared ? a.T : 0) * kDnRows * 4));
    copy_to_lds(h_l, reinterpret_cast<const uint4 *>(a.h), n_slots * a.I / 8, NT);
    uint4 *hs_l = h_l + (size_t)n_slots * a.I / 8;
    if (a.has_shared) copy_to_lds(hs_l, reinterpret_cast<const uint4 *>(a.h_s), a.T * a.I_s / 8, NT);
    hs = h_l;
    hss = hs_l;
  } else {
    hs = reinterpret_cast<const uint4 *>(a.h);
    hss = reinterpret_cast<const uint4 *>(a.h_s);
  }
  __syncthreads();

  auto compute = [&](const uint4(&w)[2][CG], const uint32_t(&ws)[2][NS], int ent) {
    const bool routed = ent < nr;
    const int e = routed ? lst.e[ent] : 0;
    const int K = routed ? a.I : a.I_s;
    const int G = K / VPG;
    const int q0 = routed ? lst.start[ent] : 0;
    const int q1 = routed ? lst.start[ent + 1] : a.T;
    float bsc[2][NS];  // MXFP4 block scales
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int c = 0; c < NS; ++c) bsc[s][c] = VPG == 32 ? e8m0_scale(ws[s][c]) : 1.0f;
    float sc0 = 1.f, sc1 = 1.f;
    if (VPG == 16) {
      const float *sc = routed ? a.s_d + (size_t)e * a.H : a.ss_d;
      sc0 = sc[o0 + rg];
      sc1 = sc[o0 + 4 + rg];
    }
    if constexpr (HLDS) {
      for (int q = q0; q < q1; ++q) {
        const int slot = routed ? lst.slots[q] : q;
        const uint4 *hr = routed ? hs + (size_t)slot * (a.I / 8) : hss + (size_t)q * (a.I_s / 8);
        float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
        for (int c = 0; c < CG; ++c) {
          const int g = l16 + 16 * c;
          if (g < G) {
            if (VPG == 8) {
              const uint4 hv = hr[g];
              acc0 = dot8_bf16(w[0][c], hv, acc0);
              acc1 = dot8_bf16(w[1][c], hv, acc1);
            } else if (VPG == 32) {
              acc0 = fmaf(dot32_fp4_bf16(w[0][c], hr + 4 * g), bsc[0][c], acc0);
              acc1 = fmaf(dot32_fp4_bf16(w[1][c], hr + 4 * g), bsc[1][c], acc1);
            } else {
              const uint4 h0 = hr[2 * g], h1 = hr[2 * g + 1];
#pragma unroll
              for (int s = 0; s < 2; ++s) {
                float acc = s == 0 ? acc0 : acc1;
                acc = dot2_bf16(fp8x2_to_bf16x2<false>(w[s][c].x), h0.x, acc);
                acc = dot2_bf16(fp8x2_to_bf16x2<true>(w[s][c].x), h0.y, acc);
                acc = dot2_bf16(fp8x2_to_bf16x2<false>(w[s][c].y), h0.z, acc);
                acc = dot2_bf16(fp8x2_to_bf16x2<true>(w[s][c].y), h0.w, acc);
                acc = dot2_bf16(fp8x2_to_bf16x2<false>(w[s][c].z), h1.x, acc);
                acc = dot2_bf16(fp8x2_to_bf16x2<true>(w[s][c].z), h1.y, acc);
                acc = dot2_bf16(fp8x2_to_bf16x2<false>(w[s][c].w), h1.z, acc);
                acc = dot2_bf16(fp8x2_to_bf16x2<true>(w[s][c].w), h1.w, acc);
                if (s == 0) acc0 = acc;
                else acc1 = acc;
              }
            }
          }
        }
        acc0 = row16_sum(acc0);
        acc1 = row16_sum(acc1);
        if (l16 == 0) {
          float *dst = routed ? s_y + (size_t)slot * kDnRows : s_ys + (size_t)q * kDnRows;
          dst[rg] = round_bf16(acc0 * sc0);
          dst[4 + rg] = round_bf16(acc1 * sc1);
        }
      }

    } else {
      // h from global memory (too large for LDS): the h of kPS slots (as many as the
      // registers hold without spilling) is loaded together, then used, so the slots' load
      // latencies overlap; each slot's sums are unchanged
      constexpr int XPG = VPG / 8, NH = CG * XPG, kPS = NH <= 4 ? 4 : NH <= 8 ? 2 : 1;
      for (int q = q0; q < q1; q += kPS) {
        uint4 hb[kPS][NH];
#pragma unroll
        for (int u = 0; u < kPS; ++u) {
          if (q + u < q1) {
            const int slot = routed ? lst.slots[q + u] : q + u;
            const uint4 *hr = routed ? hs + (size_t)slot * (a.I / 8) : hss + (size_t)(q + u) * (a.I_s / 8);
#pragma unroll
            for (int c = 0; c < CG; ++c) {
              const int g = l16 + 16 * c;
#pragma unroll
              for (int d = 0; d < XPG; ++d) hb[u][c * XPG + d] = g < G ? hr[XPG * g + d] : make_uint4(0, 0, 0, 0);
            }
          }
        }
#pragma unroll
        for (int u = 0; u < kPS; ++u) {
          if (q + u < q1) {
            const int slot = routed ? lst.slots[q + u] : q + u;
            float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
            for (int c = 0; c < CG; ++c) {
              const int g = l16 + 16 * c;
              if (g < G) {
                if (VPG == 8) {
                  acc0 = dot8_bf16(w[0][c], hb[u][c], acc0);
                  acc1 = dot8_bf16(w[1][c], hb[u][c], acc1);
                } else if (VPG == 32) {
                  acc0 = fmaf(dot32_fp4_bf16(w[0][c], &hb[u][4 * c]), bsc[0][c], acc0);
                  acc1 = fmaf(dot32_fp4_bf16(w[1][c], &hb[u][4 * c]), bsc[1][c], acc1);
                } else {
                  const uint4 h0 = hb[u][2 * c], h1 = hb[u][2 * c + 1];
#pragma unroll
                  for (int s2 = 0; s2 < 2; ++s2) {
                    float acc = s2 == 0 ? acc0 : acc1;
                    acc = dot2_bf16(fp8x2_to_bf16x2<false>(w[s2][c].x), h0.x, acc);
                    acc = dot2_bf16(fp8x2_to_bf16x2<true>(w[s2][c].x), h0.y, acc);
                    acc = dot2_bf16(fp8x2_to_bf16x2<false>(w[s2][c].y), h0.z, acc);
                    acc = dot2_bf16(fp8x2_to_bf16x2<true>(w[s2][c].y), h0.w, acc);
                    acc = dot2_bf16(fp8x2_to_bf16x2<false>(w[s2][c].z), h1.x, acc);
                    acc = dot2_bf16(fp8x2_to_bf16x2<true>(w[s2][c].z), h1.y, acc);
                    acc = dot2_bf16(fp8x2_to_bf16x2<false>(w[s2][c].w), h1.z, acc);
                    acc = dot2_bf16(fp8x2_to_bf16x2<true>(w[s2][c].w), h1.w, acc);
                    if (s2 == 0) acc0 = acc;
                    else acc1 = acc;
                  }
                }
              }
            }
            acc0 = row16_sum(acc0);
            acc1 = row16_sum(acc1);
            if (l16 == 0) {
              float *dst = routed ? s_y + (size_t)slot * kDnRows : s_ys + (size_t)(q + u) * kDnRows;
              dst[rg] = round_bf16(acc0 * sc0);
              dst[4 + rg] = round_bf16(acc1 * sc1);
            }
          }
        }
      }
    }
  };

  while (ent < NE) {
    const int e2 = ent + kDnNW;
    if (e2 < NE) load(wb, xb, e2, e2 < nr ? lst.e[e2] : 0);
    compute(wa, xa, ent);
    if (e2 >= NE) break;
    const int e3 = e2 + kDnNW;
    if (e3 < NE) load(wa, xa, e3, e3 < nr ? lst.e[e3] : 0);
    compute(wb, xb, e2);
    ent = e3;
  }
  __syncthreads();
  // combine in slot order, fp32, one write per output element
  for (int idx = threadIdx.x; idx < a.T * kDnRows; idx += NT) {
    const int t = idx / kDnRows, rr = idx % kDnRows;
    float acc = 0.0f;
    for (int j = 0; j < a.k; ++j)
      acc = fmaf(a.topk_w[t * a.k + j], s_y[(size_t)(t * a.k + j) * kDnRows + rr], acc);
    if (a.has_shared) acc = fmaf(a.gamma[t], s_ys[t * kDnRows + rr], acc);
    a.out[(size_t)t * a.H + o0 + rr] = to_bf16(acc);
  }
}

// ============================================================ launchers
static size_t list_bytes(const GemvArgs &a) { return (((size_t)(2 * a.E + 1 + a.T * a.k) * 4) + 15) & ~(size_t)15; }

// Dynamic LDS above 64 KiB has to be allowed per kernel (gfx950 has 160 KiB per CU);
// the largest size opened so far is remembered per (kernel, device).
static hipError_t set_lds(const void *kernel, size_t bytes) {
  if (bytes <= 64 * 1024) return hipSuccess;
  struct Entry {
    const void *k;
    int dev;
    size_t allowed;
  };
  static std::mutex mu;
  static Entry table[64];
  static int used = 0;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  Entry *hit = nullptr;
  for (int i = 0; i < used; ++i)
    if (table[i].k == kernel && table[i].dev == dev) hit = &table[i];
  if (hit != nullptr && bytes <= hit->allowed) return hipSuccess;
  e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (e != hipSuccess) return e;
  if (hit == nullptr && used < 64) hit = &table[used++];
  if (hit != nullptr) *hit = Entry{kernel, dev, bytes};
  return hipSuccess;
}

template <int VPG, int CG>
static hipError_t launch_gu(const GemvArgs &a, hipStream_t s, dim3 grid, bool xlds, size_t lds) {
  if (xlds) {
    auto k = gemv_gate_up_kernel<VPG, CG, true>;
    hipError_t e = set_lds(reinterpret_cast<const void *>(k), lds);
    if (e != hipSuccess) return e;
    return launch_k(k, grid, dim3(kGuNW * kWave), lds, s, a);
  }
  // (launch_k returns the launch's own status: a later hipGetLastError would read it cleared)
  return launch_k(gemv_gate_up_kernel<VPG, CG, false>, grid, dim3(kGuNW * kWave), lds, s, a);
}

hipError_t launch_gemv_gate_up(const GemvArgs &a, hipStream_t s, char *desc, size_t desc_len) {
  const int rows = a.has_shared && a.I_s > a.I ? a.I_s : a.I;
  dim3 grid(rows / 2);
  // token chunks (grid.z): the fewest whose token rows fit the LDS beside the list and the
  // chunk's entry list; past kMaxChunks, tokens come from global memory in one chunk
  constexpr int kMaxChunks = 4;
  const size_t lb1 = list_bytes(a);
  const size_t lbc = (((size_t)(2 * a.E + 1 + a.T * a.k + 3 * (a.E + 1) + kGuNW + 1) * 4) + 15) & ~(size_t)15;
  int nz = 1;
  auto xb_of = [&](int n) { return (size_t)((a.T + n - 1) / n) * a.H * 2; };
  while (nz < kMaxChunks && (nz == 1 ? lb1 : lbc) + xb_of(nz) > kLdsMax) ++nz;
  const size_t lb = nz == 1 ? lb1 : lbc;
  const size_t xbytes = xb_of(nz);
  const bool xlds = lb + xbytes <= kLdsMax;
  if (!xlds) nz = 1;
  grid.z = nz;
  const size_t lds = (nz == 1 ? lb1 : lbc) + (xlds ? xbytes : 0);
  const int vpg = a.wtype == 0 ? 8 : a.wtype == 3 ? 32 : 16;
  if (vpg == 32) grid.y = 2;                  // 4-bit rows are short: two blocks per row pair
  const int groups = a.H / vpg;               // 16-byte groups per weight row
  const int cg = (groups + 15) / 16;
  if (desc) snprintf(desc, desc_len, "gemv_gate_up<vpg=%d,CG=%d,XLDS=%d> grid=%ux%ux%u block=%d lds=%zu", vpg, cg, (int)xlds, grid.x, grid.y, grid.z, kGuNW * kWave, lds);
  if (vpg == 8) {
    if (cg <= 4) return launch_gu<8, 4>(a, s, grid, xlds, lds);
    if (cg <= 8) return launch_gu<8, 8>(a, s, grid, xlds, lds);
    if (cg <= 16) return launch_gu<8, 16>(a, s, grid, xlds, lds);
    if (cg <= 32) return launch_gu<8, 32>(a, s, grid, xlds, lds);
  } else if (vpg == 16) {
    if (cg <= 4) return launch_gu<16, 4>(a, s, grid, xlds, lds);
    if (cg <= 8) return launch_gu<16, 8>(a, s, grid, xlds, lds);
    if (cg <= 16) return launch_gu<16, 16>(a, s, grid, xlds, lds);
  } else {
    if (cg <= 1) return launch_gu<32, 1>(a, s, grid, xlds, lds);
    if (cg <= 2) return launch_gu<32, 2>(a, s, grid, xlds, lds);
    if (cg <= 4) return launch_gu<32, 4>(a, s, grid, xlds, lds);
    if (cg <= 8) return launch_gu<32, 8>(a, s, grid, xlds, lds);
    if (cg <= 16) return launch_gu<32, 16>(a, s, grid, xlds, lds);
  }
  return hipErrorInvalidValue;
}

template <int VPG, int CG>
static hipError_t launch_dn(const GemvArgs &a, hipStream_t s, dim3 grid, bool hlds, size_t lds) {
  if (hlds) {
    auto k = gemv_down_kernel<VPG, CG, true>;
    hipError_t e = set_lds(reinterpret_cast<const void *>(k), lds);
    if (e != hipSuccess) return e;
    return launch_k(k, grid, dim3(kDnNW * kWave), lds, s, a);
  }
  auto k = gemv_down_kernel<VPG, CG, false>;
  hipError_t e = set_lds(reinterpret_cast<const void *>(k), lds);
  if (e != hipSuccess) return e;
  return launch_k(k, grid, dim3(kDnNW * kWave), lds, s, a);
}

hipError_t launch_gemv_down(const GemvArgs &a, hipStream_t s, char *desc, size_t desc_len) {
  dim3 grid(a.H / kDnRows);
  const size_t n_slots = (size_t)a.T * a.k;
  const size_t base = list_bytes(a) + (((n_slots * kDnRows * 4) + 15) & ~(size_t)15) +
                      ((((size_t)(a.has_shared ? a.T : 0) * kDnRows * 4) + 15) & ~(size_t)15);
  const size_t hbytes = n_slots * a.I * 2 + (a.has_shared ? (size_t)a.T * a.I_s * 2 : 0);
  const bool hlds = base + hbytes <= kLdsMax;
  const size_t lds = base + (hlds ? hbytes : 0);
  const int vpg = a.wtype == 0 ? 8 : a.wtype == 3 ? 32 : 16;
  const int kmax = a.has_shared && a.I_s > a.I ? a.I_s : a.I;
  const int groups = kmax / vpg;
  const int cg = (groups + 15) / 16;
  if (desc) snprintf(desc, desc_len, "gemv_down_combine<vpg=%d,CG=%d,HLDS=%d> grid=%u block=%d lds=%zu", vpg, cg, (int)hlds, grid.x, kDnNW * kWave, lds);
  if (vpg == 8) {
    if (cg <= 2) return launch_dn<8, 2>(a, s, grid, hlds, lds);
    if (cg <= 4) return launch_dn<8, 4>(a, s, grid, hlds, lds);
    if (cg <= 8) return launch_dn<8, 8>(a, s, grid, hlds, lds);
  } else if (vpg == 16) {
    if (cg <= 2) return launch_dn<16, 2>(a, s, grid, hlds, lds);
    if (cg <= 4) return launch_dn<16, 4>(a, s, grid, hlds, lds);
  } else {
    if (cg <= 1) return launch_dn<32, 1>(a, s, grid, hlds, lds);
    if (cg <= 2) return launch_dn<32, 2>(a, s, grid, hlds, lds);
    if (cg <= 4) return launch_dn<32, 4>(a, s, grid, hlds, lds);
  }
  return hipErrorInvalidValue;
}

// ---------------------------------------------------------------- streaming read (measurement)
// A plain read of n16 16-byte words: each thread keeps D non-temporal loads in flight, the
// blocks stride over the buffer in chunks of 256 * D words, and each block folds what it read
// into one word of sink (so no load is dropped).  Nothing of the layer uses it: it measures
// the read rate the device attains, as context for the roofline fractions of the layer kernels.
template <int D>
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4_t *__restrict__ p, size_t n16, uint32_t *sink) {
  uint32_t acc = 0;
  const size_t stride = (size_t)gridDim.x * 256 * D;
  for (size_t base = (size_t)blockIdx.x * 256 * D + threadIdx.x; base < n16; base += stride) {
    u32x4_t v[D];
#pragma unroll
    for (int u = 0; u < D; ++u) {
      const size_t i = base + (size_t)u * 256;
      v[u] = i < n16 ? __builtin_nontemporal_load(p + i) : u32x4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < D; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  __shared__ uint32_t s_acc;
  if (threadIdx.x == 0) s_acc = 0;
  __syncthreads();
  atomicXor(&s_acc, acc);
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = s_acc;
}

hipError_t launch_stream_read(const void *buf, size_t n16, int blocks, int depth, uint32_t *sink, hipStream_t s) {
  const u32x4_t *p = static_cast<const u32x4_t *>(buf);
  if (depth == 4) return launch_k(stream_read_kernel<4>, dim3(blocks), dim3(256), 0, s, p, n16, sink);
  if (depth == 8) return launch_k(stream_read_kernel<8>, dim3(blocks), dim3(256), 0, s, p, n16, sink);
  if (depth == 16) return launch_k(stream_read_kernel<16>, dim3(blocks), dim3(256), 0, s, p, n16, sink);
  return hipErrorInvalidValue;
}

}  // namespace moe
