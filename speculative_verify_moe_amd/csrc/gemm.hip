// gemm.hip -- prefill-chunk kernels for gfx950: grouped bf16 MFMA GEMMs.
//
// veloGB10 README, "Kernel work": a prefill MoE expert kernel and an expert schedule;
// grouped expert kernels that never rebuild full weights.  At a prefill chunk every
// expert sees ~T*k/E tokens (128 at 4096 tokens, 256 experts, top-8), so the
// per-expert contraction is a real GEMM and runs on the matrix cores.
//
// One kernel template covers three contractions C[64 x 128] = A[64 x K] . B[128 x K]^T:
//   GATE_UP  A = x rows gathered through the alignment (a 64-row M-tile is one BM=64
//            block, so it belongs to one expert), B = 64 gate rows + the matching 64
//            up rows of that expert; epilogue h = bf16(silu(g) * u), stored by
//            sorted position.  The shared expert is one more segment of M-tiles over
//            the T tokens in order.
//   DOWN     A = h rows (sorted position), B = 128 rows of W_d; epilogue y = bf16(acc)
//            stored by slot (t*k + j), so the combine reads a token's k rows together.
//   ROUTER   A = x, B = the fp32 router rows split exactly into three bf16 parts
//            (w = hi + mid + lo), K = 3H: fp32 logits from bf16 products.
// Tiles: 256 threads = 4 wavefronts in 2x2, each 32 x 64 of C as 2 x 4 MFMA
// 16x16x32 bf16 tiles, fp32 accumulators.  K advances 64 per stage through a double
// LDS buffer (rows padded by 16 bytes), one barrier per stage, next stage's global
// loads in flight during the current stage's MFMAs.
// Tile order: a block's linear id L runs on XCD L % 8; each XCD takes a contiguous
// range of (N-tile major, M-tile minor) work, so the M-tiles of one expert run next
// to each other on one XCD and share its L2 copy of the expert's weight tile.
#include <cstdio>

#include "device.h"
#include "internal.h"

namespace moe {

namespace {
constexpr int TM = 64;          // tile rows (== prefill BM)
constexpr int TN = 128;         // tile B rows
constexpr int TK = 64;          // K per LDS stage
constexpr int LDSW = TK + 8;    // bf16 per LDS row
constexpr int NTHR = 256;
constexpr int kXcds = 8;
enum { MODE_GATE_UP = 0, MODE_DOWN = 1, MODE_ROUTER = 2 };

struct RouterArgs {
  const float *b_r;
  float *logits;
  float *gate_logit;
  int E, NRt;  // experts, B rows in total (E + shared gate row)
};
}  // namespace

template <int MODE>
__global__ __launch_bounds__(NTHR, 2) void grouped_gemm_kernel(GemmArgs a, RouterArgs ra, int MT_r, int MT_s,
                                                               int NN) {
  __shared__ __attribute__((aligned(16))) uint16_t sA[2][TM * LDSW];
  __shared__ __attribute__((aligned(16))) uint16_t sB[2][TN * LDSW];

  const int MT = MT_r + MT_s;
  const int ntiles = MT * NN;
  const int per_xcd = (ntiles + kXcds - 1) / kXcds;
  const int u = (blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
  if (u >= ntiles) return;
  const int mtile = u % MT, ntile = u / MT;
  const bool routed = mtile < MT_r;
  const int n_slots = a.T * a.k;

  // ---- segment: expert, K, B base, row counts
  int e = 0, K = 0, Iseg = 0;
  if (MODE == MODE_ROUTER) {
    K = 3 * a.H;
  } else if (routed) {
    e = a.block_expert[(mtile * TM) / a.BM];  // BM is 64 or 128: one expert per tile
    if (e < 0) return;  // past the padded total
    Iseg = a.I;
    K = MODE == MODE_GATE_UP ? a.H : a.I;
  } else {
    Iseg = a.I_s;
    K = MODE == MODE_GATE_UP ? a.H : a.I_s;
  }
  const int n0 = MODE == MODE_GATE_UP ? ntile * (TN / 2) : ntile * TN;
  if (MODE == MODE_GATE_UP && n0 >= Iseg) return;
  const int m0 = routed ? mtile * TM : (mtile - MT_r) * TM;  // sorted position or token

  const int tid = threadIdx.x;
  const int lane = lane_id(), wave = wave_id();
  const int wm = wave & 1, wn = wave >> 1;

  // ---- per-thread global row pointers: A rows tid/8 and 32 + tid/8, B rows tid/8 + 32i
  const int lrow = tid >> 3, lchunk = tid & 7;
  const uint16_t *arow[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = lrow + 32 * i;
    const uint16_t *p = nullptr;
    if (MODE == MODE_GATE_UP) {
      if (routed) {
        const int slot = a.sorted[m0 + r];
        if (slot < n_slots) p = a.x + (size_t)(slot / a.k) * a.H;
      } else if (m0 + r < a.T) {
        p = a.x + (size_t)(m0 + r) * a.H;
      }
    } else if (MODE == MODE_DOWN) {
      if (routed) p = a.h + (size_t)(m0 + r) * a.I;
      else if (m0 + r < a.T) p = a.h_s + (size_t)(m0 + r) * a.I_s;
    } else {
      if (m0 + r < a.T) p = a.x + (size_t)(m0 + r) * a.H;
    }
    arow[i] = p;
  }
  const uint16_t *brow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = lrow + 32 * i;
    const uint16_t *p = nullptr;
    if (MODE == MODE_GATE_UP) {
      const uint16_t *bank = routed ? a.w_gu + (size_t)e * 2 * a.I * a.H : a.ws_gu;
      const int wr = r < TN / 2 ? n0 + r : Iseg + n0 + (r - TN / 2);
      p = bank + (size_t)wr * a.H;
    } else if (MODE == MODE_DOWN) {
      const uint16_t *bank = routed ? a.w_d + (size_t)e * a.H * a.I : a.ws_d;
      p = bank + (size_t)(n0 + r) * Iseg;
    } else {
      if (n0 + r < ra.NRt) p = a.w_gu + (size_t)(n0 + r) * a.H;  // w3 passed in w_gu
    }
    brow[i] = p;
  }

  const int KT = K / TK;
  uint4 ra_reg[2], rb_reg[4];
  auto gload = [&](int kt) {
    int ka = kt * TK, kb = kt * TK;
    size_t boff = 0;
    if (MODE == MODE_ROUTER) {
      const int per = a.H / TK;
      ka = (kt % per) * TK;
      kb = ka;
      boff = (size_t)(kt / per) * ra.NRt * a.H;
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
      ra_reg[i] = arow[i] != nullptr ? *reinterpret_cast<const uint4 *>(arow[i] + ka + 8 * lchunk)
                                     : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      rb_reg[i] = brow[i] != nullptr ? ld_stream(reinterpret_cast<const uint4 *>(brow[i] + boff + kb + 8 * lchunk))
                                     : make_uint4(0, 0, 0, 0);
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
      *reinterpret_cast<uint4 *>(&sA[buf][(lrow + 32 * i) * LDSW + 8 * lchunk]) = ra_reg[i];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<uint4 *>(&sB[buf][(lrow + 32 * i) * LDSW + 8 * lchunk]) = rb_reg[i];
  };

  // B fragment rows of this wavefront
  int bfr[4];
#pragma unroll
  for (int ni = 0; ni < 4; ++ni) {
    if (MODE == MODE_GATE_UP) bfr[ni] = ni < 2 ? 32 * wn + 16 * ni : TN / 2 + 32 * wn + 16 * (ni - 2);
    else bfr[ni] = 64 * wn + 16 * ni;
  }

  f32x4_t acc[2][4];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  gload(0);
  sstore(0);
  __syncthreads();
  const int fr = lane & 15, fk = 8 * (lane >> 4);
  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < KT) gload(kt + 1);
#pragma unroll
    for (int ks = 0; ks < TK / 32; ++ks) {
      bf16x8_t af[2], bfm[4];
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
        af[mi] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4 *>(
                                                  &sA[buf][(32 * wm + 16 * mi + fr) * LDSW + ks * 32 + fk]));
#pragma unroll
      for (int ni = 0; ni < 4; ++ni)
        bfm[ni] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4 *>(
                                                   &sB[buf][(bfr[ni] + fr) * LDSW + ks * 32 + fk]));
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 4; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[mi], bfm[ni], acc[mi][ni], 0, 0, 0);
    }
    if (kt + 1 < KT) sstore(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: lane holds C[row = 4*(lane/16) + v][col = lane%16] of each 16x16 tile
  const int crow = 4 * (lane >> 4), ccol = lane & 15;
#pragma unroll
  for (int mi = 0; mi < 2; ++mi) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int row = 32 * wm + 16 * mi + crow + v;
      if (MODE == MODE_GATE_UP) {
        uint16_t *dst;
        if (routed) dst = a.h + (size_t)(m0 + row) * a.I;
        else dst = (m0 + row < a.T) ? a.h_s + (size_t)(m0 + row) * a.I_s : nullptr;
        if (dst != nullptr) {
#pragma unroll
          for (int ni = 0; ni < 2; ++ni) {
            const float g = acc[mi][ni][v], uu = acc[mi][ni + 2][v];
            dst[n0 + 32 * wn + 16 * ni + ccol] = to_bf16(g / (1.0f + expf(-g)) * uu);
          }
        }
      } else if (MODE == MODE_DOWN) {
        uint16_t *dst = nullptr;
        if (routed) {
          const int slot = a.sorted[m0 + row];
          if (slot < n_slots) dst = a.y + (size_t)slot * a.H;
        } else if (m0 + row < a.T) {
          dst = a.y_s + (size_t)(m0 + row) * a.H;
        }
        if (dst != nullptr) {
#pragma unroll
          for (int ni = 0; ni < 4; ++ni) dst[n0 + bfr[ni] + ccol] = to_bf16(acc[mi][ni][v]);
        }
      } else {
        const int t = m0 + row;
        if (t < a.T) {
#pragma unroll
          for (int ni = 0; ni < 4; ++ni) {
            const int ex = n0 + bfr[ni] + ccol;
            if (ex < ra.E) ra.logits[(size_t)t * ra.E + ex] = acc[mi][ni][v] + (ra.b_r ? ra.b_r[ex] : 0.0f);
            else if (ex < ra.NRt) ra.gate_logit[t] = acc[mi][ni][v];
          }
        }
      }
    }
  }
}

static unsigned grid_for(int tiles) { return (unsigned)(((tiles + kXcds - 1) / kXcds) * kXcds); }

hipError_t launch_gemm_gate_up(const GemmArgs &a, hipStream_t s) {
  const int MT_r = (int)(a.cap / TM);
  const int MT_s = a.has_shared ? (a.T + TM - 1) / TM : 0;
  const int imax = a.has_shared && a.I_s > a.I ? a.I_s : a.I;
  const int NN = imax / (TN / 2);
  RouterArgs ra{};
  launch_k(grouped_gemm_kernel<MODE_GATE_UP>, dim3(grid_for((MT_r + MT_s) * NN)), dim3(NTHR), 0, s, a, ra,
                     MT_r, MT_s, NN);
  return hipGetLastError();
}

hipError_t launch_gemm_down(const GemmArgs &a, hipStream_t s) {
  const int MT_r = (int)(a.cap / TM);
  const int MT_s = a.has_shared ? (a.T + TM - 1) / TM : 0;
  const int NN = a.H / TN;
  RouterArgs ra{};
  launch_k(grouped_gemm_kernel<MODE_DOWN>, dim3(grid_for((MT_r + MT_s) * NN)), dim3(NTHR), 0, s, a, ra,
                     MT_r, MT_s, NN);
  return hipGetLastError();
}

// ---------------------------------------------------------------- router on MFMA
// Exact three-way split of each fp32 router weight into bf16 parts: hi = rne(w),
// mid = rne(w - hi), lo = rne(w - hi - mid); each difference is exact in fp32 and
// hi + mid + lo == w.  Row E (when present) is the shared expert's gate vector.
__global__ __launch_bounds__(256) void router_split_kernel(const float *__restrict__ w_r,
                                                           const float *__restrict__ w_sg, int E, int H,
                                                           uint16_t *__restrict__ w3) {
  const int NRt = E + (w_sg != nullptr ? 1 : 0);
  const size_t total = (size_t)NRt * H;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (size_t)gridDim.x * blockDim.x) {
    const int n = (int)(i / H), hh = (int)(i % H);
    const float w = n < E ? w_r[(size_t)n * H + hh] : w_sg[hh];
    const float hi = round_bf16(w);
    const float r1 = w - hi;
    const float mid = round_bf16(r1);
    const float lo = round_bf16(r1 - mid);
    w3[i] = to_bf16(hi);
    w3[total + i] = to_bf16(mid);
    w3[2 * total + i] = to_bf16(lo);
  }
}

hipError_t launch_router_split(const float *w_r, const float *w_sg, int E, int H, uint16_t *w3, hipStream_t s) {
  launch_k(router_split_kernel, dim3(512), dim3(256), 0, s, w_r, w_sg, E, H, w3);
  return hipGetLastError();
}

hipError_t launch_router_gemm(const uint16_t *x, int T, int H, const uint16_t *w3, int E, int has_sg,
                              const float *b_r, float *logits, float *gate_logit, hipStream_t s) {
  GemmArgs a{};
  a.x = x;
  a.T = T;
  a.H = H;
  a.w_gu = w3;
  RouterArgs ra{b_r, logits, gate_logit, E, E + (has_sg ? 1 : 0)};
  const int MT = (T + TM - 1) / TM;
  const int NN = (ra.NRt + TN - 1) / TN;
  launch_k(grouped_gemm_kernel<MODE_ROUTER>, dim3(grid_for(MT * NN)), dim3(NTHR), 0, s, a, ra, MT, 0, NN);
  return hipGetLastError();
}

// ---------------------------------------------------------------- combine (prefill)
// out[t] = bf16(sum_{j<k} w[t][j] * y[t*k+j] + gamma_t * y_s[t]) in slot order, fp32.
__global__ __launch_bounds__(256) void combine_kernel(const uint16_t *__restrict__ y, const uint16_t *__restrict__ y_s,
                                                      const float *__restrict__ topk_w,
                                                      const float *__restrict__ gamma, int T, int H, int k,
                                                      uint16_t *__restrict__ out) {
  const int t = blockIdx.x;
  const int G8 = H / 8;
  for (int g = threadIdx.x; g < G8; g += blockDim.x) {
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
    for (int j = 0; j < k; ++j) {
      const float w = topk_w[(size_t)t * k + j];
      const uint4 v = reinterpret_cast<const uint4 *>(y + ((size_t)t * k + j) * H)[g];
      acc[0] = fmaf(w, bf16_lo(v.x), acc[0]);
      acc[1] = fmaf(w, bf16_hi(v.x), acc[1]);
      acc[2] = fmaf(w, bf16_lo(v.y), acc[2]);
      acc[3] = fmaf(w, bf16_hi(v.y), acc[3]);
      acc[4] = fmaf(w, bf16_lo(v.z), acc[4]);
      acc[5] = fmaf(w, bf16_hi(v.z), acc[5]);
      acc[6] = fmaf(w, bf16_lo(v.w), acc[6]);
      acc[7] = fmaf(w, bf16_hi(v.w), acc[7]);
    }
    if (y_s != nullptr) {
      const float gm = gamma[t];
      const uint4 v = reinterpret_cast<const uint4 *>(y_s + (size_t)t * H)[g];
      acc[0] = fmaf(gm, bf16_lo(v.x), acc[0]);
      acc[1] = fmaf(gm, bf16_hi(v.x), acc[1]);
      acc[2] = fmaf(gm, bf16_lo(v.y), acc[2]);
      acc[3] = fmaf(gm, bf16_hi(v.y), acc[3]);
      acc[4] = fmaf(gm, bf16_lo(v.z), acc[4]);
      acc[5] = fmaf(gm, bf16_hi(v.z), acc[5]);
      acc[6] = fmaf(gm, bf16_lo(v.w), acc[6]);
      acc[7] = fmaf(gm, bf16_hi(v.w), acc[7]);
    }
    uint4 o;
    o.x = pack_bf16x2(acc[0], acc[1]);
    o.y = pack_bf16x2(acc[2], acc[3]);
    o.z = pack_bf16x2(acc[4], acc[5]);
    o.w = pack_bf16x2(acc[6], acc[7]);
    reinterpret_cast<uint4 *>(out + (size_t)t * H)[g] = o;
  }
}

hipError_t launch_combine(const uint16_t *y, const uint16_t *y_s, const float *topk_w, const float *gamma, int T,
                          int H, int k, uint16_t *out, hipStream_t s) {
  launch_k(combine_kernel, dim3(T), dim3(256), 0, s, y, y_s, topk_w, gamma, T, H, k, out);
  return hipGetLastError();
}

}  // namespace moe
