// gemm.hip -- prefill-chunk kernels for gfx950: grouped bf16 MFMA GEMMs.
//
// veloGB10 README, "Kernel work": a prefill MoE expert kernel and an expert schedule;
// grouped expert kernels that never rebuild full weights.  At a prefill chunk every
// expert sees ~T*k/E tokens (128 at 4096 tokens, 256 experts, top-8), so the
// per-expert contraction is a real GEMM and runs on the matrix cores.
//
// Two kernel families:
//   expert_gemm_kernel (below, "expert-stationary GEMMs"): gate/up with the SiLU*up
//            epilogue and the down projection; a block owns one expert and a chunk of
//            its output columns, so every weight byte is read from HBM once.
//   grouped_gemm_kernel<ROUTER>: C[64 x 128] = A[64 x K] . B[128 x K]^T with A = x and
//            B = the fp32 router rows split exactly into three bf16 parts
//            (w = hi + mid + lo), K = 3H: fp32 logits from bf16 products.  (Its GATE_UP
//            and DOWN branches are the earlier tile-per-block form of those
//            contractions; no launch instantiates them.)
// grouped_gemm_kernel tiles: 256 threads = 4 wavefronts in 2x2, each 32 x 64 of C as
// 2 x 4 MFMA 16x16x32 bf16 tiles, fp32 accumulators.  K advances 64 per stage through
// a double LDS buffer (rows padded by 16 bytes), one barrier per stage, next stage's
// global loads in flight during the current stage's MFMAs.  Tile order: a block's
// linear id L runs on XCD L % 8; each XCD takes a contiguous range of (N-tile major,
// M-tile minor) work.
#include <cstdio>
#include <mutex>

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
      // plain (temporal) loads: the expert's other M-tiles, next to this one on the same XCD,
      // read the same weight tile from L2
      rb_reg[i] = brow[i] != nullptr ? *reinterpret_cast<const uint4 *>(brow[i] + boff + kb + 8 * lchunk)
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

// ---------------------------------------------------------------- expert-stationary GEMMs
// Gate/up and down of the prefill chunk.  A block owns one expert (or one 192-token
// chunk of the shared expert) and one chunk of its output columns, and runs every row
// of that expert through it (192 rows per pass), so each weight byte is read from HBM
// once.  The chunks of one expert are neighbours in the XCD-aware order, so the
// gathered token rows (gate/up) or h rows (down) they all read stay in that XCD's L2.
//   GATE_UP: B = 128 gate rows + the matching 128 up rows (columns n0 .. n0+127), K = H;
//            h[position][n0 ..] = bf16(silu(g) * u)
//   DOWN:    B = 256 rows of W_d (outputs n0 .. n0+255), K = I; y[slot][n0 ..] = bf16(acc)
// 512 threads = 8 wavefronts, 4 (M) x 2 (N); wavefront (wm, wn) owns the 16-row tiles
// wm, wm+4, wm+8 of the pass and 8 tiles of 16 columns: 3 x 8 MFMA 16x16x32 bf16.
// Global memory goes straight to LDS (buffer loads with the LDS target, 16 bytes per
// lane): no staging registers.  K advances 64 per stage; A has two LDS buffers, B (the
// weight stream) three.  At stage kt the loads of A(kt+1) and then B(kt+2) are issued, so
// waiting for A(kt) leaves B(kt+1) in flight (loads complete in issue order): 64 KiB of
// weights per block stay in flight.  LDS rows are 128 bytes with the 16-byte chunk c of
// row r stored at chunk c ^ (r & 7) (the loads pick their source so), spreading a
// fragment's 16 rows over the banks.  Every load is always issued: rows past the segment
// and stages past the end read zeros from an empty descriptor, so no count depends on a
// branch; each pass drains its loads before the buffers are reused.
namespace {
constexpr int EG_MR = 192;                         // rows per pass
constexpr int EG_NB = 256;                         // B rows per block
constexpr int EG_TK = 64;                          // K per stage (one 128-byte LDS row)
constexpr int EG_NT = 512;
constexpr int EG_ABUF = EG_MR * EG_TK * 2;         // bytes of one A stage (24 KiB)
constexpr int EG_BBUF = EG_NB * EG_TK * 2;         // bytes of one B stage (32 KiB)
constexpr size_t EG_LDS = (size_t)2 * EG_ABUF + 3 * EG_BBUF;  // 144 KiB
constexpr int kNtPolicy = 2;                       // non-temporal (weights are read once)
typedef __attribute__((address_space(3))) void lds_void;
}  // namespace

template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <int MODE>
__global__ __launch_bounds__(EG_NT) void expert_gemm_kernel(GemmArgs a, int NCH, int NSEG_R, int NSEG_S) {
  extern __shared__ __attribute__((aligned(16))) uint8_t eg_lds[];

  const int items = (NSEG_R + NSEG_S) * NCH;
  const int per_xcd = (items + kXcds - 1) / kXcds;
  const int u = (blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
  if (u >= items) return;
  const int seg = u / NCH, ch = u % NCH;
  const bool routed = seg < NSEG_R;
  const int n_slots = a.T * a.k;
  int row0, nrows;  // first sorted position (routed) or token (shared), rows of the segment
  if (routed) {
    row0 = a.offsets[seg];
    nrows = a.offsets[seg + 1] - row0;
  } else {
    row0 = (seg - NSEG_R) * EG_MR;
    nrows = min(EG_MR, a.T - row0);
  }
  if (nrows <= 0) return;
  const int e = routed ? seg : 0;
  const int Iseg = routed ? a.I : a.I_s;
  const int K = MODE == MODE_GATE_UP ? a.H : Iseg;
  const int n0 = MODE == MODE_GATE_UP ? ch * (EG_NB / 2) : ch * EG_NB;
  if (MODE == MODE_GATE_UP && n0 >= Iseg) return;

  const int lane = lane_id(), wave = wave_id();
  const int wm = wave & 3, wn = wave >> 2;
  // load mapping: a wavefront instruction fills 8 LDS rows (1 KiB); lane L writes row
  // L / 8, physical chunk L % 8, which holds logical chunk (L % 8) ^ (L / 8)
  const int lr = lane >> 3, lchunk = (lane & 7) ^ lr;

  // ---- B: the expert's weight rows (one scalar descriptor)
  const uint16_t *bank;
  size_t bank_bytes;
  if (MODE == MODE_GATE_UP) {
    bank = routed ? a.w_gu + (size_t)e * 2 * a.I * a.H : a.ws_gu;
    bank_bytes = (size_t)2 * Iseg * a.H * 2;
  } else {
    bank = routed ? a.w_d + (size_t)e * a.H * a.I : a.ws_d;
    bank_bytes = (size_t)a.H * Iseg * 2;
  }
  const __amdgpu_buffer_rsrc_t rB = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(bank), 0,
                                                                      (int)bank_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rNone = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(bank), 0, 0, 0x00020000);
  constexpr int kOff = 0x7FFFFF00;  // a row that reads zeros (past every descriptor)
  // this lane's source in the B row of instruction i (row group wave + 8 i); columns past
  // the segment (a partial last chunk) read zeros
  const int ncols = MODE == MODE_GATE_UP ? Iseg : a.H;
  int boff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 8 * (wave + 8 * i) + lr;
    const int col = MODE == MODE_GATE_UP ? n0 + (r % (EG_NB / 2)) : n0 + r;
    const int wr = MODE == MODE_GATE_UP ? (r < EG_NB / 2 ? col : Iseg + col) : col;
    boff[i] = col < ncols ? wr * K * 2 + lchunk * 16 : kOff;
  }
  // ---- A: token rows (gate/up) or h rows (down), gathered by the alignment
  const uint16_t *abase;
  size_t abytes;
  if (MODE == MODE_GATE_UP) {
    abase = a.x;
    abytes = (size_t)a.T * a.H * 2;
  } else if (routed) {
    abase = a.h;
    abytes = (size_t)a.cap * a.I * 2;
  } else {
    abase = a.h_s;
    abytes = (size_t)a.T * a.I_s * 2;
  }
  const __amdgpu_buffer_rsrc_t rA = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(abase), 0, (int)abytes,
                                                                      0x00020000);

  // B fragment rows of this wavefront
  int bfr[8];
#pragma unroll
  for (int ni = 0; ni < 8; ++ni) {
    if (MODE == MODE_GATE_UP) bfr[ni] = ni < 4 ? 64 * wn + 16 * ni : EG_NB / 2 + 64 * wn + 16 * (ni - 4);
    else bfr[ni] = 128 * wn + 16 * ni;
  }
  const int KT = K / EG_TK;
  const int fr = lane & 15, fq = lane >> 4;  // fragment row, quarter (8 bf16 of K)
  uint8_t *const ldsA = eg_lds;
  uint8_t *const ldsB = eg_lds + 2 * EG_ABUF;

  for (int pass0 = 0; pass0 < nrows; pass0 += EG_MR) {
    const int prow = min(EG_MR, nrows - pass0);
    int aoff[3];  // this lane's source in the A row of instruction i (row group wave + 8 i)
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      const int r = 8 * (wave + 8 * i) + lr;
      int off = kOff;
      if (r < prow) {
        const int m = row0 + pass0 + r;
        if (MODE == MODE_GATE_UP) {
          if (routed) {
            const int slot = a.sorted[m];
            if (slot < n_slots) off = (slot / a.k) * a.H * 2;
          } else {
            off = m * a.H * 2;
          }
        } else {
          off = m * Iseg * 2;
        }
      }
      aoff[i] = off == kOff ? kOff : off + lchunk * 16;
    }
    const int nmt = (prow + 15) / 16;  // 16-row tiles of the pass (zero rows past prow)
    const bool mv1 = wm + 4 < nmt, mv2 = wm + 8 < nmt;

    f32x4_t acc[3][8];
#pragma unroll
    for (int j = 0; j < 3; ++j)
#pragma unroll
      for (int ni = 0; ni < 8; ++ni) acc[j][ni] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // (kt is uniform; readfirstlane keeps the stage offset in a scalar register)
    auto issueA = [&](int kt) {
      kt = __builtin_amdgcn_readfirstlane(kt);
      const __amdgpu_buffer_rsrc_t rs = kt < KT ? rA : rNone;
      uint8_t *buf = ldsA + (kt & 1) * EG_ABUF;
#pragma unroll
      for (int i = 0; i < 3; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)(buf + (wave + 8 * i) * 1024), 16, aoff[i],
                                                 kt * EG_TK * 2, 0, 0);
    };
    auto issueB = [&](int kt) {
      kt = __builtin_amdgcn_readfirstlane(kt);
      const __amdgpu_buffer_rsrc_t rs = kt < KT ? rB : rNone;
      uint8_t *buf = ldsB + (kt % 3) * EG_BBUF;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)(buf + (wave + 8 * i) * 1024), 16, boff[i],
                                                 kt * EG_TK * 2, 0, kNtPolicy);
    };
    auto mfma_stage = [&](int kt) {
      const uint8_t *pa = ldsA + (kt & 1) * EG_ABUF;
      const uint8_t *pb = ldsB + (kt % 3) * EG_BBUF;
#pragma unroll
      for (int ks = 0; ks < EG_TK / 32; ++ks) {
        const int sw = ((ks * 4 + fq) ^ (fr & 7)) * 16;  // swizzled chunk of this lane's 8 bf16
        bf16x8_t bfm[8], af[3];
#pragma unroll
        for (int ni = 0; ni < 8; ++ni)
          bfm[ni] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4 *>(pb + (bfr[ni] + fr) * 128 + sw));
#pragma unroll
        for (int j = 0; j < 3; ++j)
          af[j] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4 *>(pa + ((wm + 4 * j) * 16 + fr) * 128 + sw));
#pragma unroll
        for (int ni = 0; ni < 8; ++ni) acc[0][ni] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[0], bfm[ni], acc[0][ni], 0, 0, 0);
        if (mv1) {
#pragma unroll
          for (int ni = 0; ni < 8; ++ni) acc[1][ni] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[1], bfm[ni], acc[1][ni], 0, 0, 0);
        }
        if (mv2) {
#pragma unroll
          for (int ni = 0; ni < 8; ++ni) acc[2][ni] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[2], bfm[ni], acc[2][ni], 0, 0, 0);
        }
      }
    };

    // in flight at the top of stage kt, in issue order: B(kt), A(kt), B(kt+1)
    issueB(0);
    issueA(0);
    issueB(1);
    for (int kt = 0; kt < KT; ++kt) {
      wait_vm<4>();      // A(kt) and all before it (B(kt)) are in LDS; B(kt+1) may not be
      // ... for every wavefront; and stage kt-1 is no longer read.  A bare barrier: the
      // explicit count above is the wait (a fenced one would drain B(kt+1) too)
      __builtin_amdgcn_s_barrier();
      issueA(kt + 1);    // into A buffer (kt+1) & 1, which held stage kt-1
      issueB(kt + 2);    // into B buffer (kt+2) % 3, which held stage kt-1
      mfma_stage(kt);
    }
    wait_vm<0>();        // the loads past the end have landed before the buffers are reused
    __syncthreads();

    // ---- epilogue: lane holds C[row = 4*(lane/16) + v][col = lane%16] of each 16x16 tile
    const int crow = 4 * (lane >> 4), ccol = lane & 15;
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      if ((j == 1 && !mv1) || (j == 2 && !mv2)) continue;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int r = (wm + 4 * j) * 16 + crow + v;  // row of the pass
        if (r >= prow) continue;
        const int m = row0 + pass0 + r;
        if (MODE == MODE_GATE_UP) {
          uint16_t *dst = routed ? a.h + (size_t)m * a.I : a.h_s + (size_t)m * a.I_s;
#pragma unroll
          for (int ni = 0; ni < 4; ++ni) {
            const int col = n0 + 64 * wn + 16 * ni + ccol;
            const float g = acc[j][ni][v], uu = acc[j][ni + 4][v];
            if (col < Iseg) dst[col] = to_bf16(g / (1.0f + expf(-g)) * uu);
          }
        } else {
          uint16_t *dst = nullptr;
          if (routed) {
            const int slot = a.sorted[m];
            if (slot < n_slots) dst = a.y + (size_t)slot * a.H;
          } else {
            dst = a.y_s + (size_t)m * a.H;
          }
          if (dst != nullptr) {
#pragma unroll
            for (int ni = 0; ni < 8; ++ni)
              if (n0 + bfr[ni] + ccol < a.H) dst[n0 + bfr[ni] + ccol] = to_bf16(acc[j][ni][v]);
          }
        }
      }
    }
  }
}

namespace {
template <int MODE>
hipError_t launch_expert_gemm(const GemmArgs &a, hipStream_t s) {
  auto kern = expert_gemm_kernel<MODE>;
  static std::mutex mu;
  static bool opened[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  {
    std::lock_guard<std::mutex> lock(mu);
    if (!opened[dev]) {
      e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)EG_LDS);
      if (e != hipSuccess) return e;
      opened[dev] = true;
    }
  }
  // the kernel addresses tokens, h and one expert's matrix through 32-bit buffer ranges
  const int imax = a.has_shared && a.I_s > a.I ? a.I_s : a.I;
  const size_t lim = (size_t)1 << 31;
  if ((size_t)a.T * a.H * 2 >= lim || (size_t)a.cap * a.I * 2 >= lim || (size_t)2 * imax * a.H * 2 >= lim)
    return hipErrorInvalidValue;
  if (a.H % EG_TK != 0 || a.I % EG_TK != 0 || (a.has_shared && a.I_s % EG_TK != 0)) return hipErrorInvalidValue;
  const int NCH = MODE == MODE_GATE_UP ? (imax + EG_NB / 2 - 1) / (EG_NB / 2) : (a.H + EG_NB - 1) / EG_NB;
  const int NSEG_S = a.has_shared ? (a.T + EG_MR - 1) / EG_MR : 0;
  return launch_k(kern, dim3(grid_for((a.E + NSEG_S) * NCH)), dim3(EG_NT), EG_LDS, s, a, NCH, a.E, NSEG_S);
}
}  // namespace

hipError_t launch_gemm_gate_up(const GemmArgs &a, hipStream_t s) { return launch_expert_gemm<MODE_GATE_UP>(a, s); }

hipError_t launch_gemm_down(const GemmArgs &a, hipStream_t s) { return launch_expert_gemm<MODE_DOWN>(a, s); }

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
  return launch_k(router_split_kernel, dim3(512), dim3(256), 0, s, w_r, w_sg, E, H, w3);
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
  return launch_k(grouped_gemm_kernel<MODE_ROUTER>, dim3(grid_for(MT * NN)), dim3(NTHR), 0, s, a, ra, MT, 0, NN);
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
  return launch_k(combine_kernel, dim3(T), dim3(256), 0, s, y, y_s, topk_w, gamma, T, H, k, out);
  return hipGetLastError();
}

}  // namespace moe
