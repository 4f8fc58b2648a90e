// gemm.hip -- prefill-chunk kernels for gfx950: grouped bf16 MFMA GEMMs.
//
// veloGB10 README, "Kernel work": a prefill MoE expert kernel and an expert schedule;
// grouped expert kernels that never rebuild full weights.  At a prefill chunk every
// expert sees ~T*k/E tokens (128 at 4096 tokens, 256 experts, top-8), so the
// per-expert contraction is a real GEMM and runs on the matrix cores.
//
// Kernels:
//   expert_gemm_kernel ("expert-stationary GEMMs" below): gate/up with the SiLU*up
//            epilogue and the down projection; a block owns one expert and a chunk of
//            its output columns, so every weight byte is read from HBM once.
//   router_mfma_kernel: the fp32 router logits on the matrix cores from an exact
//            three-way bf16 split of the weights, made while each tile is staged.
//   combine_kernel: the weighted sum of each token's expert outputs in slot order.
#include <cstdio>
#include <mutex>

#include "device.h"
#include "internal.h"

namespace moe {

namespace {
constexpr int kXcds = 8;
enum { MODE_GATE_UP = 0, MODE_DOWN = 1 };
// operand kinds of the expert GEMMs: bf16 weights and activations; fp8 weights widened to
// bf16 in LDS; fp8 weights and fp8 activations (one scale per activation row) on the fp8
// matrix cores
enum { KIND_BF16 = 0, KIND_FP8W = 1, KIND_A8 = 2 };
typedef int i32x8_t __attribute__((ext_vector_type(8)));
}  // namespace

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
constexpr size_t EG_LDS = (size_t)2 * EG_ABUF + 3 * EG_BBUF;  // 144 KiB (bf16 weights)
// fp8 weights: two A stages, two widened bf16 B stages, three stages of codes (160 KiB)
constexpr size_t EG_LDS_FP8 = (size_t)2 * EG_ABUF + 2 * EG_BBUF + 3 * (EG_NB * EG_TK);
constexpr int kNtPolicy = 2;                       // non-temporal (weights are read once)
typedef __attribute__((address_space(3))) void lds_void;
}  // namespace

template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// KIND_FP8W: fp8 e4m3 weight codes with one fp32 scale per weight row.  The stages arrive
// as codes in LDS (64 bytes per row and stage, 16 rows per wavefront instruction, 16-byte
// chunk c of row r at chunk c ^ ((r / 4) & 3)), three stages ahead; during each stage the
// block widens the next one exactly to bf16 into a two-stage bf16 buffer (each code once,
// not once per reading wavefront), so the MFMA loop is the bf16 one; the row scales
// multiply the finished sums.
// KIND_A8: fp8 weights and fp8 activation rows (tokens, or h), each activation row with its
// own fp32 scale.  A stage is 128 codes of K: 128 bytes per row for both operands, the bf16
// layout byte for byte, and one 16x16x128 fp8 MFMA per tile and stage; the weight-row scale
// and the activation-row scale multiply the finished sums.
// SHONLY (1: launches of the shared expert's segments alone) changes no code; it gives those
// launches a kernel name of their own, so that profiles tell them from the routed ones.
template <int MODE, int KIND, int SHONLY>
__global__ __launch_bounds__(EG_NT) void expert_gemm_kernel(GemmArgs a, int NCH, int NSEG_R, int NSEG_S) {
  extern __shared__ __attribute__((aligned(16))) uint8_t eg_lds[];
  __shared__ float s_rsc[KIND == KIND_A8 ? EG_MR : 1];  // KIND_A8: activation scale of each row
  // down: slot of each row (KIND_FP8W uses all 160 KiB of LDS and keeps them in registers)
  __shared__ int s_slot[MODE == MODE_DOWN && KIND != KIND_FP8W ? EG_MR : 1];
  constexpr int ESZ = KIND == KIND_BF16 ? 2 : 1;   // bytes per weight
  constexpr int AESZ = KIND == KIND_A8 ? 1 : 2;    // bytes per activation
  constexpr int TKE = KIND == KIND_A8 ? 128 : EG_TK;  // K per stage
  constexpr int BRB = TKE * ESZ;         // bytes of one B row in one stage
  constexpr int RPI = 1024 / BRB;        // B rows per wavefront instruction
  constexpr int CPR = BRB / 16;          // 16-byte chunks per B row
  constexpr int NBI = EG_NB / RPI / 8;   // B instructions per wavefront and stage
  constexpr int QBUF = EG_NB * BRB;      // bytes of one staged B stage (bf16, or fp8 codes)

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
    // the rows past the count up to the next offset are padding (and the count never
    // reaches past the expert's padded range)
    nrows = min(a.counts[seg], a.offsets[seg + 1] - row0);
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
  // wavefronts w and w + 4 share a SIMD: giving them different M rows (wm = w / 2)
  // spreads a pass with a ragged tile count evenly over the SIMDs
  const int wm = wave >> 1, wn = wave & 1;
  // load mapping: a wavefront instruction fills 8 LDS rows (1 KiB); lane L writes row
  // L / 8, physical chunk L % 8, which holds logical chunk (L % 8) ^ (L / 8)
  // KIND_A8: a lane's fragment is two logical chunks, 2q and 2q + 1; the logical chunk c sits
  // at physical chunk tau(c) ^ (r & 7), tau(c) = (c >> 1) | ((c & 1) << 2), so that its two
  // reads fall on the physical chunks q ^ (r & 7) and (q + 4) ^ (r & 7), the bf16 pattern,
  // which the LDS serves without bank conflicts (2q ^ (r & 7) conflicted on half the cycles)
  const int lr = lane >> 3, lphys = (lane & 7) ^ lr;
  const int lchunk = KIND == KIND_A8 ? ((lphys & 3) << 1) | (lphys >> 2) : lphys;

  // ---- B: the expert's weight rows (one scalar descriptor)
  const uint8_t *bank;
  size_t bank_bytes;
  const float *scale = nullptr;  // fp8: the row scales of this matrix
  if (MODE == MODE_GATE_UP) {
    bank = routed ? (const uint8_t *)a.w_gu + (size_t)e * 2 * a.I * a.H * ESZ : (const uint8_t *)a.ws_gu;
    bank_bytes = (size_t)2 * Iseg * a.H * ESZ;
    if (ESZ == 1) scale = routed ? a.s_gu + (size_t)e * 2 * a.I : a.ss_gu;
  } else {
    bank = routed ? (const uint8_t *)a.w_d + (size_t)e * a.H * a.I * ESZ : (const uint8_t *)a.ws_d;
    bank_bytes = (size_t)a.H * Iseg * ESZ;
    if (ESZ == 1) scale = routed ? a.s_d + (size_t)e * a.H : a.ss_d;
  }
  const __amdgpu_buffer_rsrc_t rB = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(bank), 0,
                                                                      (int)bank_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rNone = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(bank), 0, 0, 0x00020000);
  constexpr int kOff = 0x7FFFFF00;  // a row that reads zeros (past every descriptor)
  // this lane's source in the B row of instruction i (row group wave + 8 i); columns past
  // the segment (a partial last chunk) read zeros
  const int ncols = MODE == MODE_GATE_UP ? Iseg : a.H;
  const int blr = lane / CPR;  // row of the instruction's group, physical chunk lane % CPR
  const int bch = BRB == 128 ? lchunk : (lane & 3) ^ ((blr >> 2) & 3);
  int boff[4];  // NBI used (a template-dependent array size here leaves the host stub unemitted)
#pragma unroll
  for (int i = 0; i < NBI; ++i) {
    const int r = RPI * (wave + 8 * i) + blr;
    const int col = MODE == MODE_GATE_UP ? n0 + (r % (EG_NB / 2)) : n0 + r;
    const int wr = MODE == MODE_GATE_UP ? (r < EG_NB / 2 ? col : Iseg + col) : col;
    boff[i] = col < ncols ? wr * K * ESZ + bch * 16 : kOff;
  }
  // ---- A: token rows (gate/up) or h rows (down), gathered by the alignment (bf16, or
  // fp8 codes for KIND_A8)
  const uint8_t *abase;
  size_t abytes;
  if (MODE == MODE_GATE_UP) {
    abase = KIND == KIND_A8 ? a.x8 : (const uint8_t *)a.x;
    abytes = (size_t)a.T * a.H * AESZ;
  } else if (routed) {
    abase = KIND == KIND_A8 ? a.h8 : (const uint8_t *)a.h;
    abytes = (size_t)a.cap * a.I * AESZ;
  } else {
    abase = KIND == KIND_A8 ? a.hs8 : (const uint8_t *)a.h_s;
    abytes = (size_t)a.T * a.I_s * AESZ;
  }
  const __amdgpu_buffer_rsrc_t rA = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(abase), 0, (int)abytes,
                                                                      0x00020000);

  // B fragment rows of this wavefront
  int bfr[8];
#pragma unroll
  for (int ni = 0; ni < 8; ++ni) {
    if (MODE == MODE_GATE_UP) bfr[ni] = ni < 4 ? 64 * wn + 16 * ni : EG_NB / 2 + 64 * wn + 16 * (ni - 4);
    else bfr[ni] = 128 * wn + 16 * ni;
  }
  const int KT = K / TKE;
  const int fr = lane & 15, fq = lane >> 4;  // fragment row, quarter (8 bf16 of K)
  // epilogue: lane holds C[row = 4*(lane/16) + v][col = lane%16] of each 16x16 tile
  const int crow = 4 * (lane >> 4), ccol = lane & 15;
  // fp8: the row scales of this lane's output columns, loaded once before the first stage
  // (columns past the segment take the last row's scale and are never stored)
  float sc[8];
#pragma unroll
  for (int ni = 0; ni < 8; ++ni) sc[ni] = 1.0f;
  if (ESZ == 1) {
#pragma unroll
    for (int ni = 0; ni < 8; ++ni) {
      if (MODE == MODE_GATE_UP) {
        const int col = min(n0 + 64 * wn + 16 * (ni & 3) + ccol, Iseg - 1);
        sc[ni] = scale[ni < 4 ? col : Iseg + col];
      } else {
        sc[ni] = scale[min(n0 + bfr[ni] + ccol, a.H - 1)];
      }
    }
  }
  uint8_t *const ldsA = eg_lds;
  uint8_t *const ldsB = eg_lds + 2 * EG_ABUF;  // bf16 B stages: three (bf16) or two (fp8)
  uint8_t *const ldsQ = eg_lds + 2 * EG_ABUF + 2 * EG_BBUF;  // fp8: three stages of codes

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
            if (slot < n_slots) off = (slot / a.k) * a.H * AESZ;
          } else {
            off = m * a.H * AESZ;
          }
        } else {
          off = m * Iseg * AESZ;
        }
      }
      aoff[i] = off == kOff ? kOff : off + lchunk * 16;
    }
    // per row of the pass, read into LDS before the first stage (after the previous pass's
    // epilogue has read them): down, the slot of the row; KIND_A8, the activation scale (a
    // token's, or an h row's)
    int oslot[3][4];  // KIND_FP8W, down: the slot of each of this lane's output rows
    if (MODE == MODE_DOWN && KIND == KIND_FP8W) {
#pragma unroll
      for (int j = 0; j < 3; ++j)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          oslot[j][v] = routed ? a.sorted[row0 + pass0 + min((wm + 4 * j) * 16 + crow + v, prow - 1)] : 0;
    }
    if ((MODE == MODE_DOWN && KIND != KIND_FP8W) || KIND == KIND_A8) {
      if (pass0 > 0) __syncthreads();
      const int t = threadIdx.x;
      if (t < prow) {
        const int m = row0 + pass0 + t;
        if (MODE == MODE_DOWN && KIND != KIND_FP8W) s_slot[t] = routed ? a.sorted[m] : 0;
        if (KIND == KIND_A8) {
          if (MODE == MODE_GATE_UP) s_rsc[t] = routed ? a.sx[min(a.sorted[m], n_slots - 1) / a.k] : a.sx[m];
          else s_rsc[t] = routed ? a.sh[m] : a.shs[m];
        }
      }
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
                                                 kt * TKE * AESZ, 0, 0);
    };
    auto issueB = [&](int kt) {
      kt = __builtin_amdgcn_readfirstlane(kt);
      const __amdgpu_buffer_rsrc_t rs = kt < KT ? rB : rNone;
      uint8_t *buf = (KIND == KIND_FP8W ? ldsQ : ldsB) + (kt % 3) * QBUF;
#pragma unroll
      for (int i = 0; i < NBI; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)(buf + (wave + 8 * i) * 1024), 16, boff[i],
                                                 kt * BRB, 0, kNtPolicy);
    };
    auto mfma_stage = [&](int kt) {
      const uint8_t *pa = ldsA + (kt & 1) * EG_ABUF;
      const uint8_t *pb = ldsB + (KIND == KIND_FP8W ? kt & 1 : kt % 3) * EG_BBUF;
      if (KIND == KIND_A8) {
        // lane (fr, fq) holds the 32 codes of K 32 fq .. 32 fq + 31 of its row (logical
        // chunks 2 fq and 2 fq + 1), for the activation and the weight fragments alike.  The
        // fragment reads are inline asm: the compiler cannot tell them from the direct-to-LDS
        // loads still in flight into the other buffers and would otherwise wait for every one
        // of them (vmcnt 0) before the first read, draining the load queue every stage.  Each
        // block of reads waits for its own results before it ends (an asm output counts as
        // written when the block ends), and its outputs are early-clobber (no read may land in
        // a register that a later read of the block takes its address from).
        const int c0 = (fq ^ (fr & 7)) * 16, c1 = ((fq + 4) ^ (fr & 7)) * 16;
        auto addr = [&](const uint8_t *row, int c) { return (uint32_t)(uintptr_t)(row + c); };
        auto join = [](const u32x4_t &lo, const u32x4_t &hi) {
          return i32x8_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        };
        const uint8_t *ra[3], *rb[8];
#pragma unroll
        for (int j = 0; j < 3; ++j) ra[j] = pa + ((wm + 4 * j) * 16 + fr) * 128;
#pragma unroll
        for (int ni = 0; ni < 8; ++ni) rb[ni] = pb + (bfr[ni] + fr) * 128;
        u32x4_t al[3], ah[3], bl[8], bh[8];
        asm volatile(
            "ds_read_b128 %0, %14\n\tds_read_b128 %1, %15\n\tds_read_b128 %2, %16\n\t"
            "ds_read_b128 %3, %17\n\tds_read_b128 %4, %18\n\tds_read_b128 %5, %19\n\t"
            "ds_read_b128 %6, %20\n\tds_read_b128 %7, %21\n\tds_read_b128 %8, %22\n\t"
            "ds_read_b128 %9, %23\n\tds_read_b128 %10, %24\n\tds_read_b128 %11, %25\n\t"
            "ds_read_b128 %12, %26\n\tds_read_b128 %13, %27\n\ts_waitcnt lgkmcnt(0)"
            : "=&v"(al[0]), "=&v"(ah[0]), "=&v"(al[1]), "=&v"(ah[1]), "=&v"(al[2]), "=&v"(ah[2]), "=&v"(bl[0]),
              "=&v"(bh[0]), "=&v"(bl[1]), "=&v"(bh[1]), "=&v"(bl[2]), "=&v"(bh[2]), "=&v"(bl[3]), "=&v"(bh[3])
            : "v"(addr(ra[0], c0)), "v"(addr(ra[0], c1)), "v"(addr(ra[1], c0)), "v"(addr(ra[1], c1)),
              "v"(addr(ra[2], c0)), "v"(addr(ra[2], c1)), "v"(addr(rb[0], c0)), "v"(addr(rb[0], c1)),
              "v"(addr(rb[1], c0)), "v"(addr(rb[1], c1)), "v"(addr(rb[2], c0)), "v"(addr(rb[2], c1)),
              "v"(addr(rb[3], c0)), "v"(addr(rb[3], c1))
            : "memory");
        asm volatile(
            "ds_read_b128 %0, %8\n\tds_read_b128 %1, %9\n\tds_read_b128 %2, %10\n\t"
            "ds_read_b128 %3, %11\n\tds_read_b128 %4, %12\n\tds_read_b128 %5, %13\n\t"
            "ds_read_b128 %6, %14\n\tds_read_b128 %7, %15\n\ts_waitcnt lgkmcnt(0)"
            : "=&v"(bl[4]), "=&v"(bh[4]), "=&v"(bl[5]), "=&v"(bh[5]), "=&v"(bl[6]), "=&v"(bh[6]), "=&v"(bl[7]),
              "=&v"(bh[7])
            : "v"(addr(rb[4], c0)), "v"(addr(rb[4], c1)), "v"(addr(rb[5], c0)), "v"(addr(rb[5], c1)),
              "v"(addr(rb[6], c0)), "v"(addr(rb[6], c1)), "v"(addr(rb[7], c0)), "v"(addr(rb[7], c1))
            : "memory");
        i32x8_t aq[3];
#pragma unroll
        for (int j = 0; j < 3; ++j) aq[j] = join(al[j], ah[j]);
        // operand formats 0 (e4m3) for both; block scales 127 (2^0): plain products
        auto mfma_ni = [&](int ni) {
          const i32x8_t bq = join(bl[ni], bh[ni]);
          acc[0][ni] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aq[0], bq, acc[0][ni], 0, 0, 0, 127, 0, 127);
          if (mv1)
            acc[1][ni] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aq[1], bq, acc[1][ni], 0, 0, 0, 127, 0, 127);
          if (mv2)
            acc[2][ni] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aq[2], bq, acc[2][ni], 0, 0, 0, 127, 0, 127);
        };
#pragma unroll
        for (int ni = 0; ni < 8; ++ni) mfma_ni(ni);
        return;
      }
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

    // fp8: thread t widens half a row of codes (row t / 2, 32 codes) of stage kt into the
    // bf16 buffer kt & 1
    auto widen = [&](int kt) {
      const int r = threadIdx.x >> 1, hf = threadIdx.x & 1;
      const uint8_t *q = ldsQ + (kt % 3) * QBUF + r * 64;
      uint8_t *b = ldsB + (kt & 1) * EG_BBUF + r * 128;
      // the code reads are hidden from the compiler's LDS tracking: it cannot tell them from
      // the DMA writes into the other two code stages and would wait for every load in
      // flight (vmcnt 0); the stage read here landed at the wait at the top of the stage
      uint4 vv[2];
      asm volatile("ds_read_b128 %0, %2\n\tds_read_b128 %1, %3\n\ts_waitcnt lgkmcnt(0)"
                   : "=&v"(vv[0]), "=&v"(vv[1])
                   : "v"((uint32_t)(uintptr_t)(q + (((2 * hf) ^ ((r >> 2) & 3)) * 16))),
                     "v"((uint32_t)(uintptr_t)(q + (((2 * hf + 1) ^ ((r >> 2) & 3)) * 16)))
                   : "memory");
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int c = 2 * hf + u;  // logical 16-byte chunk of codes (codes 16 c ..)
        const uint4 v = vv[u];
        const uint4 lo = make_uint4(fp8x2_to_bf16x2<false>(v.x), fp8x2_to_bf16x2<true>(v.x),
                                    fp8x2_to_bf16x2<false>(v.y), fp8x2_to_bf16x2<true>(v.y));
        const uint4 hi = make_uint4(fp8x2_to_bf16x2<false>(v.z), fp8x2_to_bf16x2<true>(v.z),
                                    fp8x2_to_bf16x2<false>(v.w), fp8x2_to_bf16x2<true>(v.w));
        asm volatile("ds_write_b128 %0, %1\n\tds_write_b128 %2, %3"
                     :
                     : "v"((uint32_t)(uintptr_t)(b + (((2 * c) ^ (r & 7)) * 16))), "v"(__builtin_bit_cast(u32x4_t, lo)),
                       "v"((uint32_t)(uintptr_t)(b + (((2 * c + 1) ^ (r & 7)) * 16))), "v"(__builtin_bit_cast(u32x4_t, hi))
                     : "memory");
      }
    };
    if (KIND != KIND_FP8W) {
      // in flight at the top of stage kt, in issue order: B(kt), A(kt), B(kt+1)
      issueB(0);
      issueA(0);
      issueB(1);
      for (int kt = 0; kt < KT; ++kt) {
        wait_vm<NBI>();    // A(kt) and all before it (B(kt)) are in LDS; B(kt+1) may not be
        // ... for every wavefront; and stage kt-1 is no longer read.  A bare barrier: the
        // explicit count above is the wait (a fenced one would drain B(kt+1) too)
        __builtin_amdgcn_s_barrier();
        issueA(kt + 1);    // into A buffer (kt+1) & 1, which held stage kt-1
        issueB(kt + 2);    // into B buffer (kt+2) % 3, which held stage kt-1
        mfma_stage(kt);
      }
    } else {
      // codes of stage kt land three stages ahead and are widened one stage ahead; at the
      // top of stage kt, in issue order: A(kt), Q(kt+2) (Q(kt+1) before them has landed)
      issueA(0);
      issueB(0);
      issueB(1);
      issueB(2);
      wait_vm<2 * NBI>();  // A(0), Q(0)
      __builtin_amdgcn_s_barrier();
      widen(0);
      for (int kt = 0; kt < KT; ++kt) {
        wait_vm<NBI>();    // A(kt) and Q(kt+1) are in LDS; Q(kt+2) may not be
        // ... for every wavefront; stage kt is widened; stage kt-1 is no longer read
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        issueA(kt + 1);    // into A buffer (kt+1) & 1, which held stage kt-1
        issueB(kt + 3);    // codes into Q buffer kt % 3, widened last stage
        widen(kt + 1);     // into bf16 buffer (kt+1) & 1, which held stage kt-1
        mfma_stage(kt);
      }
    }
    wait_vm<0>();        // the loads past the end have landed before the buffers are reused
    __syncthreads();

    // ---- epilogue
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
            float g = acc[j][ni][v], uu = acc[j][ni + 4][v];
            if (col < Iseg) {
              if (ESZ == 1) {
                g *= sc[ni];
                uu *= sc[ni + 4];
              }
              if (KIND == KIND_A8) {
                g *= s_rsc[r];
                uu *= s_rsc[r];
              }
              dst[col] = to_bf16(g / (1.0f + expf(-g)) * uu);
            }
          }
        } else {
          uint16_t *dst = nullptr;
          if (routed) {
            const int slot = KIND == KIND_FP8W ? oslot[j][v] : s_slot[r];
            if (slot < n_slots) dst = a.y + (size_t)slot * a.H;
          } else {
            dst = a.y_s + (size_t)m * a.H;
          }
          if (dst != nullptr) {
#pragma unroll
            for (int ni = 0; ni < 8; ++ni) {
              const int col = n0 + bfr[ni] + ccol;
              float o = acc[j][ni][v];
              if (ESZ == 1) o *= sc[ni];
              if (KIND == KIND_A8) o *= s_rsc[r];
              if (col < a.H) dst[col] = to_bf16(o);
            }
          }
        }
      }
    }
  }
}

namespace {
template <int MODE, int KIND, int SHONLY>
hipError_t launch_expert_gemm_t(const GemmArgs &a, hipStream_t s) {
  auto kern = expert_gemm_kernel<MODE, KIND, SHONLY>;
  constexpr size_t lds = KIND == KIND_FP8W ? EG_LDS_FP8 : EG_LDS;
  constexpr size_t ESZ = KIND == KIND_BF16 ? 2 : 1;
  constexpr int TKE = KIND == KIND_A8 ? 128 : EG_TK;
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
                              (int)lds);
      if (e != hipSuccess) return e;
      opened[dev] = true;
    }
  }
  // the kernel addresses tokens, h and one expert's matrix through 32-bit buffer ranges
  const int imax = a.has_shared && a.I_s > a.I ? a.I_s : a.I;
  const size_t lim = (size_t)1 << 31;
  if ((size_t)a.T * a.H * 2 >= lim || (size_t)a.cap * a.I * 2 >= lim || (size_t)2 * imax * a.H * ESZ >= lim)
    return hipErrorInvalidValue;
  if (a.H % TKE != 0 || a.I % TKE != 0 || (a.has_shared && a.I_s % TKE != 0)) return hipErrorInvalidValue;
  const int NCH = MODE == MODE_GATE_UP ? (imax + EG_NB / 2 - 1) / (EG_NB / 2) : (a.H + EG_NB - 1) / EG_NB;
  const int NSEG_R = a.seg_mode == SEG_SHARED ? 0 : a.E;
  const int NSEG_S = a.has_shared && a.seg_mode != SEG_ROUTED ? (a.T + EG_MR - 1) / EG_MR : 0;
  if (NSEG_R + NSEG_S == 0) return hipSuccess;
  return launch_k(kern, dim3(grid_for((NSEG_R + NSEG_S) * NCH)), dim3(EG_NT), lds, s, a, NCH,
                  NSEG_R, NSEG_S);
}
}  // namespace

template <int MODE>
hipError_t launch_expert_gemm(const GemmArgs &a, hipStream_t s) {
  if (a.wtype == 1 || a.wtype == 2) {
    if (a.s_gu == nullptr || a.s_d == nullptr || (a.has_shared && (a.ss_gu == nullptr || a.ss_d == nullptr)))
      return hipErrorInvalidValue;
    if (a.wtype == 1)
      return a.seg_mode == SEG_SHARED ? launch_expert_gemm_t<MODE, KIND_FP8W, 1>(a, s)
                                      : launch_expert_gemm_t<MODE, KIND_FP8W, 0>(a, s);
    if (a.sx == nullptr || (MODE == MODE_GATE_UP ? a.x8 == nullptr : (a.h8 == nullptr || a.sh == nullptr)) ||
        (MODE == MODE_DOWN && a.has_shared && (a.hs8 == nullptr || a.shs == nullptr)))
      return hipErrorInvalidValue;
    return launch_expert_gemm_t<MODE, KIND_A8, 0>(a, s);
  }
  return a.seg_mode == SEG_SHARED ? launch_expert_gemm_t<MODE, KIND_BF16, 1>(a, s)
                                  : launch_expert_gemm_t<MODE, KIND_BF16, 0>(a, s);
}

hipError_t launch_gemm_gate_up(const GemmArgs &a, hipStream_t s) { return launch_expert_gemm<MODE_GATE_UP>(a, s); }

hipError_t launch_gemm_down(const GemmArgs &a, hipStream_t s) { return launch_expert_gemm<MODE_DOWN>(a, s); }

// ---------------------------------------------------------------- activation rows to fp8
// One wavefront per row of L bf16 values: s = 2^e for the least e with amax <= 448 * 2^e
// (1 for an all-zero row), code_i = the e4m3 code nearest a_i * 2^-e (an exact product),
// ties to an even mantissa.  A power-of-two scale costs the codes nothing (they are floating
// point) and makes every quotient exact; no quotient exceeds 448, so the hardware conversion
// (v_cvt_pk_fp8_f32, nearest even) never saturates.
// Rows whose `sorted` entry is the sentinel (padding of the alignment) are skipped.
// NG: 8-value groups per lane (L <= 512 NG); RPW rows per wavefront, all their loads in
// flight together; each row stays in registers between its amax and its encoding.
template <int NG, int RPW>
__global__ __launch_bounds__(256) void quant_rows_kernel(const uint16_t *__restrict__ src, int L, int R,
                                                         const int32_t *__restrict__ sorted, int n_slots,
                                                         uint8_t *__restrict__ dst, float *__restrict__ scale) {
  const int row0 = (blockIdx.x * 4 + wave_id()) * RPW, lane = lane_id();
  const int G = L / 8;
  uint4 v[RPW][NG];
  bool ok[RPW];
#pragma unroll
  for (int rr = 0; rr < RPW; ++rr) {
    const int row = row0 + rr;
    ok[rr] = row < R && (sorted == nullptr || sorted[row] < n_slots);
    const uint4 *r = reinterpret_cast<const uint4 *>(src + (size_t)row * L);
#pragma unroll
    for (int i = 0; i < NG; ++i)
      v[rr][i] = ok[rr] && lane + kWave * i < G ? r[lane + kWave * i] : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int rr = 0; rr < RPW; ++rr) {
    if (!ok[rr]) continue;  // uniform over the wavefront
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < NG; ++i) {
      const uint32_t w[4] = {v[rr][i].x, v[rr][i].y, v[rr][i].z, v[rr][i].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) amax = fmaxf(amax, fmaxf(fabsf(bf16_lo(w[q])), fabsf(bf16_hi(w[q]))));
    }
    // wavefront maximum: DPP within each 16-lane row, then the four rows' lane 0
    amax = fmaxf(amax, dpp_f32<kDppXor1>(amax));
    amax = fmaxf(amax, dpp_f32<kDppXor2>(amax));
    amax = fmaxf(amax, dpp_f32<kDppHalfMirror>(amax));
    amax = fmaxf(amax, dpp_f32<kDppMirror>(amax));
    amax = fmaxf(fmaxf(__builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, amax), 0)),
                       __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, amax), 16))),
                 fmaxf(__builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, amax), 32)),
                       __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, amax), 48))));
    int ex = 0;
    const float f = frexpf(amax, &ex);  // amax = f * 2^ex, f in [0.5, 1); 448 / 512 = 0.875
    const int e = amax > 0.0f ? (f <= 0.875f ? ex - 9 : ex - 8) : 0;
    const int row = row0 + rr;
    uint2 *d = reinterpret_cast<uint2 *>(dst + (size_t)row * L);
#pragma unroll
    for (int i = 0; i < NG; ++i) {
      if (lane + kWave * i >= G) continue;
      const uint32_t w[4] = {v[rr][i].x, v[rr][i].y, v[rr][i].z, v[rr][i].w};
      // v_cvt_pk_fp8_f32: two values to E4M3 codes, nearest even (no value here exceeds 448)
      int c01 = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(bf16_lo(w[0]), -e), ldexpf(bf16_hi(w[0]), -e), 0, false);
      c01 = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(bf16_lo(w[1]), -e), ldexpf(bf16_hi(w[1]), -e), c01, true);
      int c23 = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(bf16_lo(w[2]), -e), ldexpf(bf16_hi(w[2]), -e), 0, false);
      c23 = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(bf16_lo(w[3]), -e), ldexpf(bf16_hi(w[3]), -e), c23, true);
      d[lane + kWave * i] = make_uint2((uint32_t)c01, (uint32_t)c23);
    }
    if (lane == 0) scale[row] = ldexpf(1.0f, e);
  }
}

namespace {
template <int NG, int RPW>
hipError_t launch_quant_rows_t(const uint16_t *src, int L, int R, const int32_t *sorted, int n_slots, uint8_t *dst,
                               float *scale, hipStream_t s) {
  const int waves = (R + RPW - 1) / RPW;
  return launch_k(quant_rows_kernel<NG, RPW>, dim3((waves + 3) / 4), dim3(256), 0, s, src, L, R, sorted, n_slots,
                  dst, scale);
}

hipError_t launch_quant_rows(const uint16_t *src, int L, int R, const int32_t *sorted, int n_slots, uint8_t *dst,
                             float *scale, hipStream_t s) {
  if (R <= 0) return hipSuccess;
  if (L % 8 != 0 || L > 8192) return hipErrorInvalidValue;
  // one row per wavefront: the rows are short, so many wavefronts in flight hide the latency
  if (L <= 512) return launch_quant_rows_t<1, 1>(src, L, R, sorted, n_slots, dst, scale, s);
  if (L <= 1024) return launch_quant_rows_t<2, 1>(src, L, R, sorted, n_slots, dst, scale, s);
  if (L <= 2048) return launch_quant_rows_t<4, 1>(src, L, R, sorted, n_slots, dst, scale, s);
  if (L <= 4096) return launch_quant_rows_t<8, 1>(src, L, R, sorted, n_slots, dst, scale, s);
  return launch_quant_rows_t<16, 1>(src, L, R, sorted, n_slots, dst, scale, s);
}
}  // namespace

hipError_t launch_quant_tokens(const uint16_t *x, int T, int H, uint8_t *x8, float *sx, hipStream_t s) {
  return launch_quant_rows(x, H, T, nullptr, 0, x8, sx, s);
}

hipError_t launch_quant_h(const GemmArgs &a, hipStream_t s) {
  hipError_t e = launch_quant_rows((const uint16_t *)a.h, a.I, (int)a.cap, a.sorted, a.T * a.k, a.h8, a.sh, s);
  if (e != hipSuccess || !a.has_shared) return e;
  return launch_quant_rows((const uint16_t *)a.h_s, a.I_s, a.T, nullptr, 0, a.hs8, a.shs, s);
}

// ---------------------------------------------------------------- router on MFMA
// logits[t][e] = x_t . W_r[e] + b[e] and gate[t] = x_t . w_sg in fp32.  Each fp32 weight is
// split exactly into three bf16 parts while its tile is staged -- hi = rne(w),
// mid = rne(w - hi), lo = rne(w - hi - mid); each difference is exact in fp32 and
// hi + mid + lo == w -- so the MFMA sums exact bf16 products x.hi + x.mid + x.lo in fp32.
// Block: 128 tokens x 32 experts (a tall tile: each weight is split by half as many blocks
// as with a square one), 8 wavefronts in 4 (M) x 2 (N), each 32 x 16 as 2 x 1 tiles of
// 16x16x32 per part.  K in stages of 64 through a double LDS buffer fed from RT_NS
// register sets that rotate, so a stage's loads have RT_NS - 1 stages to land before they
// are staged.  The gate logit (fp32 FMAs on the staged tokens) is split among the expert
// tiles of a token tile: tile j of NN takes tokens j * ceil(128 / NN) .., 16 lanes per
// token, each lane 4 columns of every stage, then a 16-lane sum.  Blocks on one XCD take
// consecutive (token tile, expert tile) pairs, so a token tile's expert tiles share that
// XCD's L2 copy of its tokens.
namespace {
constexpr int RT_M = 128, RT_N = 32, RT_K = 64, RT_W = RT_K;  // LDS row: 64 bf16 (128 bytes)
constexpr int RT_NT = 512;
constexpr int RT_NS = 4;                                          // register sets
constexpr int RT_ABUF = RT_M * RT_W, RT_BBUF = 3 * RT_N * RT_W;  // elements per stage
constexpr size_t RT_LDS = (size_t)2 * (RT_ABUF + RT_BBUF) * 2 + 2 * RT_K * 4;  // 57856 bytes
constexpr int RT_GT = 4;                                         // gate tokens per lane at most
constexpr int RT_GR = RT_NT / 16;                                // gate token groups
}  // namespace

// fp32 pair -> exact three-way bf16 split, packed pairs (v_cvt_pk_bf16_f32 rounds both
// lanes of a pair to nearest even in one instruction)
__device__ __forceinline__ void split3_pk(float a0, float a1, uint32_t &h, uint32_t &m, uint32_t &l) {
  typedef float f2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 b2_t __attribute__((ext_vector_type(2)));
  h = __builtin_bit_cast(uint32_t, __builtin_convertvector((f2_t){a0, a1}, b2_t));
  const float r0 = a0 - bf16_lo(h), r1 = a1 - bf16_hi(h);
  m = __builtin_bit_cast(uint32_t, __builtin_convertvector((f2_t){r0, r1}, b2_t));
  l = __builtin_bit_cast(uint32_t, __builtin_convertvector((f2_t){r0 - bf16_lo(m), r1 - bf16_hi(m)}, b2_t));
}

__global__ __launch_bounds__(RT_NT) void router_mfma_kernel(const uint16_t *__restrict__ x, int T, int H,
                                                            const float *__restrict__ w_r,
                                                            const float *__restrict__ b_r, int E,
                                                            const float *__restrict__ w_sg,
                                                            float *__restrict__ logits,
                                                            float *__restrict__ gate_logit, int MT, int NN) {
  extern __shared__ __attribute__((aligned(16))) uint16_t rt_lds[];
  uint16_t *sA = rt_lds;                 // [2][128][72]: tokens
  uint16_t *sB = rt_lds + 2 * RT_ABUF;  // [2][3][32][72]: hi, mid, lo of the expert rows
  float *sG = reinterpret_cast<float *>(sB + 2 * RT_BBUF);  // [2][64]: gate weights
  const int tiles = MT * NN;
  const int per_xcd = (tiles + kXcds - 1) / kXcds;
  const int u = (blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
  if (u >= tiles) return;
  const int mt = u / NN, nt = u % NN;
  const int m0 = mt * RT_M, n0 = nt * RT_N;
  const int tid = threadIdx.x, lane = lane_id(), wave = wave_id();
  const int wm = wave & 3, wn = wave >> 2;

  // staging: token rows lrow, lrow + 64 (8 bf16 each); expert row wrow (4 fp32).  Each 8
  // lanes stage one 128-byte row; within 32 lanes the rows run 0, 1, 3, 2, so any 16 lanes
  // that the LDS serves together (consecutive eights, or eights 16 lanes apart) write one
  // even and one odd row, i.e. both halves of the banks
  const int lrow = (tid >> 3) ^ ((tid >> 4) & 1), lch = tid & 7;
  const int wrow = tid >> 4, wq = tid & 15;
  // rows past T or E load the last row (every load is issued, so the wait counts are
  // fixed) and are zeroed when staged
  const uint16_t *xr[2];
  bool xok[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int t = m0 + lrow + 64 * i;
    xok[i] = t < T;
    xr[i] = x + (size_t)min(t, T - 1) * H + 8 * lch;
  }
  const bool wok = n0 + wrow < E;
  const float *wp = w_r + (size_t)min(n0 + wrow, E - 1) * H + 4 * wq;
  // gate logit: tokens g0 + gr + RT_GR s of this tile (s < RT_GT), lane part gq
  const bool gate = w_sg != nullptr;
  const float *sgp = (gate ? w_sg : w_r) + lane;  // one weight per lane; without a gate: loaded, unused
  const int tpb = (RT_M + NN - 1) / NN;
  const int g0 = nt * tpb, g1 = min(g0 + tpb, RT_M);
  const int gr = tid >> 4, gq = tid & 15;
  float gacc[RT_GT];
#pragma unroll
  for (int s = 0; s < RT_GT; ++s) gacc[s] = 0.0f;

  // one stage of global loads in registers
  struct Stage {
    uint4 xa[2];
    float4 wv;
    float sg;
  };
  Stage st[RT_NS];
  const int KT = H / RT_K;
  auto gload = [&](Stage &S, int kt) {
    const int k0 = min(kt, KT - 1) * RT_K;  // past the end: reload the last stage (never used)
#pragma unroll
    for (int i = 0; i < 2; ++i) S.xa[i] = *reinterpret_cast<const uint4 *>(xr[i] + k0);
    S.wv = *reinterpret_cast<const float4 *>(wp + k0);
    S.sg = sgp[k0];
  };
  auto sstore = [&](const Stage &S, int buf) {
    uint16_t *A = sA + buf * RT_ABUF;
    uint16_t *B = sB + buf * RT_BBUF;
#pragma unroll
    for (int i = 0; i < 2; ++i)
      *reinterpret_cast<uint4 *>(&A[(lrow + 64 * i) * RT_W + 8 * (lch ^ (lrow & 7))]) =
          xok[i] ? S.xa[i] : make_uint4(0, 0, 0, 0);
    uint2 h, m, l;
    const float4 w = wok ? S.wv : make_float4(0.f, 0.f, 0.f, 0.f);
    split3_pk(w.x, w.y, h.x, m.x, l.x);
    split3_pk(w.z, w.w, h.y, m.y, l.y);
    const int off = wrow * RT_W + 8 * ((wq >> 1) ^ (wrow & 7)) + 4 * (wq & 1);
    *reinterpret_cast<uint2 *>(&B[off]) = h;
    *reinterpret_cast<uint2 *>(&B[RT_N * RT_W + off]) = m;
    *reinterpret_cast<uint2 *>(&B[2 * RT_N * RT_W + off]) = l;
    if (tid < RT_K) sG[buf * RT_K + tid] = S.sg;
  };

  f32x4_t acc[2];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi) acc[mi] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // a fragment row r (every fragment starts at a multiple of 16 rows, so r & 7 == fr & 7)
  // holds its K chunk q at chunk q ^ (r & 7)
  const int fr = lane & 15, fq = lane >> 4;
  auto compute = [&](int buf) {
    const uint16_t *A = sA + buf * RT_ABUF;
    const uint16_t *B = sB + buf * RT_BBUF;
#pragma unroll
    for (int ks = 0; ks < RT_K / 32; ++ks) {
      const int fc = 8 * ((4 * ks + fq) ^ (fr & 7));
      bf16x8_t af[2], bf[3];
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
        af[mi] = __builtin_bit_cast(bf16x8_t,
                                    *reinterpret_cast<const uint4 *>(&A[(32 * wm + 16 * mi + fr) * RT_W + fc]));
#pragma unroll
      for (int part = 0; part < 3; ++part)
        bf[part] = __builtin_bit_cast(
            bf16x8_t, *reinterpret_cast<const uint4 *>(&B[(part * RT_N + 16 * wn + fr) * RT_W + fc]));
#pragma unroll
      for (int part = 0; part < 3; ++part)
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
          acc[mi] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[mi], bf[part], acc[mi], 0, 0, 0);
    }
    if (gate) {
      const float4 sg = *reinterpret_cast<const float4 *>(&sG[buf * RT_K + 4 * gq]);
#pragma unroll
      for (int s = 0; s < RT_GT; ++s) {
        const int j = g0 + gr + RT_GR * s;
        if (j < g1) {
          const uint2 xv =
              *reinterpret_cast<const uint2 *>(&A[j * RT_W + 8 * ((gq >> 1) ^ (j & 7)) + 4 * (gq & 1)]);
          float g = gacc[s];
          g = fmaf(sg.x, bf16_lo(xv.x), g);
          g = fmaf(sg.y, bf16_hi(xv.x), g);
          g = fmaf(sg.z, bf16_lo(xv.y), g);
          g = fmaf(sg.w, bf16_hi(xv.y), g);
          gacc[s] = g;
        }
      }
    }
  };
  // stage kk sits in LDS buffer kk & 1 and stages kk + 1 .. kk + RT_NS - 1 in register
  // sets; stage kk + RT_NS is issued into the set that held stage kk.  The loop runs a
  // whole number of rotations: the steps past KT compute nothing, and their loads and LDS
  // stores touch stages that are never computed.
#pragma unroll
  for (int i = 0; i < RT_NS; ++i) gload(st[i], i);
  sstore(st[0], 0);
  __syncthreads();
  for (int kt0 = 0; kt0 < KT; kt0 += RT_NS) {
#pragma unroll
    for (int i = 0; i < RT_NS; ++i) {
      const int kk = kt0 + i;
      gload(st[i], kk + RT_NS);
      if (kk < KT) compute(kk & 1);
      sstore(st[(i + 1) % RT_NS], (kk + 1) & 1);
      __syncthreads();
    }
  }

  // epilogue: lane holds C[row = 4 * (lane / 16) + v][col = lane % 16] of each 16x16 tile
  const int crow = 4 * (lane >> 4), ccol = lane & 15;
  const int e = n0 + 16 * wn + ccol;
  const float bias = (e < E && b_r != nullptr) ? b_r[e] : 0.0f;
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int t = m0 + 32 * wm + 16 * mi + crow + v;
      if (t < T && e < E) logits[(size_t)t * E + e] = acc[mi][v] + bias;
    }
  if (gate) {
#pragma unroll
    for (int s = 0; s < RT_GT; ++s) {
      const float g = row16_sum(gacc[s]);  // the 16 lanes of one token are one DPP row
      const int j = g0 + gr + RT_GR * s;
      if (gq == 0 && j < g1 && m0 + j < T) gate_logit[m0 + j] = g;
    }
  }
}

hipError_t launch_router_gemm(const uint16_t *x, int T, int H, const float *w_r, const float *b_r, int E,
                              const float *w_sg, float *logits, float *gate_logit, hipStream_t s) {
  static std::mutex mu;
  static bool opened[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  {
    std::lock_guard<std::mutex> lock(mu);
    if (!opened[dev]) {
      e = hipFuncSetAttribute(reinterpret_cast<const void *>(router_mfma_kernel),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)RT_LDS);
      if (e != hipSuccess) return e;
      opened[dev] = true;
    }
  }
  if (H % RT_K != 0) return hipErrorInvalidValue;
  const int MT = (T + RT_M - 1) / RT_M, NN = (E + RT_N - 1) / RT_N;
  if ((RT_M + NN - 1) / NN > RT_GR * RT_GT) return hipErrorInvalidValue;  // gate tokens per tile
  return launch_k(router_mfma_kernel, dim3(grid_for(MT * NN)), dim3(RT_NT), RT_LDS, s, x, T, H, w_r, b_r, E, w_sg,
                  logits, gate_logit, MT, NN);
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
}

}  // namespace moe
