// device.h -- small device helpers shared by the gfx950 kernels of the MoE layer.
//
// Wave64 everywhere: a wavefront is 64 lanes in four 16-lane DPP rows.  Reductions use
// DPP permutations inside a row and readlane across rows; every step has one fixed
// pairing, so every reduction here has one fixed order (bitwise reproducible).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }
__device__ __forceinline__ int wave_id() { return threadIdx.x / kWave; }

// bf16 halves of a packed pair -> fp32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t to_bf16(float f) {
  __bf16 b = (__bf16)f;
  return __builtin_bit_cast(uint16_t, b);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)to_bf16(lo) | ((uint32_t)to_bf16(hi) << 16);
}
// fp32 rounded to the nearest bf16, returned as fp32.
__device__ __forceinline__ float round_bf16(float f) { return __uint_as_float((uint32_t)to_bf16(f) << 16); }

// c + a.lo*b.lo + a.hi*b.hi with bf16 pairs (v_dot2_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c,
                                         false);
}
__device__ __forceinline__ float dot8_bf16(const uint4 &a, const uint4 &b, float c) {
  c = dot2_bf16(a.x, b.x, c);
  c = dot2_bf16(a.y, b.y, c);
  c = dot2_bf16(a.z, b.z, c);
  c = dot2_bf16(a.w, b.w, c);
  return c;
}

// Two OCP E4M3FN codes (byte `sel*2`, `sel*2+1` of w) -> a packed bf16 pair, in one
// v_cvt_scalef32_pk_bf16_fp8 (scale 1).  Every E4M3FN value is exact in bf16 (3 mantissa
// bits, exponents 2^-9..2^8).
template <bool HI_WORD>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI_WORD));
}

// DPP lane permutations (gfx9 encodings): quad_perm [1,0,3,2] and [2,3,0,1],
// row_half_mirror (lane i <-> 7-i in each 8-lane half row), row_mirror (i <-> 15-i).
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, false);
}
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;

// Sum over each 16-lane row: every lane of the row ends with the same value (each step
// adds a lane and its mirror partner, the same two operands on both sides).
// (The DPP source is read with bound_ctrl set, the form the compiler folds into a single
// DPP-modified add; every lane of a full wavefront is a valid source for these patterns,
// so the zero fill is never taken and the sums are those of a plain move plus add.)
template <int CTRL>
__device__ __forceinline__ float dpp_add_src(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_add_src<kDppXor1>(v);
  v += dpp_add_src<kDppXor2>(v);
  v += dpp_add_src<kDppHalfMirror>(v);
  v += dpp_add_src<kDppMirror>(v);
  return v;
}
__device__ __forceinline__ float lane_value(float v, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}
// Sum over the wavefront, returned uniform: row sums, then (r0 + r1) + (r2 + r3).
__device__ __forceinline__ float wave_sum(float v) {
  v = row16_sum(v);
  return (lane_value(v, 0) + lane_value(v, 16)) + (lane_value(v, 32) + lane_value(v, 48));
}

__device__ __forceinline__ uint64_t max_u64(uint64_t a, uint64_t b) { return a > b ? a : b; }
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  return ((uint64_t)dpp_u32<CTRL>((uint32_t)(v >> 32)) << 32) | dpp_u32<CTRL>((uint32_t)v);
}
__device__ __forceinline__ uint64_t lane_value_u64(uint64_t v, int lane) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, lane);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), lane);
  return ((uint64_t)hi << 32) | lo;
}
// Maximum over the wavefront, returned uniform.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  v = max_u64(v, dpp_u64<kDppXor1>(v));
  v = max_u64(v, dpp_u64<kDppXor2>(v));
  v = max_u64(v, dpp_u64<kDppHalfMirror>(v));
  v = max_u64(v, dpp_u64<kDppMirror>(v));
  return max_u64(max_u64(lane_value_u64(v, 0), lane_value_u64(v, 16)),
                 max_u64(lane_value_u64(v, 32), lane_value_u64(v, 48)));
}

// DPP row broadcasts (GFX9): lane 15 of each row into the next row, lane 31 into rows 2
// and 3.  Rows outside the row mask keep `old`.
constexpr int kDppRowBcast15 = 0x142, kDppRowBcast31 = 0x143, kDppRowShr1 = 0x111;
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_upd_u32(uint32_t old, uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)v, CTRL, ROW_MASK, 0xF, false);
}
// Maximum / minimum over the wavefront, returned uniform: row reductions, then the row
// broadcasts carry the running value into lane 63.  `old` is the operation's identity, so
// each step compiles to a single DPP-modified max / min.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_upd_u32<kDppXor1, 0xF>(0u, v));
  v = max(v, dpp_upd_u32<kDppXor2, 0xF>(0u, v));
  v = max(v, dpp_upd_u32<kDppHalfMirror, 0xF>(0u, v));
  v = max(v, dpp_upd_u32<kDppMirror, 0xF>(0u, v));
  v = max(v, dpp_upd_u32<kDppRowBcast15, 0xA>(0u, v));
  v = max(v, dpp_upd_u32<kDppRowBcast31, 0xC>(0u, v));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  v = min(v, dpp_upd_u32<kDppXor1, 0xF>(~0u, v));
  v = min(v, dpp_upd_u32<kDppXor2, 0xF>(~0u, v));
  v = min(v, dpp_upd_u32<kDppHalfMirror, 0xF>(~0u, v));
  v = min(v, dpp_upd_u32<kDppMirror, 0xF>(~0u, v));
  v = min(v, dpp_upd_u32<kDppRowBcast15, 0xA>(~0u, v));
  v = min(v, dpp_upd_u32<kDppRowBcast31, 0xC>(~0u, v));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}
// Inclusive prefix sum over the wavefront's lanes (Hillis-Steele within each 16-lane row
// with row shifts, then the row broadcasts); lanes shifted in from outside a row add 0.
__device__ __forceinline__ uint32_t wave_incl_scan_u32(uint32_t v) {
  v += dpp_upd_u32<kDppRowShr1, 0xF>(0u, v);
  v += dpp_upd_u32<kDppRowShr1 + 1, 0xF>(0u, v);
  v += dpp_upd_u32<kDppRowShr1 + 3, 0xF>(0u, v);
  v += dpp_upd_u32<kDppRowShr1 + 7, 0xF>(0u, v);
  v += dpp_upd_u32<kDppRowBcast15, 0xA>(0u, v);
  v += dpp_upd_u32<kDppRowBcast31, 0xC>(0u, v);
  return v;
}

__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = lane_id();
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    int o = __shfl_up(v, off);
    if (lane >= off) v += o;
  }
  return v;
}

// Exclusive scan over the NT threads of a block; tmp: NT/64 + 1 ints of LDS.
template <int NT>
__device__ __forceinline__ int block_excl_scan(int v, int *tmp, int *total) {
  constexpr int NWV = NT / kWave;
  const int lane = lane_id(), w = wave_id();
  int inc = wave_incl_scan(v);
  if (lane == kWave - 1) tmp[w] = inc;
  __syncthreads();
  if (w == 0) {
    int t = lane < NWV ? tmp[lane] : 0;
    int ti = wave_incl_scan(t);
    if (lane < NWV) tmp[lane] = ti - t;
    if (lane == NWV - 1) tmp[NWV] = ti;
  }
  __syncthreads();
  int r = inc - v + tmp[w];
  *total = tmp[NWV];
  __syncthreads();
  return r;
}

// Largest e in [0, E) with off[e] <= p, for 0 <= p < off[E] (off non-decreasing):
// the expert whose padded segment holds position p.
__device__ __forceinline__ int segment_of(const int32_t *off, int E, int p) {
  int lo = 0, hi = E;
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (off[mid] <= p) lo = mid;
    else hi = mid;
  }
  return lo;
}

// Order-preserving 32-bit code of a float for the routing rank: larger float ->
// larger code; -0 and +0 share a code; every NaN gets code 0, below -inf.
__device__ __forceinline__ uint32_t rank_code(float v) {
  uint32_t b = __float_as_uint(v);
  if ((b & 0x7FFFFFFFu) > 0x7F800000u) return 0u;
  if (b == 0x80000000u) b = 0u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float rank_value(uint32_t c) {
  return __uint_as_float((c & 0x80000000u) ? (c & 0x7FFFFFFFu) : ~c);
}
// 64-bit routing key: the rank code above the complemented expert index, so that
// equal logits rank the lower index first.  0 is below every valid key.
__device__ __forceinline__ uint64_t rank_key(float v, int e) {
  return ((uint64_t)rank_code(v) << 32) | (uint32_t)(~(uint32_t)e);
}

// 16-byte load of data that is read once (weights): non-temporal, so it does not
// push the small, reused operands (tokens, intermediates) out of the caches.
__device__ __forceinline__ uint4 ld_stream(const uint4 *p) {

  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

}  // namespace moe
