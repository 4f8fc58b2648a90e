// device.h -- small device helpers shared by the gfx950 kernels of the MoE layer.
//
// Wave64 everywhere: a wavefront is 64 lanes, reductions are xor butterflies whose
// result is bitwise identical in every lane (each step adds the same two operands
// in every lane pair), so every reduction here has one fixed order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

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

// Two OCP E4M3FN codes (byte `sel*2`, `sel*2+1` of w) -> a packed bf16 pair.  Every
// E4M3FN value is exact in bf16 (3 mantissa bits, exponents 2^-9..2^8).
template <bool HI_WORD>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
  typedef float f2_t __attribute__((ext_vector_type(2)));
  f2_t f = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, HI_WORD);
  return (__float_as_uint(f.x) >> 16) | (__float_as_uint(f.y) & 0xFFFF0000u);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    uint64_t o = __shfl_xor(v, off);
    v = o > v ? o : v;
  }
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
  typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

}  // namespace moe
