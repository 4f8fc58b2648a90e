// topk.h -- one wavefront's top-k routing of one token (shared by the routing kernels
// and the fused decode kernel).
//
// Qwen3.8 Flash-Next . GB10 UltraFast, "How it works" (a sort-free verify-path top-k):
// the token's E logits sit in registers as order-preserving 32-bit codes; each of the
// k rounds takes a wavefront maximum (DPP) and breaks ties to the lower expert index
// with ballots, then retires the winner.  Gate
// weights: exp(l_j - l_0) / sum_{j'<k} exp(l_j' - l_0) (renormalised softmax), or the
// plain softmax probability when renorm == 0.
#pragma once

#include "device.h"

namespace moe {

// Writes ids_out[0..k), w_out[0..k) (lanes 0..k-1) and, when lds_ids is given, the ids
// there too.  EPL = ceil(E / 64) logits per lane (expert e = lane + 64 i in slot i).
// COHERENT: read the logits with agent-scope loads (they were written by other blocks of
// the same kernel with agent-scope stores).
// Each lane keeps its best remaining candidate (largest code, lowest slot on equal
// codes).  Each round: the wavefront maximum of those codes; a ballot names the lanes
// holding it, and on a tie between lanes the lowest expert index wins (a wavefront
// minimum), which is the order of the 64-bit key (code, ~index).  The winning lane
// retires its candidate and rescans its slots.
template <int EPL, bool COHERENT = false>
__device__ __forceinline__ void topk_wave(const float *__restrict__ l, int E, int k, int renorm,
                                          int32_t *__restrict__ ids_out, float *__restrict__ w_out,
                                          int32_t *lds_ids) {
  const int lane = lane_id();
  uint32_t code[EPL];
  float val[EPL];
  // all loads first, unguarded (index clamped into the row), so they are in flight together
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = min(lane + kWave * i, E - 1);
    val[i] = COHERENT ? __hip_atomic_load(l + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : l[e];
  }
  uint32_t alive = 0;  // bit i: slot i is a candidate
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    if (lane + kWave * i < E) {
      code[i] = rank_code(val[i]);
      alive |= 1u << i;
    } else {
      val[i] = 0.0f;
      code[i] = 0;
    }
  }
  // the lane's best candidate: the largest code, the lowest slot among equal codes
  uint32_t bc = 0;
  int bs = -1;
  // (selects, no branches: every lane runs it every round, only the winner's changes)
  auto lane_best = [&]() {
    bc = 0;
    bs = -1;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const bool take = ((alive >> i) & 1u) != 0 && (bs < 0 || code[i] > bc);
      bc = take ? code[i] : bc;
      bs = take ? i : bs;
    }
  };
  lane_best();
  int my_e = 0;
  float my_v = 0.0f, top = 0.0f;
  for (int j = 0; j < k; ++j) {
    const bool has = bs >= 0;
    const uint32_t m = wave_max_u32(has ? bc : 0u);
    const bool cand = has && bc == m;
    const uint64_t bal = __ballot(cand);
    int win;
    if (__popcll(bal) == 1) {
      const int wl = __builtin_ctzll(bal);
      win = wl + kWave * __builtin_amdgcn_readlane(bs, wl);
    } else {  // equal codes in several lanes: the lowest expert index among them
      win = (int)wave_min_u32(cand ? (uint32_t)(lane + kWave * bs) : ~0u);
    }
    const float v = rank_value(m);
    if (j == 0) top = v;
    my_e = lane == j ? win : my_e;
    my_v = lane == j ? v : my_v;
    alive = lane == (win & (kWave - 1)) ? alive & ~(1u << (win / kWave)) : alive;
    lane_best();
  }
  const float ex = lane < k ? expf(my_v - top) : 0.0f;
  float denom;
  if (renorm) {
    denom = wave_sum(ex);
  } else {
    float part = 0.0f;
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      if (lane + kWave * i < E) part += expf(val[i] - top);
    denom = wave_sum(part);
  }
  if (lane < k) {
    ids_out[lane] = my_e;
    w_out[lane] = ex / denom;
    if (lds_ids != nullptr) lds_ids[lane] = my_e;
  }
}


}  // namespace moe
