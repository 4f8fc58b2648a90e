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
// With up to four logits per lane, each lane sorts its candidates once (largest code
// first, lowest slot on equal codes) and its best remaining one is its head; with more,
// it rescans its slots for the best remaining one after each round.  Each round: the
// wavefront maximum of the lanes' best codes; a ballot names the lanes holding it, and on
// a tie between lanes the lowest expert index wins (a wavefront minimum), which is the
// order of the 64-bit key (code, ~index).  The winning lane retires that candidate.
template <int EPL, bool COHERENT = false>
__device__ __forceinline__ void topk_wave(const float *__restrict__ l, int E, int k, int renorm,
                                          int32_t *__restrict__ ids_out, float *__restrict__ w_out,
                                          int32_t *lds_ids) {
  const int lane = lane_id();
  float val[EPL];
  // all loads first, unguarded (index clamped into the row), so they are in flight together
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = min(lane + kWave * i, E - 1);
    val[i] = COHERENT ? __hip_atomic_load(l + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : l[e];
  }
  int my_e = 0;
  float my_v = 0.0f, top = 0.0f;
  if constexpr (EPL <= 4) {
    // The lane's candidates sorted once: the largest code first, the lower slot first among
    // equal codes (an odd-even transposition network on registers).  Slots past E carry
    // code 0 and the highest slot numbers, so they sort after every real candidate; nal
    // counts the real ones left.  The lane's best remaining candidate is always its head.
    uint32_t sc[EPL];
    int ss[EPL];
    int nal = 0;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const bool real = lane + kWave * i < E;
      sc[i] = real ? rank_code(val[i]) : 0u;
      ss[i] = i;
      nal += real ? 1 : 0;
      if (!real) val[i] = 0.0f;
    }
#pragma unroll
    for (int p = 0; p < EPL; ++p) {
#pragma unroll
      for (int i = p & 1; i + 1 < EPL; i += 2) {
        const bool sw = sc[i + 1] > sc[i] || (sc[i + 1] == sc[i] && ss[i + 1] < ss[i]);
        const uint32_t c0 = sw ? sc[i + 1] : sc[i], c1 = sw ? sc[i] : sc[i + 1];
        const int s0 = sw ? ss[i + 1] : ss[i], s1 = sw ? ss[i] : ss[i + 1];
        sc[i] = c0;
        sc[i + 1] = c1;
        ss[i] = s0;
        ss[i + 1] = s1;
      }
    }
    for (int j = 0; j < k; ++j) {
      const bool has = nal > 0;
      const uint32_t m = wave_max_u32(has ? sc[0] : 0u);
      const bool cand = has && sc[0] == m;
      const uint64_t bal = __ballot(cand);
      int win;
      if (__popcll(bal) == 1) {
        const int wl = __builtin_ctzll(bal);
        win = wl + kWave * __builtin_amdgcn_readlane(ss[0], wl);
      } else {  // equal codes in several lanes: the lowest expert index among their heads
        win = (int)wave_min_u32(cand ? (uint32_t)(lane + kWave * ss[0]) : ~0u);
      }
      const float v = rank_value(m);
      if (j == 0) top = v;
      my_e = lane == j ? win : my_e;
      my_v = lane == j ? v : my_v;
      // the winner's lane retires its head (selects: every lane runs it, only that one moves)
      const bool mine = lane == (win & (kWave - 1));
#pragma unroll
      for (int i = 0; i + 1 < EPL; ++i) {
        sc[i] = mine ? sc[i + 1] : sc[i];
        ss[i] = mine ? ss[i + 1] : ss[i];
      }
      nal -= mine ? 1 : 0;
    }
  } else {
    // the lane's best candidate: the largest code, the lowest slot among equal codes,
    // rescanned after every round (more slots per lane than a sort network pays for)
    uint32_t code[EPL];
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
