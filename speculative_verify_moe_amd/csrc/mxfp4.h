// mxfp4.h -- OCP MXFP4 (E2M1 codes, E8M0 block scales) for the decode kernels.
#pragma once

#include "device.h"

namespace moe {

// MXFP4: 32 E2M1 codes of one scale block (byte b holds values 2b in its low nibble and
// 2b + 1 in its high nibble) against 32 bf16 activations x[0..3]; v_cvt_scalef32_pk_bf16_fp4
// widens two codes exactly (scale 1), the block scale multiplies the finished block sum.
template <int SEL>
__device__ __forceinline__ uint32_t fp4x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, SEL));
}
__device__ __forceinline__ float dot32_fp4_bf16(const uint4 &w, const uint4 *x) {
  const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
  float acc = 0.0f;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const uint4 xv = x[d];
    acc = dot2_bf16(fp4x2_to_bf16x2<0>(wd[d]), xv.x, acc);
    acc = dot2_bf16(fp4x2_to_bf16x2<1>(wd[d]), xv.y, acc);
    acc = dot2_bf16(fp4x2_to_bf16x2<2>(wd[d]), xv.z, acc);
    acc = dot2_bf16(fp4x2_to_bf16x2<3>(wd[d]), xv.w, acc);
  }
  return acc;
}
// E8M0 scale byte -> 2^(X - 127) (0xFF: NaN)
__device__ __forceinline__ float e8m0_scale(uint32_t X) {
  return X == 0xFFu ? __builtin_nanf("") : ldexpf(1.0f, (int)X - 127);
}

}  // namespace moe
