// float32 values as float16 hi + lo pieces (gfx950), with the rounding fixed by
// the instructions used: hi is the float16 rounding of the float32 value as
// stored, lo the float16 rounding of the exact residual against that same hi
// (so a compiler cannot contract the product that formed the value into either
// conversion and round the two against different values).
#pragma once

#include <hip/hip_runtime.h>

namespace tq {

// Two floats as float16 (RNE), packed lo | hi << 16.
__device__ __forceinline__ unsigned pack_f16(float a, float b) {
  unsigned r;
  asm("v_cvt_pk_f16_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
// float16(x - hi) for each half, hi = the packed float16 roundings of (a, b):
// one mixed-precision fma per half reads its hi as float16 and writes the
// result's half (a - hi is exact in float32, so each is the float16 rounding
// of the exact residual).
__device__ __forceinline__ unsigned residual_pair(float a, float b, unsigned hi) {
  unsigned r;
  asm("v_fma_mixlo_f16 %0, %1, 1.0, -%3 op_sel_hi:[0,0,1]\n\t"
      "v_fma_mixhi_f16 %0, %2, 1.0, -%3 op_sel:[0,0,1] op_sel_hi:[0,0,1]"
      : "=&v"(r) : "v"(a), "v"(b), "v"(hi));
  return r;
}

}  // namespace tq
