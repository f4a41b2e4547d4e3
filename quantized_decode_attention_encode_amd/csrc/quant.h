// quant.h - the group quantizer's arithmetic, shared by the record encoders (KIVI, KIVI-Sink,
// SKVQ, Kitty) and the stateless block encoder. Built with FMA contraction off: each fp32
// operation rounds once, in this order ("Changelog" v0.8.0 KIVI min/max groups; v0.30.0
// lo/scale parameters in fp16).
#pragma once
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

struct GroupParams {
  float lo, inv;
  uint32_t packed;  // scale16 | zero16 << 16
};

// Parameters of one group from its exact min and max.
template <int B>
__device__ __forceinline__ GroupParams group_params(float mn, float mx) {
  constexpr float L = float((1 << B) - 1);
  GroupParams p;
  const float lo = mn + 0.0f;
  const float hi = mx + 0.0f;
  const float s32 = (hi - lo) / L;
  const __half sc16 = __float2half_rn(s32);
  const float s = __half2float(sc16);
  p.lo = lo;
  p.inv = (s != 0.0f) ? 1.0f / s : 0.0f;
  const uint32_t zb = __half_as_ushort(__float2half_rn(lo));  // exact: lo is an fp16 value
  p.packed = uint32_t(__half_as_ushort(sc16)) | (zb << 16);
  return p;
}

template <int B>
__device__ __forceinline__ uint32_t code_of(float x, const GroupParams& p) {
  constexpr float L = float((1 << B) - 1);
  const float t = (x - p.lo) * p.inv;  // with inv = 0 this is 0, so a zero scale gives code 0
  const float c = fminf(fmaxf(rintf(t), 0.0f), L);
  return uint32_t(c);
}

}  // namespace kvq
