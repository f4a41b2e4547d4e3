// decode.hip - decode launches for caches without sink tokens (the kernel is in decode_kernel.h).
#include "decode_kernel.h"

namespace kvq {

hipError_t launch_decode(uint8_t* buf, const Layout& L, const DecodeShape& ds, const PerSeq& seq, const void* q, float* ws,
                         void* out, const void* ka, const void* va, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  if (L.method == kMethodSkvq) return launch_decode_skvq(buf, L, ds, seq, q, ws, out, ka, va, s, e0, e1);
  if (L.NS > 0) return launch_decode_sink(buf, L, ds, seq, q, ws, out, ka, va, s, e0, e1);
  if (L.D == 128) return launch_split_d<128, false, false>(buf, L, ds, seq, q, ws, out, ka, va, s, e0, e1);
  if (L.D == 64) return launch_split_d<64, false, false>(buf, L, ds, seq, q, ws, out, ka, va, s, e0, e1);
  return hipErrorInvalidValue;
}

}  // namespace kvq
