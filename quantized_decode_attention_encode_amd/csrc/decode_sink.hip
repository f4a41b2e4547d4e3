// decode_sink.hip - decode launches for caches with sink tokens ("Changelog" v0.9.0, KIVI-Sink):
// the same kernel (decode_kernel.h) with one more unit per sequence, the sinks' fp16 rows, and
// the sinks' quantized slots skipped.
#include "decode_kernel.h"

namespace kvq {

hipError_t launch_decode_sink(uint8_t* buf, const Layout& L, const DecodeShape& ds, const PerSeq& seq, const void* q, float* ws,
                              void* out, const void* ka, const void* va, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  if (L.D == 128) return launch_split_d<128, true, false>(buf, L, ds, seq, q, ws, out, ka, va, s, e0, e1);
  if (L.D == 64) return launch_split_d<64, true, false>(buf, L, ds, seq, q, ws, out, ka, va, s, e0, e1);
  return hipErrorInvalidValue;
}

}  // namespace kvq
