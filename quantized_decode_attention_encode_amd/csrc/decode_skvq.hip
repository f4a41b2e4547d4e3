// decode_skvq.hip - decode launches for SKVQ-adapted caches ("Changelog" v0.30.0): the kernel of
// decode_kernel.h with per-token key groups, the query and the outputs through the cache's
// channel permutations, and the first tokens' fp16 rows as the sink unit.
#include "decode_kernel.h"

namespace kvq {

hipError_t launch_decode_skvq(uint8_t* buf, const Layout& L, const DecodeShape& ds, const PerSeq& seq, const void* q, float* ws,
                              void* out, const void* ka, const void* va, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  if (L.D == 128) return launch_split_d<128, true, true>(buf, L, ds, seq, q, ws, out, ka, va, s, e0, e1);
  if (L.D == 64) return launch_split_d<64, true, true>(buf, L, ds, seq, q, ws, out, ka, va, s, e0, e1);
  return hipErrorInvalidValue;
}

}  // namespace kvq
