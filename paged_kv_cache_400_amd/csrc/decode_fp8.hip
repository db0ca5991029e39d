// decode_fp8.hip -- the balanced (stream-K) decode of decode_streamk.h
// instantiated for 8-bit OCP E4M3 pools (pa_decode_fp8, and pa_probe_gather
// on 8-bit pools).  q and the output are bf16 or fp16.
#include "decode_streamk.h"

namespace pa {

hipError_t launch_decode_streamk_fp8(const StreamKArgs& a) {
  return a.bf16 ? launch_d<BF16, FP8>(a, false) : launch_d<F16, FP8>(a, false);
}

hipError_t launch_gather_streamk_fp8(const StreamKArgs& a) {
  return launch_d<BF16, FP8>(a, true);
}

}  // namespace pa
