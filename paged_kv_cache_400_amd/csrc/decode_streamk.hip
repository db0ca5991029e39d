// decode_streamk.hip -- the balanced (stream-K) decode of decode_streamk.h
// instantiated for 16-bit pools: with the matrix-core tile wave (pa_decode,
// pa_probe_gather) and with the vector-unit one (pa_decode_valu's balanced
// mode).
#include "decode_streamk.h"

namespace pa {

hipError_t launch_decode_streamk(const StreamKArgs& a) {
  return a.bf16 ? launch_d<BF16, BF16>(a, false) : launch_d<F16, F16>(a, false);
}

hipError_t launch_decode_streamk_valu(const StreamKArgs& a) {
  return a.bf16 ? launch_d<BF16, Vec>(a, false) : launch_d<F16, Vec>(a, false);
}

hipError_t launch_gather_streamk(const StreamKArgs& a) {
  return a.bf16 ? launch_d<BF16, BF16>(a, true) : launch_d<F16, F16>(a, true);
}

hipError_t launch_prefix_merge(const PrefixArgs& a) {
  if (a.head_dim == 64) return a.bf16 ? launch_prefix_merge_d<BF16, 64>(a)
                                      : launch_prefix_merge_d<F16, 64>(a);
  return a.bf16 ? launch_prefix_merge_d<BF16, 128>(a) : launch_prefix_merge_d<F16, 128>(a);
}

int streamk_device_waves() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    return kStreamKMaxWaves;
  return (int)min((int64_t)cus * kWorkgroupsPerCu * kWaves, (int64_t)kStreamKMaxWaves);
}

}  // namespace pa
