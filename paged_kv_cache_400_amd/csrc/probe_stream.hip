// probe_stream.hip -- measurement support (include/pa_probe.h): a plain
// streaming read of one buffer, the reference peak for the K/V gather.
//
// A segment is 1 KiB (64 lanes x 16 bytes).  Wave w of W reads segments
// w, w + W, w + 2W, ..., eight in flight, so that at any time the waves
// together sweep one contiguous window of memory (8 W KiB), with the same
// 16-byte streaming loads as the decode.  The launch shape is the one at
// which such a read peaks on this device: one workgroup of four waves per
// CU with 8 KiB in flight per wave read 2.2 GB at 7.38 TB/s; 4 or 16 KiB per
// wave, or 2, 4 or 8 workgroups per CU, read at 5.2-6.9 TB/s (more bytes in
// flight per CU than 32 KiB crowd the memory system).  Every loaded word
// enters an XOR that is stored only if it hits one particular value, so no
// load is dropped.
#include "pa_device.h"
#include "pa_launch.h"

namespace pa {

namespace {

constexpr int kProbeWaves = 4;           // waves per workgroup
constexpr int kProbeWorkgroupsPerCu = 1;
constexpr int kInFlight = 8;             // segments per wave per step

__global__ void __launch_bounds__(64 * kProbeWaves)
pa_probe_stream_kernel(uint16_t* __restrict__ sink, const uint4* __restrict__ buf, int64_t n16,
                       int64_t nwaves) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * kProbeWaves + (threadIdx.x >> 6);
  const int64_t nseg = (n16 + 63) / 64;
  uint32_t x = 0;
  for (int64_t s0 = wave; s0 < nseg; s0 += kInFlight * nwaves) {
    uint4 v[kInFlight];
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) {
      const int64_t i = (s0 + u * nwaves) * 64 + lane;
      v[u] = i < n16 ? load_stream(buf + i) : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) x ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (x == 0x9e3779b9u && lane == 0) sink[0] = (uint16_t)x;
}

}  // namespace

hipError_t launch_probe_stream(void* sink, const void* buf, size_t bytes, hipStream_t stream) {
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const int64_t groups = (int64_t)max(cus, 1) * kProbeWorkgroupsPerCu;
  hipLaunchKernelGGL(pa_probe_stream_kernel, dim3((uint32_t)groups), dim3(64 * kProbeWaves), 0,
                     stream, (uint16_t*)sink, (const uint4*)buf, (int64_t)(bytes / 16),
                     groups * kProbeWaves);
  return hipGetLastError();
}

}  // namespace pa
