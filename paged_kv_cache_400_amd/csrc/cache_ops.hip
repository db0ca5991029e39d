// cache_ops.hip -- the append (reshape_and_cache) and the copy-on-write block
// copy (copy_blocks).  Both are pure data movement: 16-byte vector loads and
// stores, one 16-byte chunk per thread, no arithmetic on the values; and the
// quantising append into 8-bit pools.
//
// Append: "Why the KV cache becomes the problem" (each decode step appends a
// small amount of new data) and "Paged attention borrows a trick from
// operating systems" (a growing request attaches another block): token i's
// rows go to slot_mapping[i], i.e. block slot / bs, offset slot % bs.
// Copy: "How PagedAttention works" (copy-on-write gives a diverging
// candidate a private copy of a shared block).
#include "pa_device.h"
#include "pa_launch.h"

namespace pa {

// One thread per (token, KV head, 16-byte chunk).  Chunks of one token row
// are consecutive threads, so a wave writes whole rows.  The thread's key
// and value chunks are loaded together with its slot (they do not depend on
// it): one memory round trip before the stores, not two.  The empty asm
// takes all three as operands, so that the compiler issues the three loads
// before it and waits for them once (rather than moving the chunks' loads
// below the slot test, or waiting for one load before issuing the next).
// I is the type of the thread index: 32-bit when the thread count allows
// (the divisions by the head count and the row's chunk count are then
// 32-bit ones).
template <typename I>
__global__ void __launch_bounds__(256)
pa_reshape_and_cache_kernel(const uint4* __restrict__ key, const uint4* __restrict__ value,
                            uint4* __restrict__ k_cache, uint4* __restrict__ v_cache,
                            const int32_t* __restrict__ slot_mapping, I total, int32_t hkv,
                            int32_t chunks, int32_t bs, int64_t num_slots) {
  const I idx = (I)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= total) return;
  const I c = idx % (I)chunks;
  const I th = idx / (I)chunks;  // token * hkv + head
  const I h = th % (I)hkv;
  const I i = th / (I)hkv;
  uint4 k = key[idx], v = value[idx];
  int32_t slot = slot_mapping[i];
  asm volatile("" : "+v"(k.x), "+v"(k.y), "+v"(k.z), "+v"(k.w), "+v"(v.x), "+v"(v.y), "+v"(v.z),
               "+v"(v.w), "+v"(slot));
  if (slot < 0 || slot >= num_slots) return;  // padding, or outside the pool
  const int32_t b = slot / bs, o = slot % bs;
  const int64_t dst = (((int64_t)b * hkv + (int64_t)h) * bs + o) * chunks + (int64_t)c;
  k_cache[dst] = k;
  v_cache[dst] = v;
}

// ---- 8-bit pools ----------------------------------------------------------
// Quantising append.  The pages name KV quantisation as the lever on bytes
// per token ("What problem does PagedAttention solve, and what is continuous
// batching?", sections "Why the KV cache becomes the problem" and "What
// they'll ask next") and fix no format; this library stores OCP FP8 E4M3
// codes with one float32 scale per pool: code = E4M3(x / scale), the
// quotient rounded once to float32 (IEEE division), then to the nearest
// E4M3 value with ties to the even code, saturating at +-448; NaN keeps its
// sign and becomes the NaN code.

// E4M3 code of y, from y's float32 bits (sign, 8-bit exponent, 23-bit
// fraction) with the E4M3 grid: normal values (1 + f/8) 2^(e-7), e = 1..15,
// and subnormals f 2^-9.
__device__ __forceinline__ uint32_t e4m3_code(float y) {
  const uint32_t u = __float_as_uint(y);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return sign | 0x7fu;      // NaN
  if (a >= 0x43e00000u) return sign | 0x7eu;     // |y| >= 448 (inf included): saturate
  if (a < 0x3c800000u) {                         // |y| < 2^-6: multiples of 2^-9
    // |y| * 2^9 is exact; rounding it to an integer (ties to even) gives the
    // code directly, 8 being the smallest normal 2^-6
    return sign | (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);
  }
  // keep 3 of the 23 fraction bits, rounding to nearest even; a carry into
  // the exponent is the correct next binade.  Code = (exponent - 120) << 3
  // | fraction, as the float32 exponent bias is 127 and E4M3's is 7.
  const uint32_t r = (a + 0x7ffffu + ((a >> 20) & 1u)) >> 20;
  return sign | (r - (120u << 3));
}

// One thread per (token, KV head, 16 elements): reads 32 bytes of key and of
// value, writes 16 bytes of codes to each pool.  As in the 16-bit append,
// the rows and the slot are loaded together (the empty asms take them all
// as operands), and I is the thread index type.
template <typename T, typename I>
__global__ void __launch_bounds__(256)
pa_reshape_and_cache_fp8_kernel(const uint4* __restrict__ key, const uint4* __restrict__ value,
                                uint4* __restrict__ k_cache, uint4* __restrict__ v_cache,
                                const int32_t* __restrict__ slot_mapping, I total, int32_t hkv,
                                int32_t chunks, int32_t bs, int64_t num_slots, float k_scale,
                                float v_scale) {
  const I idx = (I)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= total) return;
  const I c = idx % (I)chunks;
  const I th = idx / (I)chunks;  // token * hkv + head
  const I h = th % (I)hkv;
  const I i = th / (I)hkv;
  uint4 k0 = key[2 * (int64_t)idx], k1 = key[2 * (int64_t)idx + 1];
  uint4 v0 = value[2 * (int64_t)idx], v1 = value[2 * (int64_t)idx + 1];
  int32_t slot = slot_mapping[i];
  asm volatile("" : "+v"(k0.x), "+v"(k0.y), "+v"(k0.z), "+v"(k0.w), "+v"(k1.x), "+v"(k1.y),
               "+v"(k1.z), "+v"(k1.w), "+v"(slot));
  asm volatile("" : "+v"(v0.x), "+v"(v0.y), "+v"(v0.z), "+v"(v0.w), "+v"(v1.x), "+v"(v1.y),
               "+v"(v1.z), "+v"(v1.w));
  auto quantise16 = [&](const uint4& x0, const uint4& x1, float scale) {
    const uint32_t w[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
    uint32_t q[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t a = w[2 * j], b2 = w[2 * j + 1];
      q[j] = e4m3_code(lo_f32<T>(a) / scale) | (e4m3_code(hi_f32<T>(a) / scale) << 8) |
             (e4m3_code(lo_f32<T>(b2) / scale) << 16) | (e4m3_code(hi_f32<T>(b2) / scale) << 24);
    }
    return make_uint4(q[0], q[1], q[2], q[3]);
  };
  const uint4 kq = quantise16(k0, k1, k_scale);
  const uint4 vq = quantise16(v0, v1, v_scale);
  if (slot < 0 || slot >= num_slots) return;  // padding, or outside the pool
  const int32_t b = slot / bs, o = slot % bs;
  const int64_t dst = (((int64_t)b * hkv + (int64_t)h) * bs + o) * chunks + (int64_t)c;
  k_cache[dst] = kq;
  v_cache[dst] = vq;
}

// grid.x = pair; grid.y strides over the block's 16-byte chunks.
__global__ void __launch_bounds__(256)
pa_copy_blocks_kernel(uint4* __restrict__ k_cache, uint4* __restrict__ v_cache,
                      const int32_t* __restrict__ block_mapping, int64_t block_chunks,
                      int32_t num_blocks) {
  const int32_t src = block_mapping[2 * (int64_t)blockIdx.x];
  const int32_t dst = block_mapping[2 * (int64_t)blockIdx.x + 1];
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return;
  const uint4* ks = k_cache + (int64_t)src * block_chunks;
  const uint4* vs = v_cache + (int64_t)src * block_chunks;
  uint4* kd = k_cache + (int64_t)dst * block_chunks;
  uint4* vd = v_cache + (int64_t)dst * block_chunks;
  for (int64_t j = (int64_t)blockIdx.y * blockDim.x + threadIdx.x; j < block_chunks;
       j += (int64_t)gridDim.y * blockDim.x) {
    kd[j] = ks[j];
    vd[j] = vs[j];
  }
}

hipError_t launch_reshape_and_cache(const void* key, const void* value, void* k_cache,
                                    void* v_cache, const int32_t* slot_mapping,
                                    int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                                    int32_t block_size, int32_t num_blocks, hipStream_t stream) {
  const int32_t chunks = head_dim / 8;
  const int64_t total = (int64_t)num_tokens * num_kv_heads * chunks;
  const int64_t grid = (total + 255) / 256;
  const int64_t num_slots = (int64_t)num_blocks * block_size;
  if (grid * 256 <= (int64_t)UINT32_MAX)
    hipLaunchKernelGGL(pa_reshape_and_cache_kernel<uint32_t>, dim3((uint32_t)grid), dim3(256), 0,
                       stream, (const uint4*)key, (const uint4*)value, (uint4*)k_cache,
                       (uint4*)v_cache, slot_mapping, (uint32_t)total, num_kv_heads, chunks,
                       block_size, num_slots);
  else
    hipLaunchKernelGGL(pa_reshape_and_cache_kernel<int64_t>, dim3((uint32_t)grid), dim3(256), 0,
                       stream, (const uint4*)key, (const uint4*)value, (uint4*)k_cache,
                       (uint4*)v_cache, slot_mapping, total, num_kv_heads, chunks, block_size,
                       num_slots);
  return hipGetLastError();
}

hipError_t launch_reshape_and_cache_fp8(const void* key, const void* value, void* k_cache,
                                        void* v_cache, const int32_t* slot_mapping,
                                        int32_t num_tokens, int32_t num_kv_heads,
                                        int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                        float k_scale, float v_scale, bool bf16,
                                        hipStream_t stream) {
  const int32_t chunks = head_dim / 16;
  const int64_t total = (int64_t)num_tokens * num_kv_heads * chunks;
  const int64_t grid = (total + 255) / 256;
  const int64_t num_slots = (int64_t)num_blocks * block_size;
  if (grid * 256 <= (int64_t)UINT32_MAX) {
    auto kernel = bf16 ? pa_reshape_and_cache_fp8_kernel<BF16, uint32_t>
                       : pa_reshape_and_cache_fp8_kernel<F16, uint32_t>;
    hipLaunchKernelGGL(kernel, dim3((uint32_t)grid), dim3(256), 0, stream, (const uint4*)key,
                       (const uint4*)value, (uint4*)k_cache, (uint4*)v_cache, slot_mapping,
                       (uint32_t)total, num_kv_heads, chunks, block_size, num_slots, k_scale,
                       v_scale);
  } else {
    auto kernel = bf16 ? pa_reshape_and_cache_fp8_kernel<BF16, int64_t>
                       : pa_reshape_and_cache_fp8_kernel<F16, int64_t>;
    hipLaunchKernelGGL(kernel, dim3((uint32_t)grid), dim3(256), 0, stream, (const uint4*)key,
                       (const uint4*)value, (uint4*)k_cache, (uint4*)v_cache, slot_mapping,
                       total, num_kv_heads, chunks, block_size, num_slots, k_scale, v_scale);
  }
  return hipGetLastError();
}

hipError_t launch_copy_blocks(void* k_cache, void* v_cache, const int32_t* block_mapping,
                              int32_t num_pairs, int32_t num_kv_heads, int32_t head_dim,
                              int32_t block_size, int32_t num_blocks, int32_t elem_bytes,
                              hipStream_t stream) {
  const int64_t block_chunks = (int64_t)num_kv_heads * block_size * head_dim * elem_bytes / 16;
  int64_t gy = (block_chunks + 255) / 256;
  if (gy > 64) gy = 64;
  hipLaunchKernelGGL(pa_copy_blocks_kernel, dim3((uint32_t)num_pairs, (uint32_t)gy), dim3(256),
                     0, stream, (uint4*)k_cache, (uint4*)v_cache, block_mapping, block_chunks,
                     num_blocks);
  return hipGetLastError();
}

}  // namespace pa
