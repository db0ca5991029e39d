// cache_ops.hip -- the append (reshape_and_cache) and the copy-on-write block
// copy (copy_blocks).  Both are pure data movement: 16-byte vector loads and
// stores, one 16-byte chunk per thread, no arithmetic on the values.
//
// Append: "Why the KV cache becomes the problem" (each decode step appends a
// small amount of new data) and "Paged attention borrows a trick from
// operating systems" (a growing request attaches another block): token i's
// rows go to slot_mapping[i], i.e. block slot / bs, offset slot % bs.
// Copy: "How PagedAttention works" (copy-on-write gives a diverging
// candidate a private copy of a shared block).
#include "pa_launch.h"

namespace pa {

// One thread per (token, KV head, 16-byte chunk).  Chunks of one token row
// are consecutive threads, so a wave writes whole rows.
__global__ void __launch_bounds__(256)
pa_reshape_and_cache_kernel(const uint4* __restrict__ key, const uint4* __restrict__ value,
                            uint4* __restrict__ k_cache, uint4* __restrict__ v_cache,
                            const int32_t* __restrict__ slot_mapping, int64_t total,
                            int32_t hkv, int32_t chunks, int32_t bs, int64_t num_slots) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= total) return;
  const int32_t c = (int32_t)(idx % chunks);
  const int64_t th = idx / chunks;          // token * hkv + head
  const int32_t h = (int32_t)(th % hkv);
  const int64_t i = th / hkv;
  const int64_t slot = slot_mapping[i];
  if (slot < 0 || slot >= num_slots) return;  // padding, or outside the pool
  const int64_t b = slot / bs, o = slot % bs;
  const int64_t dst = ((b * hkv + h) * bs + o) * chunks + c;
  k_cache[dst] = key[idx];
  v_cache[dst] = value[idx];
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
  hipLaunchKernelGGL(pa_reshape_and_cache_kernel, dim3((uint32_t)grid), dim3(256), 0, stream,
                     (const uint4*)key, (const uint4*)value, (uint4*)k_cache, (uint4*)v_cache,
                     slot_mapping, total, num_kv_heads, chunks, block_size,
                     (int64_t)num_blocks * block_size);
  return hipGetLastError();
}

hipError_t launch_copy_blocks(void* k_cache, void* v_cache, const int32_t* block_mapping,
                              int32_t num_pairs, int32_t num_kv_heads, int32_t head_dim,
                              int32_t block_size, int32_t num_blocks, hipStream_t stream) {
  const int64_t block_chunks = (int64_t)num_kv_heads * block_size * head_dim / 8;
  int64_t gy = (block_chunks + 255) / 256;
  if (gy > 64) gy = 64;
  hipLaunchKernelGGL(pa_copy_blocks_kernel, dim3((uint32_t)num_pairs, (uint32_t)gy), dim3(256),
                     0, stream, (uint4*)k_cache, (uint4*)v_cache, block_mapping, block_chunks,
                     num_blocks);
  return hipGetLastError();
}

}  // namespace pa
