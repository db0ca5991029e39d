// pa_launch.h -- internal interface between the C ABI (pa_api.hip) and the
// kernel launchers.  Arguments are already validated when these run.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

// ---- LDS limits -----------------------------------------------------------
// gfx950 gives one workgroup at most 160 KiB of LDS.  Every kernel checks its
// static LDS against this at compile time (static_assert beside its
// __shared__ arrays); the launchers also check the kernel's LDS against the
// device's own per-workgroup limit before launching, because a launch whose
// workgroup needs more LDS than the device has is accepted by the runtime and
// then aborts the queue (HSA_STATUS_ERROR_INVALID_ALLOCATION), taking the
// process's later GPU work with it.
constexpr int kMaxLdsBytes = 160 * 1024;

// What a launcher returns when its kernel cannot be launched on the current
// device because of its resources (LDS, or no workgroup fits a CU); the C
// ABI reports it as PA_ERR_UNSUPPORTED.
constexpr hipError_t kErrDoesNotFit = hipErrorInvalidConfiguration;

constexpr int kMaxDevices = 64;

// hipSuccess if `kernel` (its static LDS plus `dynamic_bytes`) fits one
// workgroup on the current device, kErrDoesNotFit if not, another error if
// the runtime cannot tell.  `cache` is the caller's per-device memo (one per
// kernel instantiation): 1 fits, -1 does not, 0 not yet known; recomputing
// gives the same answer, so concurrent first calls are harmless.
inline hipError_t check_lds(const void* kernel, size_t dynamic_bytes,
                            int (&cache)[kMaxDevices]) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  const int known = __atomic_load_n(&cache[dev], __ATOMIC_RELAXED);
  if (known != 0) return known > 0 ? hipSuccess : kErrDoesNotFit;
  hipFuncAttributes attr;
  e = hipFuncGetAttributes(&attr, kernel);
  if (e != hipSuccess) return e;
  int limit = 0;
  e = hipDeviceGetAttribute(&limit, hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
  if (e != hipSuccess) return e;
  const bool fits = attr.sharedSizeBytes + dynamic_bytes <= (size_t)limit &&
                    attr.sharedSizeBytes + dynamic_bytes <= (size_t)kMaxLdsBytes;
  __atomic_store_n(&cache[dev], fits ? 1 : -1, __ATOMIC_RELAXED);
  return fits ? hipSuccess : kErrDoesNotFit;
}

struct DecodeArgs {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* seq_lens;
  float* ws_acc;      // [S][Hq][pmax][D]   (pmax > 1 only)
  float2* ws_ml;      // [S][Hq][pmax]      (m, l), m in base-2 units
  int32_t num_seqs, num_kv_heads, group, head_dim, block_size;
  int32_t max_blocks_per_seq, num_blocks, part, pmax;
  float qk_scale;     // scale * log2(e)
  bool bf16;
  hipStream_t stream;
};

// Balanced (stream-K) decode (decode_streamk.hip), pa_decode's automatic
// mode.  Workspace, for a launch of W waves: ws_acc float [2 * W][Gmax][D],
// then ws_ml float2 [2 * W][Gmax], then ws_meta int4 [S * Hq] (one record
// per (sequence, KV head) is used), with Gmax = min(Hq, 8);
// streamk_workspace_bytes gives the total.  W is at most kStreamKMaxWaves.
constexpr int kStreamKMaxWaves = 8192;

struct StreamKArgs {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* seq_lens;
  float* ws_acc;
  float2* ws_ml;
  int4* ws_meta;
  int32_t max_waves;  // waves the workspace holds partial slots for
  int32_t num_seqs, num_kv_heads, group, head_dim, block_size;
  int32_t max_blocks_per_seq, num_blocks;
  int32_t part_tiles; // 0: runs cut at any tile; else only at multiples of this many tiles
  float qk_scale;     // scale * log2(e) (* k_scale for 8-bit pools)
  float out_scale;    // v_scale for 8-bit pools (unused for 16-bit pools)
  bool bf16;          // q and out bf16 (else fp16)
  hipStream_t stream;
  // pa_decode_shared_prefix's tails: positions [start, L) only; a pair one
  // wave finishes leaves its state in pair_acc / pair_ml ([S * Hq] rows)
  // instead of writing out, and the merge is launched separately
  // (launch_prefix_merge).  0 / null / true for every other caller.
  int32_t start = 0;
  float* pair_acc = nullptr;
  float2* pair_ml = nullptr;
  bool merge = true;
};

// Waves a balanced decode launch has on the current device (two workgroups
// of four waves per CU), at most kStreamKMaxWaves; kStreamKMaxWaves when no
// device can be queried.
int streamk_device_waves();

inline int64_t streamk_gmax(int32_t num_q_heads) { return num_q_heads < 8 ? num_q_heads : 8; }
inline int64_t streamk_acc_bytes(int32_t num_q_heads, int32_t head_dim, int64_t waves) {
  return 2 * waves * streamk_gmax(num_q_heads) * head_dim * 4;
}
inline int64_t streamk_ml_bytes(int32_t num_q_heads, int64_t waves) {
  return 2 * waves * streamk_gmax(num_q_heads) * 8;
}
inline int64_t streamk_meta_bytes(int32_t num_seqs, int32_t num_q_heads) {
  return (int64_t)num_seqs * num_q_heads * 16;
}
inline int64_t streamk_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                       int64_t waves) {
  return streamk_acc_bytes(num_q_heads, head_dim, waves) + streamk_ml_bytes(num_q_heads, waves) +
         streamk_meta_bytes(num_seqs, num_q_heads);
}

hipError_t launch_decode_streamk(const StreamKArgs& a);

// pa_decode_shared_prefix (prefix.hip, decode_streamk.hip): the prefix's
// attention for every (sequence, query head) row, per chunk of
// kPrefixChunk positions, as partial states pre_acc [nchunks][S * Hq][D] and
// pre_ml [nchunks][S * Hq]; then, after the tails (launch_decode_streamk
// with start and pair buffers), the merge of prefix and tail into out.
constexpr int kPrefixChunk = 128;
struct PrefixArgs {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* seq_lens;
  float* pre_acc;
  float2* pre_ml;
  const float* ws_acc;   // the tails' split partials, as StreamKArgs
  const float2* ws_ml;
  const int4* ws_meta;
  const float* pair_acc; // the tails' whole-pair states
  const float2* pair_ml;
  int32_t num_seqs, num_kv_heads, group, head_dim, block_size;
  int32_t max_blocks_per_seq, num_blocks, prefix_blocks;
  float qk_scale;
  bool bf16;
  hipStream_t stream;
};
inline int64_t prefix_chunks(int32_t prefix_blocks, int32_t block_size) {
  return ((int64_t)prefix_blocks * block_size + kPrefixChunk - 1) / kPrefixChunk;
}
hipError_t launch_prefix_attend(const PrefixArgs& a);
hipError_t launch_prefix_merge(const PrefixArgs& a);
// The same split with the vector-unit tile wave (pa_valu.h), 16-bit pools.
hipError_t launch_decode_streamk_valu(const StreamKArgs& a);
// Gather-only run of the same split and loads (pa_probe_gather); uses only
// out (a sink word), the pools, block_tables, seq_lens and the sizes.
hipError_t launch_gather_streamk(const StreamKArgs& a);
// The same over 8-bit E4M3 pools (decode_fp8.hip): pa_decode_fp8, and the
// gather-only run on 8-bit pools.
hipError_t launch_decode_streamk_fp8(const StreamKArgs& a);
hipError_t launch_gather_streamk_fp8(const StreamKArgs& a);

// Chunked prefill (prefill.hip): one wave per (sequence, KV head, 16 query
// rows), causal within each chunk; no workspace.
struct PrefillArgs {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* seq_lens;
  const int32_t* query_start;
  int32_t num_seqs, total_q, num_kv_heads, group, head_dim, block_size;
  int32_t max_blocks_per_seq, num_blocks;
  float qk_scale;  // scale * log2(e)
  bool bf16;
  hipStream_t stream;
};
hipError_t launch_prefill(const PrefillArgs& a);
// Waves the prefill launch has (an upper bound on its units).
int64_t prefill_units(int32_t total_q, int32_t num_seqs, int32_t num_kv_heads, int32_t group);

// pa_decode_valu kernel (decode.hip); it launches the split-K merge itself
// when pmax > 1.
hipError_t launch_decode(const DecodeArgs& a);
hipError_t launch_splitk_reduce(const DecodeArgs& a);
int decode_max_partition_blocks();

hipError_t launch_reshape_and_cache(const void* key, const void* value, void* k_cache,
                                    void* v_cache, const int32_t* slot_mapping,
                                    int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                                    int32_t block_size, int32_t num_blocks, hipStream_t stream);

// Quantising append into 8-bit E4M3 pools; key/value bf16 (bf16) or fp16.
hipError_t launch_reshape_and_cache_fp8(const void* key, const void* value, void* k_cache,
                                        void* v_cache, const int32_t* slot_mapping,
                                        int32_t num_tokens, int32_t num_kv_heads,
                                        int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                        float k_scale, float v_scale, bool bf16,
                                        hipStream_t stream);

// elem_bytes: 2 for 16-bit pools, 1 for 8-bit ones.
hipError_t launch_copy_blocks(void* k_cache, void* v_cache, const int32_t* block_mapping,
                              int32_t num_pairs, int32_t num_kv_heads, int32_t head_dim,
                              int32_t block_size, int32_t num_blocks, int32_t elem_bytes,
                              hipStream_t stream);

}  // namespace pa
