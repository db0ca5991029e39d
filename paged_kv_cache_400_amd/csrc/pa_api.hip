// pa_api.hip -- the C ABI declared in include/pa.h: argument validation,
// partition and workspace sizing, dispatch to the kernel launchers, and the
// thread-local error text.
#include <stdarg.h>
#include <stdio.h>

#include <mutex>

#include "pa.h"
#include "pa_probe.h"
#include "pa_launch.h"

namespace pa {
// probe_stream.hip: a streaming read of `bytes` bytes of `buf` (measurement
// support, outside the decode's launch header).
hipError_t launch_probe_stream(void* sink, const void* buf, size_t bytes, hipStream_t stream);
}  // namespace pa

namespace {

thread_local char g_last_error[512] = "";

pa_status fail(pa_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return st;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Status of a launcher's result: a kernel whose resources do not fit the
// device (pa::kErrDoesNotFit) is PA_ERR_UNSUPPORTED, any other failure
// PA_ERR_HIP.
pa_status launch_status(const char* fn, hipError_t e) {
  if (e == hipSuccess) return PA_OK;
  if (e == pa::kErrDoesNotFit)
    return fail(PA_ERR_UNSUPPORTED,
                "%s: the kernel's LDS or register needs do not fit one workgroup on this device",
                fn);
  return fail(PA_ERR_HIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
}

constexpr int32_t kAutoPartition = 512;
constexpr int64_t kMaxThreadsPerLaunch = (int64_t)1 << 32;

// Partition size actually used; 0 if partition_size is invalid.  Partitions
// start at multiples of 16 positions (the decode kernels' tile) and of the
// block size.
int32_t resolve_partition(int32_t partition_size, int32_t block_size) {
  const int32_t p = partition_size == 0 ? kAutoPartition : partition_size;
  if (p <= 0 || block_size <= 0 || p % block_size != 0 || p % 16 != 0) return 0;
  if (p / block_size > pa::decode_max_partition_blocks()) return 0;
  return p;
}

int64_t partitions_needed(int32_t max_blocks_per_seq, int32_t block_size, int32_t part) {
  const int64_t max_len = (int64_t)max_blocks_per_seq * block_size;
  return (max_len + part - 1) / part;
}

// Workspace of the fixed partitions of pa_decode_valu: (m, l, acc) per
// (sequence, query head, partition); 0 when no sequence can need more than one partition or
// the partition size is invalid.
size_t partitioned_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                   int32_t max_blocks_per_seq, int32_t block_size,
                                   int32_t partition_size) {
  const int32_t part = resolve_partition(partition_size, block_size);
  if (part == 0) return 0;
  const int64_t pmax = partitions_needed(max_blocks_per_seq, block_size, part);
  if (pmax <= 1) return 0;
  const int64_t rows = (int64_t)num_seqs * num_q_heads * pmax;
  return (size_t)(rows * head_dim * (int64_t)sizeof(float) + rows * 2 * (int64_t)sizeof(float));
}

bool supported_cache_dims(int32_t head_dim, int32_t block_size) {
  return head_dim >= 8 && head_dim <= 1024 && head_dim % 8 == 0 &&
         (block_size == 8 || block_size == 16 || block_size == 32);
}

}  // namespace

extern "C" {

const char* pa_status_string(pa_status status) {
  switch (status) {
    case PA_OK: return "PA_OK";
    case PA_ERR_NULL: return "PA_ERR_NULL";
    case PA_ERR_SHAPE: return "PA_ERR_SHAPE";
    case PA_ERR_UNSUPPORTED: return "PA_ERR_UNSUPPORTED";
    case PA_ERR_WORKSPACE: return "PA_ERR_WORKSPACE";
    case PA_ERR_HIP: return "PA_ERR_HIP";
    case PA_ERR_NO_BLOCKS: return "PA_ERR_NO_BLOCKS";
  }
  return "PA_ERR_UNKNOWN";
}

const char* pa_last_error(void) { return g_last_error; }

int32_t pa_abi_version(void) { return PA_ABI_VERSION; }

size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                 int32_t max_blocks_per_seq, int32_t block_size,
                                 int32_t partition_size) {
  if (num_seqs <= 0 || num_q_heads <= 0 || head_dim <= 0 || max_blocks_per_seq <= 0 ||
      resolve_partition(partition_size, block_size) == 0)
    return 0;
  // pa_decode runs the balanced split (partition-aligned runs when
  // partition_size > 0), and so does pa_decode_valu when partition_size is
  // 0; pa_decode_valu with partition_size > 0 runs fixed partitions.  The
  // workspace serves either entry point.
  const size_t part_bytes =
      partition_size > 0 ? partitioned_workspace_bytes(num_seqs, num_q_heads, head_dim,
                                                       max_blocks_per_seq, block_size,
                                                       partition_size)
                         : 0;
  const size_t sk = (size_t)pa::streamk_workspace_bytes(num_seqs, num_q_heads, head_dim,
                                                        pa::streamk_device_waves());
  return sk > part_bytes ? sk : part_bytes;
}

}  // extern "C"

namespace {

// kAuto: pa_decode, the balanced split with the tile wave chosen by the
// query group (the vector unit at group 1, the matrix cores above; measured
// on the mixed step: at group 1 the vector unit is 1-2% faster, at groups 2,
// 4 and 8 it takes 2%, 9% and 54% longer).  kMfma: the matrix-core tile
// wave at every group (pa_probe_decode_mfma).  kValu: pa_decode_valu.
enum class Impl { kAuto, kMfma, kValu };

bool positive_finite(float x) { return x > 0.0f && x <= 3.4028234663852886e38f; }

// ---- the static scratch of pa_decode_noalloc ------------------------------
// The balanced decode's partial states and pair records, for callers that
// cannot allocate.  Each GPU the library runs on holds its own copy of this
// array until the process ends.  In host code `scratch` names a host-side
// stand-in, not a device address: the device address comes from
// hipGetSymbolAddress, once per device with that device current, and only
// that address is ever handed to a kernel.
constexpr size_t kScratchBytes = (size_t)24 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mutex;
void* g_scratch_ptr[pa::kMaxDevices];  // device address of `scratch`, per device

// The current device's address of `scratch` (looked up on the first call on
// that device).
pa_status static_scratch(const char* fn, void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(PA_ERR_HIP, "%s: no current device: %s", fn, hipGetErrorString(e));
  if (dev < 0 || dev >= pa::kMaxDevices)
    return fail(PA_ERR_UNSUPPORTED, "%s: device %d beyond the %d the library serves", fn, dev,
                pa::kMaxDevices);
  void* p = __atomic_load_n(&g_scratch_ptr[dev], __ATOMIC_ACQUIRE);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    p = g_scratch_ptr[dev];
    if (p == nullptr) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || p == nullptr)
        return fail(PA_ERR_HIP, "%s: the static scratch has no address on device %d: %s", fn,
                    dev, hipGetErrorString(e));
      __atomic_store_n(&g_scratch_ptr[dev], p, __ATOMIC_RELEASE);
    }
  }
  *ptr = p;
  return PA_OK;
}

// kv_fp8: 8-bit E4M3 pools with scales k_scale / v_scale (pa_decode_fp8;
// balanced split only).
pa_status decode_impl(Impl impl, void* out, const void* q, const void* k_cache,
                      const void* v_cache, const int32_t* block_tables, const int32_t* seq_lens,
                      int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                      int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                      int32_t num_blocks, float scale, int32_t partition_size, pa_dtype dtype,
                      void* workspace, size_t workspace_bytes, hipStream_t stream,
                      bool kv_fp8 = false, float k_scale = 1.0f, float v_scale = 1.0f,
                      bool use_static_scratch = false) {
  g_last_error[0] = '\0';
  if (kv_fp8 && (!positive_finite(k_scale) || !positive_finite(v_scale)))
    return fail(PA_ERR_SHAPE, "pa_decode_fp8: k_scale %g and v_scale %g must be positive and "
                "finite", (double)k_scale, (double)v_scale);
  if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      block_size <= 0 || max_blocks_per_seq <= 0 || num_blocks <= 0)
    return fail(PA_ERR_SHAPE,
                "pa_decode: sizes must be positive (num_seqs >= 0): S=%d Hq=%d Hkv=%d d=%d "
                "bs=%d MB=%d NB=%d",
                num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                num_blocks);
  if (dtype != PA_F16 && dtype != PA_BF16)
    return fail(PA_ERR_UNSUPPORTED, "pa_decode: dtype %d is not PA_F16 or PA_BF16", (int)dtype);
  if (head_dim != 64 && head_dim != 128)
    return fail(PA_ERR_UNSUPPORTED, "pa_decode: head_dim %d not in {64, 128}", head_dim);
  if (block_size != 8 && block_size != 16 && block_size != 32)
    return fail(PA_ERR_UNSUPPORTED, "pa_decode: block_size %d not in {8, 16, 32}", block_size);
  if (num_q_heads % num_kv_heads != 0)
    return fail(PA_ERR_SHAPE, "pa_decode: num_q_heads %d is not a multiple of num_kv_heads %d",
                num_q_heads, num_kv_heads);
  const int32_t group = num_q_heads / num_kv_heads;
  if (group != 1 && group != 2 && group != 4 && group != 8)
    return fail(PA_ERR_UNSUPPORTED, "pa_decode: query group %d not in {1, 2, 4, 8}", group);
  const int32_t part = resolve_partition(partition_size, block_size);
  if (part == 0)
    return fail(PA_ERR_SHAPE,
                "pa_decode: partition_size %d must be 0 or a positive multiple of 16 and of "
                "block_size %d, with at most %d blocks",
                partition_size, block_size, pa::decode_max_partition_blocks());
  if (num_seqs == 0) return PA_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !seq_lens)
    return fail(PA_ERR_NULL, "pa_decode: a required pointer is NULL");
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache))
    return fail(PA_ERR_SHAPE, "pa_decode: out, q, k_cache and v_cache must be 16-byte aligned");
  const int64_t pmax = partitions_needed(max_blocks_per_seq, block_size, part);
  const int64_t units = (int64_t)num_seqs * num_kv_heads * pmax;
  if (units * 256 >= kMaxThreadsPerLaunch || pmax > INT32_MAX)
    return fail(PA_ERR_SHAPE, "pa_decode: %lld work units exceed one launch",
                (long long)units);
  // the balanced split: pa_decode always, pa_decode_valu with partition_size 0
  const bool balanced = impl != Impl::kValu || partition_size == 0;
  const int waves = pa::streamk_device_waves();
  const size_t need =
      balanced ? (size_t)pa::streamk_workspace_bytes(num_seqs, num_q_heads, head_dim, waves)
               : partitioned_workspace_bytes(num_seqs, num_q_heads, head_dim, max_blocks_per_seq,
                                             block_size, partition_size);
  if (use_static_scratch) {  // pa_decode_noalloc: the scratch replaces the workspace
    if (need > kScratchBytes)
      return fail(PA_ERR_WORKSPACE,
                  "pa_decode_noalloc: these sizes need %zu bytes of scratch (the partial states "
                  "of %d waves at head_dim %d, plus 16 bytes per (sequence, query head)); the "
                  "library's static scratch holds %zu",
                  need, waves, head_dim, kScratchBytes);
    const pa_status st = static_scratch("pa_decode_noalloc", &workspace);
    if (st != PA_OK) return st;
    workspace_bytes = kScratchBytes;
  }
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(PA_ERR_WORKSPACE, "pa_decode: workspace of %zu bytes needed, %zu given%s", need,
                workspace_bytes, workspace ? "" : " (NULL)");
  if (need > 0 && !aligned16(workspace))
    return fail(PA_ERR_SHAPE, "pa_decode: workspace must be 16-byte aligned");

  if (balanced) {
    pa::StreamKArgs a;
    a.out = out;
    a.q = q;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.block_tables = block_tables;
    a.seq_lens = seq_lens;
    char* ws = (char*)workspace;
    a.ws_acc = (float*)ws;
    a.ws_ml = (float2*)(ws + pa::streamk_acc_bytes(num_q_heads, head_dim, waves));
    a.ws_meta = (int4*)(ws + pa::streamk_acc_bytes(num_q_heads, head_dim, waves) +
                        pa::streamk_ml_bytes(num_q_heads, waves));
    a.max_waves = waves;
    a.num_seqs = num_seqs;
    a.num_kv_heads = num_kv_heads;
    a.group = group;
    a.head_dim = head_dim;
    a.block_size = block_size;
    a.max_blocks_per_seq = max_blocks_per_seq;
    a.num_blocks = num_blocks;
    a.part_tiles = partition_size / 16;  // 16-position tiles (the 16-bit decode's)
    a.qk_scale = scale * 1.4426950408889634f * (kv_fp8 ? k_scale : 1.0f);
    a.out_scale = v_scale;
    a.bf16 = dtype == PA_BF16;
    a.stream = stream;
    if (kv_fp8) return launch_status("pa_decode_fp8", pa::launch_decode_streamk_fp8(a));
    if (impl == Impl::kValu || (impl == Impl::kAuto && group == 1))
      return launch_status(impl == Impl::kValu ? "pa_decode_valu" : "pa_decode",
                           pa::launch_decode_streamk_valu(a));
    return launch_status(impl == Impl::kMfma ? "pa_probe_decode_mfma" : "pa_decode",
                         pa::launch_decode_streamk(a));
  }

  pa::DecodeArgs a;
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.seq_lens = seq_lens;
  const int64_t rows = (int64_t)num_seqs * num_q_heads * pmax;
  a.ws_acc = need ? (float*)workspace : nullptr;
  a.ws_ml = need ? (float2*)((char*)workspace + rows * head_dim * sizeof(float)) : nullptr;
  a.num_seqs = num_seqs;
  a.num_kv_heads = num_kv_heads;
  a.group = group;
  a.head_dim = head_dim;
  a.block_size = block_size;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_blocks = num_blocks;
  a.part = part;
  a.pmax = (int32_t)pmax;
  a.qk_scale = scale * 1.4426950408889634f;
  a.bf16 = dtype == PA_BF16;
  a.stream = stream;
  return launch_status("pa_decode_valu", pa::launch_decode(a));
}

}  // namespace

extern "C" {

pa_status pa_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
                    const int32_t* block_tables, const int32_t* seq_lens, int32_t num_seqs,
                    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                    int32_t block_size, int32_t max_blocks_per_seq, int32_t num_blocks,
                    float scale, int32_t partition_size, pa_dtype dtype, void* workspace,
                    size_t workspace_bytes, hipStream_t stream) {
  return decode_impl(Impl::kAuto, out, q, k_cache, v_cache, block_tables, seq_lens, num_seqs,
                     num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                     num_blocks, scale, partition_size, dtype, workspace, workspace_bytes,
                     stream);
}

pa_status pa_decode_noalloc(void* out, const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* block_tables, const int32_t* seq_lens,
                            int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                            int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                            int32_t num_blocks, float scale, int32_t partition_size,
                            pa_dtype dtype, hipStream_t stream) {
  return decode_impl(Impl::kAuto, out, q, k_cache, v_cache, block_tables, seq_lens, num_seqs,
                     num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                     num_blocks, scale, partition_size, dtype, nullptr, 0, stream, false, 1.0f,
                     1.0f, true);
}

size_t pa_decode_shared_prefix_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                               int32_t head_dim, int32_t prefix_blocks,
                                               int32_t block_size) {
  if (num_seqs <= 0 || num_q_heads <= 0 || head_dim <= 0 || prefix_blocks < 0 ||
      block_size <= 0)
    return 0;
  const int64_t rows = (int64_t)num_seqs * num_q_heads;
  const int64_t sk = pa::streamk_workspace_bytes(num_seqs, num_q_heads, head_dim,
                                                 pa::streamk_device_waves());
  if (prefix_blocks == 0) return (size_t)sk;
  const int64_t nch = pa::prefix_chunks(prefix_blocks, block_size);
  return (size_t)(sk + (1 + nch) * rows * ((int64_t)head_dim * 4 + 8));
}

pa_status pa_decode_shared_prefix(void* out, const void* q, const void* k_cache,
                                  const void* v_cache, const int32_t* block_tables,
                                  const int32_t* seq_lens, int32_t num_seqs,
                                  int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                  int32_t block_size, int32_t max_blocks_per_seq,
                                  int32_t num_blocks, int32_t prefix_blocks, float scale,
                                  pa_dtype dtype, void* workspace, size_t workspace_bytes,
                                  hipStream_t stream) {
  g_last_error[0] = '\0';
  if (prefix_blocks < 0 || (max_blocks_per_seq > 0 && prefix_blocks > max_blocks_per_seq))
    return fail(PA_ERR_SHAPE,
                "pa_decode_shared_prefix: prefix_blocks %d must be in [0, max_blocks_per_seq %d]",
                prefix_blocks, max_blocks_per_seq);
  if (prefix_blocks == 0)  // nothing shared: the plain decode
    return decode_impl(Impl::kAuto, out, q, k_cache, v_cache, block_tables, seq_lens, num_seqs,
                       num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                       num_blocks, scale, 0, dtype, workspace, workspace_bytes, stream);
  // the same validation as pa_decode, with no work launched: a zero-sized call
  const pa_status st = decode_impl(Impl::kAuto, nullptr, nullptr, nullptr, nullptr, nullptr,
                                   nullptr, 0, num_q_heads, num_kv_heads, head_dim, block_size,
                                   max_blocks_per_seq, num_blocks, scale, 0, dtype, nullptr, 0,
                                   stream);
  if (st != PA_OK || num_seqs == 0) return st;
  if (num_seqs < 0)
    return fail(PA_ERR_SHAPE, "pa_decode_shared_prefix: num_seqs %d is negative", num_seqs);
  if (!out || !q || !k_cache || !v_cache || !block_tables || !seq_lens)
    return fail(PA_ERR_NULL, "pa_decode_shared_prefix: a required pointer is NULL");
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache))
    return fail(PA_ERR_SHAPE,
                "pa_decode_shared_prefix: out, q, k_cache and v_cache must be 16-byte aligned");
  const int32_t group = num_q_heads / num_kv_heads;
  const int64_t rows = (int64_t)num_seqs * num_q_heads;
  const int64_t nch = pa::prefix_chunks(prefix_blocks, block_size);
  const int64_t prefix_waves = (int64_t)num_kv_heads * ((rows / num_kv_heads + 15) / 16) * nch;
  if (prefix_waves * 64 >= kMaxThreadsPerLaunch || (int64_t)num_seqs * num_kv_heads >= INT32_MAX)
    return fail(PA_ERR_SHAPE, "pa_decode_shared_prefix: too many rows for one launch");
  const size_t need = pa_decode_shared_prefix_workspace_bytes(num_seqs, num_q_heads, head_dim,
                                                             prefix_blocks, block_size);
  if (!workspace || workspace_bytes < need)
    return fail(PA_ERR_WORKSPACE, "pa_decode_shared_prefix: workspace of %zu bytes needed, %zu "
                "given%s", need, workspace_bytes, workspace ? "" : " (NULL)");
  if (!aligned16(workspace))
    return fail(PA_ERR_SHAPE, "pa_decode_shared_prefix: workspace must be 16-byte aligned");

  // workspace: the balanced split's (acc, ml, records), then the tails'
  // whole-pair states (acc, ml), then the prefix's chunk partials (acc, ml)
  const int waves = pa::streamk_device_waves();
  char* ws = (char*)workspace;
  pa::StreamKArgs a;
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.seq_lens = seq_lens;
  a.ws_acc = (float*)ws;
  a.ws_ml = (float2*)(ws + pa::streamk_acc_bytes(num_q_heads, head_dim, waves));
  a.ws_meta = (int4*)(ws + pa::streamk_acc_bytes(num_q_heads, head_dim, waves) +
                      pa::streamk_ml_bytes(num_q_heads, waves));
  a.max_waves = waves;
  a.num_seqs = num_seqs;
  a.num_kv_heads = num_kv_heads;
  a.group = group;
  a.head_dim = head_dim;
  a.block_size = block_size;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_blocks = num_blocks;
  a.part_tiles = 0;
  a.qk_scale = scale * 1.4426950408889634f;
  a.out_scale = 1.0f;
  a.bf16 = dtype == PA_BF16;
  a.stream = stream;
  char* p = ws + pa::streamk_workspace_bytes(num_seqs, num_q_heads, head_dim, waves);
  a.pair_acc = (float*)p;
  p += rows * head_dim * 4;
  a.pair_ml = (float2*)p;
  p += rows * 8;
  a.start = prefix_blocks * block_size;
  a.merge = false;

  pa::PrefixArgs b;
  b.out = out;
  b.q = q;
  b.k_cache = k_cache;
  b.v_cache = v_cache;
  b.block_tables = block_tables;
  b.seq_lens = seq_lens;
  b.pre_acc = (float*)p;
  p += nch * rows * head_dim * 4;
  b.pre_ml = (float2*)p;
  b.ws_acc = a.ws_acc;
  b.ws_ml = a.ws_ml;
  b.ws_meta = a.ws_meta;
  b.pair_acc = a.pair_acc;
  b.pair_ml = a.pair_ml;
  b.num_seqs = num_seqs;
  b.num_kv_heads = num_kv_heads;
  b.group = group;
  b.head_dim = head_dim;
  b.block_size = block_size;
  b.max_blocks_per_seq = max_blocks_per_seq;
  b.num_blocks = num_blocks;
  b.prefix_blocks = prefix_blocks;
  b.qk_scale = a.qk_scale;
  b.bf16 = a.bf16;
  b.stream = stream;

  const char* fn = "pa_decode_shared_prefix";
  pa_status r = launch_status(fn, pa::launch_prefix_attend(b));
  if (r != PA_OK) return r;
  r = launch_status(fn, group == 1 ? pa::launch_decode_streamk_valu(a)
                                   : pa::launch_decode_streamk(a));
  if (r != PA_OK) return r;
  return launch_status(fn, pa::launch_prefix_merge(b));
}

pa_status pa_decode_valu(void* out, const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* block_tables, const int32_t* seq_lens, int32_t num_seqs,
                         int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                         int32_t block_size, int32_t max_blocks_per_seq, int32_t num_blocks,
                         float scale, int32_t partition_size, pa_dtype dtype, void* workspace,
                         size_t workspace_bytes, hipStream_t stream) {
  return decode_impl(Impl::kValu, out, q, k_cache, v_cache, block_tables, seq_lens, num_seqs,
                     num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                     num_blocks, scale, partition_size, dtype, workspace, workspace_bytes,
                     stream);
}

pa_status pa_decode_fp8(void* out, const void* q, const void* k_cache, const void* v_cache,
                        const int32_t* block_tables, const int32_t* seq_lens, int32_t num_seqs,
                        int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                        int32_t block_size, int32_t max_blocks_per_seq, int32_t num_blocks,
                        float scale, float k_scale, float v_scale, pa_dtype dtype,
                        void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return decode_impl(Impl::kAuto, out, q, k_cache, v_cache, block_tables, seq_lens, num_seqs,
                     num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                     num_blocks, scale, 0, dtype, workspace, workspace_bytes, stream, true,
                     k_scale, v_scale);
}

pa_status pa_reshape_and_cache_fp8(const void* key, const void* value, void* k_cache,
                                   void* v_cache, const int32_t* slot_mapping,
                                   int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                                   int32_t block_size, int32_t num_blocks, float k_scale,
                                   float v_scale, pa_dtype dtype, hipStream_t stream) {
  g_last_error[0] = '\0';
  if (num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
      num_blocks <= 0)
    return fail(PA_ERR_SHAPE,
                "pa_reshape_and_cache_fp8: sizes must be positive (num_tokens >= 0): T=%d "
                "Hkv=%d d=%d bs=%d NB=%d",
                num_tokens, num_kv_heads, head_dim, block_size, num_blocks);
  if (dtype != PA_F16 && dtype != PA_BF16)
    return fail(PA_ERR_UNSUPPORTED, "pa_reshape_and_cache_fp8: dtype %d is not PA_F16 or "
                "PA_BF16", (int)dtype);
  if (!supported_cache_dims(head_dim, block_size) || head_dim % 16 != 0)
    return fail(PA_ERR_UNSUPPORTED,
                "pa_reshape_and_cache_fp8: head_dim %d (multiple of 16 in [16, 1024]) or "
                "block_size %d (8, 16, 32) not supported",
                head_dim, block_size);
  if (!positive_finite(k_scale) || !positive_finite(v_scale))
    return fail(PA_ERR_SHAPE, "pa_reshape_and_cache_fp8: k_scale %g and v_scale %g must be "
                "positive and finite", (double)k_scale, (double)v_scale);
  if (num_tokens == 0) return PA_OK;
  if (!key || !value || !k_cache || !v_cache || !slot_mapping)
    return fail(PA_ERR_NULL, "pa_reshape_and_cache_fp8: a required pointer is NULL");
  if (!aligned16(key) || !aligned16(value) || !aligned16(k_cache) || !aligned16(v_cache))
    return fail(PA_ERR_SHAPE,
                "pa_reshape_and_cache_fp8: key, value and pools must be 16-byte aligned");
  const int64_t total = (int64_t)num_tokens * num_kv_heads * (head_dim / 16);
  if (total + 255 >= kMaxThreadsPerLaunch)
    return fail(PA_ERR_SHAPE, "pa_reshape_and_cache_fp8: too many tokens for one launch");
  return launch_status("pa_reshape_and_cache_fp8",
                       pa::launch_reshape_and_cache_fp8(
                           key, value, k_cache, v_cache, slot_mapping, num_tokens, num_kv_heads,
                           head_dim, block_size, num_blocks, k_scale, v_scale, dtype == PA_BF16,
                           stream));
}

pa_status pa_prefill(void* out, const void* q, const void* k_cache, const void* v_cache,
                     const int32_t* block_tables, const int32_t* seq_lens,
                     const int32_t* query_start, int32_t num_seqs, int32_t total_q,
                     int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                     int32_t block_size, int32_t max_blocks_per_seq, int32_t num_blocks,
                     float scale, pa_dtype dtype, hipStream_t stream) {
  g_last_error[0] = '\0';
  if (num_seqs < 0 || total_q < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      block_size <= 0 || max_blocks_per_seq <= 0 || num_blocks <= 0)
    return fail(PA_ERR_SHAPE,
                "pa_prefill: sizes must be positive (num_seqs, total_q >= 0): S=%d T=%d Hq=%d "
                "Hkv=%d d=%d bs=%d MB=%d NB=%d",
                num_seqs, total_q, num_q_heads, num_kv_heads, head_dim, block_size,
                max_blocks_per_seq, num_blocks);
  if (dtype != PA_F16 && dtype != PA_BF16)
    return fail(PA_ERR_UNSUPPORTED, "pa_prefill: dtype %d is not PA_F16 or PA_BF16", (int)dtype);
  if (head_dim != 64 && head_dim != 128)
    return fail(PA_ERR_UNSUPPORTED, "pa_prefill: head_dim %d not in {64, 128}", head_dim);
  if (block_size != 8 && block_size != 16 && block_size != 32)
    return fail(PA_ERR_UNSUPPORTED, "pa_prefill: block_size %d not in {8, 16, 32}", block_size);
  if (num_q_heads % num_kv_heads != 0)
    return fail(PA_ERR_SHAPE, "pa_prefill: num_q_heads %d is not a multiple of num_kv_heads %d",
                num_q_heads, num_kv_heads);
  const int32_t group = num_q_heads / num_kv_heads;
  if (group != 1 && group != 2 && group != 4 && group != 8)
    return fail(PA_ERR_UNSUPPORTED, "pa_prefill: query group %d not in {1, 2, 4, 8}", group);
  if (num_seqs == 0 || total_q == 0) return PA_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !seq_lens || !query_start)
    return fail(PA_ERR_NULL, "pa_prefill: a required pointer is NULL");
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache))
    return fail(PA_ERR_SHAPE, "pa_prefill: out, q, k_cache and v_cache must be 16-byte aligned");
  const int64_t units = pa::prefill_units(total_q, num_seqs, num_kv_heads, group);
  if (units * 64 >= kMaxThreadsPerLaunch)
    return fail(PA_ERR_SHAPE, "pa_prefill: %lld work units exceed one launch", (long long)units);
  pa::PrefillArgs a;
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.seq_lens = seq_lens;
  a.query_start = query_start;
  a.num_seqs = num_seqs;
  a.total_q = total_q;
  a.num_kv_heads = num_kv_heads;
  a.group = group;
  a.head_dim = head_dim;
  a.block_size = block_size;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_blocks = num_blocks;
  a.qk_scale = scale * 1.4426950408889634f;
  a.bf16 = dtype == PA_BF16;
  a.stream = stream;
  return launch_status("pa_prefill", pa::launch_prefill(a));
}

pa_status pa_reshape_and_cache(const void* key, const void* value, void* k_cache,
                               void* v_cache, const int32_t* slot_mapping, int32_t num_tokens,
                               int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                               int32_t num_blocks, pa_dtype dtype, hipStream_t stream) {
  g_last_error[0] = '\0';
  if (num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
      num_blocks <= 0)
    return fail(PA_ERR_SHAPE,
                "pa_reshape_and_cache: sizes must be positive (num_tokens >= 0): T=%d Hkv=%d "
                "d=%d bs=%d NB=%d",
                num_tokens, num_kv_heads, head_dim, block_size, num_blocks);
  if (dtype != PA_F16 && dtype != PA_BF16)
    return fail(PA_ERR_UNSUPPORTED, "pa_reshape_and_cache: dtype %d not supported", (int)dtype);
  if (!supported_cache_dims(head_dim, block_size))
    return fail(PA_ERR_UNSUPPORTED,
                "pa_reshape_and_cache: head_dim %d (multiple of 8 in [8, 1024]) or block_size "
                "%d (8, 16, 32) not supported",
                head_dim, block_size);
  if (num_tokens == 0) return PA_OK;
  if (!key || !value || !k_cache || !v_cache || !slot_mapping)
    return fail(PA_ERR_NULL, "pa_reshape_and_cache: a required pointer is NULL");
  if (!aligned16(key) || !aligned16(value) || !aligned16(k_cache) || !aligned16(v_cache))
    return fail(PA_ERR_SHAPE, "pa_reshape_and_cache: key, value and pools must be 16-byte aligned");
  const int64_t total = (int64_t)num_tokens * num_kv_heads * (head_dim / 8);
  if (total + 255 >= kMaxThreadsPerLaunch)
    return fail(PA_ERR_SHAPE, "pa_reshape_and_cache: too many tokens for one launch");
  return launch_status("pa_reshape_and_cache",
                       pa::launch_reshape_and_cache(key, value, k_cache, v_cache, slot_mapping,
                                                    num_tokens, num_kv_heads, head_dim,
                                                    block_size, num_blocks, stream));
}

pa_status pa_copy_blocks(void* k_cache, void* v_cache, const int32_t* block_mapping,
                         int32_t num_pairs, int32_t num_kv_heads, int32_t head_dim,
                         int32_t block_size, int32_t num_blocks, pa_dtype dtype,
                         hipStream_t stream) {
  g_last_error[0] = '\0';
  if (num_pairs < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
      num_blocks <= 0)
    return fail(PA_ERR_SHAPE,
                "pa_copy_blocks: sizes must be positive (num_pairs >= 0): n=%d Hkv=%d d=%d "
                "bs=%d NB=%d",
                num_pairs, num_kv_heads, head_dim, block_size, num_blocks);
  if (dtype != PA_F16 && dtype != PA_BF16 && dtype != PA_FP8_E4M3)
    return fail(PA_ERR_UNSUPPORTED, "pa_copy_blocks: dtype %d not supported", (int)dtype);
  if (!supported_cache_dims(head_dim, block_size) ||
      (dtype == PA_FP8_E4M3 && head_dim % 16 != 0))
    return fail(PA_ERR_UNSUPPORTED,
                "pa_copy_blocks: head_dim %d (multiple of 8 in [8, 1024], of 16 for 8-bit "
                "pools) or block_size %d (8, 16, 32) not supported",
                head_dim, block_size);
  if (num_pairs == 0) return PA_OK;
  if (!k_cache || !v_cache || !block_mapping)
    return fail(PA_ERR_NULL, "pa_copy_blocks: a required pointer is NULL");
  if (!aligned16(k_cache) || !aligned16(v_cache))
    return fail(PA_ERR_SHAPE, "pa_copy_blocks: pools must be 16-byte aligned");
  return launch_status("pa_copy_blocks",
                       pa::launch_copy_blocks(k_cache, v_cache, block_mapping, num_pairs,
                                              num_kv_heads, head_dim, block_size, num_blocks,
                                              dtype == PA_FP8_E4M3 ? 1 : 2, stream));
}

pa_status pa_probe_decode_mfma(void* out, const void* q, const void* k_cache,
                               const void* v_cache, const int32_t* block_tables,
                               const int32_t* seq_lens, int32_t num_seqs, int32_t num_q_heads,
                               int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                               int32_t max_blocks_per_seq, int32_t num_blocks, float scale,
                               int32_t partition_size, pa_dtype dtype, void* workspace,
                               size_t workspace_bytes, hipStream_t stream) {
  return decode_impl(Impl::kMfma, out, q, k_cache, v_cache, block_tables, seq_lens, num_seqs,
                     num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                     num_blocks, scale, partition_size, dtype, workspace, workspace_bytes,
                     stream);
}

pa_status pa_probe_stream(void* sink, const void* buf, size_t bytes, hipStream_t stream) {
  g_last_error[0] = '\0';
  if (bytes == 0) return PA_OK;
  if (!sink || !buf) return fail(PA_ERR_NULL, "pa_probe_stream: a required pointer is NULL");
  if (!aligned16(buf) || bytes % 16 != 0)
    return fail(PA_ERR_SHAPE, "pa_probe_stream: buf must be 16-byte aligned and bytes (%zu) a "
                "multiple of 16", bytes);
  return launch_status("pa_probe_stream", pa::launch_probe_stream(sink, buf, bytes, stream));
}

pa_status pa_probe_gather(void* sink, const void* k_cache, const void* v_cache,
                          const int32_t* block_tables, const int32_t* seq_lens,
                          int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                          int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                          int32_t num_blocks, pa_dtype dtype, hipStream_t stream) {
  g_last_error[0] = '\0';
  if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      block_size <= 0 || max_blocks_per_seq <= 0 || num_blocks <= 0)
    return fail(PA_ERR_SHAPE, "pa_probe_gather: sizes must be positive (num_seqs >= 0)");
  if (dtype != PA_F16 && dtype != PA_BF16 && dtype != PA_FP8_E4M3)
    return fail(PA_ERR_UNSUPPORTED, "pa_probe_gather: dtype %d not supported", (int)dtype);
  if ((head_dim != 64 && head_dim != 128) ||
      (block_size != 8 && block_size != 16 && block_size != 32))
    return fail(PA_ERR_UNSUPPORTED, "pa_probe_gather: head_dim %d or block_size %d not built",
                head_dim, block_size);
  if (num_q_heads % num_kv_heads != 0)
    return fail(PA_ERR_SHAPE, "pa_probe_gather: num_q_heads %d is not a multiple of %d",
                num_q_heads, num_kv_heads);
  const int32_t group = num_q_heads / num_kv_heads;
  if (group != 1 && group != 2 && group != 4 && group != 8)
    return fail(PA_ERR_UNSUPPORTED, "pa_probe_gather: query group %d not in {1, 2, 4, 8}",
                group);
  if (num_seqs == 0) return PA_OK;
  if (!sink || !k_cache || !v_cache || !block_tables || !seq_lens)
    return fail(PA_ERR_NULL, "pa_probe_gather: a required pointer is NULL");
  if (!aligned16(k_cache) || !aligned16(v_cache))
    return fail(PA_ERR_SHAPE, "pa_probe_gather: k_cache and v_cache must be 16-byte aligned");
  pa::StreamKArgs a = {};
  a.out = sink;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.seq_lens = seq_lens;
  a.num_seqs = num_seqs;
  a.num_kv_heads = num_kv_heads;
  a.group = group;
  a.head_dim = head_dim;
  a.block_size = block_size;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_blocks = num_blocks;
  a.bf16 = dtype == PA_BF16;
  a.stream = stream;
  return launch_status("pa_probe_gather", dtype == PA_FP8_E4M3
                                                ? pa::launch_gather_streamk_fp8(a)
                                                : pa::launch_gather_streamk(a));
}

}  // extern "C"
