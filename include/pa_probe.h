/*
 * pa_probe.h -- measurement support for libpa, not part of the method.
 *
 * pa_decode is bound by HBM: it reads each live key and value once, in 4 KiB
 * tiles (block 16, head_dim 128) scattered through the pool by the block
 * tables.  The fraction of the HBM peak such a gather can reach depends on
 * the access pattern, not only on the kernel, so the benchmark measures the
 * pattern's own ceiling (pa_probe_gather) and the peak of a plain streaming
 * read on the same device (pa_probe_stream), and reports pa_decode against
 * both as well as against the 8 TB/s peak.
 */
#ifndef PA_PROBE_H
#define PA_PROBE_H

#include "pa.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Reads exactly the K and V bytes that pa_decode with partition_size 0
 * (the balanced split) reads for these arguments, with the same grid, the
 * same per-wave walk and the same load instructions, and computes nothing:
 * no q, no scores, no output.  Arguments, layouts and validation are those
 * of pa_decode (the query and output arrays are replaced by `sink`).
 * `sink` is a caller-owned device buffer of at least 2 bytes; the call may
 * write it (only when the loaded data XOR to one particular word) and never
 * reads it.  Asynchronous on `stream`, like pa_decode.  dtype PA_FP8_E4M3
 * selects 8-bit pools and reads exactly what pa_decode_fp8 reads.
 *
 * Errors: PA_ERR_NULL, PA_ERR_SHAPE, PA_ERR_UNSUPPORTED, PA_ERR_HIP.
 */
pa_status pa_probe_gather(void* sink, const void* k_cache, const void* v_cache,
                          const int32_t* block_tables, const int32_t* seq_lens,
                          int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                          int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                          int32_t num_blocks, pa_dtype dtype, hipStream_t stream);

/*
 * pa_decode with the matrix-core tile wave at every query group.  pa_decode
 * chooses the tile wave by the group (the vector unit at group 1, where the
 * matrix cores save nothing; the matrix cores from group 2, where they do);
 * this entry point keeps the choice measurable at group 1, and is otherwise
 * pa_decode: same arguments, contract, workspace, results (to float32
 * rounding) and errors.
 */
pa_status pa_probe_decode_mfma(void* out, const void* q, const void* k_cache,
                               const void* v_cache, const int32_t* block_tables,
                               const int32_t* seq_lens, int32_t num_seqs, int32_t num_q_heads,
                               int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                               int32_t max_blocks_per_seq, int32_t num_blocks, float scale,
                               int32_t partition_size, pa_dtype dtype, void* workspace,
                               size_t workspace_bytes, hipStream_t stream);

/*
 * Reads `bytes` bytes of `buf` once, as a streaming read: every wave reads
 * 1 KiB segments (64 lanes x 16 bytes, the streaming hint), segment w, then
 * w + W, w + 2W, ... for wave w of W, eight in flight, so that the waves
 * together sweep one contiguous window of memory at a time; one workgroup
 * of four waves per CU, the shape at which such a read peaks on MI355X
 * (more bytes in flight per CU read slower).  Computes nothing.  `buf` is a caller-owned device buffer, 16-byte aligned, and
 * `bytes` a multiple of 16; it is only read.  `sink` as in pa_probe_gather.
 * Asynchronous on `stream`.  bytes = 0 is a no-op.
 *
 * Errors: PA_ERR_NULL, PA_ERR_SHAPE (misaligned buf, bytes not a multiple
 * of 16), PA_ERR_HIP.
 */
pa_status pa_probe_stream(void* sink, const void* buf, size_t bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_PROBE_H */
