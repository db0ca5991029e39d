/*
 * pa_probe.h -- measurement support for libpa, not part of the method.
 *
 * pa_decode is bound by HBM: it reads each live key and value once, in 4 KiB
 * tiles (block 16, head_dim 128) scattered through the pool by the block
 * tables.  The fraction of the HBM peak such a gather can reach depends on
 * the access pattern, not only on the kernel, so the benchmark measures the
 * pattern's own ceiling with the call below and reports pa_decode against
 * it as well as against the 8 TB/s peak.
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

#ifdef __cplusplus
}
#endif

#endif /* PA_PROBE_H */
