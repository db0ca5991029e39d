/*
 * pa.h -- C ABI of libpa: decode attention over a paged KV cache on AMD
 * Instinct MI355X (gfx950).
 *
 * The operations are the ones the PagedAttention pages describe:
 *   - "What problem does PagedAttention solve, and what is continuous
 *     batching?" (datarekha), section "How PagedAttention works": KV stored
 *     in fixed-size blocks of a shared pool; a per-request block table maps
 *     logical block number to physical block; the attention kernel follows
 *     the table when it reads keys and values; blocks may be shared and a
 *     diverging candidate gets a private copy (copy-on-write);
 *   - same page, "Why the KV cache becomes the problem": each decode step
 *     reads the stored keys/values and appends a little new data;
 *   - "Continuous Batching & Paged Attention" (topicspectrum), sections
 *     "Attention needs memory that grows with the conversation" (attention
 *     of the current position against the cached keys/values) and "Paged
 *     attention borrows a trick from operating systems" (a growing request
 *     attaches another block).
 *
 * Layouts (all row-major, contiguous, on one GPU, 16-byte aligned):
 *   q, out          [num_seqs][num_q_heads][head_dim]
 *   k_cache/v_cache [num_blocks][num_kv_heads][block_size][head_dim]
 *   block_tables    int32 [num_seqs][max_blocks_per_seq]
 *   seq_lens        int32 [num_seqs]
 *   key/value       [num_tokens][num_kv_heads][head_dim]
 *   slot_mapping    int32 [num_tokens]
 *   block_mapping   int32 [num_pairs][2]  (src, dst)
 * Position t of sequence s lives in physical block block_tables[s][t / bs]
 * at offset t % bs; its flat slot is block * bs + t % bs.  Query head h
 * reads KV head h / (num_q_heads / num_kv_heads).
 *
 * Conventions:
 *   - Ownership: the caller owns every buffer.  The library allocates
 *     nothing and keeps no per-call state; scratch comes from `workspace`.
 *   - Execution: every call only enqueues work on `stream` and returns; it
 *     never synchronises.  All array pointers are device pointers.
 *   - Errors: a non-PA_OK status means nothing was enqueued (except
 *     PA_ERR_HIP, a failed launch).  pa_last_error() gives the calling
 *     thread's message for its last failed call.  Every call checks, before
 *     launching, that its kernels' LDS fits one workgroup on the current
 *     device, and answers PA_ERR_UNSUPPORTED if it does not.
 *   - Device: calls run on the current HIP device; `stream` must belong to
 *     it.
 *   - Only host-visible arguments are validated.  Device-side contents that
 *     break the contract (a block id outside [0, num_blocks), a sequence
 *     longer than its table, a slot outside the pool) are never
 *     dereferenced: decode writes NaN rows for that sequence, the append
 *     and the copy skip that entry.
 *   - Zero-sized work (num_seqs, num_tokens or num_pairs == 0) is a no-op.
 *   - Thread safety: no global mutable state beyond the thread-local error
 *     text.  Calls that touch the same buffers on different streams race.
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PA_ABI_VERSION 1

typedef enum pa_status {
  PA_OK = 0,
  PA_ERR_NULL = 1,         /* a required pointer is NULL                       */
  PA_ERR_SHAPE = 2,        /* inconsistent sizes, or a misaligned pointer      */
  PA_ERR_UNSUPPORTED = 3,  /* dtype, head_dim, block_size or group not built   */
  PA_ERR_WORKSPACE = 4,    /* workspace missing or smaller than required       */
  PA_ERR_HIP = 5,          /* the HIP runtime refused a launch                 */
  PA_ERR_NO_BLOCKS = 6     /* the block manager's pool cannot supply the blocks
                              an operation needs (pa_block_manager.h)          */
} pa_status;

typedef enum pa_dtype {
  PA_F16 = 0,       /* IEEE binary16                                          */
  PA_BF16 = 1,      /* bfloat16                                               */
  PA_FP8_E4M3 = 2   /* OCP 8-bit E4M3 ("fn": no infinities, 448 largest finite,
                       S.1111.111 NaN); pool elements only (pa_copy_blocks,
                       pa_probe_gather); see pa_decode_fp8                    */
} pa_dtype;

/*
 * Decode attention of one query token per sequence over its paged cache.
 *
 *   out[s][h][:] = sum_{t < L_s} softmax_t(scale * q[s][h] . K_t) V_t
 *
 * with K_t, V_t read through block_tables[s] from KV head
 * h / (num_q_heads / num_kv_heads), L_s = seq_lens[s].  L_s = 0 gives a
 * zero row.  Slots at positions >= L_s and table entries past
 * ceil(L_s / block_size) are never read (they may hold anything, NaN
 * included).  Scores, softmax and sums are float32; each softmax weight
 * enters the P.V product as two `dtype` values, hi = round(p) and lo =
 * round(p - hi), whose sum is p to 2^-16 of p (bf16; 2^-22 for fp16), so
 * the result's error does not grow with |V|; the denominator sums the
 * float32 weights; out is rounded to `dtype` (round to nearest even).
 *
 * Supported: dtype F16/BF16 (q, pools and out share it); head_dim 64 or
 * 128; block_size 8, 16 or 32; num_q_heads / num_kv_heads in {1, 2, 4, 8}.
 *
 * Work split: the balanced split.  For each KV head the sequences are laid
 * end to end as tiles of 16 positions, and each of the launch's waves (eight
 * per CU) takes an equal run of them.  A (sequence, KV head) pair cut
 * between runs leaves partial softmax states that a second kernel merges by
 * log-sum-exp.  partition_size = 0 (automatic) lets runs start and end at
 * any tile.  partition_size > 0 (a multiple of 16 and of block_size, at
 * most 512 blocks) makes each sequence a series of partitions of that many
 * positions ([k*P, (k+1)*P)), and runs start and end only at partition
 * boundaries: every partial state covers whole partitions, and the
 * partitions one wave walks in a sequence are merged in its registers.
 * Both give the same result up to float32 summation order.  The tile wave
 * (how a run's tiles are computed) is chosen by the query group: at group 1
 * the vector unit alone (as pa_decode_valu), from group 2 on the matrix
 * cores (q.K^T and P.V as MFMA, the G query heads on the MFMA's N axis).
 * Measured on the 256-sequence mixed step at groups 1/2/4/8: at group 1
 * the vector unit is 1-2% faster; above it the vector unit takes 2%, 9% and
 * 54% longer than the matrix cores.
 * The workspace needs
 * pa_decode_workspace_bytes(...) bytes (0: may be NULL); its contents on
 * entry do not matter and on return are unspecified.
 *
 * Errors: PA_ERR_NULL, PA_ERR_SHAPE (negative sizes, num_q_heads not a
 * multiple of num_kv_heads, bad partition_size, misaligned pointer),
 * PA_ERR_UNSUPPORTED (also when the kernel's LDS or registers do not fit one
 * workgroup on the current device: nothing is launched), PA_ERR_WORKSPACE,
 * PA_ERR_HIP.
 */
pa_status pa_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
                    const int32_t* block_tables, const int32_t* seq_lens, int32_t num_seqs,
                    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                    int32_t block_size, int32_t max_blocks_per_seq, int32_t num_blocks,
                    float scale, int32_t partition_size, pa_dtype dtype, void* workspace,
                    size_t workspace_bytes, hipStream_t stream);

/*
 * pa_decode without a workspace, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation.  Same arguments (less the workspace), contract, kernels
 * and results as pa_decode; the balanced split's partial states live in a
 * static device array of 24 MiB that the library holds on each GPU it runs
 * on until the process ends.  That holds every size whose pa_decode
 * workspace (pa_decode_workspace_bytes, on the current device) fits 24 MiB:
 * on a 256-CU MI355X, the 16.3 MiB of partial states at head_dim 128 plus
 * 16 bytes per (sequence, query head), up to about 500,000 of them.  Larger
 * sizes fail with PA_ERR_WORKSPACE and launch nothing.  The call allocates
 * nothing: its first call on a device looks up the array's address there
 * (hipGetSymbolAddress), later calls reuse it.  Nothing in the array needs
 * to start at zero (every partial a call reads is written by the same call).
 * All calls on one GPU share its array: calls that overlap on one GPU (on
 * different streams, or from different threads) race and give undefined
 * results; calls in one stream are ordered and safe.
 *
 * Errors: as pa_decode, PA_ERR_WORKSPACE for sizes beyond the array, and
 * PA_ERR_HIP if the array's address cannot be found on the current device.
 */
pa_status pa_decode_noalloc(void* out, const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* block_tables, const int32_t* seq_lens,
                            int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                            int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                            int32_t num_blocks, float scale, int32_t partition_size,
                            pa_dtype dtype, hipStream_t stream);

/*
 * pa_decode for a batch whose sequences share a prefix: the first
 * prefix_blocks entries of every sequence's block table are the same
 * physical blocks (a shared system prompt, the candidates of a beam search:
 * "What problem does PagedAttention solve, and what is continuous
 * batching?", section "How PagedAttention works"; "PagedAttention &
 * Continuous Batching", section "Production defaults", prefix caching).
 * The result is pa_decode's (to float32 rounding): softmax attention of each
 * q[s][h] over positions 0..L_s-1.  The work is split at position
 * P = prefix_blocks * block_size: the prefix is attended once for all the
 * batch's query rows together (16 (sequence, head) rows per matrix-core
 * product, so each prefix block is read for 16 rows at a time rather than
 * once per sequence), each sequence's positions [P, L_s) by pa_decode's
 * balanced split, and the two are merged by log-sum-exp.
 *
 * Contract: every sequence has P <= seq_lens[s] <= max_blocks_per_seq *
 * block_size and block_tables[s][j] == block_tables[0][j] for j <
 * prefix_blocks; a sequence that breaks it gets NaN rows (the others are
 * unaffected).  prefix_blocks = 0 is pa_decode (partition_size 0).  Other
 * arguments, supported sizes and errors as pa_decode; prefix_blocks outside
 * [0, max_blocks_per_seq] is PA_ERR_SHAPE.  The workspace needs
 * pa_decode_shared_prefix_workspace_bytes(...) bytes (16-byte aligned).
 * Three kernels run in order on `stream`.
 */
pa_status pa_decode_shared_prefix(void* out, const void* q, const void* k_cache,
                                  const void* v_cache, const int32_t* block_tables,
                                  const int32_t* seq_lens, int32_t num_seqs,
                                  int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                  int32_t block_size, int32_t max_blocks_per_seq,
                                  int32_t num_blocks, int32_t prefix_blocks, float scale,
                                  pa_dtype dtype, void* workspace, size_t workspace_bytes,
                                  hipStream_t stream);

/*
 * Workspace bytes of pa_decode_shared_prefix on the current device: pa_decode's
 * balanced-split workspace, plus (m, l, acc) float32 per (sequence, query
 * head) for the tails and for each 128-position chunk of the prefix.  0 when
 * an argument is invalid.
 */
size_t pa_decode_shared_prefix_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                               int32_t head_dim, int32_t prefix_blocks,
                                               int32_t block_size);

/*
 * pa_decode computed on the vector unit alone instead of the matrix cores:
 * q.K as packed dot products reduced across the lanes of a row (DPP), the
 * online softmax per lane, P.V as float32 FMAs with the weights kept in
 * float32.  Same arguments, contract, workspace and errors as pa_decode;
 * results agree to rounding (the two sum in different orders).  Work split:
 * partition_size = 0 is pa_decode's balanced split, the same runs, launch
 * and merge with the vector tile wave in place of the matrix-core one;
 * partition_size > 0 (a multiple of 16 and of block_size, at most 512
 * blocks) gives every (sequence, KV head, partition of that many positions)
 * its own workgroup, whose four waves take the partition's tiles in turn
 * and merge through LDS, and a second kernel merges the partitions in
 * order.  With partition_size > 0 a sequence's result does not depend on
 * the other sequences of the batch, bit for bit; the balanced split's does
 * (where its runs cut the sequence depends on the whole batch), within
 * float32 rounding.
 */
pa_status pa_decode_valu(void* out, const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* block_tables, const int32_t* seq_lens, int32_t num_seqs,
                         int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                         int32_t block_size, int32_t max_blocks_per_seq, int32_t num_blocks,
                         float scale, int32_t partition_size, pa_dtype dtype, void* workspace,
                         size_t workspace_bytes, hipStream_t stream);

/*
 * Workspace bytes pa_decode (and pa_decode_valu) need for these sizes on the
 * current device; no device memory is read.  The larger of: the balanced
 * split's partial states, two per wave of the launch (two workgroups of four
 * waves per CU of the current device: 2048 waves on a 256-CU MI355X; at
 * most 8192, and 8192 when no device can be queried), min(num_q_heads, 8)
 * heads of head_dim floats plus (m, l) each, and one 16-byte record per
 * (sequence, query head), which pa_decode (and pa_decode_valu with
 * partition_size 0) uses; and, for partition_size > 0, the (m, l, acc) per
 * (sequence, query head, partition) of pa_decode_valu's fixed partitions, an
 * upper bound from max_blocks_per_seq * block_size that is 0 when no
 * sequence can need more than one partition.  0 when an argument is invalid (pa_decode then
 * reports the error).  A workspace sized on one device serves calls on any
 * device with as many CUs or fewer.
 */
size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                 int32_t max_blocks_per_seq, int32_t block_size,
                                 int32_t partition_size);

/*
 * Append: for each token i with slot_mapping[i] >= 0 and each KV head h,
 * k_cache[slot / bs][h][slot % bs][:] = key[i][h][:] (and the same for
 * value), as bit copies.  A negative slot skips the token (padding).
 * Non-negative slots must be distinct (duplicates race); slots >= num_blocks
 * * block_size are skipped.
 *
 * Errors: PA_ERR_NULL, PA_ERR_SHAPE, PA_ERR_UNSUPPORTED (dtype, head_dim not
 * a multiple of 8 in [8, 1024], block_size not in {8, 16, 32}), PA_ERR_HIP.
 */
pa_status pa_reshape_and_cache(const void* key, const void* value, void* k_cache,
                               void* v_cache, const int32_t* slot_mapping, int32_t num_tokens,
                               int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                               int32_t num_blocks, pa_dtype dtype, hipStream_t stream);

/*
 * Copy-on-write data movement: for each pair (src, dst) of block_mapping,
 * block dst of both pools (all KV heads and slots) becomes a bit copy of
 * block src.  A src may appear in several pairs; dsts must be distinct and
 * no dst may be a src (then the result equals a copy from a snapshot taken
 * before the call).  Pairs with an id outside [0, num_blocks) are skipped.
 * dtype is the pool element: PA_F16, PA_BF16 or PA_FP8_E4M3 (then head_dim
 * must be a multiple of 16).
 *
 * Errors: as pa_reshape_and_cache.
 */
pa_status pa_copy_blocks(void* k_cache, void* v_cache, const int32_t* block_mapping,
                         int32_t num_pairs, int32_t num_kv_heads, int32_t head_dim,
                         int32_t block_size, int32_t num_blocks, pa_dtype dtype,
                         hipStream_t stream);

/*
 * 8-bit KV cache.  The pages name quantising the KV cache as a way to cut
 * the bytes each token costs ("What problem does PagedAttention solve, and
 * what is continuous batching?", sections "Why the KV cache becomes the
 * problem" and "What they'll ask next") without fixing a format.  Here: the
 * pools hold OCP E4M3 codes, one byte per element in the same
 * [num_blocks][num_kv_heads][block_size][head_dim] layout, and each pool has
 * one float32 scale: a key code c stands for e4m3(c) * k_scale, a value code
 * for e4m3(c) * v_scale.
 *
 * pa_decode_fp8: pa_decode over 8-bit pools, always with the balanced split
 * (tiles of 32 positions).  q and out are `dtype` (PA_F16 or PA_BF16); keys
 * and values are widened exactly to `dtype` for the products; scores,
 * softmax and sums are float32 as in pa_decode (each softmax weight split
 * into a hi and a lo `dtype` part for the P.V product).  Workspace:
 * pa_decode_workspace_bytes(
 * num_seqs, num_q_heads, head_dim, max_blocks_per_seq, block_size, 0).  Same
 * supported sizes, contract for unused slots and table entries, NaN rows for
 * contract violations, and errors as pa_decode; k_scale and v_scale must be
 * positive and finite (PA_ERR_SHAPE).
 */
pa_status pa_decode_fp8(void* out, const void* q, const void* k_cache, const void* v_cache,
                        const int32_t* block_tables, const int32_t* seq_lens, int32_t num_seqs,
                        int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                        int32_t block_size, int32_t max_blocks_per_seq, int32_t num_blocks,
                        float scale, float k_scale, float v_scale, pa_dtype dtype,
                        void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Quantising append into 8-bit pools: for each token i with slot_mapping[i]
 * >= 0 and each KV head h, k_cache[slot / bs][h][slot % bs][j] =
 * E4M3(key[i][h][j] / k_scale) (values with v_scale), where the quotient is
 * the correctly rounded float32 quotient and E4M3(y) is the nearest E4M3
 * value, ties to the even code, saturating to +-448 (infinities included);
 * NaN gives the NaN code with its sign.  key and value are `dtype` (PA_F16
 * or PA_BF16).  Slot rules as pa_reshape_and_cache.  Errors as
 * pa_reshape_and_cache, plus PA_ERR_UNSUPPORTED for head_dim not a multiple
 * of 16 and PA_ERR_SHAPE for a scale that is not positive and finite.
 */
pa_status pa_reshape_and_cache_fp8(const void* key, const void* value, void* k_cache,
                                   void* v_cache, const int32_t* slot_mapping,
                                   int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                                   int32_t block_size, int32_t num_blocks, float k_scale,
                                   float v_scale, pa_dtype dtype, hipStream_t stream);

/*
 * Several query tokens per sequence with a causal mask (chunked prefill).
 * The pages describe prefill as the compute-heavy first pass over a prompt
 * and chunked prefill as splitting a long prompt into pieces processed over
 * several steps ("What problem does PagedAttention solve, and what is
 * continuous batching?", sections "Why the KV cache becomes the problem"
 * and "How the two fit together in production").
 *
 * Sequence s has a chunk of n_s = query_start[s+1] - query_start[s] tokens
 * whose keys and values are already in the pools (pa_reshape_and_cache),
 * at positions L_s - n_s .. L_s - 1 (L_s = seq_lens[s]).  For chunk token i
 * and query head h:
 *
 *   out[query_start[s] + i][h][:] =
 *       sum_{t <= L_s - n_s + i} softmax_t(scale * q[query_start[s] + i][h] . K_t) V_t
 *
 * with K_t, V_t read through block_tables[s] from KV head h / (num_q_heads /
 * num_kv_heads).  n_s = 1 is decode; n_s = L_s is a whole prompt; n_s = 0
 * writes nothing.  q and out are [total_q][num_q_heads][head_dim];
 * query_start holds num_seqs + 1 non-decreasing offsets from 0 to total_q
 * (device memory).  Arithmetic: float32 scores and sums; unlike pa_decode,
 * each softmax weight is rounded once to dtype for P.V (this kernel is
 * bound by the matrix cores, and the split would double its P.V work) and
 * the denominator sums the same rounded weights, so a weight errs by up to
 * 2^-8 of itself (bf16; 2^-11 for fp16) and the result by up to that
 * fraction of max_t |V_t - out|; out rounded to dtype.
 *
 * Supported: dtype F16/BF16; head_dim 64 or 128; block_size 8, 16 or 32;
 * num_q_heads / num_kv_heads in {1, 2, 4, 8}.  No workspace.
 *
 * Device data that breaks the contract is never dereferenced: a chunk
 * longer than its sequence, a length past the block table or a block id
 * outside the pool gives NaN rows for that sequence's chunk; offsets that
 * are not non-decreasing within [0, total_q] give an empty chunk (its rows
 * are left unwritten).  Rows outside [0, total_q) are never accessed.
 *
 * Errors: PA_ERR_NULL, PA_ERR_SHAPE (negative sizes, num_q_heads not a
 * multiple of num_kv_heads, misaligned pointer, too many rows for one
 * launch), PA_ERR_UNSUPPORTED, PA_ERR_HIP.
 */
pa_status pa_prefill(void* out, const void* q, const void* k_cache, const void* v_cache,
                     const int32_t* block_tables, const int32_t* seq_lens,
                     const int32_t* query_start, int32_t num_seqs, int32_t total_q,
                     int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                     int32_t block_size, int32_t max_blocks_per_seq, int32_t num_blocks,
                     float scale, pa_dtype dtype, hipStream_t stream);

/* Static name of a status code. */
const char* pa_status_string(pa_status status);

/* Message of the calling thread's last failed call ("" if none). */
const char* pa_last_error(void);

/* PA_ABI_VERSION of the built library. */
int32_t pa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
