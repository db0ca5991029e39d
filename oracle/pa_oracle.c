/*
 * pa_oracle.c -- plain CPU oracle for paged decode attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The product path
 * (the HIP library and its Python binding) never links, imports or calls it,
 * and it shares no code with that path.
 *
 * Everything here is the plain definition, in double precision, with no
 * blocking, fusion or reordering beyond what the definition states.
 *
 * Sources (three web pages on PagedAttention and continuous batching):
 *  - "What problem does PagedAttention solve, and what is continuous
 *    batching?" (datarekha), section "How PagedAttention works": a block
 *    holds a fixed number of tokens (16 in the example); a per-request block
 *    table maps logical block number -> physical block; the attention kernel
 *    follows the table when it reads keys and values, so the physical blocks
 *    may sit anywhere while positions keep their logical order.  Shared
 *    blocks and copy-on-write of a private block when a candidate diverges.
 *  - same page, "Why the KV cache becomes the problem": decode reads the
 *    stored keys/values of every earlier token and appends a small amount
 *    of new data each step.
 *  - "Continuous Batching & Paged Attention" (topicspectrum), section
 *    "Attention needs memory that grows with the conversation": attention
 *    compares the current position with the earlier tokens, whose key and
 *    value vectors are kept in the KV cache.
 *
 * Readings where the pages are silent (each one is listed with its reason
 * in the design notes of the repository):
 *  - attention is textbook softmax attention of one query vector against
 *    the L stored keys, with an explicit score scale;
 *  - query head h reads KV head h / (Hq/Hkv) (contiguous GQA groups);
 *  - position t of a sequence lives in logical block t / bs at offset
 *    t % bs, i.e. slot = table[t / bs] * bs + t % bs;
 *  - pools are laid out [num_blocks][Hkv][bs][d], K and V separate;
 *  - a negative slot in the append means "skip" (padding);
 *  - L = 0 gives an all-zero output.
 *
 * Element formats: IEEE-754 binary16 and bfloat16 (the upper half of an
 * IEEE-754 binary32).  Inputs are passed as raw 16-bit patterns and widened
 * exactly to double.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORACLE_F16 = 0, ORACLE_BF16 = 1 };

/* Error codes returned by every entry point. */
enum {
  ORACLE_OK = 0,
  ORACLE_BAD_ARG = -1,      /* sizes or dtype out of the allowed range     */
  ORACLE_BAD_BLOCK = -2,    /* a table entry that is read is out of range  */
  ORACLE_BAD_SLOT = -3,     /* slot >= num_blocks * block_size             */
  ORACLE_DUP_SLOT = -4,     /* two tokens written to the same slot         */
  ORACLE_BAD_PAIR = -5,     /* copy pair out of range, dst repeated or a src */
  ORACLE_NO_MEMORY = -6
};

/* binary16: sign, 5-bit exponent (bias 15), 10-bit fraction.
 * Normal:    (-1)^s * (1024 + f) * 2^(e - 25)
 * Subnormal: (-1)^s * f * 2^-24                                            */
double oracle_f16_to_double(uint16_t h) {
  int s = (h >> 15) & 1;
  int e = (h >> 10) & 0x1f;
  int f = h & 0x3ff;
  double v;
  if (e == 0)
    v = ldexp((double)f, -24);
  else if (e == 31)
    v = (f != 0) ? NAN : INFINITY;
  else
    v = ldexp((double)(1024 + f), e - 25);
  return s ? -v : v;
}

/* bfloat16: the 16 high bits of a binary32 value. */
double oracle_bf16_to_double(uint16_t b) {
  uint32_t u = ((uint32_t)b) << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

static double widen(uint16_t x, int dtype) {
  return dtype == ORACLE_BF16 ? oracle_bf16_to_double(x) : oracle_f16_to_double(x);
}

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Logical position t of sequence s -> flat slot in the pool. */
static int64_t slot_of(const int32_t* block_tables, int32_t max_blocks_per_seq,
                       int32_t block_size, int32_t s, int32_t t) {
  int32_t block = block_tables[(int64_t)s * max_blocks_per_seq + t / block_size];
  return (int64_t)block * block_size + t % block_size;
}

/* slots[i] = table[seq[i]][pos[i] / bs] * bs + pos[i] % bs  (used to check
 * the slot_mapping the input generator hands to the append). */
int oracle_slot_mapping(int32_t* slots, const int32_t* block_tables,
                        const int32_t* seq_ids, const int32_t* positions,
                        int32_t num_tokens, int32_t max_blocks_per_seq,
                        int32_t block_size) {
  if (block_size <= 0 || max_blocks_per_seq <= 0) return ORACLE_BAD_ARG;
  for (int32_t i = 0; i < num_tokens; ++i) {
    if (positions[i] < 0 || positions[i] / block_size >= max_blocks_per_seq)
      return ORACLE_BAD_ARG;
    int64_t v = slot_of(block_tables, max_blocks_per_seq, block_size,
                        seq_ids[i], positions[i]);
    if (v > INT32_MAX) return ORACLE_BAD_SLOT;
    slots[i] = (int32_t)v;
  }
  return ORACLE_OK;
}

/* Check that every table entry the decode of sequence s reads is a valid
 * physical block id. */
static int check_tables(const int32_t* block_tables, const int32_t* seq_lens,
                        int32_t num_seqs, int32_t max_blocks_per_seq,
                        int32_t block_size, int32_t num_blocks) {
  for (int32_t s = 0; s < num_seqs; ++s) {
    int32_t L = seq_lens[s];
    if (L < 0) return ORACLE_BAD_ARG;
    int32_t nb = (L + block_size - 1) / block_size;
    if (nb > max_blocks_per_seq) return ORACLE_BAD_ARG;
    for (int32_t j = 0; j < nb; ++j) {
      int32_t b = block_tables[(int64_t)s * max_blocks_per_seq + j];
      if (b < 0 || b >= num_blocks) return ORACLE_BAD_BLOCK;
    }
  }
  return ORACLE_OK;
}

/* Softmax attention of one (sequence, query head) over positions
 * [t0, t1) of that sequence, in double precision.
 *   z_t = scale * sum_i q[i] K_t[i]
 *   m   = max_t z_t,   l = sum_t exp(z_t - m),   acc = sum_t exp(z_t - m) V_t
 * Returns m, l and acc (length d); the attention output is acc / l. */
static void attend_range(double* m_out, double* l_out, double* acc,
                         const uint16_t* q, const uint16_t* k_cache,
                         const uint16_t* v_cache, const int32_t* block_tables,
                         int32_t s, int32_t h, int32_t t0, int32_t t1,
                         int32_t num_q_heads, int32_t num_kv_heads,
                         int32_t head_dim, int32_t block_size,
                         int32_t max_blocks_per_seq, double scale, int dtype,
                         double* z) {
  const int32_t group = num_q_heads / num_kv_heads;
  const int32_t kh = h / group;
  const uint16_t* qv = q + ((int64_t)s * num_q_heads + h) * head_dim;

  for (int32_t t = t0; t < t1; ++t) {
    int64_t slot = slot_of(block_tables, max_blocks_per_seq, block_size, s, t);
    int64_t b = slot / block_size, o = slot % block_size;
    const uint16_t* kt = k_cache + ((b * num_kv_heads + kh) * block_size + o) * head_dim;
    double dot = 0.0;
    for (int32_t i = 0; i < head_dim; ++i) dot += widen(qv[i], dtype) * widen(kt[i], dtype);
    z[t - t0] = scale * dot;
  }
  double m = -INFINITY;
  for (int32_t t = t0; t < t1; ++t) m = z[t - t0] > m ? z[t - t0] : m;
  double l = 0.0;
  for (int32_t i = 0; i < head_dim; ++i) acc[i] = 0.0;
  for (int32_t t = t0; t < t1; ++t) {
    double w = exp(z[t - t0] - m);
    l += w;
    int64_t slot = slot_of(block_tables, max_blocks_per_seq, block_size, s, t);
    int64_t b = slot / block_size, o = slot % block_size;
    const uint16_t* vt = v_cache + ((b * num_kv_heads + kh) * block_size + o) * head_dim;
    for (int32_t i = 0; i < head_dim; ++i) acc[i] += w * widen(vt[i], dtype);
  }
  *m_out = m;
  *l_out = l;
}

/*
 * out[s][h][:] = softmax over t < L_s of (scale * q[s][h] . K_t) applied to V_t,
 * with K_t, V_t read through the block table of sequence s.
 *
 * q [S][Hq][d], pools [NB][Hkv][bs][d] (raw 16-bit patterns), block_tables
 * [S][MB], seq_lens [S], out [S][Hq][d] double.  If pairs != NULL only the
 * (s, h) pairs listed there (pairs[2k], pairs[2k+1]) are written; otherwise
 * all.  scale is the float32 value the caller also hands the GPU path; it is
 * widened exactly.
 */
int oracle_decode(double* out, const uint16_t* q, const uint16_t* k_cache,
                  const uint16_t* v_cache, const int32_t* block_tables,
                  const int32_t* seq_lens, int32_t num_seqs, int32_t num_q_heads,
                  int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                  int32_t max_blocks_per_seq, int32_t num_blocks, float scale,
                  int32_t dtype, const int32_t* pairs, int32_t num_pairs) {
  if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      block_size <= 0 || max_blocks_per_seq <= 0 || num_blocks <= 0 ||
      num_q_heads % num_kv_heads != 0 || (dtype != ORACLE_F16 && dtype != ORACLE_BF16))
    return ORACLE_BAD_ARG;
  int rc = check_tables(block_tables, seq_lens, num_seqs, max_blocks_per_seq,
                        block_size, num_blocks);
  if (rc != ORACLE_OK) return rc;

  const int64_t n = pairs ? (int64_t)num_pairs : (int64_t)num_seqs * num_q_heads;
  for (int64_t k = 0; pairs && k < n; ++k)
    if (pairs[2 * k] < 0 || pairs[2 * k] >= num_seqs || pairs[2 * k + 1] < 0 ||
        pairs[2 * k + 1] >= num_q_heads)
      return ORACLE_BAD_ARG;

  int32_t max_len = 0;
  for (int32_t s = 0; s < num_seqs; ++s) max_len = seq_lens[s] > max_len ? seq_lens[s] : max_len;

  int failed = 0;
#pragma omp parallel
  {
    double* z = (double*)malloc(sizeof(double) * (size_t)(max_len > 0 ? max_len : 1));
    double* acc = (double*)malloc(sizeof(double) * (size_t)head_dim);
    if (!z || !acc) {
#pragma omp atomic write
      failed = 1;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int64_t k = 0; k < n; ++k) {
        int32_t s = pairs ? pairs[2 * k] : (int32_t)(k / num_q_heads);
        int32_t h = pairs ? pairs[2 * k + 1] : (int32_t)(k % num_q_heads);
        double* o = out + ((int64_t)s * num_q_heads + h) * head_dim;
        int32_t L = seq_lens[s];
        if (L == 0) {
          for (int32_t i = 0; i < head_dim; ++i) o[i] = 0.0;
          continue;
        }
        double m, l;
        attend_range(&m, &l, acc, q, k_cache, v_cache, block_tables, s, h, 0, L,
                     num_q_heads, num_kv_heads, head_dim, block_size,
                     max_blocks_per_seq, (double)scale, dtype, z);
        for (int32_t i = 0; i < head_dim; ++i) o[i] = acc[i] / l;
      }
    }
    free(z);
    free(acc);
  }
  return failed ? ORACLE_NO_MEMORY : ORACLE_OK;
}

/*
 * The same attention computed by partitions of `partition_size` positions
 * and merged by log-sum-exp:
 *   for each partition p: m_p, l_p, acc_p over its positions;
 *   M = max_p m_p;  out = sum_p e^{m_p - M} acc_p / sum_p e^{m_p - M} l_p.
 * In exact arithmetic this equals oracle_decode; the tests check the two
 * agree to double rounding, which pins the merge rule the split path uses.
 */
int oracle_decode_split(double* out, const uint16_t* q, const uint16_t* k_cache,
                        const uint16_t* v_cache, const int32_t* block_tables,
                        const int32_t* seq_lens, int32_t num_seqs,
                        int32_t num_q_heads, int32_t num_kv_heads,
                        int32_t head_dim, int32_t block_size,
                        int32_t max_blocks_per_seq, int32_t num_blocks,
                        float scale, int32_t dtype, int32_t partition_size) {
  if (partition_size <= 0 || num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 ||
      head_dim <= 0 || block_size <= 0 || max_blocks_per_seq <= 0 ||
      num_q_heads % num_kv_heads != 0 || (dtype != ORACLE_F16 && dtype != ORACLE_BF16))
    return ORACLE_BAD_ARG;
  int rc = check_tables(block_tables, seq_lens, num_seqs, max_blocks_per_seq,
                        block_size, num_blocks);
  if (rc != ORACLE_OK) return rc;

  double* z = (double*)malloc(sizeof(double) * (size_t)partition_size);
  double* acc_p = (double*)malloc(sizeof(double) * (size_t)head_dim);
  double* acc = (double*)malloc(sizeof(double) * (size_t)head_dim);
  if (!z || !acc_p || !acc) {
    free(z);
    free(acc_p);
    free(acc);
    return ORACLE_NO_MEMORY;
  }
  for (int32_t s = 0; s < num_seqs; ++s) {
    int32_t L = seq_lens[s];
    int32_t P = (L + partition_size - 1) / partition_size;
    for (int32_t h = 0; h < num_q_heads; ++h) {
      double* o = out + ((int64_t)s * num_q_heads + h) * head_dim;
      if (L == 0) {
        for (int32_t i = 0; i < head_dim; ++i) o[i] = 0.0;
        continue;
      }
      /* first pass: the global max of the partition maxima */
      double* m_p = (double*)malloc(sizeof(double) * (size_t)P);
      double* l_p = (double*)malloc(sizeof(double) * (size_t)P);
      double* accs = (double*)malloc(sizeof(double) * (size_t)P * (size_t)head_dim);
      if (!m_p || !l_p || !accs) {
        free(m_p);
        free(l_p);
        free(accs);
        free(z);
        free(acc_p);
        free(acc);
        return ORACLE_NO_MEMORY;
      }
      for (int32_t p = 0; p < P; ++p) {
        int32_t t0 = p * partition_size;
        int32_t t1 = t0 + partition_size < L ? t0 + partition_size : L;
        attend_range(&m_p[p], &l_p[p], acc_p, q, k_cache, v_cache, block_tables, s,
                     h, t0, t1, num_q_heads, num_kv_heads, head_dim, block_size,
                     max_blocks_per_seq, (double)scale, dtype, z);
        memcpy(accs + (int64_t)p * head_dim, acc_p, sizeof(double) * (size_t)head_dim);
      }
      double M = -INFINITY;
      for (int32_t p = 0; p < P; ++p) M = m_p[p] > M ? m_p[p] : M;
      double den = 0.0;
      for (int32_t i = 0; i < head_dim; ++i) acc[i] = 0.0;
      for (int32_t p = 0; p < P; ++p) {
        double w = exp(m_p[p] - M);
        den += w * l_p[p];
        for (int32_t i = 0; i < head_dim; ++i) acc[i] += w * accs[(int64_t)p * head_dim + i];
      }
      for (int32_t i = 0; i < head_dim; ++i) o[i] = acc[i] / den;
      free(m_p);
      free(l_p);
      free(accs);
    }
  }
  free(z);
  free(acc_p);
  free(acc);
  return ORACLE_OK;
}

/*
 * Append: for every token i with slot_mapping[i] >= 0 and every KV head h,
 * copy the bits of key[i][h][:] into k_cache[slot / bs][h][slot % bs][:]
 * (same for value).  Non-negative slots must be distinct and inside the
 * pool; the oracle refuses the call otherwise and writes nothing.
 */
int oracle_reshape_and_cache(const uint16_t* key, const uint16_t* value,
                             uint16_t* k_cache, uint16_t* v_cache,
                             const int32_t* slot_mapping, int32_t num_tokens,
                             int32_t num_kv_heads, int32_t head_dim,
                             int32_t block_size, int32_t num_blocks) {
  if (num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
      num_blocks <= 0)
    return ORACLE_BAD_ARG;
  const int64_t num_slots = (int64_t)num_blocks * block_size;
  for (int32_t i = 0; i < num_tokens; ++i) {
    if (slot_mapping[i] >= num_slots) return ORACLE_BAD_SLOT;
    for (int32_t j = 0; j < i; ++j)
      if (slot_mapping[i] >= 0 && slot_mapping[j] == slot_mapping[i]) return ORACLE_DUP_SLOT;
  }
  for (int32_t i = 0; i < num_tokens; ++i) {
    int64_t slot = slot_mapping[i];
    if (slot < 0) continue;
    int64_t b = slot / block_size, o = slot % block_size;
    for (int32_t h = 0; h < num_kv_heads; ++h) {
      int64_t src = ((int64_t)i * num_kv_heads + h) * head_dim;
      int64_t dst = ((b * num_kv_heads + h) * block_size + o) * head_dim;
      memcpy(k_cache + dst, key + src, sizeof(uint16_t) * (size_t)head_dim);
      memcpy(v_cache + dst, value + src, sizeof(uint16_t) * (size_t)head_dim);
    }
  }
  return ORACLE_OK;
}

/*
 * Copy-on-write data movement: for every pair (src, dst) in block_mapping
 * [n][2], the whole of block dst (all KV heads and slots, K and V) becomes
 * a copy of block src as it was before the call.  dsts must be distinct and
 * none may be a src; the oracle refuses the call otherwise.
 */
int oracle_copy_blocks(uint16_t* k_cache, uint16_t* v_cache,
                       const int32_t* block_mapping, int32_t num_pairs,
                       int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                       int32_t num_blocks) {
  if (num_pairs < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
      num_blocks <= 0)
    return ORACLE_BAD_ARG;
  for (int32_t i = 0; i < num_pairs; ++i) {
    int32_t src = block_mapping[2 * i], dst = block_mapping[2 * i + 1];
    if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return ORACLE_BAD_PAIR;
    for (int32_t j = 0; j < num_pairs; ++j) {
      if (j != i && block_mapping[2 * j + 1] == dst) return ORACLE_BAD_PAIR;
      if (block_mapping[2 * j] == dst) return ORACLE_BAD_PAIR;
    }
  }
  const int64_t block_elems = (int64_t)num_kv_heads * block_size * head_dim;
  /* snapshot every source first, then write the destinations */
  uint16_t* snap = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)(2 * block_elems) *
                                     (size_t)(num_pairs > 0 ? num_pairs : 1));
  if (!snap) return ORACLE_NO_MEMORY;
  for (int32_t i = 0; i < num_pairs; ++i) {
    int64_t src = block_mapping[2 * i];
    memcpy(snap + (2 * i) * block_elems, k_cache + src * block_elems,
           sizeof(uint16_t) * (size_t)block_elems);
    memcpy(snap + (2 * i + 1) * block_elems, v_cache + src * block_elems,
           sizeof(uint16_t) * (size_t)block_elems);
  }
  for (int32_t i = 0; i < num_pairs; ++i) {
    int64_t dst = block_mapping[2 * i + 1];
    memcpy(k_cache + dst * block_elems, snap + (2 * i) * block_elems,
           sizeof(uint16_t) * (size_t)block_elems);
    memcpy(v_cache + dst * block_elems, snap + (2 * i + 1) * block_elems,
           sizeof(uint16_t) * (size_t)block_elems);
  }
  free(snap);
  return ORACLE_OK;
}

/* ------------------------------------------------------------------------
 * 8-bit KV cache (OCP FP8 E4M3, one scale per pool).
 *
 * The pages name quantising the KV cache as a way to cut the bytes each
 * token costs ("What problem does PagedAttention solve, and what is
 * continuous batching?", sections "Why the KV cache becomes the problem" and
 * "What they'll ask next"), and fix neither the format nor the scaling.
 * Readings taken:
 *  - element format: OCP 8-bit floating point, E4M3 (the "fn" variant: no
 *    infinities, S.1111.111 is NaN, largest finite 448);
 *  - one float32 scale per pool: the stored code c stands for
 *    e4m3(c) * k_scale (keys) or e4m3(c) * v_scale (values);
 *  - quantising: y = x / scale rounded once to float32, then to the nearest
 *    E4M3 value, ties to the even code, saturating: |y| >= 448 (infinities
 *    included) gives +-448; NaN gives the NaN code with y's sign.
 * ------------------------------------------------------------------------ */

/* E4M3: sign, 4-bit exponent (bias 7), 3-bit fraction.
 * Normal:    (-1)^s * (8 + f) * 2^(e - 10)       (e = 1..15, not e=15,f=7)
 * Subnormal: (-1)^s * f * 2^-9                   (e = 0)
 * e = 15, f = 7: NaN.                                                       */
double oracle_e4m3_to_double(uint8_t c) {
  int s = (c >> 7) & 1;
  int e = (c >> 3) & 0xf;
  int f = c & 0x7;
  double v;
  if (e == 15 && f == 7)
    return NAN;
  if (e == 0)
    v = ldexp((double)f, -9);
  else
    v = ldexp((double)(8 + f), e - 10);
  return s ? -v : v;
}

/* Nearest E4M3 code to the float32 value y: every finite magnitude code
 * 0x00..0x7E is tried, the closest wins, and of two equally close the even
 * code (even last fraction bit) wins.  Saturating; NaN -> NaN code. */
uint8_t oracle_e4m3_from_float(float y) {
  uint32_t bits;
  memcpy(&bits, &y, sizeof bits);
  const uint8_t sign = (uint8_t)((bits >> 31) << 7);
  if (y != y) return (uint8_t)(sign | 0x7f);
  const double a = fabs((double)y);
  if (a >= 448.0) return (uint8_t)(sign | 0x7e);
  int best = 0;
  double best_err = INFINITY;
  for (int c = 0; c <= 0x7e; ++c) {
    const double err = fabs(oracle_e4m3_to_double((uint8_t)c) - a);
    if (err < best_err || (err == best_err && (c & 1) == 0)) {
      best = c;
      best_err = err;
    }
  }
  return (uint8_t)(sign | best);
}

/* The float32 quotient x / scale: the exact quotient of two float32 values
 * rounded to double and then to float32 is the correctly rounded float32
 * quotient (53 >= 2 * 24 + 2, so the double rounding is innocuous). */
static float quotient_f32(double x, float scale) { return (float)(x / (double)scale); }

/* codes[i] = E4M3 code of x[i] / scale, x raw 16-bit patterns of dtype. */
int oracle_quantize_e4m3(uint8_t* codes, const uint16_t* x, int64_t n, int32_t dtype,
                         float scale) {
  if (n < 0 || (dtype != ORACLE_F16 && dtype != ORACLE_BF16) || !(scale > 0.0f) ||
      scale == INFINITY)
    return ORACLE_BAD_ARG;
  for (int64_t i = 0; i < n; ++i)
    codes[i] = oracle_e4m3_from_float(quotient_f32(widen(x[i], dtype), scale));
  return ORACLE_OK;
}

/*
 * Append into 8-bit pools: for every token i with slot_mapping[i] >= 0 and
 * every KV head h, k_cache[slot / bs][h][slot % bs][j] = code of
 * key[i][h][j] / k_scale (values with v_scale).  Same slot rules as
 * oracle_reshape_and_cache.
 */
int oracle_reshape_and_cache_fp8(const uint16_t* key, const uint16_t* value, uint8_t* k_cache,
                                 uint8_t* v_cache, const int32_t* slot_mapping,
                                 int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                                 int32_t block_size, int32_t num_blocks, float k_scale,
                                 float v_scale, int32_t dtype) {
  if (num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
      num_blocks <= 0 || (dtype != ORACLE_F16 && dtype != ORACLE_BF16) ||
      !(k_scale > 0.0f) || !(v_scale > 0.0f) || k_scale == INFINITY || v_scale == INFINITY)
    return ORACLE_BAD_ARG;
  const int64_t num_slots = (int64_t)num_blocks * block_size;
  for (int32_t i = 0; i < num_tokens; ++i) {
    if (slot_mapping[i] >= num_slots) return ORACLE_BAD_SLOT;
    for (int32_t j = 0; j < i; ++j)
      if (slot_mapping[i] >= 0 && slot_mapping[j] == slot_mapping[i]) return ORACLE_DUP_SLOT;
  }
  for (int32_t i = 0; i < num_tokens; ++i) {
    int64_t slot = slot_mapping[i];
    if (slot < 0) continue;
    int64_t b = slot / block_size, o = slot % block_size;
    for (int32_t h = 0; h < num_kv_heads; ++h) {
      int64_t src = ((int64_t)i * num_kv_heads + h) * head_dim;
      int64_t dst = ((b * num_kv_heads + h) * block_size + o) * head_dim;
      for (int32_t j = 0; j < head_dim; ++j) {
        k_cache[dst + j] = oracle_e4m3_from_float(quotient_f32(widen(key[src + j], dtype), k_scale));
        v_cache[dst + j] =
            oracle_e4m3_from_float(quotient_f32(widen(value[src + j], dtype), v_scale));
      }
    }
  }
  return ORACLE_OK;
}

/*
 * Decode attention over 8-bit pools: exactly oracle_decode with every stored
 * key element read as e4m3(code) * k_scale and every value element as
 * e4m3(code) * v_scale (both products exact in double).  q and out as in
 * oracle_decode.
 */
int oracle_decode_fp8(double* out, const uint16_t* q, const uint8_t* k_cache,
                      const uint8_t* v_cache, const int32_t* block_tables,
                      const int32_t* seq_lens, int32_t num_seqs, int32_t num_q_heads,
                      int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                      int32_t max_blocks_per_seq, int32_t num_blocks, float scale,
                      float k_scale, float v_scale, int32_t dtype, const int32_t* pairs,
                      int32_t num_pairs) {
  if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      block_size <= 0 || max_blocks_per_seq <= 0 || num_blocks <= 0 ||
      num_q_heads % num_kv_heads != 0 || (dtype != ORACLE_F16 && dtype != ORACLE_BF16))
    return ORACLE_BAD_ARG;
  int rc = check_tables(block_tables, seq_lens, num_seqs, max_blocks_per_seq,
                        block_size, num_blocks);
  if (rc != ORACLE_OK) return rc;
  const int64_t n = pairs ? (int64_t)num_pairs : (int64_t)num_seqs * num_q_heads;
  for (int64_t k = 0; pairs && k < n; ++k)
    if (pairs[2 * k] < 0 || pairs[2 * k] >= num_seqs || pairs[2 * k + 1] < 0 ||
        pairs[2 * k + 1] >= num_q_heads)
      return ORACLE_BAD_ARG;
  int32_t max_len = 0;
  for (int32_t s = 0; s < num_seqs; ++s) max_len = seq_lens[s] > max_len ? seq_lens[s] : max_len;
  const int32_t group = num_q_heads / num_kv_heads;
  const double ks = (double)k_scale, vs = (double)v_scale, sc = (double)scale;

  int failed = 0;
#pragma omp parallel
  {
    double* z = (double*)malloc(sizeof(double) * (size_t)(max_len > 0 ? max_len : 1));
    double* acc = (double*)malloc(sizeof(double) * (size_t)head_dim);
    if (!z || !acc) {
#pragma omp atomic write
      failed = 1;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int64_t k = 0; k < n; ++k) {
        int32_t s = pairs ? pairs[2 * k] : (int32_t)(k / num_q_heads);
        int32_t h = pairs ? pairs[2 * k + 1] : (int32_t)(k % num_q_heads);
        int32_t kh = h / group;
        double* o = out + ((int64_t)s * num_q_heads + h) * head_dim;
        const uint16_t* qv = q + ((int64_t)s * num_q_heads + h) * head_dim;
        int32_t L = seq_lens[s];
        if (L == 0) {
          for (int32_t i = 0; i < head_dim; ++i) o[i] = 0.0;
          continue;
        }
        for (int32_t t = 0; t < L; ++t) {
          int64_t slot = slot_of(block_tables, max_blocks_per_seq, block_size, s, t);
          int64_t b = slot / block_size, off = slot % block_size;
          const uint8_t* kt = k_cache + ((b * num_kv_heads + kh) * block_size + off) * head_dim;
          double dot = 0.0;
          for (int32_t i = 0; i < head_dim; ++i)
            dot += widen(qv[i], dtype) * (oracle_e4m3_to_double(kt[i]) * ks);
          z[t] = sc * dot;
        }
        double m = -INFINITY;
        for (int32_t t = 0; t < L; ++t) m = z[t] > m ? z[t] : m;
        double l = 0.0;
        for (int32_t i = 0; i < head_dim; ++i) acc[i] = 0.0;
        for (int32_t t = 0; t < L; ++t) {
          double w = exp(z[t] - m);
          l += w;
          int64_t slot = slot_of(block_tables, max_blocks_per_seq, block_size, s, t);
          int64_t b = slot / block_size, off = slot % block_size;
          const uint8_t* vt = v_cache + ((b * num_kv_heads + kh) * block_size + off) * head_dim;
          for (int32_t i = 0; i < head_dim; ++i) acc[i] += w * (oracle_e4m3_to_double(vt[i]) * vs);
        }
        for (int32_t i = 0; i < head_dim; ++i) o[i] = acc[i] / l;
      }
    }
    free(z);
    free(acc);
  }
  return failed ? ORACLE_NO_MEMORY : ORACLE_OK;
}

/* ------------------------------------------------------------------------
 * Several query tokens per sequence (chunked prefill).
 *
 * "What problem does PagedAttention solve, and what is continuous
 * batching?" (datarekha): prefill is the first pass over the prompt
 * ("Why the KV cache becomes the problem"), and production servers cap the
 * tokens per scheduling step or split a long prompt into smaller pieces,
 * chunked prefill ("How the two fit together in production").  Reading:
 * a step hands sequence s a chunk of n_s = query_start[s+1] - query_start[s]
 * new tokens whose keys and values are already in the pool, at positions
 * L_s - n_s .. L_s - 1 (L_s = seq_lens[s], so 0 <= n_s <= L_s); token i of
 * the chunk attends causally, to positions 0 .. L_s - n_s + i, through the
 * sequence's block table.  n_s = 1 is decode; n_s = L_s is a whole prompt.
 * ------------------------------------------------------------------------ */

/*
 * out[query_start[s] + i][h][:] = softmax over t <= L_s - n_s + i of
 * (scale * q[query_start[s] + i][h] . K_t) applied to V_t.
 * q and out are [total_q][Hq][d] (q raw 16-bit patterns, out double);
 * query_start has num_seqs + 1 non-decreasing entries from 0 to total_q.
 */
int oracle_prefill(double* out, const uint16_t* q, const uint16_t* k_cache,
                   const uint16_t* v_cache, const int32_t* block_tables,
                   const int32_t* seq_lens, const int32_t* query_start, int32_t num_seqs,
                   int32_t total_q, int32_t num_q_heads, int32_t num_kv_heads,
                   int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                   int32_t num_blocks, float scale, int32_t dtype) {
  if (num_seqs < 0 || total_q < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      block_size <= 0 || max_blocks_per_seq <= 0 || num_blocks <= 0 ||
      num_q_heads % num_kv_heads != 0 || (dtype != ORACLE_F16 && dtype != ORACLE_BF16))
    return ORACLE_BAD_ARG;
  if (query_start[0] != 0 || query_start[num_seqs] != total_q) return ORACLE_BAD_ARG;
  for (int32_t s = 0; s < num_seqs; ++s) {
    const int32_t n = query_start[s + 1] - query_start[s];
    if (n < 0 || n > seq_lens[s]) return ORACLE_BAD_ARG;
  }
  int rc = check_tables(block_tables, seq_lens, num_seqs, max_blocks_per_seq, block_size,
                        num_blocks);
  if (rc != ORACLE_OK) return rc;
  const int32_t group = num_q_heads / num_kv_heads;
  int32_t max_len = 0;
  for (int32_t s = 0; s < num_seqs; ++s) max_len = seq_lens[s] > max_len ? seq_lens[s] : max_len;

  int failed = 0;
#pragma omp parallel
  {
    double* z = (double*)malloc(sizeof(double) * (size_t)(max_len > 0 ? max_len : 1));
    double* acc = (double*)malloc(sizeof(double) * (size_t)head_dim);
    if (!z || !acc) {
#pragma omp atomic write
      failed = 1;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int64_t k = 0; k < (int64_t)total_q * num_q_heads; ++k) {
        const int32_t row = (int32_t)(k / num_q_heads), h = (int32_t)(k % num_q_heads);
        int32_t s = 0;
        while (query_start[s + 1] <= row) ++s;  /* the sequence this token belongs to */
        const int32_t L = seq_lens[s], n = query_start[s + 1] - query_start[s];
        const int32_t p = L - n + (row - query_start[s]);  /* its position */
        const int32_t kh = h / group;
        const uint16_t* qv = q + ((int64_t)row * num_q_heads + h) * head_dim;
        double* o = out + ((int64_t)row * num_q_heads + h) * head_dim;
        for (int32_t t = 0; t <= p; ++t) {
          int64_t slot = slot_of(block_tables, max_blocks_per_seq, block_size, s, t);
          int64_t b = slot / block_size, off = slot % block_size;
          const uint16_t* kt = k_cache + ((b * num_kv_heads + kh) * block_size + off) * head_dim;
          double dot = 0.0;
          for (int32_t i = 0; i < head_dim; ++i) dot += widen(qv[i], dtype) * widen(kt[i], dtype);
          z[t] = (double)scale * dot;
        }
        double m = -INFINITY;
        for (int32_t t = 0; t <= p; ++t) m = z[t] > m ? z[t] : m;
        double l = 0.0;
        for (int32_t i = 0; i < head_dim; ++i) acc[i] = 0.0;
        for (int32_t t = 0; t <= p; ++t) {
          double w = exp(z[t] - m);
          l += w;
          int64_t slot = slot_of(block_tables, max_blocks_per_seq, block_size, s, t);
          int64_t b = slot / block_size, off = slot % block_size;
          const uint16_t* vt = v_cache + ((b * num_kv_heads + kh) * block_size + off) * head_dim;
          for (int32_t i = 0; i < head_dim; ++i) acc[i] += w * widen(vt[i], dtype);
        }
        for (int32_t i = 0; i < head_dim; ++i) o[i] = acc[i] / l;
      }
    }
    free(z);
    free(acc);
  }
  return failed ? ORACLE_NO_MEMORY : ORACLE_OK;
}
