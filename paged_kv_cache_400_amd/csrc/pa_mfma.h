// pa_mfma.h -- the per-wave machinery of the matrix-core decode kernels
// (gfx950): MFMA wrappers, the LDS layout of a V tile, and TileWave, which
// loads and consumes tiles of 16 positions x G query heads.
//
// A tile of 16 positions (one KV head) is handled as follows:
//
//  loads   K goes to registers, V goes straight from HBM into the wave's LDS
//          tile (global_load_lds_dwordx4, no VGPRs), both with the streaming
//          (nt) hint.  The caller issues a tile one step ahead of consuming
//          it.  A position past the end of the range is clamped to the last
//          valid one (so no unused slot is ever read) and its score masked.
//  q.K^T   S[t][h] = sum_d K[t][d] q[h][d] as D/32 v_mfma_f32_16x16x32
//          (A = K rows: lane l holds 16 bytes of position l%16; B = q:
//          lane l holds the same 16 bytes of head l%16, zero for l%16 >= G).
//          The d-chunk of lane l at step c is c*4 + l/16, so a load
//          instruction reads 64 contiguous bytes of each of 16 rows.  No
//          cross-lane reduction: lane l receives head l%16's scores for
//          positions 4*(l/16)+r, r = 0..3.
//  softmax scores in base 2 (scale * log2 e folded in).  The running max of
//          a head is raised only when a score exceeds it by more than 8
//          (then every weight stays <= 2^8); that test is a wave-wide
//          ballot, so the usual tile needs no lane exchange and no rescale.
//  P.V     acc[h][d] += sum_t P[h][t] V[t][d] as D/16 v_mfma_f32_16x16x32.
//          Each float32 weight p is split into two values of the input
//          type, hi = round(p) and lo = round(p - hi), so hi + lo equals p
//          to 2^-16 of p (bf16; 2^-22 for fp16) instead of the 2^-8 one
//          rounding leaves (bf16), which would err in proportion to |V|.  The
//          32-long k axis of the MFMA holds the 16 positions twice: lane
//          group g's 8 k-values are (hi of positions 4g..4g+3, lo of the
//          same), and the V operand is the same 4 rows twice, so
//          sum_k A B = sum_t (hi_t + lo_t) V_t.  On gfx950 the 16x16x32 form
//          issues at the rate of the 16x16x16 one, so the split costs no
//          matrix-core time.  A = the weights, straight from the q.K^T
//          result's layout; the V tile is stored as four 4-row regions,
//          each padded by 32 bytes, and lane group g's 4 rows of column
//          16 m + col are one LDS transpose read (ds_read_b64_tr_b16) from
//          region g.
//  The softmax denominator sums the float32 weights.  MFMA rows for heads
//  >= G compute on zero queries and are never written.
#pragma once

#include "pa_device.h"

namespace pa {

constexpr int kTile = 16;             // positions per tile
constexpr float kRescaleSlack = 8.0f;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

template <typename T> __device__ __forceinline__ f32x4_t mfma_k32(uint4 a, uint4 b, f32x4_t c);
template <> __device__ __forceinline__ f32x4_t mfma_k32<BF16>(uint4 a, uint4 b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}
template <> __device__ __forceinline__ f32x4_t mfma_k32<F16>(uint4 a, uint4 b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

// Two floats -> two 16-bit values packed in one word (round to nearest even).
template <typename T> __device__ __forceinline__ uint32_t pack2(float lo, float hi);
template <> __device__ __forceinline__ uint32_t pack2<BF16>(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, bf16x2_t{(__bf16)lo, (__bf16)hi});
}
template <> __device__ __forceinline__ uint32_t pack2<F16>(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, f16x2_t{(_Float16)lo, (_Float16)hi});
}

// Four float32 softmax weights as the k-values of a 16x16x32 P.V product:
// (hi of w0..w3, lo of w0..w3), hi = w rounded to T, lo = (w - hi) rounded
// to T; hi + lo is w to 2^-16 of w for bf16 (2^-22 for fp16, down to the
// fp16 subnormal spacing for weights below 2^-2).
template <typename T> __device__ __forceinline__ uint4 split_weights(const float (&w)[4]) {
  const uint32_t h01 = pack2<T>(w[0], w[1]), h23 = pack2<T>(w[2], w[3]);
  const uint32_t l01 = pack2<T>(w[0] - lo_f32<T>(h01), w[1] - hi_f32<T>(h01));
  const uint32_t l23 = pack2<T>(w[2] - lo_f32<T>(h23), w[3] - hi_f32<T>(h23));
  return make_uint4(h01, h23, l01, l23);
}

// s_waitcnt vmcnt(0): every outstanding vector-memory load of this wave,
// the copies of V into LDS included, has landed.  The empty asm with a memory
// clobber keeps the compiler from moving LDS reads above the wait or the next
// LDS copies above the previous tile's reads.
__device__ __forceinline__ void wait_vmem_all() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt 0, expcnt 7, lgkmcnt 15
  asm volatile("" ::: "memory");
}

// s_waitcnt vmcnt(N) (expcnt, lgkmcnt not waited for): the wave's vector
// memory operations but the N most recent have completed.  They complete
// in the order they were issued, so with the N loads of the tiles issued
// after tile j still in flight, this waits for tile j, its V copies into LDS
// included (which only this wait orders before the reads of V).
template <int N>
__device__ __forceinline__ void wait_vmem_but() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0f70);
  asm volatile("" ::: "memory");
}

// The G x D result of a matrix-core tile wave, row-major into st: lane (col,
// grp) holds acc[m][r] for head 4 grp + r, column 16 m + col, and head col's
// whole denominator in l_run (after finish).  whole: divide by the
// denominator (a finished row), else the raw accumulator (a partial state);
// every value times `scale`; NaN everywhere if bad.
template <int G, int D, int NM>
__device__ __forceinline__ void stage_mfma_result(float* st, const f32x4_t (&acc)[NM],
                                                  float l_run, bool whole, bool bad,
                                                  float scale) {
  const int lane = threadIdx.x & 63;
  const int col = lane & 15, grp = lane >> 4;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int h = 4 * grp + r;
    const float l_h = __shfl(l_run, h);
    if (h < G) {
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        const float v = (whole ? acc[m][r] / l_h : acc[m][r]) * scale;
        st[h * D + 16 * m + col] = bad ? __builtin_nanf("") : v;
      }
    }
  }
}

// One 32-bit LDS read at byte address a, completed before the asm ends (for
// the reason given at read_v_tr_twice).
__device__ __forceinline__ uint32_t lds_read_u32(uint32_t a) {
  uint32_t v;
  asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(v) : "v"(a) : "memory");
  return v;
}

// The NM transpose reads of a V tile for one lane (column block m at byte
// offset 32 m from the lane's LDS address a), as one asm block that waits for
// its own results before it ends.  Written as builtins, these reads would
// make the compiler wait first for every LDS copy the wave has in flight (it
// cannot tell the buffers apart), the next tiles' copies included; a driver
// that keeps several tiles in flight must not lose them there.  The
// caller's own vmcnt wait orders the reads after this tile's copies.
// Each read is issued twice, into w and w2: an operand that holds the same
// 64 bits twice (the V operand of the hi and lo weights) then comes straight
// from the reads, where a copy of one read took two moves per matrix-core
// product.  The second reads hit the same LDS lines.
template <int NM>
__device__ __forceinline__ void read_v_tr_twice(uint2 (&w)[NM], uint2 (&w2)[NM], uint32_t a) {
  static_assert(NM == 4 || NM == 8, "head_dim 64 or 128");
  if constexpr (NM == 8) {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %16\n\t"
        "ds_read_b64_tr_b16 %8, %16\n\t"
        "ds_read_b64_tr_b16 %1, %16 offset:32\n\t"
        "ds_read_b64_tr_b16 %9, %16 offset:32\n\t"
        "ds_read_b64_tr_b16 %2, %16 offset:64\n\t"
        "ds_read_b64_tr_b16 %10, %16 offset:64\n\t"
        "ds_read_b64_tr_b16 %3, %16 offset:96\n\t"
        "ds_read_b64_tr_b16 %11, %16 offset:96\n\t"
        "ds_read_b64_tr_b16 %4, %16 offset:128\n\t"
        "ds_read_b64_tr_b16 %12, %16 offset:128\n\t"
        "ds_read_b64_tr_b16 %5, %16 offset:160\n\t"
        "ds_read_b64_tr_b16 %13, %16 offset:160\n\t"
        "ds_read_b64_tr_b16 %6, %16 offset:192\n\t"
        "ds_read_b64_tr_b16 %14, %16 offset:192\n\t"
        "ds_read_b64_tr_b16 %7, %16 offset:224\n\t"
        "ds_read_b64_tr_b16 %15, %16 offset:224\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(w[0]), "=&v"(w[1]), "=&v"(w[2]), "=&v"(w[3]), "=&v"(w[4]), "=&v"(w[5]),
          "=&v"(w[6]), "=&v"(w[7]), "=&v"(w2[0]), "=&v"(w2[1]), "=&v"(w2[2]), "=&v"(w2[3]),
          "=&v"(w2[4]), "=&v"(w2[5]), "=&v"(w2[6]), "=&v"(w2[7])
        : "v"(a)
        : "memory");
  } else {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %8\n\t"
        "ds_read_b64_tr_b16 %4, %8\n\t"
        "ds_read_b64_tr_b16 %1, %8 offset:32\n\t"
        "ds_read_b64_tr_b16 %5, %8 offset:32\n\t"
        "ds_read_b64_tr_b16 %2, %8 offset:64\n\t"
        "ds_read_b64_tr_b16 %6, %8 offset:64\n\t"
        "ds_read_b64_tr_b16 %3, %8 offset:96\n\t"
        "ds_read_b64_tr_b16 %7, %8 offset:96\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(w[0]), "=&v"(w[1]), "=&v"(w[2]), "=&v"(w[3]), "=&v"(w2[0]), "=&v"(w2[1]),
          "=&v"(w2[2]), "=&v"(w2[3])
        : "v"(a)
        : "memory");
  }
}

template <int D>
struct Geo {
  static constexpr int KC = D / 32;                 // q.K^T MFMA steps
  static constexpr int NM = D / 16;                 // P.V MFMAs
  static constexpr int ROW = D * 2;                 // bytes of one V row
  static constexpr int REGION = 4 * ROW + 32;       // 4 rows + padding
  static constexpr int TILE = 4 * REGION;           // one LDS V tile
  static constexpr int LANES = 4 * ROW / 16;        // lanes that fill a region
};

// One wave's softmax state for the G query heads of one KV head, and the
// loading and consuming of its tiles.  vtile points at the wave's two LDS V
// tiles (2 * Geo<D>::TILE bytes).
template <typename T, int D, int BS, int G>
struct TileWave {
  using GE = Geo<D>;
  static constexpr int KC = GE::KC, NM = GE::NM;
  static_assert(G <= 16, "one MFMA row per query head");
  // What the balanced driver needs to know of a tile wave.
  using Out = T;                  // q and output type
  using Elem = uint16_t;          // pool element
  static constexpr int kD = D, kBS = BS, kG = G;
  static constexpr int kTileLen = kTile;                  // positions per tile
  static constexpr int KL = KC;                           // 16-byte K loads per lane
  static constexpr int kIds = BS < kTile ? kTile / BS : 1;  // blocks per tile
  static constexpr int kTileBytes = GE::TILE;             // one LDS V tile

  const uint16_t* kc;
  const uint16_t* vc;
  int64_t blk_stride;  // elements per block of a pool
  int64_t head_off;    // elements to the KV head within a block
  unsigned char* vtile;
  int lane, col, grp;

  struct QRegs {     // q operand (B of q.K^T): head col, d-chunk c*4 + grp
    uint4 r[KC];
  };
  QRegs qr;
  f32x4_t acc[NM];   // P.V accumulators: head 4*grp + r, column 16*m + col
  float m_run;       // running max of head col (same in the 4 lane groups)
  float l_run;       // this lane's share of head col's denominator

  __device__ __forceinline__ void init(const uint16_t* kc_, const uint16_t* vc_, int hkv, int kh,
                                       unsigned char* vtile_) {
    kc = kc_;
    vc = vc_;
    blk_stride = (int64_t)hkv * BS * D;
    head_off = (int64_t)kh * BS * D;
    vtile = vtile_;
    lane = threadIdx.x & 63;
    col = lane & 15;
    grp = lane >> 4;
  }

  // q rows of the G heads start at q_rows ([G][D]); zero operand for col >= G.
  static __device__ __forceinline__ void fetch_q(QRegs& dst, const uint16_t* q_rows) {
    const int l = threadIdx.x & 63, c16 = l & 15, g4 = l >> 4;
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      dst.r[c] = make_uint4(0u, 0u, 0u, 0u);
      if (c16 < G) dst.r[c] = *reinterpret_cast<const uint4*>(q_rows + c16 * D + (c * 4 + g4) * 8);
    }
  }
  __device__ __forceinline__ void load_q(const uint16_t* q_rows) { fetch_q(qr, q_rows); }

  __device__ __forceinline__ void reset() {
#pragma unroll
    for (int m = 0; m < NM; ++m) acc[m] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    m_run = kNegInf;
    l_run = 0.0f;
  }

  // Issue the K (to registers kr) and V (to LDS buffer `buf`) loads of the
  // tile at positions t0..t0+15, clamped to t_last.  id0 is the block of t0;
  // for blocks of 8 positions id1 is the block of t0 + 8.
  __device__ __forceinline__ void issue(uint4 (&kr)[KC], int buf, int t0, int t_last, int id0,
                                        int id1) {
    const uint16_t* kb0 = kc + (int64_t)id0 * blk_stride + head_off;
    const uint16_t* kb1 = kc + (int64_t)id1 * blk_stride + head_off;
    const uint16_t* vb0 = vc + (int64_t)id0 * blk_stride + head_off;
    const uint16_t* vb1 = vc + (int64_t)id1 * blk_stride + head_off;
    // K: position col (clamped), chunk c*4 + grp
    {
      const int t = min(t0 + col, t_last);
      const uint16_t* kr_base = (BS < kTile && t - t0 >= BS) ? kb1 : kb0;
      const uint16_t* ptr = kr_base + ((uint32_t)t % BS) * D + grp * 8;
#pragma unroll
      for (int c = 0; c < KC; ++c) kr[c] = load_stream(ptr + c * 32);
    }
    // V: region i holds rows 4i..4i+3; lane l (< LANES) loads row 4i + l/(D/8),
    // chunk l%(D/8), landing at region i + 16*l bytes
    unsigned char* vt = vtile + buf * GE::TILE;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tau = 4 * i + lane / (D / 8);
      const int t = min(t0 + tau, t_last);
      const uint16_t* vrow =
          ((BS < kTile && t - t0 >= BS) ? vb1 : vb0) + ((uint32_t)t % BS) * D;
      if (GE::LANES == 64 || lane < GE::LANES)
        __builtin_amdgcn_global_load_lds(
            (const void*)(vrow + (lane % (D / 8)) * 8),
            (void __attribute__((address_space(3)))*)(vt + i * GE::REGION), 16, 0,
            kCachePolicyStream);
    }
  }

  // The same, with the tile's block ids in an array (ids[j]: the block of
  // positions t0 + j * BS ...).
  __device__ __forceinline__ void issue_ids(uint4 (&kr)[KC], int buf, int t0, int t_last,
                                            const int (&ids)[kIds]) {
    issue(kr, buf, t0, t_last, ids[0], ids[kIds - 1]);
  }

  // issue_ids with the V copies as buffer loads: every load of the tile is
  // then one the compiler counts, so a driver may keep the next tile in
  // flight and wait for this one with wait_vmem_but<kLoadsPerTile>.  The
  // rows of one copy lie in one block (for 8-position blocks, rows 8..15 in
  // the second one unless all of them clamp back into the first).
  // kNt: the streaming hint on every load (each byte read once, the batch's
  // K/V far larger than the caches); without it, K/V that the last-level
  // cache holds is read from there.  Positions are never negative: the row
  // within a block is an unsigned remainder, one AND (signed, five
  // instructions per address).
  static constexpr int kLoadsPerTile = KL + 4;
  template <bool kNt = true>
  __device__ __forceinline__ void issue_ids_counted(uint4 (&kr)[KC], int buf, int t0, int t_last,
                                                    const int (&ids)[kIds]) {
    const int id0 = ids[0], id1 = ids[kIds - 1];
    {
      const uint16_t* kb0 = kc + (int64_t)id0 * blk_stride + head_off;
      const uint16_t* kb1 = kc + (int64_t)id1 * blk_stride + head_off;
      const int t = min(t0 + col, t_last);
      const uint16_t* ptr =
          ((BS < kTile && t - t0 >= BS) ? kb1 : kb0) + ((uint32_t)t % BS) * D + grp * 8;
#pragma unroll
      for (int c = 0; c < KC; ++c) kr[c] = load_kv<kNt>(ptr + c * 32);
    }
    unsigned char* vt = vtile + buf * GE::TILE;
    const __amdgpu_buffer_rsrc_t r0 = buffer_rsrc(vc + (int64_t)id0 * blk_stride + head_off,
                                                  BS * D * 2);
    const __amdgpu_buffer_rsrc_t r1 = buffer_rsrc(vc + (int64_t)id1 * blk_stride + head_off,
                                                  BS * D * 2);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = min(t0 + 4 * i + lane / (D / 8), t_last);
      const bool second = BS < kTile && 4 * i >= BS && t0 + BS <= t_last;
      const uint32_t off = (((uint32_t)t % BS) * D + (lane % (D / 8)) * 8) * 2;
      if (GE::LANES == 64 || lane < GE::LANES)
        copy_to_lds16<kNt ? kCachePolicyStream : kCachePolicyReuse>(second ? r1 : r0, off,
                                                                     vt + i * GE::REGION);
    }
  }

  // Compute the tile at t0 (positions >= t_end masked) whose K is in kr and
  // V in LDS buffer `buf`.  kDrain: wait for every load the wave has in
  // flight before reading V, the next tile's included.  The decode drivers
  // keep one tile in flight and drain: with the next tile's loads kept in
  // flight through P.V instead, the bandwidth-bound batches ran 0.3-0.5%
  // slower (more scattered requests outstanding than the memory system
  // serves well).  A driver that keeps several tiles in flight and waits for
  // each with wait_vmem_but does not drain.
  template <bool kDrain = true>
  __device__ __forceinline__ void consume(const uint4 (&kr)[KC], int buf, int t0, int t_end,
                                          float qk_scale) {
    f32x4_t sc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int c = 0; c < KC; ++c) sc = mfma_k32<T>(kr[c], qr.r[c], sc);

    float sr[4];
    float lm = kNegInf;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      sr[r] = (t0 + 4 * grp + r < t_end) ? sc[r] * qk_scale : kNegInf;
      lm = fmaxf(lm, sr[r]);
    }
    if (__builtin_amdgcn_ballot_w64(lm > m_run + kRescaleSlack) != 0) {
      float mx = fmaxf(lm, __shfl_xor(lm, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx);
      const float corr = exp2_fast(m_run - m_new);  // 0 when m_run = -inf
      m_run = m_new;
      l_run *= corr;
      // as whole vectors: scaled element by element, the accumulators
      // took new registers, and the path without a rescale copied them
      // there (16 moves a tile)
      f32x4_t cr;
#pragma unroll
      for (int r = 0; r < 4; ++r) cr[r] = __shfl(corr, 4 * grp + r);
#pragma unroll
      for (int m = 0; m < NM; ++m) acc[m] = acc[m] * cr;
    }
    float pw[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) pw[r] = exp2_fast(sr[r] - m_run);
    l_run += (pw[0] + pw[1]) + (pw[2] + pw[3]);
    const uint4 pa_op = split_weights<T>(pw);

    // B operand: V[4*grp + r][16*m + col] from region grp, row r, given
    // twice (for the hi and the lo weights).  ds_read_b64_tr_b16 transposes
    // within each group of 16 lanes: lanes 4r .. 4r + 3 give row r (columns
    // 16 m .. 16 m + 15, 4 each) and lane col receives element col of every
    // row.
    const unsigned char* vb = vtile + buf * GE::TILE + grp * GE::REGION + (col >> 2) * GE::ROW +
                              8 * (col & 3);
    uint2 w[NM], w2[NM];
    if constexpr (kDrain) wait_vmem_all();
    read_v_tr_twice<NM>(w, w2, (uint32_t)(uintptr_t)vb);
#pragma unroll
    for (int m = 0; m < NM; ++m)
      acc[m] = mfma_k32<T>(pa_op, make_uint4(w[m].x, w[m].y, w2[m].x, w2[m].y), acc[m]);
  }

  // After the last tile: every lane holds head col's whole denominator.
  __device__ __forceinline__ void finish() {
    l_run += __shfl_xor(l_run, 16);
    l_run += __shfl_xor(l_run, 32);
  }

  // After finish: the result row-major into st ([G][D] floats), and (m, l)
  // of head `lane` for lanes < G.
  __device__ __forceinline__ void stage(float* st, bool whole, bool bad, float scale) const {
    stage_mfma_result<G, D, NM>(st, acc, l_run, whole, bad, scale);
  }
  __device__ __forceinline__ float2 ml_of_lane() const { return make_float2(m_run, l_run); }
};

}  // namespace pa
