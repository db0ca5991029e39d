// pa_mfma_fp8.h -- TileWave8: the per-wave machinery of decode over 8-bit
// KV pools (OCP FP8 E4M3 codes, one float32 scale per pool).  Same contract
// as TileWave (pa_mfma.h) with a tile of 32 positions.
//
// Quantising the KV cache is the pages' lever on bytes per token ("What
// problem does PagedAttention solve, and what is continuous batching?",
// sections "Why the KV cache becomes the problem" and "What they'll ask
// next"); they fix no format.  Every E4M3 value is exactly a bf16 and an
// fp16 value, so codes are widened in registers (v_cvt_scalef32_pk_*_fp8,
// scale 1) and the products run on the same 16-bit MFMAs as the 16-bit path;
// k_scale is folded into the score scale and v_scale into the output by the
// caller.
//
// Why 32 positions: at one byte per element a 16-position tile moves half
// the bytes of the 16-bit one, and with one tile in flight per wave the HBM
// queue would hold half as much.  A 32-position tile keeps the bytes per
// wave in flight and makes P.V one 16x16x32 MFMA per 16 columns:
//
//  loads   K: the tile is two halves of 16 rows; lane l loads 16 bytes of
//          row (half u, position l%16), d = 64c + 16*(l/16) .. +16, c < D/64.
//          V: straight into the wave's LDS tile, stored as four regions of
//          8 rows (region i: rows 4i..4i+3 of each half), 16 bytes of padding
//          after each region so the four lane groups of a read hit disjoint
//          banks.
//  q.K^T   per half, D/32 v_mfma_f32_16x16x32: the 16 codes of a load are
//          widened to two 8-element operands, the first for d = 64c +
//          16*grp + 0..7 and the second for + 8..15; q is held in the same
//          d order.  Lane l receives head l%16's scores for positions
//          4*(l/16) + r of each half.
//  P.V     2 D/16 v_mfma_f32_16x16x32 with the 32 positions on k in the
//          order (half 0: 4*grp + 0..3, half 1: 4*grp + 0..3) for lane group
//          grp: that is exactly what the lane holds of P after q.K^T, and
//          exactly the 8 rows of region grp of the V tile.  Each float32
//          weight is split as in TileWave into hi = round(p) and lo =
//          round(p - hi), one MFMA per part against the same V operand, so
//          the weights err by 2^-16 of p (bf16) and not by the 2^-8 a single
//          rounding leaves, which would err in proportion to |V|.  The B
//          operand of MFMA m (the 8 rows' bytes of column 16 m + col) is one
//          LDS transpose read (ds_read_b64_tr_b8) widened to 16 bits.
//          Reading it byte by byte instead costs 64 LDS reads per tile and
//          10% of the mixed decode step; reading whole rows and transposing
//          in registers, 3%.  The denominator sums the float32 weights.
#pragma once

#include "pa_mfma.h"

namespace pa {

struct FP8 {};  // tag: pools of OCP E4M3 codes

template <int D>
struct Geo8 {
  static constexpr int ROW = D;                 // bytes of one row
  static constexpr int REGION = 8 * ROW + 16;   // 8 rows + padding
  static constexpr int TILE = 4 * REGION;       // one LDS V tile
  static constexpr int LANES = 8 * ROW / 16;    // lanes that fill a region
};

// Four E4M3 codes (one word) -> four 16-bit values in two words, exactly.
template <typename T> __device__ __forceinline__ uint2 widen4(uint32_t w);
template <> __device__ __forceinline__ uint2 widen4<BF16>(uint32_t w) {
  return make_uint2(
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false)),
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true)));
}
template <> __device__ __forceinline__ uint2 widen4<F16>(uint32_t w) {
  return make_uint2(
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false)),
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true)));
}
template <typename T> __device__ __forceinline__ uint4 widen8(uint32_t w0, uint32_t w1) {
  const uint2 a = widen4<T>(w0), b = widen4<T>(w1);
  return make_uint4(a.x, a.y, b.x, b.y);
}

// The NM byte-transpose reads of an 8-bit V tile for one lane (column block
// m at byte offset 16 m from a), as one asm block that waits for its own
// results, for the reason given at read_v_tr_twice: builtins would make the
// compiler wait for every LDS copy in flight, the next tiles' included.
template <int NM>
__device__ __forceinline__ void read_v_tr8(uint2 (&w)[NM], uint32_t a) {
  static_assert(NM == 4 || NM == 8, "head_dim 64 or 128");
  if constexpr (NM == 8) {
    asm volatile(
        "ds_read_b64_tr_b8 %0, %8\n\t"
        "ds_read_b64_tr_b8 %1, %8 offset:16\n\t"
        "ds_read_b64_tr_b8 %2, %8 offset:32\n\t"
        "ds_read_b64_tr_b8 %3, %8 offset:48\n\t"
        "ds_read_b64_tr_b8 %4, %8 offset:64\n\t"
        "ds_read_b64_tr_b8 %5, %8 offset:80\n\t"
        "ds_read_b64_tr_b8 %6, %8 offset:96\n\t"
        "ds_read_b64_tr_b8 %7, %8 offset:112\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(w[0]), "=&v"(w[1]), "=&v"(w[2]), "=&v"(w[3]), "=&v"(w[4]), "=&v"(w[5]),
          "=&v"(w[6]), "=&v"(w[7])
        : "v"(a)
        : "memory");
  } else {
    asm volatile(
        "ds_read_b64_tr_b8 %0, %4\n\t"
        "ds_read_b64_tr_b8 %1, %4 offset:16\n\t"
        "ds_read_b64_tr_b8 %2, %4 offset:32\n\t"
        "ds_read_b64_tr_b8 %3, %4 offset:48\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(w[0]), "=&v"(w[1]), "=&v"(w[2]), "=&v"(w[3])
        : "v"(a)
        : "memory");
  }
}

template <typename T, int D, int BS, int G>
struct TileWave8 {
  using GE = Geo8<D>;
  using Out = T;
  using Elem = uint8_t;
  static_assert(G <= 16, "one MFMA row per query head");
  static constexpr int kD = D, kBS = BS, kG = G;
  static constexpr int kTileLen = 32;
  static constexpr int KC = D / 32;              // q.K^T MFMA steps per half
  static constexpr int KCH = D / 64;             // 16-byte K loads per half
  static constexpr int KL = 2 * KCH;             // 16-byte K loads per lane per tile
  static constexpr int NM = D / 16;              // P.V MFMAs
  static constexpr int kIds = BS < kTileLen ? kTileLen / BS : 1;
  static constexpr int kTileBytes = GE::TILE;

  const uint8_t* kc;
  const uint8_t* vc;
  int64_t blk_stride;  // bytes per block of a pool
  int64_t head_off;    // bytes to the KV head within a block
  unsigned char* vtile;
  int lane, col, grp;

  struct QRegs {     // q operand, step 2c + h: head col, d = 64c + 16 grp + 8h .. +8
    uint4 r[KC];
  };
  QRegs qr;
  f32x4_t acc[NM];   // P.V accumulators: head 4*grp + r, column 16*m + col
  float m_run;       // running max of head col
  float l_run;       // this lane's share of head col's denominator

  __device__ __forceinline__ void init(const uint8_t* kc_, const uint8_t* vc_, int hkv, int kh,
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

  static __device__ __forceinline__ void fetch_q(QRegs& dst, const uint16_t* q_rows) {
    const int l = threadIdx.x & 63, c16 = l & 15, g4 = l >> 4;
#pragma unroll
    for (int c = 0; c < KCH; ++c) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        dst.r[2 * c + h] = make_uint4(0u, 0u, 0u, 0u);
        if (c16 < G)
          dst.r[2 * c + h] =
              *reinterpret_cast<const uint4*>(q_rows + c16 * D + 64 * c + 16 * g4 + 8 * h);
      }
    }
  }
  __device__ __forceinline__ void load_q(const uint16_t* q_rows) { fetch_q(qr, q_rows); }

  __device__ __forceinline__ void reset() {
#pragma unroll
    for (int m = 0; m < NM; ++m) acc[m] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    m_run = kNegInf;
    l_run = 0.0f;
  }

  // Byte offset of the KV head's rows in the block holding position t
  // (t0 <= t < t0 + 32), picked from the tile's block offsets.
  __device__ __forceinline__ uint64_t block_of(int t, int t0, const uint64_t (&boff)[kIds]) const {
    uint64_t o = boff[0];
#pragma unroll
    for (int j = 1; j < kIds; ++j)
      if (t - t0 >= j * BS) o = boff[j];
    return o;
  }

  // Issue the K (registers) and V (LDS buffer buf) loads of the tile at
  // positions t0..t0+31, clamped to t_last; ids[j] is the block of positions
  // t0 + j * BS ... (entries past t_last are not used).  The ids are the
  // same in every lane, so their offsets are scalar work; a lane only
  // picks one.  Positions are never negative: the row within a block is an
  // unsigned remainder, one AND (signed, five instructions).
  __device__ __forceinline__ void issue_ids(uint4 (&kr)[KL], int buf, int t0, int t_last,
                                            const int (&ids)[kIds]) {
    uint64_t boff[kIds];
#pragma unroll
    for (int j = 0; j < kIds; ++j)
      boff[j] = (uint64_t)(uint32_t)ids[j] * (uint64_t)blk_stride + (uint64_t)head_off;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int t = min(t0 + 16 * u + col, t_last);
      const uint8_t* p = kc + block_of(t, t0, boff) + ((uint32_t)t % BS) * D + grp * 16;
#pragma unroll
      for (int c = 0; c < KCH; ++c) kr[u * KCH + c] = load_stream(p + c * 64);
    }
    // V: lane l (< LANES) loads row r8 = l / (D/16) of region i, 16-byte
    // chunk l % (D/16), landing at region i + 16 l bytes
    unsigned char* vt = vtile + buf * GE::TILE;
    const int r8 = lane / (D / 16);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tau = r8 < 4 ? 4 * i + r8 : 16 + 4 * i + (r8 - 4);
      const int t = min(t0 + tau, t_last);
      const uint8_t* vrow = vc + block_of(t, t0, boff) + ((uint32_t)t % BS) * D;
      if (GE::LANES == 64 || lane < GE::LANES)
        __builtin_amdgcn_global_load_lds(
            (const void*)(vrow + (lane % (D / 16)) * 16),
            (void __attribute__((address_space(3)))*)(vt + i * GE::REGION), 16, 0,
            kCachePolicyStream);
    }
  }

  __device__ __forceinline__ void consume(const uint4 (&kr)[KL], int buf, int t0, int t_end,
                                          float qk_scale) {
    f32x4_t sc[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      sc[u] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int c = 0; c < KCH; ++c) {
        const uint4 k8 = kr[u * KCH + c];
        sc[u] = mfma_k32<T>(widen8<T>(k8.x, k8.y), qr.r[2 * c], sc[u]);
        sc[u] = mfma_k32<T>(widen8<T>(k8.z, k8.w), qr.r[2 * c + 1], sc[u]);
      }
    }

    float sr[8];
    float lm = kNegInf;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float v = (t0 + 16 * u + 4 * grp + r < t_end) ? sc[u][r] * qk_scale : kNegInf;
        sr[4 * u + r] = v;
        lm = fmaxf(lm, v);
      }
    }
    if (__builtin_amdgcn_ballot_w64(lm > m_run + kRescaleSlack) != 0) {
      float mx = fmaxf(lm, __shfl_xor(lm, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx);
      const float corr = exp2_fast(m_run - m_new);  // 0 when m_run = -inf
      m_run = m_new;
      l_run *= corr;
      f32x4_t cr;
#pragma unroll
      for (int r = 0; r < 4; ++r) cr[r] = __shfl(corr, 4 * grp + r);
#pragma unroll
      for (int m = 0; m < NM; ++m) acc[m] = acc[m] * cr;
    }
    float pw[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) pw[j] = exp2_fast(sr[j] - m_run);
    l_run += ((pw[0] + pw[1]) + (pw[2] + pw[3])) + ((pw[4] + pw[5]) + (pw[6] + pw[7]));
    uint32_t ph[4], pl[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      ph[j] = pack2<T>(pw[2 * j], pw[2 * j + 1]);
      pl[j] = pack2<T>(pw[2 * j] - lo_f32<T>(ph[j]), pw[2 * j + 1] - hi_f32<T>(ph[j]));
    }
    const uint4 pa_hi = make_uint4(ph[0], ph[1], ph[2], ph[3]);
    const uint4 pa_lo = make_uint4(pl[0], pl[1], pl[2], pl[3]);

    // B operand of MFMA m: V[row j of region grp][16 m + col], j = 0..7.
    // ds_read_b64_tr_b8 transposes within each group of 16 lanes: lanes 2j
    // and 2j + 1 give the two 8-byte halves of row j (columns 16 m ..
    // 16 m + 15) and lane col receives byte col of every row.
    const unsigned char* vb =
        vtile + buf * GE::TILE + grp * GE::REGION + (col >> 1) * GE::ROW + 8 * (col & 1);
    uint2 w[NM];
    wait_vmem_all();  // as TileWave's consume with kDrain
    read_v_tr8<NM>(w, (uint32_t)(uintptr_t)vb);
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      const uint4 vop = widen8<T>(w[m].x, w[m].y);
      acc[m] = mfma_k32<T>(pa_hi, vop, acc[m]);
      acc[m] = mfma_k32<T>(pa_lo, vop, acc[m]);
    }
  }

  __device__ __forceinline__ void finish() {
    l_run += __shfl_xor(l_run, 16);
    l_run += __shfl_xor(l_run, 32);
  }

  __device__ __forceinline__ void stage(float* st, bool whole, bool bad, float scale) const {
    stage_mfma_result<G, D, NM>(st, acc, l_run, whole, bad, scale);
  }
  __device__ __forceinline__ float2 ml_of_lane() const { return make_float2(m_run, l_run); }
};

}  // namespace pa
