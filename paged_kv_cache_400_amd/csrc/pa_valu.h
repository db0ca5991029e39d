// pa_valu.h -- TileWaveV: the per-wave machinery of decode on the vector
// unit alone (no matrix cores), for the balanced driver of decode_streamk.h.
// Same contract as TileWave (pa_mfma.h): tiles of 16 positions of one KV
// head for its G query heads, each tile issued one tile ahead of its use.
//
//  lanes   a position row of D elements is D/8 lanes holding 16 bytes each
//          (16 lanes at d 128, 8 at d 64), so one 16-byte load per lane
//          reads 64/(D/8) whole rows (1 KiB) and a tile is 16/(64/(D/8))
//          loads of K and as many of V, both straight to registers with the
//          streaming hint.
//  q.K     per load and head: four v_dot2_f32_{bf16,f16} over the lane's 8
//          elements, then a DPP butterfly over the row's lanes (4 steps at
//          d 128, 3 at d 64), after which every lane of the row holds the
//          score.  This is the wave-level form of the dot product: the
//          reduction the matrix cores do inside one instruction costs here
//          one exchange step per halving.
//  softmax the positions a lane sees (its row of every load) form their own
//          stream with its own running max and sum; the streams of the rows
//          are merged by log-sum-exp after the last tile.  Base 2, the
//          scale times log2 e folded into the scores; the running max is
//          raised only when a score exceeds it by more than 8, decided by a
//          wave-wide ballot, as in TileWave.
//  P.V     float32 FMAs, acc[h][e] += p V[e], over the lane's 8 elements;
//          the weights stay float32.
// Every exponential is computed by all D/8 lanes of a row (the row's lanes
// hold the same score), and q.K needs its exchange steps: the cost the
// matrix-core tile wave avoids.  Both are kept so the two can be measured on
// the same driver, run for run.
#pragma once

#include "pa_device.h"
#include "pa_mfma.h"

namespace pa {

struct Vec {};  // tag: 16-bit pools, vector-unit tile wave

template <typename T, int D, int BS, int G>
struct TileWaveV {
  static_assert(D == 64 || D == 128, "head_dim 64 or 128");
  using Out = T;
  using Elem = uint16_t;
  static constexpr int kD = D, kBS = BS, kG = G;
  static constexpr int LPT = D / 8;              // lanes per position row
  static constexpr int RPL = 64 / LPT;           // rows per load instruction
  static constexpr int kTileLen = 16;            // positions per tile
  static constexpr int NI = kTileLen / RPL;      // loads per tile, of K and of V each
  static constexpr int KL = 2 * NI;              // kr[0, NI): K, kr[NI, 2 NI): V
  static constexpr int kIds = BS < kTileLen ? kTileLen / BS : 1;
  static constexpr int kTileBytes = G * D * 4;   // LDS: the result's staging only

  const uint16_t* kc;
  const uint16_t* vc;
  int64_t blk_stride;  // elements per block of a pool
  int64_t head_off;    // elements to the KV head within a block
  int lane, row, col;

  struct QRegs {       // q of head h, elements 8 col .. 8 col + 7
    uint4 r[G];
  };
  QRegs qr;
  float acc[G][8];     // the lane's stream: sum of p V over its 8 elements
  float m[G], l[G];    // the lane's stream: running max and sum

  __device__ __forceinline__ void init(const uint16_t* kc_, const uint16_t* vc_, int hkv, int kh,
                                       unsigned char*) {
    kc = kc_;
    vc = vc_;
    blk_stride = (int64_t)hkv * BS * D;
    head_off = (int64_t)kh * BS * D;
    lane = threadIdx.x & 63;
    row = lane / LPT;
    col = lane % LPT;
  }

  static __device__ __forceinline__ void fetch_q(QRegs& dst, const uint16_t* q_rows) {
    const int c = (threadIdx.x & 63) % LPT;
#pragma unroll
    for (int h = 0; h < G; ++h) dst.r[h] = *reinterpret_cast<const uint4*>(q_rows + h * D + c * 8);
  }
  __device__ __forceinline__ void load_q(const uint16_t* q_rows) { fetch_q(qr, q_rows); }

  __device__ __forceinline__ void reset() {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      m[h] = kNegInf;
      l[h] = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] = 0.0f;
    }
  }

  // Offset (elements) of the KV head's rows in the block holding position
  // t (t0 <= t < t0 + 16), picked from the tile's block offsets.
  __device__ __forceinline__ uint64_t block_of(int t, int t0, const uint64_t (&boff)[kIds]) const {
    uint64_t o = boff[0];
#pragma unroll
    for (int j = 1; j < kIds; ++j)
      if (t - t0 >= j * BS) o = boff[j];
    return o;
  }

  // Issue the K and V loads of the tile at positions t0..t0+15, clamped to
  // t_last (a clamped row re-reads the last valid position; its score is
  // masked).  ids[j] is the block of positions t0 + j * BS ...; the ids are
  // the same in every lane, so their offsets are scalar work.  Positions are
  // never negative: the row within a block is an unsigned remainder.
  __device__ __forceinline__ void issue_ids(uint4 (&kr)[KL], int, int t0, int t_last,
                                            const int (&ids)[kIds]) {
    uint64_t boff[kIds];
#pragma unroll
    for (int j = 0; j < kIds; ++j)
      boff[j] = (uint64_t)(uint32_t)ids[j] * (uint64_t)blk_stride + (uint64_t)head_off;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int t = min(t0 + i * RPL + row, t_last);
      const uint64_t off = block_of(t, t0, boff) + ((uint32_t)t % BS) * D + col * 8;
      kr[i] = load_stream(kc + off);
      kr[NI + i] = load_stream(vc + off);
    }
  }

  // Compute the tile at t0 (positions >= t_end masked) whose K and V are in kr.
  __device__ __forceinline__ void consume(const uint4 (&kr)[KL], int, int t0, int t_end,
                                          float qk_scale) {
    bool valid[NI];
    float s[NI][G];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      valid[i] = t0 + i * RPL + row < t_end;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float a = dot2<T>(qr.r[h].x, kr[i].x, 0.0f);
        a = dot2<T>(qr.r[h].y, kr[i].y, a);
        a = dot2<T>(qr.r[h].z, kr[i].z, a);
        a = dot2<T>(qr.r[h].w, kr[i].w, a);
        s[i][h] = valid[i] ? group_sum<LPT>(a) * qk_scale : kNegInf;
      }
    }
    bool raise = false;
    float mx[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      mx[h] = s[0][h];
#pragma unroll
      for (int i = 1; i < NI; ++i) mx[h] = fmaxf(mx[h], s[i][h]);
      raise |= mx[h] > m[h] + kRescaleSlack;
    }
    if (__builtin_amdgcn_ballot_w64(raise) != 0) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float mn = fmaxf(m[h], mx[h]);
        const float corr = (mn == m[h]) ? 1.0f : exp2_fast(m[h] - mn);  // 0 from -inf
        m[h] = mn;
        l[h] *= corr;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] *= corr;
      }
    }
    float vf[NI][8];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const uint4 v = kr[NI + i];
      vf[i][0] = lo_f32<T>(v.x);
      vf[i][1] = hi_f32<T>(v.x);
      vf[i][2] = lo_f32<T>(v.y);
      vf[i][3] = hi_f32<T>(v.y);
      vf[i][4] = lo_f32<T>(v.z);
      vf[i][5] = hi_f32<T>(v.z);
      vf[i][6] = lo_f32<T>(v.w);
      vf[i][7] = hi_f32<T>(v.w);
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        // a valid score has m[h] >= it - 8 (finite); a masked one weighs 0
        const float p = valid[i] ? exp2_fast(s[i][h] - m[h]) : 0.0f;
        l[h] += p;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(p, vf[i][e], acc[h][e]);
      }
    }
  }

  // After the last tile: the rows' streams merged by log-sum-exp, so every
  // lane holds the whole state of its 8 elements.
  __device__ __forceinline__ void finish() {
#pragma unroll
    for (int mask = LPT; mask < 64; mask <<= 1) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float mo = __shfl_xor(m[h], mask);
        const float lo = __shfl_xor(l[h], mask);
        const float mn = fmaxf(m[h], mo);
        const float base = (mn == kNegInf) ? 0.0f : mn;
        const float f = exp2_fast(m[h] - base), fo = exp2_fast(mo - base);
        l[h] = l[h] * f + lo * fo;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float ao = __shfl_xor(acc[h][e], mask);
          acc[h][e] = acc[h][e] * f + ao * fo;
        }
        m[h] = mn;
      }
    }
  }

  // The result row-major into st ([G][D] floats), by the lanes of row 0.
  __device__ __forceinline__ void stage(float* st, bool whole, bool bad, float scale) const {
    if (row != 0) return;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float o[8];
#pragma unroll
      for (int e = 0; e < 8; ++e)
        o[e] = bad ? __builtin_nanf("") : (whole ? acc[h][e] / l[h] : acc[h][e]) * scale;
      *reinterpret_cast<float4*>(st + h * D + col * 8) = make_float4(o[0], o[1], o[2], o[3]);
      *reinterpret_cast<float4*>(st + h * D + col * 8 + 4) = make_float4(o[4], o[5], o[6], o[7]);
    }
  }

  // (m, l) of head `lane`, for lanes < G (0 bits for the others).  Built by
  // masking, with the mask hidden from the optimizer: written as a chain of
  // selects, it became an index into m[] and l[] by the lane, which put the
  // whole tile wave's state in scratch memory at G >= 4.
  __device__ __forceinline__ float2 ml_of_lane() const {
    uint32_t rm = 0u, rl = 0u;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      uint32_t sel = lane == h ? 0xffffffffu : 0u;
      asm volatile("" : "+v"(sel));
      rm |= __float_as_uint(m[h]) & sel;
      rl |= __float_as_uint(l[h]) & sel;
    }
    return make_float2(__uint_as_float(rm), __uint_as_float(rl));
  }
};

}  // namespace pa
