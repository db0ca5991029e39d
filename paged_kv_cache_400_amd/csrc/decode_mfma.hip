// decode_mfma.hip -- paged decode attention with q.K^T and P.V on the matrix
// cores (gfx950 MFMA), for head_dim 64/128, block 8/16/32, group 1..8.
//
// Same result and work decomposition as the VALU kernel (decode.hip): one
// workgroup of 4 waves per (sequence, KV head, partition), numbered
// partition-major so that the XCDs share the work evenly, waves taking
// 16-position tiles in turn, a per-wave online softmax in base 2, a
// log-sum-exp merge of the waves and, for split sequences, of the partitions.
// How a wave handles a tile of 16 positions x G query heads:
//
//  loads   K goes to registers, V goes straight from HBM into the wave's LDS
//          tile (global_load_lds_dwordx4, no VGPRs), both with the
//          streaming (nt) hint.  Both are issued one tile ahead: the loop
//          waits for tile k, issues tile k+1, then computes tile k.  Block ids are wave-uniform scalar loads; a
//          position past the end is clamped to the last valid one (so no
//          unused slot is ever read) and its score is masked.
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
//  P.V     acc[h][d] += sum_t P[h][t] V[t][d] as D/16 v_mfma_f32_16x16x16
//          (A = P: the q.K^T result is already in the A layout; B = V with
//          the 16 positions along k, read column-wise from LDS as 16-bit
//          values).  The V tile is stored as four 4-row regions, each
//          padded by 32 bytes, so the four lane groups of a read hit
//          disjoint LDS banks and every read address is a lane base plus an
//          immediate offset.
//  P is rounded to the input type for the P.V product and the softmax
//  denominator sums the same rounded weights.
//
// MFMA rows for heads >= G compute on zero queries and are never written.
#include "pa_device.h"
#include "pa_launch.h"

namespace pa {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kTile = 16;          // positions per tile
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

template <typename T> __device__ __forceinline__ f32x4_t mfma_k16(uint2 a, uint2 b, f32x4_t c);
template <> __device__ __forceinline__ f32x4_t mfma_k16<BF16>(uint2 a, uint2 b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4_t, a),
                                                   __builtin_bit_cast(i16x4_t, b), c, 0, 0, 0);
}
template <> __device__ __forceinline__ f32x4_t mfma_k16<F16>(uint2 a, uint2 b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4_t, a),
                                               __builtin_bit_cast(f16x4_t, b), c, 0, 0, 0);
}

// Two floats -> two 16-bit values packed in one word (round to nearest even).
template <typename T> __device__ __forceinline__ uint32_t pack2(float lo, float hi);
template <> __device__ __forceinline__ uint32_t pack2<BF16>(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, bf16x2_t{(__bf16)lo, (__bf16)hi});
}
template <> __device__ __forceinline__ uint32_t pack2<F16>(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, f16x2_t{(_Float16)lo, (_Float16)hi});
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

template <int D>
struct Geo {
  static constexpr int KC = D / 32;                 // q.K^T MFMA steps
  static constexpr int NM = D / 16;                 // P.V MFMAs
  static constexpr int ROW = D * 2;                 // bytes of one V row
  static constexpr int REGION = 4 * ROW + 32;       // 4 rows + padding
  static constexpr int TILE = 4 * REGION;           // one LDS V tile
  static constexpr int LANES = 4 * ROW / 16;        // lanes that fill a region
};

}  // namespace

template <typename T, int D, int BS, int G>
__global__ void __launch_bounds__(kThreads)
pa_decode_mfma(uint16_t* __restrict__ out, float* __restrict__ ws_acc, float2* __restrict__ ws_ml,
               const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
               const uint16_t* __restrict__ vc, const int32_t* __restrict__ block_tables,
               const int32_t* __restrict__ seq_lens, int32_t hkv, int32_t mb, int32_t nb,
               int32_t part, int32_t pmax, float qk_scale) {
  using GE = Geo<D>;
  constexpr int KC = GE::KC, NM = GE::NM;
  static_assert(G <= 16, "one MFMA row per query head");
  static_assert(kWaves * 2 * GE::TILE >= (int)(sizeof(float) * kWaves * G * (D + 2)),
                "merge buffers alias the V tiles");

  // per wave: two V tiles (double buffer); reused for the wave merge
  __shared__ __attribute__((aligned(16))) unsigned char s_mem[kWaves * 2 * GE::TILE];
  __shared__ int s_bad[kWaves];

  const Unit u = unit_of(blockIdx.x, hkv, pmax);
  const int s = u.s, kh = u.kh, p = u.p;
  const int hq = hkv * G;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, grp = lane >> 4;
  const int64_t row0 = (int64_t)s * hq + (int64_t)kh * G;

  const int L = seq_lens[s];
  if (L < 0 || (int64_t)L > (int64_t)mb * BS) {
    if (p == 0)
      for (int i = tid; i < G * D; i += kThreads) out[row0 * D + i] = to_bits<T>(__builtin_nanf(""));
    return;
  }
  const int t_begin = p * part;
  if (t_begin >= L) {
    if (p == 0)
      for (int i = tid; i < G * D; i += kThreads) out[row0 * D + i] = to_bits<T>(0.0f);
    return;
  }
  const int t_end = min(L, t_begin + part);
  const int nparts = (L + part - 1) / part;
  const int ntiles = (t_end - t_begin + kTile - 1) / kTile;
  const int32_t* bt_row = block_tables + (int64_t)s * mb;
  const int64_t blk_stride = (int64_t)hkv * BS * D;  // elements
  const int64_t head_off = (int64_t)kh * BS * D;

  // q operand (B of q.K^T): head col, d-chunk c*4 + grp; zero for col >= G
  uint4 qb[KC];
#pragma unroll
  for (int c = 0; c < KC; ++c) {
    qb[c] = make_uint4(0u, 0u, 0u, 0u);
    if (col < G) qb[c] = *reinterpret_cast<const uint4*>(q + (row0 + col) * D + (c * 4 + grp) * 8);
  }

  unsigned char* vtile = s_mem + w * 2 * GE::TILE;
  bool bad = false;

  // Issue the K (to registers) and V (to LDS buffer `buf`) loads of the tile
  // that starts at position t0.
  auto issue = [&](uint4 (&kr)[KC], int buf, int t0) {
    int id0 = bt_row[t0 / BS];
    int id1 = id0;
    if constexpr (BS < kTile) id1 = (t0 + BS < t_end) ? bt_row[t0 / BS + 1] : id0;
    if (id0 < 0 || id0 >= nb) { bad = true; id0 = 0; }
    if (id1 < 0 || id1 >= nb) { bad = true; id1 = 0; }
    const uint16_t* kb0 = kc + (int64_t)id0 * blk_stride + head_off;
    const uint16_t* kb1 = kc + (int64_t)id1 * blk_stride + head_off;
    const uint16_t* vb0 = vc + (int64_t)id0 * blk_stride + head_off;
    const uint16_t* vb1 = vc + (int64_t)id1 * blk_stride + head_off;
    // K: position col (clamped), chunk c*4 + grp
    {
      const int t = min(t0 + col, t_end - 1);
      const uint16_t* kr_base = (BS < kTile && t - t0 >= BS) ? kb1 : kb0;
      const uint16_t* ptr = kr_base + (t % BS) * D + grp * 8;
#pragma unroll
      for (int c = 0; c < KC; ++c) kr[c] = load_stream(ptr + c * 32);
    }
    // V: region i holds rows 4i..4i+3; lane l (< LANES) loads row 4i + l/(D/8),
    // chunk l%(D/8), landing at region i + 16*l bytes
    unsigned char* vt = vtile + buf * GE::TILE;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tau = 4 * i + lane / (D / 8);
      const int t = min(t0 + tau, t_end - 1);
      const uint16_t* vrow = ((BS < kTile && t - t0 >= BS) ? vb1 : vb0) + (t % BS) * D;
      if (GE::LANES == 64 || lane < GE::LANES)
        __builtin_amdgcn_global_load_lds(
            (const void*)(vrow + (lane % (D / 8)) * 8),
            (void __attribute__((address_space(3)))*)(vt + i * GE::REGION), 16, 0,
            kCachePolicyStream);
    }
  };

  f32x4_t acc[NM];
#pragma unroll
  for (int m = 0; m < NM; ++m) acc[m] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  float m_run = kNegInf;  // running max of head col (same in the 4 lane groups)
  float l_run = 0.0f;     // this lane's share of head col's denominator

  // Compute the tile at t0 whose K is in kr and V in LDS buffer `buf`.
  auto consume = [&](const uint4 (&kr)[KC], int buf, int t0) {
    f32x4_t sc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int c = 0; c < KC; ++c) sc = mfma_k32<T>(kr[c], qb[c], sc);

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
      float cr[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) cr[r] = __shfl(corr, 4 * grp + r);
#pragma unroll
      for (int m = 0; m < NM; ++m) {
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[m][r] *= cr[r];
      }
    }
    const uint32_t p01 = pack2<T>(exp2_fast(sr[0] - m_run), exp2_fast(sr[1] - m_run));
    const uint32_t p23 = pack2<T>(exp2_fast(sr[2] - m_run), exp2_fast(sr[3] - m_run));
    l_run += (lo_f32<T>(p01) + hi_f32<T>(p01)) + (lo_f32<T>(p23) + hi_f32<T>(p23));
    const uint2 pa_op = make_uint2(p01, p23);

    // B operand: V[4*grp + r][16*m + col] from region grp, row r
    const uint16_t* vr = reinterpret_cast<const uint16_t*>(vtile + buf * GE::TILE +
                                                           grp * GE::REGION) + col;
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      const uint32_t b0 = vr[0 * D + 16 * m];
      const uint32_t b1 = vr[1 * D + 16 * m];
      const uint32_t b2 = vr[2 * D + 16 * m];
      const uint32_t b3 = vr[3 * D + 16 * m];
      acc[m] = mfma_k16<T>(pa_op, make_uint2(b0 | (b1 << 16), b2 | (b3 << 16)), acc[m]);
    }
  };

  uint4 ka[KC], kb[KC];
  int tile = w;
  if (tile < ntiles) issue(ka, 0, t_begin + tile * kTile);
  while (tile < ntiles) {
    wait_vmem_all();
    if (tile + kWaves < ntiles) issue(kb, 1, t_begin + (tile + kWaves) * kTile);
    consume(ka, 0, t_begin + tile * kTile);
    tile += kWaves;
    if (tile >= ntiles) break;
    wait_vmem_all();
    if (tile + kWaves < ntiles) issue(ka, 0, t_begin + (tile + kWaves) * kTile);
    consume(kb, 1, t_begin + tile * kTile);
    tile += kWaves;
  }

  // ---- merge: lane groups' denominators, then the waves through LDS
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  if (lane == 0) s_bad[w] = bad ? 1 : 0;
  __syncthreads();  // every wave is done with its V tiles
  float* s_acc = reinterpret_cast<float*>(s_mem);           // [kWaves][G][D]
  float* s_m = s_acc + kWaves * G * D;                       // [kWaves][G]
  float* s_l = s_m + kWaves * G;                             // [kWaves][G]
  if (lane < G) {
    s_m[w * G + lane] = m_run;
    s_l[w * G + lane] = l_run;
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int h = 4 * grp + r;
    if (h < G) {
#pragma unroll
      for (int m = 0; m < NM; ++m) s_acc[(w * G + h) * D + 16 * m + col] = acc[m][r];
    }
  }
  __syncthreads();

  const bool any_bad = s_bad[0] | s_bad[1] | s_bad[2] | s_bad[3];
  for (int i = tid; i < G * D; i += kThreads) {
    const int h = i / D, d = i % D;
    float M = kNegInf;
#pragma unroll
    for (int k = 0; k < kWaves; ++k) M = fmaxf(M, s_m[k * G + h]);
    const float base = (M == kNegInf) ? 0.0f : M;
    float num = 0.0f, den = 0.0f;
#pragma unroll
    for (int k = 0; k < kWaves; ++k) {
      const float f = exp2_fast(s_m[k * G + h] - base);
      num = fmaf(f, s_acc[(k * G + h) * D + d], num);
      den = fmaf(f, s_l[k * G + h], den);
    }
    if (any_bad) {
      num = __builtin_nanf("");
      den = __builtin_nanf("");
    }
    if (nparts == 1) {
      out[(row0 + h) * D + d] = to_bits<T>(num / den);
    } else {
      ws_acc[((row0 + h) * pmax + p) * D + d] = num;
      if (d == 0) ws_ml[(row0 + h) * pmax + p] = make_float2(any_bad ? 0.0f : M, den);
    }
  }
}

// ---------------------------------------------------------------------------
template <typename T, int D, int BS, int G>
static hipError_t launch_t(const DecodeArgs& a) {
  const int64_t units = (int64_t)a.num_seqs * a.num_kv_heads * a.pmax;
  hipLaunchKernelGGL((pa_decode_mfma<T, D, BS, G>), dim3((uint32_t)units), dim3(kThreads), 0,
                     a.stream, (uint16_t*)a.out, a.ws_acc, a.ws_ml, (const uint16_t*)a.q,
                     (const uint16_t*)a.k_cache, (const uint16_t*)a.v_cache, a.block_tables,
                     a.seq_lens, a.num_kv_heads, a.max_blocks_per_seq, a.num_blocks, a.part,
                     a.pmax, a.qk_scale);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.pmax <= 1) return e;
  return launch_splitk_reduce(a);
}

template <typename T, int D, int BS>
static hipError_t launch_g(const DecodeArgs& a) {
  switch (a.group) {
    case 1: return launch_t<T, D, BS, 1>(a);
    case 2: return launch_t<T, D, BS, 2>(a);
    case 4: return launch_t<T, D, BS, 4>(a);
    case 8: return launch_t<T, D, BS, 8>(a);
  }
  return hipErrorInvalidValue;
}

template <typename T, int D>
static hipError_t launch_bs(const DecodeArgs& a) {
  switch (a.block_size) {
    case 8: return launch_g<T, D, 8>(a);
    case 16: return launch_g<T, D, 16>(a);
    case 32: return launch_g<T, D, 32>(a);
  }
  return hipErrorInvalidValue;
}

template <typename T>
static hipError_t launch_d(const DecodeArgs& a) {
  switch (a.head_dim) {
    case 64: return launch_bs<T, 64>(a);
    case 128: return launch_bs<T, 128>(a);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode_mfma(const DecodeArgs& a) {
  return a.bf16 ? launch_d<BF16>(a) : launch_d<F16>(a);
}

}  // namespace pa
