// decode_mfma.hip -- paged decode attention with q.K^T and P.V on the matrix
// cores (gfx950 MFMA), for head_dim 64/128, block 8/16/32, group 1..8: the
// partitioned kernel (explicit partition_size).
//
// Same result and work decomposition as the VALU kernel (decode.hip): one
// workgroup of 4 waves per (sequence, KV head, partition), numbered
// partition-major so that the XCDs share the work evenly, waves taking
// 16-position tiles in turn (TileWave in pa_mfma.h: K to registers, V to
// LDS, q.K^T and P.V on MFMA, base-2 online softmax), a log-sum-exp merge of
// the waves through LDS and, for split sequences, of the partitions
// (pa_splitk_reduce).  Block ids are wave-uniform scalar loads; each tile is
// issued one tile ahead of being consumed.
#include "pa_launch.h"
#include "pa_mfma.h"

namespace pa {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

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

  TileWave<T, D, BS, G> tw;
  tw.init(kc, vc, hkv, kh, s_mem + w * 2 * GE::TILE);
  tw.load_q(q + row0 * D);
  tw.reset();
  bool bad = false;

  // Block ids of the tile at t0: wave-uniform scalar loads; an id outside
  // the pool is never dereferenced (block 0 is read instead, rows become NaN).
  auto issue = [&](uint4 (&kr)[KC], int buf, int t0) {
    int id0 = bt_row[t0 / BS];
    int id1 = id0;
    if constexpr (BS < kTile) id1 = (t0 + BS < t_end) ? bt_row[t0 / BS + 1] : id0;
    if (id0 < 0 || id0 >= nb) { bad = true; id0 = 0; }
    if (id1 < 0 || id1 >= nb) { bad = true; id1 = 0; }
    tw.issue(kr, buf, t0, t_end - 1, id0, id1);
  };

  uint4 ka[KC], kb[KC];
  int tile = w;
  if (tile < ntiles) issue(ka, 0, t_begin + tile * kTile);
  while (tile < ntiles) {
    wait_vmem_all();
    if (tile + kWaves < ntiles) issue(kb, 1, t_begin + (tile + kWaves) * kTile);
    tw.consume(ka, 0, t_begin + tile * kTile, t_end, qk_scale);
    tile += kWaves;
    if (tile >= ntiles) break;
    wait_vmem_all();
    if (tile + kWaves < ntiles) issue(ka, 0, t_begin + (tile + kWaves) * kTile);
    tw.consume(kb, 1, t_begin + tile * kTile, t_end, qk_scale);
    tile += kWaves;
  }

  // ---- merge: lane groups' denominators, then the waves through LDS
  tw.finish();
  if (lane == 0) s_bad[w] = bad ? 1 : 0;
  __syncthreads();  // every wave is done with its V tiles
  float* s_acc = reinterpret_cast<float*>(s_mem);           // [kWaves][G][D]
  float* s_m = s_acc + kWaves * G * D;                       // [kWaves][G]
  float* s_l = s_m + kWaves * G;                             // [kWaves][G]
  if (lane < G) {
    s_m[w * G + lane] = tw.m_run;
    s_l[w * G + lane] = tw.l_run;
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int h = 4 * grp + r;
    if (h < G) {
#pragma unroll
      for (int m = 0; m < NM; ++m) s_acc[(w * G + h) * D + 16 * m + col] = tw.acc[m][r];
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
