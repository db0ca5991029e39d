// decode.hip -- paged decode attention kernels (gfx950, wave64).
//
// What is computed: for every sequence s and query head h, softmax attention
// of q[s][h] against the keys/values of positions 0..L_s-1, read through the
// sequence's block table ("What problem does PagedAttention solve ...",
// section "How PagedAttention works": the kernel follows the block table;
// "Continuous Batching & Paged Attention", section "Attention needs memory
// that grows with the conversation").
//
// Work decomposition.  One workgroup (4 waves) per work unit
// (sequence s, KV head kh, partition p), numbered partition-major so that
// the XCDs share the work evenly (unit_of in pa_device.h); a partition is
// `part` consecutive positions.  The G = Hq/Hkv query heads that share kh share every K/V load.
// The unit stages its block ids in LDS, then its waves take 16-token (d 128)
// or 32-token (d 64) tiles in turn:
//   - lane layout: a token row is D/8 lanes, each holding 8 elements
//     (16 bytes) of it; a wave covers 64/(D/8) rows per 128-bit load, 4
//     loads per tile, so every load instruction reads whole 256-byte
//     (d 128) or 128-byte (d 64) rows and a 4 KiB K tile takes 4 loads;
//   - q.K with v_dot2_f32_{f16,bf16} on the packed pairs, then a DPP
//     butterfly over the row's lanes (every lane ends with the score);
//   - online softmax per row in base 2 (scores carry scale*log2 e);
//   - P.V as float32 FMAs into a per-lane accumulator of G x 8 floats;
//   - positions >= L are never loaded: their score is -inf and their V row
//     is zero, so NaN in unused slots cannot leak in.
// At the end, rows and then waves are merged by log-sum-exp.  A sequence
// with one partition writes its output; otherwise the unit writes
// (m, l, acc) to the workspace and pa_splitk_reduce merges the partitions:
//   M = max_p m_p,  out = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p.
#include "pa_device.h"
#include "pa_launch.h"

namespace pa {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kMaxPartBlocks = 512;

template <typename T, int D, int G>
__device__ __forceinline__ void write_rows(uint16_t* out, int64_t row0, float v) {
  for (int i = threadIdx.x; i < G * D; i += kThreads) out[row0 * D + i] = to_bits<T>(v);
}

template <typename T, int D, int BS, int G>
__global__ void __launch_bounds__(kThreads)
pa_decode_valu(uint16_t* __restrict__ out, float* __restrict__ ws_acc, float2* __restrict__ ws_ml,
               const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
               const uint16_t* __restrict__ vc, const int32_t* __restrict__ block_tables,
               const int32_t* __restrict__ seq_lens, int32_t hkv, int32_t mb, int32_t nb,
               int32_t part, int32_t pmax, float qk_scale) {
  constexpr int LPT = D / 8;        // lanes per token row
  constexpr int RPW = 64 / LPT;     // token rows per load instruction
  constexpr int NI = 4;             // load instructions per tile
  constexpr int TT = NI * RPW;      // tokens per tile

  __shared__ int32_t s_bt[kMaxPartBlocks];
  __shared__ float s_acc[kWaves][G][D];
  __shared__ float s_m[kWaves][G];
  __shared__ float s_l[kWaves][G];
  __shared__ int s_bad;
  static_assert(sizeof(s_bt) + sizeof(s_acc) + sizeof(s_m) + sizeof(s_l) + sizeof(s_bad) <=
                    kMaxLdsBytes,
                "one workgroup's LDS fits gfx950's 160 KiB");

  const Unit u = unit_of(blockIdx.x, hkv, pmax);
  const int s = u.s, kh = u.kh, p = u.p;
  const int hq = hkv * G;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int64_t row0 = (int64_t)s * hq + (int64_t)kh * G;  // first output row

  const int L = seq_lens[s];
  if (L < 0 || (int64_t)L > (int64_t)mb * BS) {  // breaks the contract: NaN rows
    if (p == 0) write_rows<T, D, G>(out, row0, __builtin_nanf(""));
    return;
  }
  const int t_begin = p * part;
  if (t_begin >= L) {
    if (p == 0) write_rows<T, D, G>(out, row0, 0.0f);  // L == 0
    return;
  }
  const int t_end = min(L, t_begin + part);
  const int nparts = (L + part - 1) / part;
  const int blk0 = t_begin / BS;
  const int nblk = (t_end - t_begin + BS - 1) / BS;

  if (tid == 0) s_bad = 0;
  __syncthreads();
  for (int j = tid; j < nblk; j += kThreads) {
    int b = block_tables[(int64_t)s * mb + blk0 + j];
    if (b < 0 || b >= nb) {
      s_bad = 1;
      b = 0;
    }
    s_bt[j] = b;
  }
  __syncthreads();
  if (s_bad) {  // an id outside the pool: never dereferenced, rows become NaN
    if (nparts == 1) {
      write_rows<T, D, G>(out, row0, __builtin_nanf(""));
    } else {
      for (int i = tid; i < G * D; i += kThreads) {
        const int h = i / D, d = i % D;
        ws_acc[((row0 + h) * pmax + p) * D + d] = __builtin_nanf("");
        if (d == 0) ws_ml[(row0 + h) * pmax + p] = make_float2(0.0f, __builtin_nanf(""));
      }
    }
    return;
  }

  const int col = lane % LPT;
  const int row = lane / LPT;

  uint4 qv[G];
  {
    const uint16_t* qb = q + row0 * D + col * 8;
#pragma unroll
    for (int h = 0; h < G; ++h) qv[h] = *reinterpret_cast<const uint4*>(qb + h * D);
  }

  float m[G], l[G], acc[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = kNegInf;
    l[h] = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.0f;
  }

  const int64_t blk_stride = (int64_t)hkv * BS * D;
  const int64_t lane_off = (int64_t)kh * BS * D + col * 8;
  const int ntiles = (t_end - t_begin + TT - 1) / TT;

  for (int tile = w; tile < ntiles; tile += kWaves) {
    const int t0 = t_begin + tile * TT;
    uint4 kr[NI], vr[NI];
    bool valid[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int t = t0 + i * RPW + row;
      valid[i] = t < t_end;
      kr[i] = make_uint4(0u, 0u, 0u, 0u);
      vr[i] = make_uint4(0u, 0u, 0u, 0u);
      if (valid[i]) {
        const int64_t off = (int64_t)s_bt[t / BS - blk0] * blk_stride + lane_off + (t % BS) * D;
        kr[i] = load_stream(kc + off);
        vr[i] = load_stream(vc + off);
      }
    }

    float sc[NI][G];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float a = dot2<T>(qv[h].x, kr[i].x, 0.0f);
        a = dot2<T>(qv[h].y, kr[i].y, a);
        a = dot2<T>(qv[h].z, kr[i].z, a);
        a = dot2<T>(qv[h].w, kr[i].w, a);
        sc[i][h] = group_sum<LPT>(a);
      }
    }

    float vf[NI][8];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      vf[i][0] = lo_f32<T>(vr[i].x);
      vf[i][1] = hi_f32<T>(vr[i].x);
      vf[i][2] = lo_f32<T>(vr[i].y);
      vf[i][3] = hi_f32<T>(vr[i].y);
      vf[i][4] = lo_f32<T>(vr[i].z);
      vf[i][5] = hi_f32<T>(vr[i].z);
      vf[i][6] = lo_f32<T>(vr[i].w);
      vf[i][7] = hi_f32<T>(vr[i].w);
    }

#pragma unroll
    for (int h = 0; h < G; ++h) {
      float mx = kNegInf;
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        sc[i][h] = valid[i] ? sc[i][h] * qk_scale : kNegInf;
        mx = fmaxf(mx, sc[i][h]);
      }
      const float mnew = fmaxf(m[h], mx);
      const float base = (mnew == kNegInf) ? 0.0f : mnew;
      const float corr = exp2_fast(m[h] - base);
      l[h] *= corr;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] *= corr;
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const float pr = exp2_fast(sc[i][h] - base);
        l[h] += pr;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(pr, vf[i][e], acc[h][e]);
      }
      m[h] = mnew;
    }
  }

  // merge the rows of the wave (lane groups LPT apart)
#pragma unroll
  for (int mask = LPT; mask < 64; mask <<= 1) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float mo = __shfl_xor(m[h], mask);
      const float lo = __shfl_xor(l[h], mask);
      const float mn = fmaxf(m[h], mo);
      const float base = (mn == kNegInf) ? 0.0f : mn;
      const float f = exp2_fast(m[h] - base);
      const float fo = exp2_fast(mo - base);
      l[h] = l[h] * f + lo * fo;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float ao = __shfl_xor(acc[h][e], mask);
        acc[h][e] = acc[h][e] * f + ao * fo;
      }
      m[h] = mn;
    }
  }
  if (row == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int e = 0; e < 8; ++e) s_acc[w][h][col * 8 + e] = acc[h][e];
      if (col == 0) {
        s_m[w][h] = m[h];
        s_l[w][h] = l[h];
      }
    }
  }
  __syncthreads();

  // merge the waves and write
  for (int i = tid; i < G * D; i += kThreads) {
    const int h = i / D, d = i % D;
    float M = kNegInf;
#pragma unroll
    for (int k = 0; k < kWaves; ++k) M = fmaxf(M, s_m[k][h]);
    const float base = (M == kNegInf) ? 0.0f : M;
    float num = 0.0f, den = 0.0f;
#pragma unroll
    for (int k = 0; k < kWaves; ++k) {
      const float f = exp2_fast(s_m[k][h] - base);
      num = fmaf(f, s_acc[k][h][d], num);
      den = fmaf(f, s_l[k][h], den);
    }
    if (nparts == 1) {
      out[(row0 + h) * D + d] = to_bits<T>(num / den);
    } else {
      ws_acc[((row0 + h) * pmax + p) * D + d] = num;
      if (d == 0) ws_ml[(row0 + h) * pmax + p] = make_float2(M, den);
    }
  }
}

// Merge of the partitions of every (sequence, query head) with more than one:
// one thread per output element; the partition states are read in batches of
// 8 independent loads so the loop is not a chain of dependent load latencies.
template <typename T, int D>
__global__ void __launch_bounds__(256)
pa_splitk_reduce(uint16_t* __restrict__ out, const float* __restrict__ ws_acc,
                 const float2* __restrict__ ws_ml, const int32_t* __restrict__ seq_lens,
                 int32_t hq, int32_t max_len, int32_t part, int32_t pmax) {
  constexpr int HPB = 256 / D;  // query heads per workgroup
  constexpr int U = 8;
  const int s = blockIdx.y;
  const int h = blockIdx.x * HPB + threadIdx.x / D;
  const int d = threadIdx.x % D;
  if (h >= hq) return;
  const int L = seq_lens[s];
  if (L < 0 || L > max_len) return;  // the decode kernel wrote NaN rows
  const int nparts = (L + part - 1) / part;
  if (nparts <= 1) return;
  const int64_t r = (int64_t)s * hq + h;
  const float2* ml = ws_ml + r * pmax;
  const float* ac = ws_acc + r * pmax * D + d;
  float M = kNegInf;
  for (int k0 = 0; k0 < nparts; k0 += U) {
    float mk[U];
#pragma unroll
    for (int u = 0; u < U; ++u) mk[u] = (k0 + u < nparts) ? ml[k0 + u].x : kNegInf;
#pragma unroll
    for (int u = 0; u < U; ++u) M = fmaxf(M, mk[u]);
  }
  float num = 0.0f, den = 0.0f;
  for (int k0 = 0; k0 < nparts; k0 += U) {
    float2 v[U];
    float a[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool ok = k0 + u < nparts;
      v[u] = ok ? ml[k0 + u] : make_float2(kNegInf, 0.0f);
      a[u] = ok ? ac[(int64_t)(k0 + u) * D] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float f = exp2_fast(v[u].x - M);
      num = fmaf(f, a[u], num);
      den = fmaf(f, v[u].y, den);
    }
  }
  out[r * D + d] = to_bits<T>(num / den);
}

template <typename T, int D>
static hipError_t launch_reduce_t(const DecodeArgs& a) {
  constexpr int HPB = 256 / D;
  const int hq = a.num_kv_heads * a.group;
  hipLaunchKernelGGL((pa_splitk_reduce<T, D>),
                     dim3((uint32_t)((hq + HPB - 1) / HPB), (uint32_t)a.num_seqs), dim3(256), 0,
                     a.stream, (uint16_t*)a.out, a.ws_acc, a.ws_ml, a.seq_lens, hq,
                     a.max_blocks_per_seq * a.block_size, a.part, a.pmax);
  return hipGetLastError();
}

hipError_t launch_splitk_reduce(const DecodeArgs& a) {
  if (a.bf16) return a.head_dim == 64 ? launch_reduce_t<BF16, 64>(a) : launch_reduce_t<BF16, 128>(a);
  return a.head_dim == 64 ? launch_reduce_t<F16, 64>(a) : launch_reduce_t<F16, 128>(a);
}

// ---------------------------------------------------------------------------
template <typename T, int D, int BS, int G>
static hipError_t launch_decode_t(const DecodeArgs& a) {
  static int lds_cache[kMaxDevices];
  const hipError_t fit = check_lds((const void*)pa_decode_valu<T, D, BS, G>, 0, lds_cache);
  if (fit != hipSuccess) return fit;
  const int64_t units = (int64_t)a.num_seqs * a.num_kv_heads * a.pmax;
  hipLaunchKernelGGL((pa_decode_valu<T, D, BS, G>), dim3((uint32_t)units), dim3(kThreads), 0,
                     a.stream, (uint16_t*)a.out, a.ws_acc, a.ws_ml, (const uint16_t*)a.q,
                     (const uint16_t*)a.k_cache, (const uint16_t*)a.v_cache, a.block_tables,
                     a.seq_lens, a.num_kv_heads, a.max_blocks_per_seq, a.num_blocks, a.part,
                     a.pmax, a.qk_scale);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.pmax <= 1) return e;
  return launch_splitk_reduce(a);
}

template <typename T, int D, int BS>
static hipError_t launch_decode_g(const DecodeArgs& a) {
  switch (a.group) {
    case 1: return launch_decode_t<T, D, BS, 1>(a);
    case 2: return launch_decode_t<T, D, BS, 2>(a);
    case 4: return launch_decode_t<T, D, BS, 4>(a);
    case 8: return launch_decode_t<T, D, BS, 8>(a);
  }
  return hipErrorInvalidValue;
}

template <typename T, int D>
static hipError_t launch_decode_bs(const DecodeArgs& a) {
  switch (a.block_size) {
    case 8: return launch_decode_g<T, D, 8>(a);
    case 16: return launch_decode_g<T, D, 16>(a);
    case 32: return launch_decode_g<T, D, 32>(a);
  }
  return hipErrorInvalidValue;
}

template <typename T>
static hipError_t launch_decode_d(const DecodeArgs& a) {
  switch (a.head_dim) {
    case 64: return launch_decode_bs<T, 64>(a);
    case 128: return launch_decode_bs<T, 128>(a);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode(const DecodeArgs& a) {
  return a.bf16 ? launch_decode_d<BF16>(a) : launch_decode_d<F16>(a);
}

int decode_max_partition_blocks() { return kMaxPartBlocks; }

}  // namespace pa
