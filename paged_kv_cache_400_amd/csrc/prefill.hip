// prefill.hip -- paged attention of several query tokens per sequence with a
// causal mask (chunked prefill), over the same pools and block tables as
// decode.
//
// "What problem does PagedAttention solve, and what is continuous
// batching?" (datarekha): prefill is the compute-heavy first pass over a
// prompt ("Why the KV cache becomes the problem"), and servers split a long
// prompt into chunks processed over several steps ("How the two fit
// together in production").  A step gives sequence s a chunk of n_s =
// query_start[s+1] - query_start[s] tokens whose keys and values are
// already in the pool; chunk token i sits at position L_s - n_s + i and
// attends to positions 0 .. L_s - n_s + i (n_s = 1 is decode).
//
// Row block: 16 query rows = 16 / G consecutive chunk tokens x the G query
// heads of one KV head, so the q.K^T MFMA (16 positions x 16 rows) has no
// idle rows.  Work unit: one wave per (sequence, KV head, kNrb = 3
// consecutive row blocks).  The wave walks the sequence's tiles of 16
// positions from 0 up to its last row's position with TileWave (pa_mfma.h):
// K to registers and V to LDS once per tile, each tile issued one tile
// ahead, consumed by the three row blocks' tile waves; each lane's row has
// its own causal end, which masks its scores.  No split and no merge: a
// chunk has many units per (sequence, head).
//
// Placement: workgroup g runs on XCD g % 8; pair (s, kh) belongs to XCD
// (s * hkv + kh) % 8, whose waves take its units consecutively (the last,
// longest ones first), so the units of a pair share one L2 for the pair's
// keys and values.
//
// Roofline: the useful work is 4 d FLOPs per (query row, visible
// position); the kernel is bound by on-chip work (matrix cores, the softmax,
// the per-tile loads from L2), not by HBM.  Measured on the 32 x 512-token
// chunked-prefill step: one row block per unit, units in plain order
// 5.39 ms; units grouped per XCD 3.99 ms; two row blocks per unit (2 waves
// per SIMD) 1.86 ms; three 1.55 ms (four, at one wave per SIMD, 3.27 ms).
#include "pa_launch.h"
#include "pa_mfma.h"

namespace pa {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRows = 16;  // query rows per row block
constexpr int kNrb = 3;    // row blocks per unit

__device__ __forceinline__ int wave_inclusive_scan(int x, int lane) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    const int y = __shfl_up(x, m);
    if (lane >= m) x += y;
  }
  return x;
}

}  // namespace

template <typename T, int D, int BS, int G>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
pa_prefill_kernel(uint16_t* __restrict__ out, const uint16_t* __restrict__ q,
                  const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc,
                  const int32_t* __restrict__ block_tables, const int32_t* __restrict__ seq_lens,
                  const int32_t* __restrict__ query_start, int32_t num_seqs, int32_t total_q,
                  int32_t hkv, int32_t mb, int32_t nb, float qk_scale) {
  using GE = Geo<D>;
  constexpr int KC = GE::KC, NM = GE::NM;
  constexpr int R1 = kRows / G;   // chunk tokens per row block
  constexpr int R = kNrb * R1;     // chunk tokens per unit
  static_assert(kRows % G == 0, "whole tokens per unit");
  __shared__ __attribute__((aligned(16))) unsigned char s_mem[kWaves * 2 * GE::TILE];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hq = hkv * G;
  const int64_t max_len = (int64_t)mb * BS;

  // chunk of sequence j: [qs, qe) if the offsets are consistent, else empty
  auto chunk_of = [&](int j, int& qs, int& n) {
    qs = query_start[j];
    const int qe = query_start[j + 1];
    n = (qs >= 0 && qe >= qs && qe <= total_q) ? qe - qs : 0;
  };

  // ---- this wave's (sequence, KV head, unit).  Workgroup g runs on XCD
  // g % 8; pair p = s * hkv + kh belongs to XCD p % 8, and an XCD's waves
  // take its pairs in order, a pair's units consecutively, so the units of
  // one pair share that XCD's L2 for the pair's keys and values.
  const int xcd = blockIdx.x % 8;
  const int un = (blockIdx.x / 8) * kWaves + w;  // unit index within the XCD
  const int npairs = num_seqs * hkv;
  int s = -1, kh = 0, rb_local = 0;
  {
    int run = 0;
    for (int j0 = 0; xcd + 8 * j0 < npairs; j0 += 64) {
      const int p = xcd + 8 * (j0 + lane);
      int cnt = 0;
      if (p < npairs) {
        int qs_, n_;
        chunk_of(p / hkv, qs_, n_);
        cnt = (n_ + R - 1) / R;
      }
      const int incl = wave_inclusive_scan(cnt, lane);
      const uint64_t hit = __builtin_amdgcn_ballot_w64(run + incl > un);
      if (hit != 0) {
        const int i = __builtin_ctzll(hit);
        const int pp = xcd + 8 * (j0 + i);
        s = pp / hkv;
        kh = pp % hkv;
        rb_local = un - (run + __builtin_amdgcn_readlane(incl, i) -
                         __builtin_amdgcn_readlane(cnt, i));
        break;
      }
      run += __builtin_amdgcn_readlane(incl, 63);
    }
  }
  if (s < 0) return;  // past the last unit
  int qs, n;
  chunk_of(s, qs, n);
  const int L = seq_lens[s];
  const int nrb = (n + R - 1) / R;    // units of this pair
  const int rb = nrb - 1 - rb_local;  // last units first: they see the most positions
  const int i0 = rb * R;              // first chunk token of this unit
  const int col = lane & 15, grp = lane >> 4;
  const bool valid = n <= L && (int64_t)L <= max_len;
  // the lane's query row in row block h (h < kNrb): chunk token i0 + h R1 +
  // col / G, head kh * G + col % G; its causal end (exclusive)
  int tok[kNrb], lane_end[kNrb];
  bool active[kNrb];
#pragma unroll
  for (int h = 0; h < kNrb; ++h) {
    tok[h] = i0 + h * R1 + col / G;
    active[h] = tok[h] < n;
    lane_end[h] = active[h] ? L - n + tok[h] + 1 : 1;
  }
  const int p_end = L - n + min(i0 + R, n);
  auto store_rows = [&](const float* st, int tfirst) {
    // st: [16 rows][D] floats staged in LDS; row r -> (token tfirst + r / G, head r % G)
    for (int i = lane * 8; i < kRows * D; i += 64 * 8) {
      const int r = i / D, d = i % D;
      const int t_r = tfirst + r / G;
      if (t_r < n) {
        const float4 a = *reinterpret_cast<const float4*>(st + i);
        const float4 b = *reinterpret_cast<const float4*>(st + i + 4);
        *reinterpret_cast<uint4*>(out + (((int64_t)qs + t_r) * hq + kh * G + r % G) * D + d) =
            make_uint4(pack2<T>(a.x, a.y), pack2<T>(a.z, a.w), pack2<T>(b.x, b.y),
                       pack2<T>(b.z, b.w));
      }
    }
  };

  unsigned char* vtile = s_mem + w * 2 * GE::TILE;
  float* st = reinterpret_cast<float*>(vtile);  // [16][D] staging once the tiles are consumed
  static_assert(sizeof(float) * kRows * D <= 2 * GE::TILE, "the result fits the wave's V tiles");

  if (!valid) {  // lengths break the contract: NaN rows, nothing read
    for (int i = lane; i < kRows * D; i += 64) st[i] = __builtin_nanf("");
#pragma unroll
    for (int h = 0; h < kNrb; ++h) store_rows(st, i0 + h * R1);
    return;
  }

  TileWave<T, D, BS, kRows> tws[kNrb];
#pragma unroll
  for (int h = 0; h < kNrb; ++h) {
    tws[h].init(kc, vc, hkv, kh, vtile);
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      tws[h].qb[c] = make_uint4(0u, 0u, 0u, 0u);
      if (active[h])
        tws[h].qb[c] = *reinterpret_cast<const uint4*>(
            q + (((int64_t)qs + tok[h]) * hq + kh * G + col % G) * D + (c * 4 + grp) * 8);
    }
    tws[h].reset();
  }
  auto& tw = tws[0];  // issues the loads every row block consumes

  // block ids of the positions [0, p_end), 64 at a time: lane j holds block base + j
  const int32_t* bt_row = block_tables + (int64_t)s * mb;
  const int blk_last = (p_end - 1) / BS;
  int blk_base = 0;
  bool bad = false;
  auto load_ids = [&]() {
    int id = 0;
    if (blk_base + lane <= blk_last) {
      id = bt_row[blk_base + lane];
      if (id < 0 || id >= nb) {
        bad = true;  // never dereferenced: block 0 is read, the rows become NaN
        id = 0;
      }
    }
    bad = __builtin_amdgcn_ballot_w64(bad) != 0;
    return id;
  };
  int vid = load_ids();
  const int ntiles = (p_end + kTile - 1) / kTile;

  auto issue = [&](uint4 (&kr)[KC], int buf, int j) {
    const int t0 = j * kTile;
    int b = t0 / BS - blk_base;
    if (b + TileWave<T, D, BS, kRows>::kIds - 1 >= 64) {
      blk_base += b;
      b = 0;
      vid = load_ids();
    }
    const int id0 = __builtin_amdgcn_readlane(vid, b);
    int id1 = id0;
    if constexpr (BS < kTile) id1 = (t0 + BS < p_end) ? __builtin_amdgcn_readlane(vid, b + 1) : id0;
    tw.issue(kr, buf, t0, p_end - 1, id0, id1);
  };

  uint4 ka[KC], kb[KC];
  issue(ka, 0, 0);
  for (int j = 0;;) {
    wait_vmem_all();
    if (j + 1 < ntiles) issue(kb, 1, j + 1);
#pragma unroll
    for (int h = 0; h < kNrb; ++h) tws[h].consume(ka, 0, j * kTile, lane_end[h], qk_scale);
    if (++j >= ntiles) break;
    wait_vmem_all();
    if (j + 1 < ntiles) issue(ka, 0, j + 1);
#pragma unroll
    for (int h = 0; h < kNrb; ++h) tws[h].consume(kb, 1, j * kTile, lane_end[h], qk_scale);
    if (++j >= ntiles) break;
  }
#pragma unroll
  for (int h = 0; h < kNrb; ++h) tws[h].finish();

  // out = acc / l, staged row-major in the wave's V tiles, stored whole lines
  auto put = [&](const TileWave<T, D, BS, kRows>& t) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int h = 4 * grp + r;
      const float l_h = __shfl(t.l_run, h);
#pragma unroll
      for (int m = 0; m < NM; ++m)
        st[h * D + 16 * m + col] = bad ? __builtin_nanf("") : t.acc[m][r] / l_h;
    }
  };
#pragma unroll
  for (int h = 0; h < kNrb; ++h) {
    put(tws[h]);
    store_rows(st, i0 + h * R1);
  }
}

// Units one XCD can get at most: each sequence has at most ceil(hkv / 8)
// of its (sequence, KV head) pairs on one XCD.
static int64_t units_per_xcd(int32_t total_q, int32_t num_seqs, int32_t hkv, int32_t group) {
  return ((int64_t)hkv + 7) / 8 *
         (((int64_t)total_q * group + kNrb * kRows - 1) / (kNrb * kRows) + num_seqs);
}

template <typename T, int D, int BS, int G>
static hipError_t launch_t(const PrefillArgs& a) {
  const int64_t per_xcd = units_per_xcd(a.total_q, a.num_seqs, a.num_kv_heads, G);
  const int64_t grid = 8 * ((per_xcd + kWaves - 1) / kWaves);
  hipLaunchKernelGGL((pa_prefill_kernel<T, D, BS, G>), dim3((uint32_t)grid), dim3(kThreads), 0,
                     a.stream, (uint16_t*)a.out, (const uint16_t*)a.q,
                     (const uint16_t*)a.k_cache, (const uint16_t*)a.v_cache, a.block_tables,
                     a.seq_lens, a.query_start, a.num_seqs, a.total_q, a.num_kv_heads,
                     a.max_blocks_per_seq, a.num_blocks, a.qk_scale);
  return hipGetLastError();
}

template <typename T, int D, int BS>
static hipError_t launch_g(const PrefillArgs& a) {
  switch (a.group) {
    case 1: return launch_t<T, D, BS, 1>(a);
    case 2: return launch_t<T, D, BS, 2>(a);
    case 4: return launch_t<T, D, BS, 4>(a);
    case 8: return launch_t<T, D, BS, 8>(a);
  }
  return hipErrorInvalidValue;
}

template <typename T, int D>
static hipError_t launch_bs(const PrefillArgs& a) {
  switch (a.block_size) {
    case 8: return launch_g<T, D, 8>(a);
    case 16: return launch_g<T, D, 16>(a);
    case 32: return launch_g<T, D, 32>(a);
  }
  return hipErrorInvalidValue;
}

template <typename T>
static hipError_t launch_d(const PrefillArgs& a) {
  switch (a.head_dim) {
    case 64: return launch_bs<T, 64>(a);
    case 128: return launch_bs<T, 128>(a);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_prefill(const PrefillArgs& a) {
  return a.bf16 ? launch_d<BF16>(a) : launch_d<F16>(a);
}

int64_t prefill_units(int32_t total_q, int32_t num_seqs, int32_t num_kv_heads, int32_t group) {
  return 8 * kWaves * ((units_per_xcd(total_q, num_seqs, num_kv_heads, group) + kWaves - 1) / kWaves);
}

}  // namespace pa
