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
// idle rows.  Work unit: one workgroup of 4 waves per (sequence, KV head,
// 4 x kNrb consecutive row blocks); each wave owns kNrb = 3 row blocks.
// The workgroup walks the sequence's positions from 0 up to its last row's
// position in tiles of 32, double-buffered in LDS: after a wait and a
// barrier, the four waves copy the next tile's keys and values from HBM
// straight into LDS (global_load_lds) while they compute the current one,
// so each key and value is fetched once per unit, not once per wave.
//
// Per wave and 32-position slab: q.K^T as two 16-position halves (K read
// from LDS in the MFMA operand layout); the softmax on the 8 scores a lane
// holds per row, masked only where the slab reaches past the wave's first
// token; P.V as v_mfma_f32_16x16x32 (the lane's 8 weights, positions
// 4 grp + r then 16 + 4 grp + r, are its k-values, and the V operand is the
// two halves' transpose reads side by side), which runs at twice the rate
// of the 16x16x16 form on gfx950; the denominator as one more MFMA of the
// weights against a column of ones, so it accumulates in the rows' own
// layout (no lane exchange at the end).  No split and no merge.
//
// Placement: workgroup g runs on XCD g % 8; pair (s, kh) belongs to XCD
// (s * hkv + kh) % 8, whose workgroups take its units consecutively (the
// last, longest ones first), so the units of a pair share one L2.  With at
// most 64 pairs per XCD the pairs are taken in order of their sequence's
// context before the chunk, longest first: a unit's time is mostly its
// context, so the XCD's last units are its shortest (5% on the
// chunked-prefill step, as a greedy-dispatch model of the units predicts).
//
// Copies: each lane's byte offset within a pool block is fixed per copy, so
// a tile that lies wholly below the unit's last position costs a readlane of
// its block id, a scalar multiply and one add per copy; only the unit's last
// tile clamps rows one by one.  V sub-tiles are stored with a chunk swizzle
// (VGeo below) that halves the bank conflicts of the transpose reads.
//
// Roofline: the useful work is 4 d FLOPs per (query row, visible
// position); the kernel is bound by on-chip work (matrix cores, the softmax
// and the LDS traffic), not by HBM.  Measured on the 32 x 512-token
// chunked-prefill step: one wave per unit, each loading its own tiles,
// 1.52 ms; tiles shared by the workgroup through LDS 1.25 ms; 32-position
// tiles and the 16x16x32 P.V form 1.02 ms; the mask only on the diagonal,
// the scale folded into one FMA per weight and the denominator on the
// matrix cores 0.93 ms; scalar block addressing for whole tiles and the
// swizzled V layout 0.85 ms; pairs ordered by context 0.80 ms.
#include "pa_launch.h"
#include "pa_mfma.h"

namespace pa {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRows = 16;          // query rows per row block
constexpr int kNrb = 3;            // row blocks per wave
constexpr int kSub = 2;            // 16-position sub-tiles per tile
constexpr int kTP = kTile * kSub;  // positions per tile

// LDS layout of the V sub-tiles (16 rows each): four regions of 4 rows,
// regions 128 bytes apart modulo the 256-byte bank period, and within a
// region the 16-byte chunks of row r stored at chunk index c ^ (2 sw(r)).
// A transpose read (ds_read_b64_tr_b16) of column block m gives each group
// of 16 lanes 32 bytes of each of its region's 4 rows: with the swizzle the
// 4 rows fall on distinct banks, and the 4 groups pair up on the two halves
// of the bank period, so an instruction meets each bank twice (the least
// for its 512 bytes) instead of four times.
template <int D>
struct VGeo {
  static constexpr int ROW = 2 * D;             // bytes of one V row
  static constexpr int CHUNKS = D / 8;          // 16-byte chunks per row
  static constexpr int REGION = 4 * ROW + 128;  // 4 rows + padding
  static constexpr int TILE = 4 * REGION;       // one 16-row sub-tile
  static constexpr int LANES = 4 * CHUNKS;      // lanes that fill a region
  static constexpr int SWDIV = 256 / ROW;       // rows per bank period
  static_assert(TILE % 32 == 0 && (REGION % 256) == 128, "bank layout");
};
template <int D>
__device__ __forceinline__ int v_swizzle(int r) {
  return r / VGeo<D>::SWDIV;
}

// LDS of one tile (one stage of the double buffer): the K operand blocks,
// then the V sub-tiles.  K block (sub-tile st, d-chunk c) holds, at byte
// 16 l, the 16 bytes lane l feeds the q.K^T MFMA: position 16 st + l % 16,
// elements 32 c + 8 (l / 16) .. + 7, so a wave reads it back linearly.
template <int D>
struct Stage {
  using GE = Geo<D>;
  static constexpr int KBLK = 64 * 16;
  static constexpr int KSUB = GE::KC * KBLK;
  static constexpr int KBYTES = kSub * KSUB;
  static constexpr int BYTES = KBYTES + kSub * VGeo<D>::TILE;
  static constexpr int KJOBS = kSub * GE::KC;  // DMA instructions per tile: K blocks,
  static constexpr int JOBS = KJOBS + kSub * 4;  // then V regions
  static_assert(JOBS % kWaves == 0, "every wave issues the same number of copies");
  static_assert(kSub % 2 == 0, "whole 32-position slabs");
  static_assert(BYTES % 32 == 0, "stages and the per-wave staging stay 16-byte aligned");
};

// The V operands of one 32-position slab: for each column block m, the
// transpose reads of the first sub-tile (lo) and of the second (hi, one
// VGeo tile further).  a[i] is the lane's address of column block i ^ sw
// in the first sub-tile (i < 4); block m is at a[m & 3] + 128 (m >> 2).
// One asm block, completed before it ends: the compiler would otherwise
// make these reads wait for every LDS copy in flight, the next tile's
// included.  The caller's wait and barrier order them after the copies of
// this tile.
template <int NM>
__device__ __forceinline__ void read_v_slab(uint2 (&lo)[NM], uint2 (&hi)[NM],
                                            const uint32_t (&a)[4]) {
  static_assert(NM == 4 || NM == 8, "head_dim 64 or 128");
  if constexpr (NM == 8) {
    static_assert(VGeo<128>::TILE == 4608, "offsets below");
    asm volatile(
        "ds_read_b64_tr_b16 %0, %16\n\t"
        "ds_read_b64_tr_b16 %1, %16 offset:4608\n\t"
        "ds_read_b64_tr_b16 %2, %17\n\t"
        "ds_read_b64_tr_b16 %3, %17 offset:4608\n\t"
        "ds_read_b64_tr_b16 %4, %18\n\t"
        "ds_read_b64_tr_b16 %5, %18 offset:4608\n\t"
        "ds_read_b64_tr_b16 %6, %19\n\t"
        "ds_read_b64_tr_b16 %7, %19 offset:4608\n\t"
        "ds_read_b64_tr_b16 %8, %16 offset:128\n\t"
        "ds_read_b64_tr_b16 %9, %16 offset:4736\n\t"
        "ds_read_b64_tr_b16 %10, %17 offset:128\n\t"
        "ds_read_b64_tr_b16 %11, %17 offset:4736\n\t"
        "ds_read_b64_tr_b16 %12, %18 offset:128\n\t"
        "ds_read_b64_tr_b16 %13, %18 offset:4736\n\t"
        "ds_read_b64_tr_b16 %14, %19 offset:128\n\t"
        "ds_read_b64_tr_b16 %15, %19 offset:4736\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(lo[0]), "=&v"(hi[0]), "=&v"(lo[1]), "=&v"(hi[1]), "=&v"(lo[2]), "=&v"(hi[2]),
          "=&v"(lo[3]), "=&v"(hi[3]), "=&v"(lo[4]), "=&v"(hi[4]), "=&v"(lo[5]), "=&v"(hi[5]),
          "=&v"(lo[6]), "=&v"(hi[6]), "=&v"(lo[7]), "=&v"(hi[7])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3])
        : "memory");
  } else {
    static_assert(VGeo<64>::TILE == 2560, "offsets below");
    asm volatile(
        "ds_read_b64_tr_b16 %0, %8\n\t"
        "ds_read_b64_tr_b16 %1, %8 offset:2560\n\t"
        "ds_read_b64_tr_b16 %2, %9\n\t"
        "ds_read_b64_tr_b16 %3, %9 offset:2560\n\t"
        "ds_read_b64_tr_b16 %4, %10\n\t"
        "ds_read_b64_tr_b16 %5, %10 offset:2560\n\t"
        "ds_read_b64_tr_b16 %6, %11\n\t"
        "ds_read_b64_tr_b16 %7, %11 offset:2560\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(lo[0]), "=&v"(hi[0]), "=&v"(lo[1]), "=&v"(hi[1]), "=&v"(lo[2]), "=&v"(hi[2]),
          "=&v"(lo[3]), "=&v"(hi[3])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3])
        : "memory");
  }
}

// The larger of a and b, NaN if either is NaN (llvm.maximum).
__device__ __forceinline__ float fmax_nan(float a, float b) {
  return __builtin_elementwise_maximum(a, b);
}

// Two 16-bit ones packed in a word (the B operand of a row sum).
template <typename T> constexpr uint32_t kOnes2 = 0x3c003c00u;  // fp16 1.0
template <> constexpr uint32_t kOnes2<BF16> = 0x3f803f80u;      // bf16 1.0

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
  using SG = Stage<D>;
  constexpr int KC = GE::KC, NM = GE::NM;
  constexpr int R1 = kRows / G;   // chunk tokens per row block
  constexpr int R = kNrb * R1;     // chunk tokens per wave
  constexpr int RW = kWaves * R;   // chunk tokens per workgroup
  static_assert(kRows % G == 0, "whole tokens per row block");
  __shared__ __attribute__((aligned(16))) unsigned char s_st0[SG::BYTES];
  __shared__ __attribute__((aligned(16))) unsigned char s_st1[SG::BYTES];
  static_assert(sizeof(s_st0) + sizeof(s_st1) <= kMaxLdsBytes,
                "one workgroup's LDS fits gfx950's 160 KiB");
  unsigned char* const s_mem = s_st0;
  static_assert(sizeof(float) * kRows * D <= 2 * SG::BYTES / kWaves,
                "a row block's result fits the wave's quarter of the LDS");

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

  // ---- this workgroup's (sequence, KV head, unit).  Workgroup g runs on
  // XCD g % 8; pair p = s * hkv + kh belongs to XCD p % 8, and an XCD's
  // workgroups take its pairs in order, a pair's units consecutively, so the
  // units of one pair share that XCD's L2.
  const int xcd = blockIdx.x % 8;
  const int un = blockIdx.x / 8;  // unit index within the XCD
  const int npairs = num_seqs * hkv;
  int s = -1, kh = 0, u_local = 0;
  if (npairs <= 8 * 64) {
    // at most 64 pairs on this XCD, one per lane: taken in order of their
    // sequence's context before the chunk (L - n), longest first, ties by
    // index, so the longest units start first and the XCD's last ones are
    // short (a unit's time is mostly its context)
    const int p = xcd + 8 * lane;
    int cnt = 0, ctx = -1;
    if (p < npairs) {
      int qs_, n_;
      chunk_of(p / hkv, qs_, n_);
      cnt = (n_ + RW - 1) / RW;
      if (cnt > 0) ctx = seq_lens[p / hkv] - n_;
    }
    int before = 0;  // units of the pairs taken before this lane's
    for (int j = 0; j < 64; ++j) {
      const int cj = __builtin_amdgcn_readlane(ctx, j);
      const int nj = __builtin_amdgcn_readlane(cnt, j);
      if (cj > ctx || (cj == ctx && j < lane)) before += nj;
    }
    const uint64_t hit = __builtin_amdgcn_ballot_w64(cnt > 0 && before <= un && un < before + cnt);
    if (hit != 0) {
      const int i = __builtin_ctzll(hit);
      const int pp = xcd + 8 * i;
      s = pp / hkv;
      kh = pp % hkv;
      u_local = un - __builtin_amdgcn_readlane(before, i);
    }
  } else {
    int run = 0;
    for (int j0 = 0; xcd + 8 * j0 < npairs; j0 += 64) {
      const int p = xcd + 8 * (j0 + lane);
      int cnt = 0;
      if (p < npairs) {
        int qs_, n_;
        chunk_of(p / hkv, qs_, n_);
        cnt = (n_ + RW - 1) / RW;
      }
      const int incl = wave_inclusive_scan(cnt, lane);
      const uint64_t hit = __builtin_amdgcn_ballot_w64(run + incl > un);
      if (hit != 0) {
        const int i = __builtin_ctzll(hit);
        const int pp = xcd + 8 * (j0 + i);
        s = pp / hkv;
        kh = pp % hkv;
        u_local = un - (run + __builtin_amdgcn_readlane(incl, i) -
                        __builtin_amdgcn_readlane(cnt, i));
        break;
      }
      run += __builtin_amdgcn_readlane(incl, 63);
    }
  }
  if (s < 0) return;  // past the last unit (the same for every wave)
  int qs, n;
  chunk_of(s, qs, n);
  const int L = seq_lens[s];
  const int nu = (n + RW - 1) / RW;  // units of this pair
  const int i0 = (nu - 1 - u_local) * RW;  // last units first: they see the most positions
  const int iw = i0 + w * R;               // this wave's first chunk token
  const int col = lane & 15, grp = lane >> 4;
  const bool valid = n <= L && (int64_t)L <= max_len;
  const bool wave_on = iw < n;
  // the lane's query row in row block h: chunk token iw + h R1 + col / G,
  // head kh * G + col % G; its causal end (exclusive)
  int tok[kNrb], lane_end[kNrb];
  bool active[kNrb];
#pragma unroll
  for (int h = 0; h < kNrb; ++h) {
    tok[h] = iw + h * R1 + col / G;
    active[h] = tok[h] < n;
    lane_end[h] = active[h] ? L - n + tok[h] + 1 : 1;
  }
  const int wave_end = L - n + min(iw + R, n);  // positions this wave needs
  const int p_end = L - n + min(i0 + RW, n);    // positions the workgroup loads

  float* st = reinterpret_cast<float*>(s_mem + w * (2 * SG::BYTES / kWaves));  // [16][D]
  auto store_rows = [&](int tfirst) {
    // st: 16 rows staged in LDS; row r -> (token tfirst + r / G, head r % G)
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

  if (!valid) {  // lengths break the contract: NaN rows, nothing read
    if (!wave_on) return;
    for (int i = lane; i < kRows * D; i += 64) st[i] = __builtin_nanf("");
#pragma unroll
    for (int h = 0; h < kNrb; ++h) store_rows(iw + h * R1);
    return;
  }

  // per row block: q operand, P.V accumulators, running max (scaled, base
  // 2) and the denominator, accumulated by the matrix cores as P times a
  // column of ones, so it lands in the accumulators' row layout.  A
  // negative scale is moved into q (exact sign flips), so the running max
  // can be taken on the raw scores.
  const uint32_t q_sign = qk_scale < 0.0f ? 0x80008000u : 0u;
  const float sc_scale = fabsf(qk_scale);
  uint4 qb[kNrb][KC];
  f32x4_t acc[kNrb][NM], lacc[kNrb];
  float m_run[kNrb];
#pragma unroll
  for (int h = 0; h < kNrb; ++h) {
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      qb[h][c] = make_uint4(0u, 0u, 0u, 0u);
      if (active[h]) {
        const uint4 v = *reinterpret_cast<const uint4*>(
            q + (((int64_t)qs + tok[h]) * hq + kh * G + col % G) * D + (c * 4 + grp) * 8);
        qb[h][c] = make_uint4(v.x ^ q_sign, v.y ^ q_sign, v.z ^ q_sign, v.w ^ q_sign);
      }
    }
#pragma unroll
    for (int m = 0; m < NM; ++m) acc[h][m] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    lacc[h] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    m_run[h] = kNegInf;
  }
  const uint4 ones = make_uint4(kOnes2<T>, kOnes2<T>, kOnes2<T>, kOnes2<T>);
  // positions every stored row of the wave sees (its first token's end)
  const int wave_min_end = L - n + iw + 1;

  // block ids of the positions [0, p_end), 64 at a time: lane j holds block blk_base + j
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
  const int ntiles = (p_end + kTP - 1) / kTP;
  const uint16_t* kh_k = kc + (int64_t)kh * BS * D;
  const uint16_t* kh_v = vc + (int64_t)kh * BS * D;

  // The workgroup's copies of tile j into a stage, straight from HBM to LDS;
  // wave w issues copies w, w + 4, ...  Every unit of a (sequence, KV head)
  // copies the same tiles, so they keep the default cache policy: with the
  // streaming hint the decode uses (each byte read once), L2 dropped the
  // tiles before the pair's other units reached them, and the kernel read
  // 1.61 GB from HBM per call instead of 0.58 GB and took 7% longer.  Copy k of this wave moves, for each
  // lane, 16 bytes of tile row row0_of(k) + lane_row(k) at byte coff[k] of
  // that row's (block, head) slice of the pool; tiles start at multiples of
  // every block size, so the row's block is the tile's block row / BS.
  constexpr int kCopies = SG::JOBS / kWaves;
  // tile row of lane 0 of copy k (wave-uniform) and the lane's row above it
  auto row0_of = [&](int k) -> int {
    const int job = k * kWaves + w;
    return job < SG::KJOBS ? kTile * (job / KC)
                           : kTile * ((job - SG::KJOBS) / 4) + 4 * ((job - SG::KJOBS) % 4);
  };
  const int vrow = lane / VGeo<D>::CHUNKS;  // a V copy's row within its region
  auto lane_row = [&](int k) -> int { return k * kWaves + w < SG::KJOBS ? col : vrow; };
  uint32_t coff[kCopies];
#pragma unroll
  for (int k = 0; k < kCopies; ++k) {
    const int job = k * kWaves + w;
    const int row = row0_of(k) + lane_row(k);
    if (job < SG::KJOBS) {
      const int c = job % KC;
      coff[k] = 2u * (uint32_t)((row % BS) * D + 32 * c + 8 * grp);
    } else {
      const int chunk = (lane % VGeo<D>::CHUNKS) ^ (2 * v_swizzle<D>(vrow));
      coff[k] = 2u * (uint32_t)((row % BS) * D + chunk * 8);
    }
  }
  const uint32_t blk_bytes = 2u * (uint32_t)hkv * BS * D;
  const unsigned char* kh_kb = reinterpret_cast<const unsigned char*>(kh_k);
  const unsigned char* kh_vb = reinterpret_cast<const unsigned char*>(kh_v);

  auto issue = [&](int j, unsigned char* stage) {
    const int t0 = j * kTP;
    if ((min(t0 + kTP, p_end) - 1) / BS - blk_base >= 64) {
      blk_base = t0 / BS;
      vid = load_ids();
    }
    const int b0 = t0 / BS - blk_base;  // the tile's first block in vid
    if (t0 + kTP <= p_end) {
      // a whole tile: every row is in range, block ids are wave-uniform
      // (one of two for the key copies at block size 8)
#pragma unroll
      for (int k = 0; k < kCopies; ++k) {
        const int job = k * kWaves + w;
        const bool is_k = job < SG::KJOBS;
        const int bi = row0_of(k) / BS;  // lane 0's row is the lowest
        const int id_lo = __builtin_amdgcn_readlane(vid, b0 + bi);
        const unsigned char* pool = is_k ? kh_kb : kh_vb;
        // the block's base in scalar registers, then the lane's offset (the
        // empty asm keeps the compiler from hoisting a 64-bit pool + offset
        // per copy into vector registers)
        uint64_t base = (uint64_t)pool + (uint64_t)(uint32_t)id_lo * blk_bytes;
        asm volatile("" : "+s"(base));
        const unsigned char* src = (const unsigned char*)base + coff[k];
        if constexpr (BS < kTile) {
          if (is_k) {
            const int id_hi = __builtin_amdgcn_readlane(vid, b0 + bi + 1);
            uint64_t base_hi = (uint64_t)pool + (uint64_t)(uint32_t)id_hi * blk_bytes;
            asm volatile("" : "+s"(base_hi));
            if (col >= BS) src = (const unsigned char*)base_hi + coff[k];  // rows 16 sb + col
          }
        }
        unsigned char* dst = is_k ? stage + job * SG::KBLK
                                  : stage + SG::KBYTES + ((job - SG::KJOBS) / 4) * VGeo<D>::TILE +
                                        ((job - SG::KJOBS) % 4) * VGeo<D>::REGION;
        if (is_k || VGeo<D>::LANES == 64 || lane < VGeo<D>::LANES)
          __builtin_amdgcn_global_load_lds((const void*)src,
                                           (void __attribute__((address_space(3)))*)dst, 16, 0,
                                           kCachePolicyReuse);
      }
      return;
    }
    // the unit's last tile: rows past p_end - 1 read row p_end - 1
#pragma unroll
    for (int k = 0; k < kCopies; ++k) {
      const int job = k * kWaves + w;
      const int row = row0_of(k) + lane_row(k);
      const int t = min(t0 + row, p_end - 1);
      const int id = __shfl(vid, t / BS - blk_base);
      const unsigned char* pool = job < SG::KJOBS ? kh_kb : kh_vb;
      const uint32_t off = coff[k] - 2u * (uint32_t)((row % BS) * D) + 2u * (uint32_t)((t % BS) * D);
      const unsigned char* src = pool + (uint64_t)(uint32_t)id * blk_bytes + off;
      unsigned char* dst = job < SG::KJOBS ? stage + job * SG::KBLK
                                           : stage + SG::KBYTES + ((job - SG::KJOBS) / 4) * VGeo<D>::TILE +
                                                 ((job - SG::KJOBS) % 4) * VGeo<D>::REGION;
      if (job < SG::KJOBS || VGeo<D>::LANES == 64 || lane < VGeo<D>::LANES)
        __builtin_amdgcn_global_load_lds((const void*)src,
                                         (void __attribute__((address_space(3)))*)dst, 16, 0,
                                         kCachePolicyReuse);
    }
  };

  // the lane's offsets, within a V sub-tile, of column blocks i ^ sw (i < 4)
  // of rows 4 grp + (col >> 2): its transpose reads
  uint32_t vlane[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    vlane[i] = (uint32_t)(grp * VGeo<D>::REGION + (col >> 2) * VGeo<D>::ROW + 8 * (col & 3) +
                          32 * (i ^ v_swizzle<D>(col >> 2)));

  // The wave's row blocks over tile j, in slabs of 32 positions (two
  // sub-tiles): slabs past the wave's last position are skipped; each lane
  // masks at its own row's end.  q.K^T per sub-tile gives lane (col, grp)
  // the scores of positions 4 grp + r (first sub-tile) and 16 + 4 grp + r
  // (second); these 8 weights, in that order, are the lane's k-values of
  // the 16x16x32 P.V product, whose V operand is therefore the two
  // sub-tiles' transpose reads side by side.
  auto compute = [&](int j, const unsigned char* stage) {
#pragma unroll 1
    for (int sl = 0; sl < kSub / 2; ++sl) {
      const int t0 = j * kTP + 2 * kTile * sl;
      if (t0 >= wave_end) break;
      uint4 k0[KC], k1[KC];
      const unsigned char* kb = stage + 2 * sl * KC * SG::KBLK + 16 * lane;
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        k0[c] = *reinterpret_cast<const uint4*>(kb + c * SG::KBLK);
        k1[c] = *reinterpret_cast<const uint4*>(kb + (KC + c) * SG::KBLK);
      }
      uint4 pa_op[kNrb];
#pragma unroll
      for (int h = 0; h < kNrb; ++h) {
        f32x4_t s0 = {0.0f, 0.0f, 0.0f, 0.0f}, s1 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int c = 0; c < KC; ++c) s0 = mfma_k32<T>(k0[c], qb[h][c], s0);
#pragma unroll
        for (int c = 0; c < KC; ++c) s1 = mfma_k32<T>(k1[c], qb[h][c], s1);
        // only slabs that reach past the first token's end need the mask;
        // rows of tokens past the chunk are never stored
        if (t0 + 2 * kTile > wave_min_end) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            if (t0 + 4 * grp + r >= lane_end[h]) s0[r] = kNegInf;
            if (t0 + kTile + 4 * grp + r >= lane_end[h]) s1[r] = kNegInf;
          }
        }
        // the lane's largest score: llvm.maximum maps to v_maximum3_f32,
        // four instructions for the eight scores; fmaxf's IEEE semantics had
        // the compiler quiet each raw matrix-core result first (eleven)
        const float ma = fmax_nan(fmax_nan(s0[0], s0[1]), s0[2]);
        const float mb = fmax_nan(fmax_nan(s0[3], s1[0]), s1[1]);
        const float lm = fmax_nan(mb, fmax_nan(fmax_nan(s1[2], s1[3]), ma)) * sc_scale;
        if (__builtin_amdgcn_ballot_w64(lm > m_run[h] + kRescaleSlack) != 0) {
          float mx = fmaxf(lm, __shfl_xor(lm, 16));
          mx = fmaxf(mx, __shfl_xor(mx, 32));
          const float m_new = fmaxf(m_run[h], mx);
          const float corr = exp2_fast(m_run[h] - m_new);  // 0 when m_run = -inf
          m_run[h] = m_new;
          float cr[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) cr[r] = __shfl(corr, 4 * grp + r);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            lacc[h][r] *= cr[r];
#pragma unroll
            for (int m = 0; m < NM; ++m) acc[h][m][r] *= cr[r];
          }
        }
        // weight = 2^(score * scale - m), one FMA and one exp each
        const float nm = -m_run[h];
        pa_op[h] = make_uint4(
            pack2<T>(exp2_fast(fmaf(s0[0], sc_scale, nm)), exp2_fast(fmaf(s0[1], sc_scale, nm))),
            pack2<T>(exp2_fast(fmaf(s0[2], sc_scale, nm)), exp2_fast(fmaf(s0[3], sc_scale, nm))),
            pack2<T>(exp2_fast(fmaf(s1[0], sc_scale, nm)), exp2_fast(fmaf(s1[1], sc_scale, nm))),
            pack2<T>(exp2_fast(fmaf(s1[2], sc_scale, nm)), exp2_fast(fmaf(s1[3], sc_scale, nm))));
        lacc[h] = mfma_k32<T>(pa_op[h], ones, lacc[h]);
      }
      // V operand of column block m: rows 4 grp + r of the first sub-tile,
      // then of the second, column 16 m + col
      const uint32_t vb = (uint32_t)(uintptr_t)(stage + SG::KBYTES + 2 * sl * VGeo<D>::TILE);
      const uint32_t va[4] = {vb + vlane[0], vb + vlane[1], vb + vlane[2], vb + vlane[3]};
      uint2 vlo[NM], vhi[NM];
      read_v_slab<NM>(vlo, vhi, va);
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        const uint4 vop = make_uint4(vlo[m].x, vlo[m].y, vhi[m].x, vhi[m].y);
#pragma unroll
        for (int h = 0; h < kNrb; ++h) acc[h][m] = mfma_k32<T>(pa_op[h], vop, acc[h][m]);
      }
    }
  };

  // one tile in flight while the previous one is computed; one barrier a tile
  issue(0, s_st0);
  for (int j = 0;;) {
    wait_vmem_all();
    __syncthreads();  // tile j is in LDS; every wave is done with tile j - 1
    if (j + 1 < ntiles) issue(j + 1, s_st1);
    if (wave_on) compute(j, s_st0);
    if (++j >= ntiles) break;
    wait_vmem_all();
    __syncthreads();
    if (j + 1 < ntiles) issue(j + 1, s_st0);
    if (wave_on) compute(j, s_st1);
    if (++j >= ntiles) break;
  }
  __syncthreads();  // the stages are free: each wave stages its rows in its quarter
  if (!wave_on) return;

  // out = acc / l, staged row-major, stored whole lines
#pragma unroll
  for (int h = 0; h < kNrb; ++h) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 4 * grp + r;
#pragma unroll
      for (int m = 0; m < NM; ++m)
        st[row * D + 16 * m + col] = bad ? __builtin_nanf("") : acc[h][m][r] / lacc[h][r];
    }
    store_rows(iw + h * R1);
  }
}

// Units (workgroups) one XCD can get at most: each sequence has at most
// ceil(hkv / 8) of its (sequence, KV head) pairs on one XCD, and a pair's
// chunk of n tokens has ceil(n / tokens per unit) units.
static int64_t units_per_xcd(int32_t total_q, int32_t num_seqs, int32_t hkv, int32_t group) {
  const int64_t per_unit = kWaves * kNrb * kRows / group;
  return ((int64_t)hkv + 7) / 8 * (((int64_t)total_q + per_unit - 1) / per_unit + num_seqs);
}

template <typename T, int D, int BS, int G>
static hipError_t launch_t(const PrefillArgs& a) {
  static int lds_cache[kMaxDevices];
  const hipError_t fit = check_lds((const void*)pa_prefill_kernel<T, D, BS, G>, 0, lds_cache);
  if (fit != hipSuccess) return fit;
  const int64_t grid = 8 * units_per_xcd(a.total_q, a.num_seqs, a.num_kv_heads, G);
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
  return 8 * kWaves * units_per_xcd(total_q, num_seqs, num_kv_heads, group);
}

}  // namespace pa
