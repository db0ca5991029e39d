// decode_streamk.h -- paged decode attention, the balanced (stream-K)
// decomposition used by pa_decode (runs cut at partition boundaries when
// partition_size is given) and by pa_decode_fp8, as templates:
// decode_streamk.hip instantiates them for 16-bit pools, decode_fp8.hip for
// 8-bit E4M3 pools.
//
// What is computed is the same as the vector kernel's: for every
// sequence s and query head h, softmax attention of q[s][h] over positions
// 0..L_s-1 read through the sequence's block table ("What problem does
// PagedAttention solve ...", section "How PagedAttention works").  What
// differs is how the work is cut.
//
// Tile order: for each KV head, the sequences' tiles back to back, sequence
// s holding ceil(L_s / n) tiles of n positions (n = 16 for 16-bit pools, 32
// for 8-bit ones).  The launch has two workgroups (8 waves) per CU, or one
// on batches of few long sequences for the 16-bit matrix-core tile wave,
// all resident at once (a whole number of waves per KV head); wave w works on
// head w % hkv and takes the (w / hkv)-th of that head's equal runs of
// units.  A unit is a tile, or with an explicit partition_size a partition
// of that many positions (runs then start and end only at partition
// boundaries).  Adjacent waves therefore read the same positions of
// adjacent heads, neighbouring pieces of the same pool blocks, at about the
// same time: 2% faster on the mixed decode step than the pairs in
// (sequence, head) order, 4% with 8-bit pools.  Every wave streams the same
// number of units, never waits for another wave, and never sits idle at the
// end of a work unit: a kernel with one workgroup per (sequence, head,
// 512-position) unit spent a merge through LDS and a barrier on every unit,
// and its units differed in size.  Each wave finds its first sequence from
// a prefix sum of the unit counts (recomputed by every wave from seq_lens; a
// few hundred integers from L2), then walks its run sequence by sequence:
//   - a pair that lies wholly inside the run is finished in place: out =
//     acc / l, rounded to the output type;
//   - a pair cut by the run's start or end leaves a partial (m, l, acc) in
//     the wave's slot 0 (the pair it starts in) or slot 1 (the pair it ends
//     in) of the workspace;
//   - the wave that processes a pair's last tile records which runs of the
//     head hold its partials (meta; run c of head kh is wave c * hkv + kh,
//     and unit u of the head's order lies in run u / C, C units per run),
//     and pa_streamk_reduce merges them by log-sum-exp
//     ("Continuous Batching & Paged Attention", section "Attention needs
//     memory that grows with the conversation": plain softmax attention; the
//     merge is the identity M = max m_p, out = sum 2^(m_p - M) acc_p /
//     sum 2^(m_p - M) l_p) and writes the zero rows of empty sequences and
//     the NaN rows of sequences whose length breaks the contract.
// Within a pair a wave consumes its tiles in order with TileWave
// (pa_mfma.h) or TileWave8 (pa_mfma_fp8.h) -- K to registers, V to LDS,
// q.K^T and P.V on MFMA -- or with TileWaveV (pa_valu.h, the vector unit
// alone, K and V to registers).  Each tile is issued one tile ahead of its
// use, two tiles ahead for the 16-bit matrix-core tile wave (kDeep).  The
// run's block ids are staged in a register, one per lane, and read with
// v_readlane: no memory access between two tiles.
#pragma once

#include <type_traits>

#include "pa_launch.h"
#include "pa_mfma.h"
#include "pa_mfma_fp8.h"
#include "pa_valu.h"

namespace pa {

namespace {

constexpr int kWaves = 4;              // waves per workgroup (independent)
constexpr int kThreads = 64 * kWaves;
constexpr int kMinChunk = 4;           // tiles per wave at least

// Workgroups per CU the launch uses: two (8 waves), not the three that fit.
// The K/V gather saturates with as few as 4 waves per CU (the gather-only
// probe takes the same time with 4 to 20), so the third workgroup adds no
// loads in flight that the memory system can use; it only makes the runs a
// third shorter (more pairs cut, more partials, more wave starts) and puts
// a third more waves on each SIMD.  Measured with two instead of three:
// mixed decode step 358 -> 346 us, the same over 8-bit pools 222 -> 204 us,
// long context at block 16 416 -> 394 us.
constexpr int kWorkgroupsPerCu = 2;

// Sum over the wave, returned as a wave-uniform (scalar) value.
__device__ __forceinline__ int wave_sum(int x) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) x += __shfl_xor(x, m);
  return __builtin_amdgcn_readfirstlane(x);
}

// Lane i's value as a wave-uniform (scalar) value; i must be uniform.
__device__ __forceinline__ int lane_value(int x, int i) {
  return __builtin_amdgcn_readlane(x, i);
}

__device__ __forceinline__ int wave_inclusive_scan(int x, int lane) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    const int y = __shfl_up(x, m);
    if (lane >= m) x += y;
  }
  return x;
}

}  // namespace

// The tile wave of a pool element type: TileWave (pa_mfma.h) for 16-bit
// pools, TileWave8 (pa_mfma_fp8.h) for 8-bit E4M3 pools, TileWaveV
// (pa_valu.h, the vector unit alone) for 16-bit pools tagged Vec.
template <typename T, typename KV, int D, int BS, int G>
struct TileWaveOf {
  using type = TileWave<T, D, BS, G>;
};
template <typename T, int D, int BS, int G>
struct TileWaveOf<T, FP8, D, BS, G> {
  using type = TileWave8<T, D, BS, G>;
};
template <typename T, int D, int BS, int G>
struct TileWaveOf<T, Vec, D, BS, G> {
  using type = TileWaveV<T, D, BS, G>;
};

// kGather = true is the gather-only instantiation behind pa_probe_gather:
// the same split, walk and K/V loads, no q, no arithmetic on the data and no
// results (a word is written to `out` only if the XOR of the loaded data hits
// a value it cannot be expected to hit).  KV is the pool element type (T, or
// FP8 with out_scale = v_scale applied to every result; for 16-bit pools
// out_scale is not used).  Two waves per SIMD are all the launch uses
// (kWorkgroupsPerCu), so the compiler may take up to 256 registers; at
// d 128 and block 16 the 8-bit tile wave uses 207-217 of them (with the 168
// that three waves allow it spent 8% more time on the mixed step), the
// 16-bit matrix-core one 183-195, the vector-unit one 148-256 (at group 8
// all of them, and it spills 80-160 bytes per lane; the 8-bit one spills
// 48 bytes at block 8).
//
// kDeep: each wave with two tiles in flight instead of one (the 16-bit
// matrix-core tile wave only, whose loads the compiler counts exactly; see
// the walk below).  The launch puts one workgroup of these on each CU for
// batches of few long sequences, two for the rest (launch_t).
//
// kNt: the K/V loads carry the streaming hint (kDeep only may drop it; see
// launch_t).
template <typename T, int D, int BS, int G, bool kGather, typename KV, bool kDeep = false,
          bool kNt = true>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
pa_decode_streamk(uint16_t* __restrict__ out, float* __restrict__ ws_acc,
                  float2* __restrict__ ws_ml, int4* __restrict__ ws_meta,
                  const uint16_t* __restrict__ q,
                  const typename TileWaveOf<T, KV, D, BS, G>::type::Elem* __restrict__ kc,
                  const typename TileWaveOf<T, KV, D, BS, G>::type::Elem* __restrict__ vc,
                  const int32_t* __restrict__ block_tables,
                  const int32_t* __restrict__ seq_lens, int32_t num_seqs, int32_t hkv,
                  int32_t mb, int32_t nb, int32_t nwaves, int32_t part_tiles, float qk_scale,
                  float out_scale, int32_t start, float* __restrict__ pair_acc,
                  float2* __restrict__ pair_ml) {
  using TW = typename TileWaveOf<T, KV, D, BS, G>::type;
  constexpr int KL = TW::KL, kT = TW::kTileLen, kIds = TW::kIds;
  constexpr bool kScaled = std::is_same<KV, FP8>::value;
  static_assert(!kDeep || std::is_same<KV, T>::value, "kDeep: the 16-bit matrix-core tile wave");
  static_assert(kNt || kDeep, "the K/V loads without the streaming hint: kDeep only");
  __shared__ __attribute__((aligned(16))) unsigned char s_mem[kWaves * 2 * TW::kTileBytes];
  static_assert(sizeof(s_mem) <= kMaxLdsBytes, "one workgroup's LDS fits gfx950's 160 KiB");
  static_assert(kWorkgroupsPerCu * sizeof(s_mem) <= kMaxLdsBytes,
                "the workgroups the launch puts on one CU fit its LDS together");

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wave = blockIdx.x * kWaves + w;
  const int hq = hkv * G;
  const int64_t max_len = (int64_t)mb * BS;
  // Positions [start, L) of each sequence are walked (start = 0 but for the
  // tails of pa_decode_shared_prefix, whose first `start` positions are a
  // prefix attended separately).
  auto tiles_of = [&](int L) -> int {
    return (L > start && (int64_t)L <= max_len) ? (L - start + kT - 1) / kT : 0;
  };

  // ---- this wave's run: wave w works on KV head w % hkv, and the waves of
  // one head split that head's order of units (the sequences' units back to
  // back) into equal runs.  A unit is one tile, or with part_tiles > 0 a
  // partition of part_tiles tiles (the last of a sequence may be shorter):
  // runs then start and end only at partition boundaries, and the
  // partitions a wave walks in one sequence are merged in its registers.
  // Adjacent waves take adjacent heads of the same positions, so they read
  // neighbouring pieces of the same pool blocks at about the same time.
  const int pt = part_tiles > 0 ? part_tiles : 1;  // tiles per unit
  auto units_of = [&](int L) -> int { return (tiles_of(L) + pt - 1) / pt; };
  const int nwh = nwaves / hkv;  // waves per head (the launch has nwaves >= hkv)
  const int kh0 = wave % hkv, jw = wave / hkv;
  if (jw >= nwh) return;
  // seq_lens is read kLenBatch x 64 lengths at a time, all loads in flight
  // together: these scans come before the wave's first K/V load, so each
  // round trip delays the whole wave.  The first 256 lengths stay in
  // registers for the search below (a batch of up to 256 sequences is read
  // once).  Reading 1,024 at a time saved another 2% on 4,096 short
  // sequences but cost the mixed step and the long-context batch 1%.
  constexpr int kLenBatch = 4;
  auto load_lens = [&](int b, int (&Lb)[kLenBatch]) {
#pragma unroll
    for (int k = 0; k < kLenBatch; ++k) {
      const int j = b + 64 * k + lane;
      Lb[k] = j < num_seqs ? seq_lens[j] : 0;
    }
  };
  int Lb0[kLenBatch];
  load_lens(0, Lb0);
  int64_t per_head = 0, per_head_tiles = 0;  // units and tiles of all sequences
  for (int b = 0; b < num_seqs; b += 64 * kLenBatch) {
    int Lb[kLenBatch];
    if (b == 0) {
#pragma unroll
      for (int k = 0; k < kLenBatch; ++k) Lb[k] = Lb0[k];
    } else {
      load_lens(b, Lb);
    }
#pragma unroll
    for (int k = 0; k < kLenBatch; ++k) {
      per_head += wave_sum(units_of(Lb[k]));
      per_head_tiles += wave_sum(tiles_of(Lb[k]));
    }
  }
  const int64_t chunk =
      max((int64_t)(pt == 1 ? kMinChunk : 1), (per_head + nwh - 1) / nwh);  // units per run
  const int64_t u0 = (int64_t)jw * chunk;
  if (u0 >= per_head) return;
  const int64_t u1 = min(per_head, u0 + chunk);

  // The sequence holding unit u, its length, where its units start, and
  // where its tiles start (index of its first unit / tile in the head's
  // order).
  struct Where { int s, L; int64_t ustart, tstart; };
  auto locate = [&](int64_t u) -> Where {
    int64_t urun = 0, trun = 0;
    for (int b = 0; b < num_seqs; b += 64 * kLenBatch) {
      int Lb[kLenBatch];
      if (b == 0) {
#pragma unroll
        for (int k = 0; k < kLenBatch; ++k) Lb[k] = Lb0[k];
      } else {
        load_lens(b, Lb);
      }
#pragma unroll
      for (int k = 0; k < kLenBatch; ++k) {
        const int un = units_of(Lb[k]), tn = tiles_of(Lb[k]);
        const int uincl = wave_inclusive_scan(un, lane);
        const int tincl = wave_inclusive_scan(tn, lane);
        const uint64_t hit = __builtin_amdgcn_ballot_w64(urun + uincl > u);
        if (hit != 0) {
          const int i = __builtin_ctzll(hit);
          return {b + 64 * k + i, lane_value(Lb[k], i),
                  urun + lane_value(uincl, i) - lane_value(un, i),
                  trun + lane_value(tincl, i) - lane_value(tn, i)};
        }
        urun += lane_value(uincl, 63);
        trun += lane_value(tincl, 63);
      }
    }
    return {-1, 0, urun, trun};
  };
  const Where w0 = locate(u0);
  int s = w0.s;
  if (s < 0) return;  // unreachable: u0 < per_head
  int64_t seq_ustart = w0.ustart;  // the current sequence's first unit
  const int64_t g0 = w0.tstart + (u0 - w0.ustart) * pt;  // the run's first tile
  int64_t g1 = per_head_tiles;                          // one past its last tile
  if (u1 < per_head) {
    if (pt == 1) {
      g1 = u1;
    } else {
      const Where w1 = locate(u1);
      g1 = w1.tstart + (u1 - w1.ustart) * pt;
    }
  }
  int L = w0.L;
  int ns = tiles_of(L);
  if (ns == 0) return;  // unreachable: the first hit has units
  const int kh = kh0;
  int t_lo = (int)(g0 - w0.tstart);

  // The segment's result: final rows for a pair wholly inside the run, else
  // a partial in slot 0 (the run's first pair) or 1 (its last); the wave
  // holding a pair's last tile records where its partials are.  The G x D
  // result leaves the MFMA layout 64 bytes per head row at a time, so it is
  // staged row-major in the wave's V tiles (idle once the last tile is
  // consumed) and stored 16 bytes per lane: whole, contiguous cache lines.
  // (Stores of 32 or 64 bytes per instruction cost the mixed decode step 2%.)
  unsigned char* vtile = s_mem + w * 2 * TW::kTileBytes;
  auto write_result = [&](const TW& t, bool bad, int64_t row0, int t_lo,
                          int t_hi, int ns, bool first, int64_t pair_ustart) {
    const bool whole = t_lo == 0 && t_hi == ns;
    float* st = reinterpret_cast<float*>(vtile);  // [G][D]
    t.stage(st, whole && pair_acc == nullptr, bad, kScaled ? out_scale : 1.0f);
    // one wave's LDS accesses take effect in program order
    if (whole && pair_acc != nullptr) {
      // a shared-prefix tail: the whole pair's state, for the merge with the prefix
      for (int i = lane * 4; i < G * D; i += 64 * 4)
        *reinterpret_cast<float4*>(pair_acc + row0 * D + i) =
            *reinterpret_cast<const float4*>(st + i);
      const float2 ml = t.ml_of_lane();
      if (lane < G) pair_ml[row0 + lane] = make_float2(ml.x, bad ? __builtin_nanf("") : ml.y);
    } else if (whole) {
      for (int i = lane * 8; i < G * D; i += 64 * 8) {
        const float4 a = *reinterpret_cast<const float4*>(st + i);
        const float4 b = *reinterpret_cast<const float4*>(st + i + 4);
        *reinterpret_cast<uint4*>(out + row0 * D + i) =
            make_uint4(pack2<T>(a.x, a.y), pack2<T>(a.z, a.w), pack2<T>(b.x, b.y),
                       pack2<T>(b.z, b.w));
      }
    } else {
      const int64_t slot = (int64_t)wave * 2 + (first ? 0 : 1);
      for (int i = lane * 4; i < G * D; i += 64 * 4)
        *reinterpret_cast<float4*>(ws_acc + slot * G * D + i) =
            *reinterpret_cast<const float4*>(st + i);
      const float2 ml = t.ml_of_lane();
      if (lane < G) ws_ml[slot * G + lane] = make_float2(ml.x, bad ? __builtin_nanf("") : ml.y);
    }
    if (t_hi == ns && lane == 0) {
      const int c_first = (int)(pair_ustart / chunk);
      const int c_last = (int)((pair_ustart + (ns + pt - 1) / pt - 1) / chunk);
      ws_meta[row0 / G] = make_int4(c_first, c_last, pair_ustart % chunk != 0, 0);
    }
  };
  static_assert(sizeof(float) * G * D <= 2 * TW::kTileBytes, "the result fits the wave's V tiles");

  TW tw;
  // The next sequence's length, first 64 table entries and q rows, fetched
  // when a segment starts so that the next segment does not begin with
  // three dependent round trips.  All initialised: a register left undefined
  // on some path can make the compiler wait for every outstanding load when
  // it copies that register inside the tile loop.
  int next_L = 0, next_raw = 0;
  bool have_next = false, use_next = false;
  typename TW::QRegs next_q{};
  // The vector tile wave at group 8 holds 8 heads' q, scores and sums per
  // lane; the prefetch's registers (32 for q alone) made it spill 320 bytes
  // per lane, so it reads the next sequence when its segment starts.
  constexpr bool kPrefetch = !(std::is_same<KV, Vec>::value && G >= 8);

  int64_t g = g0;
  while (true) {
    // ---- one segment: pair (s, kh), tiles [t_lo, t_hi)
    const int t_hi = (int)min((int64_t)ns, (int64_t)t_lo + (g1 - g));
    const int p_lo = start + t_lo * kT;
    const int p_end = min(L, start + t_hi * kT);  // positions [p_lo, p_end)
    const int ntiles = t_hi - t_lo;
    const int64_t row0 = (int64_t)s * hq + (int64_t)kh * G;
    const int32_t* bt_row = block_tables + (int64_t)s * mb;

    tw.init(kc, vc, hkv, kh, vtile);
    if constexpr (!kGather) {
      if (kPrefetch && use_next)
        tw.qr = next_q;
      else
        tw.load_q(q + row0 * D);
    }
    tw.reset();
    uint32_t gathered = 0;
    auto consume = [&](const uint4 (&kr)[KL], int buf, int t0) {
      if constexpr (kGather) {
        // every loaded K word enters the XOR, or the compiler narrows the loads
#pragma unroll
        for (int c = 0; c < KL; ++c) gathered ^= kr[c].x ^ kr[c].y ^ kr[c].z ^ kr[c].w;
        if constexpr (kDeep)
          gathered ^= lds_read_u32((uint32_t)(uintptr_t)(vtile + buf * TW::kTileBytes) + 4 * lane);
        else
          gathered ^= reinterpret_cast<const uint32_t*>(vtile + buf * TW::kTileBytes)[lane];
      } else if constexpr (kDeep) {
        tw.template consume<false>(kr, buf, t0, p_end, qk_scale);
      } else {
        tw.consume(kr, buf, t0, p_end, qk_scale);
      }
    };

    // block ids of the segment, 64 at a time: lane j holds block blk_base + j
    const int blk_last = (p_end - 1) / BS;
    int blk_base = p_lo / BS;
    bool bad = false;
    // raw: lane j's table entry blk_base + j (loaded here, or prefetched)
    auto take_ids = [&](int raw) {
      int id = 0;
      if (blk_base + lane <= blk_last) {
        id = raw;
        if (id < 0 || id >= nb) {
          bad = true;  // never dereferenced: block 0 is read, the rows become NaN
          id = 0;
        }
      }
      bad = __builtin_amdgcn_ballot_w64(bad) != 0;
      return id;
    };
    auto load_ids = [&]() {
      return take_ids(blk_base + lane <= blk_last ? bt_row[blk_base + lane] : 0);
    };
    int vid = use_next ? take_ids(next_raw) : load_ids();  // prefetched from block start / BS

    auto issue = [&](uint4 (&kr)[KL], int buf, int j) {
      const int t0 = p_lo + j * kT;
      int b = t0 / BS - blk_base;
      if (b + kIds - 1 >= 64) {  // past this batch of ids
        blk_base += b;
        b = 0;
        vid = load_ids();
      }
      int ids[kIds];
      ids[0] = __builtin_amdgcn_readlane(vid, b);
#pragma unroll
      for (int i = 1; i < kIds; ++i)
        ids[i] = (t0 + i * BS < p_end) ? __builtin_amdgcn_readlane(vid, b + i) : ids[0];
      if constexpr (kDeep)
        tw.template issue_ids_counted<kNt>(kr, buf, t0, p_end - 1, ids);
      else
        tw.issue_ids(kr, buf, t0, p_end - 1, ids);
    };

    uint4 ka[KL], kb[KL];
    issue(ka, 0, 0);
    // the run goes on past this sequence
    have_next = kPrefetch && g + ntiles < g1 && s + 1 < num_seqs;
    if (have_next) {
      next_L = seq_lens[s + 1];
      const int b0 = start / BS;  // the next segment's first block
      next_raw = b0 + lane < mb ? block_tables[(int64_t)(s + 1) * mb + b0 + lane] : 0;
      if constexpr (!kGather)
        TW::fetch_q(next_q, q + ((int64_t)(s + 1) * hq + (int64_t)kh * G) * D);
    }
    // Tile j + 1 goes into the other buffer.  Without kDeep the wave waits
    // for everything, then issues it, so one tile is in flight per wave
    // while it computes.  kDeep: tile j + 1 is issued before the wait for
    // tile j, so two are in flight while the wave waits, and the wait leaves
    // tile j + 1's loads outstanding.  On the bandwidth-bound batches, eight
    // waves per CU with two tiles each were 1.5-2.5% slower than with one
    // (more scattered requests outstanding than the memory system serves
    // well), and four waves with two tiles each 1.5-2% faster than eight
    // with one; on many short sequences eight waves with two tiles each are
    // the fastest.
    auto next = [&](uint4 (&kn)[KL], int buf, int jn) {
      if constexpr (kDeep) {
        if (jn < ntiles) {
          issue(kn, buf, jn);
          wait_vmem_but<TW::kLoadsPerTile>();
        } else {
          wait_vmem_all();
        }
      } else {
        wait_vmem_all();
        if (jn < ntiles) issue(kn, buf, jn);
      }
    };
    // Tiles in pairs, the loop's only exit at its top: a loop left from its
    // middle gave the compiler undefined loop values to copy, and the copy
    // of an undefined register made it wait for every outstanding load.
    if constexpr (std::is_same<KV, Vec>::value) {
      // the vector tile wave waits for everything before each issue, so a
      // loop left from its middle costs it nothing, and its two copies of
      // the tile step (not three) leave it fewer registers to spill at
      // group 8
      for (int j = 0;;) {
        next(kb, 1, j + 1);
        consume(ka, 0, p_lo + j * kT);
        if (++j >= ntiles) break;
        next(ka, 0, j + 1);
        consume(kb, 1, p_lo + j * kT);
        if (++j >= ntiles) break;
      }
    } else {
      int j = 0;
      for (; j + 1 < ntiles; j += 2) {
        next(kb, 1, j + 1);
        consume(ka, 0, p_lo + j * kT);
        next(ka, 0, j + 2);
        consume(kb, 1, p_lo + (j + 1) * kT);
      }
      if (j < ntiles) {
        next(kb, 1, j + 1);
        consume(ka, 0, p_lo + j * kT);
      }
    }
    if constexpr (kGather) {
      if (gathered == 0x9e3779b9u && lane == 0) out[0] = (uint16_t)gathered;
    } else {
      tw.finish();
      write_result(tw, bad, row0, t_lo, t_hi, ns, g == g0, seq_ustart);
    }

    g += ntiles;
    if (g >= g1) break;
    // the run goes on, so this sequence ended here: the next one, same head
    t_lo = 0;
    seq_ustart += (ns + pt - 1) / pt;
    use_next = have_next && tiles_of(next_L) > 0;
    if (use_next) {
      ++s;
      L = next_L;
      ns = tiles_of(L);
    } else {
      do {
        if (++s >= num_seqs) return;  // unreachable: tiles remain in the run
        L = seq_lens[s];
        ns = tiles_of(L);
      } while (ns == 0);
    }
  }
}

// Merge of the partials of every (sequence, KV head) pair split between
// waves, plus the rows no wave writes: zero rows for empty sequences, NaN
// rows for lengths outside [0, max_blocks_per_seq * block_size].  TPP
// threads per pair, 256 / TPP pairs per workgroup: 256 when pairs are few
// (each long pair has many partials, and the more threads merge it the
// less of their load latency is in series), 64 when they are many (4,096
// sequences x 8 heads in workgroups of one pair launched 32,768 workgroups,
// most for pairs no run cut, and the merge took 15 us).  A thread merges 4
// consecutive elements of one query head at a time.  The length and the
// pair's record are loaded together, then the partials four at a time with
// all their loads in flight at once.
constexpr int kManyPairs = 4096;  // from this many pairs on, one wave per pair

template <typename T, int D, int G, int TPP>
__global__ void __launch_bounds__(256)
pa_streamk_reduce(uint16_t* __restrict__ out, const float* __restrict__ ws_acc,
                  const float2* __restrict__ ws_ml, const int4* __restrict__ ws_meta,
                  const int32_t* __restrict__ seq_lens, int32_t num_pairs, int32_t hkv,
                  int32_t max_len) {
  static_assert(TPP == 64 || TPP == 256, "a wave or a workgroup per pair");
  const int lane = threadIdx.x % TPP;
  const int pair = blockIdx.x * (256 / TPP) + threadIdx.x / TPP;
  if (pair >= num_pairs) return;
  const int s = pair / hkv, kh = pair % hkv;
  const int64_t row0 = (int64_t)s * hkv * G + (int64_t)kh * G;
  const int L = seq_lens[s];
  const int4 meta = ws_meta[pair];  // meaningful only when L is in range
  if (L <= 0 || L > max_len) {
    const uint32_t v = L == 0 ? 0u : (uint32_t)to_bits<T>(__builtin_nanf("")) * 0x10001u;
    for (int i = lane * 8; i < G * D; i += TPP * 8)
      *reinterpret_cast<uint4*>(out + row0 * D + i) = make_uint4(v, v, v, v);
    return;
  }
  const int c_first = meta.x, c_last = meta.y;
  if (c_first == c_last) return;  // finished by one wave
  // the pair's partials, kBatch read per round trip
  auto merge = [&](auto batch) {
    constexpr int kBatch = decltype(batch)::value;
    for (int i = lane * 4; i < G * D; i += TPP * 4) {
      const int h = i / D, d = i % D;
      float M = kNegInf, den = 0.0f;
      float num[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      for (int c0 = c_first; c0 <= c_last; c0 += kBatch) {
        float2 ml[kBatch];
        float4 a[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const int c = c0 + u;
          ml[u] = make_float2(kNegInf, 0.0f);
          a[u] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
          if (c <= c_last) {
            const int64_t slot = 2 * ((int64_t)c * hkv + kh) + (c == c_first ? meta.z : 0);
            ml[u] = ws_ml[slot * G + h];
            a[u] = *reinterpret_cast<const float4*>(ws_acc + (slot * G + h) * D + d);
          }
        }
        float Mb = M;
#pragma unroll
        for (int u = 0; u < kBatch; ++u) Mb = fmaxf(Mb, ml[u].x);
        const float base = (Mb == kNegInf) ? 0.0f : Mb;
        const float r = exp2_fast(M - base);  // rescale what is summed so far
        den *= r;
#pragma unroll
        for (int e = 0; e < 4; ++e) num[e] *= r;
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const float f = exp2_fast(ml[u].x - base);
          den = fmaf(f, ml[u].y, den);
          num[0] = fmaf(f, a[u].x, num[0]);
          num[1] = fmaf(f, a[u].y, num[1]);
          num[2] = fmaf(f, a[u].z, num[2]);
          num[3] = fmaf(f, a[u].w, num[3]);
        }
        M = Mb;
      }
      const uint2 o = make_uint2(pack2<T>(num[0] / den, num[1] / den),
                                 pack2<T>(num[2] / den, num[3] / den));
      *reinterpret_cast<uint2*>(out + (row0 + h) * D + d) = o;
    }
  };
  // A pair cut into many runs (a long sequence in a small batch: 61 partials
  // per pair of the pages' worked example) is merged 16 partials per round
  // trip (6.6 us against 10.3 us 4 at a time); the usual one or two
  // partials 4 at a time (16, mostly predicated off, cost the mixed step
  // 0.5 us and 4,096 short sequences 3%).
  if (TPP == 256 && c_last - c_first >= 4)
    merge(std::integral_constant<int, 16>{});
  else
    merge(std::integral_constant<int, 4>{});
}

// The merge of pa_decode_shared_prefix, one workgroup per (sequence, KV
// head) pair: the prefix's chunk partials (pre_*, rows [chunk][S * Hq]) and
// the tail's state (the pair buffer when one wave finished the tail, else
// the waves' slots named by the pair's record), folded four at a time by
// log-sum-exp in that order.  A sequence shorter than the prefix, longer
// than its table, or whose table's first prefix_blocks entries differ from
// sequence 0's breaks the contract: NaN rows.  One with no positions past
// the prefix takes the prefix's result alone.
template <typename T, int D, int G>
__global__ void __launch_bounds__(256)
pa_prefix_merge(uint16_t* __restrict__ out, const float* __restrict__ ws_acc,
                const float2* __restrict__ ws_ml, const int4* __restrict__ ws_meta,
                const float* __restrict__ pair_acc, const float2* __restrict__ pair_ml,
                const float* __restrict__ pre_acc, const float2* __restrict__ pre_ml,
                const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ block_tables,
                int32_t num_seqs, int32_t hkv, int32_t mb, int32_t max_len, int32_t start,
                int32_t prefix_blocks, int32_t nchunks) {
  constexpr int kBatch = 4;
  const int pair = blockIdx.x;
  const int s = pair / hkv, kh = pair % hkv;
  const int64_t rows = (int64_t)num_seqs * hkv * G;  // rows of one chunk's partials
  const int64_t row0 = (int64_t)s * hkv * G + (int64_t)kh * G;
  const int L = seq_lens[s];
  const int4 meta = ws_meta[pair];  // meaningful only when the tail was walked
  int differs = 0;
  for (int j = threadIdx.x; j < prefix_blocks; j += 256)
    differs |= block_tables[(int64_t)s * mb + j] != block_tables[j];
  differs = __syncthreads_or(differs);
  if (differs || L < start || L > max_len) {
    const uint32_t v = (uint32_t)to_bits<T>(__builtin_nanf("")) * 0x10001u;
    for (int i = threadIdx.x * 8; i < G * D; i += 256 * 8)
      *reinterpret_cast<uint4*>(out + row0 * D + i) = make_uint4(v, v, v, v);
    return;
  }
  const bool tail = L > start, split = tail && meta.x != meta.y;
  const int n = nchunks + (!tail ? 0 : split ? meta.y - meta.x + 1 : 1);
  for (int i = threadIdx.x * 4; i < G * D; i += 256 * 4) {
    const int h = i / D, d = i % D;
    auto source = [&](int k, float2& ml, float4& a) {
      if (k < nchunks) {
        const int64_t r = (int64_t)k * rows + row0 + h;
        ml = pre_ml[r];
        a = *reinterpret_cast<const float4*>(pre_acc + r * D + d);
      } else if (!split) {
        ml = pair_ml[row0 + h];
        a = *reinterpret_cast<const float4*>(pair_acc + (row0 + h) * D + d);
      } else {
        const int c = meta.x + (k - nchunks);
        const int64_t slot = 2 * ((int64_t)c * hkv + kh) + (c == meta.x ? meta.z : 0);
        ml = ws_ml[slot * G + h];
        a = *reinterpret_cast<const float4*>(ws_acc + (slot * G + h) * D + d);
      }
    };
    float M = kNegInf, den = 0.0f;
    float num[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int k0 = 0; k0 < n; k0 += kBatch) {
      float2 ml[kBatch];
      float4 a[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        ml[u] = make_float2(kNegInf, 0.0f);
        a[u] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        if (k0 + u < n) source(k0 + u, ml[u], a[u]);
      }
      float Mb = M;
#pragma unroll
      for (int u = 0; u < kBatch; ++u) Mb = fmaxf(Mb, ml[u].x);
      const float base = (Mb == kNegInf) ? 0.0f : Mb;
      const float r = exp2_fast(M - base);
      den *= r;
#pragma unroll
      for (int e = 0; e < 4; ++e) num[e] *= r;
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const float f = exp2_fast(ml[u].x - base);
        den = fmaf(f, ml[u].y, den);
        num[0] = fmaf(f, a[u].x, num[0]);
        num[1] = fmaf(f, a[u].y, num[1]);
        num[2] = fmaf(f, a[u].z, num[2]);
        num[3] = fmaf(f, a[u].w, num[3]);
      }
      M = Mb;
    }
    *reinterpret_cast<uint2*>(out + (row0 + h) * D + d) =
        make_uint2(pack2<T>(num[0] / den, num[1] / den), pack2<T>(num[2] / den, num[3] / den));
  }
}

template <typename T, int D, int G>
static hipError_t launch_prefix_merge_t(const PrefixArgs& a) {
  hipLaunchKernelGGL((pa_prefix_merge<T, D, G>), dim3((uint32_t)a.num_seqs * a.num_kv_heads),
                     dim3(256), 0, a.stream, (uint16_t*)a.out, a.ws_acc, a.ws_ml, a.ws_meta,
                     a.pair_acc, a.pair_ml, a.pre_acc, a.pre_ml, a.seq_lens, a.block_tables,
                     a.num_seqs, a.num_kv_heads, a.max_blocks_per_seq,
                     a.max_blocks_per_seq * a.block_size, a.prefix_blocks * a.block_size,
                     a.prefix_blocks, (int32_t)prefix_chunks(a.prefix_blocks, a.block_size));
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_prefix_merge_d(const PrefixArgs& a) {
  switch (a.group) {
    case 1: return launch_prefix_merge_t<T, D, 1>(a);
    case 2: return launch_prefix_merge_t<T, D, 2>(a);
    case 4: return launch_prefix_merge_t<T, D, 4>(a);
    case 8: return launch_prefix_merge_t<T, D, 8>(a);
  }
  return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------

// Waves of one decode launch on the current device: per_cu_max (1 or
// kWorkgroupsPerCu) workgroups per CU, or fewer if fewer fit;
// kErrDoesNotFit if not one workgroup fits a CU or its LDS exceeds the
// device's per-workgroup limit (cached per instantiation, device and
// per_cu_max; recomputing gives the same answer, so concurrent first calls
// are harmless).
template <typename T, typename KV, int D, int BS, int G, bool kDeep = false, bool kNt = true>
static hipError_t launch_waves(int* waves, int per_cu_max) {
  if (per_cu_max < 1 || per_cu_max > kWorkgroupsPerCu) return hipErrorInvalidValue;
  static int cache[kMaxDevices][kWorkgroupsPerCu + 1];  // > 0 waves, -1 does not fit, 0 unknown
  static int lds_cache[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  const int cached = __atomic_load_n(&cache[dev][per_cu_max], __ATOMIC_RELAXED);
  if (cached != 0) {
    *waves = cached;
    return cached > 0 ? hipSuccess : kErrDoesNotFit;
  }
  auto kernel = pa_decode_streamk<T, D, BS, G, false, KV, kDeep, kNt>;
  e = check_lds((const void*)kernel, 0, lds_cache);
  if (e != hipSuccess && e != kErrDoesNotFit) return e;
  int cus = 0, per_cu = 0;
  if (e == hipSuccess) {
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kThreads, 0);
    if (e != hipSuccess) return e;
  }
  const int n = (per_cu > 0 && cus > 0) ? cus * min(per_cu, per_cu_max) * kWaves : -1;
  __atomic_store_n(&cache[dev][per_cu_max], n, __ATOMIC_RELAXED);
  *waves = n;
  return n > 0 ? hipSuccess : kErrDoesNotFit;
}

template <typename T, typename KV, int D, int BS, int G, bool kDeep, bool kNt = true>
static hipError_t launch_k(const StreamKArgs& a, bool gather, int per_cu_max) {
  using Elem = typename TileWaveOf<T, KV, D, BS, G>::type::Elem;
  int waves = 0;
  hipError_t e = launch_waves<T, KV, D, BS, G, kDeep, kNt>(&waves, per_cu_max);
  if (e != hipSuccess) return e;
  // no more waves than the workspace holds partial slots for, a whole
  // number per KV head, at least one
  const int cap = gather ? kStreamKMaxWaves : min(a.max_waves, kStreamKMaxWaves);
  if (a.num_kv_heads > cap) return hipErrorInvalidValue;
  waves = max(min(waves, cap) / a.num_kv_heads, 1) * a.num_kv_heads;
  if constexpr (!std::is_same<KV, Vec>::value) {  // the gather probe reads as the matrix-core wave
    if (gather) {  // the same grid, gather-only (the group does not change the loads)
      static int lds_cache[kMaxDevices];
      auto kernel = pa_decode_streamk<T, D, BS, 1, true, KV, kDeep, kNt>;
      e = check_lds((const void*)kernel, 0, lds_cache);
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL(kernel, dim3((uint32_t)((waves + kWaves - 1) / kWaves)),
                         dim3(kThreads), 0, a.stream, (uint16_t*)a.out, nullptr, nullptr,
                         nullptr, nullptr, (const Elem*)a.k_cache, (const Elem*)a.v_cache,
                         a.block_tables, a.seq_lens, a.num_seqs, a.num_kv_heads,
                         a.max_blocks_per_seq, a.num_blocks, waves, 0, 0.0f, 0.0f, 0, nullptr,
                         nullptr);
      return hipGetLastError();
    }
  } else {
    if (gather) return hipErrorInvalidValue;
  }
  hipLaunchKernelGGL((pa_decode_streamk<T, D, BS, G, false, KV, kDeep, kNt>),
                     dim3((uint32_t)((waves + kWaves - 1) / kWaves)),
                     dim3(kThreads), 0, a.stream, (uint16_t*)a.out, a.ws_acc, a.ws_ml, a.ws_meta,
                     (const uint16_t*)a.q, (const Elem*)a.k_cache, (const Elem*)a.v_cache,
                     a.block_tables, a.seq_lens, a.num_seqs, a.num_kv_heads,
                     a.max_blocks_per_seq, a.num_blocks, waves, a.part_tiles, a.qk_scale,
                     a.out_scale, a.start, a.pair_acc, a.pair_ml);
  e = hipGetLastError();
  if (e != hipSuccess || !a.merge) return e;
  const int64_t pairs = (int64_t)a.num_seqs * a.num_kv_heads;
  if (pairs >= kManyPairs)
    hipLaunchKernelGGL((pa_streamk_reduce<T, D, G, 64>), dim3((uint32_t)((pairs + 3) / 4)),
                       dim3(256), 0, a.stream, (uint16_t*)a.out, a.ws_acc, a.ws_ml, a.ws_meta,
                       a.seq_lens, (int32_t)pairs, a.num_kv_heads,
                       a.max_blocks_per_seq * a.block_size);
  else
    hipLaunchKernelGGL((pa_streamk_reduce<T, D, G, 256>), dim3((uint32_t)pairs), dim3(256), 0,
                       a.stream, (uint16_t*)a.out, a.ws_acc, a.ws_ml, a.ws_meta, a.seq_lens,
                       (int32_t)pairs, a.num_kv_heads, a.max_blocks_per_seq * a.block_size);
  return hipGetLastError();
}

// The 16-bit matrix-core tile wave always keeps two tiles in flight
// (kDeep).  On batches of few, long sequences, where every wave's run is
// long and the launch is bound by the gather (at most kDeepMaxPairs
// (sequence, KV head) pairs, tables of at least kDeepMinLen positions), the
// launch puts one workgroup on each CU; measured against two workgroups of
// one tile in flight each: the 256-sequence mixed step 344.5 -> 339.4 us,
// the 32-sequence long context 391.6 -> 384.0 us.  Other batches get two
// workgroups per CU: with one, 4,096 sequences of 16-64 positions took 245
// us and 8,192 of 1-8 positions 339 us, against 220 and 256 us with two
// (225 and 258 us with two of one tile in flight each).  The shared-prefix
// tails (start > 0) are short too.  The 8-bit and vector tile waves keep
// one tile in flight, two workgroups per CU.
constexpr int64_t kDeepMaxPairs = 4096;
constexpr int64_t kDeepMinLen = 1024;

// The streaming hint lets the caches drop each K/V line once it is read:
// right when the batch's K/V is far larger than the last-level cache (256
// MiB on MI355X), as on the mixed step (without it 340 -> 384 us) and the
// long context (384 -> 437 us).  When all the K/V a call can read fits in
// that cache -- the smaller of the pool and the tables' capacity -- the
// lines stay there across calls and across the sequences that share them:
// without the hint the 64 sequences on one 2048-position prefix decode in
// 64.6 instead of 82.5 us (their 81 MB of distinct K/V is read 7.5 times),
// the pages' worked example (64 MB of tables) in 24.1 instead of 25.4 us.
constexpr int64_t kCacheResidentBytes = int64_t(256) << 20;

template <typename T, typename KV, int D, int BS, int G>
static hipError_t launch_t(const StreamKArgs& a, bool gather) {
  if constexpr (std::is_same<KV, T>::value) {
    const int64_t pairs = (int64_t)a.num_seqs * a.num_kv_heads;
    const int64_t max_len = (int64_t)a.max_blocks_per_seq * a.block_size;
    const bool few_long = a.start == 0 && pairs <= kDeepMaxPairs && max_len >= kDeepMinLen;
    const int per_cu = few_long ? 1 : kWorkgroupsPerCu;
    const int64_t block_bytes = (int64_t)2 * a.num_kv_heads * BS * D * sizeof(uint16_t);  // K + V
    const int64_t reach = min((int64_t)a.num_blocks, (int64_t)a.num_seqs * a.max_blocks_per_seq);
    if (reach * block_bytes <= kCacheResidentBytes)
      return launch_k<T, KV, D, BS, G, true, false>(a, gather, per_cu);
    return launch_k<T, KV, D, BS, G, true, true>(a, gather, per_cu);
  } else {
    return launch_k<T, KV, D, BS, G, false>(a, gather, kWorkgroupsPerCu);
  }
}

template <typename T, typename KV, int D, int BS>
static hipError_t launch_g(const StreamKArgs& a, bool gather) {
  switch (a.group) {
    case 1: return launch_t<T, KV, D, BS, 1>(a, gather);
    case 2: return launch_t<T, KV, D, BS, 2>(a, gather);
    case 4: return launch_t<T, KV, D, BS, 4>(a, gather);
    case 8: return launch_t<T, KV, D, BS, 8>(a, gather);
  }
  return hipErrorInvalidValue;
}

template <typename T, typename KV, int D>
static hipError_t launch_bs(const StreamKArgs& a, bool gather) {
  switch (a.block_size) {
    case 8: return launch_g<T, KV, D, 8>(a, gather);
    case 16: return launch_g<T, KV, D, 16>(a, gather);
    case 32: return launch_g<T, KV, D, 32>(a, gather);
  }
  return hipErrorInvalidValue;
}

template <typename T, typename KV>
static hipError_t launch_d(const StreamKArgs& a, bool gather) {
  switch (a.head_dim) {
    case 64: return launch_bs<T, KV, 64>(a, gather);
    case 128: return launch_bs<T, KV, 128>(a, gather);
  }
  return hipErrorInvalidValue;
}

}  // namespace pa
