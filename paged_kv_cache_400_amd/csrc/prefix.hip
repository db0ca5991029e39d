// prefix.hip -- the shared prefix of pa_decode_shared_prefix, attended once
// for every sequence that shares it.
//
// The pages name prefix sharing (a system prompt, the candidates of a beam
// search) as the case where several sequences hold the same physical blocks
// ("What problem does PagedAttention solve, and what is continuous
// batching?", section "How PagedAttention works"; "PagedAttention &
// Continuous Batching", section "Production defaults": prefix caching).
// Decoded one sequence at a time, those blocks are read once per sequence.
// Here the query rows of all sequences are stacked instead: for KV head kh,
// the rows (s, h) with h in kh's group, 16 to a row block (16 / G sequences
// x G heads), attend the prefix's positions as one product of 16 rows per
// MFMA, the matrix-core tile wave of the decode (pa_mfma.h) with its 16 MFMA
// columns holding 16 rows instead of at most 8 heads.
//
// Work: a workgroup takes one (KV head kh, chunk c of kPrefixChunk
// positions) pair and four row blocks, one per wave.  The four waves share
// each tile of the chunk: every wave copies a quarter of it (K and V) from
// memory straight into LDS, a barrier makes the whole tile visible, and each
// wave computes its 16 rows from LDS.  kStages tiles are in LDS at once, so
// the copies of the next kStages - 1 tiles are in flight while a tile is
// computed.
// The workgroups of one (head, chunk) pair run on one XCD (workgroups are
// dealt to the 8 XCDs in turn), so each prefix block is fetched into one L2
// and served from there to all the row blocks.  Each row's partial state (m,
// l, acc: base-2 running max, sum of weights, weighted sum of V) is left for
// the merge with the row's tail.  The block ids come from sequence 0's
// table; the merge checks that every other sequence's table starts with the
// same ids.
#include <type_traits>
#include <utility>

#include "pa_launch.h"
#include "pa_mfma.h"

namespace pa {

namespace {

constexpr int kWaves = 4;                       // row blocks per workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kRows = 16;                       // rows per row block: the MFMA's columns
constexpr int kStages = 4;                      // tiles held in LDS at once
constexpr int kChunkTiles = kPrefixChunk / 16;  // tiles of one chunk
constexpr int kXcds = 8;                        // MI355X: workgroups dealt to 8 XCDs in turn

// LDS of one workgroup: kStages V tiles (the tile wave's layout), then
// kStages K tiles, each K tile KC blocks of 1 KiB holding, at byte 16 l,
// the 16 bytes lane l feeds the q.K^T MFMA at that step (position l % 16,
// elements 32 c + 8 (l / 16) .. + 7): a wave reads its operand back
// linearly.  After the walk the same bytes stage the four waves' results.
template <int D>
struct PrefixLds {
  using GE = Geo<D>;
  static constexpr int KTILE = GE::KC * 1024;
  static constexpr int V0 = 0;
  static constexpr int K0 = kStages * GE::TILE;
  static constexpr int TILES = K0 + kStages * KTILE;
  static constexpr int RESULT = kWaves * kRows * D * 4;
  static constexpr int BYTES = TILES > RESULT ? TILES : RESULT;
  static constexpr int JOBS = GE::KC + 4;       // copies per tile: K blocks, then V regions
};

// f(integral_constant<int, j>) for j = 0 .. N-1, in order, at compile time.
template <int N, typename F, int... J>
__device__ __forceinline__ void unroll_impl(F&& f, std::integer_sequence<int, J...>) {
  (f(std::integral_constant<int, J>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void unroll(F&& f) {
  unroll_impl<N>(f, std::make_integer_sequence<int, N>{});
}

// Wait until this wave's copies of the tiles issued after tile j are all
// that remain in flight (`after` such tiles).  Wave w issues the copies
// w, w + 4, ... of each tile's kJobs, so waves below kJobs % 4 issue one
// more than the others.
template <int kJobs, int kAfter>
__device__ __forceinline__ void wait_own_tiles(int w) {
  constexpr int hi = (kJobs + 3) / 4, lo = kJobs / 4;
  if (kJobs % 4 == 0 || w < kJobs % 4)
    wait_vmem_but<hi * kAfter>();
  else
    wait_vmem_but<lo * kAfter>();
}

// The KC 16-byte K operands of this lane from a K tile in LDS, read as one
// asm block that waits for its own results (the reason is read_v_tr_twice's).
template <int KC>
__device__ __forceinline__ void read_k(uint4 (&kr)[KC], uint32_t a) {
  static_assert(KC == 2 || KC == 4, "head_dim 64 or 128");
  if constexpr (KC == 4) {
    asm volatile(
        "ds_read_b128 %0, %4\n\t"
        "ds_read_b128 %1, %4 offset:1024\n\t"
        "ds_read_b128 %2, %4 offset:2048\n\t"
        "ds_read_b128 %3, %4 offset:3072\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(kr[0]), "=&v"(kr[1]), "=&v"(kr[2]), "=&v"(kr[3])
        : "v"(a)
        : "memory");
  } else {
    asm volatile(
        "ds_read_b128 %0, %2\n\t"
        "ds_read_b128 %1, %2 offset:1024\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(kr[0]), "=&v"(kr[1])
        : "v"(a)
        : "memory");
  }
}

template <typename T, int D, int BS, int G>
__global__ void __launch_bounds__(kThreads)
pa_prefix_attend(float* __restrict__ pre_acc, float2* __restrict__ pre_ml,
                 const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
                 const uint16_t* __restrict__ vc, const int32_t* __restrict__ block_tables,
                 int32_t num_seqs, int32_t hkv, int32_t nb, int32_t prefix_len, int32_t nrb,
                 int32_t nchunks, float qk_scale) {
  using TW = TileWave<T, D, BS, kRows>;
  using L = PrefixLds<D>;
  using GE = Geo<D>;
  constexpr int KC = TW::KC, kT = TW::kTileLen;
  static_assert(kRows % G == 0, "whole sequences per row block");
  static_assert(kPrefixChunk % 64 == 0 && kPrefixChunk / 8 <= 64, "a chunk's ids fit one wave");
  static_assert(kT == 16 && kChunkTiles >= kStages, "16-position tiles, at least kStages a chunk");
  static_assert(L::JOBS <= 2 * kWaves, "at most two copies per wave and tile");
  __shared__ __attribute__((aligned(16))) unsigned char s_mem[L::BYTES];
  static_assert(sizeof(s_mem) <= kMaxLdsBytes, "one workgroup's LDS fits gfx950's 160 KiB");

  // workgroup -> (pair p = (kh, c), row quad r): the pairs with p % 8 == x
  // go to XCD x, all row quads of a pair one after the other
  const int nquads = (nrb + kWaves - 1) / kWaves;
  const int xcd = blockIdx.x % kXcds, slot = blockIdx.x / kXcds;
  const int p = (slot / nquads) * kXcds + xcd;
  if (p >= hkv * nchunks) return;  // the whole workgroup
  const int kh = p % hkv, c = p / hkv;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rb = (slot % nquads) * kWaves + w;  // rb >= nrb: copies only, no rows
  const int hq = hkv * G;
  const int p_lo = c * kPrefixChunk;
  const int p_end = min(prefix_len, p_lo + kPrefixChunk);
  const int col = lane & 15, grp = lane >> 4;
  // MFMA column r is row (s_r, h_r): sequence rb * 16 / G + r / G, query head
  // kh * G + r % G; columns past the last sequence compute on zero queries
  auto seq_of = [&](int r) { return rb * (kRows / G) + r / G; };
  auto head_of = [&](int r) { return kh * G + r % G; };

  TW tw;
  tw.init(kc, vc, hkv, kh, s_mem + L::V0);
  {
    const int s = seq_of(col);
#pragma unroll
    for (int k = 0; k < KC; ++k) {
      tw.qr.r[k] = make_uint4(0u, 0u, 0u, 0u);
      if (s < num_seqs)
        tw.qr.r[k] = *reinterpret_cast<const uint4*>(
            q + ((int64_t)s * hq + head_of(col)) * D + (k * 4 + grp) * 8);
    }
  }
  tw.reset();

  // the chunk's block ids, one per lane (at most kPrefixChunk / 8 blocks)
  const int blk_base = p_lo / BS, blk_last = (p_end - 1) / BS;
  bool bad = false;
  int vid = 0;
  if (blk_base + lane <= blk_last) {
    vid = block_tables[blk_base + lane];
    if (vid < 0 || vid >= nb) {
      bad = true;  // never dereferenced: block 0 is read, the rows become NaN
      vid = 0;
    }
  }
  bad = __builtin_amdgcn_ballot_w64(bad) != 0;
  wait_vmem_all();  // q and the ids, before the first copies

  const int64_t blk_stride = (int64_t)hkv * BS * D, head_off = (int64_t)kh * BS * D;
  const uint32_t lds0 = (uint32_t)(uintptr_t)s_mem;
  // This wave's copies of tile j into stage j % kStages.  A position past
  // the chunk's end (in a prefix's last, partial chunk) re-reads the last
  // valid one; its scores are masked.
  auto issue = [&](int j) {
    const int t0 = p_lo + j * kT, t_last = p_end - 1;
    const int st = j % kStages;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int jb = w + kWaves * u;
      if (jb >= L::JOBS) break;
      int t, chunk8;  // position and 8-element chunk this lane copies
      unsigned char* dst;
      if (jb < KC) {  // K block jb: position col, elements 32 jb + 8 grp ..
        t = min(t0 + col, t_last);
        chunk8 = jb * 4 + grp;
        dst = s_mem + L::K0 + st * L::KTILE + jb * 1024;
      } else {  // V region i: rows 4i .., as the tile wave lays them out
        const int i = jb - KC;
        t = min(t0 + 4 * i + lane / (D / 8), t_last);
        chunk8 = lane % (D / 8);
        dst = s_mem + L::V0 + st * GE::TILE + i * GE::REGION;
      }
      const int id = __builtin_amdgcn_ds_bpermute(4 * (t / BS - blk_base), vid);
      const uint16_t* src = (jb < KC ? kc : vc) + (int64_t)id * blk_stride + head_off +
                            ((uint32_t)t % BS) * D + chunk8 * 8;
      // the default cache policy: the (head, chunk)'s other workgroups copy
      // the same tile from this L2 (43.5-43.9 against 44.1-44.2 us per call
      // with the streaming hint)
      if (jb < KC || GE::LANES == 64 || lane < GE::LANES)
        __builtin_amdgcn_global_load_lds((const void*)src,
                                         (void __attribute__((address_space(3)))*)dst, 16, 0,
                                         kCachePolicyReuse);
    }
  };

#pragma unroll
  for (int j = 0; j < kStages - 1; ++j) issue(j);
  unroll<kChunkTiles>([&](auto jc) {
    constexpr int j = decltype(jc)::value;
    // this wave's copies of tile j have landed; after the barrier, every
    // wave's have, and every wave is done with tile j - 1, whose stage the
    // copies of tile j + kStages - 1 then overwrite
    constexpr int kAfter = kStages - 2 < kChunkTiles - 1 - j ? kStages - 2 : kChunkTiles - 1 - j;
    wait_own_tiles<L::JOBS, kAfter>(w);
    __builtin_amdgcn_s_barrier();
    if constexpr (j + kStages - 1 < kChunkTiles) issue(j + kStages - 1);
    uint4 kr[KC];
    read_k<KC>(kr, lds0 + L::K0 + (j % kStages) * L::KTILE + 16 * lane);
    tw.template consume<false>(kr, j % kStages, p_lo + j * kT, p_end, qk_scale);
  });
  tw.finish();

  // the rows' partial states: acc staged row-major in LDS (after a barrier:
  // the other waves may still read the last tiles), then stored 16 bytes
  // per lane; (m, l) by the lane of each column
  wait_vmem_all();
  __builtin_amdgcn_s_barrier();
  float* st = reinterpret_cast<float*>(s_mem) + w * kRows * D;  // [16][D]
  tw.stage(st, false, bad, 1.0f);
  if (rb >= nrb) return;
  const int64_t chunk_row0 = (int64_t)c * num_seqs * hq;
  for (int i = lane * 4; i < kRows * D; i += 64 * 4) {
    const int r = i / D;
    if (seq_of(r) < num_seqs)
      *reinterpret_cast<float4*>(
          pre_acc + (chunk_row0 + (int64_t)seq_of(r) * hq + head_of(r)) * D + i % D) =
          *reinterpret_cast<const float4*>(st + i);
  }
  const float2 ml = tw.ml_of_lane();
  if (lane < kRows && seq_of(lane) < num_seqs)
    pre_ml[chunk_row0 + (int64_t)seq_of(lane) * hq + head_of(lane)] =
        make_float2(ml.x, bad ? __builtin_nanf("") : ml.y);
}

template <typename T, int D, int BS, int G>
hipError_t launch_t(const PrefixArgs& a) {
  static int lds_cache[kMaxDevices];
  const hipError_t fit = check_lds((const void*)pa_prefix_attend<T, D, BS, G>, 0, lds_cache);
  if (fit != hipSuccess) return fit;
  const int64_t nrb = ((int64_t)a.num_seqs * G + kRows - 1) / kRows;
  const int64_t nquads = (nrb + kWaves - 1) / kWaves;
  const int64_t nchunks = prefix_chunks(a.prefix_blocks, a.block_size);
  const int64_t pairs = (int64_t)a.num_kv_heads * nchunks;
  const int64_t groups = ((pairs + kXcds - 1) / kXcds) * kXcds * nquads;
  hipLaunchKernelGGL((pa_prefix_attend<T, D, BS, G>), dim3((uint32_t)groups), dim3(kThreads), 0,
                     a.stream, a.pre_acc, a.pre_ml, (const uint16_t*)a.q,
                     (const uint16_t*)a.k_cache, (const uint16_t*)a.v_cache, a.block_tables,
                     a.num_seqs, a.num_kv_heads, a.num_blocks, a.prefix_blocks * a.block_size,
                     (int32_t)nrb, (int32_t)nchunks, a.qk_scale);
  return hipGetLastError();
}

template <typename T, int D, int BS>
hipError_t launch_g(const PrefixArgs& a) {
  switch (a.group) {
    case 1: return launch_t<T, D, BS, 1>(a);
    case 2: return launch_t<T, D, BS, 2>(a);
    case 4: return launch_t<T, D, BS, 4>(a);
    case 8: return launch_t<T, D, BS, 8>(a);
  }
  return hipErrorInvalidValue;
}

template <typename T, int D>
hipError_t launch_bs(const PrefixArgs& a) {
  switch (a.block_size) {
    case 8: return launch_g<T, D, 8>(a);
    case 16: return launch_g<T, D, 16>(a);
    case 32: return launch_g<T, D, 32>(a);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_prefix_attend(const PrefixArgs& a) {
  if (a.head_dim == 64) return a.bf16 ? launch_bs<BF16, 64>(a) : launch_bs<F16, 64>(a);
  return a.bf16 ? launch_bs<BF16, 128>(a) : launch_bs<F16, 128>(a);
}

}  // namespace pa
