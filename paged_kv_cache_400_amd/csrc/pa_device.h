// pa_device.h -- device helpers shared by the libpa kernels (gfx950).
//
// Element formats: IEEE binary16 and bfloat16, stored as raw 16-bit words;
// two neighbouring elements share one 32-bit register word (element 2k in
// the low half, 2k+1 in the high half).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

struct F16 {};
struct BF16 {};

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf162_t __attribute__((ext_vector_type(2)));

constexpr float kNegInf = -__builtin_inff();
constexpr float kLog2e = 1.4426950408889634f;

// ---- widening of packed pairs -------------------------------------------
template <typename T> __device__ __forceinline__ float lo_f32(uint32_t w);
template <typename T> __device__ __forceinline__ float hi_f32(uint32_t w);

template <> __device__ __forceinline__ float lo_f32<BF16>(uint32_t w) {
  return __uint_as_float(w << 16);
}
template <> __device__ __forceinline__ float hi_f32<BF16>(uint32_t w) {
  return __uint_as_float(w & 0xffff0000u);
}
template <> __device__ __forceinline__ float lo_f32<F16>(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
}
template <> __device__ __forceinline__ float hi_f32<F16>(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

// ---- a.lo*b.lo + a.hi*b.hi + c, float32 accumulate (v_dot2_f32_*) -------
template <typename T> __device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c);

template <> __device__ __forceinline__ float dot2<F16>(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a), __builtin_bit_cast(half2_t, b), c,
                                false);
}
template <> __device__ __forceinline__ float dot2<BF16>(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, a),
                                         __builtin_bit_cast(bf162_t, b), c, false);
}

// ---- float -> 16-bit word, round to nearest even -----------------------
template <typename T> __device__ __forceinline__ uint16_t to_bits(float x);

template <> __device__ __forceinline__ uint16_t to_bits<F16>(float x) {
  return __builtin_bit_cast(uint16_t, (_Float16)x);  // v_cvt_f16_f32, RNE
}
template <> __device__ __forceinline__ uint16_t to_bits<BF16>(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);  // quiet NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// ---- streaming loads ------------------------------------------------------
// Every K/V byte is read exactly once per call, so the loads carry the
// non-temporal hint: they stream through the caches instead of displacing
// the small, soon-reused data (the split-K partials the same launch writes,
// the block tables, q).  Without it, the partials' write-back interleaves
// with the K/V read stream at the memory controllers, which cost the mixed
// decode step about 3% of its bandwidth.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_stream(const void* p) {
  return __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p)));
}
// The same load without the hint when kNt is false.
template <bool kNt>
__device__ __forceinline__ uint4 load_kv(const void* p) {
  if constexpr (kNt)
    return load_stream(p);
  else
    return *reinterpret_cast<const uint4*>(p);
}
// Cache-policy operand of the copies into LDS (global_load_lds, buffer_load
// ... lds) for the same hint (the nt bit), and the default policy for data
// that other workgroups read again soon (prefill's K/V tiles).
constexpr int kCachePolicyStream = 2;
constexpr int kCachePolicyReuse = 0;

// A buffer resource for `bytes` bytes at p (raw: no stride, no format; a
// load past the range reads 0; the last word is the gfx9 resource format).
// Copies into LDS issued as buffer loads (buffer_load_dwordx4 ... lds) are
// counted by the compiler among the wave's vector-memory operations like any
// load.  A pending global_load_lds instead makes it wait for every
// outstanding load (vmcnt(0)) before any use of a register another load
// filled, which a driver that keeps several tiles in flight cannot afford.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* p, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, bytes, 0x00020000);
}
// 16 bytes per lane from the resource at byte voffset into LDS at lds +
// 16 * lane (the copy's destination is per instruction, not per lane).
template <int kPolicy = kCachePolicyStream>
__device__ __forceinline__ void copy_to_lds16(__amdgpu_buffer_rsrc_t r, uint32_t voffset,
                                              void* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16,
                                           voffset, 0, 0, kPolicy);
}

// ---- 2^x on the transcendental unit (v_exp_f32; 2^-inf = 0) -------------
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// ---- DPP lane exchange within 16-lane rows -----------------------------
template <int CTRL> __device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
constexpr int kQuadXor1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;
constexpr int kRowMirror = 0x140;

// Sum over groups of N consecutive lanes (N = 8 or 16); every lane of a
// group ends with the same bits (each exchange adds a pair in both lanes).
template <int N> __device__ __forceinline__ float group_sum(float x) {
  static_assert(N == 8 || N == 16, "group of 8 or 16 lanes");
  x += dpp<kQuadXor1>(x);
  x += dpp<kQuadXor2>(x);
  x += dpp<kRowHalfMirror>(x);
  if constexpr (N == 16) x += dpp<kRowMirror>(x);
  return x;
}


// ---- work-unit order ------------------------------------------------------
// A decode launch has one workgroup per unit (sequence s, KV head kh,
// partition p), num_seqs * hkv * pmax in all; units with p past a sequence's
// last partition exit at once.  The hardware deals workgroup i to XCD i % 8,
// and each XCD has its own L2 and dispatcher, so the order decides how the
// work is split between XCDs.  Units are numbered partition-major:
//   i = (pmax - 1 - p) * (num_seqs * hkv) + s * hkv + kh,
// so consecutive workgroups walk the sequences and heads of one partition
// index, each XCD gets every sequence in equal measure (with hkv = 8, XCD x
// gets KV head x of every sequence), and the sparse high partition indices,
// which only long sequences have, come first instead of leaving the chip
// half idle at the end.  (Numbering (s, kh, p) with p fastest sent every
// first partition to XCD 0 and every eighth to XCD 7.)
struct Unit {
  int s, kh, p;
};
__device__ __forceinline__ Unit unit_of(int i, int hkv, int pmax) {
  const int per_part = (int)(gridDim.x / (unsigned)pmax);  // num_seqs * hkv
  const int rest = i % per_part;
  return Unit{rest / hkv, rest % hkv, pmax - 1 - i / per_part};
}

}  // namespace pa
