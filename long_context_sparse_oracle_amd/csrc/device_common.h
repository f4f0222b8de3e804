// Device helpers shared by the ctxsparse kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cs {

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------- bf16 unpacking
// A bf16 is the upper half of a binary32, so widening is a shift (low half of a 32-bit word) or
// a mask (high half).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ void unpack8(const uint4& u, float (&f)[8]) {
  f[0] = bf16_lo(u.x); f[1] = bf16_hi(u.x);
  f[2] = bf16_lo(u.y); f[3] = bf16_hi(u.y);
  f[4] = bf16_lo(u.z); f[5] = bf16_hi(u.z);
  f[6] = bf16_lo(u.w); f[7] = bf16_hi(u.w);
}

// ---------------------------------------------------------------------------- DPP lane moves
// Row = 16 lanes in DPP terms.  Control codes: quad_perm [1,0,3,2] = 0xB1, [2,3,0,1] = 0x4E,
// row_half_mirror = 0x141 (lane i <-> 7-i within 8), row_mirror = 0x140 (i <-> 15-i within 16).
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}

// Sum over aligned groups of N lanes (N = 8 or 16); every lane of the group gets the total.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  v += dpp<0xB1>(v);
  v += dpp<0x4E>(v);
  v += dpp<0x141>(v);
  if constexpr (N == 16) v += dpp<0x140>(v);
  return v;
}
template <int N>
__device__ __forceinline__ float group_max(float v) {
  v = fmaxf(v, dpp<0xB1>(v));
  v = fmaxf(v, dpp<0x4E>(v));
  v = fmaxf(v, dpp<0x141>(v));
  if constexpr (N == 16) v = fmaxf(v, dpp<0x140>(v));
  return v;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// ---------------------------------------------------------------------------- ordered keys
// Order-preserving map float32 -> uint32: a > b (as floats) iff key(a) > key(b).  -0.0 is first
// folded onto +0.0 so the two zeros are an exact tie, as for the floating-point comparison.
__device__ __forceinline__ uint32_t ord_key(float s) {
  uint32_t u = __float_as_uint(s);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ---------------------------------------------------------------------------- KV addressing
struct KVArgs {
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* page_table;
  const int32_t* seq_lens;
  int32_t max_len;
  int32_t page_shift;  // log2(page_size) (paged)
  int32_t max_pages;
  int32_t num_pages;
  int32_t num_kv_heads;
};

__device__ __forceinline__ int seq_len_of(const KVArgs& kv, int b) {
  int L = kv.seq_lens[b];
  return L < 0 ? 0 : (L > kv.max_len ? kv.max_len : L);
}

// Element offset of row (b, h, n) in the K or V buffer; n must be < L_b.
template <int D, bool PAGED>
__device__ __forceinline__ int64_t kv_row(const KVArgs& kv, int b, int h, int n) {
  if constexpr (!PAGED) {
    return ((int64_t)(b * kv.num_kv_heads + h) * kv.max_len + n) * D;
  } else {
    int page = kv.page_table[(int64_t)b * kv.max_pages + (n >> kv.page_shift)];
    page = page < 0 ? 0 : (page >= kv.num_pages ? kv.num_pages - 1 : page);
    int slot = n & ((1 << kv.page_shift) - 1);
    return ((((int64_t)page * kv.num_kv_heads + h) << kv.page_shift) + slot) * D;
  }
}

// Same, for a 16-aligned tile start n0 (every position of the tile lies in one page because
// page sizes are powers of two >= 16): returns the offset of row n0; rows n0 + j follow at + j*D.
template <int D, bool PAGED>
__device__ __forceinline__ int64_t kv_tile(const KVArgs& kv, int b, int h, int n0) {
  return kv_row<D, PAGED>(kv, b, h, n0);
}

__device__ __forceinline__ uint4 ld16(const uint16_t* p) {
  return *reinterpret_cast<const uint4*>(p);
}

}  // namespace cs
