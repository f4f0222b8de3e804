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
typedef int i32x4 __attribute__((ext_vector_type(4)));

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

// Sum over aligned groups of N lanes (N = 4, 8 or 16); every lane of the group gets the total.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(N == 4 || N == 8 || N == 16, "group size");
  v += dpp<0xB1>(v);
  v += dpp<0x4E>(v);
  if constexpr (N >= 8) v += dpp<0x141>(v);
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

// Sum of v over the wave, in every lane (row sums by DPP, then the four rows by readlane).
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xf, 0xf, false);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xf, 0xf, false);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xf, 0xf, false);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xf, 0xf, false);
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 0) + (uint32_t)__builtin_amdgcn_readlane((int)v, 16) +
         (uint32_t)__builtin_amdgcn_readlane((int)v, 32) + (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
}

// Minimum and maximum of v over the wave, in every lane (the same row permutations as
// wave_sum_u32, then the four rows by readlane).
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xf, 0xf, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xf, 0xf, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xf, 0xf, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xf, 0xf, false));
  return min(min((uint32_t)__builtin_amdgcn_readlane((int)v, 0), (uint32_t)__builtin_amdgcn_readlane((int)v, 16)),
             min((uint32_t)__builtin_amdgcn_readlane((int)v, 32), (uint32_t)__builtin_amdgcn_readlane((int)v, 48)));
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xf, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xf, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xf, 0xf, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xf, 0xf, false));
  return max(max((uint32_t)__builtin_amdgcn_readlane((int)v, 0), (uint32_t)__builtin_amdgcn_readlane((int)v, 16)),
             max((uint32_t)__builtin_amdgcn_readlane((int)v, 32), (uint32_t)__builtin_amdgcn_readlane((int)v, 48)));
}

// Inclusive prefix sum over the wave's lanes: shifts by 1, 2, 4, 8 within each row of 16 lanes
// (lanes shifted in from outside the row add 0), then row 0's total into row 1 and row 2's into
// row 3 (row_bcast:15), then lane 31's running total into rows 2 and 3 (row_bcast:31).
__device__ __forceinline__ uint32_t wave_incl_scan_u32(uint32_t x) {
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xf, 0xf, false);
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xf, 0xf, false);
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xf, 0xf, false);
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xf, 0xf, false);
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xa, 0xf, false);
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xc, 0xf, false);
  return x;
}

// Orders this wave's LDS accesses before and after the call (same-wave producer/consumer).
__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Workgroup barrier that orders LDS accesses only: global loads in flight stay in flight across
// it (a full __syncthreads waits for them).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// a.lo * b.lo + a.hi * b.hi + c for two packed bf16 pairs (v_dot2_f32_bf16; the bf16 products
// are exact in float32).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c,
                                         false);
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

// Inverse of ord_key: the float whose key is k.
__device__ __forceinline__ float key_to_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
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

// The same value held in a vector register, for kernels that need it only after their first
// vector loads: a scalar load shares the scalar counter with the kernel-argument loads, whose
// out-of-order returns make every wait on that counter wait for all of them, so the first
// vector loads would queue behind this cold read; as a vector load nothing waits for it until
// its first use.
__device__ __forceinline__ int seq_len_vec(const KVArgs& kv, int b) {
  const int L = __hip_atomic_load(kv.seq_lens + b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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

// Page ids of logical positions [start, end) of request b, clamped to the pool, copied into LDS
// by the whole workgroup (paged caches only; the caller synchronises before use).  Entry i holds
// the page of position ((start >> page_shift) + i) << page_shift.
__device__ __forceinline__ void stage_pages(const KVArgs& kv, int b, int start, int end,
                                            int* lds_pages) {
  const int p0 = start >> kv.page_shift;
  const int n = ((end - 1) >> kv.page_shift) - p0 + 1;
  const int32_t* pt = kv.page_table + (int64_t)b * kv.max_pages + p0;
  // 8 independent loads per thread in flight before any store
  for (int i0 = threadIdx.x; i0 < n; i0 += 8 * blockDim.x) {
    int pg[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = i0 + u * blockDim.x;
      pg[u] = i < n ? pt[i] : 0;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = i0 + u * blockDim.x;
      if (i < n) lds_pages[i] = pg[u] < 0 ? 0 : (pg[u] >= kv.num_pages ? kv.num_pages - 1 : pg[u]);
    }
  }
}

// Offset of row n0 (a wave-uniform, 16-aligned tile start inside [start, end)) using the page ids
// staged by stage_pages; contiguous caches ignore the staging.
template <int D, bool PAGED>
__device__ __forceinline__ int64_t kv_tile_staged(const KVArgs& kv, const int* lds_pages, int start,
                                                  int b, int h, int n0) {
  n0 = __builtin_amdgcn_readfirstlane(n0);
  if constexpr (!PAGED) {
    return ((int64_t)(b * kv.num_kv_heads + h) * kv.max_len + n0) * D;
  } else {
    const int page = __builtin_amdgcn_readfirstlane(
        lds_pages[(n0 >> kv.page_shift) - (start >> kv.page_shift)]);
    const int slot = n0 & ((1 << kv.page_shift) - 1);
    return ((((int64_t)page * kv.num_kv_heads + h) << kv.page_shift) + slot) * D;
  }
}

// Row (b * T + t) * Hq + hq handled by workgroup `wid` of a per-row grid of
// grouped_row_blocks() workgroups: the G * T rows of one (request, KV head) group run on one XCD
// (workgroups go to the 8 XCDs round-robin by linear id; group g takes the ids congruent to
// g mod 8), so rows of a GQA group that read the same token find its lines in that XCD's L2.
// -1 for the padding workgroups of the last groups.
__device__ __forceinline__ int grouped_row(int wid, int B, int T, int Hq, int G, int Hkv) {
  const int GT = G * T;
  const int xcd = wid & 7, j = wid >> 3;
  const int lg = j / GT, r = j - (j / GT) * GT;
  const int g = lg * 8 + xcd;
  if (g >= B * Hkv) return -1;
  const int b = g / Hkv, h = g - (g / Hkv) * Hkv;
  const int t = r / G, gi = r - (r / G) * G;
  return (b * T + t) * Hq + h * G + gi;
}
__host__ __device__ inline unsigned grouped_row_blocks(int B, int Hkv, int GT) {
  return 8u * (unsigned)((B * Hkv + 7) / 8) * (unsigned)GT;
}

// Chunk of a (request, KV head) group that the workgroup in chunk slot `slot` (blockIdx.x of a
// (chunks, groups, tiles) grid) streams: the slots of a group are rotated by the group index.
// Workgroups go to the 8 XCDs round-robin by linear id, so with the plain order chunk c of every
// group ran on XCD c mod 8 (chunk counts are mostly multiples of 8); in a ragged batch, whose
// late chunks are mostly empty, the XCDs holding late chunks idled (32 requests of 8192-131072
// positions: the indexer's K stream at 3.4 TB/s).  Rotated, XCD x gets chunk x - g (mod 8) of
// group g, the same mix of early and late chunks on every XCD, while a group's chunks are still
// dispatched together (concurrent workgroups sweep neighbouring addresses: the same chunks
// ordered group-major over the whole grid streamed 4-6% slower on full-length caches).
__device__ __forceinline__ int rotated_chunk(int slot, int group, int chunks) {
  return (int)(((unsigned)slot + (unsigned)group) % (unsigned)chunks);
}

__device__ __forceinline__ uint4 ld16(const uint16_t* p) {
  return *reinterpret_cast<const uint4*>(p);
}

}  // namespace cs
