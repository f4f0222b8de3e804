// int8 sketches of key and query rows for the reduced-byte indexer.
//
// A row x of D bf16 values becomes D int8 codes and one float32 scale:
//   m = max_i |x_i|,  scale = m / 127,  c_i = rint(x_i / scale)  (clamped to [-127, 127]),
// both divisions correctly rounded in float32 and rint rounding half to even; a zero row has
// scale 0 and codes 0.  The sketch score of a query row against a key row is then
// (scale_q * scale_k) * (c_q . c_k) with an exact integer dot product, so every step of it is
// reproducible bit for bit.  The indexer ranks candidates by this score and re-ranks them by the
// exact one; the pages count such an indexer's cost against the sparse kernel's gain (technical
// summary, section 3.C, indexing-overhead bullet).
#include "launch.h"

namespace cs {

constexpr int kSketchThreads = 256;

// Quantises one row held by D / 8 consecutive lanes, 8 values per lane (raw: their bf16 bits).
// Returns this lane's 8 codes packed little-endian in two words; `scale` gets the row's scale.
// Every lane of the row group must be active.
template <int D>
__device__ __forceinline__ uint2 quantize8(const uint4& raw, float& scale) {
  float x[8];
  unpack8(raw, x);
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(x[i]));
  m = group_max<D / 8>(m);
  scale = __fdiv_rn(m, 127.f);
  uint32_t w[2] = {0u, 0u};
  if (scale > 0.f) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float c = fminf(fmaxf(rintf(__fdiv_rn(x[i], scale)), -127.f), 127.f);
      w[i >> 2] |= ((uint32_t)(int)c & 0xffu) << (8 * (i & 3));
    }
  }
  return make_uint2(w[0], w[1]);
}

// Key rows: blockIdx.y = b * Hkv + h; rows [n0, L_b) with n0 = max(0, L_b - last_n) (0 when
// last_n <= 0), kSketchThreads / (D / 8) rows per workgroup and iteration.
template <int D, bool PAGED>
__global__ __launch_bounds__(kSketchThreads) void key_sketch_kernel(KVArgs kv, int last_n,
                                                                    int8_t* __restrict__ codes,
                                                                    float* __restrict__ scales) {
  constexpr int LPR = D / 8;
  constexpr int RPB = kSketchThreads / LPR;
  const int bh = blockIdx.y;
  const int b = bh / kv.num_kv_heads, h = bh - (bh / kv.num_kv_heads) * kv.num_kv_heads;
  const int L = seq_len_of(kv, b);
  const int n0 = last_n > 0 ? max(0, L - last_n) : 0;
  const int c = threadIdx.x % LPR;
  for (int base = n0 + blockIdx.x * RPB; base < L; base += gridDim.x * RPB) {
    const int n = base + threadIdx.x / LPR;
    const int nc = min(n, L - 1);  // whole row groups stay active for the lane reduction
    const int64_t off = kv_row<D, PAGED>(kv, b, h, nc);
    float scale;
    const uint2 w = quantize8<D>(ld16(kv.k + off + c * 8), scale);
    if (n < L) {
      *reinterpret_cast<uint2*>(codes + off + c * 8) = w;
      if (c == 0) scales[off / D] = scale;
    }
  }
}

template <int D>
__global__ __launch_bounds__(kSketchThreads) void q_sketch_kernel(const uint16_t* __restrict__ q, int rows,
                                                                  int8_t* __restrict__ codes,
                                                                  float* __restrict__ scales) {
  constexpr int LPR = D / 8;
  constexpr int RPB = kSketchThreads / LPR;
  const int c = threadIdx.x % LPR;
  const int r = blockIdx.x * RPB + threadIdx.x / LPR;
  const int rc = min(r, rows - 1);
  float scale;
  const uint2 w = quantize8<D>(ld16(q + (int64_t)rc * D + c * 8), scale);
  if (r < rows) {
    *reinterpret_cast<uint2*>(codes + (int64_t)r * D + c * 8) = w;
    if (c == 0) scales[r] = scale;
  }
}

hipError_t launch_key_sketch(const KVArgs& kv, int B, int D, int last_n, int8_t* codes, float* scales,
                             hipStream_t stream) {
  const int rpb = kSketchThreads / (D / 8);
  const int span = last_n > 0 && last_n < kv.max_len ? last_n : kv.max_len;
  int gx = (span + rpb - 1) / rpb;
  if (gx > 1024) gx = 1024;  // the workgroups loop over longer ranges
  const dim3 grid(gx, B * kv.num_kv_heads);
  const bool paged = kv.page_table != nullptr;
  if (D == 128) {
    if (paged)
      hipLaunchKernelGGL((key_sketch_kernel<128, true>), grid, dim3(kSketchThreads), 0, stream, kv, last_n, codes, scales);
    else
      hipLaunchKernelGGL((key_sketch_kernel<128, false>), grid, dim3(kSketchThreads), 0, stream, kv, last_n, codes, scales);
  } else {
    if (paged)
      hipLaunchKernelGGL((key_sketch_kernel<64, true>), grid, dim3(kSketchThreads), 0, stream, kv, last_n, codes, scales);
    else
      hipLaunchKernelGGL((key_sketch_kernel<64, false>), grid, dim3(kSketchThreads), 0, stream, kv, last_n, codes, scales);
  }
  return hipGetLastError();
}

hipError_t launch_q_sketch(const uint16_t* q, int rows, int D, int8_t* codes, float* scales,
                           hipStream_t stream) {
  const int rpb = kSketchThreads / (D / 8);
  const dim3 grid((rows + rpb - 1) / rpb);
  if (D == 128)
    hipLaunchKernelGGL(q_sketch_kernel<128>, grid, dim3(kSketchThreads), 0, stream, q, rows, codes, scales);
  else
    hipLaunchKernelGGL(q_sketch_kernel<64>, grid, dim3(kSketchThreads), 0, stream, q, rows, codes, scales);
  return hipGetLastError();
}

}  // namespace cs
