// Sparse and dense decode attention for gfx950.
//
// Sparse: softmax attention restricted to an index list per (request, token, query head); only
// the listed K/V rows are read, so a decode step moves O(k d) bytes instead of O(N d) ("Inference
// Time Context Sparsity: Illusion or Opportunity?", technical summary, section 3.C).  Each list is
// cut into splits evaluated with an online softmax and merged by log-sum-exp, the tiling with
// online softmax of the FlashSFA summary ("Scaling Attention via Feature Sparsity").
// Dense: the same with every visible position, the baseline whose linear-in-N bandwidth cost the
// pages set out to remove (section 1).
#include "device_common.h"
#include "launch.h"

namespace cs {

constexpr int kAttnThreads = 256;  // 4 waves
constexpr int kAttnWaves = kAttnThreads / kWave;

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Writes either the final (o, lse) of a row (single split) or its partial (o~, m, l).
__device__ __forceinline__ void store_result(float O, float M, float Lsum, int col, int D, int64_t row,
                                             int s, int S, float* part_o, float* part_ml,
                                             float* out, float* lse) {
  if (S == 1) {
    out[row * D + col] = Lsum > 0.f ? O / Lsum : 0.f;
    if (col == 0) lse[row] = Lsum > 0.f ? (M + fast_log2(Lsum)) * kLn2 : -INFINITY;
  } else {
    part_o[(row * S + s) * D + col] = O;
    if (col == 0) {
      part_ml[(row * S + s) * 2 + 0] = M;
      part_ml[(row * S + s) * 2 + 1] = Lsum;
    }
  }
}

// ============================================================================ sparse partial
// One workgroup per (row, split), rows of one (request, KV head) kept on one XCD: workgroup w runs
// on XCD w % 8, so group g is given the ids congruent to g mod 8 and rows of a GQA group that pick
// the same token find its K/V lines in that XCD's L2.
// Inside a wave, D/8 lanes hold one selected position (8 dims = 16 bytes of K and of V each), so
// a wave gathers 64/(D/8) whole 256-byte (D=128) rows per step, kUnroll steps in flight.
template <int D, bool PAGED>
__global__ __launch_bounds__(kAttnThreads) void sparse_partial_kernel(
    const uint16_t* __restrict__ q, KVArgs kv, const int32_t* __restrict__ indices, int T, int Hq,
    int G, int k_max, float scale_log2, int S, int chunk, int n_groups, int items_per_group,
    float* __restrict__ part_o, float* __restrict__ part_ml, float* __restrict__ out,
    float* __restrict__ lse) {
  constexpr int LPP = D / 8;        // lanes per position
  constexpr int PPW = kWave / LPP;  // positions per wave step
  constexpr int U = 4;              // steps in flight
  __shared__ float red_m[kAttnWaves * PPW];
  __shared__ float red_l[kAttnWaves * PPW];
  __shared__ float red_o[kAttnWaves * PPW][D];

  const int wid = blockIdx.x;
  const int xcd = wid & 7;
  const int j = wid >> 3;
  const int lg = j / items_per_group;
  const int within = j - lg * items_per_group;
  const int gidx = lg * 8 + xcd;
  if (gidx >= n_groups) return;
  const int r = within / S;
  const int s = within - r * S;
  const int Hkv = kv.num_kv_heads;
  const int b = gidx / Hkv, h = gidx - (gidx / Hkv) * Hkv;
  const int t = r / G, gi = r - (r / G) * G;
  const int hq = h * G + gi;
  const int64_t row = ((int64_t)b * T + t) * Hq + hq;

  const int L = seq_len_of(kv, b);
  const int vis = L - T + t + 1;
  const int lo = s * chunk;
  const int hi = min(lo + chunk, k_max);

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int p = lane / LPP;
  const int c = lane - p * LPP;

  float qf[8];
  unpack8(ld16(q + row * D + c * 8), qf);

  float m = -INFINITY, l = 0.f;
  float o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = 0.f;

  const int32_t* irow = indices + row * k_max;
  for (int e0 = lo + wave * PPW * U; e0 < hi; e0 += kAttnWaves * PPW * U) {
    int idx[U];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int e = e0 + u * PPW + p;
      idx[u] = e < hi ? irow[e] : -1;
      ok[u] = idx[u] >= 0 && idx[u] < vis;
    }
    uint4 kr[U], vr[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      kr[u] = make_uint4(0, 0, 0, 0);
      vr[u] = make_uint4(0, 0, 0, 0);
      if (ok[u]) {
        const int64_t off = kv_row<D, PAGED>(kv, b, h, idx[u]) + c * 8;
        kr[u] = ld16(kv.k + off);
        vr[u] = ld16(kv.v + off);
      }
    }
    float sv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float kf[8];
      unpack8(kr[u], kf);
      float dot = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) dot = fmaf(qf[i], kf[i], dot);
      dot = group_sum<LPP>(dot);
      sv[u] = ok[u] ? dot * scale_log2 : -INFINITY;
    }
    float mx = sv[0];
#pragma unroll
    for (int u = 1; u < U; ++u) mx = fmaxf(mx, sv[u]);
    const float m_new = fmaxf(m, mx);
    if (m_new == -INFINITY) continue;
    const float alpha = fast_exp2(m - m_new);
    l *= alpha;
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] *= alpha;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float pw = fast_exp2(sv[u] - m_new);
      l += pw;
      float vf[8];
      unpack8(vr[u], vf);
#pragma unroll
      for (int i = 0; i < 8; ++i) o[i] = fmaf(pw, vf[i], o[i]);
    }
    m = m_new;
  }

  const int slot = wave * PPW + p;
  if (c == 0) {
    red_m[slot] = m;
    red_l[slot] = l;
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) red_o[slot][c * 8 + i] = o[i];
  __syncthreads();
  if (threadIdx.x < D) {
    const int col = threadIdx.x;
    float M = -INFINITY;
    for (int k = 0; k < kAttnWaves * PPW; ++k) M = fmaxf(M, red_m[k]);
    float Lsum = 0.f, O = 0.f;
    if (M != -INFINITY) {
      for (int k = 0; k < kAttnWaves * PPW; ++k) {
        const float w = fast_exp2(red_m[k] - M);
        Lsum = fmaf(w, red_l[k], Lsum);
        O = fmaf(w, red_o[k][col], O);
      }
    }
    store_result(O, M, Lsum, col, D, row, s, S, part_o, part_ml, out, lse);
  }
}

// ============================================================================ combine
// out = sum_s e^{m_s - M} o~_s / sum_s e^{m_s - M} l_s,  lse = (M + log2 sum_s e^{m_s - M} l_s) ln 2
// with M = max_s m_s (m in log2 units).  One workgroup of D threads per row.
__global__ void combine_kernel(const float* __restrict__ part_o, const float* __restrict__ part_ml,
                               int S, int D, float* __restrict__ out, float* __restrict__ lse) {
  const int64_t row = blockIdx.x;
  const int col = threadIdx.x;
  const float* ml = part_ml + row * S * 2;
  float M = -INFINITY;
  for (int s = 0; s < S; ++s) M = fmaxf(M, ml[2 * s]);
  float Lsum = 0.f, O = 0.f;
  if (M != -INFINITY) {
    for (int s = 0; s < S; ++s) {
      const float w = fast_exp2(ml[2 * s] - M);
      Lsum = fmaf(w, ml[2 * s + 1], Lsum);
      O = fmaf(w, part_o[(row * S + s) * D + col], O);
    }
  }
  out[row * D + col] = Lsum > 0.f ? O / Lsum : 0.f;
  if (col == 0) lse[row] = Lsum > 0.f ? (M + fast_log2(Lsum)) * kLn2 : -INFINITY;
}

// ============================================================================ dense partial
// Grid: (splits, B * Hkv, ceil(G*T / 16)).  A workgroup streams one chunk of positions of one
// (request, KV head) once for up to 16 query rows: q.K^T per 16-position tile on MFMA (as in the
// indexer), online softmax per row in the MFMA output layout (rows spread over 16-lane DPP rows),
// then P.V in float32 on the vector ALUs: each lane owns D/64 output columns of every row and
// reads the tile's probabilities from a per-wave LDS buffer.
template <int D, bool PAGED, int MR>
__global__ __launch_bounds__(kAttnThreads) void dense_partial_kernel(
    const uint16_t* __restrict__ q, KVArgs kv, int T, int Hq, int G, float scale_log2, int S,
    int chunk, float* __restrict__ part_o, float* __restrict__ part_ml, float* __restrict__ out,
    float* __restrict__ lse) {
  constexpr int KS = D / 32;
  constexpr int DC = D / 64;  // output columns per lane
  constexpr int U = 2;        // tiles in flight per wave
  __shared__ __attribute__((aligned(16))) float pbuf[kAttnWaves][16][16];  // [wave][position][row]
  __shared__ float abuf[kAttnWaves][16];      // per-row rescale of the tile
  __shared__ float red_m[kAttnWaves][16];
  __shared__ float red_l[kAttnWaves][16];
  __shared__ float red_o[kAttnWaves][MR][D];

  const int s = blockIdx.x;
  const int bh = blockIdx.y;
  const int mt = blockIdx.z;
  const int Hkv = kv.num_kv_heads;
  const int b = bh / Hkv, h = bh - (bh / Hkv) * Hkv;
  const int GT = G * T;
  const int r0 = mt * 16;
  const int rows_here = min(16, GT - r0);
  const int L = seq_len_of(kv, b);
  const int start = s * chunk;
  const int end = min(start + chunk, L);

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int mm = lane & 15;
  const int g4 = lane >> 4;
  const int c0 = lane * DC;

  bf16x8 a[KS];
  {
    const int r = r0 + mm;
    if (r < GT) {
      const int t = r / G, gi = r - (r / G) * G;
      const uint16_t* qp = q + (((int64_t)b * T + t) * Hq + (h * G + gi)) * D + g4 * 8;
#pragma unroll
      for (int j = 0; j < KS; ++j) a[j] = __builtin_bit_cast(bf16x8, ld16(qp + j * 32));
    } else {
#pragma unroll
      for (int j = 0; j < KS; ++j) a[j] = __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0));
    }
  }
  int vis[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rl = 4 * g4 + i;
    vis[i] = rl < rows_here ? L - T + (r0 + rl) / G + 1 : 0;
  }
  float mrow[4], lrow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    mrow[i] = -INFINITY;
    lrow[i] = 0.f;
  }
  float o[MR][DC];
#pragma unroll
  for (int r = 0; r < MR; ++r)
#pragma unroll
    for (int d = 0; d < DC; ++d) o[r][d] = 0.f;

  for (int n0 = start + wave * 16; n0 < end; n0 += kAttnWaves * 16 * U) {
    uint4 kb[U][KS];
    uint32_t vb[U][16];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int tile = n0 + u * kAttnWaves * 16;
      if (tile < end) {
        const int64_t base = kv_tile<D, PAGED>(kv, b, h, tile);
        const int nk = min(mm, L - 1 - tile);
#pragma unroll
        for (int j = 0; j < KS; ++j) kb[u][j] = ld16(kv.k + base + (int64_t)nk * D + g4 * 8 + j * 32);
#pragma unroll
        for (int n = 0; n < 16; ++n) {
          const int nv = min(n, L - 1 - tile);
          const uint16_t* vp = kv.v + base + (int64_t)nv * D + c0;
          if constexpr (DC == 2)
            vb[u][n] = *reinterpret_cast<const uint32_t*>(vp);
          else
            vb[u][n] = (uint32_t)(*vp);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int tile = n0 + u * kAttnWaves * 16;
      if (tile >= end) break;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < KS; ++j)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[j], __builtin_bit_cast(bf16x8, kb[u][j]),
                                                      acc, 0, 0, 0);
      const int n = tile + mm;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float sc = n < vis[i] ? acc[i] * scale_log2 : -INFINITY;
        const float tmax = group_max<16>(sc);
        const float m_new = fmaxf(mrow[i], tmax);
        float alpha, pr;
        if (m_new == -INFINITY) {
          alpha = 1.f;
          pr = 0.f;
        } else {
          alpha = fast_exp2(mrow[i] - m_new);
          pr = fast_exp2(sc - m_new);
        }
        lrow[i] = fmaf(lrow[i], alpha, pr);
        mrow[i] = m_new;
        pbuf[wave][mm][4 * g4 + i] = pr;
        if (mm == 0) abuf[wave][4 * g4 + i] = alpha;
      }
      wave_lds_sync();
#pragma unroll
      for (int r = 0; r < MR; ++r) {
        const float al = abuf[wave][r];
#pragma unroll
        for (int d = 0; d < DC; ++d) o[r][d] *= al;
      }
#pragma unroll
      for (int n = 0; n < 16; ++n) {
        float vf[DC];
        if constexpr (DC == 2) {
          vf[0] = bf16_lo(vb[u][n]);
          vf[1] = bf16_hi(vb[u][n]);
        } else {
          vf[0] = bf16_lo(vb[u][n]);
        }
#pragma unroll
        for (int r4 = 0; r4 < MR; r4 += 4) {
          const float4 pv = *reinterpret_cast<const float4*>(&pbuf[wave][n][r4]);
#pragma unroll
          for (int d = 0; d < DC; ++d) {
            o[r4 + 0][d] = fmaf(pv.x, vf[d], o[r4 + 0][d]);
            o[r4 + 1][d] = fmaf(pv.y, vf[d], o[r4 + 1][d]);
            o[r4 + 2][d] = fmaf(pv.z, vf[d], o[r4 + 2][d]);
            o[r4 + 3][d] = fmaf(pv.w, vf[d], o[r4 + 3][d]);
          }
        }
      }
      wave_lds_sync();
    }
  }

#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float lt = group_sum<16>(lrow[i]);
    if (mm == 0) {
      red_m[wave][4 * g4 + i] = mrow[i];
      red_l[wave][4 * g4 + i] = lt;
    }
  }
#pragma unroll
  for (int r = 0; r < MR; ++r)
#pragma unroll
    for (int d = 0; d < DC; ++d) red_o[wave][r][c0 + d] = o[r][d];
  __syncthreads();

  for (int idx = threadIdx.x; idx < rows_here * D; idx += kAttnThreads) {
    const int rl = idx / D;
    const int col = idx - rl * D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) M = fmaxf(M, red_m[w][rl]);
    float Lsum = 0.f, O = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kAttnWaves; ++w) {
        const float wt = fast_exp2(red_m[w][rl] - M);
        Lsum = fmaf(wt, red_l[w][rl], Lsum);
        O = fmaf(wt, red_o[w][rl][col], O);
      }
    }
    const int r = r0 + rl;
    const int t = r / G, gi = r - (r / G) * G;
    const int64_t row = ((int64_t)b * T + t) * Hq + (h * G + gi);
    store_result(O, M, Lsum, col, D, row, s, S, part_o, part_ml, out, lse);
  }
}

// ============================================================================ launchers
template <int D, bool PAGED>
static hipError_t launch_sparse_t(const AttnLaunch& a, hipStream_t stream) {
  const int n_groups = a.B * a.kv.num_kv_heads;
  const int items = a.GT * a.S;
  const int64_t blocks = 8LL * ((n_groups + 7) / 8) * items;
  hipLaunchKernelGGL((sparse_partial_kernel<D, PAGED>), dim3((unsigned)blocks), dim3(kAttnThreads),
                     0, stream, a.q, a.kv, a.indices, a.T, a.Hq, a.G, a.k_max, a.scale_log2, a.S,
                     a.chunk, n_groups, items, a.part_o, a.part_ml, a.out, a.lse);
  return hipGetLastError();
}

static hipError_t launch_combine(const AttnLaunch& a, hipStream_t stream) {
  if (a.S == 1) return hipSuccess;
  hipLaunchKernelGGL(combine_kernel, dim3(a.rows), dim3(a.D), 0, stream, a.part_o, a.part_ml, a.S,
                     a.D, a.out, a.lse);
  return hipGetLastError();
}

hipError_t launch_sparse(const AttnLaunch& a, hipStream_t stream) {
  hipError_t e;
  if (a.D == 128)
    e = a.paged ? launch_sparse_t<128, true>(a, stream) : launch_sparse_t<128, false>(a, stream);
  else
    e = a.paged ? launch_sparse_t<64, true>(a, stream) : launch_sparse_t<64, false>(a, stream);
  if (e != hipSuccess) return e;
  return launch_combine(a, stream);
}

template <int D, bool PAGED, int MR>
static hipError_t launch_dense_t(const AttnLaunch& a, hipStream_t stream) {
  dim3 grid(a.S, a.B * a.kv.num_kv_heads, (a.GT + 15) / 16);
  hipLaunchKernelGGL((dense_partial_kernel<D, PAGED, MR>), grid, dim3(kAttnThreads), 0, stream, a.q,
                     a.kv, a.T, a.Hq, a.G, a.scale_log2, a.S, a.chunk, a.part_o, a.part_ml, a.out,
                     a.lse);
  return hipGetLastError();
}

template <int D, bool PAGED>
static hipError_t launch_dense_d(const AttnLaunch& a, hipStream_t stream) {
  const int rows_tile = a.GT < 16 ? a.GT : 16;
  if (rows_tile <= 4) return launch_dense_t<D, PAGED, 4>(a, stream);
  if (rows_tile <= 8) return launch_dense_t<D, PAGED, 8>(a, stream);
  return launch_dense_t<D, PAGED, 16>(a, stream);
}

hipError_t launch_dense(const AttnLaunch& a, hipStream_t stream) {
  hipError_t e;
  if (a.D == 128)
    e = a.paged ? launch_dense_d<128, true>(a, stream) : launch_dense_d<128, false>(a, stream);
  else
    e = a.paged ? launch_dense_d<64, true>(a, stream) : launch_dense_d<64, false>(a, stream);
  if (e != hipSuccess) return e;
  return launch_combine(a, stream);
}

}  // namespace cs
