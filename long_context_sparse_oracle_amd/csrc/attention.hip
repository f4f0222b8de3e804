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
// One workgroup per (row, split) of up to MAXW waves; each wave takes E entries of the row's
// index list per round and loops, so many short rounds of different waves overlap and the data
// that arrives last leaves little compute behind it.  Rows of one (request, KV head) are kept on
// one XCD (workgroup w runs on XCD w % 8, so group g gets the ids congruent to g mod 8): rows of
// a GQA group that pick the same token find its K/V lines in that XCD's L2.
// Indices are loaded one round ahead with one coalesced load and handed to the lanes with
// ds_bpermute (paged caches: the entries two rounds ahead and their page ids one round ahead, so
// no round's gathers wait on a page-table lookup); a round then issues all of its K loads and then all of its V loads before using
// any: D/8 lanes hold one position (8 dims = 16 bytes of K and of V), 64/(D/8) positions per
// step.  Scores are reduced across the D/8 lanes with DPP, the round's softmax statistics are
// merged into the running (m, l, o); at the end the wave's position groups are merged with lane
// shuffles and the waves through LDS.
template <int D, bool PAGED, int E, int MAXW>
__global__ void __launch_bounds__(MAXW * 64)
sparse_partial_kernel(
    const uint16_t* __restrict__ q, KVArgs kv, const int32_t* __restrict__ indices, int T, int Hq,
    int G, int k_max, float scale_log2, int S, int chunk, int n_groups, int items_per_group,
    float* __restrict__ part_o, float* __restrict__ part_ml, float* __restrict__ out,
    float* __restrict__ lse) {
  constexpr int LPP = D / 8;                        // lanes per position
  constexpr int PPW = kWave / LPP;                  // positions per wave step
  constexpr int NSTEP = E / PPW;                    // steps per round
  __shared__ float red_m[MAXW];
  __shared__ float red_l[MAXW];
  __shared__ float red_o[MAXW][D];

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

  const int vis = seq_len_vec(kv, b) - T + t + 1;  // per lane, wanted only by the validity test
  const int lo = s * chunk;
  const int hi = min(lo + chunk, k_max);

  const int nwaves = blockDim.x >> 6;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int p = lane / LPP;
  const int c = lane - p * LPP;

  // q slice of this lane as 4 packed bf16 pairs (dims c*8 .. c*8+7)
  const uint4 qv = ld16(q + row * D + c * 8);
  const uint32_t qw[4] = {qv.x, qv.y, qv.z, qv.w};

  float m = -INFINITY, l = 0.f;
  float o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = 0.f;

  // Contiguous caches address rows of this (request, KV head) from one base with 32-bit
  // offsets; paged caches translate every position through the page table.
  const int64_t slab = PAGED ? 0 : (int64_t)(b * kv.num_kv_heads + h) * kv.max_len * D;
  const uint16_t* kbase = kv.k + slab;
  const uint16_t* vbase = kv.v + slab;
  const int32_t* irow = indices + row * k_max;
  // Index loads run one round ahead of the gathers, and the first is issued next to the q load,
  // so neither waits for the other.  They are unconditional and clamped to the last entry of the
  // split (k_max >= 1 makes hi - 1 a valid entry): the compiler then counts them like the
  // gathers and never has to drain the memory counter at the loop head.
  const int round_step = nwaves * E;
  // One round: the K/V rows at element offsets off[u] (entry u valid when bit u of okm is set),
  // all K loads then all V loads in flight before any is used, then the online-softmax update.
  auto gather_round = [&](const int64_t (&off)[NSTEP], uint32_t okm) __attribute__((always_inline)) {
    uint4 kr[NSTEP], vr[NSTEP];
#pragma unroll
    for (int u = 0; u < NSTEP; ++u) kr[u] = ld16(kbase + off[u]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < NSTEP; ++u) vr[u] = ld16(vbase + off[u]);
    __builtin_amdgcn_sched_barrier(0);
    float sv[NSTEP];
    float mx = -INFINITY;
#pragma unroll
    for (int u = 0; u < NSTEP; ++u) {
      float dot = 0.f;
      dot = dot2_bf16(qw[0], kr[u].x, dot);
      dot = dot2_bf16(qw[1], kr[u].y, dot);
      dot = dot2_bf16(qw[2], kr[u].z, dot);
      dot = dot2_bf16(qw[3], kr[u].w, dot);
      dot = group_sum<LPP>(dot);
      sv[u] = ((okm >> u) & 1u) ? dot * scale_log2 : -INFINITY;
      mx = fmaxf(mx, sv[u]);
    }
    const float m_new = fmaxf(m, mx);
    if (m_new == -INFINITY) return;
    const float alpha = fast_exp2(m - m_new);
    l *= alpha;
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] *= alpha;
#pragma unroll
    for (int u = 0; u < NSTEP; ++u) {
      const float pw = fast_exp2(sv[u] - m_new);
      l += pw;
      float vf[8];
      unpack8(vr[u], vf);
#pragma unroll
      for (int i = 0; i < 8; ++i) o[i] = fmaf(pw, vf[i], o[i]);
    }
    m = m_new;
  };
  if constexpr (PAGED) {
    // The page ids of a round's positions are loaded one round ahead (the entries two rounds
    // ahead), so a round's K/V loads wait on no page-table lookup.  An invalid entry reads
    // position 0's page and is masked out.
    const int64_t pt_row = (int64_t)b * kv.max_pages;
    auto pages_of = [&](int entry, int (&pg)[NSTEP]) __attribute__((always_inline)) {
#pragma unroll
      for (int u = 0; u < NSTEP; ++u) {
        const int x = __shfl(entry, u * PPW + p);
        const int n = (x >= 0 && x < vis) ? x : 0;
        pg[u] = kv.page_table[pt_row + (n >> kv.page_shift)];
      }
    };
    int base = lo + wave * E;
    int mine = base + lane < hi ? irow[min(base + lane, hi - 1)] : -1;
    int pgc[NSTEP];
    pages_of(mine, pgc);
    int next_idx = irow[min(base + round_step + lane, hi - 1)];
    for (; base < hi; base += round_step) {
      const int nmine = base + round_step + lane < hi ? next_idx : -1;
      next_idx = irow[min(base + 2 * round_step + lane, hi - 1)];
      int pgn[NSTEP];
      pages_of(nmine, pgn);
      // a round of padding (-1) or otherwise invalid entries issues no loads
      if (__ballot(mine >= 0 && mine < vis) != 0ull) {
        uint32_t okm = 0;
        int64_t off[NSTEP];
#pragma unroll
        for (int u = 0; u < NSTEP; ++u) {
          const int x = __shfl(mine, u * PPW + p);
          const bool ok = x >= 0 && x < vis;
          okm |= (uint32_t)ok << u;
          const int n = ok ? x : 0;
          int page = pgc[u];
          page = page < 0 ? 0 : (page >= kv.num_pages ? kv.num_pages - 1 : page);
          off[u] = ((((int64_t)page * kv.num_kv_heads + h) << kv.page_shift) + (n & ((1 << kv.page_shift) - 1))) * D +
                   c * 8;
        }
        gather_round(off, okm);
      }
      mine = nmine;
#pragma unroll
      for (int u = 0; u < NSTEP; ++u) pgc[u] = pgn[u];
    }
  } else {
    int base = lo + wave * E;
    int next_idx = irow[min(base + lane, hi - 1)];
    for (; base < hi; base += round_step) {
      const int mine = base + lane < hi ? next_idx : -1;
      next_idx = irow[min(base + round_step + lane, hi - 1)];
      // a round of padding (-1) or otherwise invalid entries issues no loads
      if (__ballot(mine >= 0 && mine < vis) == 0ull) continue;
      uint32_t okm = 0;
      int64_t off[NSTEP];
#pragma unroll
      for (int u = 0; u < NSTEP; ++u) {
        const int x = __shfl(mine, u * PPW + p);
        const bool ok = x >= 0 && x < vis;
        okm |= (uint32_t)ok << u;
        off[u] = (int64_t)(ok ? x : 0) * D + c * 8;
      }
      gather_round(off, okm);
    }
  }

  // merge the wave's PPW position groups (lanes c + LPP p) with lane shuffles, then the waves
  // through LDS
#pragma unroll
  for (int x = LPP; x < kWave; x *= 2) {
    const float m_o = __shfl_xor(m, x);
    const float l_o = __shfl_xor(l, x);
    const float M = fmaxf(m, m_o);
    const float a = m == -INFINITY ? 0.f : fast_exp2(m - M);
    const float bw = m_o == -INFINITY ? 0.f : fast_exp2(m_o - M);
    l = a * l + bw * l_o;
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = a * o[i] + bw * __shfl_xor(o[i], x);
    m = M;
  }
  const int slot = wave;
  if (lane == 0) {
    red_m[slot] = m;
    red_l[slot] = l;
  }
  if (p == 0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) red_o[slot][c * 8 + i] = o[i];
  }
  __syncthreads();
  const int nslots = nwaves;
  for (int col = threadIdx.x; col < D; col += blockDim.x) {
    float M = -INFINITY;
    for (int k = 0; k < nslots; ++k) M = fmaxf(M, red_m[k]);
    float Lsum = 0.f, O = 0.f;
    if (M != -INFINITY) {
      for (int k = 0; k < nslots; ++k) {
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
// with M = max_s m_s (m in log2 units).  One workgroup of D threads per row; the split weights
// e^{m_s - M} are computed once into LDS (dynamic, 2 * S floats).
__global__ void combine_kernel(const float* __restrict__ part_o, const float* __restrict__ part_ml,
                               int S, int D, float* __restrict__ out, float* __restrict__ lse) {
  extern __shared__ float cw[];  // [S] weights, then [S] weighted l
  __shared__ float red[8];
  const int64_t row = blockIdx.x;
  const int col = threadIdx.x;
  const float* ml = part_ml + row * S * 2;
  float M = -INFINITY;
  for (int s = col; s < S; s += blockDim.x) M = fmaxf(M, ml[2 * s]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
  if ((col & 63) == 0) red[col >> 6] = M;
  __syncthreads();
  M = red[0];
  for (int w = 1; w < (int)(blockDim.x >> 6); ++w) M = fmaxf(M, red[w]);
  for (int s = col; s < S; s += blockDim.x) {
    const float w = M == -INFINITY ? 0.f : fast_exp2(ml[2 * s] - M);
    cw[s] = w;
    cw[S + s] = w * ml[2 * s + 1];
  }
  __syncthreads();
  float Lsum = 0.f, O = 0.f;
  const float* po = part_o + row * S * D + col;
  for (int s = 0; s < S; ++s) {
    Lsum += cw[S + s];
    O = fmaf(cw[s], po[(int64_t)s * D], O);
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
  extern __shared__ int lds_pages[];          // paged caches: page ids of this chunk
  __shared__ __attribute__((aligned(16))) float pbuf[kAttnWaves][16][16];  // [wave][position][row]
  __shared__ float abuf[kAttnWaves][16];      // per-row rescale of the tile
  __shared__ float red_m[kAttnWaves][16];
  __shared__ float red_l[kAttnWaves][16];
  __shared__ float red_o[kAttnWaves][MR][D];

  const int bh = blockIdx.y;
  const int s = rotated_chunk(blockIdx.x, bh, gridDim.x);
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

  if constexpr (PAGED) stage_pages(kv, b, start, end, lds_pages);
  __syncthreads();

  // Tiles of this wave: start + 16 * wave + 64 * it.  The K tile (MFMA B operand) and this lane's
  // V columns of tile it+1 are loaded before tile it is processed.
  auto load_tile = [&](int tile, uint4 (&kb)[KS], uint32_t (&vb)[16]) {
    const int64_t base = kv_tile_staged<D, PAGED>(kv, lds_pages, start, b, h, tile);
    const int nk = min(mm, L - 1 - tile);
#pragma unroll
    for (int j = 0; j < KS; ++j) kb[j] = ld16(kv.k + base + (int64_t)nk * D + g4 * 8 + j * 32);
#pragma unroll
    for (int n = 0; n < 16; ++n) {
      const int nv = min(n, L - 1 - tile);
      const uint16_t* vp = kv.v + base + (int64_t)nv * D + c0;
      if constexpr (DC == 2)
        vb[n] = *reinterpret_cast<const uint32_t*>(vp);
      else
        vb[n] = (uint32_t)(*vp);
    }
  };
  auto process = [&](int tile, const uint4 (&kc)[KS], const uint32_t (&vc)[16]) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  #pragma unroll
      for (int j = 0; j < KS; ++j)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[j], __builtin_bit_cast(bf16x8, kc[j]), acc, 0, 0, 0);
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
      for (int nn = 0; nn < 16; ++nn) {
        float vf[DC];
        if constexpr (DC == 2) {
          vf[0] = bf16_lo(vc[nn]);
          vf[1] = bf16_hi(vc[nn]);
        } else {
          vf[0] = bf16_lo(vc[nn]);
        }
  #pragma unroll
        for (int r4 = 0; r4 < MR; r4 += 4) {
          const float4 pv = *reinterpret_cast<const float4*>(&pbuf[wave][nn][r4]);
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
  };
  // ping-pong buffers: tile it+1 loads while tile it is processed, with no register copies
  // Prefetches are unconditional (a tile past the chunk reloads the chunk's last tile, which is
  // cached) so the loads stay straight-line and the compiler's load counters stay exact.
  uint4 ka[KS], kb2[KS];
  uint32_t va[16], vb2[16];
  constexpr int kStride = kAttnWaves * 16;
  if (start < end) {
    const int last = (end - 1) & ~15;
    int tile = start + wave * 16;
    load_tile(min(tile, last), ka, va);
    for (; tile < end; tile += 2 * kStride) {
      load_tile(min(tile + kStride, last), kb2, vb2);
      process(tile, ka, va);
      if (tile + kStride >= end) break;
      load_tile(min(tile + 2 * kStride, last), ka, va);
      process(tile + kStride, kb2, vb2);
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

// ============================================================================ dense partial, MFMA P.V
// For G*T >= 5 query rows per KV head the float32 P.V of dense_partial_kernel is VALU-bound, so
// here both products run on MFMA.  Scores are computed as K q^T (A = 16 tokens x 32 dims of K,
// B = the query rows): lane l then holds tokens 4*(l/16)..+3 of query row l%16, which is exactly
// the A-operand layout of v_mfma_f32_16x16x16_bf16 for P (rows x tokens).  P is split into bf16
// hi + lo parts (two MFMAs, ~16 significant bits), V (tokens x dims, bf16) is staged row-major in
// a per-wave LDS buffer and read as the B operand with ds_read_b64_tr_b16 (lane s of 16-lane
// group g addresses token 4g + s/4, dims 16 nb + 4 (s%4); the transpose hands lane i the
// values of tokens 4g..4g+3 at dim 16 nb + i).  The running max of a row is raised only when a
// tile exceeds it by more than 2^8 (in log2 units), so O is rescaled rarely; P <= 2^8 is exact
// enough in hi + lo bf16.
typedef short v4i16 __attribute__((ext_vector_type(4)));

template <int D, bool PAGED>
__global__ __launch_bounds__(kAttnThreads) void dense_partial_mfma_kernel(
    const uint16_t* __restrict__ q, KVArgs kv, int T, int Hq, int G, float scale_log2, int S,
    int chunk, float* __restrict__ part_o, float* __restrict__ part_ml, float* __restrict__ out,
    float* __restrict__ lse) {
  constexpr int KS = D / 32;        // k-steps of K q^T
  constexpr int NB = D / 16;        // 16-column blocks of P.V
  constexpr int VROW = D * 2 + 32;  // LDS bytes per staged V token (padded against bank conflicts)
  constexpr int VLD = D / 32;       // 16-byte V loads per lane per tile
  constexpr int VBUF = 16 * VROW;   // bytes per wave
  constexpr int RED = kAttnWaves * 16 * D * 4;  // final merge of the waves' O tiles
  constexpr int SHARED = (kAttnWaves * VBUF > RED) ? kAttnWaves * VBUF : RED;
  extern __shared__ int lds_pages[];
  __shared__ __attribute__((aligned(16))) char smem[SHARED];
  __shared__ float red_m[kAttnWaves][16];
  __shared__ float red_l[kAttnWaves][16];

  const int bh = blockIdx.y;
  const int s = rotated_chunk(blockIdx.x, bh, gridDim.x);
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
  const int mm = lane & 15;   // query row (softmax layout) / token of the K operand
  const int g4 = lane >> 4;

  bf16x8 qb[KS];
  int vis_row = 0;
  {
    const int r = r0 + mm;
    if (mm < rows_here) {
      const int t = r / G, gi = r - (r / G) * G;
      const uint16_t* qp = q + (((int64_t)b * T + t) * Hq + (h * G + gi)) * D + g4 * 8;
#pragma unroll
      for (int j = 0; j < KS; ++j) qb[j] = __builtin_bit_cast(bf16x8, ld16(qp + j * 32));
      vis_row = L - T + t + 1;
    } else {
#pragma unroll
      for (int j = 0; j < KS; ++j) qb[j] = __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0));
    }
  }
  float m_row = -INFINITY;  // running max of row mm (log2 units)
  float l_part = 0.f;       // this lane's share of the row sum
  f32x4 oacc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) oacc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  if constexpr (PAGED) stage_pages(kv, b, start, end, lds_pages);
  __syncthreads();

  char* vb = smem + wave * VBUF;
  auto load_tile = [&](int tile, uint4 (&kt)[KS], uint4 (&vt)[VLD]) {
    const int64_t base = kv_tile_staged<D, PAGED>(kv, lds_pages, start, b, h, tile);
    const int nk = min(mm, L - 1 - tile);
#pragma unroll
    for (int j = 0; j < KS; ++j) kt[j] = ld16(kv.k + base + (int64_t)nk * D + g4 * 8 + j * 32);
    const int nv = min(lane >> 2, L - 1 - tile);
#pragma unroll
    for (int x = 0; x < VLD; ++x) vt[x] = ld16(kv.v + base + (int64_t)nv * D + (lane & 3) * (D / 4) + x * 8);
  };
  auto process = [&](int tile, const uint4 (&kt)[KS], const uint4 (&vt)[VLD]) {
#pragma unroll
    for (int x = 0; x < VLD; ++x)
      *reinterpret_cast<uint4*>(vb + (lane >> 2) * VROW + (lane & 3) * (D / 2) + x * 16) = vt[x];
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < KS; ++j)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kt[j]), qb[j], acc, 0, 0, 0);
    float sc[4];
    float tmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sc[i] = tile + 4 * g4 + i < vis_row ? acc[i] * scale_log2 : -INFINITY;
      tmax = fmaxf(tmax, sc[i]);
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const bool raise = tmax > m_row + 8.f;
    if (__ballot(raise)) {
      const float m_new = raise ? tmax : m_row;
      const float alpha = m_row == -INFINITY ? 0.f : fast_exp2(m_row - m_new);
      l_part *= alpha;
      m_row = m_new;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float ai = __shfl(alpha, 4 * g4 + i);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) oacc[nb][i] *= ai;
      }
    }
    uint32_t hi[4], lo[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float p = sc[i] == -INFINITY ? 0.f : fast_exp2(sc[i] - m_row);
      l_part += p;
      const uint32_t pb = __float_as_uint(p);
      hi[i] = pb >> 16;
      lo[i] = __float_as_uint(p - __uint_as_float(pb & 0xffff0000u)) >> 16;
    }
    const v4i16 ahi = __builtin_bit_cast(v4i16, make_uint2(hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16)));
    const v4i16 alo = __builtin_bit_cast(v4i16, make_uint2(lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16)));
    wave_lds_sync();
    const char* vrd = vb + (4 * g4 + (mm >> 2)) * VROW + 4 * (mm & 3) * 2;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const v4i16 bv = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) v4i16*)(vrd + nb * 32));
      oacc[nb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ahi, bv, oacc[nb], 0, 0, 0);
      oacc[nb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(alo, bv, oacc[nb], 0, 0, 0);
    }
    wave_lds_sync();
  };

  uint4 ka[KS], kb2[KS], va[VLD], vb2[VLD];
  constexpr int kStride = kAttnWaves * 16;
  if (start < end) {
    const int last = (end - 1) & ~15;
    int tile = start + wave * 16;
    load_tile(min(tile, last), ka, va);
    for (; tile < end; tile += 2 * kStride) {
      load_tile(min(tile + kStride, last), kb2, vb2);
      process(tile, ka, va);
      if (tile + kStride >= end) break;
      load_tile(min(tile + 2 * kStride, last), ka, va);
      process(tile + kStride, kb2, vb2);
    }
  }

  // row sums over the 4 lanes holding a row; merge the waves
  float l_row = l_part + __shfl_xor(l_part, 16);
  l_row += __shfl_xor(l_row, 32);
  __syncthreads();  // every wave is done with its V buffer before the merge area reuses it
  float* red_o = reinterpret_cast<float*>(smem);  // [wave][16 rows][D]
  if (g4 == 0) {
    red_m[wave][mm] = m_row;
    red_l[wave][mm] = l_row;
  }
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int i = 0; i < 4; ++i) red_o[(wave * 16 + 4 * g4 + i) * D + nb * 16 + mm] = oacc[nb][i];
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
        O = fmaf(wt, red_o[(w * 16 + rl) * D + col], O);
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
  const int waves = a.waves < 1 ? 1 : (a.waves > kSparseWaves ? kSparseWaves : a.waves);
  auto kern = a.entries == kSparseWaveEntriesBig ? sparse_partial_kernel<D, PAGED, kSparseWaveEntriesBig, kSparseWaves>
                                                 : sparse_partial_kernel<D, PAGED, kSparseWaveEntries, kSparseWaves>;
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(waves * kWave), 0, stream, a.q, a.kv, a.indices,
                     a.T, a.Hq, a.G, a.k_max, a.scale_log2, a.S, a.chunk, n_groups, items,
                     a.part_o, a.part_ml, a.out, a.lse);
  return hipGetLastError();
}

static hipError_t launch_combine(const AttnLaunch& a, hipStream_t stream) {
  if (a.S == 1) return hipSuccess;
  hipLaunchKernelGGL(combine_kernel, dim3(a.rows), dim3(a.D), 2 * a.S * sizeof(float), stream,
                     a.part_o, a.part_ml, a.S,
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
  const size_t lds = PAGED ? ((size_t)(a.chunk >> a.kv.page_shift) + 2) * sizeof(int) : 0;
  hipLaunchKernelGGL((dense_partial_kernel<D, PAGED, MR>), grid, dim3(kAttnThreads), lds, stream, a.q,
                     a.kv, a.T, a.Hq, a.G, a.scale_log2, a.S, a.chunk, a.part_o, a.part_ml, a.out,
                     a.lse);
  return hipGetLastError();
}

template <int D, bool PAGED>
static hipError_t launch_dense_mfma_t(const AttnLaunch& a, hipStream_t stream) {
  dim3 grid(a.S, a.B * a.kv.num_kv_heads, (a.GT + 15) / 16);
  const size_t lds = PAGED ? ((size_t)(a.chunk >> a.kv.page_shift) + 2) * sizeof(int) : 0;
  hipLaunchKernelGGL((dense_partial_mfma_kernel<D, PAGED>), grid, dim3(kAttnThreads), lds, stream,
                     a.q, a.kv, a.T, a.Hq, a.G, a.scale_log2, a.S, a.chunk, a.part_o, a.part_ml,
                     a.out, a.lse);
  return hipGetLastError();
}

// Up to 4 query rows per KV head: float32 P.V on the VALU is cheap enough; more rows: MFMA P.V.
template <int D, bool PAGED>
static hipError_t launch_dense_d(const AttnLaunch& a, hipStream_t stream) {
  const int rows_tile = a.GT < 16 ? a.GT : 16;
  if (rows_tile <= 4) return launch_dense_t<D, PAGED, 4>(a, stream);
  return launch_dense_mfma_t<D, PAGED>(a, stream);
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
