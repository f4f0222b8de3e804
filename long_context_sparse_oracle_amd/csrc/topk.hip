// Oracle top-k indexer for gfx950, and the parts of the decode step that sit on its scores.
//  * full-score path: a streaming score kernel (q.K^T on MFMA, fused 12-bit radix histogram) and
//    a per-row select kernel (LDS radix refinement, ballot compaction);
//  * candidate path (short lists): sampled thresholds, a streaming pass that keeps only the
//    candidates above them, and a per-row radix select over the candidates;
//  * the one-call step's attention on the selected lists with the indexer's own scores;
//  * the reduced-byte indexer: the same passes on an int8 key sketch, then an exact re-rank.
//
// Method: exact top-k selection of cached tokens per (request, token, query head), as used by the
// oracle indexer of "Inference Time Context Sparsity: Illusion or Opportunity?" (technical
// summary, section 2, sparsity mechanisms).  Ranking is by the float32 score
// s = (q . K) * sm_scale, larger first, lower position first among equal scores.
#include "device_common.h"
#include "launch.h"

namespace cs {

typedef uint32_t v2u32 __attribute__((ext_vector_type(2)));
typedef uint32_t v4u32 __attribute__((ext_vector_type(4)));

constexpr int kHistBins = 4096;      // 12 leading bits of the ordered key
constexpr int kScoreMaxThreads = 1024;  // up to 16 waves (4 per 4 query rows of the group)
constexpr int kScoreUnroll = 2;      // 16-position tiles in flight per wave
constexpr int kSelThreads = 1024;    // 16 waves
constexpr int kSelWaves = kSelThreads / kWave;
constexpr int kCandCap = 8192;       // threshold-bin candidates held in LDS
constexpr int kSelVecUnroll = 8;     // 16-byte score loads in flight per lane in the select pass

// ============================================================================ clear
// Fills n 32-bit words (n a multiple of 4, p 16-byte aligned) with 16-byte stores.
__global__ void fill_u32_kernel(uint32_t* __restrict__ p, int64_t n, uint32_t value) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const uint4 v = make_uint4(value, value, value, value);
  uint4* p4 = reinterpret_cast<uint4*>(p);
  for (; i < n / 4; i += stride) p4[i] = v;
}

// 16 bytes of int8 codes
__device__ __forceinline__ uint4 ld16i8(const int8_t* p) { return *reinterpret_cast<const uint4*>(p); }

// Scores of one 16-position tile for the 4 MFMA rows 4 * (lane / 16) + i of this lane, from the
// operand steps a (query rows) and kt (key rows, this lane's position lane % 16):
//   exact   bf16 dot products times `scale`;
//   SK      sketch scores (qsc[i] * ksc) * (c_q . c_k), the integer dot product exact in int32.
template <bool SK, int KS>
__device__ __forceinline__ void tile_scores(const uint4 (&a)[KS], const uint4 (&kt)[KS], float scale,
                                            const float (&qsc)[4], float ksc, float (&sc)[4]) {
  if constexpr (SK) {
    i32x4 acc = {0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < KS; ++j)
      acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, a[j]), __builtin_bit_cast(i32x4, kt[j]),
                                                  acc, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) sc[i] = (qsc[i] * ksc) * (float)acc[i];
  } else {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < KS; ++j)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[j]), __builtin_bit_cast(bf16x8, kt[j]),
                                                    acc, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) sc[i] = acc[i] * scale;
  }
}

// ============================================================================ score + histogram
// Grid: (chunks, B * Hkv, ceil(G*T / 16)).  One workgroup (4 waves per 4 query rows, so the
// LDS histogram never starves a CU of waves) streams `chunk` positions of one (request, KV head)
// and scores them against up to 16 of the G*T query rows that read that head
// (row r = t * G + g, query head h * G + g).  Per 16-position tile a wave issues D/32
// v_mfma_f32_16x16x32_bf16: A = the 16 query rows (lane l: row l%16, 8 dims), B = K^T (lane l:
// position l%16, the same 8 dims), so each K row is read once for all rows of the group.
// Scores of visible positions go to scores[row][n]; their 12-bit key prefix is counted in an LDS
// histogram (two 16-bit counters per word) that is added to the global one at the end.
// SK: sketch scores instead (int8 codes of q and K, v_mfma_i32_16x16x64_i8).
template <int D, bool PAGED, bool SK>
__global__ __launch_bounds__(kScoreMaxThreads) void score_hist_kernel(
    const uint16_t* __restrict__ q, KVArgs kv, SketchArgs sk, int T, int Hq, int G, float scale,
    float* __restrict__ scores, uint32_t* __restrict__ hist, int chunk, int hist_rows,
    int64_t score_stride) {
  extern __shared__ uint32_t lds_hist[];  // [hist_rows][kHistBins / 2], then the chunk's page ids
  int* lds_pages = reinterpret_cast<int*>(lds_hist + hist_rows * (kHistBins / 2));
  constexpr int KS = SK ? D / 64 : D / 32;  // MFMA k-steps per tile
  const int bh = blockIdx.y;
  const int c = rotated_chunk(blockIdx.x, bh, gridDim.x);
  const int mt = blockIdx.z;
  const int Hkv = kv.num_kv_heads;
  const int b = bh / Hkv, h = bh - (bh / Hkv) * Hkv;
  const int GT = G * T;
  const int r0 = mt * 16;
  const int rows_here = min(16, GT - r0);
  const int L = seq_len_of(kv, b);
  const int start = c * chunk;
  if (start >= L) return;
  const int end = min(start + chunk, L);

  for (int i = threadIdx.x; i < rows_here * (kHistBins / 2); i += blockDim.x) lds_hist[i] = 0u;
  if constexpr (PAGED) stage_pages(kv, b, start, end, lds_pages);

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int m = lane & 15;
  const int g4 = lane >> 4;

  // A operand: query row r0 + m, dims j*32 + g4*8 .. +8 (SK: codes j*64 + g4*16 .. +16).
  uint4 a[KS];
  {
    const int r = r0 + m;
    if (r < GT) {
      const int t = r / G, gi = r - (r / G) * G;
      const int64_t qr = ((int64_t)b * T + t) * Hq + (h * G + gi);
#pragma unroll
      for (int j = 0; j < KS; ++j)
        a[j] = SK ? ld16i8(sk.q_codes + qr * D + g4 * 16 + j * 64) : ld16(q + qr * D + g4 * 8 + j * 32);
    } else {
#pragma unroll
      for (int j = 0; j < KS; ++j) a[j] = make_uint4(0, 0, 0, 0);
    }
  }
  // Output rows held by this lane: 4*g4 + i (i = 0..3).
  int vis[4];
  float* srow[4];
  float qsc[4];  // SK: the rows' scales
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rl = 4 * g4 + i;
    const int r = r0 + rl;
    if (rl < rows_here) {
      const int t = r / G, gi = r - (r / G) * G;
      const int64_t qr = ((int64_t)b * T + t) * Hq + (h * G + gi);
      vis[i] = L - T + t + 1;
      srow[i] = scores + qr * score_stride;
      qsc[i] = SK ? sk.q_scales[qr] : 0.f;
    } else {
      vis[i] = 0;
      srow[i] = scores;
      qsc[i] = 0.f;
    }
  }
  __syncthreads();

  // Iteration `it` covers positions start + kStep * it .. + kStep; wave w scores the kScoreUnroll
  // adjacent tiles at start + kStep * it + 16 * (kScoreUnroll * w + u), so each of its score
  // stores per row fills consecutive 64-byte pieces of one line.  The K tiles of iteration it+1
  // load while iteration it is scored (ping-pong buffers, no register copies); loads are
  // unconditional (a tile past the chunk reloads the chunk's last tile, which is cached) so they
  // stay straight-line and the compiler's load counters stay exact.
  const uint16_t* kbase = kv.k;
  const int kStep = (int)(blockDim.x >> 6) * 16 * kScoreUnroll;
  const int last = (end - 1) & ~15;
  uint4 cur[kScoreUnroll][KS], nxt[kScoreUnroll][KS];
  float csc[kScoreUnroll], nsc[kScoreUnroll];  // SK: the tiles' key scales (this lane's position)
  auto load_tiles = [&](int n0, uint4 (&dst)[kScoreUnroll][KS], float (&dsc)[kScoreUnroll]) {
#pragma unroll
    for (int u = 0; u < kScoreUnroll; ++u) {
      const int tile = min(n0 + u * 16, last);
      const int64_t off = kv_tile_staged<D, PAGED>(kv, lds_pages, start, b, h, tile) +
                          (int64_t)min(m, L - 1 - tile) * D;
#pragma unroll
      for (int j = 0; j < KS; ++j)
        dst[u][j] = SK ? ld16i8(sk.codes + off + g4 * 16 + j * 64) : ld16(kbase + off + g4 * 8 + j * 32);
      dsc[u] = SK ? sk.scales[off / D] : 0.f;
    }
  };
  auto score_tiles = [&](int n0, const uint4 (&kt)[kScoreUnroll][KS], const float (&ksc)[kScoreUnroll]) {
#pragma unroll
    for (int u = 0; u < kScoreUnroll; ++u) {
      const int tile = n0 + u * 16;
      if (tile >= end) break;
      float sc[4];
      tile_scores<SK, KS>(a, kt[u], scale, qsc, ksc[u], sc);
      const int n = tile + m;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (n < vis[i]) {
          const float s = sc[i];
          srow[i][n] = s;
          const uint32_t bin = ord_key(s) >> 20;
          atomicAdd(&lds_hist[(4 * g4 + i) * (kHistBins / 2) + (bin >> 1)], 1u << ((bin & 1u) * 16));
        }
      }
    }
  };
  int n0 = start + wave * 16 * kScoreUnroll;
  load_tiles(n0, cur, csc);
  for (; n0 < end; n0 += 2 * kStep) {
    load_tiles(n0 + kStep, nxt, nsc);
    score_tiles(n0, cur, csc);
    if (n0 + kStep >= end) break;
    load_tiles(n0 + 2 * kStep, cur, csc);
    score_tiles(n0 + kStep, nxt, nsc);
  }
  __syncthreads();

  for (int w = threadIdx.x; w < rows_here * (kHistBins / 2); w += blockDim.x) {
    const uint32_t v = lds_hist[w];
    if (v == 0u) continue;
    const int rl = w / (kHistBins / 2);
    const int r = r0 + rl;
    const int t = r / G, gi = r - (r / G) * G;
    const int64_t grow = ((int64_t)b * T + t) * Hq + (h * G + gi);
    uint32_t* hp = hist + grow * kHistBins + 2 * (w - rl * (kHistBins / 2));
    if (v & 0xffffu) __hip_atomic_fetch_add(hp, v & 0xffffu, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (v >> 16) __hip_atomic_fetch_add(hp + 1, v >> 16, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// ============================================================================ select
// Block-wide exclusive prefix sum over the NW * 64 threads' values.  SYNC_AFTER = false leaves
// out the closing barrier, for callers that pass another barrier before wsum is written again.
template <int NW = kSelWaves, bool SYNC_AFTER = true>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* wsum, uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t x = wave_incl_scan_u32(v);
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const uint32_t t = wsum[w];
    before += w < wave ? t : 0u;
    all += t;
  }
  if (total) *total = all;
  if constexpr (SYNC_AFTER) __syncthreads();  // wsum may be reused right away
  return before + x - v;
}

struct SelShared {
  uint32_t wsum[kSelWaves + 1];
  uint32_t kmin, kmax;  // key range of a candidate list
  uint32_t cand_count;
  uint32_t thr_bin;    // bin holding the k-th largest key
  uint32_t thr_above;  // keys in higher bins
  uint32_t thr_count;  // keys in the threshold bin
  uint32_t found;
};

// Folds this thread's key range into sh.kmin / sh.kmax (which start at ~0 / 0): reduced over the
// wave first, so one lane per wave issues the LDS atomics (the compiler otherwise serialises a
// same-address atomic through a 64-step loop on the scalar unit that the CU's waves share).  All
// lanes of the wave take part.
__device__ __forceinline__ void block_key_range(uint32_t lmin, uint32_t lmax, SelShared& sh) {
  lmin = wave_min_u32(lmin);
  lmax = wave_max_u32(lmax);
  if ((threadIdx.x & 63) == 0) {
    atomicMin(&sh.kmin, lmin);
    atomicMax(&sh.kmax, lmax);
  }
}

// Finds, over `nbins` counters hist[0..nbins) (bin nbins-1 highest), the bin holding the need-th
// largest key.  Each of the NW * 64 threads covers PER = nbins / (NW * 64) consecutive bins,
// highest bins on thread 0.  Returns the total count.
template <int PER, int NW = kSelWaves>
__device__ uint32_t find_threshold(const uint32_t* hist, int nbins, uint32_t need, SelShared& sh) {
  uint32_t cnt[PER];
  uint32_t sum = 0;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int bin = nbins - 1 - (threadIdx.x * PER + e);
    cnt[e] = hist[bin];
    sum += cnt[e];
  }
  if (threadIdx.x == 0) sh.found = 0u;
  uint32_t total;
  uint32_t above = block_excl_scan<NW, false>(sum, sh.wsum, &total);  // the barrier below closes it
  if (above < need && above + sum >= need) {
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      if (above + cnt[e] >= need) {
        sh.thr_bin = (uint32_t)(nbins - 1 - (threadIdx.x * PER + e));
        sh.thr_above = above;
        sh.thr_count = cnt[e];
        sh.found = 1u;
        break;
      }
      above += cnt[e];
    }
  }
  __syncthreads();
  return total;
}

// Shared memory of the select kernels (dynamic part; the layout select_lds_bytes sizes).
struct SelLds {
  uint32_t* hist;      // kHistBins
  uint32_t* gt_bits;   // bitmap words: positions taken
  uint32_t* eq_bits;   // bitmap words: positions whose key equals the k-th key
  uint32_t* cand_key;  // kCandCap
  uint32_t* cand_pos;  // kCandCap
};

__device__ __forceinline__ SelLds sel_lds(uint32_t* smem, int bitmap_words) {
  SelLds l;
  l.hist = smem;
  l.gt_bits = l.hist + kHistBins;
  l.eq_bits = l.gt_bits + bitmap_words;
  l.cand_key = l.eq_bits + bitmap_words;
  l.cand_pos = l.cand_key + kCandCap;
  return l;
}

// Keeps the `need` lowest positions flagged in eq_bits (keys equal to the k-th key) unless all of
// them are taken, then writes the positions flagged in gt_bits in ascending order (kk of them)
// and pads the row to k_max with -1.  The caller synchronises before.
__device__ void emit_selection(const SelLds& l, int words, uint32_t need, bool take_all_eq, int kk,
                               int k_max, int32_t* __restrict__ out, SelShared& sh) {
  const int tid = threadIdx.x;
  const int wpt = (words + kSelThreads - 1) / kSelThreads;  // bitmap words per thread
  const int w0 = tid * wpt;
  if (!take_all_eq) {
    // keep the `need` lowest positions among keys equal to K*
    uint32_t cnt = 0;
    for (int w = w0; w < min(w0 + wpt, words); ++w) cnt += __popc(l.eq_bits[w]);
    uint32_t before = block_excl_scan(cnt, sh.wsum, nullptr);
    for (int w = w0; w < min(w0 + wpt, words); ++w) {
      uint32_t bits = l.eq_bits[w];
      while (bits) {
        const uint32_t bit = bits & (0u - bits);
        if (before < need) l.gt_bits[w] |= bit;
        ++before;
        bits ^= bit;
      }
    }
    __syncthreads();
  }

  uint32_t cnt = 0;
  for (int w = w0; w < min(w0 + wpt, words); ++w) cnt += __popc(l.gt_bits[w]);
  uint32_t pos = block_excl_scan(cnt, sh.wsum, nullptr);
  for (int w = w0; w < min(w0 + wpt, words); ++w) {
    uint32_t bits = l.gt_bits[w];
    while (bits) {
      const int bit = __ffs(bits) - 1;
      if (pos < (uint32_t)k_max) out[pos] = w * 32 + bit;
      ++pos;
      bits &= bits - 1;
    }
  }
  for (int i = kk + tid; i < k_max; i += kSelThreads) out[i] = -1;
}

// Selects the kk largest of srow[0, vis) (1 <= kk < vis) into out, ascending, padded to k_max
// with -1.  hist_row is the row's 12-bit key-prefix histogram, or nullptr to build it here.
//  1. threshold bin T12 of the 12-bit prefix from the histogram (rebuilt from the scores when it
//     does not add up to the visible count);
//  2. one pass over the scores (16-byte loads): keys above T12 are marked in an LDS bitmap (8
//     lanes' 4-bit nibbles OR-reduced per 32-bit word), keys in T12 are appended to an LDS
//     candidate list;
//  3. two 10-bit radix rounds over the candidates give the exact k-th key K* and how many keys
//     equal to K* are taken (lowest positions first); when T12 holds more than kCandCap keys the
//     rounds read the scores instead;
//  4. the bitmap is emitted in ascending position order by a block prefix sum of popcounts.
__device__ void select_dense_row(const float* __restrict__ srow, const uint32_t* __restrict__ hist_row,
                                 int vis, int kk, int k_max, int32_t* __restrict__ out,
                                 const SelLds& l, SelShared& sh) {
  uint32_t* hist_s = l.hist;
  uint32_t* gt_bits = l.gt_bits;
  uint32_t* eq_bits = l.eq_bits;
  uint32_t* cand_key = l.cand_key;
  uint32_t* cand_pos = l.cand_pos;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;

  const int words = ((vis + 255) >> 8) * 8;  // bitmap words touched (256-position granules)
  for (int i = tid; i < words; i += kSelThreads) {
    gt_bits[i] = 0u;
    eq_bits[i] = 0u;
  }
  if (tid == 0) sh.cand_count = 0u;

  // Scores are read 16 bytes (4 positions) per lane: iteration B covers kSelIter positions, wave w
  // the 256-position blocks B + 256 * (kSelWaves * u + w).  The first iteration's loads are issued
  // before the threshold search so they are in flight meanwhile.
  constexpr int kSelIter = kSelThreads * 4 * kSelVecUnroll;
  // the row's histogram: one 16-byte load per thread, issued first
  static_assert(kHistBins == 4 * kSelThreads, "one uint4 of histogram bins per thread");
  const uint4 hv = hist_row ? reinterpret_cast<const uint4*>(hist_row)[tid] : make_uint4(0, 0, 0, 0);
  float4 sv[kSelVecUnroll];
  auto load_iter = [&](int B) {
#pragma unroll
    for (int u = 0; u < kSelVecUnroll; ++u) {
      const int n4 = B + (u * kSelWaves + wave) * 256 + lane * 4;
      sv[u] = n4 < vis ? *reinterpret_cast<const float4*>(srow + n4) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  load_iter(0);

  // ---- 1. threshold bin of the 12-bit prefix
  reinterpret_cast<uint4*>(hist_s)[tid] = hv;
  __syncthreads();
  uint32_t total = find_threshold<kHistBins / kSelThreads>(hist_s, kHistBins, (uint32_t)kk, sh);
  if (!hist_row || total != (uint32_t)vis || !sh.found) {
    // histogram does not describe this row: rebuild it from the scores
    for (int i = tid; i < kHistBins; i += kSelThreads) hist_s[i] = 0u;
    __syncthreads();
    for (int n = tid; n < vis; n += kSelThreads) atomicAdd(&hist_s[ord_key(srow[n]) >> 20], 1u);
    __syncthreads();
    find_threshold<kHistBins / kSelThreads>(hist_s, kHistBins, (uint32_t)kk, sh);
  }
  const uint32_t T12 = sh.thr_bin;
  uint32_t need = (uint32_t)kk - sh.thr_above;  // keys still to take from bin T12
  const uint32_t cntT = sh.thr_count;
  const bool fast = cntT <= (uint32_t)kCandCap;
  __syncthreads();

  // ---- 2. mark keys above T12 in the bitmap, collect keys in T12
  // A lane's 4 flags form a nibble; 8 lanes' nibbles OR-reduced with DPP give one 32-bit word.
  // Candidate slots: ballots of all blocks first, then one LDS atomic per wave and iteration.
  // bin(s) > T12  <=>  s >= lo_next,  bin(s) == T12  <=>  lo <= s < lo_next, where lo and lo_next
  // are the smallest scores of bins T12 and T12 + 1 (the key map is monotone and float compares
  // treat -0 and +0 as equal, like the keys); no score lies above bin 4095.
  const float lo = key_to_float(T12 << 20);
  const bool has_next = T12 < (uint32_t)(kHistBins - 1);
  const float lo_next = has_next ? key_to_float((T12 + 1u) << 20) : 0.f;
  auto process_iter = [&](int B) {
    uint32_t eqm[kSelVecUnroll];
#pragma unroll
    for (int u = 0; u < kSelVecUnroll; ++u) {
      eqm[u] = 0u;
      const int nb = B + (u * kSelWaves + wave) * 256;
      if (nb >= vis) continue;
      const int n4 = nb + lane * 4;
      const float vals[4] = {sv[u].x, sv[u].y, sv[u].z, sv[u].w};
      const uint32_t valid = n4 + 3 < vis ? 0xfu : (n4 >= vis ? 0u : (1u << (vis - n4)) - 1u);
      uint32_t gt = 0u;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bool above = has_next && vals[j] >= lo_next;
        gt |= (uint32_t)above << j;
        eqm[u] |= (uint32_t)(!above && vals[j] >= lo) << j;
      }
      gt &= valid;
      eqm[u] &= valid;
      uint32_t word = gt << (4 * (lane & 7));
      word |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)word, 0xB1, 0xf, 0xf, false);
      word |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)word, 0x4E, 0xf, 0xf, false);
      word |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)word, 0x141, 0xf, 0xf, false);
      if ((lane & 7) == 0) gt_bits[(nb >> 5) + (lane >> 3)] = word;
    }
    if (!fast) return;
    // per-lane candidate count over all blocks, wave prefix via ballots of its 5 bits
    uint32_t cnt = 0;
#pragma unroll
    for (int u = 0; u < kSelVecUnroll; ++u) cnt += __popc(eqm[u]);
    uint32_t before = 0, tot = 0;
#pragma unroll
    for (int bit = 0; bit < 6; ++bit) {
      const uint64_t bm = __ballot((cnt >> bit) & 1u);
      before += __builtin_amdgcn_mbcnt_hi((uint32_t)(bm >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bm, 0u)) << bit;
      tot += (uint32_t)__popcll(bm) << bit;
    }
    if (tot == 0) return;
    uint32_t slot0 = 0;
    if (lane == 0) slot0 = atomicAdd(&sh.cand_count, tot);
    uint32_t slot = __shfl(slot0, 0) + before;
#pragma unroll
    for (int u = 0; u < kSelVecUnroll; ++u) {
      if (eqm[u] == 0u) continue;
      const int n4 = B + (u * kSelWaves + wave) * 256 + lane * 4;
      const float vals[4] = {sv[u].x, sv[u].y, sv[u].z, sv[u].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if ((eqm[u] >> j) & 1u) {
          if (slot < (uint32_t)kCandCap) {
            cand_key[slot] = ord_key(vals[j]);
            cand_pos[slot] = (uint32_t)(n4 + j);
          }
          ++slot;
        }
      }
    }
  };
  for (int B = 0; B < vis; B += kSelIter) {
    if (B > 0) load_iter(B);
    process_iter(B);
  }
  __syncthreads();

  // ---- 3. exact threshold key K* inside bin T12 (two 10-bit rounds)
  uint32_t prefix = T12;  // resolved leading bits
  uint32_t cnt_eq = 0;
  for (int round = 0; round < 2; ++round) {
    const int shift = round == 0 ? 10 : 0;
    for (int i = tid; i < 1024; i += kSelThreads) hist_s[i] = 0u;
    __syncthreads();
    if (fast) {
      const uint32_t c = min(sh.cand_count, (uint32_t)kCandCap);
      for (uint32_t i = tid; i < c; i += kSelThreads) {
        const uint32_t key = cand_key[i];
        if ((key >> (shift + 10)) == prefix) atomicAdd(&hist_s[(key >> shift) & 1023u], 1u);
      }
    } else {
      for (int n = tid; n < vis; n += kSelThreads) {
        const uint32_t key = ord_key(srow[n]);
        if ((key >> (shift + 10)) == prefix) atomicAdd(&hist_s[(key >> shift) & 1023u], 1u);
      }
    }
    __syncthreads();
    find_threshold<1>(hist_s, 1024, need, sh);
    prefix = (prefix << 10) | sh.thr_bin;
    need -= sh.thr_above;
    cnt_eq = sh.thr_count;
    __syncthreads();
  }
  const uint32_t kstar = prefix;  // exact key of the kk-th largest score
  const bool take_all_eq = (cnt_eq == need);

  // mark keys of bin T12 that are > K* (and == K*)
  if (fast) {
    const uint32_t c = min(sh.cand_count, (uint32_t)kCandCap);
    for (uint32_t i = tid; i < c; i += kSelThreads) {
      const uint32_t key = cand_key[i];
      const uint32_t p = cand_pos[i];
      if (key > kstar || (key == kstar && take_all_eq))
        atomicOr(&gt_bits[p >> 5], 1u << (p & 31));
      else if (key == kstar)
        atomicOr(&eq_bits[p >> 5], 1u << (p & 31));
    }
  } else {
    for (int nb = wave * 64; nb < vis; nb += kSelThreads) {
      const int n = nb + lane;
      const bool valid = n < vis;
      const uint32_t key = valid ? ord_key(srow[n]) : 0u;
      const bool inbin = valid && (key >> 20) == T12;
      const uint64_t gm = __ballot(inbin && (key > kstar || (key == kstar && take_all_eq)));
      const uint64_t em = __ballot(inbin && key == kstar && !take_all_eq);
      if (lane == 0) {
        gt_bits[nb >> 5] |= (uint32_t)gm;
        gt_bits[(nb >> 5) + 1] |= (uint32_t)(gm >> 32);
        eq_bits[nb >> 5] |= (uint32_t)em;
        eq_bits[(nb >> 5) + 1] |= (uint32_t)(em >> 32);
      }
    }
  }
  __syncthreads();

  emit_selection(l, words, need, take_all_eq, kk, k_max, out, sh);
}

// One workgroup per row (b, t, hq): the min(mult * k', visible) largest scores of the row
// (k' = min(k_b, visible); mult = 1 for the top-k itself), from the scores and histogram of
// score_hist_kernel, into rows of out_stride entries.
__global__ __launch_bounds__(kSelThreads) void select_kernel(
    const float* __restrict__ scores, const uint32_t* __restrict__ hist,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ k_per_req, int T, int Hq,
    int max_len, int64_t score_stride, int k_max, int mult, int out_stride, int bitmap_words,
    int32_t* __restrict__ indices) {
  extern __shared__ uint32_t smem[];
  __shared__ SelShared sh;
  const int row = blockIdx.x;
  const int b = row / (T * Hq);
  const int t = (row / Hq) - (row / (T * Hq)) * T;
  int L = seq_lens[b];
  L = L < 0 ? 0 : (L > max_len ? max_len : L);
  const int vis = max(0, L - T + t + 1);
  int kb = k_per_req ? k_per_req[b] : k_max;
  kb = kb < 0 ? 0 : (kb > k_max ? k_max : kb);
  const int kk = (int)min((int64_t)mult * min(kb, vis), (int64_t)vis);
  int32_t* out = indices + (int64_t)row * out_stride;
  if (kk == vis || kk == 0) {  // everything visible is selected, or nothing
    for (int i = threadIdx.x; i < out_stride; i += kSelThreads) out[i] = i < kk ? i : -1;
    return;
  }
  select_dense_row(scores + (int64_t)row * score_stride, hist + (int64_t)row * kHistBins, vis, kk,
                   out_stride, out, sel_lds(smem, bitmap_words), sh);
}

// ============================================================================ filtered indexer
// Writing every fp32 score and reading it back costs more than the 4 or 16 bytes per position
// suggest (the writes interleave with the K stream), so for k <= N/8 the indexer avoids them:
//  A. sample_tau_kernel scores a strided sample of at most kTauSamples positions per (request,
//     KV head) and sets, per row, a threshold tau: the 16-bit key prefix of the sample's r-th
//     largest score, r from cand_rank (about 2.5 k samples / visible at 50x sparsity);
//  B. score_cand_kernel then scores
//     every position once, as score_hist_kernel does, and keeps only the candidates s >= tau as
//     (score, position) entries, staged in LDS and written a 128-byte line at a time into per-wave
//     slots of the workspace.  A wave scans one contiguous range, so the slots concatenated in
//     (chunk, wave) order list a row's candidates in ascending position order;
//  C. cand_select_kernel selects the k largest candidates by radix select and writes them in that
//     order.  They are the exact top-k whenever there are at least k candidates (then the k-th
//     largest score is >= tau, so every position of the top-k is a candidate) and no slot
//     overflowed; otherwise the workgroup recomputes every score of its row and selects from
//     those (exact, slow, rare).
// The rank r of the threshold among a row's ns_row samples.  About mu = kk * ns_row / vis samples
// fall among the row's kk largest scores; when r or more do, fewer than kk positions reach tau and
// the row falls back.  r = ceil(mu + 4.8 sqrt(mu) + 9.5) keeps that chance below 1e-8 per row for
// every mu (binomial upper tail, 1024 samples of i.i.d. scores) with as few candidates as that
// allows: their lines are the indexer's only writes and cost about 1 TB/s against the K stream.
// It matches 2.5 mu at 50x sparsity (r = 52); a fixed 3 mu with a minimum of 32 measured 2% slower
// on the indexer and 6% on the sketch step at 50x, and wrote more lines than needed at 10x
// (3 mu = 308 where 160 suffice) and 1000x (32 where 16 suffice).
__host__ __device__ inline int64_t cand_rank(int64_t kk, int64_t ns_row, int64_t vis) {
  const float mu = (float)kk * (float)ns_row / (float)vis;
  return (int64_t)ceilf(mu + 4.8f * sqrtf(mu) + 9.5f);
}

// Sampling stride of a request of length L: every stride-th position, at most kTauSamples.
__device__ __forceinline__ int tau_stride(int L) { return L > kTauSamples ? (L + kTauSamples - 1) / kTauSamples : 1; }

// Candidate slots: wave w of workgroup (chunk c) of row `row` scans the positions
// [c * chunk + w * chunk / kCandWaves, + chunk / kCandWaves) and owns slot s = c * kCandWaves + w
// of the row's workspace area: up to cand_cap(chunk) candidates in 128-byte lines of
// kLinePairs = 20 -- words 0..19 their float32 scores, words 20..29 their positions as 16-bit
// offsets from the slot's first position (a slot spans at most 4096), words 30..31 unused; 20
// candidates in 128 bytes instead of 16 (position, score) pairs, since these lines are the
// indexer's only writes and cost far more per byte than the K stream (measured: 1-2% faster
// indexer calls, less than the bytes suggested).  Lines are interleaved
// across the row's nsub = chunks * kCandWaves slots -- line l of slot s is line l * nsub + s of
// the area -- so the first lines of all slots, the ones most written, lie together.
constexpr int kCandWaves = 4;
constexpr int kLinePairs = 20;

// Byte offset, in a staging ring of 2 * kLinePairs entries (scores, then 16-bit offsets), of 8-byte
// part p (0..15) of the line whose first entry is hd (0 or kLinePairs): parts 0..9 hold scores
// hd + 2p, hd + 2p + 1; parts 10..14 offsets hd + 4 (p - 10) .. + 3; part 15 is unused and reads
// the last four offsets of the line again.
__device__ __forceinline__ uint32_t line_part_8(uint32_t hd, uint32_t p) {
  constexpr uint32_t kOffsets = 2 * kLinePairs * 4;  // byte offset of the ring's 16-bit offsets
  return p < 10u ? (hd + 2u * p) * 4u : kOffsets + (hd + 4u * (p < 15u ? p - 10u : 4u)) * 2u;
}
__host__ __device__ constexpr int cand_cap(int chunk) {
  return chunk / (2 * kCandWaves) / kLinePairs * kLinePairs;
}

// tau of one row from its sample keys (one wave): the largest 16-bit prefix P with at least r
// keys >= P << 16, r = cand_rank(kk, samples_visible, vis); -inf when every visible position has
// to be a candidate, +inf when the selection needs none (k = 0 or k >= visible).  The fraction of
// the row scoring >= tau then has mean about r / samples and relative spread about 1 / sqrt(r).

// The search for P on the 16-bit key prefixes of NR rows' samples, 16 per lane and row in any
// order (0 for a sample the row does not see), for ranks rr; the rows' searches are interleaved
// so that their wave sums overlap.
template <int NR>
__device__ void search_prefixes(const uint32_t (&k16)[NR][kTauSamples / kWave], const int (&rr)[NR],
                                uint32_t (&P)[NR]) {
#pragma unroll
  for (int x = 0; x < NR; ++x) P[x] = 0;
  for (int bit = 15; bit >= 0; --bit) {
    uint32_t c[NR];
#pragma unroll
    for (int x = 0; x < NR; ++x) {
      const uint32_t cand = P[x] | (1u << bit);
      c[x] = 0;
#pragma unroll
      for (int e = 0; e < kTauSamples / kWave; ++e) c[x] += k16[x][e] >= cand ? 1u : 0u;
    }
#pragma unroll
    for (int x = 0; x < NR; ++x) c[x] = wave_sum_u32(c[x]);
#pragma unroll
    for (int x = 0; x < NR; ++x)
      if (c[x] >= (uint32_t)rr[x]) P[x] |= 1u << bit;
  }
}

// The rank r of a row's threshold, or 0 when the row needs no rank search (tau = *special).
__device__ __forceinline__ int tau_rank(int vis, int kk, int stride, float* special) {
  if (kk <= 0 || kk >= vis) {
    *special = INFINITY;
    return 0;
  }
  const int ns_row = (vis + stride - 1) / stride;
  const int64_t rr = cand_rank(kk, ns_row, vis);
  if (rr >= ns_row) {
    *special = -INFINITY;
    return 0;
  }
  return (int)rr;
}

// tau of a row whose sample keys (32-bit, kTauSamples of them) lie in LDS.
__device__ float row_tau(const uint32_t* __restrict__ krow, int vis, int kk, int stride) {
  const int lane = threadIdx.x & 63;
  float special;
  const int rr = tau_rank(vis, kk, stride, &special);
  if (rr == 0) return special;
  uint32_t k16[1][kTauSamples / kWave];
#pragma unroll
  for (int e = 0; e < kTauSamples / kWave / 4; ++e) {
    const uint4 v = reinterpret_cast<const uint4*>(krow)[e * kWave + lane];
    k16[0][4 * e] = v.x >> 16;
    k16[0][4 * e + 1] = v.y >> 16;
    k16[0][4 * e + 2] = v.z >> 16;
    k16[0][4 * e + 3] = v.w >> 16;
  }
  const int rrs[1] = {rr};
  uint32_t P[1];
  search_prefixes<1>(k16, rrs, P);
  return key_to_float(P[0] << 16);
}

// A lane's share of a row's sample key prefixes (16-bit, kTauSamples of them, 16-byte aligned) as
// a split sample pass leaves them in global memory: 16 prefixes in two 16-byte words.
__device__ __forceinline__ void load_prefixes(const uint16_t* __restrict__ krow, uint4 (&w)[2]) {
  const int lane = threadIdx.x & 63;
  w[0] = reinterpret_cast<const uint4*>(krow)[lane];
  w[1] = reinterpret_cast<const uint4*>(krow)[kWave + lane];
}

// The 16 prefixes of two words from load_prefixes, one per entry.
__device__ __forceinline__ void unpack_prefixes(const uint4 (&pw)[2], uint32_t (&k16)[kTauSamples / kWave]) {
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const uint32_t w[4] = {pw[e].x, pw[e].y, pw[e].z, pw[e].w};
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      k16[8 * e + 2 * x] = w[x] & 0xffffu;
      k16[8 * e + 2 * x + 1] = w[x] >> 16;
    }
  }
}

// The whole selection of one row whose every position has its key in krow (one wave; krow 16-byte
// aligned, kTauSamples keys, 0 for a position not visible to the row, every visible key >= 1):
// the kk largest keys (lower position first among equal keys) as ascending positions into out,
// padded with -1 to k_max.  The kk-th largest key is found bit by bit with DPP wave sums.
__device__ void row_select_all(const uint32_t* __restrict__ krow, int vis, int kk, int k_max,
                               int32_t* __restrict__ out) {
  constexpr int PER = kTauSamples / kWave;  // keys per lane: positions e * 64 + lane
  const int lane = threadIdx.x & 63;
  kk = kk < 0 ? 0 : (kk > vis ? vis : kk);
  if (kk > 0 && kk < vis) {
    uint32_t key[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) key[e] = krow[e * kWave + lane];
    uint32_t P = 0;  // the largest P with at least kk keys >= P: the kk-th largest key
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t cand = P | (1u << bit);
      uint32_t c = 0;
#pragma unroll
      for (int e = 0; e < PER; ++e) c += key[e] >= cand ? 1u : 0u;
      if (wave_sum_u32(c) >= (uint32_t)kk) P = cand;
    }
    uint32_t gt = 0;
#pragma unroll
    for (int e = 0; e < PER; ++e) gt += key[e] > P ? 1u : 0u;
    const uint32_t need = (uint32_t)kk - wave_sum_u32(gt);  // keys equal to P that are taken
    uint32_t eq_base = 0, out_base = 0;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const bool is_eq = key[e] == P;
      const uint64_t eqb = __ballot(is_eq);
      const uint32_t eq_rank =
          eq_base + __builtin_amdgcn_mbcnt_hi((uint32_t)(eqb >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)eqb, 0u));
      const bool sel = key[e] > P || (is_eq && eq_rank < need);
      const uint64_t sb = __ballot(sel);
      const uint32_t o =
          out_base + __builtin_amdgcn_mbcnt_hi((uint32_t)(sb >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)sb, 0u));
      if (sel) out[o] = e * kWave + lane;
      eq_base += (uint32_t)__popcll(eqb);
      out_base += (uint32_t)__popcll(sb);
    }
  } else {
    for (int i = lane; i < kk; i += kWave) out[i] = i;  // none, or every visible position
  }
  for (int i = kk + lane; i < k_max; i += kWave) out[i] = -1;
}

// SK: this lane's A operand of query row qrow -- the 16 values j * 64 + g4 * 16 .. + 16 of each
// k-step j -- as int8 codes, quantised as the key sketch is: the row's maximum comes from the four
// lanes m, m + 16, m + 32, m + 48 that hold it, scale = max / 127 and code = rint(x / scale),
// both divisions correctly rounded, clamped to +-127; an invalid row gives zeros.  Returns the
// row's scale.
template <int D>
__device__ __forceinline__ float quantize_q_operand(const uint16_t* __restrict__ qrow, bool valid, int g4,
                                                    uint4 (&a)[D / 64]) {
  constexpr int KS = D / 64;
  float x[KS][16];
#pragma unroll
  for (int j = 0; j < KS; ++j) {
    const uint4 lo = valid ? ld16(qrow + j * 64 + g4 * 16) : make_uint4(0, 0, 0, 0);
    const uint4 hi = valid ? ld16(qrow + j * 64 + g4 * 16 + 8) : make_uint4(0, 0, 0, 0);
    float f[8];
    unpack8(lo, f);
#pragma unroll
    for (int e = 0; e < 8; ++e) x[j][e] = f[e];
    unpack8(hi, f);
#pragma unroll
    for (int e = 0; e < 8; ++e) x[j][8 + e] = f[e];
  }
  float mx = 0.f;
#pragma unroll
  for (int j = 0; j < KS; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) mx = fmaxf(mx, fabsf(x[j][e]));
  mx = fmaxf(mx, __shfl_xor(mx, 16));
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  const float scale = __fdiv_rn(mx, 127.f);
#pragma unroll
  for (int j = 0; j < KS; ++j) {
    uint32_t w[4] = {0u, 0u, 0u, 0u};
    if (scale > 0.f) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float c = fminf(fmaxf(rintf(__fdiv_rn(x[j][e], scale)), -127.f), 127.f);
        w[e >> 2] |= ((uint32_t)(int)c & 0xffu) << (8 * (e & 3));
      }
    }
    a[j] = make_uint4(w[0], w[1], w[2], w[3]);
  }
  return scale;
}

// A and the thresholds in one workgroup per (request, KV head, 16-row tile): kSampleWaves waves
// score the kTauSamples sampled positions (sample j = 64 w + 16 u + m of wave w, tile u, lane
// row m, at position j * stride; loads clamped to the last sample) against the tile's query rows
// on MFMA and keep the samples' ordered keys in LDS (0 marks "not visible to this row"; every
// finite score has a larger key); then wave w sets tau of the tile's row w with row_tau.
// SK: sketch scores (int8 codes of q and K), and tau for the row's min(cand_mult * k', visible)
// largest of them; the workgroup also quantises its query rows and stores their codes and scales
// for the later passes.
// EXACT (every request at most kTauSamples long, so stride 1 and the sample is the whole row):
// wave w selects row w's top-k from the keys itself (row_select_all) into `indices` instead of
// setting tau, and with `scores` keeps every visible score at scores[row * score_stride + n].
// SPLIT > 1: SPLIT workgroups (blockIdx.z) share a tile's samples, a quarter or half each, and
// store the samples' 16-bit key prefixes at prefixes[row * kTauSamples + j] instead of setting tau;
// the candidate pass then sets tau from them.  With EXACT they store the whole 32-bit keys
// (prefixes read as uint32_t) and small_select_kernel selects.  A sample pass is bound by the sampled rows one
// compute unit has in flight, so spreading a tile over several units shortens it when there are
// fewer tiles than units.
constexpr int kSampleWaves = kTauSamples / 64;  // 16
template <int D, bool PAGED, bool SK, bool EXACT, int SPLIT>
__global__ __launch_bounds__(kSampleWaves * kWave) void sample_tau_kernel(
    const uint16_t* __restrict__ q, KVArgs kv, SketchArgs sk, int T, int Hq, int G, float scale,
    const int32_t* __restrict__ k_per_req, int k_max, int cand_mult, float* __restrict__ tau,
    int32_t* __restrict__ indices, float* __restrict__ scores, int64_t score_stride,
    uint16_t* __restrict__ prefixes) {
  static_assert(SPLIT == 1 || SPLIT == 2 || SPLIT == 4, "a tile's samples split into 1, 2 or 4 parts");
  extern __shared__ uint32_t lkeys[];  // [16][kTauSamples] (SPLIT == 1)
  constexpr int KS = SK ? D / 64 : D / 32;  // 16-byte operand steps per lane
  constexpr int kTiles = 4 / SPLIT;         // 16-sample tiles per wave
  const int bh = blockIdx.x;
  const int mt = blockIdx.y;
  const int Hkv = kv.num_kv_heads;
  const int b = bh / Hkv, h = bh - (bh / Hkv) * Hkv;
  const int GT = G * T;
  const int r0 = mt * 16;
  const int rows_here = min(16, GT - r0);
  const int L = seq_len_of(kv, b);
  const int stride = tau_stride(L);
  const int ns = (L + stride - 1) / stride;  // samples j * stride < L
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int m = lane & 15;
  const int g4 = lane >> 4;
  // the request's k, read now so that its latency overlaps the sample loads
  const int k_req = k_per_req ? k_per_req[b] : k_max;

  uint4 a[KS];
  float my_qsc = 0.f;  // SK: scale of query row r0 + m
  {
    const int r = r0 + m;
    const int t = r / G, gi = r - (r / G) * G;
    const int64_t qr = ((int64_t)b * T + t) * Hq + (h * G + gi);
    if constexpr (SK) {
      my_qsc = quantize_q_operand<D>(q + (r < GT ? qr : 0) * D, r < GT, g4, a);
      if (r < GT && wave == 0 && blockIdx.z == 0) {
#pragma unroll
        for (int j = 0; j < KS; ++j) *reinterpret_cast<uint4*>(sk.q_codes + qr * D + g4 * 16 + j * 64) = a[j];
        if (g4 == 0) sk.q_scales[qr] = my_qsc;
      }
    } else if (r < GT) {
#pragma unroll
      for (int j = 0; j < KS; ++j) a[j] = ld16(q + qr * D + g4 * 8 + j * 32);
    } else {
#pragma unroll
      for (int j = 0; j < KS; ++j) a[j] = make_uint4(0, 0, 0, 0);
    }
  }
  const int j0 = (int)blockIdx.z * (kTauSamples / SPLIT) + 16 * kTiles * wave;
  uint4 kt[kTiles][KS];
  float ksc[kTiles];  // SK: the sampled rows' scales
  const int jlast = max(ns - 1, 0);
#pragma unroll
  for (int u = 0; u < kTiles; ++u) {
    const int j = min(j0 + 16 * u + m, jlast);
    ksc[u] = 0.f;
    if (L > 0) {
      const int64_t off = kv_row<D, PAGED>(kv, b, h, j * stride);
#pragma unroll
      for (int kq = 0; kq < KS; ++kq)
        kt[u][kq] = SK ? ld16i8(sk.codes + off + g4 * 16 + kq * 64) : ld16(kv.k + off + g4 * 8 + kq * 32);
      if constexpr (SK) ksc[u] = sk.scales[off / D];
    } else {
#pragma unroll
      for (int kq = 0; kq < KS; ++kq) kt[u][kq] = make_uint4(0, 0, 0, 0);
    }
  }
  int vis_i[4];
  float qsc[4];  // SK: scales of this lane's output rows
  int64_t grow_i[4];  // EXACT: the rows' indices
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rl = 4 * g4 + i;
    const int r = r0 + rl;
    const int t = r / G, gi = r - (r / G) * G;
    vis_i[i] = rl < rows_here ? L - T + t + 1 : 0;
    qsc[i] = SK ? __shfl(my_qsc, rl) : 0.f;  // lane rl holds row r0 + rl's scale
    grow_i[i] = ((int64_t)b * T + t) * Hq + (h * G + gi);
  }
#pragma unroll
  for (int u = 0; u < kTiles; ++u) {
    float sc[4];
    tile_scores<SK, KS>(a, kt[u], scale, qsc, ksc[u], sc);
    const int j = j0 + 16 * u + m;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool ok = j < ns && j * stride < vis_i[i];
      const uint32_t key = ok ? max(ord_key(sc[i]), 1u) : 0u;
      if constexpr (SPLIT == 1) {
        lkeys[(4 * g4 + i) * kTauSamples + j] = key;
      } else if (4 * g4 + i < rows_here) {
        if constexpr (EXACT)
          reinterpret_cast<uint32_t*>(prefixes)[grow_i[i] * kTauSamples + j] = key;
        else
          prefixes[grow_i[i] * kTauSamples + j] = (uint16_t)(key >> 16);
      }
      if constexpr (EXACT) {  // every position is sampled (stride 1): keep the score for the step
        if (ok && scores) scores[grow_i[i] * score_stride + j] = sc[i];
      }
    }
  }
  if constexpr (SPLIT > 1) return;
  __syncthreads();
  if (wave < rows_here) {
    const int r = r0 + wave;
    const int t = r / G, gi = r - (r / G) * G;
    const int vis = L - T + t + 1;
    const int kb = k_req < 0 ? 0 : (k_req > k_max ? k_max : k_req);
    const int kk = min(kb, max(vis, 0));
    const int keep = SK ? (int)min((int64_t)cand_mult * kk, (int64_t)max(vis, 0)) : kk;
    const int64_t grow = ((int64_t)b * T + t) * Hq + (h * G + gi);
    if constexpr (EXACT) {
      row_select_all(lkeys + wave * kTauSamples, max(vis, 0), kk, k_max, indices + grow * k_max);
    } else {
      const float th = row_tau(lkeys + wave * kTauSamples, vis, keep, stride);
      if (lane == 0) tau[grow] = th;
    }
  }
}

// Row mapping of the candidate pass: query row r of a 16-row tile sits in MFMA row
// 4 * (r % 4) + r / 4, so lane group g4 (lanes 16 g4 .. 16 g4 + 15) holds rows 4 i + g4 for
// i = 0..3 and, with 4 or 8 query rows, every lane group holds valid rows for the same i.
//
// SK (reduced-byte indexer): positions are scored on the sketch, and each row keeps the
// candidates for its min(cand_mult * k, visible) largest sketch scores.
// PREFIX (after a split sample pass): the workgroup sets its rows' thresholds itself from the
// sample key prefixes, wave w those of rows w, w + 4, ..., instead of reading tau.
template <int D, bool PAGED, int NI, bool SK, bool PREFIX>
__global__ __launch_bounds__(kCandWaves * kWave) void score_cand_kernel(
    const uint16_t* __restrict__ q, KVArgs kv, SketchArgs sk, int T, int Hq, int G, float scale,
    const float* __restrict__ tau, const uint16_t* __restrict__ prefixes,
    const int32_t* __restrict__ k_per_req, int k_max, int cand_mult, float* __restrict__ region,
    int64_t score_stride, uint32_t* __restrict__ counts, int chunk, int chunks) {
  extern __shared__ int lds_pages[];
  // per wave and row: a ring of kRing staged candidates, their scores (4 bytes each) then their
  // slot offsets (2 bytes each), so that a line's 20 scores and 20 offsets lie together
  constexpr int kRing = 2 * kLinePairs;
  __shared__ __align__(16) unsigned char stage[kCandWaves][16][kRing * 6];
  __shared__ float tau_sh[16];                                 // PREFIX: the tile's thresholds
  constexpr int KS = SK ? D / 64 : D / 32;  // 16-byte operand steps per lane
  constexpr int UNR = kScoreUnroll;  // tiles per step (twice as many for the sketch measured no faster)
  const int bh = blockIdx.y;
  const int c = rotated_chunk(blockIdx.x, bh, gridDim.x);
  const int mt = blockIdx.z;
  const int Hkv = kv.num_kv_heads;
  const int b = bh / Hkv, h = bh - (bh / Hkv) * Hkv;
  const int GT = G * T;
  const int r0 = mt * 16;
  const int rows_here = min(16, GT - r0);
  const int L = seq_len_of(kv, b);
  const int start = c * chunk;
  if (start >= L) return;
  const int end = min(start + chunk, L);
  if constexpr (PAGED) stage_pages(kv, b, start, end, lds_pages);

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int m = lane & 15;
  const int g4 = lane >> 4;
  const int cap = cand_cap(chunk);
  const int span = chunk / kCandWaves;
  const int wbeg = start + wave * span;
  const int wend = min(wbeg + span, end);

  uint4 a[KS];
  {
    const int rl = 4 * (m & 3) + (m >> 2);  // query row of MFMA row m
    const int r = r0 + rl;
    if (rl < rows_here) {
      const int t = r / G, gi = r - (r / G) * G;
      const int64_t qr = ((int64_t)b * T + t) * Hq + (h * G + gi);
#pragma unroll
      for (int j = 0; j < KS; ++j)
        a[j] = SK ? ld16i8(sk.q_codes + qr * D + g4 * 16 + j * 64) : ld16(q + qr * D + g4 * 8 + j * 32);
    } else {
#pragma unroll
      for (int j = 0; j < KS; ++j) a[j] = make_uint4(0, 0, 0, 0);
    }
  }
  __syncthreads();  // page ids
  // UNR adjacent 16-position tiles per iteration; the next iteration's K loads while this one
  // is scored (ping-pong, unconditional loads clamped to the range's last tile; a wave with no
  // range loads the chunk's first tile)
  constexpr int kStep = 16 * UNR;
  const int last = wend > wbeg ? (wend - 1) & ~15 : (PREFIX ? start : wbeg);
  uint4 cur[UNR][KS], nxt[UNR][KS];
  float csc[UNR], nsc[UNR];  // SK: the tiles' key scales (this lane's position)
  auto load_tiles = [&](int n0, uint4 (&dst)[UNR][KS], float (&dsc)[UNR]) {
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int tile = min(n0 + u * 16, last);
      const int64_t off = kv_tile_staged<D, PAGED>(kv, lds_pages, start, b, h, tile) +
                          (int64_t)min(m, L - 1 - tile) * D;
#pragma unroll
      for (int j = 0; j < KS; ++j)
        dst[u][j] = SK ? ld16i8(sk.codes + off + g4 * 16 + j * 64) : ld16(kv.k + off + g4 * 8 + j * 32);
      dsc[u] = SK ? sk.scales[off / D] : 0.f;
    }
  };
  // PREFIX: wave w sets the thresholds of rows w + 4 x (x < NI, as rows <= 4 NI).  Their
  // prefixes load first, then the first tiles (every wave, unconditionally: a wave with no range
  // loads the chunk's first tile, so no branch precedes the loop), and the searches run while
  // the tiles are in flight.
  if constexpr (PREFIX) {
    uint4 pref[NI][2];
#pragma unroll
    for (int x = 0; x < NI; ++x) {
      const int r = r0 + wave + kCandWaves * x;
      const int t = r / G, gi = r - (r / G) * G;
      if (wave + kCandWaves * x < rows_here) {
        load_prefixes(prefixes + (((int64_t)b * T + t) * Hq + (h * G + gi)) * kTauSamples, pref[x]);
      } else {
        pref[x][0] = pref[x][1] = make_uint4(0, 0, 0, 0);
      }
    }
    load_tiles(wbeg, cur, csc);
    const int k_req = k_per_req ? k_per_req[b] : k_max;
    const int kb = k_req < 0 ? 0 : (k_req > k_max ? k_max : k_req);
    const int stride = tau_stride(L);
    int rr[NI];
    float special[NI];
    uint32_t k16[NI][kTauSamples / kWave];
#pragma unroll
    for (int x = 0; x < NI; ++x) {
      const int t = (r0 + wave + kCandWaves * x) / G;
      const int vis = L - T + t + 1;
      const int kk = min(kb, max(vis, 0));
      const int keep = SK ? (int)min((int64_t)cand_mult * kk, (int64_t)max(vis, 0)) : kk;
      rr[x] = tau_rank(vis, keep, stride, &special[x]);
      unpack_prefixes(pref[x], k16[x]);
    }
    uint32_t P[NI];
    search_prefixes<NI>(k16, rr, P);
#pragma unroll
    for (int x = 0; x < NI; ++x) {
      const int rl = wave + kCandWaves * x;
      if (rl < rows_here && lane == 0) tau_sh[rl] = rr[x] ? key_to_float(P[x] << 16) : special[x];
    }
    lds_barrier();
  }
  // Candidate lines are written with buffer stores through one resource spanning this
  // workgroup's rows; a lane with nothing to write passes an offset past the resource, which
  // the hardware drops.  Every tile thus issues the same stores with no branch around them, and
  // the compiler keeps the K prefetch in flight across loop iterations.
  int64_t row_lo, row_hi;
  {
    const int t0 = r0 / G, t1 = (r0 + rows_here - 1) / G;
    row_lo = ((int64_t)b * T + t0) * Hq + (h * G + r0 - t0 * G);
    row_hi = ((int64_t)b * T + t1) * Hq + (h * G + (r0 + rows_here - 1) - t1 * G);
  }
  // (base and size pass through readfirstlane: they are workgroup-uniform, and the compiler
  // otherwise may keep the descriptor in vector registers and wrap every store in a loop over
  // its distinct values)
  const uint64_t out_addr = reinterpret_cast<uint64_t>(region + row_lo * score_stride);
  const uint64_t out_base = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(out_addr >> 32)) << 32) |
                            (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)out_addr);
  const int out_bytes = __builtin_amdgcn_readfirstlane((int)((row_hi - row_lo + 1) * score_stride * 4));
  const __amdgpu_buffer_rsrc_t out_rsrc =
      __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<float*>(out_base), (short)0, out_bytes, 0x00020000);
  constexpr uint32_t kDrop = 0xfffffff0u;
  const uint32_t line_stride = (uint32_t)chunks * kCandWaves * 128u;  // bytes from line l to l + 1 of a slot
  // rows 4 i + g4 (i < NI = ceil(rows / 4), fixed at compile time) of this lane: visibility,
  // threshold, byte offset of the slot; ring head, staged count, written count
  int vis[4];
  float th[4];
  float qsc[4];  // SK: the rows' scales
  uint32_t slot[4];
  int64_t grow[4];
  bool valid[4];
  uint32_t head[4] = {0u, 0u, 0u, 0u}, fill[4] = {0u, 0u, 0u, 0u}, done[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rl = 4 * i + g4;
    const int r = r0 + rl;
    valid[i] = rl < rows_here;
    if (valid[i]) {
      const int t = r / G, gi = r - (r / G) * G;
      grow[i] = ((int64_t)b * T + t) * Hq + (h * G + gi);
      vis[i] = L - T + t + 1;
      th[i] = PREFIX ? tau_sh[rl] : tau[grow[i]];
      qsc[i] = SK ? sk.q_scales[grow[i]] : 0.f;
    } else {
      grow[i] = 0;
      vis[i] = 0;
      th[i] = INFINITY;
      qsc[i] = 0.f;
    }
    slot[i] = (uint32_t)(((valid[i] ? grow[i] - row_lo : 0) * score_stride) * 4 +
                         (int64_t)(c * kCandWaves + wave) * 128);
  }

  // Per tile and row: candidates s >= tau join the row's 32-entry LDS ring; once it holds 16, the
  // 16 from its head are written as one 128-byte line.
  // Tiles past the range (the second of a pair at the end) are scored on reloaded data and
  // keep nothing, so every iteration runs the same instructions.
  auto score_tiles = [&](int n0, const uint4 (&kt)[UNR][KS], const float (&ksc)[UNR]) {
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int tile = n0 + u * 16;
      float sc[4];
      tile_scores<SK, KS>(a, kt[u], scale, qsc, ksc[u], sc);
      const int n = tile + m;
      const bool in_range = n < wend;
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        unsigned char* st = stage[wave][4 * i + g4];
        const float s = sc[i];
        const bool pred = in_range && n < vis[i] && s >= th[i];
        const uint64_t mask = __ballot(pred);
        const uint32_t seg = (uint32_t)(mask >> (16 * g4)) & 0xffffu;
        if (pred) {
          // head + fill <= 39 and the rank < 16: one wrap at most
          uint32_t e = head[i] + fill[i] + __popc(seg & ((1u << m) - 1u));
          e = e >= (uint32_t)kRing ? e - kRing : e;
          *reinterpret_cast<float*>(st + e * 4) = s;
          *reinterpret_cast<uint16_t*>(st + kRing * 4 + e * 2) = (uint16_t)(n - wbeg);
        }
        fill[i] += __popc(seg);
        if constexpr (NI == 1) {
          wave_lds_fence();
          const uint2 v = *reinterpret_cast<const uint2*>(st + line_part_8(head[i], (uint32_t)m));
          const bool full = fill[i] >= (uint32_t)kLinePairs;
          const bool write = full && valid[i] && done[i] + kLinePairs <= (uint32_t)cap;
          __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(v2u32, v), out_rsrc,
                                                (int)(write ? slot[i] + (done[i] / kLinePairs) * line_stride + m * 8u : kDrop), 0, 0);
        }
      }
      if constexpr (NI >= 2) {
        // rows 4 i + g4 and 4 (i + 1) + g4 share one 16-byte store per lane: lanes 8 h .. 8 h + 7
        // of lane group g4 write the line of row 4 (i + h) + g4, 16 bytes (two 8-byte parts) each
        wave_lds_fence();
        const uint32_t h = (uint32_t)(m >> 3) & 1u, j = (uint32_t)m & 7u;
#pragma unroll
        for (int i = 0; i < NI; i += 2) {
          const uint32_t hd = h ? head[i + 1] : head[i];
          const uint32_t fl = h ? fill[i + 1] : fill[i];
          const uint32_t dn = h ? done[i + 1] : done[i];
          const uint32_t sl = h ? slot[i + 1] : slot[i];
          const bool vd = h ? valid[i + 1] : valid[i];
          const unsigned char* st = stage[wave][4 * (i + (int)h) + g4];
          const uint2 lo = *reinterpret_cast<const uint2*>(st + line_part_8(hd, 2u * j));
          const uint2 hi = *reinterpret_cast<const uint2*>(st + line_part_8(hd, 2u * j + 1u));
          const uint4 v = make_uint4(lo.x, lo.y, hi.x, hi.y);
          const bool write = fl >= (uint32_t)kLinePairs && vd && dn + kLinePairs <= (uint32_t)cap;
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u32, v), out_rsrc,
                                                 (int)(write ? sl + (dn / kLinePairs) * line_stride + j * 16u : kDrop), 0, 0);
        }
      }
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const bool full = fill[i] >= (uint32_t)kLinePairs;
        head[i] = full ? (uint32_t)kLinePairs - head[i] : head[i];  // 0 <-> 20
        done[i] += full ? (uint32_t)kLinePairs : 0u;
        fill[i] -= full ? (uint32_t)kLinePairs : 0u;
      }
    }
  };
  if (wbeg < wend) {
    int n0 = wbeg;
    if constexpr (!PREFIX) load_tiles(n0, cur, csc);
    do {
      load_tiles(n0 + kStep, nxt, nsc);
      score_tiles(n0, cur, csc);
      load_tiles(n0 + 2 * kStep, cur, csc);
      score_tiles(n0 + kStep, nxt, nsc);
      n0 += 2 * kStep;
    } while (n0 < wend);
  }
  // the last, partial line of each row (its count says how many entries are valid)
  wave_lds_fence();
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const uint2 v = *reinterpret_cast<const uint2*>(stage[wave][4 * i + g4] + line_part_8(head[i], (uint32_t)m));
    const bool write = valid[i] && fill[i] > 0u && done[i] < (uint32_t)cap;
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(v2u32, v), out_rsrc,
                                          (int)(write ? slot[i] + (done[i] / kLinePairs) * line_stride + m * 8u : kDrop), 0, 0);
    if (valid[i] && m == 0) counts[(grow[i] * chunks + c) * kCandWaves + wave] = done[i] + fill[i];
  }
}

// ---- C: selection over a position-ordered list of (position, key) items
constexpr int kCsThreads = 512;
constexpr int kCsWaves = kCsThreads / kWave;
constexpr int kMaxCandSlots = (262144 / 1024) * kCandWaves;  // chunks of >= 1024 positions
constexpr int kCsPer = 8;  // consecutive items per thread in the ordered passes
constexpr int kFallbackUnroll = 8;  // key rows per lane group in flight when a row is rescored whole

// Candidates of a row in position order, from the slots: item f lives in the slot s with
// prefix[s] <= f < prefix[s + 1], as entry j = f - prefix[s] of it.  Keys come from LDS when
// lds_key is set.
struct CandSource {
  const uint32_t* base;    // the row's slot area, as 32-bit words
  const uint32_t* prefix;  // [nsub + 1] exclusive prefix of the slot counts (LDS)
  int nsub, cap;
  int nsub_all;            // slots of a row (chunks * kCandWaves): the line interleave
  int span;                // positions per slot (chunk / kCandWaves): slot s starts at s * span
  const uint32_t* lds_key;
  // first word of the line holding entry j of slot sl (lines interleaved across nsub_all slots)
  __device__ __forceinline__ int64_t line_word(int sl, int j) const {
    return ((int64_t)(j / kLinePairs) * nsub_all + sl) * 32;
  }
  __device__ __forceinline__ int slot_of(int f) const {
    int lo = 0, hi = nsub - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if ((int)prefix[mid] <= f) lo = mid; else hi = mid - 1;
    }
    return lo;
  }
  // items f0 .. f0 + kCsPer - 1 (the valid ones, f < total; others 0): the word index of each
  // score, the 16-bit index of each offset and the first position of each slot
  __device__ __forceinline__ void locate(int f0, int total, int64_t (&sw)[kCsPer], int64_t (&ow)[kCsPer],
                                         int (&first)[kCsPer]) const {
    int sl = f0 < total ? slot_of(f0) : 0;
#pragma unroll
    for (int e = 0; e < kCsPer; ++e) {
      const int f = f0 + e;
      if (f < total) {
        while ((int)prefix[sl + 1] <= f) ++sl;
        const int j = f - (int)prefix[sl];
        const int64_t lw = line_word(sl, j);
        sw[e] = lw + j % kLinePairs;
        ow[e] = (lw + kLinePairs) * 2 + j % kLinePairs;
        first[e] = sl * span;
      } else {
        sw[e] = 0;
        ow[e] = 0;
        first[e] = 0;
      }
    }
  }
  __device__ __forceinline__ uint32_t key(int f) const {
    if (lds_key) return lds_key[f];
    const int sl = slot_of(f);
    const int j = f - (int)prefix[sl];
    return ord_key(__uint_as_float(base[line_word(sl, j) + j % kLinePairs]));
  }
  __device__ __forceinline__ void pos8(int f0, int total, uint32_t sel, uint32_t (&p)[kCsPer]) const {
    int64_t sw[kCsPer], ow[kCsPer];
    int first[kCsPer];
    locate(f0, total, sw, ow, first);
    const uint16_t* off16 = reinterpret_cast<const uint16_t*>(base);
#pragma unroll
    for (int e = 0; e < kCsPer; ++e) p[e] = ((sel >> e) & 1u) ? (uint32_t)first[e] + off16[ow[e]] : 0u;
  }
};

// Every score of a row (the exact fallback), position = index.
struct DenseSource {
  const float* s;
  __device__ __forceinline__ uint32_t key(int f) const { return ord_key(s[f]); }
  __device__ __forceinline__ void pos8(int f0, int, uint32_t, uint32_t (&p)[kCsPer]) const {
#pragma unroll
    for (int e = 0; e < kCsPer; ++e) p[e] = (uint32_t)(f0 + e);
  }
};

// Candidate blocks of kCsThreads * kCsPer held in LDS with their positions in registers: MB =
// kCsBlocks, or kCsBlocksBig for long lists (more registers, fewer workgroups per CU).
constexpr int kCsBlocks = 3;
constexpr int kCsBlocksBig = 6;

// Finds the kk-th largest key of the list (kmin <= every key <= kmax) by radix select over the
// bits below their common prefix, in digits of up to 11 bits.  hist holds two areas of 2048
// counters used in turn: the next digit's area is cleared while this digit is counted, so a digit
// costs three barriers (after the counts, and the two of find_threshold).
// Returns the key and sets need (items equal to it that are taken) and cnt_eq (items equal to it).
template <class KeyAt>
__device__ uint32_t radix_kth(KeyAt key_at, int total, int kk, uint32_t kmin, uint32_t kmax,
                              uint32_t* hist, SelShared& sh, uint32_t& need, uint32_t& cnt_eq) {
  const int tid = threadIdx.x;
  need = (uint32_t)kk;
  cnt_eq = (uint32_t)total;
  if (kmin == kmax) return kmin;  // one key value
  int lo = 32 - __clz(kmin ^ kmax);  // bits [0, lo) vary
  uint32_t prefix = lo >= 32 ? 0u : kmin >> lo;
  for (int i = tid; i < 2048; i += kCsThreads) hist[i] = 0u;
  __syncthreads();
  int area = 0;
  while (lo > 0) {
    const int width = lo >= 11 ? 11 : lo;
    const int shift = lo - width;
    const int nb = 1 << width;
    uint32_t* h = hist + area * 2048;
    // the other area was last read by the previous digit's find_threshold, which ended in a barrier
    if (shift > 0) {
      uint32_t* next = hist + (area ^ 1) * 2048;
      for (int i = tid; i < 2048; i += kCsThreads) next[i] = 0u;
    }
    for (int f = tid; f < total; f += kCsThreads) {
      const uint32_t key = key_at(f);
      if (lo >= 32 || (key >> lo) == prefix) atomicAdd(&h[(key >> shift) & (uint32_t)(nb - 1)], 1u);
    }
    __syncthreads();
    // bins at and above nb count nothing: they were cleared and no key maps there
    find_threshold<2048 / kCsThreads, kCsWaves>(h, 2048, need, sh);
    // sh.thr_* are read here, before this thread reaches the next digit's first barrier, and
    // written again only after it
    prefix = (prefix << width) | sh.thr_bin;
    need -= sh.thr_above;
    cnt_eq = sh.thr_count;
    lo = shift;
    area ^= 1;
  }
  return prefix;
}

// Where a selection goes: the index row (or nullptr) and, for the fused decode step, the row's
// selected (position, score) list (or nullptrs).
struct SelOut {
  int32_t* idx;
  int32_t* pos;
  float* score;
};

// Emission of one block of list items in list order: item fb + e (e < kCsPer) of this thread, key
// keys[e], position pos[e]; selected are keys > kstar and the first `need` keys == kstar (unless
// take_all_eq).  eq_base / out_base carry the counts of the earlier blocks.
__device__ __forceinline__ void emit_block(int fb, int total, const uint32_t (&keys)[kCsPer],
                                           const uint32_t (&pos)[kCsPer], uint32_t kstar, uint32_t need,
                                           bool take_all_eq, uint32_t& eq_base, uint32_t& out_base,
                                           const SelOut& so, SelShared& sh) {
  uint32_t eq_tot = 0, sel_tot;
  uint32_t eq_rank = eq_base;
  if (!take_all_eq) {  // workgroup-uniform: the ranks among keys equal to kstar decide
    uint32_t eqc = 0;
#pragma unroll
    for (int e = 0; e < kCsPer; ++e) eqc += (fb + e < total && keys[e] == kstar) ? 1u : 0u;
    eq_rank += block_excl_scan<kCsWaves>(eqc, sh.wsum, &eq_tot);
  }
  uint32_t selc = 0, selm = 0;
#pragma unroll
  for (int e = 0; e < kCsPer; ++e) {
    if (fb + e >= total) continue;
    bool sel = keys[e] > kstar;
    if (keys[e] == kstar) {
      sel = take_all_eq || eq_rank < need;
      ++eq_rank;
    }
    selm |= (uint32_t)sel << e;
    selc += sel ? 1u : 0u;
  }
  uint32_t o = out_base + block_excl_scan<kCsWaves>(selc, sh.wsum, &sel_tot);
#pragma unroll
  for (int e = 0; e < kCsPer; ++e) {
    if ((selm >> e) & 1u) {
      if (so.idx) so.idx[o] = (int32_t)pos[e];
      if (so.pos) {
        so.pos[o] = (int32_t)pos[e];
        so.score[o] = key_to_float(keys[e]);
      }
      ++o;
    }
  }
  eq_base += eq_tot;
  out_base += sel_tot;
}

// Writes, in list order, the kk items of the largest keys (ties at the k-th key: earliest items)
// and pads out to k_max with -1.  Keys and positions come from src (list in global memory).
// kmin / kmax: bounds of the keys, when known.
template <class Src>
__device__ void select_ordered(const Src& src, int total, int kk, int k_max, const SelOut& so,
                               uint32_t* hist, SelShared& sh, uint32_t kmin = 0u, uint32_t kmax = 0xffffffffu) {
  const int tid = threadIdx.x;
  uint32_t need, cnt_eq;
  const uint32_t kstar = radix_kth([&](int f) { return src.key(f); }, total, kk, kmin, kmax, hist, sh,
                                   need, cnt_eq);
  const bool take_all_eq = cnt_eq == need;
  uint32_t eq_base = 0, out_base = 0;
  for (int f0 = 0; f0 < total; f0 += kCsThreads * kCsPer) {
    const int fb = f0 + tid * kCsPer;
    uint32_t keys[kCsPer], pos[kCsPer];
#pragma unroll
    for (int e = 0; e < kCsPer; ++e) keys[e] = fb + e < total ? src.key(fb + e) : 0u;
    src.pos8(fb, total, 0xffu, pos);
    emit_block(fb, total, keys, pos, kstar, need, take_all_eq, eq_base, out_base, so, sh);
  }
  if (so.idx)
    for (int i = kk + tid; i < k_max; i += kCsThreads) so.idx[i] = -1;
}

// Attention of one row over its selected list (kk positions; score_at(i, position) gives the
// scaled score of entry i), for the fused decode step: the scores come with the list, so only V
// rows are read.  Each of the
// kCsWaves waves takes kCsAttnEntries entries per round (D/8 lanes per position, all V loads of
// the round in flight before use), keeps an online softmax in log2 units, and the position groups
// and waves are merged at the end (lane shuffles, then `red`: kCsWaves * (D + 2) floats of LDS).
constexpr int kCsAttnEntries = 64;
template <int D, bool PAGED, class ScoreAt>
__device__ void attend_list(const KVArgs& kv, int b, int h, const int32_t* __restrict__ pos,
                            ScoreAt score_at, int kk, float* red,
                            float* __restrict__ out_row, float* __restrict__ lse_row) {
  constexpr int LPP = D / 8, PPW = kWave / LPP, NSTEP = kCsAttnEntries / PPW;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int p = lane / LPP, c = lane - (lane / LPP) * LPP;
  float m = -INFINITY, l = 0.f;
  float o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = 0.f;
  for (int base = wave * kCsAttnEntries; base < kk; base += kCsWaves * kCsAttnEntries) {
    const bool mine_ok = base + lane < kk;
    const int my_pos = mine_ok ? pos[base + lane] : 0;
    const float my_s = mine_ok ? score_at(base + lane, my_pos) * kLog2e : -INFINITY;
    int idx[NSTEP];
    float sv[NSTEP];
#pragma unroll
    for (int u = 0; u < NSTEP; ++u) {
      idx[u] = __shfl(my_pos, u * PPW + p);
      sv[u] = __shfl(my_s, u * PPW + p);
    }
    uint4 vr[NSTEP];
#pragma unroll
    for (int u = 0; u < NSTEP; ++u) vr[u] = ld16(kv.v + kv_row<D, PAGED>(kv, b, h, idx[u]) + c * 8);
    float mx = -INFINITY;
#pragma unroll
    for (int u = 0; u < NSTEP; ++u) mx = fmaxf(mx, sv[u]);
    const float m_new = fmaxf(m, mx);
    if (m_new != -INFINITY) {
      const float alpha = fast_exp2(m - m_new);
      l *= alpha;
#pragma unroll
      for (int i = 0; i < 8; ++i) o[i] *= alpha;
#pragma unroll
      for (int u = 0; u < NSTEP; ++u) {
        const float w = fast_exp2(sv[u] - m_new);
        l += w;
        float vf[8];
        unpack8(vr[u], vf);
#pragma unroll
        for (int i = 0; i < 8; ++i) o[i] = fmaf(w, vf[i], o[i]);
      }
      m = m_new;
    }
  }
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
  float* red_m = red;
  float* red_l = red + kCsWaves;
  float* red_o = red + 2 * kCsWaves;  // [kCsWaves][D]
  if (lane == 0) {
    red_m[wave] = m;
    red_l[wave] = l;
  }
  if (p == 0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) red_o[wave * D + c * 8 + i] = o[i];
  }
  __syncthreads();
  for (int col = tid; col < D; col += kCsThreads) {
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kCsWaves; ++w) M = fmaxf(M, red_m[w]);
    float Lsum = 0.f, O = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kCsWaves; ++w) {
        const float wt = fast_exp2(red_m[w] - M);
        Lsum = fmaf(wt, red_l[w], Lsum);
        O = fmaf(wt, red_o[w * D + col], O);
      }
    }
    out_row[col] = Lsum > 0.f ? O / Lsum : 0.f;
    if (col == 0) *lse_row = Lsum > 0.f ? (M + fast_log2(Lsum)) * kLn2 : -INFINITY;
  }
}

// The candidate part of cand_select_kernel: select from the row's slots (held in LDS when at most
// lds_cap <= MB * kCsThreads * kCsPer of them).
template <int MB>
__device__ void cand_path(uint32_t total, int nsub, int cap, const SelOut& so, int kk, int k_max,
                          int row, float* __restrict__ region, int64_t score_stride, int chunk, int chunks,
                          const uint32_t* prefix_s, uint32_t* lds_key, int lds_cap, uint32_t* hist,
                          SelShared& sh) {
  const int tid = threadIdx.x;
  CandSource src;
  src.base = reinterpret_cast<const uint32_t*>(region + (int64_t)row * score_stride);
  src.prefix = prefix_s;
  src.nsub = nsub;
  src.cap = cap;
  src.nsub_all = chunks * kCandWaves;
  src.span = chunk / kCandWaves;
  src.lds_key = nullptr;
  if (total > (uint32_t)lds_cap) {  // too many to hold: every pass reads the slots
    select_ordered(src, (int)total, kk, k_max, so, hist, sh);
    return;
  }
  // keys into LDS and positions into registers, kCsPer consecutive items per thread and block
  // (the same items the emission gives this thread), loads of a block in flight together
  if (tid == 0) {
    sh.kmin = 0xffffffffu;
    sh.kmax = 0u;
  }
  __syncthreads();
  // every block's loads are issued before any is used
  const int nblk = ((int)total + kCsThreads * kCsPer - 1) / (kCsThreads * kCsPer);  // <= MB
  uint32_t preg[MB][kCsPer];  // the slot's first position, then the item's position
  uint32_t sc[MB][kCsPer], of[MB][kCsPer];
  const uint16_t* off16 = reinterpret_cast<const uint16_t*>(src.base);
#pragma unroll
  for (int blk = 0; blk < MB; ++blk) {
    if (blk < nblk) {
      int64_t sw[kCsPer], ow[kCsPer];
      int first[kCsPer];
      src.locate(blk * kCsThreads * kCsPer + tid * kCsPer, (int)total, sw, ow, first);
#pragma unroll
      for (int e = 0; e < kCsPer; ++e) {
        sc[blk][e] = src.base[sw[e]];
        of[blk][e] = off16[ow[e]];
        preg[blk][e] = (uint32_t)first[e];
      }
    }
  }
  uint32_t lmin = 0xffffffffu, lmax = 0u;
#pragma unroll
  for (int blk = 0; blk < MB; ++blk) {
    if (blk >= nblk) break;
    const int fb = blk * kCsThreads * kCsPer + tid * kCsPer;
#pragma unroll
    for (int e = 0; e < kCsPer; ++e) {
      preg[blk][e] += of[blk][e];
      if (fb + e < (int)total) {
        const uint32_t key = ord_key(__uint_as_float(sc[blk][e]));
        lds_key[fb + e] = key;
        lmin = min(lmin, key);
        lmax = max(lmax, key);
      }
    }
  }
  block_key_range(lmin, lmax, sh);
  __syncthreads();
  uint32_t need, cnt_eq;
  const uint32_t kstar = radix_kth([&](int f) { return lds_key[f]; }, (int)total, kk, sh.kmin, sh.kmax,
                                   hist, sh, need, cnt_eq);
  const bool take_all_eq = cnt_eq == need;
  uint32_t eq_base = 0, out_base = 0;
#pragma unroll
  for (int blk = 0; blk < MB; ++blk) {
    if (blk * kCsThreads * kCsPer >= (int)total) break;
    const int fb = blk * kCsThreads * kCsPer + tid * kCsPer;
    uint32_t keys[kCsPer];
#pragma unroll
    for (int e = 0; e < kCsPer; ++e) keys[e] = fb + e < (int)total ? lds_key[fb + e] : 0u;
    emit_block(fb, (int)total, keys, preg[blk], kstar, need, take_all_eq, eq_base, out_base, so, sh);
  }
  if (so.idx)
    for (int i = kk + tid; i < k_max; i += kCsThreads) so.idx[i] = -1;
}


// Slot counts of the row's chunks that hold positions < L (nsub slots, each capped at cap) and
// their exclusive prefix sums into prefix_s[0 .. kMaxCandSlots]; returns the total and sets
// overflow when a slot lost candidates.  Ends with a barrier.
__device__ uint32_t slot_prefix(const uint32_t* __restrict__ counts, int row, int chunks, int nsub,
                                int cap, uint32_t* prefix_s, SelShared& sh, bool& overflow) {
  const int tid = threadIdx.x;
  constexpr int kPerT = kMaxCandSlots / kCsThreads;  // slots per thread
  uint32_t cc[kPerT];
  uint32_t local = 0;
  bool over = false;
#pragma unroll
  for (int e = 0; e < kPerT; ++e) {
    const int sidx = tid * kPerT + e;
    const uint32_t cnt = sidx < nsub ? counts[(int64_t)row * chunks * kCandWaves + sidx] : 0u;
    over |= cnt > (uint32_t)cap;
    cc[e] = cnt > (uint32_t)cap ? (uint32_t)cap : cnt;
    local += cc[e];
  }
  uint32_t total;
  uint32_t run = block_excl_scan<kCsWaves>(local, sh.wsum, &total);
#pragma unroll
  for (int e = 0; e < kPerT; ++e) {
    prefix_s[tid * kPerT + e] = run;
    run += cc[e];
  }
  if (tid == 0) prefix_s[kMaxCandSlots] = total;
  overflow = __syncthreads_or(over) != 0;
  return total;
}

// FUSED (the decode step): the selection also goes to the row's (position, score) list in
// sel_pos / sel_score, the workgroup then attends to it (attend_list) and writes out / lse;
// indices may then be nullptr.
template <int D, bool PAGED, bool FUSED, int MB>
__global__ __launch_bounds__(kCsThreads) void cand_select_kernel(
    const uint16_t* __restrict__ q, KVArgs kv, int T, int Hq, int G, float scale,
    const int32_t* __restrict__ k_per_req, float* __restrict__ region, int64_t score_stride,
    const uint32_t* __restrict__ counts, int chunk, int chunks, int k_max, int lds_cap,
    int32_t* __restrict__ indices, int32_t* __restrict__ sel_pos, float* __restrict__ sel_score,
    float* __restrict__ out, float* __restrict__ lse, int B) {
  extern __shared__ uint32_t smem[];  // lds_cap candidate keys, then 2 x 2048 histogram counters
  __shared__ SelShared sh;
  __shared__ uint32_t prefix_s[kMaxCandSlots + 1];
  uint32_t* lds_key = smem;
  uint32_t* hist = smem + lds_cap;
  const int row = grouped_row(blockIdx.x, B, T, Hq, G, kv.num_kv_heads);
  if (row < 0) return;
  const int b = row / (T * Hq);
  const int t = (row / Hq) - (row / (T * Hq)) * T;
  const int hq = row - (row / Hq) * Hq;
  const int L = seq_len_of(kv, b);
  const int vis = max(0, L - T + t + 1);
  int kb = k_per_req ? k_per_req[b] : k_max;
  kb = kb < 0 ? 0 : (kb > k_max ? k_max : kb);
  const int kk = min(kb, vis);
  SelOut so;
  so.idx = indices ? indices + (int64_t)row * k_max : nullptr;
  so.pos = FUSED ? sel_pos + (int64_t)row * k_max : nullptr;
  so.score = FUSED ? sel_score + (int64_t)row * k_max : nullptr;
  const int tid = threadIdx.x;
  // nothing to select; or (index-only) everything visible is selected -- the fused step needs the
  // scores of every visible position then, which its fallback computes
  if (kk == 0 || (!FUSED && kk == vis)) {
    if (so.idx)
      for (int i = tid; i < k_max; i += kCsThreads) so.idx[i] = i < kk ? i : -1;
    if (FUSED) {
      for (int i = tid; i < D; i += kCsThreads) out[(int64_t)row * D + i] = 0.f;
      if (tid == 0) lse[row] = -INFINITY;
    }
    return;
  }

  const int cap = cand_cap(chunk);
  const int nsub = ((L + chunk - 1) / chunk) * kCandWaves;
  bool overflow;
  const uint32_t total = slot_prefix(counts, row, chunks, nsub, cap, prefix_s, sh, overflow);

  if (overflow || total < (uint32_t)kk) {
    // ---- exact fallback: every score of the row into its workspace area, then select
    float* srow = region + (int64_t)row * score_stride;
    constexpr int LPP = D / 8, PPW = kWave / LPP;
    const int lane = tid & 63, wave = tid >> 6;
    const int p = lane / LPP, cdim = lane - (lane / LPP) * LPP;
    const int h = hq / G;
    const uint4 qv = ld16(q + (int64_t)row * D + cdim * 8);
    // kFallbackUnroll rows per lane group in flight (one at a time, a 10^5-position row took
    // milliseconds on one workgroup)
    constexpr int U = kFallbackUnroll, STRIDE = kCsWaves * PPW;
    for (int n0 = wave * PPW; n0 < vis; n0 += STRIDE * U) {
      uint4 kr[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int n = n0 + u * STRIDE + p;
        kr[u] = ld16(kv.k + kv_row<D, PAGED>(kv, b, h, n < vis ? n : 0) + cdim * 8);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int n = n0 + u * STRIDE + p;
        float dot = 0.f;
        dot = dot2_bf16(qv.x, kr[u].x, dot);
        dot = dot2_bf16(qv.y, kr[u].y, dot);
        dot = dot2_bf16(qv.z, kr[u].z, dot);
        dot = dot2_bf16(qv.w, kr[u].w, dot);
        dot = group_sum<LPP>(dot);
        if (n < vis && cdim == 0) srow[n] = dot * scale;
      }
    }
    __syncthreads();
    select_ordered(DenseSource{srow}, vis, kk, k_max, so, hist, sh);
  } else {
    cand_path<MB>(total, nsub, cap, so, kk, k_max, row, region, score_stride, chunk, chunks, prefix_s, lds_key,
              lds_cap, hist, sh);
  }
  if constexpr (FUSED) {
    __syncthreads();  // the selected list is complete, LDS free again
    const float* sel = so.score;
    attend_list<D, PAGED>(kv, b, hq / G, so.pos, [sel](int i, int) { return sel[i]; }, kk,
                          reinterpret_cast<float*>(smem),
                          out + (int64_t)row * D, lse + row);
  }
}

// The decode step on the full-score path (k > N/8): each row's index list (from select_kernel,
// ascending) with the scores score_hist_kernel already wrote for every visible position, so the
// attention gathers V rows only.  One workgroup per row.
template <int D, bool PAGED>
__global__ __launch_bounds__(kCsThreads) void attend_scores_kernel(
    KVArgs kv, int T, int Hq, int G, const int32_t* __restrict__ k_per_req, int k_max,
    const int32_t* __restrict__ indices, const float* __restrict__ scores, int64_t score_stride,
    float* __restrict__ out, float* __restrict__ lse, int B) {
  __shared__ float red[kCsWaves * (D + 2)];
  const int row = grouped_row(blockIdx.x, B, T, Hq, G, kv.num_kv_heads);
  if (row < 0) return;
  const int b = row / (T * Hq);
  const int t = (row / Hq) - (row / (T * Hq)) * T;
  const int hq = row - (row / Hq) * Hq;
  const int L = seq_len_of(kv, b);
  const int vis = max(0, L - T + t + 1);
  int kb = k_per_req ? k_per_req[b] : k_max;
  kb = kb < 0 ? 0 : (kb > k_max ? k_max : kb);
  const int kk = min(kb, vis);
  const float* srow = scores + (int64_t)row * score_stride;
  attend_list<D, PAGED>(kv, b, hq / G, indices + (int64_t)row * k_max, [srow](int, int p) { return srow[p]; }, kk,
                        red, out + (int64_t)row * D, lse + row);
}

// ============================================================================ reduced-byte indexer
// C of the sketch pipeline (A and B are sample_tau_kernel / score_cand_kernel with SK): per row,
// the nc = min(cand_mult * k', visible) positions with the largest sketch scores (lower position
// first among equal values) go to the row's list -- from the candidates, or from every sketch
// score of the row when the candidates may not hold them (too few, or a slot overflowed), or
// every visible position when nc = visible; the list entries then get their exact scores and
// the k' largest of those (lower position first) are the selection.

// A row's list in position order: positions in global memory, keys in LDS (key_lds) or from the
// scores in global memory.
struct ListSource {
  const int32_t* pos;
  const float* score;
  const uint32_t* key_lds;
  __device__ __forceinline__ uint32_t key(int f) const { return key_lds ? key_lds[f] : ord_key(score[f]); }
  __device__ __forceinline__ void pos8(int f0, int total, uint32_t, uint32_t (&p)[kCsPer]) const {
#pragma unroll
    for (int e = 0; e < kCsPer; ++e) p[e] = f0 + e < total ? (uint32_t)pos[f0 + e] : 0u;
  }
};

// Sketch score of every visible position of query row `qr` into srow: D / 16 lanes per position,
// 16 codes each, integer dot products (v_dot4) summed exactly (every partial sum is an integer
// below 2^24) -- the same values as the MFMA pass.
template <int D, bool PAGED>
__device__ void sketch_row_scores(const KVArgs& kv, const SketchArgs& sk, int b, int h, int64_t qr,
                                  int vis, float* __restrict__ srow) {
  constexpr int LPP = D / 16, PPW = kWave / LPP;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int p = lane / LPP, c = lane - (lane / LPP) * LPP;
  const uint4 qc = ld16i8(sk.q_codes + qr * D + c * 16);
  const float qs = sk.q_scales[qr];
  constexpr int U = kFallbackUnroll, STRIDE = kCsWaves * PPW;
  for (int n0 = wave * PPW; n0 < vis; n0 += STRIDE * U) {
    uint4 kc[U];
    float ks[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int n = n0 + u * STRIDE + p;
      const int64_t off = kv_row<D, PAGED>(kv, b, h, n < vis ? n : 0);
      kc[u] = ld16i8(sk.codes + off + c * 16);
      ks[u] = sk.scales[off / D];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int n = n0 + u * STRIDE + p;
      int d = 0;
      d = __builtin_amdgcn_sdot4((int)qc.x, (int)kc[u].x, d, false);
      d = __builtin_amdgcn_sdot4((int)qc.y, (int)kc[u].y, d, false);
      d = __builtin_amdgcn_sdot4((int)qc.z, (int)kc[u].z, d, false);
      d = __builtin_amdgcn_sdot4((int)qc.w, (int)kc[u].w, d, false);
      const float dot = group_sum<LPP>((float)d);
      if (n < vis && c == 0) srow[n] = (qs * ks[u]) * dot;
    }
  }
}

// Exact scores of list entries [0, n) (positions pos[f], all visible): each wave takes kWave
// entries per round, D / 8 lanes per entry (D / 8 entries per lane group, their K loads in flight
// together); a round's positions arrive with one coalesced load, issued a round ahead, and are
// spread by lane shuffles.  The ordered keys go to key_lds[f] when it is set, else the scores to
// score[f]; the keys' bounds to sh.kmin / sh.kmax (initialised by the caller).
template <int D, bool PAGED>
__device__ void rerank_exact(const KVArgs& kv, int b, int h, const uint16_t* __restrict__ qrow, float scale,
                             const int32_t* __restrict__ pos, float* __restrict__ score,
                             uint32_t* key_lds, int n, SelShared& sh) {
  constexpr int LPP = D / 8, PPW = kWave / LPP, NSTEP = kWave / PPW;
  constexpr int kRound = kCsWaves * kWave;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int p = lane / LPP, c = lane - (lane / LPP) * LPP;
  const uint4 qv = ld16(qrow + c * 8);
  uint32_t lmin = 0xffffffffu, lmax = 0u;
  int base = wave * kWave;
  int my = base < n ? pos[min(base + lane, n - 1)] : 0;
  for (; base < n; base += kRound) {
    const int nb = base + kRound;
    const int nxt = nb < n ? pos[min(nb + lane, n - 1)] : 0;
    uint4 kr[NSTEP];
#pragma unroll
    for (int u = 0; u < NSTEP; ++u) kr[u] = ld16(kv.k + kv_row<D, PAGED>(kv, b, h, __shfl(my, u * PPW + p)) + c * 8);
#pragma unroll
    for (int u = 0; u < NSTEP; ++u) {
      float dot = 0.f;
      dot = dot2_bf16(qv.x, kr[u].x, dot);
      dot = dot2_bf16(qv.y, kr[u].y, dot);
      dot = dot2_bf16(qv.z, kr[u].z, dot);
      dot = dot2_bf16(qv.w, kr[u].w, dot);
      dot = group_sum<LPP>(dot);
      const int f = base + u * PPW + p;
      if (f < n && c == 0) {
        const float sc = dot * scale;
        const uint32_t key = ord_key(sc);
        lmin = min(lmin, key);
        lmax = max(lmax, key);
        if (key_lds) key_lds[f] = key; else score[f] = sc;
      }
    }
    my = nxt;
  }
  block_key_range(lmin, lmax, sh);
}

// list_pos / list_score: the rows' lists (list_stride >= min(cand_mult * k_max, max_len) entries);
// with `listed` the positions are already there (select_kernel over every sketch score).
// FUSED: as for cand_select_kernel, the selection also goes to sel_pos / sel_score and the row's
// attention over it to out / lse.
template <int D, bool PAGED, bool FUSED, int MB>
__global__ __launch_bounds__(kCsThreads) void sketch_select_kernel(
    const uint16_t* __restrict__ q, KVArgs kv, SketchArgs sk, int T, int Hq, int G, float scale,
    const int32_t* __restrict__ k_per_req, float* __restrict__ region, int64_t score_stride,
    const uint32_t* __restrict__ counts, int chunk, int chunks, int k_max, int cand_mult, int lds_cap,
    int32_t* __restrict__ list_pos, float* __restrict__ list_score, int list_stride, bool listed,
    int32_t* __restrict__ indices, int32_t* __restrict__ sel_pos, float* __restrict__ sel_score,
    float* __restrict__ out, float* __restrict__ lse, int B) {
  extern __shared__ uint32_t smem[];  // lds_cap candidate keys, then 2 x 2048 histogram counters
  __shared__ SelShared sh;
  __shared__ uint32_t prefix_s[kMaxCandSlots + 1];
  uint32_t* lds_key = smem;
  uint32_t* hist = smem + lds_cap;
  const int row = grouped_row(blockIdx.x, B, T, Hq, G, kv.num_kv_heads);
  if (row < 0) return;
  const int b = row / (T * Hq);
  const int t = (row / Hq) - (row / (T * Hq)) * T;
  const int hq = row - (row / Hq) * Hq;
  const int h = hq / G;
  const int L = seq_len_of(kv, b);
  const int vis = max(0, L - T + t + 1);
  int kb = k_per_req ? k_per_req[b] : k_max;
  kb = kb < 0 ? 0 : (kb > k_max ? k_max : kb);
  const int kk = min(kb, vis);
  const int nc = (int)min((int64_t)cand_mult * kk, (int64_t)vis);
  SelOut so;
  so.idx = indices ? indices + (int64_t)row * k_max : nullptr;
  so.pos = FUSED ? sel_pos + (int64_t)row * k_max : nullptr;
  so.score = FUSED ? sel_score + (int64_t)row * k_max : nullptr;
  const int tid = threadIdx.x;
  if (kk == 0 || (!FUSED && kk == vis)) {
    if (so.idx)
      for (int i = tid; i < k_max; i += kCsThreads) so.idx[i] = i < kk ? i : -1;
    if (FUSED) {
      for (int i = tid; i < D; i += kCsThreads) out[(int64_t)row * D + i] = 0.f;
      if (tid == 0) lse[row] = -INFINITY;
    }
    return;
  }
  int32_t* lpos = list_pos + (int64_t)row * list_stride;
  float* lsc = list_score + (int64_t)row * list_stride;
  if (listed) {
    // the list is in place
  } else if (nc == vis) {
    for (int f = tid; f < vis; f += kCsThreads) lpos[f] = f;
  } else {
    const int cap = cand_cap(chunk);
    const int nsub = ((L + chunk - 1) / chunk) * kCandWaves;
    bool overflow;
    const uint32_t total = slot_prefix(counts, row, chunks, nsub, cap, prefix_s, sh, overflow);
    // index lists only, one candidate per selected position (cand_mult = 1): the list is the
    // selection, written straight to the row's indices
    const bool direct = !FUSED && nc == kk;
    SelOut lo;
    lo.idx = direct ? so.idx : nullptr;
    lo.pos = direct ? nullptr : lpos;
    lo.score = direct ? nullptr : lsc;
    const int lk = direct ? k_max : nc;
    if (overflow || total < (uint32_t)nc) {
      float* srow = region + (int64_t)row * score_stride;
      sketch_row_scores<D, PAGED>(kv, sk, b, h, row, vis, srow);
      __syncthreads();
      select_ordered(DenseSource{srow}, vis, nc, lk, lo, hist, sh);
    } else {
      cand_path<MB>(total, nsub, cap, lo, nc, lk, row, region, score_stride, chunk, chunks, prefix_s, lds_key,
                lds_cap, hist, sh);
    }
    if (direct) return;
  }
  if (tid == 0) {
    sh.kmin = 0xffffffffu;
    sh.kmax = 0u;
  }
  __syncthreads();  // the list is complete
  uint32_t* rkey = nc <= lds_cap ? lds_key : nullptr;  // exact keys in LDS when they fit
  rerank_exact<D, PAGED>(kv, b, h, q + (int64_t)row * D, scale, lpos, lsc, rkey, nc, sh);
  __syncthreads();
  select_ordered(ListSource{lpos, lsc, rkey}, nc, kk, k_max, so, hist, sh, sh.kmin, sh.kmax);
  if constexpr (FUSED) {
    __syncthreads();  // the selected list is complete, LDS free again
    const float* sel = so.score;
    attend_list<D, PAGED>(kv, b, h, so.pos, [sel](int i, int) { return sel[i]; }, kk, reinterpret_cast<float*>(smem),
                          out + (int64_t)row * D, lse + row);
  }
}

// ============================================================================ launchers
int score_threads(int GT) {
  const int rows = GT < 16 ? GT : 16;
  return 256 * ((rows + 3) / 4);
}

size_t select_lds_bytes(int max_len) {
  const int words = ((max_len + 255) / 256) * 8;
  return sizeof(uint32_t) * ((size_t)kHistBins + 2 * (size_t)words + 2 * (size_t)kCandCap);
}

hipError_t launch_fill_u32(uint32_t* p, int64_t n, uint32_t value, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  if (n % 4 != 0 || reinterpret_cast<uintptr_t>(p) % 16 != 0) return hipErrorInvalidValue;
  int64_t blocks = (n / 4 + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(fill_u32_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p, n, value);
  return hipGetLastError();
}

template <int D, bool PAGED, bool SK>
static hipError_t launch_score_t(const TopkLaunch& a, hipStream_t stream) {
  const int rows_tile = a.GT < 16 ? a.GT : 16;
  const size_t page_ids = PAGED ? (size_t)(a.chunk >> a.kv.page_shift) + 2 : 0;
  const size_t lds = (size_t)rows_tile * (kHistBins / 2) * sizeof(uint32_t) + page_ids * sizeof(int);
  auto kern = score_hist_kernel<D, PAGED, SK>;
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  dim3 grid(a.chunks, a.B * a.kv.num_kv_heads, (a.GT + 15) / 16);
  hipLaunchKernelGGL(kern, grid, dim3(score_threads(a.GT)), lds, stream, a.q, a.kv, a.sk, a.T, a.Hq, a.G,
                     a.scale, a.scores, a.hist, a.chunk, rows_tile, a.score_stride);
  return hipGetLastError();
}

// Full-score path: every visible position's score (SK: sketch score) and the rows' histograms,
// then the min(mult * k', visible) largest per row into `out` (rows of out_stride entries).
template <int D, bool PAGED, bool SK>
static hipError_t launch_full_select_t(const TopkLaunch& a, int mult, int out_stride, int32_t* out,
                                       hipStream_t stream) {
  hipError_t e = launch_fill_u32(a.hist, (int64_t)a.rows * kHistBins, 0u, stream);
  if (e != hipSuccess) return e;
  if ((e = launch_score_t<D, PAGED, SK>(a, stream)) != hipSuccess) return e;
  const size_t lds = select_lds_bytes(a.kv.max_len);
  if (lds > 65536) {
    e = hipFuncSetAttribute((const void*)select_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  const int words = ((a.kv.max_len + 255) / 256) * 8;
  hipLaunchKernelGGL(select_kernel, dim3(a.rows), dim3(kSelThreads), lds, stream, a.scores,
                     a.hist, a.kv.seq_lens, a.k_per_req, a.T, a.Hq, a.kv.max_len, a.score_stride,
                     a.k_max, mult, out_stride, words, out);
  return hipGetLastError();
}

// Candidate pipeline (A, B, C above); SK: the reduced-byte indexer, whose lists come from the
// full-score path instead when a.sketch_full is set.
template <int D, bool PAGED, bool SK>
static hipError_t launch_filtered_t(const TopkLaunch& a, hipStream_t stream) {
  // candidate positions are stored as 16-bit offsets within a wave's slot
  if (a.cand_chunk / kCandWaves > 65536) return hipErrorInvalidValue;
  const int tiles = (a.GT + 15) / 16;
  const int groups = a.B * a.kv.num_kv_heads;
  hipError_t e;
  const bool listed = SK && a.sketch_full;
  if (listed) {  // otherwise sample_tau_kernel quantises the query rows
    if ((e = launch_q_sketch(a.q, a.rows, D, a.sk.q_codes, a.sk.q_scales, stream)) != hipSuccess) return e;
  }
  if (listed && a.cand_mult == 1 && !a.fused)  // the selection is the sketch's own top-k
    return launch_full_select_t<D, PAGED, true>(a, 1, a.k_max, a.indices, stream);
  if (listed) {
    if ((e = launch_full_select_t<D, PAGED, true>(a, a.cand_mult, a.list_stride, a.list_pos, stream)) != hipSuccess)
      return e;
  } else {
    // At most half as many tiles as compute units: four workgroups per tile sample, and every
    // candidate workgroup sets its rows' thresholds.  Measured: the sample pass drops from 15-16
    // to 7-8 us, the candidate pass grows by 1-3 us; on the sketch, whose candidate workgroups
    // are short, with 8 rows per tile the growth exceeds the saving.
    const int rows_tile = a.GT < 16 ? a.GT : 16;
    const bool split = 2 * groups * tiles <= a.cus && (!SK || rows_tile <= 4);
    if (split) {
      hipLaunchKernelGGL((sample_tau_kernel<D, PAGED, SK, false, 4>), dim3(groups, tiles, 4),
                         dim3(kSampleWaves * kWave), 0, stream, a.q, a.kv, a.sk, a.T, a.Hq, a.G, a.scale,
                         a.k_per_req, a.k_max, a.cand_mult, a.tau, nullptr, nullptr, (int64_t)0, a.tau_prefixes);
    } else {
      auto samp = sample_tau_kernel<D, PAGED, SK, false, 1>;
      const size_t lds_keys = (size_t)16 * kTauSamples * sizeof(uint32_t);
      if ((e = hipFuncSetAttribute((const void*)samp, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_keys)) !=
          hipSuccess)
        return e;
      hipLaunchKernelGGL(samp, dim3(groups, tiles), dim3(kSampleWaves * kWave), lds_keys, stream, a.q, a.kv, a.sk,
                         a.T, a.Hq, a.G, a.scale, a.k_per_req, a.k_max, a.cand_mult, a.tau, nullptr, nullptr,
                         (int64_t)0, nullptr);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const size_t page_ids = PAGED ? (size_t)(a.cand_chunk >> a.kv.page_shift) + 2 : 0;
    auto cand = split ? (rows_tile <= 4 ? score_cand_kernel<D, PAGED, 1, SK, true>
                                        : (rows_tile <= 8 ? score_cand_kernel<D, PAGED, 2, SK, true>
                                                          : score_cand_kernel<D, PAGED, 4, SK, true>))
                      : (rows_tile <= 4 ? score_cand_kernel<D, PAGED, 1, SK, false>
                                        : (rows_tile <= 8 ? score_cand_kernel<D, PAGED, 2, SK, false>
                                                          : score_cand_kernel<D, PAGED, 4, SK, false>));
    hipLaunchKernelGGL(cand, dim3(a.cand_chunks, groups, tiles), dim3(kCandWaves * kWave),
                       page_ids * sizeof(int), stream, a.q, a.kv, a.sk, a.T, a.Hq, a.G, a.scale, a.tau,
                       a.tau_prefixes, a.k_per_req, a.k_max, a.cand_mult, a.scores,
                       a.score_stride, a.counts, a.cand_chunk, a.cand_chunks);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // candidate keys held in LDS: 1.6 times the count expected at the longest row (cand_rank of
  // its samples), at least twice the largest list, at most kCsBlocks * kCsThreads * kCsPer = 12288;
  // when there are no more rows than compute units (one workgroup per unit anyway), up to twice
  // that.  Rows with more candidates select from the slots in global memory.
  const int64_t keep_max = SK ? (int64_t)a.list_stride : (int64_t)a.k_max;
  const int64_t ns_max = a.kv.max_len < kTauSamples ? a.kv.max_len : kTauSamples;
  const int64_t expect = cand_rank(keep_max, ns_max, a.kv.max_len) * a.kv.max_len / ns_max;
  const int64_t want = expect * 8 / 5 > 2 * keep_max ? expect * 8 / 5 : 2 * keep_max;
  int lds_cap = (int)((min(want, (int64_t)kCsBlocksBig * kCsThreads * kCsPer) + 255) / 256 * 256);
  const bool big = lds_cap > kCsBlocks * kCsThreads * kCsPer && a.rows <= a.cus;
  const int cap_max = (big ? kCsBlocksBig : kCsBlocks) * kCsThreads * kCsPer;
  if (lds_cap > cap_max) lds_cap = cap_max;
  const size_t lds = ((size_t)lds_cap + 4096) * sizeof(uint32_t);  // keys, two histogram areas
  if constexpr (SK) {
    auto sel = a.fused ? (big ? sketch_select_kernel<D, PAGED, true, kCsBlocksBig> : sketch_select_kernel<D, PAGED, true, kCsBlocks>)
                       : (big ? sketch_select_kernel<D, PAGED, false, kCsBlocksBig> : sketch_select_kernel<D, PAGED, false, kCsBlocks>);
    if (lds > 65536) {
      e = hipFuncSetAttribute((const void*)sel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(sel, dim3(grouped_row_blocks(a.B, a.kv.num_kv_heads, a.GT)), dim3(kCsThreads), lds, stream,
                       a.q, a.kv, a.sk, a.T, a.Hq, a.G, a.scale, a.k_per_req, a.scores, a.score_stride, a.counts,
                       a.cand_chunk, a.cand_chunks, a.k_max, a.cand_mult, lds_cap, a.list_pos, a.list_score,
                       a.list_stride, listed, a.indices, a.sel_pos, a.sel_score, a.out, a.lse, a.B);
  } else {
    auto sel = a.fused ? (big ? cand_select_kernel<D, PAGED, true, kCsBlocksBig> : cand_select_kernel<D, PAGED, true, kCsBlocks>)
                       : (big ? cand_select_kernel<D, PAGED, false, kCsBlocksBig> : cand_select_kernel<D, PAGED, false, kCsBlocks>);
    if (lds > 65536) {
      e = hipFuncSetAttribute((const void*)sel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(sel, dim3(grouped_row_blocks(a.B, a.kv.num_kv_heads, a.GT)), dim3(kCsThreads), lds, stream,
                       a.q, a.kv, a.T, a.Hq, a.G, a.scale, a.k_per_req, a.scores, a.score_stride, a.counts,
                       a.cand_chunk, a.cand_chunks, a.k_max, lds_cap, a.indices, a.sel_pos, a.sel_score, a.out,
                       a.lse, a.B);
  }
  return hipGetLastError();
}

template <bool SK>
static hipError_t launch_filtered(const TopkLaunch& a, hipStream_t stream) {
  if (a.D == 128)
    return a.paged ? launch_filtered_t<128, true, SK>(a, stream) : launch_filtered_t<128, false, SK>(a, stream);
  return a.paged ? launch_filtered_t<64, true, SK>(a, stream) : launch_filtered_t<64, false, SK>(a, stream);
}

hipError_t launch_attend_scores(const TopkLaunch& a, hipStream_t stream) {
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3(grouped_row_blocks(a.B, a.kv.num_kv_heads, a.GT)), dim3(kCsThreads), 0, stream,
                       a.kv, a.T, a.Hq, a.G, a.k_per_req, a.k_max, a.indices, a.scores, a.score_stride, a.out,
                       a.lse, a.B);
  };
  if (a.D == 128) {
    if (a.paged) go(attend_scores_kernel<128, true>); else go(attend_scores_kernel<128, false>);
  } else {
    if (a.paged) go(attend_scores_kernel<64, true>); else go(attend_scores_kernel<64, false>);
  }
  return hipGetLastError();
}

// Selection of caches of at most kTauSamples positions whose keys a split whole-row pass stored
// (keys[row * kTauSamples + n], 0 for a position the row does not see): one wave per row.
__global__ __launch_bounds__(4 * kWave) void small_select_kernel(KVArgs kv, int T, int Hq, int rows,
                                                                 const int32_t* __restrict__ k_per_req, int k_max,
                                                                 const uint32_t* __restrict__ keys,
                                                                 int32_t* __restrict__ indices) {
  const int row = (int)blockIdx.x * 4 + (int)(threadIdx.x >> 6);
  if (row >= rows) return;
  const int b = row / (T * Hq);
  const int t = row / Hq - b * T;
  const int vis = max(seq_len_of(kv, b) - T + t + 1, 0);
  const int k_req = k_per_req ? k_per_req[b] : k_max;
  const int kb = k_req < 0 ? 0 : (k_req > k_max ? k_max : k_req);
  row_select_all(keys + (int64_t)row * kTauSamples, vis, min(kb, vis), k_max, indices + (int64_t)row * k_max);
}

// Caches of at most kTauSamples positions: the sample kernel scores every position, so it finishes
// the selection itself (and, for the one-call step, keeps every score for the attention).  With
// at most half as many tiles as compute units, four workgroups per tile score a quarter of the
// positions each and store the keys, and small_select_kernel selects: the scoring is bound by the
// rows one compute unit has in flight, which one workgroup per tile leaves on a few units.
template <int D, bool PAGED>
static hipError_t launch_small_t(const TopkLaunch& a, hipStream_t stream) {
  const int groups = a.B * a.kv.num_kv_heads, tiles = (a.GT + 15) / 16;
  if (2 * groups * tiles <= a.cus) {
    hipLaunchKernelGGL((sample_tau_kernel<D, PAGED, false, true, 4>), dim3(groups, tiles, 4),
                       dim3(kSampleWaves * kWave), 0, stream, a.q, a.kv, a.sk, a.T, a.Hq, a.G, a.scale,
                       a.k_per_req, a.k_max, 1, a.tau, nullptr, a.keep_scores ? a.scores : nullptr,
                       a.score_stride, a.tau_prefixes);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(small_select_kernel, dim3((a.rows + 3) / 4), dim3(4 * kWave), 0, stream, a.kv, a.T, a.Hq,
                       a.rows, a.k_per_req, a.k_max, reinterpret_cast<const uint32_t*>(a.tau_prefixes), a.indices);
    return hipGetLastError();
  }
  auto kern = sample_tau_kernel<D, PAGED, false, true, 1>;
  const size_t lds_keys = (size_t)16 * kTauSamples * sizeof(uint32_t);
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_keys);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(a.B * a.kv.num_kv_heads, (a.GT + 15) / 16), dim3(kSampleWaves * kWave), lds_keys,
                     stream, a.q, a.kv, a.sk, a.T, a.Hq, a.G, a.scale, a.k_per_req, a.k_max, 1, a.tau, a.indices,
                     a.keep_scores ? a.scores : nullptr, a.score_stride, nullptr);
  return hipGetLastError();
}

hipError_t launch_topk(const TopkLaunch& a, hipStream_t stream) {
  if (a.sketch) return launch_filtered<true>(a, stream);
  if (a.small) {
    if (a.D == 128) return a.paged ? launch_small_t<128, true>(a, stream) : launch_small_t<128, false>(a, stream);
    return a.paged ? launch_small_t<64, true>(a, stream) : launch_small_t<64, false>(a, stream);
  }
  if (a.filtered) return launch_filtered<false>(a, stream);
  if (a.D == 128)
    return a.paged ? launch_full_select_t<128, true, false>(a, 1, a.k_max, a.indices, stream)
                   : launch_full_select_t<128, false, false>(a, 1, a.k_max, a.indices, stream);
  return a.paged ? launch_full_select_t<64, true, false>(a, 1, a.k_max, a.indices, stream)
                 : launch_full_select_t<64, false, false>(a, 1, a.k_max, a.indices, stream);
}

}  // namespace cs
