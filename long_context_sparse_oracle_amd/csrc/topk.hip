// Oracle top-k indexer for gfx950: a streaming score kernel (q.K^T on MFMA, fused 12-bit
// radix histogram) and a per-row select kernel (LDS radix refinement, ballot compaction).
//
// Method: exact top-k selection of cached tokens per (request, token, query head), as used by the
// oracle indexer of "Inference Time Context Sparsity: Illusion or Opportunity?" (technical
// summary, section 2, sparsity mechanisms).  Ranking is by the float32 score
// s = (q . K) * sm_scale, larger first, lower position first among equal scores.
#include "device_common.h"
#include "launch.h"

namespace cs {

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

// ============================================================================ score + histogram
// Grid: (chunks, B * Hkv, ceil(G*T / 16)).  One workgroup (4 waves per 4 query rows, so the
// LDS histogram never starves a CU of waves) streams `chunk` positions of one (request, KV head)
// and scores them against up to 16 of the G*T query rows that read that head
// (row r = t * G + g, query head h * G + g).  Per 16-position tile a wave issues D/32
// v_mfma_f32_16x16x32_bf16: A = the 16 query rows (lane l: row l%16, 8 dims), B = K^T (lane l:
// position l%16, the same 8 dims), so each K row is read once for all rows of the group.
// Scores of visible positions go to scores[row][n]; their 12-bit key prefix is counted in an LDS
// histogram (two 16-bit counters per word) that is added to the global one at the end.
template <int D, bool PAGED>
__global__ __launch_bounds__(kScoreMaxThreads) void score_hist_kernel(
    const uint16_t* __restrict__ q, KVArgs kv, int T, int Hq, int G, float scale,
    float* __restrict__ scores, uint32_t* __restrict__ hist, int chunk, int hist_rows,
    int64_t score_stride) {
  extern __shared__ uint32_t lds_hist[];  // [hist_rows][kHistBins / 2], then the chunk's page ids
  int* lds_pages = reinterpret_cast<int*>(lds_hist + hist_rows * (kHistBins / 2));
  constexpr int KS = D / 32;              // MFMA k-steps per tile
  const int c = blockIdx.x;
  const int bh = blockIdx.y;
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

  // A operand: query row r0 + m, dims j*32 + g4*8 .. +8.
  bf16x8 a[KS];
  {
    const int r = r0 + m;
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
  // Output rows held by this lane: 4*g4 + i (i = 0..3).
  int vis[4];
  float* srow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rl = 4 * g4 + i;
    const int r = r0 + rl;
    if (rl < rows_here) {
      const int t = r / G, gi = r - (r / G) * G;
      vis[i] = L - T + t + 1;
      srow[i] = scores + (((int64_t)b * T + t) * Hq + (h * G + gi)) * score_stride;
    } else {
      vis[i] = 0;
      srow[i] = scores;
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
  auto load_tiles = [&](int n0, uint4 (&dst)[kScoreUnroll][KS]) {
#pragma unroll
    for (int u = 0; u < kScoreUnroll; ++u) {
      const int tile = min(n0 + u * 16, last);
      const int64_t off = kv_tile_staged<D, PAGED>(kv, lds_pages, start, b, h, tile) +
                          (int64_t)min(m, L - 1 - tile) * D + g4 * 8;
#pragma unroll
      for (int j = 0; j < KS; ++j) dst[u][j] = ld16(kbase + off + j * 32);
    }
  };
  auto score_tiles = [&](int n0, const uint4 (&kt)[kScoreUnroll][KS]) {
#pragma unroll
    for (int u = 0; u < kScoreUnroll; ++u) {
      const int tile = n0 + u * 16;
      if (tile >= end) break;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < KS; ++j)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[j], __builtin_bit_cast(bf16x8, kt[u][j]),
                                                      acc, 0, 0, 0);
      const int n = tile + m;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (n < vis[i]) {
          const float s = acc[i] * scale;
          srow[i][n] = s;
          const uint32_t bin = ord_key(s) >> 20;
          atomicAdd(&lds_hist[(4 * g4 + i) * (kHistBins / 2) + (bin >> 1)], 1u << ((bin & 1u) * 16));
        }
      }
    }
  };
  int n0 = start + wave * 16 * kScoreUnroll;
  load_tiles(n0, cur);
  for (; n0 < end; n0 += 2 * kStep) {
    load_tiles(n0 + kStep, nxt);
    score_tiles(n0, cur);
    if (n0 + kStep >= end) break;
    load_tiles(n0 + 2 * kStep, cur);
    score_tiles(n0 + kStep, nxt);
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
// Block-wide exclusive prefix sum over kSelThreads values.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* wsum, uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t acc = 0;
    for (int w = 0; w < kSelWaves; ++w) {
      const uint32_t t = wsum[w];
      wsum[w] = acc;
      acc += t;
    }
    wsum[kSelWaves] = acc;
  }
  __syncthreads();
  const uint32_t r = wsum[wave] + x - v;
  if (total) *total = wsum[kSelWaves];
  __syncthreads();
  return r;
}

struct SelShared {
  uint32_t wsum[kSelWaves + 1];
  uint32_t cand_count;
  uint32_t thr_bin;    // bin holding the k-th largest key
  uint32_t thr_above;  // keys in higher bins
  uint32_t thr_count;  // keys in the threshold bin
  uint32_t found;
};

// Finds, over `nbins` counters hist[0..nbins) (bin nbins-1 highest), the bin holding the need-th
// largest key.  Each thread covers nbins / kSelThreads consecutive bins, highest bins on thread 0.
// Returns the total count.
template <int PER>
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
  uint32_t above = block_excl_scan(sum, sh.wsum, &total);
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

// Per row (b, t, hq): select the kk = min(k_b, visible) largest scores.
//  1. threshold bin T12 of the 12-bit key prefix from the fused histogram (rebuilt from the scores
//     when it does not add up to the visible count);
//  2. one pass over the scores (16-byte loads): keys above T12 are marked in an LDS bitmap (8
//     lanes' 4-bit nibbles OR-reduced per 32-bit word), keys in T12 are appended to an LDS
//     candidate list;
//  3. two 10-bit radix rounds over the candidates give the exact k-th key K* and how many keys
//     equal to K* are taken (lowest positions first); when T12 holds more than kCandCap keys the
//     rounds read the scores instead;
//  4. the bitmap is emitted in ascending position order by a block prefix sum of popcounts.
__global__ __launch_bounds__(kSelThreads) void select_kernel(
    const float* __restrict__ scores, const uint32_t* __restrict__ hist,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ k_per_req, int T, int Hq,
    int max_len, int64_t score_stride, int k_max, int bitmap_words, int32_t* __restrict__ indices) {
  extern __shared__ uint32_t smem[];
  uint32_t* hist_s = smem;                      // kHistBins
  uint32_t* gt_bits = hist_s + kHistBins;       // bitmap_words
  uint32_t* eq_bits = gt_bits + bitmap_words;   // bitmap_words
  uint32_t* cand_key = eq_bits + bitmap_words;  // kCandCap
  uint32_t* cand_pos = cand_key + kCandCap;     // kCandCap
  __shared__ SelShared sh;

  const int row = blockIdx.x;
  const int b = row / (T * Hq);
  const int t = (row / Hq) - (row / (T * Hq)) * T;
  int L = seq_lens[b];
  L = L < 0 ? 0 : (L > max_len ? max_len : L);
  const int vis = max(0, L - T + t + 1);
  int kb = k_per_req ? k_per_req[b] : k_max;
  kb = kb < 0 ? 0 : (kb > k_max ? k_max : kb);
  const int kk = min(kb, vis);
  int32_t* out = indices + (int64_t)row * k_max;
  const float* srow = scores + (int64_t)row * score_stride;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;

  if (kk == vis) {  // everything visible is selected (also kk == 0)
    for (int i = tid; i < k_max; i += kSelThreads) out[i] = i < vis ? i : -1;
    return;
  }

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
  const uint4 hv = reinterpret_cast<const uint4*>(hist + (int64_t)row * kHistBins)[tid];
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
  if (total != (uint32_t)vis || !sh.found) {
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

  const int wpt = (words + kSelThreads - 1) / kSelThreads;  // bitmap words per thread
  const int w0 = tid * wpt;
  if (!take_all_eq) {
    // keep the `need` lowest positions among keys equal to K*
    uint32_t cnt = 0;
    for (int w = w0; w < min(w0 + wpt, words); ++w) cnt += __popc(eq_bits[w]);
    uint32_t before = block_excl_scan(cnt, sh.wsum, nullptr);
    for (int w = w0; w < min(w0 + wpt, words); ++w) {
      uint32_t bits = eq_bits[w];
      while (bits) {
        const uint32_t bit = bits & (0u - bits);
        if (before < need) gt_bits[w] |= bit;
        ++before;
        bits ^= bit;
      }
    }
    __syncthreads();
  }

  // ---- 4. emit ascending positions
  uint32_t cnt = 0;
  for (int w = w0; w < min(w0 + wpt, words); ++w) cnt += __popc(gt_bits[w]);
  uint32_t pos = block_excl_scan(cnt, sh.wsum, nullptr);
  for (int w = w0; w < min(w0 + wpt, words); ++w) {
    uint32_t bits = gt_bits[w];
    while (bits) {
      const int bit = __ffs(bits) - 1;
      if (pos < (uint32_t)k_max) out[pos] = w * 32 + bit;
      ++pos;
      bits &= bits - 1;
    }
  }
  for (int i = kk + tid; i < k_max; i += kSelThreads) out[i] = -1;
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

template <int D, bool PAGED>
static hipError_t launch_score_t(const TopkLaunch& a, hipStream_t stream) {
  const int rows_tile = a.GT < 16 ? a.GT : 16;
  const size_t page_ids = PAGED ? (size_t)(a.chunk >> a.kv.page_shift) + 2 : 0;
  const size_t lds = (size_t)rows_tile * (kHistBins / 2) * sizeof(uint32_t) + page_ids * sizeof(int);
  auto kern = score_hist_kernel<D, PAGED>;
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  dim3 grid(a.chunks, a.B * a.kv.num_kv_heads, (a.GT + 15) / 16);
  hipLaunchKernelGGL(kern, grid, dim3(score_threads(a.GT)), lds, stream, a.q, a.kv, a.T, a.Hq, a.G,
                     a.scale, a.scores, a.hist, a.chunk, rows_tile, a.score_stride);
  return hipGetLastError();
}

hipError_t launch_topk(const TopkLaunch& a, hipStream_t stream) {
  hipError_t e = launch_fill_u32(a.hist, (int64_t)a.rows * kHistBins, 0u, stream);
  if (e != hipSuccess) return e;
  if (a.D == 128)
    e = a.paged ? launch_score_t<128, true>(a, stream) : launch_score_t<128, false>(a, stream);
  else
    e = a.paged ? launch_score_t<64, true>(a, stream) : launch_score_t<64, false>(a, stream);
  if (e != hipSuccess) return e;
  const size_t lds = select_lds_bytes(a.kv.max_len);
  if (lds > 65536) {
    e = hipFuncSetAttribute((const void*)select_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  const int words = ((a.kv.max_len + 255) / 256) * 8;
  hipLaunchKernelGGL(select_kernel, dim3(a.rows), dim3(kSelThreads), lds, stream, a.scores,
                     a.hist, a.kv.seq_lens, a.k_per_req, a.T, a.Hq, a.kv.max_len, a.score_stride,
                     a.k_max, words, a.indices);
  return hipGetLastError();
}

}  // namespace cs
