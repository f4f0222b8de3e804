// Internal launch descriptors shared by the C-ABI layer and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"

namespace cs {

// Sparse attention launch shape: index entries a wave takes per round, and waves per workgroup.
constexpr int kSparseWaveEntries = 16;
constexpr int kSparseWaves = 8;
// With at least twice as many rows as compute units (several workgroups per unit, the gather
// bandwidth-bound) and lists long enough to give all waves full rounds, a wave takes twice as
// many entries per round: fewer, longer rounds.
constexpr int kSparseWaveEntriesBig = 32;

// Positions sampled per (request, KV head) to set the candidate threshold of the filtered indexer;
// caches of at most this many positions are scored whole and selected in one kernel.
constexpr int kTauSamples = 1024;

// int8 key sketch of the reduced-byte indexer: per key row, int8 codes in the K cache's layout
// (element offset e of K holds code e) and one float32 scale (index e / D); the query rows'
// codes and scales live in the indexer's workspace.
struct SketchArgs {
  const int8_t* codes;
  const float* scales;
  int8_t* q_codes;   // [rows, D]
  float* q_scales;   // [rows]
};

struct TopkLaunch {
  const uint16_t* q;
  KVArgs kv;
  int B, T, Hq, G, GT, D, rows;
  int cus;  // compute units of the device
  bool paged;
  float scale;
  const int32_t* k_per_req;
  int k_max;
  int chunk, chunks;
  float* scores;    // [rows, score_stride]
  int64_t score_stride;  // max_len rounded up to 64 floats
  uint32_t* hist;   // [rows, 4096]
  int32_t* indices; // [rows, k_max]
  // filtered indexer (k_max <= max_len / 8): sampled thresholds, then candidates only
  bool filtered;
  uint32_t* counts;   // [rows, cand_chunks, 4]: candidates per workgroup wave
  float* tau;         // [rows]: candidate thresholds
  uint16_t* tau_prefixes;  // [rows, kTauSamples]: sample key prefixes of a split sample pass
  // max_len <= kTauSamples: one kernel scores every position and selects; keep_scores: it also
  // writes every visible score to `scores` (the one-call step's attention reads them)
  bool small;
  bool keep_scores;
  // fused decode step (filtered path): selection and attention per row in one kernel
  bool fused;
  int32_t* sel_pos;   // [rows, k_max]
  float* sel_score;   // [rows, k_max]
  float* out;         // [rows, D]
  float* lse;         // [rows]
  int cand_chunk, cand_chunks;
  // reduced-byte indexer: candidates ranked on the sketch, cand_mult * k of them re-ranked on
  // exact scores through the list area (positions and scores, list_stride entries per row)
  bool sketch;
  bool sketch_full;  // lists from every sketch score (score + histogram, select) instead of candidates
  SketchArgs sk;
  int cand_mult;
  int32_t* list_pos;
  float* list_score;
  int list_stride;
};

struct AttnLaunch {
  const uint16_t* q;
  KVArgs kv;
  int B, T, Hq, G, GT, D, rows;
  bool paged;
  float scale_log2;
  const int32_t* indices;  // sparse only
  int k_max;               // sparse only
  int S, chunk;
  int waves;       // sparse only: waves per workgroup
  int entries;     // sparse only: index entries a wave takes per round
  float* part_o;   // [rows, S, D]
  float* part_ml;  // [rows, S, 2]
  float* out;
  float* lse;
};

size_t select_lds_bytes(int max_len);
int score_threads(int GT);  // workgroup size of the score kernel for G*T query rows
hipError_t launch_fill_u32(uint32_t* p, int64_t n, uint32_t value, hipStream_t stream);
hipError_t launch_topk(const TopkLaunch& a, hipStream_t stream);
// after launch_topk on the full-score path: attention of every row over its index list with the
// scores the indexer left in a.scores (V rows only), into a.out / a.lse
hipError_t launch_attend_scores(const TopkLaunch& a, hipStream_t stream);
// int8 sketch of key rows [max(0, L_b - last_n), L_b) of every (request, KV head) (last_n <= 0:
// all of [0, L_b)), and of `rows` contiguous query rows
hipError_t launch_key_sketch(const KVArgs& kv, int B, int D, int last_n, int8_t* codes, float* scales,
                             hipStream_t stream);
hipError_t launch_q_sketch(const uint16_t* q, int rows, int D, int8_t* codes, float* scales,
                           hipStream_t stream);
hipError_t launch_sparse(const AttnLaunch& a, hipStream_t stream);
hipError_t launch_dense(const AttnLaunch& a, hipStream_t stream);

}  // namespace cs
