// Internal launch descriptors shared by the C-ABI layer and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"

namespace cs {

// Sparse attention launch shape: index entries a wave takes per round, and waves per workgroup.
constexpr int kSparseWaveEntries = 16;
constexpr int kSparseWaves = 8;

struct TopkLaunch {
  const uint16_t* q;
  KVArgs kv;
  int B, T, Hq, G, GT, D, rows;
  bool paged;
  float scale;
  const int32_t* k_per_req;
  int k_max;
  int chunk, chunks;
  float* scores;    // [rows, score_stride]
  int64_t score_stride;  // max_len rounded up to 64 floats
  uint32_t* hist;   // [rows, 4096]
  int32_t* indices; // [rows, k_max]
  // filtered indexer (k_max <= max_len / 16): sampled thresholds, then candidates only
  bool filtered;
  uint32_t* sample_keys;  // [rows, 1024]: ordered keys of the sampled scores
  uint32_t* counts;   // [rows, cand_chunks, 4]: candidates per workgroup wave
  // fused decode step (filtered path): selection and attention per row in one kernel
  bool fused;
  int32_t* sel_pos;   // [rows, k_max]
  float* sel_score;   // [rows, k_max]
  float* out;         // [rows, D]
  float* lse;         // [rows]
  int cand_chunk, cand_chunks;
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
  float* part_o;   // [rows, S, D]
  float* part_ml;  // [rows, S, 2]
  float* out;
  float* lse;
};

size_t select_lds_bytes(int max_len);
int score_threads(int GT);  // workgroup size of the score kernel for G*T query rows
hipError_t launch_fill_u32(uint32_t* p, int64_t n, uint32_t value, hipStream_t stream);
hipError_t launch_topk(const TopkLaunch& a, hipStream_t stream);
hipError_t launch_sparse(const AttnLaunch& a, hipStream_t stream);
hipError_t launch_dense(const AttnLaunch& a, hipStream_t stream);

}  // namespace cs
