// Host-only stand-ins for the kernel launchers, so that the C-ABI layer (argument validation,
// workspace sizing and layout, split plans) can be built and run under AddressSanitizer and
// UndefinedBehaviorSanitizer without a GPU.  Each stub checks the launch descriptor it receives
// the way the kernels rely on it and queues nothing.
#include <cstdio>
#include <cstdlib>

#include "launch.h"

namespace cs {

static void require(bool ok, const char* what) {
  if (!ok) {
    std::fprintf(stderr, "launch descriptor check failed: %s\n", what);
    std::abort();
  }
}

size_t select_lds_bytes(int max_len) { return (size_t)max_len / 4 + 4096; }
int score_threads(int GT) { return GT <= 4 ? 256 : 1024; }
hipError_t launch_fill_u32(uint32_t* p, int64_t n, uint32_t, hipStream_t) {
  require(p != nullptr && n >= 0, "fill");
  return hipSuccess;
}
hipError_t launch_topk(const TopkLaunch& a, hipStream_t) {
  require(a.B >= 1 && a.T >= 1 && a.G >= 1 && a.GT == a.G * a.T && a.rows == a.B * a.T * a.Hq, "topk shape");
  require(a.k_max >= 1 && a.k_max <= a.kv.max_len, "topk k_max");
  require(a.chunk >= 1 && a.chunks >= 1 && (int64_t)a.chunk * a.chunks >= a.kv.max_len, "topk chunking");
  require(a.cand_chunk >= 1 && (int64_t)a.cand_chunk * a.cand_chunks >= a.kv.max_len, "cand chunking");
  require(a.score_stride >= a.kv.max_len, "score stride");
  return hipSuccess;
}
hipError_t launch_attend_scores(const TopkLaunch& a, hipStream_t) {
  require(a.out != nullptr && a.lse != nullptr, "attend outputs");
  return hipSuccess;
}
hipError_t launch_key_sketch(const KVArgs& kv, int B, int D, int, int8_t* codes, float* scales, hipStream_t) {
  require(B >= 1 && (D == 64 || D == 128) && codes && scales && kv.k, "sketch");
  return hipSuccess;
}
hipError_t launch_q_sketch(const uint16_t* q, int rows, int D, int8_t* codes, float* scales, hipStream_t) {
  require(q && rows >= 1 && (D == 64 || D == 128) && codes && scales, "q sketch");
  return hipSuccess;
}
hipError_t launch_sparse(const AttnLaunch& a, hipStream_t) {
  require(a.S >= 1 && a.chunk >= 1 && (int64_t)a.S * a.chunk >= a.k_max, "sparse plan");
  require(a.S == 1 || (a.part_o && a.part_ml), "sparse partials");
  require(a.waves >= 1 && a.waves <= kSparseWaves, "sparse waves");
  require(a.entries == kSparseWaveEntries || a.entries == kSparseWaveEntriesBig, "sparse entries");
  return hipSuccess;
}
hipError_t launch_dense(const AttnLaunch& a, hipStream_t) {
  require(a.S >= 1 && a.chunk >= 64 && (int64_t)a.S * a.chunk >= a.kv.max_len, "dense plan");
  require(a.S == 1 || (a.part_o && a.part_ml), "dense partials");
  return hipSuccess;
}

}  // namespace cs
