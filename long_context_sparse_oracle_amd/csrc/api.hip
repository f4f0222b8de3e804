// C ABI of libctxsparse.so: argument validation, workspace layout and launch sizing.  Every
// entry point validates on the host before touching the GPU and queues its kernels on the
// caller's stream without synchronising or allocating.
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>

#include "../../include/ctxsparse.h"
#include "launch.h"

// Fixed device scratch of sparse_decode_attn_noalloc (split partials), one copy per GPU, held
// until the process ends.  Host code never uses this name as an address: the device address is
// resolved per device with hipGetSymbolAddress (noalloc_scratch below).
static __device__ __align__(256) unsigned char scratch[CS_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxGT = 64;             // query rows per KV head (G * T): four 16-row MFMA tiles
constexpr int kTopkMaxLen = 262144;    // select kernel keeps two position bitmaps in LDS
constexpr int kMaxDevices = 64;
constexpr size_t kAlign = 256;

std::atomic<int> g_cu_count[kMaxDevices];

// Compute-unit count of the current device (an immutable property, cached per device).
int cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  int n = g_cu_count[dev].load(std::memory_order_relaxed);
  if (n > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = 256;
  g_cu_count[dev].store(n, std::memory_order_relaxed);
  return n;
}

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }
bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
int ilog2(int x) {
  int r = 0;
  while ((1 << r) < x) ++r;
  return r;
}

cs_status check_shape(const cs_decode_shape* s) {
  if (!s) return CS_ERR_INVALID_ARG;
  if (s->batch < 1 || s->q_len < 1 || s->num_q_heads < 1 || s->num_kv_heads < 1)
    return CS_ERR_INVALID_ARG;
  if (s->num_q_heads % s->num_kv_heads) return CS_ERR_INVALID_ARG;
  if (s->head_dim != 64 && s->head_dim != 128) return CS_ERR_UNSUPPORTED;
  const int64_t gt = (int64_t)(s->num_q_heads / s->num_kv_heads) * s->q_len;
  if (gt > kMaxGT) return CS_ERR_UNSUPPORTED;
  if ((int64_t)s->batch * s->num_kv_heads > 65535) return CS_ERR_UNSUPPORTED;
  if ((int64_t)s->batch * s->q_len * s->num_q_heads > (int64_t)INT32_MAX / 4096)
    return CS_ERR_UNSUPPORTED;
  return CS_OK;
}

cs_status check_kv(const cs_decode_shape* s, const cs_kv_desc* kv) {
  if (!kv) return CS_ERR_INVALID_ARG;
  if (!kv->k || !kv->v || !kv->seq_lens) return CS_ERR_INVALID_ARG;
  if (!aligned(kv->k, 16) || !aligned(kv->v, 16) || !aligned(kv->seq_lens, 4))
    return CS_ERR_INVALID_ARG;
  if (kv->max_len < 1 || kv->max_len < s->q_len) return CS_ERR_INVALID_ARG;
  if (kv->layout == CS_KV_CONTIGUOUS) return CS_OK;
  if (kv->layout != CS_KV_PAGED) return CS_ERR_INVALID_ARG;
  if (kv->page_size < 1 || kv->max_pages < 1 || kv->num_pages < 1 || !kv->page_table)
    return CS_ERR_INVALID_ARG;
  if (!is_pow2(kv->page_size) || kv->page_size < 16 || kv->page_size > 4096)
    return CS_ERR_UNSUPPORTED;
  if ((int64_t)kv->max_len > (int64_t)kv->max_pages * kv->page_size) return CS_ERR_INVALID_ARG;
  if (!aligned(kv->page_table, 4)) return CS_ERR_INVALID_ARG;
  return CS_OK;
}

cs::KVArgs make_kv(const cs_decode_shape* s, const cs_kv_desc* kv) {
  cs::KVArgs a;
  a.k = static_cast<const uint16_t*>(kv->k);
  a.v = static_cast<const uint16_t*>(kv->v);
  a.seq_lens = kv->seq_lens;
  a.max_len = kv->max_len;
  a.num_kv_heads = s->num_kv_heads;
  if (kv->layout == CS_KV_PAGED) {
    a.page_table = kv->page_table;
    a.page_shift = ilog2(kv->page_size);
    a.max_pages = kv->max_pages;
    a.num_pages = kv->num_pages;
  } else {
    a.page_table = nullptr;
    a.page_shift = 0;
    a.max_pages = 0;
    a.num_pages = 0;
  }
  return a;
}

int64_t rows_of(const cs_decode_shape* s) {
  return (int64_t)s->batch * s->q_len * s->num_q_heads;
}
int gt_of(const cs_decode_shape* s) { return (s->num_q_heads / s->num_kv_heads) * s->q_len; }

// ---- indexer sizing
void topk_chunking(const cs_decode_shape* s, const cs_kv_desc* kv, int* chunk, int* chunks) {
  const int64_t groups = (int64_t)s->batch * s->num_kv_heads * ceil_div(gt_of(s), 16);
  const int64_t target = 4LL * cu_count();
  int64_t c = ceil_div(groups * kv->max_len, target);
  c = ceil_div(c, 256) * 256;
  if (c < 1024) c = 1024;
  if (c > 16384) c = 16384;
  *chunk = (int)c;
  *chunks = (int)ceil_div(kv->max_len, c);
}

// Filtered indexer (candidates only) for lists of at most 1/16 of the cache; its score pass
// runs 4-wave workgroups over chunks of >= 1024 positions, about 16 per compute unit over the
// call, so ragged lengths still leave the last wave of workgroups short.  When the sample pass is
// split (at most half as many (request, KV head, 16-row tile) groups as compute units, and on the
// sketch at most 4 query rows per tile), every candidate workgroup repeats its rows' threshold
// searches, and longer chunks pay: about 4 per unit on the exact indexer (Qwen-shaped tiles of 8
// rows at 131072 positions 6% faster, 16 requests x 8 KV heads at 131072 2%, 4 rows at 32768 1%)
// and 8 on the sketch, whose short candidate workgroups lost 2% at 4 per unit on the last.
// `sketch` selects the reduced-byte indexer's rule.
void cand_chunking(const cs_decode_shape* s, const cs_kv_desc* kv, bool sketch, int* chunk, int* chunks) {
  const int64_t groups = (int64_t)s->batch * s->num_kv_heads * ceil_div(gt_of(s), 16);
  const bool split = 2 * groups <= cu_count() && (!sketch || gt_of(s) <= 4);
  const int64_t target = (split ? (sketch ? 8LL : 4LL) : 16LL) * cu_count();
  int64_t c = ceil_div(groups * kv->max_len, target);
  c = ceil_div(c, 256) * 256;
  if (c < 1024) c = 1024;
  if (c > 16384) c = 16384;
  *chunk = (int)c;
  *chunks = (int)ceil_div(kv->max_len, c);
}

// Per-row pitch (floats) of the score area: the scores of every position, or the candidate slots
// of the filtered indexer (half a pair per position of every chunk).
int64_t score_stride(const cs_decode_shape* s, const cs_kv_desc* kv, bool sketch) {
  int cc, cn;
  cand_chunking(s, kv, sketch, &cc, &cn);
  const int64_t dense = ceil_div(kv->max_len, 64) * 64;
  const int64_t cand = (int64_t)cc * cn;
  return dense > cand ? dense : cand;
}

// The filtered indexer takes lists of at most 1/8 of the cache: at that bound the candidate
// threshold keeps about 19% of a row's positions, well inside a slot's capacity (half of its
// positions), and rows with more candidates than the selection's LDS key area select from the
// slots in global memory.  Against the full-score path on 16 requests x 131072 positions: k = N/20
// indexer 1033 -> 915 us, one-call step 1219 -> 1028 us; k = N/10 1055 -> 1030 and 1367 -> 1304;
// k = N/5 measured 8% slower, so it stays on the full-score path.  The candidate pass addresses the
// rows of one (request, KV head) through a buffer resource, whose size field is 32-bit: their
// score areas must span less than 2 GiB.
bool topk_filtered(const cs_decode_shape* s, const cs_kv_desc* kv, int k_max) {
  const int64_t span = (int64_t)s->q_len * s->num_q_heads * score_stride(s, kv, false) * 4;
  return (int64_t)k_max * 8 <= kv->max_len && span < (1LL << 31);
}

// ---- reduced-byte indexer sizing
constexpr int kMaxCandMult = 64;

// Entries of a row's candidate list: min(cand_mult * k_max, max_len), rounded up to 64.
int64_t sketch_list_stride(const cs_kv_desc* kv, int32_t k_max, int32_t cand_mult) {
  int64_t n = (int64_t)cand_mult * k_max;
  if (n > kv->max_len) n = kv->max_len;
  return ceil_div(n, 64) * 64;
}

// The sketch path always runs the candidate pipeline, whose buffer resource spans the score areas
// of one (request, KV head)'s rows.
bool sketch_supported(const cs_decode_shape* s, const cs_kv_desc* kv) {
  const int64_t span = (int64_t)s->q_len * s->num_q_heads * score_stride(s, kv, true) * 4;
  return span < (1LL << 31);
}

cs_status check_sketch(const cs_key_sketch* sk) {
  if (!sk || !sk->codes || !sk->scales) return CS_ERR_INVALID_ARG;
  if (!aligned(sk->codes, 16) || !aligned(sk->scales, 4)) return CS_ERR_INVALID_ARG;
  return CS_OK;
}

// Workspace of the sketch indexer (and, with `step`, of the fused step): candidate slots (or every
// sketch score), histograms of the full-score mode, slot counts, thresholds, the query rows'
// codes and scales, the candidate lists (positions, scores), then the selected lists of the step.
struct SketchWs {
  size_t scores, hist, counts, tau, q_codes, q_scales, list_pos, list_score, sel_pos, sel_score, total;
};

// Lists (m * k entries) longer than 1/16 of the cache come from every sketch score; shorter ones
// from the candidate path, whose selection reads the slots from global memory for rows with more
// candidates than its LDS key area (m = 1 at k = N/20: 939 -> 874 us; lists of N/10 measured no
// faster than from every sketch score).
bool sketch_full(const cs_decode_shape*, const cs_kv_desc* kv, int32_t k_max, int32_t cand_mult) {
  const int64_t keep = (int64_t)cand_mult * k_max;
  return keep * 16 > kv->max_len;
}

SketchWs sketch_ws_layout(const cs_decode_shape* s, const cs_kv_desc* kv, int32_t k_max, int32_t cand_mult,
                          bool step) {
  const size_t rows = (size_t)rows_of(s);
  int cc, cn;
  cand_chunking(s, kv, true, &cc, &cn);
  const size_t ls = (size_t)sketch_list_stride(kv, k_max, cand_mult);
  SketchWs w;
  w.scores = 0;
  w.hist = w.scores + align_up(rows * (size_t)score_stride(s, kv, true) * sizeof(float));
  // histograms of the full-score mode, else the sample key prefixes of a split sample pass
  w.counts = w.hist + (sketch_full(s, kv, k_max, cand_mult) ? align_up(rows * 4096 * sizeof(uint32_t))
                                                            : align_up(rows * cs::kTauSamples * sizeof(uint16_t)));
  w.tau = w.counts + align_up(rows * (size_t)cn * 4 * sizeof(uint32_t));
  w.q_codes = w.tau + align_up(rows * sizeof(float));
  w.q_scales = w.q_codes + align_up(rows * (size_t)s->head_dim);
  w.list_pos = w.q_scales + align_up(rows * sizeof(float));
  w.list_score = w.list_pos + align_up(rows * ls * sizeof(int32_t));
  w.sel_pos = w.list_score + align_up(rows * ls * sizeof(float));
  w.sel_score = w.sel_pos + (step ? align_up(rows * (size_t)k_max * sizeof(int32_t)) : 0);
  w.total = w.sel_score + (step ? align_up(rows * (size_t)k_max * sizeof(float)) : 0);
  return w;
}

struct TopkWs {
  size_t scores, hist, counts, tau, total;
};

TopkWs topk_ws_layout(const cs_decode_shape* s, const cs_kv_desc* kv) {
  const size_t rows = (size_t)rows_of(s);
  int cc, cn;
  cand_chunking(s, kv, false, &cc, &cn);
  TopkWs w;
  w.scores = 0;
  w.hist = w.scores + align_up(rows * (size_t)score_stride(s, kv, false) * sizeof(float));
  w.counts = w.hist + align_up(rows * 4096 * sizeof(uint32_t));
  w.tau = w.counts + align_up(rows * (size_t)cn * 4 * sizeof(uint32_t));
  w.total = w.tau + align_up(rows * sizeof(float));
  return w;
}

size_t topk_ws(const cs_decode_shape* s, const cs_kv_desc* kv) { return topk_ws_layout(s, kv).total; }

// ---- attention sizing
// Gather plan: splits per row, entries per split, waves per workgroup and the entries a wave
// takes per round (kSparseWaveEntries, or kSparseWaveEntriesBig for many rows).
struct SparsePlan {
  int S, chunk, waves, entries;
};

SparsePlan sparse_plan(const cs_decode_shape* s, int k_max, int requested) {
  // One workgroup of up to kSparseWaves waves per row, looping over its list kSparseWaveEntries
  // entries per wave and round: no partials and no combine pass.  Only when there are fewer rows
  // than compute units are lists split, to put every unit to work, and only lists that take more
  // than one round of a workgroup (splitting a one-round list shortens nothing and adds the
  // combine pass).
  const int64_t rows = rows_of(s);
  const int entries = rows >= 2LL * cu_count() && k_max >= cs::kSparseWaves * cs::kSparseWaveEntriesBig
                          ? cs::kSparseWaveEntriesBig
                          : cs::kSparseWaveEntries;
  const int64_t waves_needed = ceil_div(k_max, entries);
  int64_t S;
  if (requested > 0) {
    S = requested;
  } else if (rows >= cu_count() || waves_needed <= cs::kSparseWaves) {
    S = 1;
  } else {
    S = ceil_div(cu_count(), rows);
    if (S > waves_needed) S = waves_needed;
  }
  if (S > k_max) S = k_max;
  if (S > 1024) S = 1024;
  if (S < 1) S = 1;
  const int64_t chunk = ceil_div(k_max, S);  // every split non-empty
  SparsePlan p;
  p.S = (int)ceil_div(k_max, chunk);
  p.chunk = (int)chunk;
  const int64_t w = ceil_div(chunk, entries);
  p.waves = (int)(w > cs::kSparseWaves ? cs::kSparseWaves : w);
  p.entries = entries;
  return p;
}

int dense_splits(const cs_decode_shape* s, const cs_kv_desc* kv, int requested, int* chunk_out) {
  int64_t S;
  if (requested > 0) {
    S = requested;
  } else {
    const int64_t groups = (int64_t)s->batch * s->num_kv_heads * ceil_div(gt_of(s), 16);
    S = ceil_div(4LL * cu_count(), groups);
    // chunks of at most 16384 positions: in a ragged batch a workgroup's chunk may be the last
    // one still streaming, and longer chunks leave a long tail (32 requests of 8192-131072
    // positions: 1837 us with 32768-position chunks, 1673 us with 16384)
    const int64_t min_S = ceil_div(kv->max_len, 16384);
    if (S < min_S) S = min_S;
    const int64_t by_len = ceil_div(kv->max_len, 256);
    if (S > by_len) S = by_len;
  }
  if (kv->layout == CS_KV_PAGED) {
    // a paged chunk's page ids are staged in LDS: keep them within 8192 ids (32 KB)
    const int64_t max_chunk = (8190LL * kv->page_size) / 64 * 64;
    const int64_t min_S = ceil_div(kv->max_len, max_chunk);
    if (S < min_S) S = min_S;
  }
  if (S > 1024) S = 1024;
  if (S < 1) S = 1;
  int64_t chunk = ceil_div(ceil_div(kv->max_len, S), 64) * 64;
  S = ceil_div(kv->max_len, chunk);
  *chunk_out = (int)chunk;
  return (int)S;
}

size_t attn_ws(const cs_decode_shape* s, int S) {
  if (S <= 1) return 0;
  const size_t rows = (size_t)rows_of(s);
  return align_up(rows * S * (size_t)s->head_dim * sizeof(float)) + align_up(rows * S * 2 * sizeof(float));
}

// Device address of `scratch` on the current device, resolved on the first call on that device
// and kept per device (each GPU holds its own copy at its own address).
std::atomic<void*> g_scratch_ptr[kMaxDevices];

hipError_t noalloc_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return hipSuccess;
}

cs_status check_ws(void* ws, size_t bytes, size_t need) {
  if (need == 0) return CS_OK;
  if (!ws || !aligned(ws, 16)) return CS_ERR_INVALID_ARG;
  if (bytes < need) return CS_ERR_WORKSPACE_TOO_SMALL;
  return CS_OK;
}


// ---- launch descriptors
cs::TopkLaunch topk_launch(const cs_decode_shape* shape, const void* q, const cs_kv_desc* kv,
                           float sm_scale, const int32_t* k_per_req, int32_t k_max, int32_t* indices,
                           void* workspace) {
  cs::TopkLaunch a;
  a.fused = false;
  a.sketch = false;
  a.sketch_full = false;
  a.sk = cs::SketchArgs{nullptr, nullptr, nullptr, nullptr};
  a.cand_mult = 1;
  a.list_pos = nullptr;
  a.list_score = nullptr;
  a.list_stride = 0;
  a.sel_pos = nullptr;
  a.sel_score = nullptr;
  a.out = nullptr;
  a.lse = nullptr;
  a.q = static_cast<const uint16_t*>(q);
  a.kv = make_kv(shape, kv);
  a.B = shape->batch;
  a.T = shape->q_len;
  a.Hq = shape->num_q_heads;
  a.G = shape->num_q_heads / shape->num_kv_heads;
  a.GT = gt_of(shape);
  a.D = shape->head_dim;
  a.rows = (int)rows_of(shape);
  a.cus = cu_count();
  a.paged = kv->layout == CS_KV_PAGED;
  a.scale = sm_scale;
  a.k_per_req = k_per_req;
  a.k_max = k_max;
  topk_chunking(shape, kv, &a.chunk, &a.chunks);
  cand_chunking(shape, kv, false, &a.cand_chunk, &a.cand_chunks);
  a.filtered = topk_filtered(shape, kv, k_max);
  a.small = kv->max_len <= cs::kTauSamples;  // every position is scored and selected in one kernel
  a.keep_scores = false;
  char* ws = static_cast<char*>(workspace);
  const TopkWs lay = topk_ws_layout(shape, kv);
  a.score_stride = score_stride(shape, kv, false);
  a.scores = reinterpret_cast<float*>(ws + lay.scores);
  a.hist = reinterpret_cast<uint32_t*>(ws + lay.hist);
  a.counts = reinterpret_cast<uint32_t*>(ws + lay.counts);
  a.tau = reinterpret_cast<float*>(ws + lay.tau);
  a.tau_prefixes = reinterpret_cast<uint16_t*>(ws + lay.hist);  // the histograms' area (unused by that path)
  a.indices = indices;
  return a;
}

cs::AttnLaunch sparse_launch(const cs_decode_shape* shape, const void* q, const cs_kv_desc* kv,
                             const int32_t* indices, int32_t k_max, float sm_scale,
                             const SparsePlan& plan, float* out, float* lse, void* workspace) {
  const int S = plan.S;
  cs::AttnLaunch a;
  a.q = static_cast<const uint16_t*>(q);
  a.kv = make_kv(shape, kv);
  a.B = shape->batch;
  a.T = shape->q_len;
  a.Hq = shape->num_q_heads;
  a.G = shape->num_q_heads / shape->num_kv_heads;
  a.GT = gt_of(shape);
  a.D = shape->head_dim;
  a.rows = (int)rows_of(shape);
  a.paged = kv->layout == CS_KV_PAGED;
  a.scale_log2 = sm_scale * 1.4426950408889634f;
  a.indices = indices;
  a.k_max = k_max;
  a.S = S;
  a.chunk = plan.chunk;
  a.waves = plan.waves;
  a.entries = plan.entries;
  char* ws = static_cast<char*>(workspace);
  a.part_o = S > 1 ? reinterpret_cast<float*>(ws) : nullptr;
  a.part_ml = S > 1 ? reinterpret_cast<float*>(ws + align_up((size_t)a.rows * S * a.D * sizeof(float)))
                    : nullptr;
  a.out = out;
  a.lse = lse;
  return a;
}

// ---- fused decode step: indexer + sparse attention in one call
// Workspace: the indexer's, then the selected lists (int32 positions and float32 scores,
// [rows, k_max] each; on the full-score path the positions only, when the caller passes no
// index buffer).
struct StepWs {
  size_t topk, sel_pos, sel_score, total;
};

StepWs step_ws_layout(const cs_decode_shape* s, const cs_kv_desc* kv, int32_t k_max) {
  const size_t rows = (size_t)rows_of(s);
  StepWs w;
  w.topk = 0;
  w.sel_pos = align_up(topk_ws(s, kv));
  w.sel_score = w.sel_pos + align_up(rows * (size_t)k_max * sizeof(int32_t));
  w.total = w.sel_score + align_up(rows * (size_t)k_max * sizeof(float));
  return w;
}

cs_status check_sketch_call(const cs_decode_shape* shape, const void* q, const cs_kv_desc* kv,
                            const cs_key_sketch* sketch, float sm_scale, const int32_t* k_per_req,
                            int32_t k_max, int32_t cand_mult, const int32_t* indices) {
  cs_status st = check_shape(shape);
  if (st != CS_OK) return st;
  if ((st = check_kv(shape, kv)) != CS_OK) return st;
  if ((st = check_sketch(sketch)) != CS_OK) return st;
  if (!q || !aligned(q, 16)) return CS_ERR_INVALID_ARG;
  if ((indices && !aligned(indices, 4)) || (k_per_req && !aligned(k_per_req, 4))) return CS_ERR_INVALID_ARG;
  if (k_max < 1 || k_max > kv->max_len || !std::isfinite(sm_scale)) return CS_ERR_INVALID_ARG;
  if (cand_mult < 1 || cand_mult > kMaxCandMult) return CS_ERR_INVALID_ARG;
  if (kv->max_len > kTopkMaxLen || !sketch_supported(shape, kv)) return CS_ERR_UNSUPPORTED;
  return CS_OK;
}

cs::TopkLaunch sketch_launch(const cs_decode_shape* shape, const void* q, const cs_kv_desc* kv,
                             const cs_key_sketch* sketch, float sm_scale, const int32_t* k_per_req,
                             int32_t k_max, int32_t cand_mult, int32_t* indices, char* ws,
                             const SketchWs& lay) {
  cs::TopkLaunch a = topk_launch(shape, q, kv, sm_scale, k_per_req, k_max, indices, ws);
  cand_chunking(shape, kv, true, &a.cand_chunk, &a.cand_chunks);
  a.score_stride = score_stride(shape, kv, true);
  a.filtered = true;
  a.small = false;
  a.sketch = true;
  a.cand_mult = cand_mult;
  a.sk.codes = static_cast<const int8_t*>(sketch->codes);
  a.sk.scales = sketch->scales;
  a.sk.q_codes = reinterpret_cast<int8_t*>(ws + lay.q_codes);
  a.sk.q_scales = reinterpret_cast<float*>(ws + lay.q_scales);
  a.scores = reinterpret_cast<float*>(ws + lay.scores);
  a.sketch_full = sketch_full(shape, kv, k_max, cand_mult);
  a.hist = reinterpret_cast<uint32_t*>(ws + lay.hist);
  a.counts = reinterpret_cast<uint32_t*>(ws + lay.counts);
  a.tau = reinterpret_cast<float*>(ws + lay.tau);
  a.tau_prefixes = reinterpret_cast<uint16_t*>(ws + lay.hist);
  a.list_pos = reinterpret_cast<int32_t*>(ws + lay.list_pos);
  a.list_score = reinterpret_cast<float*>(ws + lay.list_score);
  a.list_stride = (int)sketch_list_stride(kv, k_max, cand_mult);
  return a;
}

}  // namespace

extern "C" {

const char* cs_status_str(cs_status s) {
  switch (s) {
    case CS_OK: return "CS_OK";
    case CS_ERR_INVALID_ARG: return "CS_ERR_INVALID_ARG";
    case CS_ERR_UNSUPPORTED: return "CS_ERR_UNSUPPORTED";
    case CS_ERR_WORKSPACE_TOO_SMALL: return "CS_ERR_WORKSPACE_TOO_SMALL";
    case CS_ERR_HIP: return "CS_ERR_HIP";
    case CS_ERR_SCRATCH_LIMIT: return "CS_ERR_SCRATCH_LIMIT";
  }
  return "CS_ERR_UNKNOWN";
}

int32_t cs_version(void) { return 100; }

size_t topk_index_workspace_size(const cs_decode_shape* shape, const cs_kv_desc* kv, int32_t k_max) {
  (void)k_max;
  if (check_shape(shape) != CS_OK || check_kv(shape, kv) != CS_OK) return 0;
  return topk_ws(shape, kv);
}

cs_status topk_index(const cs_decode_shape* shape, const void* q, const cs_kv_desc* kv,
                     float sm_scale, const int32_t* k_per_req, int32_t k_max, int32_t* indices,
                     void* workspace, size_t workspace_bytes, void* stream) {
  cs_status st = check_shape(shape);
  if (st != CS_OK) return st;
  if ((st = check_kv(shape, kv)) != CS_OK) return st;
  if (!q || !indices || !aligned(q, 16) || !aligned(indices, 4)) return CS_ERR_INVALID_ARG;
  if (k_per_req && !aligned(k_per_req, 4)) return CS_ERR_INVALID_ARG;
  if (k_max < 1 || k_max > kv->max_len) return CS_ERR_INVALID_ARG;
  if (!std::isfinite(sm_scale)) return CS_ERR_INVALID_ARG;
  if (kv->max_len > kTopkMaxLen) return CS_ERR_UNSUPPORTED;
  const size_t need = topk_ws(shape, kv);
  if ((st = check_ws(workspace, workspace_bytes, need)) != CS_OK) return st;

  cs::TopkLaunch a = topk_launch(shape, q, kv, sm_scale, k_per_req, k_max, indices, workspace);
  hipError_t e = cs::launch_topk(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? CS_OK : CS_ERR_HIP;
}

size_t sparse_decode_attn_workspace_size(const cs_decode_shape* shape, int32_t k_max,
                                         int32_t num_splits) {
  if (check_shape(shape) != CS_OK || k_max < 1 || num_splits < 0) return 0;
  return attn_ws(shape, sparse_plan(shape, k_max, num_splits).S);
}

cs_status sparse_decode_attn(const cs_decode_shape* shape, const void* q, const cs_kv_desc* kv,
                             const int32_t* indices, int32_t k_max, float sm_scale,
                             int32_t num_splits, float* out, float* lse, void* workspace,
                             size_t workspace_bytes, void* stream) {
  cs_status st = check_shape(shape);
  if (st != CS_OK) return st;
  if ((st = check_kv(shape, kv)) != CS_OK) return st;
  if (!q || !indices || !out || !lse) return CS_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(indices, 4) || !aligned(out, 4) || !aligned(lse, 4))
    return CS_ERR_INVALID_ARG;
  if (k_max < 1 || num_splits < 0 || !std::isfinite(sm_scale)) return CS_ERR_INVALID_ARG;
  const SparsePlan plan = sparse_plan(shape, k_max, num_splits);
  const int S = plan.S;
  const size_t need = attn_ws(shape, S);
  if ((st = check_ws(workspace, workspace_bytes, need)) != CS_OK) return st;

  cs::AttnLaunch a = sparse_launch(shape, q, kv, indices, k_max, sm_scale, plan, out, lse, workspace);
  hipError_t e = cs::launch_sparse(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? CS_OK : CS_ERR_HIP;
}

cs_status sparse_decode_attn_noalloc(const cs_decode_shape* shape, const void* q, const cs_kv_desc* kv,
                                     const int32_t* indices, int32_t k_max, float sm_scale,
                                     int32_t num_splits, float* out, float* lse, void* stream) {
  cs_status st = check_shape(shape);
  if (st != CS_OK) return st;
  if ((st = check_kv(shape, kv)) != CS_OK) return st;
  if (!q || !indices || !out || !lse) return CS_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(indices, 4) || !aligned(out, 4) || !aligned(lse, 4))
    return CS_ERR_INVALID_ARG;
  if (k_max < 1 || num_splits < 0 || !std::isfinite(sm_scale)) return CS_ERR_INVALID_ARG;
  const SparsePlan plan = sparse_plan(shape, k_max, num_splits);
  if (attn_ws(shape, plan.S) > CS_NOALLOC_SCRATCH_BYTES) return CS_ERR_SCRATCH_LIMIT;
  void* ws = nullptr;
  if (plan.S > 1 && noalloc_scratch(&ws) != hipSuccess) return CS_ERR_HIP;
  // the partials of every split are written before the combine reads them: nothing to clear
  cs::AttnLaunch a = sparse_launch(shape, q, kv, indices, k_max, sm_scale, plan, out, lse, ws);
  hipError_t e = cs::launch_sparse(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? CS_OK : CS_ERR_HIP;
}

size_t sparse_decode_step_workspace_size(const cs_decode_shape* shape, const cs_kv_desc* kv,
                                         int32_t k_max) {
  if (check_shape(shape) != CS_OK || check_kv(shape, kv) != CS_OK || k_max < 1 || k_max > kv->max_len)
    return 0;
  return step_ws_layout(shape, kv, k_max).total;
}

cs_status sparse_decode_step(const cs_decode_shape* shape, const void* q, const cs_kv_desc* kv,
                             float sm_scale, const int32_t* k_per_req, int32_t k_max,
                             int32_t* indices, float* out, float* lse, void* workspace,
                             size_t workspace_bytes, void* stream) {
  cs_status st = check_shape(shape);
  if (st != CS_OK) return st;
  if ((st = check_kv(shape, kv)) != CS_OK) return st;
  if (!q || !out || !lse || !aligned(q, 16) || !aligned(out, 4) || !aligned(lse, 4))
    return CS_ERR_INVALID_ARG;
  if ((indices && !aligned(indices, 4)) || (k_per_req && !aligned(k_per_req, 4))) return CS_ERR_INVALID_ARG;
  if (k_max < 1 || k_max > kv->max_len || !std::isfinite(sm_scale)) return CS_ERR_INVALID_ARG;
  if (kv->max_len > kTopkMaxLen) return CS_ERR_UNSUPPORTED;
  const StepWs lay = step_ws_layout(shape, kv, k_max);
  if ((st = check_ws(workspace, workspace_bytes, lay.total)) != CS_OK) return st;
  char* ws = static_cast<char*>(workspace);
  hipStream_t hs = static_cast<hipStream_t>(stream);
  int32_t* sel_pos = reinterpret_cast<int32_t*>(ws + lay.sel_pos);
  cs::TopkLaunch a = topk_launch(shape, q, kv, sm_scale, k_per_req, k_max, indices, ws + lay.topk);
  if (a.filtered && !a.small) {
    // selection and attention of a row in one workgroup, on the candidates' own scores
    a.fused = true;
    a.sel_pos = sel_pos;
    a.sel_score = reinterpret_cast<float*>(ws + lay.sel_score);
    a.out = out;
    a.lse = lse;
    hipError_t e = cs::launch_topk(a, hs);
    return e == hipSuccess ? CS_OK : CS_ERR_HIP;
  }
  // full-score path (or a cache short enough to be scored whole in one kernel): the index lists
  // (the caller's buffer, else the workspace), then the attention over them on the scores the
  // indexer left in its workspace (V rows only)
  a.indices = indices ? indices : sel_pos;
  a.keep_scores = true;
  a.out = out;
  a.lse = lse;
  hipError_t e = cs::launch_topk(a, hs);
  if (e != hipSuccess) return CS_ERR_HIP;
  e = cs::launch_attend_scores(a, hs);
  return e == hipSuccess ? CS_OK : CS_ERR_HIP;
}

// ---- reduced-byte indexer
cs_status key_sketch_build(const cs_decode_shape* shape, const cs_kv_desc* kv, int32_t last_n,
                           const cs_key_sketch* sketch, void* stream) {
  cs_status st = check_shape(shape);
  if (st != CS_OK) return st;
  if ((st = check_kv(shape, kv)) != CS_OK) return st;
  if ((st = check_sketch(sketch)) != CS_OK) return st;
  if (last_n < 0) return CS_ERR_INVALID_ARG;
  hipError_t e = cs::launch_key_sketch(make_kv(shape, kv), shape->batch, shape->head_dim, last_n,
                                       static_cast<int8_t*>(sketch->codes), sketch->scales,
                                       static_cast<hipStream_t>(stream));
  return e == hipSuccess ? CS_OK : CS_ERR_HIP;
}

size_t topk_index_sketch_workspace_size(const cs_decode_shape* shape, const cs_kv_desc* kv, int32_t k_max,
                                        int32_t cand_mult) {
  if (check_shape(shape) != CS_OK || check_kv(shape, kv) != CS_OK || k_max < 1 || k_max > kv->max_len ||
      cand_mult < 1 || cand_mult > kMaxCandMult)
    return 0;
  return sketch_ws_layout(shape, kv, k_max, cand_mult, false).total;
}

cs_status topk_index_sketch(const cs_decode_shape* shape, const void* q, const cs_kv_desc* kv,
                            const cs_key_sketch* sketch, float sm_scale, const int32_t* k_per_req,
                            int32_t k_max, int32_t cand_mult, int32_t* indices, void* workspace,
                            size_t workspace_bytes, void* stream) {
  cs_status st = check_sketch_call(shape, q, kv, sketch, sm_scale, k_per_req, k_max, cand_mult, indices);
  if (st != CS_OK) return st;
  if (!indices) return CS_ERR_INVALID_ARG;
  const SketchWs lay = sketch_ws_layout(shape, kv, k_max, cand_mult, false);
  if ((st = check_ws(workspace, workspace_bytes, lay.total)) != CS_OK) return st;
  cs::TopkLaunch a = sketch_launch(shape, q, kv, sketch, sm_scale, k_per_req, k_max, cand_mult, indices,
                                   static_cast<char*>(workspace), lay);
  hipError_t e = cs::launch_topk(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? CS_OK : CS_ERR_HIP;
}

size_t sparse_decode_step_sketch_workspace_size(const cs_decode_shape* shape, const cs_kv_desc* kv,
                                                int32_t k_max, int32_t cand_mult) {
  if (check_shape(shape) != CS_OK || check_kv(shape, kv) != CS_OK || k_max < 1 || k_max > kv->max_len ||
      cand_mult < 1 || cand_mult > kMaxCandMult)
    return 0;
  return sketch_ws_layout(shape, kv, k_max, cand_mult, true).total;
}

cs_status sparse_decode_step_sketch(const cs_decode_shape* shape, const void* q, const cs_kv_desc* kv,
                                    const cs_key_sketch* sketch, float sm_scale, const int32_t* k_per_req,
                                    int32_t k_max, int32_t cand_mult, int32_t* indices, float* out,
                                    float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  cs_status st = check_sketch_call(shape, q, kv, sketch, sm_scale, k_per_req, k_max, cand_mult, indices);
  if (st != CS_OK) return st;
  if (!out || !lse || !aligned(out, 4) || !aligned(lse, 4)) return CS_ERR_INVALID_ARG;
  const SketchWs lay = sketch_ws_layout(shape, kv, k_max, cand_mult, true);
  if ((st = check_ws(workspace, workspace_bytes, lay.total)) != CS_OK) return st;
  char* ws = static_cast<char*>(workspace);
  cs::TopkLaunch a = sketch_launch(shape, q, kv, sketch, sm_scale, k_per_req, k_max, cand_mult, indices, ws, lay);
  a.fused = true;
  a.sel_pos = reinterpret_cast<int32_t*>(ws + lay.sel_pos);
  a.sel_score = reinterpret_cast<float*>(ws + lay.sel_score);
  a.out = out;
  a.lse = lse;
  hipError_t e = cs::launch_topk(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? CS_OK : CS_ERR_HIP;
}

size_t dense_decode_attn_workspace_size(const cs_decode_shape* shape, const cs_kv_desc* kv,
                                        int32_t num_splits) {
  if (check_shape(shape) != CS_OK || check_kv(shape, kv) != CS_OK || num_splits < 0) return 0;
  int chunk;
  return attn_ws(shape, dense_splits(shape, kv, num_splits, &chunk));
}

cs_status dense_decode_attn(const cs_decode_shape* shape, const void* q, const cs_kv_desc* kv,
                            float sm_scale, int32_t num_splits, float* out, float* lse,
                            void* workspace, size_t workspace_bytes, void* stream) {
  cs_status st = check_shape(shape);
  if (st != CS_OK) return st;
  if ((st = check_kv(shape, kv)) != CS_OK) return st;
  if (!q || !out || !lse || !aligned(q, 16) || !aligned(out, 4) || !aligned(lse, 4))
    return CS_ERR_INVALID_ARG;
  if (num_splits < 0 || !std::isfinite(sm_scale)) return CS_ERR_INVALID_ARG;
  int chunk;
  const int S = dense_splits(shape, kv, num_splits, &chunk);
  const size_t need = attn_ws(shape, S);
  if ((st = check_ws(workspace, workspace_bytes, need)) != CS_OK) return st;

  cs::AttnLaunch a;
  a.q = static_cast<const uint16_t*>(q);
  a.kv = make_kv(shape, kv);
  a.B = shape->batch;
  a.T = shape->q_len;
  a.Hq = shape->num_q_heads;
  a.G = shape->num_q_heads / shape->num_kv_heads;
  a.GT = gt_of(shape);
  a.D = shape->head_dim;
  a.rows = (int)rows_of(shape);
  a.paged = kv->layout == CS_KV_PAGED;
  a.scale_log2 = sm_scale * 1.4426950408889634f;
  a.indices = nullptr;
  a.k_max = 0;
  a.S = S;
  a.chunk = chunk;
  a.waves = 0;
  a.entries = 0;
  char* ws = static_cast<char*>(workspace);
  a.part_o = S > 1 ? reinterpret_cast<float*>(ws) : nullptr;
  a.part_ml = S > 1 ? reinterpret_cast<float*>(ws + align_up((size_t)a.rows * S * a.D * sizeof(float)))
                    : nullptr;
  a.out = out;
  a.lse = lse;
  hipError_t e = cs::launch_dense(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? CS_OK : CS_ERR_HIP;
}

}  // extern "C"
