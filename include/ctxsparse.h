/*
 * ctxsparse — oracle top-k context-sparse decode attention for AMD Instinct MI355X (gfx950).
 *
 * C ABI of libctxsparse.so.  Every pointer argument named "device" is GPU memory; the library
 * never allocates, frees or synchronises: all work is queued on the caller's HIP stream and the
 * caller owns every buffer, including the workspace.  Calls return before the GPU work finishes.
 * No global mutable state is kept, so calls from several host threads are safe as long as they
 * do not share a workspace while in flight.
 *
 * The method follows the pages summarising "Inference Time Context Sparsity: Illusion or
 * Opportunity?":
 *   - oracle top-k: exact selection of the k highest-scoring cached tokens, made separately for
 *     every decode token, query and head (technical summary, section 2, sparsity mechanisms);
 *   - sparse decode attention: softmax attention over only the selected tokens, so a decode step
 *     moves O(k d) instead of O(N d) bytes (section 3.C, bandwidth-efficiency bullet);
 *   - dense decode attention over every cached token as the same-GPU baseline (section 1: the
 *     linear bandwidth cost of dense decoding).
 * Split evaluation with a log-sum-exp merge is the tiling-with-online-softmax technique named in
 * the FlashSFA summary ("Scaling Attention via Feature Sparsity", system implementation).
 *
 * Notation.  B requests, T new query tokens per request, Hq query heads, Hkv KV heads,
 * G = Hq / Hkv, d = head_dim.  L_b = seq_lens[b] is request b's cached length counting its T new
 * tokens.  Query head hq reads KV head hq / G.  A "row" is one (b, t, hq).  Token t sees the
 * positions 0 .. L_b - T + t (its "visible" range, of length L_b - T + t + 1).
 * Scores are s_n = (q . K_n) * sm_scale in float32; sm_scale is normally 1/sqrt(d).
 */
#ifndef CTXSPARSE_H_
#define CTXSPARSE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes.  Any non-OK return means nothing was queued on the stream, except
 * CS_ERR_HIP, which reports a failed kernel launch (work queued before it may have run). */
typedef enum {
  CS_OK = 0,
  CS_ERR_INVALID_ARG = 1,         /* null pointer, non-positive or inconsistent size */
  CS_ERR_UNSUPPORTED = 2,         /* valid but not implemented: head_dim other than 64/128, ... */
  CS_ERR_WORKSPACE_TOO_SMALL = 3, /* workspace_bytes below the *_workspace_size() figure */
  CS_ERR_HIP = 4,                 /* hipGetLastError() reported a launch failure */
  CS_ERR_SCRATCH_LIMIT = 5,       /* sparse_decode_attn_noalloc: the call needs more scratch than
                                     CS_NOALLOC_SCRATCH_BYTES */
  /* not statuses: they give the type the range of a 32-bit int, so any int a caller passes to
     cs_status_str is a valid value of the type */
  CS_STATUS_RANGE_MIN_ = -2147483647 - 1,
  CS_STATUS_RANGE_MAX_ = 2147483647
} cs_status;

/* Problem shape of one decode step (host memory). */
typedef struct {
  int32_t batch;        /* B  >= 1 */
  int32_t q_len;        /* T  >= 1: new tokens per request (multi-token decode when > 1) */
  int32_t num_q_heads;  /* Hq >= 1, a multiple of num_kv_heads */
  int32_t num_kv_heads; /* Hkv >= 1 */
  int32_t head_dim;     /* d: 64 or 128 */
} cs_decode_shape;

enum { CS_KV_CONTIGUOUS = 0, CS_KV_PAGED = 1 };

/* KV cache descriptor (host struct, device pointers).  K and V are bf16.
 *   CS_KV_CONTIGUOUS: k, v are [B, Hkv, max_len, d]; position n of (b, h) is row n.
 *   CS_KV_PAGED:      k, v are pools [num_pages, Hkv, page_size, d]; logical position n of request
 *                     b lives in page page_table[b * max_pages + n / page_size], slot
 *                     n % page_size.  page_size is a power of two in [16, 4096].
 * max_len is a host-side bound on every seq_lens[b] (for paged caches at most
 * max_pages * page_size); it sizes grids and workspaces.  Device data is trusted as follows:
 * seq_lens[b] is clamped to [0, max_len] and page ids to [0, num_pages - 1] inside the kernels, so
 * bad values give wrong results but never out-of-bounds reads. */
typedef struct {
  const void* k;             /* device bf16 */
  const void* v;             /* device bf16 */
  int32_t layout;            /* CS_KV_CONTIGUOUS or CS_KV_PAGED */
  int32_t max_len;           /* >= 1 */
  int32_t page_size;         /* paged only */
  int32_t max_pages;         /* paged only: columns of page_table */
  int32_t num_pages;         /* paged only: pool size */
  const int32_t* page_table; /* paged only: device int32 [B, max_pages] */
  const int32_t* seq_lens;   /* device int32 [B]: L_b, each >= T for a meaningful step */
} cs_kv_desc;

/* Human-readable name of a status code (static string, never NULL). */
const char* cs_status_str(cs_status s);

/* Library version as major * 10000 + minor * 100 + patch. */
int32_t cs_version(void);

/* ------------------------------------------------------------------------------------------
 * topk_index — oracle top-k indexer (a1 score + a2 select).
 *
 * For every row (b, t, hq) with k' = min(k_b, visible), writes the k' visible positions with the
 * largest float32 scores s_n = (q[b,t,hq] . K[b, hq/G, n]) * sm_scale, the lower position first
 * among equal scores (-0.0 equals +0.0), in ascending position order, then -1 up to k_max.
 *
 *   q          device bf16 [B, T, Hq, d]
 *   k_per_req  device int32 [B] (k_b, clamped to [0, k_max]) or NULL: every request uses k_max
 *   k_max      1 <= k_max <= max_len; row stride of `indices`
 *   indices    device int32 [B, T, Hq, k_max] (written)
 *   workspace  device scratch of at least topk_index_workspace_size() bytes, 256-byte aligned
 *   stream     hipStream_t (NULL: the default stream)
 * Errors: CS_ERR_INVALID_ARG for null pointers / bad sizes / non-finite sm_scale,
 * CS_ERR_UNSUPPORTED for head_dim not in {64, 128} or G * T > 64, CS_ERR_WORKSPACE_TOO_SMALL.
 * ------------------------------------------------------------------------------------------ */
size_t topk_index_workspace_size(const cs_decode_shape* shape, const cs_kv_desc* kv, int32_t k_max);
cs_status topk_index(const cs_decode_shape* shape, const void* q, const cs_kv_desc* kv,
                     float sm_scale, const int32_t* k_per_req, int32_t k_max, int32_t* indices,
                     void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------------------------
 * sparse_decode_attn — attention over index lists (a3 split partials + a4 log-sum-exp combine).
 *
 * For every row, over the entries I of indices[b, t, hq, 0:k_max]: entries outside the row's
 * visible range (in particular -1 padding) are skipped; every other entry counts once per
 * occurrence, in any order.  With s_i as above, m = max s_i:
 *   out[b,t,hq,:] = sum_i e^{s_i - m} V[b, hq/G, i, :] / sum_i e^{s_i - m}
 *   lse[b,t,hq]   = m + ln sum_i e^{s_i - m}          (natural log, scaled-score units)
 * A row with no valid entry gets out = 0 and lse = -inf.
 *
 *   indices     device int32 [B, T, Hq, k_max]
 *   num_splits  pieces each row's list is cut into (partials merged by log-sum-exp);
 *               0 picks a value from the shape and the GPU's compute-unit count
 *   out         device float32 [B, T, Hq, d];  lse: device float32 [B, T, Hq]
 * The workspace size depends on num_splits; pass the same value to both calls.
 * ------------------------------------------------------------------------------------------ */
size_t sparse_decode_attn_workspace_size(const cs_decode_shape* shape, int32_t k_max,
                                         int32_t num_splits);
cs_status sparse_decode_attn(const cs_decode_shape* shape, const void* q, const cs_kv_desc* kv,
                             const int32_t* indices, int32_t k_max, float sm_scale,
                             int32_t num_splits, float* out, float* lse, void* workspace,
                             size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------------------------
 * sparse_decode_attn_noalloc — sparse_decode_attn for callers that cannot allocate device
 * memory or pass a workspace (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation).  Same arguments, results and errors as sparse_decode_attn, without the
 * workspace: the split partials live in a fixed static device buffer of the library,
 * CS_NOALLOC_SCRATCH_BYTES per GPU, held until the process ends.  A call whose split plan needs
 * more (rows * splits * (d + 2) * 4 bytes, rounded up; only plans with splits > 1 use any) returns
 * CS_ERR_SCRATCH_LIMIT with nothing queued; the automatic plan (num_splits = 0) needs at most
 * about 270 KB.  Nothing is allocated or freed.  The first call on a device resolves the
 * buffer's device address (hipGetSymbolAddress), so make that first call outside graph capture.
 * Every call on one GPU shares that GPU's buffer: calls that overlap in time on one GPU (on
 * different streams, or from several threads) race and give wrong results.  Each call writes
 * the partials it reads, so the contents left by an earlier call never matter.
 * ------------------------------------------------------------------------------------------ */
#define CS_NOALLOC_SCRATCH_BYTES ((size_t)4 << 20)
cs_status sparse_decode_attn_noalloc(const cs_decode_shape* shape, const void* q,
                                     const cs_kv_desc* kv, const int32_t* indices, int32_t k_max,
                                     float sm_scale, int32_t num_splits, float* out, float* lse,
                                     void* stream);

/* ------------------------------------------------------------------------------------------
 * sparse_decode_step — the oracle-indexed decode step in one call: topk_index followed by
 * sparse_decode_attn over the lists it selects (the end-to-end step whose indexer overhead the
 * technical summary, section 3.C, counts against the sparse kernel's gain).  Same arguments and
 * results as those two calls; `indices` (device int32 [B, T, Hq, k_max]) may be NULL when the
 * lists themselves are not wanted.  For k_max <= max_len / 8 (and max_len > 1024) each row's
 * selection and its attention run in one workgroup on the scores the indexer already computed;
 * otherwise the indexer (its full-score pass, or for max_len <= 1024 the whole-row pass that
 * scores every position and selects) leaves every score in the workspace and a further kernel
 * attends over each row's list on those scores.  Either way only the V rows of the selected positions are
 * read for the attention.  out / lse agree with sparse_decode_attn over the exact top-k lists within the
 * same tolerances (the scores come from the indexer's float32 dot products).
 * Errors: as topk_index and sparse_decode_attn.
 * ------------------------------------------------------------------------------------------ */
size_t sparse_decode_step_workspace_size(const cs_decode_shape* shape, const cs_kv_desc* kv,
                                         int32_t k_max);
cs_status sparse_decode_step(const cs_decode_shape* shape, const void* q, const cs_kv_desc* kv,
                             float sm_scale, const int32_t* k_per_req, int32_t k_max,
                             int32_t* indices, float* out, float* lse, void* workspace,
                             size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------------------------
 * Reduced-byte indexer.  The technical summary (section 3.C, indexing-overhead bullet) counts
 * an indexer's own cost against the sparse kernel's gain and estimates it with an indexer that
 * scores a reduced form of each key.  This library's reduced form is an int8 key sketch: a key
 * row K_n of d bf16 values is stored as d int8 codes and one float32 scale,
 *   scale_n = max_i |K_n,i| / 127,   code_n,i = rint(K_n,i / scale_n)   (clamped to +-127),
 * divisions correctly rounded in float32, rint rounding half to even, a zero row giving scale 0
 * and codes 0.  The query row is quantised the same way, and the sketch score of position n is
 *   a_n = (scale_q * scale_n) * (codes_q . codes_n)      (exact int32 dot product, two float32
 *                                                         products rounded in that order),
 * reading d + 4 bytes per position instead of 2 d.
 *
 * Selection of a row (k' = min(k_b, visible), m = cand_mult):
 *   1. the min(m k', visible) visible positions with the largest a_n, the lower position first
 *      among equal values (exact: count(a_n >= a sampled threshold) >= m k' is checked, and a
 *      row short of candidates is rescored in full);
 *   2. of those, the k' with the largest exact float32 scores s_n, as topk_index ranks them.
 * With m k' >= visible the result is topk_index's.  Otherwise it may differ from the exact top-k
 * where the sketch ranks an exact top-k position below m k' others.
 * ------------------------------------------------------------------------------------------ */

/* An int8 key sketch (host struct, device pointers owned by the caller). */
typedef struct {
  void* codes;   /* device int8 with the K cache's shape: [B, Hkv, max_len, d] (contiguous) or
                    [num_pages, Hkv, page_size, d] (paged); 16-byte aligned */
  float* scales; /* device float32 with the same shape without d */
} cs_key_sketch;

/* key_sketch_build — writes the sketch of key positions [max(0, L_b - last_n), L_b) of every
 * request b and KV head (last_n = 0: every position [0, L_b)), through the page table for paged
 * caches; other entries are left as they are.  A decode step that appended T tokens per request
 * calls it with last_n = T.
 * Errors: CS_ERR_INVALID_ARG for null or misaligned pointers and last_n < 0; as topk_index. */
cs_status key_sketch_build(const cs_decode_shape* shape, const cs_kv_desc* kv, int32_t last_n,
                           const cs_key_sketch* sketch, void* stream);

/* topk_index_sketch — the reduced-byte indexer: topk_index's arguments and output layout, plus
 * the sketch of the cache (current for every visible position) and cand_mult in [1, 64].
 * Errors: as topk_index; CS_ERR_INVALID_ARG for a bad sketch or cand_mult; CS_ERR_UNSUPPORTED
 * when one (request, KV head)'s candidate areas would span 2 GiB or more. */
size_t topk_index_sketch_workspace_size(const cs_decode_shape* shape, const cs_kv_desc* kv,
                                        int32_t k_max, int32_t cand_mult);
cs_status topk_index_sketch(const cs_decode_shape* shape, const void* q, const cs_kv_desc* kv,
                            const cs_key_sketch* sketch, float sm_scale, const int32_t* k_per_req,
                            int32_t k_max, int32_t cand_mult, int32_t* indices, void* workspace,
                            size_t workspace_bytes, void* stream);

/* sparse_decode_step_sketch — sparse_decode_step with the reduced-byte indexer: each row's
 * selection and its attention run in one workgroup, on the exact scores of the re-rank, so only
 * the V rows of the selected positions are read for the attention.  `indices` may be NULL.
 * Errors: as topk_index_sketch and sparse_decode_step. */
size_t sparse_decode_step_sketch_workspace_size(const cs_decode_shape* shape, const cs_kv_desc* kv,
                                                int32_t k_max, int32_t cand_mult);
cs_status sparse_decode_step_sketch(const cs_decode_shape* shape, const void* q, const cs_kv_desc* kv,
                                    const cs_key_sketch* sketch, float sm_scale,
                                    const int32_t* k_per_req, int32_t k_max, int32_t cand_mult,
                                    int32_t* indices, float* out, float* lse, void* workspace,
                                    size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------------------------
 * dense_decode_attn — the same-GPU dense baseline (a5): sparse_decode_attn with every visible
 * position selected, computed by streaming each (b, KV head)'s cache once for all G * T rows.
 * num_splits: pieces the sequence axis is cut into (0: automatic).
 * ------------------------------------------------------------------------------------------ */
size_t dense_decode_attn_workspace_size(const cs_decode_shape* shape, const cs_kv_desc* kv,
                                        int32_t num_splits);
cs_status dense_decode_attn(const cs_decode_shape* shape, const void* q, const cs_kv_desc* kv,
                            float sm_scale, int32_t num_splits, float* out, float* lse,
                            void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* CTXSPARSE_H_ */
