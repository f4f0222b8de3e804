// Drives the C ABI of libctxsparse's host layer (built with launch_stubs.cpp) through the
// argument-validation, workspace-sizing and split-plan cases, including extreme sizes, under
// AddressSanitizer and UndefinedBehaviorSanitizer.  Prints "abi cases: N passed" on success;
// any sanitizer report or mismatched status fails the run.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "ctxsparse.h"

static int failures = 0, passed = 0;
#define EXPECT(cond)                                                     \
  do {                                                                   \
    if (cond) {                                                          \
      ++passed;                                                          \
    } else {                                                             \
      ++failures;                                                        \
      std::fprintf(stderr, "FAILED line %d: %s\n", __LINE__, #cond);     \
    }                                                                    \
  } while (0)

static void* const FAKE = reinterpret_cast<void*>(0x10000);  // aligned, never dereferenced

static cs_decode_shape shape(int B = 2, int T = 1, int Hq = 8, int Hkv = 2, int d = 128) {
  return cs_decode_shape{B, T, Hq, Hkv, d};
}
static cs_kv_desc kv(int layout = CS_KV_CONTIGUOUS, int max_len = 1000, int page_size = 0, int max_pages = 0,
                     int num_pages = 0, const void* pt = nullptr, const void* k = FAKE) {
  return cs_kv_desc{k, FAKE, layout, max_len, page_size, max_pages, num_pages,
                    static_cast<const int32_t*>(pt), static_cast<const int32_t*>(FAKE)};
}

int main() {
  // ---- shapes
  const int bad_shapes[][5] = {{0, 1, 8, 2, 128}, {2, 0, 8, 2, 128}, {2, 1, 0, 2, 128}, {2, 1, 8, 0, 128},
                               {2, 1, 6, 4, 128}, {2, 1, 8, 2, 96},  {2, 2, 64, 1, 128}, {65536, 1, 8, 2, 128}};
  for (auto& s : bad_shapes) {
    cs_decode_shape sh = shape(s[0], s[1], s[2], s[3], s[4]);
    cs_kv_desc k = kv();
    EXPECT(topk_index(&sh, FAKE, &k, 0.088f, nullptr, 10, (int32_t*)FAKE, FAKE, 1ull << 40, nullptr) != CS_OK);
    EXPECT(sparse_decode_attn(&sh, FAKE, &k, (int32_t*)FAKE, 10, 0.088f, 0, (float*)FAKE, (float*)FAKE, FAKE,
                              1ull << 40, nullptr) != CS_OK);
    EXPECT(dense_decode_attn(&sh, FAKE, &k, 0.088f, 0, (float*)FAKE, (float*)FAKE, FAKE, 1ull << 40, nullptr) != CS_OK);
    EXPECT(sparse_decode_attn_noalloc(&sh, FAKE, &k, (int32_t*)FAKE, 10, 0.088f, 0, (float*)FAKE, (float*)FAKE,
                                      nullptr) != CS_OK);
    EXPECT(topk_index_workspace_size(&sh, &k, 10) == 0);
  }
  EXPECT(topk_index(nullptr, FAKE, nullptr, 0.088f, nullptr, 10, (int32_t*)FAKE, FAKE, 1, nullptr) == CS_ERR_INVALID_ARG);

  // ---- KV descriptors
  {
    cs_decode_shape sh = shape();
    cs_kv_desc bad[] = {kv(CS_KV_CONTIGUOUS, 1000, 0, 0, 0, nullptr, nullptr),
                        kv(CS_KV_CONTIGUOUS, 0),
                        kv(7),
                        kv(CS_KV_PAGED, 1000, 16, 100, 10, nullptr),
                        kv(CS_KV_PAGED, 1000, 8, 200, 10, FAKE),
                        kv(CS_KV_PAGED, 1000, 24, 100, 10, FAKE),
                        kv(CS_KV_PAGED, 1000, 16, 10, 10, FAKE),
                        kv(CS_KV_PAGED, 1000, 16, 100, 0, FAKE),
                        kv(CS_KV_CONTIGUOUS, 1000, 0, 0, 0, nullptr, reinterpret_cast<void*>(0x10002))};
    for (auto& k : bad) {
      EXPECT(topk_index(&sh, FAKE, &k, 0.088f, nullptr, 10, (int32_t*)FAKE, FAKE, 1ull << 40, nullptr) != CS_OK);
      EXPECT(dense_decode_attn_workspace_size(&sh, &k, 0) == 0);
      EXPECT(sparse_decode_step_workspace_size(&sh, &k, 10) == 0);
    }
  }

  // ---- workspace sizes over a sweep of shapes, including the largest accepted ones; every
  // valid call with a sufficient workspace reaches the (stubbed) launch and returns CS_OK
  const int Bs[] = {1, 3, 64, 4096};
  const int lens[] = {1, 15, 1024, 1025, 32768, 131072, 262144};
  const int dims[] = {64, 128};
  std::vector<char> dummy(16);
  for (int B : Bs)
    for (int L : lens)
      for (int d : dims)
        for (int T : {1, 4})
          for (int layout : {CS_KV_CONTIGUOUS, CS_KV_PAGED}) {
            if (T > L) continue;
            cs_decode_shape sh = shape(B, T, 32, 8, d);
            const int pages = (L + 15) / 16;
            cs_kv_desc k = layout == CS_KV_PAGED ? kv(CS_KV_PAGED, L, 16, pages, pages * B, FAKE) : kv(CS_KV_CONTIGUOUS, L);
            if (topk_index_workspace_size(&sh, &k, 1) == 0) {
              // shapes beyond the supported range (here: more than 2^31 / 4096 query rows) are
              // refused by every entry point before any sizing
              EXPECT(topk_index(&sh, FAKE, &k, 0.088f, nullptr, 1, (int32_t*)FAKE, FAKE, 1ull << 40, nullptr) ==
                     CS_ERR_UNSUPPORTED);
              EXPECT(sparse_decode_attn(&sh, FAKE, &k, (int32_t*)FAKE, 1, 0.088f, 0, (float*)FAKE, (float*)FAKE, FAKE,
                                        1ull << 40, nullptr) == CS_ERR_UNSUPPORTED);
              EXPECT(dense_decode_attn(&sh, FAKE, &k, 0.088f, 0, (float*)FAKE, (float*)FAKE, FAKE, 1ull << 40,
                                       nullptr) == CS_ERR_UNSUPPORTED);
              continue;
            }
            for (int kmax : {1, L / 50 > 0 ? L / 50 : 1, L / 10 > 0 ? L / 10 : 1, L}) {
              const size_t wt = topk_index_workspace_size(&sh, &k, kmax);
              const size_t ws = sparse_decode_attn_workspace_size(&sh, kmax, 0);
              const size_t wd = dense_decode_attn_workspace_size(&sh, &k, 0);
              const size_t wst = sparse_decode_step_workspace_size(&sh, &k, kmax);
              const size_t wsk = topk_index_sketch_workspace_size(&sh, &k, kmax, 2);
              EXPECT(wt > 0 && wt % 256 == 0);
              EXPECT(wst >= wt);
              EXPECT(topk_index(&sh, FAKE, &k, 0.088f, nullptr, kmax, (int32_t*)FAKE, FAKE, wt, nullptr) == CS_OK);
              EXPECT(topk_index(&sh, FAKE, &k, 0.088f, nullptr, kmax, (int32_t*)FAKE, FAKE, wt - 1, nullptr) ==
                     CS_ERR_WORKSPACE_TOO_SMALL);
              EXPECT(sparse_decode_attn(&sh, FAKE, &k, (int32_t*)FAKE, kmax, 0.088f, 0, (float*)FAKE, (float*)FAKE,
                                        ws ? FAKE : nullptr, ws, nullptr) == CS_OK);
              EXPECT(dense_decode_attn(&sh, FAKE, &k, 0.088f, 0, (float*)FAKE, (float*)FAKE, wd ? FAKE : nullptr, wd,
                                       nullptr) == CS_OK);
              EXPECT(sparse_decode_step(&sh, FAKE, &k, 0.088f, nullptr, kmax, nullptr, (float*)FAKE, (float*)FAKE, FAKE,
                                        wst, nullptr) == CS_OK);
              if (wsk > 0) {
                cs_key_sketch sk{FAKE, (float*)FAKE};
                const cs_status st = topk_index_sketch(&sh, FAKE, &k, &sk, 0.088f, nullptr, kmax, 2, (int32_t*)FAKE,
                                                       FAKE, wsk, nullptr);
                EXPECT(st == CS_OK || st == CS_ERR_UNSUPPORTED);
              }
              for (int S : {1, 2, 7, 1024, 5000}) {
                const size_t w2 = sparse_decode_attn_workspace_size(&sh, kmax, S);
                EXPECT(w2 < (size_t)1 << 50);
                EXPECT(sparse_decode_attn(&sh, FAKE, &k, (int32_t*)FAKE, kmax, 0.088f, S, (float*)FAKE, (float*)FAKE,
                                          w2 ? FAKE : nullptr, w2, nullptr) == CS_OK);
                const size_t w3 = dense_decode_attn_workspace_size(&sh, &k, S);
                EXPECT(dense_decode_attn(&sh, FAKE, &k, 0.088f, S, (float*)FAKE, (float*)FAKE, w3 ? FAKE : nullptr, w3,
                                         nullptr) == CS_OK);
                // the allocation-free variant: refused beyond its fixed scratch, else it needs the
                // device (hipGetSymbolAddress), which a CPU-only run does not have
                const cs_status na = sparse_decode_attn_noalloc(&sh, FAKE, &k, (int32_t*)FAKE, kmax, 0.088f, S,
                                                                (float*)FAKE, (float*)FAKE, nullptr);
                EXPECT(w2 > CS_NOALLOC_SCRATCH_BYTES ? na == CS_ERR_SCRATCH_LIMIT : (na == CS_OK || na == CS_ERR_HIP));
              }
            }
          }
  // non-finite scales, bad k
  {
    cs_decode_shape sh = shape();
    cs_kv_desc k = kv();
    EXPECT(topk_index(&sh, FAKE, &k, NAN, nullptr, 10, (int32_t*)FAKE, FAKE, 1ull << 40, nullptr) == CS_ERR_INVALID_ARG);
    EXPECT(topk_index(&sh, FAKE, &k, INFINITY, nullptr, 10, (int32_t*)FAKE, FAKE, 1ull << 40, nullptr) == CS_ERR_INVALID_ARG);
    EXPECT(topk_index(&sh, FAKE, &k, 0.088f, nullptr, 0, (int32_t*)FAKE, FAKE, 1ull << 40, nullptr) == CS_ERR_INVALID_ARG);
    EXPECT(topk_index(&sh, FAKE, &k, 0.088f, nullptr, 1001, (int32_t*)FAKE, FAKE, 1ull << 40, nullptr) == CS_ERR_INVALID_ARG);
    cs_kv_desc big = kv(CS_KV_CONTIGUOUS, 262145);
    EXPECT(topk_index(&sh, FAKE, &big, 0.088f, nullptr, 10, (int32_t*)FAKE, FAKE, 1ull << 40, nullptr) == CS_ERR_UNSUPPORTED);
    EXPECT(sparse_decode_attn(&sh, FAKE, &k, (int32_t*)FAKE, 10, 0.088f, -1, (float*)FAKE, (float*)FAKE, FAKE, 1ull << 40,
                              nullptr) == CS_ERR_INVALID_ARG);
    EXPECT(key_sketch_build(&sh, &k, -1, nullptr, nullptr) == CS_ERR_INVALID_ARG);
  }
  for (int s = -1; s < 8; ++s) EXPECT(cs_status_str((cs_status)s) != nullptr);
  EXPECT(cs_version() >= 100);
  std::printf("abi cases: %d passed, %d failed\n", passed, failures);
  return failures ? 1 : 0;
}
