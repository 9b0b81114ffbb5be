// Host-side checks of the C ABI, built with AddressSanitizer and
// UndefinedBehaviorSanitizer on the host code only (the kernels are not
// compiled in; nothing here launches one). Exercises argument validation,
// planning over a grid of shapes up to the 32-bit limits, the error paths of
// the prepare / launch / append entry points, and the thread-local error
// message under concurrent use. Prints "ALL OK" and exits 0 when every
// expectation holds; a sanitizer report aborts the run.
#include "gqa_decode.h"

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <limits>
#include <thread>
#include <vector>

namespace {

int g_failures = 0;

void expect(bool ok, const char* what, int line) {
  if (!ok) {
    ++g_failures;
    std::printf("FAIL line %d: %s (last error: '%s')\n", line, what, gqa_last_error());
  }
}
#define EXPECT(c) expect((c), #c, __LINE__)

// Fake, aligned, well-separated device addresses: validation compares them only.
constexpr uintptr_t kGiB = uintptr_t(1) << 30;
const void* const Q = reinterpret_cast<const void*>(1 * kGiB);
const void* const KV = reinterpret_cast<const void*>(64 * kGiB);
const void* const SCALES = reinterpret_cast<const void*>(128 * kGiB);
const int32_t* const LENS = reinterpret_cast<const int32_t*>(192 * kGiB);
void* const OUT = reinterpret_cast<void*>(200 * kGiB);
const int32_t* const TABLE = reinterpret_cast<const int32_t*>(208 * kGiB);

gqa_desc_t desc(int32_t batch = 2, int32_t capacity = 1024, int32_t kv = GQA_BF16,
                int32_t q = GQA_BF16, int32_t hq = 32) {
  gqa_desc_t d;
  std::memset(&d, 0, sizeof d);
  d.batch = batch;
  d.capacity = capacity;
  d.num_q_heads = hq;
  d.num_kv_heads = 8;
  d.head_dim = 128;
  d.q_dtype = q;
  d.kv_dtype = kv;
  const bool quant = kv == GQA_FP8_E4M3 || kv == GQA_INT8_ROWSCALE;
  d.k_scale = quant ? 0.5f : 1.f;
  d.v_scale = quant ? 0.25f : 1.f;
  return d;
}

gqa_paged_desc_t pdesc(int32_t batch = 2, int32_t T = 1, int32_t P = 16, int32_t num_pages = 64,
                       int32_t max_pages = 32, int32_t kv = GQA_BF16, int32_t hq = 32) {
  gqa_paged_desc_t d;
  std::memset(&d, 0, sizeof d);
  d.batch = batch;
  d.q_tokens = T;
  d.num_q_heads = hq;
  d.num_kv_heads = 8;
  d.head_dim = 128;
  d.q_dtype = GQA_BF16;
  d.kv_dtype = kv;
  const bool quant = kv == GQA_FP8_E4M3 || kv == GQA_INT8_ROWSCALE;
  d.k_scale = quant ? 0.5f : 1.f;
  d.v_scale = quant ? 0.25f : 1.f;
  d.page_size = P;
  d.num_pages = num_pages;
  d.max_pages = max_pages;
  return d;
}

gqa_status_t v(const gqa_desc_t& d, const void* q = Q, const void* kv = KV,
               const int32_t* lens = LENS, float qs = 1.f, const void* out = OUT, int32_t ns = 0) {
  return gqa_validate_args(&d, q, kv, lens, qs, out, ns);
}

void contiguous_validation() {
  EXPECT(v(desc()) == GQA_OK);
  EXPECT(std::strcmp(gqa_last_error(), "") == 0);
  EXPECT(v(desc(), nullptr) == GQA_ERR_INVALID_ARG);
  EXPECT(std::strlen(gqa_last_error()) > 0);
  EXPECT(v(desc(), Q, nullptr) == GQA_ERR_INVALID_ARG);
  EXPECT(v(desc(), Q, KV, nullptr) == GQA_ERR_INVALID_ARG);
  EXPECT(v(desc(), Q, KV, LENS, 1.f, nullptr) == GQA_ERR_INVALID_ARG);
  EXPECT(gqa_validate_args(nullptr, Q, KV, LENS, 1.f, OUT, 0) == GQA_ERR_INVALID_ARG);
  const float bad_scales[] = {0.f, -1.f, std::numeric_limits<float>::infinity(),
                              std::numeric_limits<float>::quiet_NaN()};
  for (float s : bad_scales) {
    EXPECT(v(desc(), Q, KV, LENS, s) == GQA_ERR_INVALID_ARG);
    gqa_desc_t d = desc(2, 1024, GQA_FP8_E4M3);
    d.k_scale = s;
    EXPECT(v(d) == GQA_ERR_INVALID_ARG);
    d = desc(2, 1024, GQA_FP8_E4M3);
    d.v_scale = s;
    EXPECT(v(d) == GQA_ERR_INVALID_ARG);
  }
  {
    gqa_desc_t d = desc();
    d.k_scale = 2.f;   // a scale other than 1 needs a quantised cache
    EXPECT(v(d) == GQA_ERR_INVALID_ARG);
  }
  const int32_t geometry[][3] = {{31, 8, 128}, {32, 4, 128}, {32, 8, 64}, {0, 8, 128}, {-32, 8, 128}};
  for (const auto& g : geometry) {
    gqa_desc_t d = desc();
    d.num_q_heads = g[0];
    d.num_kv_heads = g[1];
    d.head_dim = g[2];
    EXPECT(v(d) == GQA_ERR_INVALID_ARG);
  }
  for (int32_t C : {0, -1, GQA_MAX_CAPACITY + 1, std::numeric_limits<int32_t>::max()})
    EXPECT(v(desc(2, C)) == GQA_ERR_INVALID_ARG);
  EXPECT(v(desc(-1)) == GQA_ERR_INVALID_ARG);
  for (int32_t dt : {-1, 4, 99}) {
    EXPECT(v(desc(2, 1024, dt)) == GQA_ERR_INVALID_ARG);
    EXPECT(v(desc(2, 1024, GQA_BF16, dt)) == GQA_ERR_INVALID_ARG);
  }
  EXPECT(v(desc(2, 1024, GQA_FP8_E4M3, GQA_FP8_E4M3)) == GQA_ERR_INVALID_ARG);  // fp8 queries
  EXPECT(v(desc(2, 1024, GQA_INT8_ROWSCALE, GQA_BF16, 16)) == GQA_ERR_INVALID_ARG);  // needs _int8
  // alignment and aliasing
  EXPECT(v(desc(), reinterpret_cast<const char*>(Q) + 4) == GQA_ERR_INVALID_ARG);
  EXPECT(v(desc(), Q, KV, LENS, 1.f, reinterpret_cast<char*>(OUT) + 8) == GQA_ERR_INVALID_ARG);
  EXPECT(v(desc(), Q, KV, LENS, 1.f, const_cast<void*>(Q)) == GQA_ERR_ALIAS);
  EXPECT(v(desc(), Q, KV, LENS, 1.f, const_cast<void*>(KV)) == GQA_ERR_ALIAS);
  EXPECT(v(desc(), Q, Q) == GQA_OK);   // inputs may overlap each other
  // split counts
  EXPECT(v(desc(), Q, KV, LENS, 1.f, OUT, -1) == GQA_ERR_INVALID_ARG);
  EXPECT(v(desc(), Q, KV, LENS, 1.f, OUT, 10) == GQA_OK);
  EXPECT(v(desc(), Q, KV, LENS, 1.f, OUT, 1025) == GQA_ERR_INVALID_ARG);
  EXPECT(v(desc(), Q, KV, LENS, 1.f, OUT, std::numeric_limits<int32_t>::max()) ==
         GQA_ERR_INVALID_ARG);
  {
    gqa_desc_t d = desc();
    d.flags = 2;
    EXPECT(v(d) == GQA_ERR_INVALID_ARG);
    d.flags = GQA_FLAG_FUSED_COMBINE;
    EXPECT(v(d) == GQA_OK);
  }
  // batch 0: a valid no-op, whatever the pointers
  EXPECT(v(desc(0), nullptr, nullptr, nullptr, 1.f, nullptr) == GQA_OK);
}

void int8_validation() {
  const gqa_desc_t d = desc(2, 1024, GQA_INT8_ROWSCALE, GQA_BF16, 16);
  EXPECT(gqa_validate_args_int8(&d, Q, KV, SCALES, LENS, 1.f, OUT, 0) == GQA_OK);
  EXPECT(gqa_validate_args_int8(&d, Q, KV, nullptr, LENS, 1.f, OUT, 0) == GQA_ERR_INVALID_ARG);
  EXPECT(gqa_validate_args_int8(&d, Q, KV, SCALES, LENS, 1.f, const_cast<void*>(SCALES), 0) ==
         GQA_ERR_ALIAS);
  const gqa_desc_t bf = desc();
  EXPECT(gqa_validate_args_int8(&bf, Q, KV, SCALES, LENS, 1.f, OUT, 0) == GQA_ERR_INVALID_ARG);
}

// Route 0: capacity <= 64; 1: chunks of chunk_tokens (num_splits of them, a
// second kernel merges when more than one); 2: the balanced split.
void check_plan(const gqa_plan_t& p, int32_t batch, int32_t C, int32_t ns) {
  EXPECT(p.route >= 0 && p.route <= 2);
  EXPECT((p.route == 0) == (C <= GQA_SHORT_CAPACITY_MAX));
  if (batch == 0) {
    EXPECT(p.workspace_bytes == 0);
    return;
  }
  EXPECT(p.num_workgroups > 0);
  if (ns > 0) EXPECT(p.route != 2 && p.num_splits == ns);
  if (p.route == 2) {
    EXPECT(p.num_splits == 0 && p.chunk_tokens == 64 && p.workspace_bytes > 0);
  } else {
    EXPECT(p.chunk_tokens > 0 && p.chunk_tokens % GQA_CHUNK_GRANULE == 0);
    EXPECT((int64_t)p.num_splits * p.chunk_tokens >= C);
    EXPECT((int64_t)(p.num_splits - 1) * p.chunk_tokens < C);
    EXPECT((p.num_splits > 1) == (p.workspace_bytes > 0));
    EXPECT((int64_t)p.num_workgroups == (int64_t)batch * 8 * p.num_splits);
    if (p.fused_merge) EXPECT(p.num_splits > 1);
  }
}

void planning() {
  const int32_t batches[] = {0, 1, 2, 8, 31, 4096, 4097, 65535, 1 << 20};
  const int32_t caps[] = {1, 63, 64, 65, 1000, 1024, 8192, 65536, 131072, GQA_MAX_CAPACITY};
  const int32_t splits[] = {0, 1, 2, 7, 64};
  const int32_t kvs[] = {GQA_F16, GQA_BF16, GQA_FP8_E4M3, GQA_INT8_ROWSCALE};
  int planned = 0, refused = 0;
  for (int32_t kv : kvs)
    for (int32_t B : batches)
      for (int32_t C : caps)
        for (int32_t ns : splits)
          for (int32_t flags : {0, (int32_t)GQA_FLAG_FUSED_COMBINE}) {
            const int32_t hq = kv == GQA_INT8_ROWSCALE ? 16 : 32;
            gqa_desc_t d = desc(B, C, kv, kv == GQA_F16 ? GQA_F16 : GQA_BF16, hq);
            d.flags = flags;
            gqa_plan_t p;
            std::memset(&p, 0xff, sizeof p);
            const gqa_status_t st = gqa_plan_decode(&d, ns, &p);
            if (st == GQA_OK) {
              ++planned;
              check_plan(p, B, C, ns);
            } else {
              ++refused;   // too large for one launch, or a split count that cannot be honoured
              EXPECT(st == GQA_ERR_INVALID_ARG);
              EXPECT(std::strlen(gqa_last_error()) > 0);
            }
          }
  EXPECT(planned > 1000 && refused > 0);
  gqa_plan_t p;
  EXPECT(gqa_plan_decode(nullptr, 0, &p) == GQA_ERR_INVALID_ARG);
  const gqa_desc_t d = desc();
  EXPECT(gqa_plan_decode(&d, 0, nullptr) == GQA_ERR_INVALID_ARG);
  EXPECT(gqa_plan_decode(&d, -3, &p) == GQA_ERR_INVALID_ARG);
}

void paged() {
  const gqa_paged_desc_t ok = pdesc();
  EXPECT(gqa_validate_args_paged(&ok, Q, KV, nullptr, TABLE, LENS, 1.f, OUT, 0) == GQA_OK);
  EXPECT(gqa_validate_args_paged(&ok, Q, KV, nullptr, nullptr, LENS, 1.f, OUT, 0) ==
         GQA_ERR_INVALID_ARG);
  EXPECT(gqa_validate_args_paged(&ok, Q, KV, nullptr, TABLE, LENS, 1.f, const_cast<int32_t*>(TABLE),
                                 0) == GQA_ERR_ALIAS);
  for (int32_t P : {0, 8, 24, 100, GQA_MAX_PAGE_SIZE * 2, -16}) {
    const gqa_paged_desc_t d = pdesc(2, 1, P);
    EXPECT(gqa_validate_args_paged(&d, Q, KV, nullptr, TABLE, LENS, 1.f, OUT, 0) ==
           GQA_ERR_INVALID_ARG);
  }
  for (int32_t n : {0, -1}) {
    gqa_paged_desc_t d = pdesc();
    d.num_pages = n;
    EXPECT(gqa_validate_args_paged(&d, Q, KV, nullptr, TABLE, LENS, 1.f, OUT, 0) ==
           GQA_ERR_INVALID_ARG);
    d = pdesc();
    d.max_pages = n;
    EXPECT(gqa_validate_args_paged(&d, Q, KV, nullptr, TABLE, LENS, 1.f, OUT, 0) ==
           GQA_ERR_INVALID_ARG);
  }
  {
    gqa_paged_desc_t d = pdesc(2, 1, 1 << 16, 64, 1 << 12);   // logical capacity past the maximum
    EXPECT(gqa_validate_args_paged(&d, Q, KV, nullptr, TABLE, LENS, 1.f, OUT, 0) ==
           GQA_ERR_INVALID_ARG);
    d = pdesc(2, 5);   // 5 tokens x 4 heads = 20 rows > 16
    EXPECT(gqa_validate_args_paged(&d, Q, KV, nullptr, TABLE, LENS, 1.f, OUT, 0) ==
           GQA_ERR_INVALID_ARG);
    d = pdesc(2, 8, 16, 64, 32, GQA_INT8_ROWSCALE, 16);   // 8 tokens x 2 heads = 16 rows
    EXPECT(gqa_validate_args_paged(&d, Q, KV, SCALES, TABLE, LENS, 1.f, OUT, 0) == GQA_OK);
    EXPECT(gqa_validate_args_paged(&d, Q, KV, nullptr, TABLE, LENS, 1.f, OUT, 0) ==
           GQA_ERR_INVALID_ARG);
    d = pdesc();
    d.flags = GQA_FLAG_FUSED_COMBINE;
    EXPECT(gqa_validate_args_paged(&d, Q, KV, nullptr, TABLE, LENS, 1.f, OUT, 0) ==
           GQA_ERR_INVALID_ARG);
    d.flags = GQA_PAGED_SCALES_BY_POSITION;   // a bf16 pool has no scales to index
    EXPECT(gqa_validate_args_paged(&d, Q, KV, nullptr, TABLE, LENS, 1.f, OUT, 0) ==
           GQA_ERR_INVALID_ARG);
    d = pdesc(4096, 2, 16, 1 << 20, 8192, GQA_INT8_ROWSCALE, 16);
    d.flags = GQA_PAGED_SCALES_BY_POSITION;   // scales [4096, 2, 8, 131072]: 16 GiB
    EXPECT(gqa_validate_args_paged(&d, Q, KV, SCALES, TABLE, LENS, 1.f, OUT, 0) == GQA_OK);
    gqa_plan_t p;
    EXPECT(gqa_plan_decode_paged(&d, 0, &p) == GQA_OK && p.route == 2);
  }
  for (int32_t P : {16, 64, 4096})
    for (int32_t B : {1, 3, 64, 4096})
      for (int32_t T : {1, 2, 4})
        for (int32_t ns : {0, 1, 3}) {
          const int32_t max_pages = std::max(1, 131072 / P);
          const gqa_paged_desc_t d = pdesc(B, T, P, 1 << 20, max_pages);
          gqa_plan_t p;
          if (gqa_plan_decode_paged(&d, ns, &p) == GQA_OK) check_plan(p, B, max_pages * P, ns);
        }
}

void append_and_device_paths(bool have_device) {
  const gqa_desc_t d = desc();
  EXPECT(gqa_kv_append(&d, nullptr, Q, LENS, OUT, nullptr) == GQA_ERR_INVALID_ARG);
  EXPECT(gqa_kv_append(&d, Q, nullptr, LENS, OUT, nullptr) == GQA_ERR_INVALID_ARG);
  EXPECT(gqa_kv_append(&d, Q, Q, nullptr, OUT, nullptr) == GQA_ERR_INVALID_ARG);
  EXPECT(gqa_kv_append(nullptr, Q, Q, LENS, OUT, nullptr) == GQA_ERR_INVALID_ARG);
  const gqa_paged_desc_t pd = pdesc(2, 3);
  EXPECT(gqa_kv_append_paged(&pd, Q, Q, LENS, nullptr, OUT, nullptr) == GQA_ERR_INVALID_ARG);
  EXPECT(gqa_kv_append_paged(&pd, reinterpret_cast<const char*>(Q) + 4, Q, LENS, TABLE, OUT,
                             nullptr) == GQA_ERR_INVALID_ARG);

  // INT8 appends: INT8 descriptors only, a scales buffer overlapping nothing.
  const gqa_desc_t d8 = desc(2, 1024, GQA_INT8_ROWSCALE, GQA_BF16, 16);
  void* const sc = const_cast<void*>(SCALES);
  EXPECT(gqa_kv_append_int8(&d8, Q, Q, LENS, OUT, nullptr, nullptr) == GQA_ERR_INVALID_ARG);
  EXPECT(gqa_kv_append_int8(&d, Q, Q, LENS, OUT, sc, nullptr) == GQA_ERR_INVALID_ARG);
  EXPECT(gqa_kv_append_int8(&d8, Q, Q, LENS, OUT, OUT, nullptr) == GQA_ERR_ALIAS);
  EXPECT(gqa_kv_append_int8(&d8, Q, Q, LENS, OUT, static_cast<char*>(sc) + 1, nullptr) ==
         GQA_ERR_INVALID_ARG);
  EXPECT(gqa_kv_append(&d8, Q, Q, LENS, OUT, nullptr) == GQA_ERR_INVALID_ARG);
  const gqa_paged_desc_t pd8 = pdesc(2, 2, 16, 64, 32, GQA_INT8_ROWSCALE, 16);
  EXPECT(gqa_kv_append_paged_int8(&pd8, Q, Q, LENS, TABLE, OUT, nullptr, nullptr) ==
         GQA_ERR_INVALID_ARG);
  EXPECT(gqa_kv_append_paged_int8(&pd, Q, Q, LENS, TABLE, OUT, sc, nullptr) == GQA_ERR_INVALID_ARG);
  EXPECT(gqa_kv_append_paged_int8(&pd8, Q, Q, LENS, TABLE, OUT, const_cast<int32_t*>(TABLE),
                                  nullptr) == GQA_ERR_ALIAS);

  gqa_prepared_t* h = nullptr;
  EXPECT(launch_gqa_decode_prepared(nullptr, nullptr) == GQA_ERR_INVALID_ARG);
  EXPECT(gqa_prepared_workspace_bytes(nullptr) == 0);
  gqa_plan_t p;
  EXPECT(gqa_prepared_plan(nullptr, &p) == GQA_ERR_INVALID_ARG);
  gqa_prepared_destroy(nullptr);
  EXPECT(prepare_gqa_decode(&d, Q, KV, LENS, 1.f, OUT, -1, &h) == GQA_ERR_INVALID_ARG && !h);
  EXPECT(prepare_gqa_decode(&d, Q, KV, LENS, 1.f, OUT, 0, nullptr) == GQA_ERR_INVALID_ARG);
  if (!have_device) {
    // Valid arguments reach the device check, which fails without a GPU:
    // no handle, no launch, a message.
    EXPECT(prepare_gqa_decode(&d, Q, KV, LENS, 1.f, OUT, 0, &h) != GQA_OK && !h);
    EXPECT(std::strlen(gqa_last_error()) > 0);
    EXPECT(gqa_decode(&d, Q, KV, LENS, 1.f, OUT, nullptr) != GQA_OK);
    EXPECT(gqa_kv_append(&d, Q, Q, LENS, OUT, nullptr) != GQA_OK);
    EXPECT(gqa_kv_append_int8(&d8, Q, Q, LENS, OUT, sc, nullptr) != GQA_OK);
    EXPECT(gqa_kv_append_paged_int8(&pd8, Q, Q, LENS, TABLE, OUT, sc, nullptr) != GQA_OK);
    EXPECT(prepare_gqa_decode_paged(&pd, Q, KV, nullptr, TABLE, LENS, 1.f, OUT, 0, &h) != GQA_OK &&
           !h);
  }
}

void threads() {
  // The last-error message is per thread: each thread sees its own outcome.
  std::atomic<int> bad{0};
  std::vector<std::thread> ts;
  for (int t = 0; t < 8; ++t)
    ts.emplace_back([t, &bad] {
      for (int i = 0; i < 2000; ++i) {
        const bool fail = ((i + t) & 1) != 0;
        const gqa_desc_t d = desc(fail ? -1 : 2);
        const gqa_status_t st = v(d);
        const bool empty = gqa_last_error()[0] == '\0';
        if ((st == GQA_OK) == fail || empty != !fail) ++bad;
        gqa_plan_t p;
        if (gqa_plan_decode(&d, 0, &p) != (fail ? GQA_ERR_INVALID_ARG : GQA_OK)) ++bad;
      }
    });
  for (auto& th : ts) th.join();
  EXPECT(bad.load() == 0);
}

}  // namespace

int main() {
  int devices = 0;
  const bool have_device = hipGetDeviceCount(&devices) == hipSuccess && devices > 0;
  contiguous_validation();
  int8_validation();
  planning();
  paged();
  append_and_device_paths(have_device);
  threads();
  if (g_failures) {
    std::printf("%d expectation(s) failed\n", g_failures);
    return 1;
  }
  std::printf("ALL OK\n");
  return 0;
}
