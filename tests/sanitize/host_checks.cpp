// Host-side checks of the C-ABI, built with AddressSanitizer and
// UndefinedBehaviorSanitizer (host code only, no GPU): the argument checks,
// workspace queries, status strings and per-thread error messages, and every
// entry point with arguments that must be rejected before anything is
// launched.  The kernel launchers are stubs that count calls: a call that
// reaches one here is a failure.  Exit status 0 when every check holds.
#include <climits>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <thread>
#include <vector>

#include "dg.h"

extern "C" int dg_stub_launches(void);

static int failures = 0;
#define EXPECT(c)                                                              \
  do {                                                                         \
    if (!(c)) {                                                                \
      std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c);     \
      ++failures;                                                              \
    }                                                                          \
  } while (0)

static dg_dims make_dims(int d, int hq, int hkv, int hd, int V, int C, int W, int dt) {
  dg_dims x;
  x.d_model = d;
  x.n_q_heads = hq;
  x.n_kv_heads = hkv;
  x.head_dim = hd;
  x.vocab = V;
  x.canvas = C;
  x.window = W;
  x.mask_id = V - 1;
  x.dtype = dt;
  return x;
}

// aligned fake device addresses: never dereferenced on the host
static void *fake(uintptr_t a) { return reinterpret_cast<void *>(a); }

static void workspace_queries(const dg_dims &d) {
  const int32_t batches[] = {0, 1, 3, 32, 512, 4096};
  const int32_t lens[] = {0, 1, 255, 256, 257, 2048, 8192, 110707, 1 << 20};
  for (int32_t B : batches) {
    size_t prev[7] = {0, 0, 0, 0, 0, 0, 0};
    bool capped[7] = {false, false, false, false, false, false, false};
    for (int32_t m : lens) {
      const size_t w[7] = {dg_denoise_step_workspace(&d, B, m), dg_denoise_loop_workspace(&d, B, m),
                           dg_slot_read_workspace(&d, B, 4, m, 4),
                           dg_slot_read_full_canvas_workspace(&d, B, 4, m, 4),
                           dg_slot_read_staged_workspace(&d, B, 4, m, 4),
                           dg_prefill_encode_workspace(&d, B, m),
                           dg_slot_read_workspace(&d, B, 26, m, 16)};
      // non-decreasing in max_prompt while the sizes fit; once a query says 0
      // (out of range) after a size, every longer prompt is out of range too
      for (int i = 0; i < 7; ++i) {
        if (w[i] == 0 && prev[i] > 0) capped[i] = true;
        if (capped[i]) {
          EXPECT(w[i] == 0);
        } else if (w[i] < prev[i]) {
          std::fprintf(stderr, "query %d: batch %d, max_prompt %d: %zu < %zu\n", i, B, m, w[i], prev[i]);
          EXPECT(false);
        }
        prev[i] = w[i];
      }
    }
  }
  // bad arguments give 0, extreme ones a size or 0, never undefined behaviour
  EXPECT(dg_denoise_step_workspace(nullptr, 1, 1) == 0);
  EXPECT(dg_denoise_step_workspace(&d, -1, 1) == 0);
  EXPECT(dg_slot_read_workspace(&d, 1, -1, 1, 4) == 0);
  const int32_t big[] = {INT_MAX / 256, INT_MAX};
  for (int32_t b : big) {
    (void)dg_denoise_step_workspace(&d, b, INT_MAX);
    (void)dg_denoise_loop_workspace(&d, b, INT_MAX);
    (void)dg_slot_read_workspace(&d, b, 64, INT_MAX, 16);
    (void)dg_slot_read_staged_workspace(&d, b, 64, INT_MAX, 16);
    (void)dg_slot_read_full_canvas_workspace(&d, b, 64, INT_MAX, 16);
    (void)dg_prefill_encode_workspace(&d, b, INT_MAX);
  }
}

static void validators(const dg_dims &d) {
  dg_weights w;
  std::memset(&w, 0, sizeof w);
  w.embed = w.embed_t = w.wq = w.wk = w.wv = w.wo = fake(0x10000);
  dg_prompt_kv kv = {fake(0x20000), fake(0x30000), static_cast<const int32_t *>(fake(0x40000)), 128, 128};
  EXPECT(dg_denoise_step_validate(&d, 1, 128, &w, &kv) == DG_OK);
  EXPECT(dg_denoise_step_validate(nullptr, 1, 128, &w, &kv) == DG_ERR_INVALID_ARG);
  EXPECT(dg_denoise_step_validate(&d, 1, 64, &w, &kv) == DG_ERR_INVALID_ARG);   // max_len > planned
  dg_weights bad = w;
  bad.wq = fake(0x10002);
  EXPECT(dg_denoise_step_validate(&d, 1, 128, &bad, &kv) == DG_ERR_INVALID_ARG);
  bad = w;
  bad.lm_fp8_act = 1;
  EXPECT(dg_denoise_step_validate(&d, 1, 128, &bad, &kv) == DG_ERR_INVALID_ARG);
  EXPECT(std::strlen(dg_last_error()) > 0);
  dg_dims e = d;
  e.head_dim = 96;
  EXPECT(dg_denoise_step_validate(&e, 1, 128, &w, &kv) == DG_ERR_UNSUPPORTED);
  e = d;
  e.canvas = 0;
  EXPECT(dg_denoise_step_validate(&e, 1, 128, &w, &kv) == DG_ERR_INVALID_ARG);
  e = d;
  e.mask_id = d.vocab;
  EXPECT(dg_denoise_step_validate(&e, 1, 128, &w, &kv) == DG_ERR_INVALID_ARG);
  e = d;
  e.window = INT_MAX;   // a full-block window is valid
  EXPECT(dg_denoise_step_validate(&e, 1, 128, &w, &kv) == DG_OK);
  EXPECT(dg_slot_read_validate(&d, 2, 4, 4, 0.1f) == DG_OK);
  EXPECT(dg_slot_read_validate(&d, 2, 4, 0, 0.1f) == DG_ERR_INVALID_ARG);
  EXPECT(dg_slot_read_validate(&d, 2, 4, 4, -1.f) == DG_ERR_INVALID_ARG);
  EXPECT(dg_commit_validate(2, 256) == DG_OK);
  EXPECT(dg_commit_validate(2, 0) == DG_ERR_INVALID_ARG);
  EXPECT(dg_check_label_count(26) == DG_OK);
  EXPECT(dg_check_label_count(27) == DG_ERR_TOO_MANY_LABELS);
  EXPECT(dg_check_label_count(0) == DG_ERR_INVALID_ARG);
  EXPECT(dg_check_label_count(INT_MIN) == DG_ERR_INVALID_ARG);
  // (values outside the enumerators are checked from Python, where they are plain ints)
  const dg_status all[] = {DG_OK, DG_ERR_INVALID_ARG, DG_ERR_TOO_MANY_LABELS, DG_ERR_UNSUPPORTED,
                           DG_ERR_WORKSPACE, DG_ERR_HIP};
  for (dg_status s : all) EXPECT(std::strcmp(dg_status_string(s), "unknown status") != 0);
  EXPECT(std::strstr(dg_version(), "gfx950") != nullptr);
}

// every entry point with an argument that must be rejected on the host
static void rejected_calls(const dg_dims &d) {
  dg_weights w;
  std::memset(&w, 0, sizeof w);
  w.embed = w.embed_t = w.wq = w.wk = w.wv = w.wo = fake(0x10000);
  dg_prompt_kv kv = {fake(0x20000), fake(0x30000), static_cast<const int32_t *>(fake(0x40000)), 128, 128};
  int32_t *ip = static_cast<int32_t *>(fake(0x50000));
  float *fp = static_cast<float *>(fake(0x60000));
  void *ws = fake(0x70000);
  const size_t small = 16;
  EXPECT(dg_denoise_step(&d, &w, &kv, 2, ip, nullptr, 1.f, nullptr, fp, fp, ip, nullptr, nullptr,
                         nullptr, ws, small, nullptr) == DG_ERR_WORKSPACE);
  EXPECT(dg_denoise_step(&d, &w, &kv, 2, nullptr, nullptr, 1.f, nullptr, fp, fp, ip, nullptr,
                         nullptr, nullptr, ws, 1 << 30, nullptr) == DG_ERR_INVALID_ARG);
  EXPECT(dg_denoise_loop(&d, &w, &kv, 2, ip, nullptr, 1.f, nullptr, 2.f, 4, 1, ip, ip, nullptr,
                         nullptr, ws, small, nullptr) == DG_ERR_WORKSPACE);
  EXPECT(dg_commit(2, 0, 0, ip, fp, fp, ip, 1.f, nullptr, ip, ip, nullptr) == DG_ERR_INVALID_ARG);
  EXPECT(dg_prefill_kv(&d, &w, -1, ip, ws, ws, nullptr, nullptr) == DG_ERR_INVALID_ARG);
  EXPECT(dg_prefill_encode(&d, &w, 2, ip, 700, 900, ip, ws, ws, ws, nullptr, nullptr, ws, small,
                           nullptr) == DG_ERR_WORKSPACE);
  EXPECT(dg_slot_read(&d, &w, &kv, 2, ip, 4, ip, ip, ip, ip, 1.f, nullptr, 0.1f, 4, fp, fp, fp, fp,
                      ip, ip, ip, ws, small, nullptr) == DG_ERR_WORKSPACE);
  EXPECT(dg_slot_read_full_canvas(&d, &w, &kv, 2, ip, 4, ip, ip, ip, ip, 1.f, nullptr, 0.1f, 17, fp,
                                  fp, fp, fp, ip, ip, ip, ws, 1 << 30, nullptr) == DG_ERR_INVALID_ARG);
  const int32_t stage[4] = {0, 0, 1, 2};   // stage 2 does not exist
  const int32_t ask[4] = {-1, -1, 0, -1}, lab[4] = {0, 0, 0, 0};
  EXPECT(dg_slot_read_staged(&d, &w, &kv, 2, ip, 4, ip, ip, ip, ip, stage, ask, lab, 1.f, nullptr,
                             0.1f, 4, fp, fp, fp, fp, ip, ip, ip, ws, 1 << 30, nullptr) ==
         DG_ERR_INVALID_ARG);
  EXPECT(dg_prepare_lm_fp8(nullptr, ws, ws, ip, nullptr) == DG_ERR_INVALID_ARG);
}

int main() {
  const dg_dims tiny = make_dims(256, 4, 4, 64, 2048, 256, 16, DG_F32);
  const dg_dims tiny_bf = make_dims(256, 4, 4, 64, 2048, 256, 16, DG_BF16);
  const dg_dims head = make_dims(2816, 8, 2, 512, 262144, 256, 128, DG_BF16);
  for (const dg_dims &d : {tiny, tiny_bf, head}) {
    workspace_queries(d);
    validators(d);
    rejected_calls(d);
  }
  // the detail message is per thread: each thread sees its own last error
  std::vector<std::thread> th;
  std::vector<int> ok(8, 0);
  for (int t = 0; t < 8; ++t)
    th.emplace_back([t, &ok, &tiny] {
      int good = 1;
      for (int i = 0; i < 200; ++i) {
        const int32_t n = 27 + t;   // distinct per thread
        if (dg_check_label_count(n) != DG_ERR_TOO_MANY_LABELS) good = 0;
        char want[32];
        std::snprintf(want, sizeof want, "%d", n);
        if (!std::strstr(dg_last_error(), want)) good = 0;
        (void)dg_denoise_step_workspace(&tiny, 1 + t, 100 * i);
      }
      ok[t] = good;
    });
  for (auto &x : th) x.join();
  for (int t = 0; t < 8; ++t) EXPECT(ok[t] == 1);
  EXPECT(dg_stub_launches() == 0);
  if (failures) std::fprintf(stderr, "%d checks failed\n", failures);
  else std::printf("host checks passed\n");
  return failures ? 1 : 0;
}
