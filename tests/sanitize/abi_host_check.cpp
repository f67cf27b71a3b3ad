// Host-side check of the C ABI (include/aq.h) built with AddressSanitizer and
// UndefinedBehaviorSanitizer over the library's real host code (aq_api.cpp,
// aq_plan.cpp) and stand-in launchers (launch_stubs.cpp).  Every entry point
// is called with invalid arguments (each must be rejected with its status
// before any launch) and with valid ones, once with a forced launch failure
// (each must return AQ_ERR_HIP) and once with success.  Device pointers are
// aligned addresses in host memory that the stand-ins never dereference.
#include <hip/hip_runtime_api.h>

#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "../../include/aq.h"

extern hipError_t g_forced;
extern int g_launches;

static int failures = 0;
#define CHECK(cond)                                                   \
  do {                                                                \
    if (!(cond)) {                                                    \
      std::printf("FAIL %s:%d: %s\n", __FILE__, __LINE__, #cond);     \
      ++failures;                                                     \
    }                                                                 \
  } while (0)

alignas(256) static unsigned char pool[1 << 20];
static void *dev(size_t off) { return pool + off; }

// A packed projection with fake device buffers and host labels.
struct Fake {
  aq_packed p;
  std::vector<uint8_t> labels;
  std::vector<uint32_t> meta;
};

static Fake make(int N, int K, int bK, double frac4, unsigned seed) {
  Fake f;
  const int R = N / 64, C = K / bK;
  std::vector<uint8_t> z((size_t)R * C);
  srand(seed);
  for (auto &v : z) v = (rand() % 1000) < frac4 * 1000 ? 4 : 8;
  f.labels.assign(((size_t)R * C + 7) / 8, 0);
  CHECK(aq_labels_from_map(z.data(), R, C, f.labels.data()) == AQ_OK);
  aq_plan plan;
  CHECK(aq_plan_pack(N, K, 64, bK, f.labels.data(), &plan) == AQ_OK);
  f.meta.assign(plan.meta_bytes / 4 + 1, 0);
  f.p = aq_packed{N, K, 64, bK, plan.T4, plan.T8,
                  (uint8_t *)dev(0), (int32_t *)dev(4096), (int32_t *)dev(8192),
                  (uint8_t *)dev(16384), (int8_t *)dev(32768), (float *)dev(49152), (float *)dev(65536),
                  plan.meta_bytes ? f.meta.data() : nullptr};
  return f;
}

// Valid transform tables: signed permutations of 64 elements.
static aq_transform_tables make_tables() {
  aq_transform_tables t{};
  for (int s = 0; s < AQ_TRANSFORM_SEEDS; ++s)
    for (int e = 0; e < 64; ++e) {
      t.perm[s][e] = (uint8_t)((e * 5 + s) % 64);
      t.dl[s][e] = (e + s) % 3 ? 1 : -1;
      t.dr[s][e] = (e * s) % 2 ? -1 : 1;
    }
  return t;
}
static const aq_transform_tables g_tables = make_tables();

// launches: whether the failure comes from a launcher (else from the HIP
// copies that precede it, as in packing)
static void expect_launch(aq_status (*call)(void *), void *ctx, const char *name, bool launches = true) {
  g_forced = hipErrorLaunchFailure;
  const int before = g_launches;
  const aq_status st = call(ctx);
  if (st != AQ_ERR_HIP) std::printf("FAIL %s: forced launch failure gave %d\n", name, (int)st), ++failures;
  if (launches && g_launches == before) std::printf("FAIL %s: no launch\n", name), ++failures;
  g_forced = hipSuccess;
  const aq_status ok = call(ctx);
  if (ok != AQ_OK) std::printf("FAIL %s: successful launch gave %d\n", name, (int)ok), ++failures;
}

int main() {
  CHECK(aq_abi_version() == AQ_ABI_VERSION);
  for (int s = -9; s <= 0; ++s) CHECK(aq_status_string((aq_status)s) != nullptr);

  // labels and plans
  {
    uint8_t z[6] = {4, 8, 4, 8, 8, 4}, lab[1] = {0xFF};
    CHECK(aq_labels_from_map(z, 2, 3, lab) == AQ_OK && lab[0] == (1 | 4 | 32));
    z[2] = 5;
    CHECK(aq_labels_from_map(z, 2, 3, lab) == AQ_ERR_MAP);
    CHECK(aq_labels_from_map(nullptr, 2, 3, lab) == AQ_ERR_NULL);
    CHECK(aq_labels_from_map(z, 0, 3, lab) == AQ_ERR_SHAPE);
    aq_plan p;
    uint8_t l8[16] = {0};
    CHECK(aq_plan_pack(256, 512, 64, 128, l8, &p) == AQ_OK && p.T4 == 0 && p.T8 == 16);
    CHECK(aq_plan_pack(256, 512, 64, 48, l8, &p) == AQ_ERR_TILE);
    CHECK(aq_plan_pack(256, 512, 64, 96, l8, &p) == AQ_ERR_SHAPE);
    CHECK(aq_plan_pack(250, 512, 64, 128, l8, &p) == AQ_ERR_SHAPE);
    CHECK(aq_plan_pack(256, 512, 64, 128, nullptr, &p) == AQ_ERR_NULL);
    int bM, rows, cols;
    CHECK(aq_act_group_shape(1, 128, &bM, &rows, &cols) == AQ_OK && bM == 1 && rows == 1 && cols == 2);
    CHECK(aq_act_group_shape(33, 64, &bM, &rows, &cols) == AQ_OK && bM == 16 && rows == 3 && cols == 1);
    CHECK(aq_act_group_shape(4, 96, &bM, &rows, &cols) == AQ_ERR_SHAPE);
    CHECK(aq_act_group_shape(4, 64, nullptr, &rows, &cols) == AQ_ERR_NULL);
  }

  // packing: validation, the host metadata image, a forced copy failure
  for (int bK : {64, 128}) {
    Fake f = make(512, 1024, bK, 0.6, 3 + bK);
    struct Ctx { Fake *f; bool mse; } c{&f, false};
    auto pack = [](void *v) {
      Ctx *c = (Ctx *)v;
      return c->mse ? aq_pack_weights_mse((const float *)dev(0), c->f->labels.data(), &c->f->p, nullptr)
                    : aq_pack_weights((const float *)dev(0), c->f->labels.data(), &c->f->p, nullptr);
    };
    expect_launch(pack, &c, "aq_pack_weights", false);
    c.mse = true;
    expect_launch(pack, &c, "aq_pack_weights_mse", false);
    CHECK(aq_pack_weights((const float *)dev(4), f.labels.data(), &f.p, nullptr) == AQ_ERR_ALIGN);
    aq_packed bad = f.p;
    bad.T4 += 1;
    CHECK(aq_pack_weights((const float *)dev(0), f.labels.data(), &bad, nullptr) == AQ_ERR_MAP);
    bad = f.p;
    bad.bN = 32;
    CHECK(aq_pack_weights((const float *)dev(0), f.labels.data(), &bad, nullptr) == AQ_ERR_TILE);
  }

  // activation quantizers
  {
    auto qa = [](void *) { return aq_quant_act((const float *)dev(0), 7, 192, (int8_t *)dev(4096), (float *)dev(8192), nullptr); };
    expect_launch(qa, nullptr, "aq_quant_act");
    CHECK(aq_quant_act((const float *)dev(0), 7, 100, (int8_t *)dev(4096), (float *)dev(8192), nullptr) == AQ_ERR_SHAPE);
    CHECK(aq_quant_act((const float *)dev(8), 7, 192, (int8_t *)dev(4096), (float *)dev(8192), nullptr) == AQ_ERR_ALIGN);
    CHECK(aq_quant_act(nullptr, 7, 192, (int8_t *)dev(4096), (float *)dev(8192), nullptr) == AQ_ERR_NULL);
    CHECK(aq_quant_act(nullptr, 0, 192, nullptr, nullptr, nullptr) == AQ_OK);
    auto qg = [](void *) { return aq_quant_act_grouped((const float *)dev(0), 17, 128, (int8_t *)dev(4096), (float *)dev(8192), nullptr); };
    expect_launch(qg, nullptr, "aq_quant_act_grouped");
  }

  // linears: every shape class of the planner, invalid arguments, forced failures
  const int shapes[][3] = {{256, 512, 128}, {3072, 8192, 128}, {16384, 3072, 128}, {6144, 2560, 128},
                           {19456, 2560, 128}, {192, 640, 64}, {256, 65536, 128}};
  for (const auto &sh : shapes) {
    Fake f = make(sh[0], sh[1], sh[2], 0.7, sh[0] + sh[1]);
    for (int M : {1, 4, 16, 33, 64, 100, 1024, 2048}) {
      const size_t wd = aq_workspace_bytes(&f.p, M, AQ_PHASE_DECODE, 0);
      const size_t wp = aq_workspace_bytes(&f.p, M, AQ_PHASE_PREFILL, 0);
      std::vector<unsigned char> wsd(wd + 256), wsp(wp + 256);
      unsigned char *wsd_a = wsd.data() + (256 - (uintptr_t)wsd.data() % 256) % 256;
      unsigned char *wsp_a = wsp.data() + (256 - (uintptr_t)wsp.data() % 256) % 256;
      struct Ctx { Fake *f; int M; void *wd; size_t nd; void *wp; size_t np; } c{&f, M, wd ? wsd_a : nullptr, wd,
                                                                                 wp ? wsp_a : nullptr, wp};
      expect_launch([](void *v) { Ctx *c = (Ctx *)v;
        return aq_linear_decode(&c->f->p, (const int8_t *)dev(0), (const float *)dev(4096), c->M, nullptr,
                                (float *)dev(8192), 0, c->wd, c->nd, nullptr); }, &c, "aq_linear_decode");
      expect_launch([](void *v) { Ctx *c = (Ctx *)v;
        return aq_linear_prefill(&c->f->p, (const int8_t *)dev(0), (const float *)dev(4096), c->M,
                                 (const float *)dev(12288), (float *)dev(8192), c->wp, c->np, nullptr); }, &c,
                    "aq_linear_prefill");
      expect_launch([](void *v) { Ctx *c = (Ctx *)v;
        return aq_linear_tile_partials(&c->f->p, (const int8_t *)dev(0), c->M, AQ_PHASE_PREFILL,
                                       (int32_t *)dev(8192), c->wp, c->np, nullptr); }, &c, "aq_linear_tile_partials");
      if (wd <= AQ_DECODE_SCRATCH_BYTES)
        expect_launch([](void *v) { Ctx *c = (Ctx *)v;
          return aq_linear_decode_noalloc(&c->f->p, (const int8_t *)dev(0), (const float *)dev(4096), c->M,
                                          nullptr, (float *)dev(8192), 0, nullptr); }, &c, "aq_linear_decode_noalloc");
      else
        CHECK(aq_linear_decode_noalloc(&f.p, (const int8_t *)dev(0), (const float *)dev(4096), M, nullptr,
                                       (float *)dev(8192), 0, nullptr) == AQ_ERR_WORKSPACE);
      if (M <= 64 && sh[1] % 64 == 0) {
        int bM, rows, cols;
        CHECK(aq_act_group_shape(M, sh[1], &bM, &rows, &cols) == AQ_OK);
        expect_launch([](void *v) { Ctx *c = (Ctx *)v;
          return aq_linear_decode_grouped(&c->f->p, (const int8_t *)dev(0), (const float *)dev(4096), c->M,
                                          nullptr, (float *)dev(8192), 0, c->wd, c->nd, nullptr); }, &c,
                      "aq_linear_decode_grouped");
      }
      {
        // the transformed decode: its own workspace size (hand-over of tile rows)
        const size_t wx = aq_workspace_bytes(&f.p, M, AQ_PHASE_DECODE_TRANSFORMED, 0);
        CHECK(wx >= wd);
        std::vector<unsigned char> wsx(wx + 256);
        unsigned char *wsx_a = wsx.data() + (256 - (uintptr_t)wsx.data() % 256) % 256;
        struct X { Fake *f; int M; void *w; size_t n; } xc{&f, M, wx ? wsx_a : nullptr, wx};
        expect_launch([](void *v) { X *c = (X *)v;
          return aq_linear_decode_transformed(&c->f->p, (const int8_t *)dev(0), (const float *)dev(4096), c->M,
                                              (const float *)dev(12288), (const int8_t *)dev(16384), &g_tables,
                                              (float *)dev(8192), 0, c->w, c->n, nullptr); }, &xc,
                      "aq_linear_decode_transformed");
        const int before = g_launches;
        if (wx)
          CHECK(aq_linear_decode_transformed(&f.p, (const int8_t *)dev(0), (const float *)dev(4096), M, nullptr,
                                             (const int8_t *)dev(16384), &g_tables, (float *)dev(8192), 0, wsx_a,
                                             wx - 1, nullptr) == AQ_ERR_WORKSPACE);
        CHECK(aq_linear_decode_transformed(&f.p, (const int8_t *)dev(0), (const float *)dev(4096), M, nullptr,
                                           nullptr, &g_tables, (float *)dev(8192), 0, xc.w, xc.n,
                                           nullptr) == AQ_ERR_NULL);
        aq_transform_tables bad = g_tables;
        bad.dl[1][3] = 2;
        CHECK(aq_linear_decode_transformed(&f.p, (const int8_t *)dev(0), (const float *)dev(4096), M, nullptr,
                                           (const int8_t *)dev(16384), &bad, (float *)dev(8192), 0, xc.w, xc.n,
                                           nullptr) == AQ_ERR_ARG);
        CHECK(aq_linear_decode_transformed(&f.p, (const int8_t *)dev(0), (const float *)dev(4096), M, nullptr,
                                           (const int8_t *)dev(16384), &g_tables, (float *)dev(8192), 5, xc.w,
                                           xc.n, nullptr) == AQ_ERR_ARG);
        CHECK(g_launches == before);
      }
      {
        // decode from FP32 activations: one kernel (no workspace) or the
        // quantizer into the workspace behind a whole counter block
        const size_t wf = aq_workspace_bytes(&f.p, M, AQ_PHASE_DECODE_FP32, 0);
        CHECK(wf == 0 || wf >= wd + (size_t)M * sh[1]);
        CHECK(wf == 0 || wf >= ((size_t)256 << 10));
        std::vector<unsigned char> wsf(wf + 256);
        unsigned char *wsf_a = wsf.data() + (256 - (uintptr_t)wsf.data() % 256) % 256;
        struct F32 { Fake *f; int M; void *w; size_t n; } fc{&f, M, wf ? wsf_a : nullptr, wf};
        expect_launch([](void *v) { F32 *c = (F32 *)v;
          return aq_linear_decode_fp32(&c->f->p, (const float *)dev(0), c->M, (const float *)dev(12288),
                                       (float *)dev(8192), 0, c->w, c->n, nullptr); }, &fc, "aq_linear_decode_fp32");
        const int before = g_launches;
        if (wf)
          CHECK(aq_linear_decode_fp32(&f.p, (const float *)dev(0), M, nullptr, (float *)dev(8192), 0, wsf_a, wf - 1,
                                      nullptr) == AQ_ERR_WORKSPACE);
        CHECK(aq_linear_decode_fp32(&f.p, nullptr, M, nullptr, (float *)dev(8192), 0, fc.w, fc.n, nullptr) ==
              AQ_ERR_NULL);
        CHECK(aq_linear_decode_fp32(&f.p, (const float *)dev(4), M, nullptr, (float *)dev(8192), 0, fc.w, fc.n,
                                    nullptr) == AQ_ERR_ALIGN);
        CHECK(aq_linear_decode_fp32(&f.p, (const float *)dev(0), M, nullptr, (float *)dev(8192), 5, fc.w, fc.n,
                                    nullptr) == AQ_ERR_ARG);
        CHECK(aq_linear_decode_fp32(&f.p, (const float *)dev(0), -1, nullptr, (float *)dev(8192), 0, fc.w, fc.n,
                                    nullptr) == AQ_ERR_SHAPE);
        CHECK(aq_linear_decode_fp32(&f.p, (const float *)dev(0), 0, nullptr, nullptr, 0, nullptr, 0, nullptr) ==
              AQ_OK);
        CHECK(g_launches == before);
      }
      {
        const size_t wg = aq_workspace_bytes(&f.p, M, AQ_PHASE_PREFILL_GROUPED, 0);
        std::vector<unsigned char> wsg(wg + 256);
        unsigned char *wsg_a = wsg.data() + (256 - (uintptr_t)wsg.data() % 256) % 256;
        struct G { Fake *f; int M; void *w; size_t n; } gc{&f, M, wg ? wsg_a : nullptr, wg};
        expect_launch([](void *v) { G *c = (G *)v;
          return aq_linear_prefill_grouped(&c->f->p, (const int8_t *)dev(0), (const float *)dev(4096), c->M,
                                           nullptr, (float *)dev(8192), c->w, c->n, nullptr); }, &gc,
                      "aq_linear_prefill_grouped");
        expect_launch([](void *v) { G *c = (G *)v;
          return aq_linear_tile_partials_grouped(&c->f->p, (const int8_t *)dev(0), c->M, (int32_t *)dev(8192),
                                                 c->w, c->n, nullptr); }, &gc, "aq_linear_tile_partials_grouped");
        if (wg)
          CHECK(aq_linear_prefill_grouped(&f.p, (const int8_t *)dev(0), (const float *)dev(4096), M, nullptr,
                                          (float *)dev(8192), wsg_a, wg - 1, nullptr) == AQ_ERR_WORKSPACE);
      }
      // rejected before any launch
      const int before = g_launches;
      if (wd) CHECK(aq_linear_decode(&f.p, (const int8_t *)dev(0), (const float *)dev(4096), M, nullptr,
                                     (float *)dev(8192), 0, wsd_a, wd - 1, nullptr) == AQ_ERR_WORKSPACE);
      if (wp) CHECK(aq_linear_prefill(&f.p, (const int8_t *)dev(0), (const float *)dev(4096), M, nullptr,
                                      (float *)dev(8192), nullptr, 0, nullptr) == AQ_ERR_WORKSPACE);
      CHECK(aq_linear_decode(&f.p, (const int8_t *)dev(4), (const float *)dev(4096), M, nullptr,
                             (float *)dev(8192), 0, c.wd, c.nd, nullptr) == AQ_ERR_ALIGN);
      CHECK(aq_linear_prefill(&f.p, nullptr, (const float *)dev(4096), M, nullptr, (float *)dev(8192), c.wp,
                              c.np, nullptr) == AQ_ERR_NULL);
      CHECK(aq_linear_decode(&f.p, (const int8_t *)dev(0), (const float *)dev(4096), M, nullptr,
                             (float *)dev(8192), 3, c.wd, c.nd, nullptr) == AQ_ERR_ARG);
      CHECK(aq_linear_decode(&f.p, (const int8_t *)dev(0), (const float *)dev(4096), -1, nullptr,
                             (float *)dev(8192), 0, nullptr, 0, nullptr) == AQ_ERR_SHAPE);
      CHECK(g_launches == before);
    }
  }

  // the long-prompt operand preparation and the transformed route
  {
    Fake f = make(6144, 2560, 128, 0.7, 11);
    const size_t wp = aq_workspace_bytes(&f.p, 2048, AQ_PHASE_PREFILL, 0);
    std::vector<unsigned char> ws(wp + 256);
    unsigned char *w = ws.data() + (256 - (uintptr_t)ws.data() % 256) % 256;
    struct Ctx { Fake *f; void *w; size_t n; aq_transform_tables t; } c{&f, w, wp, {}};
    for (int s = 0; s < AQ_TRANSFORM_SEEDS; ++s)
      for (int e = 0; e < 64; ++e) {
        c.t.perm[s][e] = (uint8_t)((e * 5 + s) % 64);
        c.t.dl[s][e] = (e + s) % 3 ? 1 : -1;
        c.t.dr[s][e] = (e * s) % 2 ? -1 : 1;
      }
    expect_launch([](void *v) { Ctx *c = (Ctx *)v; return aq_prefill_prepare(&c->f->p, c->w, c->n, nullptr); }, &c,
                  "aq_prefill_prepare");
    expect_launch([](void *v) { Ctx *c = (Ctx *)v;
      return aq_linear_prefill_prepared(&c->f->p, (const int8_t *)dev(0), (const float *)dev(4096), 2048, nullptr,
                                        (float *)dev(8192), c->w, c->n, nullptr); }, &c, "aq_linear_prefill_prepared");
    expect_launch([](void *v) { Ctx *c = (Ctx *)v;
      return aq_linear_prefill_transformed(&c->f->p, (const int8_t *)dev(0), (const float *)dev(4096), 2048,
                                           nullptr, (const int8_t *)dev(12288), &c->t, (float *)dev(8192), c->w, c->n,
                                           nullptr); }, &c, "aq_linear_prefill_transformed");
    expect_launch([](void *v) { Ctx *c = (Ctx *)v;
      return aq_transform_rows((const float *)dev(0), 5, 640, (const int8_t *)dev(4096), &c->t, (float *)dev(8192),
                               nullptr); }, &c, "aq_transform_rows");
    expect_launch([](void *v) { Ctx *c = (Ctx *)v;
      return aq_transform_out((const float *)dev(0), 5, 640, (const int8_t *)dev(4096), &c->t, nullptr,
                              (float *)dev(8192), nullptr); }, &c, "aq_transform_out");
    expect_launch([](void *v) { Ctx *c = (Ctx *)v;
      return aq_quant_act_transformed((const float *)dev(0), 5, 640, (const int8_t *)dev(4096), &c->t,
                                      (int8_t *)dev(8192), (float *)dev(12288), nullptr); }, &c,
                  "aq_quant_act_transformed");
    expect_launch([](void *v) { Ctx *c = (Ctx *)v;
      return aq_transform_weights((const float *)dev(0), 128, 640, (const int8_t *)dev(1 << 19),
                                  (const int8_t *)dev((1 << 19) + 256), &c->t, (float *)dev(409600), nullptr); }, &c,
                  "aq_transform_weights");
    aq_transform_tables bad = c.t;
    bad.perm[2][7] = bad.perm[2][8];  // not a permutation
    CHECK(aq_transform_rows((const float *)dev(0), 5, 640, (const int8_t *)dev(4096), &bad, (float *)dev(8192),
                            nullptr) == AQ_ERR_ARG);
    bad = c.t;
    bad.dr[0][0] = 0;
    CHECK(aq_transform_out((const float *)dev(0), 5, 640, (const int8_t *)dev(4096), &bad, nullptr,
                           (float *)dev(8192), nullptr) == AQ_ERR_ARG);
    CHECK(aq_transform_weights((const float *)dev(0), 128, 640, (const int8_t *)dev(1 << 19),
                               (const int8_t *)dev((1 << 19) + 256), &c.t, (float *)dev(4096), nullptr) == AQ_ERR_ARG);
  }

  std::printf(failures ? "host ABI check: %d failure(s)\n" : "host ABI check: ok\n", failures);
  return failures ? 1 : 0;
}
