// Host-only check of libdspark's argument validation and workspace layout
// (csrc/plan.cpp), built with AddressSanitizer and UndefinedBehaviorSanitizer
// by tests/test_plan_sanitized.py.  Every validate_* / plan_* function is
// called on a seeded sweep of sizes (extremes included) and struct contents;
// for each accepted argument set the workspace layout must be 256-byte
// aligned, ordered and inside the reported total.  A sanitizer report or a
// failed invariant ends the run with a nonzero status.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

#include "plan.h"

using namespace dspark;

static int g_fail = 0;
#define EXPECT(c)                                                   \
  do {                                                              \
    if (!(c)) {                                                     \
      std::fprintf(stderr, "invariant failed line %d: %s\n", __LINE__, #c); \
      ++g_fail;                                                     \
    }                                                               \
  } while (0)

static const int32_t kInts[] = {INT32_MIN, -1024, -1, 0, 1, 2, 3, 7, 8, 15, 16, 17, 24, 64, 65, 512, 513, 1023,
                                1024, 1025, 4096, 151936, (1 << 24), (1 << 24) + 1, (1 << 30), (1 << 30) + 1,
                                INT32_MAX};
static const int64_t kLongs[] = {INT64_MIN, -1, 0, 1, 5, 448, 1LL << 31, 1LL << 40, INT64_MAX};

static void* fake(std::mt19937_64& g, bool allow_null = true) {
  // plausible addresses: 256-aligned, slightly misaligned, or NULL
  const unsigned k = g() % 8;
  if (allow_null && k == 0) return nullptr;
  uintptr_t base = 0x100000 + ((g() % 4096) << 8);
  if (k == 1) base += 4;
  if (k == 2) base += 2;
  return reinterpret_cast<void*>(base);
}

template <class T>
static T pick(std::mt19937_64& g, const T* v, size_t n) { return v[g() % n]; }

static void check_layout(const DraftPlan& p) {
  EXPECT(p.part_off == kHeaderBytes);
  EXPECT(p.total >= p.part_off);
  EXPECT(p.total % kWsAlign == 0);
  EXPECT(p.n_seg >= 1);
}

static void check_layout(const VerifyPlan& p) {
  EXPECT(p.vpart_off == kHeaderBytes);
  EXPECT(p.vpart_off <= p.rsinfo_off && p.rsinfo_off <= p.rsstats_off && p.rsstats_off <= p.rpart_off);
  EXPECT(p.rpart_off <= p.total);
  for (std::size_t o : {p.vpart_off, p.rsinfo_off, p.rsstats_off, p.rpart_off, p.total}) EXPECT(o % kWsAlign == 0);
  if (p.seg_rows == kSegWide) {
    EXPECT(p.rpart_off < p.rcount_off && p.rcount_off < p.rlist_off && p.rlist_off <= p.total);
  }
}

int main(int argc, char** argv) {
  const int iters = argc > 1 ? std::atoi(argv[1]) : 200000;
  std::mt19937_64 g(20261203);
  const size_t NI = sizeof(kInts) / sizeof(kInts[0]), NL = sizeof(kLongs) / sizeof(kLongs[0]);
  long accepted = 0;
  for (int it = 0; it < iters; ++it) {
    // every other iteration starts from a valid argument set (sizes in range,
    // aligned pointers, a large enough workspace) and perturbs one field
    const bool valid = (it & 1) != 0;
    const int perturb = valid ? static_cast<int>(g() % 24) : -1;
    auto I = [&]() { return (g() % 3 == 0) ? static_cast<int32_t>(g() % 2000) : pick(g, kInts, NI); };
    auto P = [&](int field) -> void* {  // pointer for field number `field`
      if (valid && field != perturb) return reinterpret_cast<void*>(0x100000 + ((g() % 4096) << 8));
      return fake(g);
    };
    {
      dspark_draft_args a;
      std::memset(&a, 0, sizeof(a));
      a.struct_size = (!valid && g() % 16 == 0) ? 8u : static_cast<uint32_t>(sizeof(a));
      if (valid) {
        a.R = static_cast<int32_t>(g() % 3000); a.gamma = 1 + static_cast<int32_t>(g() % 16);
        a.V = 1 + static_cast<int32_t>(g() % 300000); a.rank = 8 * (1 + static_cast<int32_t>(g() % 64));
        a.wdtype = static_cast<int32_t>(g() % 2);
        a.flags = static_cast<uint32_t>(g() % 2);
        if (perturb == 20) a.R = I();
        if (perturb == 21) a.V = I();
        if (perturb == 22) a.rank = I();
        if (perturb == 23) a.flags = static_cast<uint32_t>(g());
      } else {
        a.R = I(); a.gamma = I(); a.V = I(); a.rank = I();
        a.wdtype = static_cast<int32_t>(g() % 3);
        a.flags = (g() % 8 == 0) ? static_cast<uint32_t>(g()) : static_cast<uint32_t>(g() % 2);
      }
      a.U = static_cast<const float*>(P(0)); a.W1 = P(1); a.W2 = P(2);
      a.anchor = static_cast<const int32_t*>(P(3)); a.temp = static_cast<const float*>(P(4));
      a.u_draft = static_cast<const float*>(P(5)); a.y = static_cast<int32_t*>(P(6));
      a.q_tok = static_cast<float*>(P(7)); a.q_stats = static_cast<float*>(P(8));
      a.workspace = P(9);
      DraftPlan sz;
      a.workspace_bytes = (valid && perturb != 10 && plan_draft(&a, &sz) == DSPARK_OK) ? sz.total
                          : ((g() % 2) ? (g() % (1ull << 34)) : SIZE_MAX);
      a.W2_packed = (g() % 2) ? P(11) : nullptr;
      a.W2_packed_bytes = (valid && perturb != 12 && a.wdtype == DSPARK_W_BF16 && a.V > 0 && a.rank > 0)
                              ? w2_packed_bytes(a.V, a.rank) : g() % (1ull << 33);
      DraftPlan p;
      const int st = validate_draft(&a, &p);
      std::size_t bytes = 0;
      DraftPlan q;
      const int st2 = plan_draft(&a, &q);
      if (st2 == DSPARK_OK) {
        check_layout(q);
        bytes = q.total;
        EXPECT(a.R >= 0 && a.gamma >= 1 && a.gamma <= DSPARK_MAX_GAMMA && a.rank % 8 == 0);
      }
      if (st == DSPARK_OK && a.R > 0) {
        ++accepted;
        EXPECT(st2 == DSPARK_OK && a.workspace_bytes >= bytes && a.workspace != nullptr);
        if (a.W2_packed) EXPECT(a.W2_packed_bytes >= w2_packed_bytes(a.V, a.rank));
      }
    }
    {
      dspark_verify_args a;
      std::memset(&a, 0, sizeof(a));
      a.struct_size = static_cast<uint32_t>(sizeof(a));
      if (valid) {
        a.R = static_cast<int32_t>(g() % 3000); a.gamma = 1 + static_cast<int32_t>(g() % 16);
        a.V = 1 + static_cast<int32_t>(g() % 300000); a.rank = 8 * (1 + static_cast<int32_t>(g() % 64));
        a.wdtype = static_cast<int32_t>(g() % 2);
        a.flags = static_cast<uint32_t>(g() % 2);
        a.n_rows = a.R + static_cast<int64_t>(g() % (static_cast<uint64_t>(a.R) * a.gamma + 1));
        if (perturb == 20) a.n_rows = pick(g, kLongs, NL);
        if (perturb == 21) a.V = I();
      } else {
        a.R = I(); a.gamma = I(); a.V = I(); a.rank = I();
        a.wdtype = static_cast<int32_t>(g() % 3);
        a.flags = static_cast<uint32_t>(g() % 3);
        a.n_rows = (g() % 2) ? pick(g, kLongs, NL) : static_cast<int64_t>(a.R) * static_cast<int64_t>(1 + g() % 17);
      }
      void** ptrs[] = {(void**)&a.target, (void**)&a.row_offsets, (void**)&a.U, (void**)&a.W1, (void**)&a.W2,
                       (void**)&a.anchor, (void**)&a.temp, (void**)&a.y, (void**)&a.q_tok, (void**)&a.q_stats,
                       (void**)&a.u_accept, (void**)&a.u_final, (void**)&a.n_accept, (void**)&a.out_tok,
                       (void**)&a.p_tok};
      int fi = 0;
      for (void** pp : ptrs) *pp = valid ? P(fi++) : fake(g, g() % 4 == 0);
      a.workspace = P(16);
      VerifyPlan sz;
      a.workspace_bytes = (valid && perturb != 17 && plan_verify(&a, &sz) == DSPARK_OK) ? sz.total
                          : g() % (1ull << 36);
      a.W2_packed = (g() % 2) ? P(18) : nullptr;
      a.W2_packed_bytes = (valid && perturb != 19 && a.wdtype == DSPARK_W_BF16 && a.V > 0 && a.rank > 0)
                              ? w2_packed_bytes(a.V, a.rank) : g() % (1ull << 33);
      VerifyPlan p;
      const int st = validate_verify(&a, &p);
      VerifyPlan q;
      if (plan_verify(&a, &q) == DSPARK_OK) {
        check_layout(q);
        EXPECT(a.n_rows >= a.R && a.n_rows <= static_cast<int64_t>(a.R) * (a.gamma + 1));
      }
      if (st == DSPARK_OK && a.R > 0) {
        ++accepted;
        EXPECT(a.workspace_bytes >= q.total);
      }
    }
    {
      dspark_schedule_args a;
      std::memset(&a, 0, sizeof(a));
      a.struct_size = static_cast<uint32_t>(sizeof(a));
      a.R = valid ? static_cast<int32_t>(g() % 20000) : I();
      a.gamma = valid ? 1 + static_cast<int32_t>(g() % 16) : I();
      a.K = pick(g, kLongs, NL);
      a.flags = static_cast<uint32_t>(g() % 3);
      void** ptrs[] = {(void**)&a.c, (void**)&a.anchor, (void**)&a.y, (void**)&a.a, (void**)&a.l,
                       (void**)&a.row_offsets, (void**)&a.row_req, (void**)&a.row_pos, (void**)&a.row_tok};
      int fi = 0;
      for (void** pp : ptrs) *pp = valid ? P(fi++) : fake(g, g() % 4 == 0);
      a.workspace = P(10); a.workspace_bytes = (valid && perturb != 11) ? 256 : g() % 1024;
      std::size_t need = 0;
      const int sp = plan_schedule(&a, &need);
      if (sp == DSPARK_OK) EXPECT(need == ((a.flags & DSPARK_CHECK_INPUTS) ? kHeaderBytes : 0));
      const int st = validate_schedule(&a);
      if (st == DSPARK_OK && a.R > 0 && need) EXPECT(a.workspace_bytes >= need);
      const int64_t rows = schedule_rows(a.R, a.gamma, a.K);
      if (a.R >= 0 && a.gamma >= 1) EXPECT(rows >= a.R && rows <= static_cast<int64_t>(a.R) * (static_cast<int64_t>(a.gamma) + 1));
      else EXPECT(rows == -1);
    }
    {
      dspark_cutoff_args a;
      std::memset(&a, 0, sizeof(a));
      a.struct_size = static_cast<uint32_t>(sizeof(a));
      a.R = I(); a.gamma = I();
      const float cm[] = {-1.f, 0.f, 0.5f, 1.f, 2.f, __builtin_nanf("")};
      a.conf_min = cm[g() % 6];
      a.flags = static_cast<uint32_t>(g() % 3);
      void** ptrs[] = {(void**)&a.c, (void**)&a.anchor, (void**)&a.y, (void**)&a.a, (void**)&a.l,
                       (void**)&a.row_offsets, (void**)&a.row_req, (void**)&a.row_pos, (void**)&a.row_tok};
      for (void** pp : ptrs) *pp = fake(g, g() % 4 == 0);
      a.workspace = fake(g); a.workspace_bytes = g() % 1024;
      (void)validate_cutoff(&a);
      std::size_t need = 0;
      (void)plan_cutoff(&a, &need);
    }
    {
      dspark_pack_w2_args a;
      std::memset(&a, 0, sizeof(a));
      a.struct_size = static_cast<uint32_t>(sizeof(a));
      a.V = I(); a.rank = I();
      a.W2 = fake(g); a.W2_packed = fake(g); a.W2_packed_bytes = g() % (1ull << 34);
      if (validate_pack_w2(&a) == DSPARK_OK) EXPECT(a.W2_packed_bytes >= w2_packed_bytes(a.V, a.rank));
    }
    {
      dspark_capacity_args a;
      std::memset(&a, 0, sizeof(a));
      a.struct_size = static_cast<uint32_t>(sizeof(a));
      a.R = I(); a.gamma = I(); a.n_sps = I();
      a.a_lag = static_cast<const float*>(fake(g)); a.sps = static_cast<const float*>(fake(g));
      a.K = static_cast<int32_t*>(fake(g)); a.expected = static_cast<double*>(fake(g));
      a.theta = static_cast<double*>(fake(g));
      if (validate_capacity(&a) == DSPARK_OK)
        EXPECT(static_cast<int64_t>(a.R) * a.gamma <= DSPARK_CAPACITY_MAX_CANDIDATES && a.n_sps >= a.R + 1);
    }
    {
      dspark_sts_fit_args f;
      std::memset(&f, 0, sizeof(f));
      f.struct_size = static_cast<uint32_t>(sizeof(f));
      f.N = I(); f.gamma = I();
      f.z = static_cast<const float*>(fake(g)); f.n_acc = static_cast<const int32_t*>(fake(g));
      f.tau = static_cast<float*>(fake(g));
      (void)validate_sts_fit(&f);
      dspark_sts_apply_args s;
      std::memset(&s, 0, sizeof(s));
      s.struct_size = static_cast<uint32_t>(sizeof(s));
      s.R = I(); s.gamma = I();
      s.z = static_cast<const float*>(fake(g)); s.tau = static_cast<const float*>(fake(g));
      s.c = static_cast<float*>(fake(g));
      (void)validate_sts_apply(&s);
    }
    for (int st = -2; st < 12; ++st) EXPECT(status_string(st) != nullptr);
    (void)w2_packed_bytes(1 << 30, 512);
  }
  // NULL argument structs
  DraftPlan dp;
  VerifyPlan vp;
  std::size_t n = 0;
  EXPECT(validate_draft(nullptr, &dp) == DSPARK_ERR_NULL);
  EXPECT(validate_verify(nullptr, &vp) == DSPARK_ERR_NULL);
  EXPECT(plan_schedule(nullptr, &n) == DSPARK_ERR_NULL);
  EXPECT(plan_cutoff(nullptr, &n) == DSPARK_ERR_NULL);
  EXPECT(validate_schedule(nullptr) == DSPARK_ERR_NULL);
  EXPECT(validate_cutoff(nullptr) == DSPARK_ERR_NULL);
  EXPECT(validate_pack_w2(nullptr) == DSPARK_ERR_NULL);
  EXPECT(validate_capacity(nullptr) == DSPARK_ERR_NULL);
  EXPECT(validate_sts_fit(nullptr) == DSPARK_ERR_NULL);
  EXPECT(validate_sts_apply(nullptr) == DSPARK_ERR_NULL);
  std::printf("plan_sanitize: %d iterations, %ld accepted argument sets, %d failures\n", iters, accepted, g_fail);
  // the valid half of the sweep must mostly pass validation, or it tests little
  EXPECT(accepted > iters / 4);
  return g_fail == 0 ? 0 : 1;
}
