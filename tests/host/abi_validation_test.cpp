// Host-only check of the C ABI's argument validation, built together with the
// library's host code under AddressSanitizer + UndefinedBehaviorSanitizer and
// run where no GPU is visible.  Every call below must be rejected on the host
// with the documented status before anything is enqueued; the fake device
// pointers are never dereferenced.  The size sweep drives natsl_workspace_size
// through extreme shapes so that an overflow in its size arithmetic is caught
// as undefined behaviour; the thread part exercises the thread-local error
// text from several threads at once.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <string>
#include <thread>
#include <vector>

#include "../../include/natsl.h"

static int g_fail = 0, g_run = 0;
#define EXPECT(cond)                                                              \
  do {                                                                            \
    ++g_run;                                                                      \
    if (!(cond)) {                                                                \
      ++g_fail;                                                                   \
      printf("FAILED %s:%d: %s (last error: %s)\n", __FILE__, __LINE__, #cond,    \
             natsl_last_error());                                                 \
    }                                                                             \
  } while (0)

static void* const FAKE = (void*)0x10000;

static natsl_dims dims(int B, int H, int L, int D, int dm, natsl_dtype io) {
  natsl_dims d;
  memset(&d, 0, sizeof d);
  d.B = B; d.H = H; d.L = L; d.Dk = D; d.Dv = D; d.d_model = dm; d.chunk = 64; d.route_groups = 1; d.io = io;
  return d;
}
static natsl_dims good() { return dims(2, 4, 256, 128, 256, NATSL_BF16); }

static void fill_cache(natsl_decode_cache* c) {
  memset(c, 0, sizeof *c);
  c->k_cache = c->v_cache = FAKE;
  c->n_committed = c->n_open = c->err_flag = (int32_t*)FAKE;
  c->S_carry = c->S_work = c->x_sum = (float*)FAKE;
  c->cap = 1024;
}

static void dims_checks() {
  size_t n = 0;
  natsl_dims d = good();
  EXPECT(natsl_workspace_size(NATSL_ENTRY_FORWARD, &d, &n) == NATSL_OK);
  EXPECT(natsl_workspace_size(NATSL_ENTRY_FORWARD, nullptr, &n) == NATSL_ERR_INVALID_ARG);
  EXPECT(natsl_workspace_size(NATSL_ENTRY_FORWARD, &d, nullptr) == NATSL_ERR_INVALID_ARG);
  EXPECT(natsl_workspace_size(99, &d, &n) != NATSL_OK);
  d.chunk = 32;  EXPECT(natsl_workspace_size(NATSL_ENTRY_FORWARD, &d, &n) == NATSL_ERR_UNSUPPORTED);
  d = good(); d.Dv = 64;  EXPECT(natsl_workspace_size(NATSL_ENTRY_FORWARD, &d, &n) == NATSL_ERR_UNSUPPORTED);
  d = good(); d.L = 100;  EXPECT(natsl_workspace_size(NATSL_ENTRY_FORWARD, &d, &n) == NATSL_ERR_UNSUPPORTED);
  d = good(); d.route_groups = 3;  EXPECT(natsl_workspace_size(NATSL_ENTRY_FORWARD, &d, &n) == NATSL_ERR_UNSUPPORTED);
  d = good(); d.H = 0;  EXPECT(natsl_workspace_size(NATSL_ENTRY_FORWARD, &d, &n) == NATSL_ERR_INVALID_ARG);
  d = good(); d.B = -1;  EXPECT(natsl_workspace_size(NATSL_ENTRY_FORWARD, &d, &n) == NATSL_ERR_INVALID_ARG);
  d = good(); d.io = (natsl_dtype)7;  EXPECT(natsl_workspace_size(NATSL_ENTRY_FORWARD, &d, &n) == NATSL_ERR_INVALID_ARG);
  // B * H * L must stay below 2^31
  d = dims(1 << 16, 16, 1 << 12, 128, 256, NATSL_BF16);
  EXPECT(natsl_workspace_size(NATSL_ENTRY_FORWARD, &d, &n) != NATSL_OK);
  d = dims(1, 1, 64 * 15233, 128, 256, NATSL_BF16);
  EXPECT(natsl_workspace_size(NATSL_ENTRY_FORWARD, &d, &n) == NATSL_ERR_UNSUPPORTED);
}

// Every entry id over a grid of shapes, including the largest accepted ones.
static void workspace_sweep() {
  const int Bs[] = {0, 1, 3, 64, 4096, 1 << 20};
  const int Hs[] = {1, 16, 1024, 1025};
  const int Ls[] = {64, 4096, 64 * 15232, 64 * 15233, 1 << 30, 2147483647};
  const int Ds[] = {64, 128};
  const int dms[] = {8, 256, 32768, 32776};
  int accepted = 0;
  for (int B : Bs)
    for (int H : Hs)
      for (int L : Ls)
        for (int D : Ds)
          for (int dm : dms)
            for (int io = 0; io < 2; ++io)
              for (int g = 0; g < 2; ++g)
                for (int entry = 0; entry <= NATSL_ENTRY_ROUTE_BACKWARD; ++entry) {
                  natsl_dims d = dims(B, H, L, D, dm, (natsl_dtype)io);
                  d.route_groups = g ? H : 1;
                  size_t n = 12345;
                  natsl_status s = natsl_workspace_size(entry, &d, &n);
                  EXPECT(s == NATSL_OK || s == NATSL_ERR_INVALID_ARG || s == NATSL_ERR_UNSUPPORTED);
                  if (s == NATSL_OK) {
                    ++accepted;
                    // no size arithmetic wrapped around
                    EXPECT(n < ((size_t)1 << 50));
                    // prefill entries bound B * H * L (decode takes dims->L as its capacity)
                    if (entry != NATSL_ENTRY_DECODE_STEP) EXPECT((long long)B * H * L <= (1LL << 28));
                  }
                }
  EXPECT(accepted > 100);
  for (int slots : {-1, 0, 1, 64, 65, 1 << 20})
    for (int window : {-64, 0, 64, 2048, 1 << 30}) {
      natsl_dims d = dims(1, 16, 32768, 128, 256, NATSL_BF16);
      size_t n = 0;
      natsl_status s = natsl_nha_workspace_size(&d, slots, window, &n);
      EXPECT(s == NATSL_OK || s == NATSL_ERR_INVALID_ARG || s == NATSL_ERR_UNSUPPORTED);
    }
}

static void entry_checks() {
  natsl_dims d = good();
  void* F = FAKE;
  const float* Ff = (const float*)FAKE;
  float* Fw = (float*)FAKE;
  int32_t* Fi = (int32_t*)FAKE;
  // router
  EXPECT(natsl_route(nullptr, F, Ff, Ff, nullptr, Fi, Fi, Fi, Fw, nullptr) == NATSL_ERR_INVALID_ARG);
  EXPECT(natsl_route(&d, nullptr, Ff, Ff, nullptr, Fi, Fi, Fi, Fw, nullptr) == NATSL_ERR_INVALID_ARG);
  EXPECT(natsl_route(&d, F, Ff, Ff, nullptr, Fi, nullptr, Fi, Fw, nullptr) == NATSL_ERR_INVALID_ARG);
  d.d_model = 12;
  EXPECT(natsl_route(&d, F, Ff, Ff, nullptr, Fi, Fi, Fi, Fw, nullptr) == NATSL_ERR_UNSUPPORTED);
  d = good();
  // Gated DeltaNet chunk: workspace missing, misaligned, too small; route missing; bad dtype
  size_t need = 0;
  EXPECT(natsl_workspace_size(NATSL_ENTRY_GDN_CHUNK, &d, &need) == NATSL_OK && need > 0);
  EXPECT(natsl_gdn_chunk(&d, F, F, F, Ff, Ff, Fi, nullptr, F, NATSL_F32, nullptr, nullptr, need, nullptr) ==
         NATSL_ERR_WORKSPACE);
  EXPECT(natsl_gdn_chunk(&d, F, F, F, Ff, Ff, Fi, nullptr, F, NATSL_F32, nullptr, (char*)F + 8, need, nullptr) ==
         NATSL_ERR_WORKSPACE);
  EXPECT(natsl_gdn_chunk(&d, F, F, F, Ff, Ff, Fi, nullptr, F, NATSL_F32, nullptr, F, need - 1, nullptr) ==
         NATSL_ERR_WORKSPACE);
  EXPECT(natsl_gdn_chunk(&d, F, F, F, Ff, Ff, nullptr, nullptr, F, NATSL_F32, nullptr, F, need, nullptr) ==
         NATSL_ERR_INVALID_ARG);
  EXPECT(natsl_gdn_chunk(&d, F, F, F, Ff, Ff, Fi, nullptr, F, (natsl_dtype)5, nullptr, F, need, nullptr) ==
         NATSL_ERR_INVALID_ARG);
  // softmax and merge
  EXPECT(natsl_softmax_masked(&d, F, F, F, nullptr, Fi, F, NATSL_F32, nullptr, nullptr, 0, nullptr) ==
         NATSL_ERR_INVALID_ARG);
  EXPECT(natsl_softmax_masked(&d, F, F, F, Fi, Fi, F, (natsl_dtype)9, nullptr, nullptr, 0, nullptr) ==
         NATSL_ERR_INVALID_ARG);
  EXPECT(natsl_merge(&d, F, F, F, NATSL_F32, nullptr, 0, nullptr, nullptr, F, nullptr) == NATSL_ERR_INVALID_ARG);
  EXPECT(natsl_merge(&d, F, F, F, NATSL_F32, Ff, -2, nullptr, nullptr, F, nullptr) == NATSL_ERR_INVALID_ARG);
  // forward
  natsl_forward_args a;
  memset(&a, 0, sizeof a);
  EXPECT(natsl_forward(&d, nullptr, F, (size_t)1 << 30, nullptr) == NATSL_ERR_INVALID_ARG);
  a.q = a.k = a.v = F;
  a.alpha = a.beta = a.w_mix = Ff;
  a.out = F;
  EXPECT(natsl_forward(&d, &a, F, (size_t)1 << 30, nullptr) == NATSL_ERR_INVALID_ARG);  // no x, no override
  a.route_override = Fi;
  EXPECT(natsl_workspace_size(NATSL_ENTRY_FORWARD, &d, &need) == NATSL_OK);
  EXPECT(natsl_forward(&d, &a, F, need / 4, nullptr) == NATSL_ERR_WORKSPACE);
  a.branch_dtype = (natsl_dtype)3;
  EXPECT(natsl_forward(&d, &a, F, need, nullptr) == NATSL_ERR_INVALID_ARG);
  a.branch_dtype = NATSL_BF16;
  natsl_decode_cache pc;
  memset(&pc, 0, sizeof pc);
  a.prefix = &pc;
  EXPECT(natsl_forward(&d, &a, F, need, nullptr) == NATSL_ERR_INVALID_ARG);  // prefix tensors missing
  fill_cache(&pc);
  a.S_init = Ff;
  EXPECT(natsl_forward(&d, &a, F, need, nullptr) == NATSL_ERR_INVALID_ARG);  // S_init with a prefix
  // decode
  natsl_decode_cache c;
  memset(&c, 0, sizeof c);
  natsl_decode_args da;
  memset(&da, 0, sizeof da);
  EXPECT(natsl_decode_step(&d, &c, &da, nullptr, 0, nullptr) == NATSL_ERR_INVALID_ARG);
  fill_cache(&c);
  c.cap = 0;
  EXPECT(natsl_decode_step(&d, &c, &da, nullptr, 0, nullptr) == NATSL_ERR_INVALID_ARG);
  c.cap = 1024;
  da.x = da.q = da.k = da.v = F;
  da.alpha = da.beta = da.w_score = da.w_mix = Ff;
  da.out = F;
  EXPECT(natsl_decode_step(&d, &c, &da, nullptr, 0, nullptr) == NATSL_ERR_WORKSPACE);
  EXPECT(natsl_decode_step_noalloc(&d, nullptr, &da, nullptr) == NATSL_ERR_INVALID_ARG);
  natsl_dims big = dims(64, 16, 1, 128, 256, NATSL_BF16);
  c.cap = 40000;
  EXPECT(natsl_decode_step_noalloc(&big, &c, &da, nullptr) == NATSL_ERR_WORKSPACE);
  // handoff
  EXPECT(natsl_workspace_size(NATSL_ENTRY_DECODE_HANDOFF, &d, &need) == NATSL_OK);
  c.cap = 1024;
  EXPECT(natsl_decode_handoff(&d, nullptr, F, F, nullptr, 0, &c, F, need, nullptr) == NATSL_ERR_INVALID_ARG);
  EXPECT(natsl_decode_handoff(&d, Fi, F, F, nullptr, 0, &c, F, need - 4, nullptr) == NATSL_ERR_WORKSPACE);
  EXPECT(natsl_decode_handoff(&d, Fi, F, F, nullptr, 1, &c, F, need, nullptr) == NATSL_ERR_INVALID_ARG);
  EXPECT(natsl_decode_handoff(&d, Fi, F, F, Ff, 2, &c, F, need, nullptr) == NATSL_ERR_INVALID_ARG);
  // gradients: missing workspace or tensors
  EXPECT(natsl_softmax_masked_backward(&d, F, F, F, Fi, Fi, F, Ff, F, Fw, Fw, Fw, nullptr, nullptr, 0, nullptr) !=
         NATSL_OK);
  EXPECT(natsl_gdn_backward(&d, F, F, F, Ff, Ff, Fi, nullptr, Ff, nullptr, Fw, Fw, Fw, Fw, Fw, nullptr, nullptr,
                            nullptr, 0, nullptr) != NATSL_OK);
  EXPECT(natsl_merge_backward(&d, F, F, F, NATSL_F32, Ff, 0, nullptr, nullptr, nullptr, Fw, Fw, Fw, Fw, nullptr,
                              nullptr, nullptr, 0, nullptr) == NATSL_ERR_INVALID_ARG);
  EXPECT(natsl_route_backward(&d, F, Ff, Ff, Ff, Ff, Fw, Fw, Fw, nullptr, 0, nullptr) != NATSL_OK);
  EXPECT(natsl_nha_attention(&d, F, F, F, Ff, 0, 64, F, nullptr, 0, nullptr) != NATSL_OK);
  // empty batch: a no-op that succeeds with NULL tensors
  natsl_dims e = good();
  e.B = 0;
  EXPECT(natsl_route(&e, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr) == NATSL_OK);
  EXPECT(natsl_forward(&e, &a, nullptr, 0, nullptr) == NATSL_OK);
  // debug and timing controls (host state only)
  EXPECT(natsl_set_sync_check(3) == NATSL_ERR_INVALID_ARG);
  EXPECT(natsl_set_sync_check(-1) == NATSL_ERR_INVALID_ARG);
  EXPECT(natsl_set_sync_check(2) == NATSL_OK && natsl_get_sync_check() == 2);
  EXPECT(natsl_set_sync_check(0) == NATSL_OK && natsl_get_sync_check() == 0);
  EXPECT(natsl_profile_select("no_such_kernel") == NATSL_ERR_INVALID_ARG);
  EXPECT(natsl_profile_select(nullptr) == NATSL_OK);
  int cnt = 0;
  double ms = 0;
  EXPECT(natsl_profile_read(nullptr, &cnt, &ms) == NATSL_ERR_INVALID_ARG);
  EXPECT(natsl_profile_read("no_such_kernel", &cnt, &ms) == NATSL_ERR_INVALID_ARG);
}

// Several threads fail different validations at once; each must read back
// its own message (the error text is thread-local).
static void thread_checks() {
  std::atomic<int> bad{0};
  std::vector<std::thread> ts;
  for (int t = 0; t < 8; ++t)
    ts.emplace_back([t, &bad] {
      for (int i = 0; i < 2000; ++i) {
        natsl_dims d = good();
        size_t n = 0;
        if (t & 1) {
          d.chunk = 16 + t;
          if (natsl_workspace_size(NATSL_ENTRY_FORWARD, &d, &n) != NATSL_ERR_UNSUPPORTED) ++bad;
          if (!strstr(natsl_last_error(), "chunk")) ++bad;
        } else {
          if (natsl_profile_select("kernel_of_thread") != NATSL_ERR_INVALID_ARG) ++bad;
          if (!strstr(natsl_last_error(), "kernel_of_thread")) ++bad;
        }
        if (natsl_workspace_size(NATSL_ENTRY_FORWARD, &d, &n) == NATSL_OK && natsl_last_error()[0]) ++bad;
      }
    });
  for (auto& t : ts) t.join();
  EXPECT(bad.load() == 0);
}

int main() {
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) == hipSuccess && ndev > 0) {
    printf("a GPU is visible: this host-only check runs without one\n");
    return 77;
  }
  dims_checks();
  workspace_sweep();
  entry_checks();
  thread_checks();
  printf("%d checks, %d errors\n", g_run, g_fail);
  return g_fail ? 1 : 0;
}
