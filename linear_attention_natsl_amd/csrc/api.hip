// C ABI of the NAtS-L hybrid layer: argument validation (before anything is
// enqueued), workspace carving, dtype / head-dim dispatch, the prefill
// fork-join (Gated DeltaNet on a helper stream, softmax on the caller's
// stream), and optional per-kernel event timing.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <set>
#include <string>
#include <utility>
#include <vector>

#include "../../include/natsl.h"
#include "helper_pool.hpp"
#include "kernels.hpp"

namespace natsl {

// (device, kernel) pairs whose dynamic LDS limit has been raised
static std::mutex g_attr_mu;
static std::set<std::pair<int, const void*>> g_attr_done;

hipError_t set_lds_limit(const void* fn, int bytes) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lk(g_attr_mu);
  if (g_attr_done.count({dev, fn})) return hipSuccess;
  e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess) g_attr_done.insert({dev, fn});
  return e;
}

}  // namespace natsl

using namespace natsl;

namespace {

thread_local std::string g_err;

natsl_status fail(natsl_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
natsl_status fail(natsl_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}
natsl_status ok() {
  g_err.clear();
  return NATSL_OK;
}
natsl_status dev_fail(hipError_t e, const char* where) {
  return fail(NATSL_ERR_DEVICE, "%s: %s", where, hipGetErrorString(e));
}

// ------------------------------------------------------------- sync check ----
// Debug mode.  Level 1: every entry point that enqueues work waits for its
// stream before it returns and turns the first error the runtime reports into
// NATSL_ERR_DEVICE naming the entry point.  Level 2 also writes the entry
// point's name to stderr (flushed) before the wait, so that a fault which ends
// the process still names the call that raised it.  A stream under graph
// capture is not waited for.  The level comes from natsl_set_sync_check, else
// from NATSL_SYNC_CHECK in the environment at the first call ("1", "2").
std::atomic<int> g_sync_level{-1};
int sync_level() {
  int v = g_sync_level.load(std::memory_order_acquire);
  if (v >= 0) return v;
  const char* s = getenv("NATSL_SYNC_CHECK");
  int want = 0;
  if (s && s[0] && strcmp(s, "0") != 0) want = strcmp(s, "2") == 0 ? 2 : 1;
  int expect = -1;
  g_sync_level.compare_exchange_strong(expect, want, std::memory_order_acq_rel);
  return g_sync_level.load(std::memory_order_acquire);
}
natsl_status done(hipStream_t st, const char* where) {
  const int lv = sync_level();
  if (lv > 0) {
    if (lv > 1) {
      fprintf(stderr, "natsl sync check: %s\n", where);
      fflush(stderr);
    }
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    hipError_t e = hipStreamIsCapturing(st, &cs);
    if (e == hipSuccess && cs == hipStreamCaptureStatusNone) e = hipStreamSynchronize(st);
    if (e == hipSuccess) e = hipGetLastError();
    if (e != hipSuccess) return fail(NATSL_ERR_DEVICE, "%s (sync check): %s", where, hipGetErrorString(e));
  }
  return ok();
}

size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

// ---------------------------------------------------------------- timing ----
const char* kKernelNames[KID_COUNT] = {"route",        "compact",       "gdn_prep",   "gdn_scan",
                                       "softmax_masked", "merge",       "decode_route", "decode_gdn",
                                       "decode_attn",  "decode_combine", "decode_commit", "softmax_backward", "decode_handoff",
                                       "gdn_backward", "merge_backward", "nha", "nha_window", "nha_chunk", "nha_scan",
                                       "nha_slots", "route_backward"};
struct ProfRec {
  int kid;
  hipEvent_t a, b;
};
std::mutex g_prof_mu;
bool g_prof_on = false;
std::vector<ProfRec> g_prof_pool;  // created on enable
size_t g_prof_used = 0;
int g_prof_open[KID_COUNT];         // index of the record whose start was recorded

int g_prof_only = -1;                // record only this kernel id (-1: all)

void prof_hook(int kid, hipStream_t st, int phase) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (!g_prof_on) return;
  if (g_prof_only >= 0 && kid != g_prof_only) return;
  if (phase == 0) {
    if (g_prof_used >= g_prof_pool.size()) {
      g_prof_open[kid] = -1;
      return;
    }
    ProfRec& r = g_prof_pool[g_prof_used];
    r.kid = kid;
    g_prof_open[kid] = (int)g_prof_used++;
    (void)hipEventRecord(r.a, st);
  } else if (g_prof_open[kid] >= 0) {
    (void)hipEventRecord(g_prof_pool[g_prof_open[kid]].b, st);
  }
}
void (*prof_fn())(int, hipStream_t, int) { return g_prof_on ? prof_hook : nullptr; }

// ------------------------------------------------------------ helper streams ----
// natsl_forward runs the Gated DeltaNet branch on a helper stream (default
// priority) ordered against the caller's stream by three events.  A helper
// (stream + events) belongs to one call for the whole of that call's enqueue
// (HelperPool: taken from a per-device free list, given back when the call
// returns), so concurrent calls from several host threads never share events
// and never serialise on one helper stream.  A helper is reused only after
// its previous call has enqueued all its waits, and a HIP event wait captures
// the record that precedes it, so reuse cannot alias two calls' records.
struct Helper {
  hipStream_t aux = nullptr;
  hipEvent_t fork = nullptr, join = nullptr, routed = nullptr;
};
HelperPool<Helper> g_helpers;

Helper* make_helper(int /*dev: current*/) {
  Helper* h = new Helper();
  if (hipStreamCreateWithFlags(&h->aux, hipStreamNonBlocking) != hipSuccess) {
    delete h;
    return nullptr;
  }
  if (hipEventCreateWithFlags(&h->fork, hipEventDisableTiming) != hipSuccess ||
      hipEventCreateWithFlags(&h->join, hipEventDisableTiming) != hipSuccess ||
      hipEventCreateWithFlags(&h->routed, hipEventDisableTiming) != hipSuccess)
    return nullptr;  // the stream is kept: nothing may destroy a stream another call could use
  return h;
}

natsl_status acquire_helper(HelperPool<Helper>::Lease* lease) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return dev_fail(e, "hipGetDevice");
  Helper* h = g_helpers.acquire(dev, make_helper);
  if (!h) {
    e = hipGetLastError();
    return e != hipSuccess ? dev_fail(e, "helper stream / events") : fail(NATSL_ERR_UNSUPPORTED, "device ordinal %d", dev);
  }
  lease->pool = &g_helpers;
  lease->dev = dev;
  lease->ctx = h;
  return NATSL_OK;
}

// ------------------------------------------------------------ validation ----
natsl_status check_dims(const natsl_dims* d, bool need_L, bool need_dmodel) {
  if (!d) return fail(NATSL_ERR_INVALID_ARG, "dims is NULL");
  if (d->B < 0 || d->H < 1) return fail(NATSL_ERR_INVALID_ARG, "bad B=%d / H=%d", d->B, d->H);
  if (d->io != NATSL_F32 && d->io != NATSL_BF16) return fail(NATSL_ERR_INVALID_ARG, "bad io dtype %d", (int)d->io);
  if (d->chunk != 64) return fail(NATSL_ERR_UNSUPPORTED, "chunk must be 64 (got %d)", d->chunk);
  if (d->Dk != d->Dv) return fail(NATSL_ERR_UNSUPPORTED, "Dk (%d) != Dv (%d)", d->Dk, d->Dv);
  if (d->Dk != 64 && d->Dk != 128) return fail(NATSL_ERR_UNSUPPORTED, "head dim %d not in {64, 128}", d->Dk);
  if (d->H > 1024) return fail(NATSL_ERR_UNSUPPORTED, "H=%d above 1024", d->H);
  if (d->route_groups != 1 && d->route_groups != d->H)
    return fail(NATSL_ERR_UNSUPPORTED, "route_groups %d not in {1, H=%d}", d->route_groups, d->H);
  if (need_L) {
    if (d->L < 64 || d->L % 64 != 0) return fail(NATSL_ERR_UNSUPPORTED, "L=%d must be a positive multiple of 64", d->L);
    // keeps every launch's work-item count (e.g. one 256-lane workgroup per
    // chunk-head, 1024 lanes per chunk in the router) below 2^32
    if ((int64_t)d->B * d->H * d->L > ((int64_t)1 << 28))
      return fail(NATSL_ERR_UNSUPPORTED, "B*H*L = %lld above 2^28", (long long)d->B * d->H * d->L);
  }
  if (need_dmodel) {
    // the router keeps the chunk mean (d_model floats) and 2G scores in LDS
    if (d->d_model < 8 || d->d_model % 8 != 0 || d->d_model > 32768)
      return fail(NATSL_ERR_UNSUPPORTED, "d_model=%d must be a multiple of 8 in [8, 32768]", d->d_model);
  }
  return NATSL_OK;
}
#define NEED(p, name) \
  if (!(p)) return fail(NATSL_ERR_INVALID_ARG, "%s is NULL", name)
#define CHECK(x)                                \
  do {                                          \
    natsl_status _s = (x);                      \
    if (_s != NATSL_OK) return _s;              \
  } while (0)

float eff_scale(const natsl_dims* d) { return d->sm_scale > 0.f ? d->sm_scale : 1.0f / sqrtf((float)d->Dk); }
float eff_eps(const natsl_dims* d) { return d->rms_eps > 0.f ? d->rms_eps : 1e-6f; }
int nchunks(const natsl_dims* d) { return d->L / 64; }

struct FwdWs {
  int32_t *route, *sel, *nsb;
  void *o_sm, *o_gdn, *gdn;
  float* mixd;  // per token z0 - z1 of the mixing scores (softmax branch -> merge)
};
size_t fwd_ws(const natsl_dims* d, natsl_dtype branch, FwdWs* w, void* base) {
  const int64_t nc = nchunks(d), BG = (int64_t)d->B * d->route_groups;
  const size_t bsz = (size_t)d->B * d->H * d->L * d->Dv * (branch == NATSL_BF16 ? 2 : 4);
  size_t off = 0;
  auto take = [&](size_t n) {
    size_t o = off;
    off += al256(n);
    return o;
  };
  const size_t o_r = take(BG * nc * 4), o_s = take(BG * nc * 4), o_n = take(BG * (nc + 1) * 4);
  const size_t o_sm = take(bsz), o_gd = take(bsz);
  const size_t o_gdn = take(gdn_ws_bytes(d->io == NATSL_BF16, d->Dk, (int64_t)d->B * d->H * nc));
  const size_t o_mix = take((size_t)d->B * d->H * d->L * 4);
  if (w) {
    char* p = (char*)base;
    w->route = (int32_t*)(p + o_r);
    w->sel = (int32_t*)(p + o_s);
    w->nsb = (int32_t*)(p + o_n);
    w->o_sm = p + o_sm;
    w->o_gdn = p + o_gd;
    w->gdn = p + o_gdn;
    w->mixd = (float*)(p + o_mix);
  }
  return off;
}

// the Gated DeltaNet branch's sequence-length limit (checked before any launch)
natsl_status check_gdn_len(const natsl_dims* d) {
  const int maxc = gdn_max_chunks(d->io == NATSL_BF16, d->Dk);
  if (nchunks(d) > maxc)
    return fail(NATSL_ERR_UNSUPPORTED, "L=%d: the Gated DeltaNet branch supports at most %d chunks (L <= %lld) "
                "for this io dtype and head dim", d->L, maxc, (long long)maxc * 64);
  return NATSL_OK;
}

natsl_status check_ws(void* ws, size_t have, size_t need) {
  if (need == 0) return NATSL_OK;
  if (!ws) return fail(NATSL_ERR_WORKSPACE, "workspace is NULL (need %zu bytes)", need);
  if (((uintptr_t)ws & 255) != 0) return fail(NATSL_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (have < need) return fail(NATSL_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", have, need);
  return NATSL_OK;
}

// --------------------------------------------------------------- launches ----
hipError_t do_route(const natsl_dims* d, const void* x, const float* w, const float* b,
                    const int32_t* route_in, int32_t* route_out, int32_t* sel, int32_t* nsb,
                    float* scores, hipStream_t st) {
  const int nc = nchunks(d), G = d->route_groups;
  auto prof = prof_fn();
  hipError_t e = hipSuccess;
  const int32_t* rsrc = route_in;
  if (!route_in) {
    if (prof) prof(KID_ROUTE, st, 0);
    if (d->io == NATSL_BF16)
      e = launch_route<bf16>((const bf16*)x, w, b, d->B, d->L, d->d_model, G, route_out, scores, st);
    else
      e = launch_route<float>((const float*)x, w, b, d->B, d->L, d->d_model, G, route_out, scores, st);
    if (e != hipSuccess) return e;
    if (prof) prof(KID_ROUTE, st, 1);
    rsrc = route_out;
  }
  if (prof) prof(KID_COMPACT, st, 0);
  e = launch_compact(rsrc, route_out, d->B, G, nc, sel, nsb, st);
  if (e != hipSuccess) return e;
  if (prof) prof(KID_COMPACT, st, 1);
  return hipSuccess;
}

template <typename T, typename To>
hipError_t do_softmax_t(const natsl_dims* d, const void* q, const void* k, const void* v,
                        const int32_t* sel, const int32_t* nsb, void* o, float* lse, hipStream_t st,
                        const SmPrefix& pre, const SmMix& mix) {
  if (d->Dk == 64)
    return launch_softmax_masked<T, To, 64>((const T*)q, (const T*)k, (const T*)v, sel, nsb, (To*)o, lse,
                                            d->B, d->H, d->L, d->route_groups, eff_scale(d), st, pre, mix);
  return launch_softmax_masked<T, To, 128>((const T*)q, (const T*)k, (const T*)v, sel, nsb, (To*)o, lse,
                                           d->B, d->H, d->L, d->route_groups, eff_scale(d), st, pre, mix);
}
hipError_t do_softmax(const natsl_dims* d, const void* q, const void* k, const void* v, const int32_t* sel,
                      const int32_t* nsb, void* o, natsl_dtype od, float* lse, hipStream_t st,
                      const SmPrefix& pre = SmPrefix(), const SmMix& mix = SmMix()) {
  auto prof = prof_fn();
  if (prof) prof(KID_SOFTMAX, st, 0);
  hipError_t e;
  if (d->io == NATSL_BF16)
    e = od == NATSL_BF16 ? do_softmax_t<bf16, bf16>(d, q, k, v, sel, nsb, o, lse, st, pre, mix)
                         : do_softmax_t<bf16, float>(d, q, k, v, sel, nsb, o, lse, st, pre, mix);
  else
    e = od == NATSL_BF16 ? do_softmax_t<float, bf16>(d, q, k, v, sel, nsb, o, lse, st, pre, mix)
                         : do_softmax_t<float, float>(d, q, k, v, sel, nsb, o, lse, st, pre, mix);
  if (e == hipSuccess && prof) prof(KID_SOFTMAX, st, 1);
  return e;
}

// The chunk prep runs on st_prep; the scan runs on st_scan (after an event
// wait when the two differ).
template <typename T, typename To>
hipError_t do_gdn_t(const natsl_dims* d, const void* q, const void* k, const void* v, const float* a,
                    const float* b, const int32_t* route, const float* S0, void* o, float* Sf, void* ws,
                    hipStream_t st_prep, hipStream_t st_scan, hipEvent_t ev, hipEvent_t dep) {
  if (d->Dk == 64)
    return launch_gdn<T, To, 64>((const T*)q, (const T*)k, (const T*)v, a, b, route, S0, (To*)o, Sf, ws,
                                 d->B, d->H, d->L, d->route_groups, st_prep, st_scan, ev, dep, prof_fn());
  return launch_gdn<T, To, 128>((const T*)q, (const T*)k, (const T*)v, a, b, route, S0, (To*)o, Sf, ws,
                                d->B, d->H, d->L, d->route_groups, st_prep, st_scan, ev, dep, prof_fn());
}
// st_prep / st_scan: streams of the chunk prep and of the scan (an event orders
// them when they differ); dep: an event the scan waits for (the routes), or null
hipError_t do_gdn(const natsl_dims* d, const void* q, const void* k, const void* v, const float* a,
                  const float* b, const int32_t* route, const float* S0, void* o, natsl_dtype od, float* Sf,
                  void* ws, hipStream_t st_prep, hipStream_t st_scan = nullptr, hipEvent_t ev = nullptr,
                  hipEvent_t dep = nullptr) {
  if (!st_scan) st_scan = st_prep;
  if (d->io == NATSL_BF16)
    return od == NATSL_BF16 ? do_gdn_t<bf16, bf16>(d, q, k, v, a, b, route, S0, o, Sf, ws, st_prep, st_scan, ev, dep)
                            : do_gdn_t<bf16, float>(d, q, k, v, a, b, route, S0, o, Sf, ws, st_prep, st_scan, ev, dep);
  return od == NATSL_BF16 ? do_gdn_t<float, bf16>(d, q, k, v, a, b, route, S0, o, Sf, ws, st_prep, st_scan, ev, dep)
                          : do_gdn_t<float, float>(d, q, k, v, a, b, route, S0, o, Sf, ws, st_prep, st_scan, ev, dep);
}

template <typename Tq, typename Tb>
hipError_t do_merge_t(const natsl_dims* d, const void* q, const void* osm, const void* ogd, const float* wm,
                      int64_t hs, const float* gs, const float* gl, void* out, hipStream_t st, const float* mixd) {
  if (d->Dk == 64)
    return launch_merge<Tq, Tb, 64>((const Tq*)q, (const Tb*)osm, (const Tb*)ogd, wm, hs, gs, gl, (Tq*)out,
                                    d->B, d->H, d->L, eff_eps(d), st, mixd);
  return launch_merge<Tq, Tb, 128>((const Tq*)q, (const Tb*)osm, (const Tb*)ogd, wm, hs, gs, gl, (Tq*)out,
                                   d->B, d->H, d->L, eff_eps(d), st, mixd);
}
template <typename Tq, typename Tb>
hipError_t do_merge_bwd_t(const natsl_dims* d, const void* q, const void* osm, const void* ogd, const float* wm,
                          int64_t hs, const float* gs, const float* gl, const float* d_out, float* d_sm, float* d_gdn,
                          float* dq, float* dwm, float* dgs, float* dgl, void* ws, hipStream_t st) {
  if (d->Dk == 64)
    return launch_merge_backward<Tq, Tb, 64>((const Tq*)q, (const Tb*)osm, (const Tb*)ogd, wm, hs, gs, gl, d_out, d_sm,
                                             d_gdn, dq, dwm, dgs, dgl, ws, d->B, d->H, d->L, eff_eps(d), st);
  return launch_merge_backward<Tq, Tb, 128>((const Tq*)q, (const Tb*)osm, (const Tb*)ogd, wm, hs, gs, gl, d_out, d_sm,
                                            d_gdn, dq, dwm, dgs, dgl, ws, d->B, d->H, d->L, eff_eps(d), st);
}

// mixd (nullable): the mixing scores' difference per token, from the softmax branch
hipError_t do_merge(const natsl_dims* d, const void* q, const void* osm, const void* ogd, natsl_dtype bd,
                    const float* wm, int64_t hs, const float* gs, const float* gl, void* out, hipStream_t st,
                    const float* mixd = nullptr) {
  auto prof = prof_fn();
  if (prof) prof(KID_MERGE, st, 0);
  hipError_t e;
  if (d->io == NATSL_BF16)
    e = bd == NATSL_BF16 ? do_merge_t<bf16, bf16>(d, q, osm, ogd, wm, hs, gs, gl, out, st, mixd)
                         : do_merge_t<bf16, float>(d, q, osm, ogd, wm, hs, gs, gl, out, st, mixd);
  else
    e = bd == NATSL_BF16 ? do_merge_t<float, bf16>(d, q, osm, ogd, wm, hs, gs, gl, out, st, mixd)
                         : do_merge_t<float, float>(d, q, osm, ogd, wm, hs, gs, gl, out, st, mixd);
  if (e == hipSuccess && prof) prof(KID_MERGE, st, 1);
  return e;
}

}  // namespace

extern "C" {

int natsl_version(void) { return 100; }

const char* natsl_last_error(void) { return g_err.c_str(); }

natsl_status natsl_workspace_size(int entry, const natsl_dims* dims, size_t* bytes) {
  if (!bytes) return fail(NATSL_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = 0;
  switch (entry) {
    case NATSL_ENTRY_ROUTE:
    case NATSL_ENTRY_SOFTMAX_MASKED:
    case NATSL_ENTRY_MERGE:
      CHECK(check_dims(dims, true, false));
      return ok();
    case NATSL_ENTRY_GDN_CHUNK:
      CHECK(check_dims(dims, true, false));
      CHECK(check_gdn_len(dims));
      *bytes = gdn_ws_bytes(dims->io == NATSL_BF16, dims->Dk, (int64_t)dims->B * dims->H * nchunks(dims));
      return ok();
    case NATSL_ENTRY_FORWARD:
      CHECK(check_dims(dims, true, false));
      CHECK(check_gdn_len(dims));
      *bytes = fwd_ws(dims, NATSL_F32, nullptr, nullptr);  // fp32 branches: the larger of the two
      return ok();
    case NATSL_ENTRY_DECODE_STEP:
      CHECK(check_dims(dims, false, false));
      if (dims->L < 1) return fail(NATSL_ERR_INVALID_ARG, "decode: dims->L must hold the cache capacity");
      if (const char* why = decode_dims_problem(dims->B, dims->H, dims->L))
        return fail(NATSL_ERR_UNSUPPORTED, "decode: %s", why);
      *bytes = decode_ws_bytes(dims->B, dims->H, dims->route_groups, dims->Dk, dims->L);
      return ok();
    case NATSL_ENTRY_SOFTMAX_BACKWARD:
      CHECK(check_dims(dims, true, false));
      *bytes = sm_bwd_ws_bytes(dims->B, dims->H, dims->L);
      return ok();
    case NATSL_ENTRY_DECODE_HANDOFF:
      CHECK(check_dims(dims, true, false));
      *bytes = handoff_ws_bytes(dims->B, dims->route_groups, nchunks(dims));
      return ok();
    case NATSL_ENTRY_GDN_BACKWARD:
    case NATSL_ENTRY_GDN_BACKWARD_OVERLAP:
      CHECK(check_dims(dims, true, false));
      CHECK(check_gdn_len(dims));
      *bytes = gdn_bwd_ws_bytes(dims->io == NATSL_BF16, dims->B, dims->H, dims->L, dims->Dk,
                                entry == NATSL_ENTRY_GDN_BACKWARD_OVERLAP);
      return ok();
    case NATSL_ENTRY_MERGE_BACKWARD:
      CHECK(check_dims(dims, true, false));
      *bytes = merge_bwd_ws_bytes(dims->B, dims->H, dims->L, dims->Dk);
      return ok();
    case NATSL_ENTRY_ROUTE_BACKWARD:
      CHECK(check_dims(dims, true, true));
      *bytes = route_bwd_ws_bytes(dims->B, dims->route_groups, dims->L, dims->d_model);
      return ok();
    default:
      return fail(NATSL_ERR_INVALID_ARG, "unknown entry id %d", entry);
  }
}

natsl_status natsl_route(const natsl_dims* dims, const void* x, const float* w_score, const float* b_score,
                         const int32_t* route_in, int32_t* route_out, int32_t* sel_idx, int32_t* nsel_before,
                         float* scores, hipStream_t stream) {
  CHECK(check_dims(dims, true, route_in == nullptr));
  if (dims->B == 0) return ok();  // empty batch: nothing to do, pointers may be NULL
  if (!route_in) {
    NEED(x, "x");
    NEED(w_score, "w_score");
  }
  NEED(route_out, "route_out");
  NEED(sel_idx, "sel_idx");
  NEED(nsel_before, "nsel_before");
  hipError_t e = do_route(dims, x, w_score, b_score, route_in, route_out, sel_idx, nsel_before, scores, stream);
  if (e != hipSuccess) return dev_fail(e, "natsl_route");
  return done(stream, "natsl_route");
}

natsl_status natsl_gdn_chunk(const natsl_dims* dims, const void* q, const void* k, const void* v,
                             const float* alpha, const float* beta, const int32_t* route, const float* S_init,
                             void* o_gdn, natsl_dtype o_dtype, float* S_final, void* ws, size_t ws_bytes,
                             hipStream_t stream) {
  CHECK(check_dims(dims, true, false));
  if (dims->B == 0) return ok();  // empty batch: nothing to do, pointers may be NULL
  NEED(q, "q");
  NEED(k, "k");
  NEED(v, "v");
  NEED(alpha, "alpha");
  NEED(beta, "beta");
  NEED(route, "route");
  NEED(o_gdn, "o_gdn");
  if (o_dtype != NATSL_F32 && o_dtype != NATSL_BF16) return fail(NATSL_ERR_INVALID_ARG, "bad o_dtype");
  CHECK(check_gdn_len(dims));
  const size_t need = gdn_ws_bytes(dims->io == NATSL_BF16, dims->Dk, (int64_t)dims->B * dims->H * nchunks(dims));
  CHECK(check_ws(ws, ws_bytes, need));
  hipError_t e = do_gdn(dims, q, k, v, alpha, beta, route, S_init, o_gdn, o_dtype, S_final, ws, stream);
  if (e != hipSuccess) return dev_fail(e, "natsl_gdn_chunk");
  return done(stream, "natsl_gdn_chunk");
}

natsl_status natsl_softmax_masked(const natsl_dims* dims, const void* q, const void* k, const void* v,
                                  const int32_t* sel_idx, const int32_t* nsel_before, void* o_sm,
                                  natsl_dtype o_dtype, float* lse, void* ws, size_t ws_bytes, hipStream_t stream) {
  (void)ws;
  (void)ws_bytes;
  CHECK(check_dims(dims, true, false));
  if (dims->B == 0) return ok();  // empty batch: nothing to do, pointers may be NULL
  NEED(q, "q");
  NEED(k, "k");
  NEED(v, "v");
  NEED(sel_idx, "sel_idx");
  NEED(nsel_before, "nsel_before");
  NEED(o_sm, "o_sm");
  if (o_dtype != NATSL_F32 && o_dtype != NATSL_BF16) return fail(NATSL_ERR_INVALID_ARG, "bad o_dtype");
  hipError_t e = do_softmax(dims, q, k, v, sel_idx, nsel_before, o_sm, o_dtype, lse, stream);
  if (e != hipSuccess) return dev_fail(e, "natsl_softmax_masked");
  return done(stream, "natsl_softmax_masked");
}

natsl_status natsl_merge(const natsl_dims* dims, const void* q, const void* o_sm, const void* o_gdn,
                         natsl_dtype branch_dtype, const float* w_mix, int64_t w_mix_head_stride,
                         const float* g_sm, const float* g_lin, void* out, hipStream_t stream) {
  CHECK(check_dims(dims, true, false));
  if (dims->B == 0) return ok();  // empty batch: nothing to do, pointers may be NULL
  NEED(q, "q");
  NEED(o_sm, "o_sm");
  NEED(o_gdn, "o_gdn");
  NEED(w_mix, "w_mix");
  NEED(out, "out");
  if (branch_dtype != NATSL_F32 && branch_dtype != NATSL_BF16) return fail(NATSL_ERR_INVALID_ARG, "bad branch dtype");
  if (w_mix_head_stride < 0) return fail(NATSL_ERR_INVALID_ARG, "negative w_mix head stride");
  hipError_t e = do_merge(dims, q, o_sm, o_gdn, branch_dtype, w_mix, w_mix_head_stride, g_sm, g_lin, out, stream);
  if (e != hipSuccess) return dev_fail(e, "natsl_merge");
  return done(stream, "natsl_merge");
}

natsl_status natsl_forward(const natsl_dims* dims, const natsl_forward_args* a, void* ws, size_t ws_bytes,
                           hipStream_t stream) {
  CHECK(check_dims(dims, true, a && !a->route_override));
  if (dims->B == 0) return ok();  // empty batch: nothing to do, pointers may be NULL
  NEED(a, "args");
  NEED(a->q, "q");
  NEED(a->k, "k");
  NEED(a->v, "v");
  NEED(a->alpha, "alpha");
  NEED(a->beta, "beta");
  NEED(a->w_mix, "w_mix");
  NEED(a->out, "out");
  if (!a->route_override) {
    NEED(a->x, "x");
    NEED(a->w_score, "w_score");
  }
  if (a->branch_dtype != NATSL_F32 && a->branch_dtype != NATSL_BF16)
    return fail(NATSL_ERR_INVALID_ARG, "bad branch dtype");
  if (a->w_mix_head_stride < 0) return fail(NATSL_ERR_INVALID_ARG, "negative w_mix head stride");
  CHECK(check_gdn_len(dims));
  // chunked prefill: the segment continues a decode cache at a chunk boundary
  SmPrefix pre;
  const float* S_init = a->S_init;
  if (a->prefix) {
    const natsl_decode_cache* c = a->prefix;
    NEED(c->k_cache, "prefix k_cache");
    NEED(c->v_cache, "prefix v_cache");
    NEED(c->n_committed, "prefix n_committed");
    NEED(c->S_carry, "prefix S_carry");
    if (a->S_init) return fail(NATSL_ERR_INVALID_ARG, "S_init and prefix are exclusive (the prefix's S_carry is used)");
    if (c->cap < 0) return fail(NATSL_ERR_INVALID_ARG, "prefix capacity %d", c->cap);
    pre.k = c->k_cache;
    pre.v = c->v_cache;
    pre.n_committed = c->n_committed;
    pre.cap = c->cap;
    S_init = c->S_carry;
  }
  FwdWs w;
  const size_t need = fwd_ws(dims, a->branch_dtype, nullptr, nullptr);
  CHECK(check_ws(ws, ws_bytes, need));
  fwd_ws(dims, a->branch_dtype, &w, ws);
  HelperPool<Helper>::Lease lease;
  CHECK(acquire_helper(&lease));
  Helper* ctx = lease.ctx;
  int32_t* route = a->route_out ? a->route_out : w.route;
  void* o_sm = a->o_sm_dbg ? a->o_sm_dbg : w.o_sm;
  void* o_gd = a->o_gdn_dbg ? a->o_gdn_dbg : w.o_gdn;
  // Fork: the helper stream waits for the caller's stream (inputs ready) and
  // runs the chunk prep, which does not depend on the routes, while the caller's
  // stream routes; the scan then waits for the routes.  The softmax branch runs
  // on the caller's stream meanwhile; the merge waits for both.
  hipError_t e;
  if ((e = hipEventRecord(ctx->fork, stream)) != hipSuccess) return dev_fail(e, "hipEventRecord");
  if ((e = hipStreamWaitEvent(ctx->aux, ctx->fork, 0)) != hipSuccess) return dev_fail(e, "hipStreamWaitEvent");
  // from here on, a failure still joins the helper stream back into the
  // caller's stream (best effort), so that nothing the call queued can outlive
  // what the caller orders after it
  auto fail_joined = [&](hipError_t err, const char* where) {
    if (hipEventRecord(ctx->join, ctx->aux) == hipSuccess) (void)hipStreamWaitEvent(stream, ctx->join, 0);
    return dev_fail(err, where);
  };
  e = do_route(dims, a->x, a->w_score, a->b_score, a->route_override, route, w.sel, w.nsb, a->scores_out, stream);
  if (e != hipSuccess) return fail_joined(e, "natsl_forward/route");
  if ((e = hipEventRecord(ctx->routed, stream)) != hipSuccess) return fail_joined(e, "hipEventRecord");
  e = do_gdn(dims, a->q, a->k, a->v, a->alpha, a->beta, route, S_init, o_gd, a->branch_dtype, a->S_final,
             w.gdn, ctx->aux, ctx->aux, nullptr, ctx->routed);
  if (e != hipSuccess) return fail_joined(e, "natsl_forward/gdn");
  // the softmax branch also leaves the merge's mixing scores (bf16 D = 128 kernel)
  bool mix_done = false;
  SmMix mix;
  mix.w_mix = a->w_mix;
  mix.hs = a->w_mix_head_stride;
  mix.d = w.mixd;
  mix.done = &mix_done;
  e = do_softmax(dims, a->q, a->k, a->v, w.sel, w.nsb, o_sm, a->branch_dtype, nullptr, stream, pre, mix);
  if (e != hipSuccess) return fail_joined(e, "natsl_forward/softmax");
  if ((e = hipEventRecord(ctx->join, ctx->aux)) != hipSuccess) return dev_fail(e, "hipEventRecord");
  if ((e = hipStreamWaitEvent(stream, ctx->join, 0)) != hipSuccess) return dev_fail(e, "hipStreamWaitEvent");
  e = do_merge(dims, a->q, o_sm, o_gd, a->branch_dtype, a->w_mix, a->w_mix_head_stride, a->g_sm, a->g_lin, a->out,
               stream, mix_done ? w.mixd : nullptr);
  if (e != hipSuccess) return dev_fail(e, "natsl_forward/merge");
  return done(stream, "natsl_forward");
}

namespace {
// Validation and launch of a decode step whose scratch is `ws` (ws_bytes
// available; checked before anything is enqueued).  noalloc: ws is null and
// the device's static scratch array is used instead.
natsl_status decode_step_impl(const natsl_dims* dims, const natsl_decode_cache* c, const natsl_decode_args* a,
                              void* ws, size_t ws_bytes, bool noalloc, hipStream_t stream) {
  CHECK(check_dims(dims, false, true));
  if (dims->B == 0) return ok();  // empty batch: nothing to do, pointers may be NULL
  NEED(c, "cache");
  NEED(a, "args");
  NEED(c->k_cache, "k_cache");
  NEED(c->v_cache, "v_cache");
  NEED(c->n_committed, "n_committed");
  NEED(c->n_open, "n_open");
  NEED(c->S_carry, "S_carry");
  NEED(c->S_work, "S_work");
  NEED(c->x_sum, "x_sum");
  NEED(c->err_flag, "err_flag");
  if (c->cap < 1) return fail(NATSL_ERR_INVALID_ARG, "cache capacity %d", c->cap);
  if (const char* why = decode_dims_problem(dims->B, dims->H, c->cap)) return fail(NATSL_ERR_UNSUPPORTED, "decode: %s", why);
  NEED(a->x, "x");
  NEED(a->q, "q");
  NEED(a->k, "k");
  NEED(a->v, "v");
  NEED(a->alpha, "alpha");
  NEED(a->beta, "beta");
  NEED(a->w_score, "w_score");
  NEED(a->w_mix, "w_mix");
  NEED(a->out, "out");
  if (a->w_mix_head_stride < 0) return fail(NATSL_ERR_INVALID_ARG, "negative w_mix head stride");
  const size_t need = decode_ws_bytes(dims->B, dims->H, dims->route_groups, dims->Dk, c->cap);
  if (noalloc) {
    if (need > DECODE_SCRATCH_BYTES)
      return fail(NATSL_ERR_WORKSPACE, "natsl_decode_step_noalloc: these dims need %zu bytes of scratch, above the "
                  "%zu the allocation-free entry point holds per device (use natsl_decode_step with a workspace)",
                  need, (size_t)DECODE_SCRATCH_BYTES);
    const hipError_t e = decode_scratch_address(&ws);
    if (e != hipSuccess) return dev_fail(e, "natsl_decode_step_noalloc: scratch address");
  } else {
    CHECK(check_ws(ws, ws_bytes, need));
  }
  DecodeLaunch L;
  L.B = dims->B;
  L.H = dims->H;
  L.G = dims->route_groups;
  L.d = dims->d_model;
  L.cap = c->cap;
  L.scale = eff_scale(dims);
  L.eps = eff_eps(dims);
  L.x = a->x;
  L.q = a->q;
  L.k = a->k;
  L.v = a->v;
  L.alpha = a->alpha;
  L.beta = a->beta;
  L.w_score = a->w_score;
  L.b_score = a->b_score;
  L.w_mix = a->w_mix;
  L.w_mix_hs = a->w_mix_head_stride;
  L.g_sm = a->g_sm;
  L.g_lin = a->g_lin;
  L.k_cache = c->k_cache;
  L.v_cache = c->v_cache;
  L.n_committed = c->n_committed;
  L.n_open = c->n_open;
  L.err_flag = c->err_flag;
  L.route_out = a->route_out;
  L.S_carry = c->S_carry;
  L.S_work = c->S_work;
  L.x_sum = c->x_sum;
  L.out = a->out;
  L.o_sm_dbg = a->o_sm_dbg;
  L.o_gdn_dbg = a->o_gdn_dbg;
  hipError_t e;
  auto prof = prof_fn();
  if (dims->io == NATSL_BF16)
    e = dims->Dk == 64 ? launch_decode<bf16, 64>(L, ws, stream, prof) : launch_decode<bf16, 128>(L, ws, stream, prof);
  else
    e = dims->Dk == 64 ? launch_decode<float, 64>(L, ws, stream, prof) : launch_decode<float, 128>(L, ws, stream, prof);
  if (e != hipSuccess) return dev_fail(e, noalloc ? "natsl_decode_step_noalloc" : "natsl_decode_step");
  return done(stream, noalloc ? "natsl_decode_step_noalloc" : "natsl_decode_step");
}
}  // namespace

natsl_status natsl_decode_step(const natsl_dims* dims, const natsl_decode_cache* c, const natsl_decode_args* a,
                               void* ws, size_t ws_bytes, hipStream_t stream) {
  return decode_step_impl(dims, c, a, ws, ws_bytes, false, stream);
}

natsl_status natsl_decode_step_noalloc(const natsl_dims* dims, const natsl_decode_cache* c,
                                       const natsl_decode_args* a, hipStream_t stream) {
  return decode_step_impl(dims, c, a, nullptr, 0, true, stream);
}

natsl_status natsl_softmax_masked_backward(const natsl_dims* dims, const void* q, const void* k, const void* v,
                                           const int32_t* sel_idx, const int32_t* nsel_before, const void* o_sm,
                                           const float* lse, const void* d_o, float* dq, float* dk, float* dv,
                                           float* dgate, void* ws, size_t ws_bytes, hipStream_t stream) {
  CHECK(check_dims(dims, true, false));
  if (dims->B == 0) return ok();  // empty batch: nothing to do, pointers may be NULL
  NEED(q, "q");
  NEED(k, "k");
  NEED(v, "v");
  NEED(sel_idx, "sel_idx");
  NEED(nsel_before, "nsel_before");
  NEED(o_sm, "o_sm");
  NEED(lse, "lse");
  NEED(d_o, "d_o");
  NEED(dq, "dq");
  NEED(dk, "dk");
  NEED(dv, "dv");
  CHECK(check_ws(ws, ws_bytes, sm_bwd_ws_bytes(dims->B, dims->H, dims->L)));
  const float sc = eff_scale(dims);
  const int B = dims->B, H = dims->H, L = dims->L, G = dims->route_groups;
  hipError_t e;
  auto prof = prof_fn();
  if (prof) prof(KID_SOFTMAX_BWD, stream, 0);
  if (dims->io == NATSL_BF16)
    e = dims->Dk == 64
            ? launch_softmax_backward<bf16, bf16, 64>((const bf16*)q, (const bf16*)k, (const bf16*)v, sel_idx,
                                                      nsel_before, (const bf16*)o_sm, lse, (const bf16*)d_o, dq, dk,
                                                      dv, dgate, ws, B, H, L, G, sc, stream)
            : launch_softmax_backward<bf16, bf16, 128>((const bf16*)q, (const bf16*)k, (const bf16*)v, sel_idx,
                                                       nsel_before, (const bf16*)o_sm, lse, (const bf16*)d_o, dq, dk,
                                                       dv, dgate, ws, B, H, L, G, sc, stream);
  else
    e = dims->Dk == 64
            ? launch_softmax_backward<float, float, 64>((const float*)q, (const float*)k, (const float*)v, sel_idx,
                                                        nsel_before, (const float*)o_sm, lse, (const float*)d_o, dq,
                                                        dk, dv, dgate, ws, B, H, L, G, sc, stream)
            : launch_softmax_backward<float, float, 128>((const float*)q, (const float*)k, (const float*)v, sel_idx,
                                                         nsel_before, (const float*)o_sm, lse, (const float*)d_o, dq,
                                                         dk, dv, dgate, ws, B, H, L, G, sc, stream);
  if (prof) prof(KID_SOFTMAX_BWD, stream, 1);
  if (e != hipSuccess) return dev_fail(e, "natsl_softmax_masked_backward");
  return done(stream, "natsl_softmax_masked_backward");
}

natsl_status natsl_gdn_backward(const natsl_dims* dims, const void* q, const void* k, const void* v,
                                const float* alpha, const float* beta, const int32_t* route, const float* S_init,
                                const float* d_o, const float* dS_final, float* dq, float* dk, float* dv,
                                float* dalpha, float* dbeta, float* dS_init, float* dgate, void* ws, size_t ws_bytes,
                                hipStream_t stream) {
  CHECK(check_dims(dims, true, false));
  if (dims->B == 0) return ok();  // empty batch: nothing to do, pointers may be NULL
  NEED(q, "q");
  NEED(k, "k");
  NEED(v, "v");
  NEED(alpha, "alpha");
  NEED(beta, "beta");
  NEED(route, "route");
  NEED(d_o, "d_o");
  NEED(dq, "dq");
  NEED(dk, "dk");
  NEED(dv, "dv");
  NEED(dalpha, "dalpha");
  NEED(dbeta, "dbeta");
  CHECK(check_gdn_len(dims));
  const bool bf = dims->io == NATSL_BF16;
  CHECK(check_ws(ws, ws_bytes, gdn_bwd_ws_bytes(bf, dims->B, dims->H, dims->L, dims->Dk, false)));
  // a workspace of the overlap layout's size: the two sweeps on two streams
  SideStream ov;
  HelperPool<Helper>::Lease lease;
  if (ws_bytes >= gdn_bwd_ws_bytes(bf, dims->B, dims->H, dims->L, dims->Dk, true)) {
    CHECK(acquire_helper(&lease));
    ov.aux = lease.ctx->aux;
    ov.fork = lease.ctx->fork;
    ov.join = lease.ctx->join;
  }
  const int B = dims->B, H = dims->H, L = dims->L, G = dims->route_groups;
  hipError_t e;
  auto prof = prof_fn();
  if (prof) prof(KID_GDN_BWD, stream, 0);
  if (dims->io == NATSL_BF16)
    e = dims->Dk == 64 ? launch_gdn_backward<bf16, 64>((const bf16*)q, (const bf16*)k, (const bf16*)v, alpha, beta,
                                                       route, S_init, d_o, dS_final, dq, dk, dv, dalpha, dbeta,
                                                       dS_init, dgate, ws, B, H, L, G, stream, ov)
                       : launch_gdn_backward<bf16, 128>((const bf16*)q, (const bf16*)k, (const bf16*)v, alpha, beta,
                                                        route, S_init, d_o, dS_final, dq, dk, dv, dalpha, dbeta,
                                                        dS_init, dgate, ws, B, H, L, G, stream, ov);
  else
    e = dims->Dk == 64 ? launch_gdn_backward<float, 64>((const float*)q, (const float*)k, (const float*)v, alpha,
                                                        beta, route, S_init, d_o, dS_final, dq, dk, dv, dalpha,
                                                        dbeta, dS_init, dgate, ws, B, H, L, G, stream, ov)
                       : launch_gdn_backward<float, 128>((const float*)q, (const float*)k, (const float*)v, alpha,
                                                         beta, route, S_init, d_o, dS_final, dq, dk, dv, dalpha,
                                                         dbeta, dS_init, dgate, ws, B, H, L, G, stream, ov);
  if (prof) prof(KID_GDN_BWD, stream, 1);
  if (e != hipSuccess) return dev_fail(e, "natsl_gdn_backward");
  return done(stream, "natsl_gdn_backward");
}

natsl_status natsl_merge_backward(const natsl_dims* dims, const void* q, const void* o_sm, const void* o_gdn,
                                  natsl_dtype branch_dtype, const float* w_mix, int64_t w_mix_head_stride,
                                  const float* g_sm, const float* g_lin, const float* d_out, float* d_o_sm,
                                  float* d_o_gdn, float* dq, float* dw_mix, float* dg_sm, float* dg_lin, void* ws,
                                  size_t ws_bytes, hipStream_t stream) {
  CHECK(check_dims(dims, true, false));
  if (dims->B == 0) return ok();  // empty batch: nothing to do, pointers may be NULL
  NEED(q, "q");
  NEED(o_sm, "o_sm");
  NEED(o_gdn, "o_gdn");
  NEED(w_mix, "w_mix");
  NEED(d_out, "d_out");
  NEED(d_o_sm, "d_o_sm");
  NEED(d_o_gdn, "d_o_gdn");
  NEED(dq, "dq");
  if (branch_dtype != NATSL_F32 && branch_dtype != NATSL_BF16) return fail(NATSL_ERR_INVALID_ARG, "bad branch dtype");
  if (w_mix_head_stride != 0 && w_mix_head_stride != 2 * dims->Dk)
    return fail(NATSL_ERR_INVALID_ARG, "w_mix head stride must be 0 or 2 Dk (got %lld)", (long long)w_mix_head_stride);
  CHECK(check_ws(ws, ws_bytes, merge_bwd_ws_bytes(dims->B, dims->H, dims->L, dims->Dk)));
  auto prof = prof_fn();
  if (prof) prof(KID_MERGE_BWD, stream, 0);
  hipError_t e;
  const int64_t hs = w_mix_head_stride;
  if (dims->io == NATSL_BF16)
    e = branch_dtype == NATSL_BF16
            ? do_merge_bwd_t<bf16, bf16>(dims, q, o_sm, o_gdn, w_mix, hs, g_sm, g_lin, d_out, d_o_sm, d_o_gdn, dq,
                                         dw_mix, dg_sm, dg_lin, ws, stream)
            : do_merge_bwd_t<bf16, float>(dims, q, o_sm, o_gdn, w_mix, hs, g_sm, g_lin, d_out, d_o_sm, d_o_gdn, dq,
                                          dw_mix, dg_sm, dg_lin, ws, stream);
  else
    e = branch_dtype == NATSL_BF16
            ? do_merge_bwd_t<float, bf16>(dims, q, o_sm, o_gdn, w_mix, hs, g_sm, g_lin, d_out, d_o_sm, d_o_gdn, dq,
                                          dw_mix, dg_sm, dg_lin, ws, stream)
            : do_merge_bwd_t<float, float>(dims, q, o_sm, o_gdn, w_mix, hs, g_sm, g_lin, d_out, d_o_sm, d_o_gdn, dq,
                                           dw_mix, dg_sm, dg_lin, ws, stream);
  if (prof) prof(KID_MERGE_BWD, stream, 1);
  if (e != hipSuccess) return dev_fail(e, "natsl_merge_backward");
  return done(stream, "natsl_merge_backward");
}

natsl_status natsl_decode_handoff(const natsl_dims* dims, const int32_t* route, const void* k, const void* v,
                                  const float* S_final, int append, const natsl_decode_cache* c, void* ws,
                                  size_t ws_bytes, hipStream_t stream) {
  CHECK(check_dims(dims, true, true));
  if (dims->B == 0) return ok();  // empty batch: nothing to do, pointers may be NULL
  NEED(route, "route");
  NEED(k, "k");
  NEED(v, "v");
  NEED(c, "cache");
  NEED(c->k_cache, "k_cache");
  NEED(c->v_cache, "v_cache");
  NEED(c->n_committed, "n_committed");
  NEED(c->n_open, "n_open");
  NEED(c->S_carry, "S_carry");
  NEED(c->S_work, "S_work");
  NEED(c->x_sum, "x_sum");
  NEED(c->err_flag, "err_flag");
  if (c->cap < 1) return fail(NATSL_ERR_INVALID_ARG, "cache capacity %d", c->cap);
  if (append != 0 && append != 1) return fail(NATSL_ERR_INVALID_ARG, "append must be 0 or 1 (got %d)", append);
  if (append && !S_final) return fail(NATSL_ERR_INVALID_ARG, "appending needs the segment's S_final");
  CHECK(check_ws(ws, ws_bytes, handoff_ws_bytes(dims->B, dims->route_groups, nchunks(dims))));
  HandoffLaunch L;
  L.append = append;
  L.B = dims->B;
  L.H = dims->H;
  L.G = dims->route_groups;
  L.L = dims->L;
  L.D = dims->Dk;
  L.d = dims->d_model;
  L.cap = c->cap;
  L.route = route;
  L.k = k;
  L.v = v;
  L.S_final = S_final;
  L.k_cache = c->k_cache;
  L.v_cache = c->v_cache;
  L.n_committed = c->n_committed;
  L.n_open = c->n_open;
  L.err_flag = c->err_flag;
  L.S_carry = c->S_carry;
  L.S_work = c->S_work;
  L.x_sum = c->x_sum;
  auto prof = prof_fn();
  if (prof) prof(KID_HANDOFF, stream, 0);
  const hipError_t e = dims->io == NATSL_BF16 ? launch_handoff<bf16>(L, ws, stream) : launch_handoff<float>(L, ws, stream);
  if (prof) prof(KID_HANDOFF, stream, 1);
  if (e != hipSuccess) return dev_fail(e, "natsl_decode_handoff");
  return done(stream, "natsl_decode_handoff");
}

natsl_status natsl_route_backward(const natsl_dims* dims, const void* x, const float* w_score, const float* scores,
                                  const float* dgate_sm, const float* dgate_lin, float* dx, float* dw_score,
                                  float* db_score, void* ws, size_t ws_bytes, hipStream_t stream) {
  CHECK(check_dims(dims, true, true));
  if (dims->B == 0) return ok();  // empty batch: nothing to do, pointers may be NULL
  NEED(x, "x");
  NEED(w_score, "w_score");
  NEED(scores, "scores");
  NEED(dgate_sm, "dgate_sm");
  NEED(dgate_lin, "dgate_lin");
  NEED(dw_score, "dw_score");
  CHECK(check_ws(ws, ws_bytes, route_bwd_ws_bytes(dims->B, dims->route_groups, dims->L, dims->d_model)));
  auto prof = prof_fn();
  if (prof) prof(KID_ROUTE_BWD, stream, 0);
  const hipError_t e =
      dims->io == NATSL_BF16
          ? launch_route_backward<bf16>((const bf16*)x, w_score, scores, dgate_sm, dgate_lin, dx, dw_score, db_score,
                                        ws, dims->B, dims->H, dims->L, dims->d_model, dims->route_groups, stream)
          : launch_route_backward<float>((const float*)x, w_score, scores, dgate_sm, dgate_lin, dx, dw_score,
                                         db_score, ws, dims->B, dims->H, dims->L, dims->d_model, dims->route_groups,
                                         stream);
  if (prof) prof(KID_ROUTE_BWD, stream, 1);
  if (e != hipSuccess) return dev_fail(e, "natsl_route_backward");
  return done(stream, "natsl_route_backward");
}

natsl_status natsl_nha_workspace_size(const natsl_dims* dims, int slots, int window, size_t* bytes) {
  if (!bytes) return fail(NATSL_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = 0;
  CHECK(check_dims(dims, true, false));
  if (slots != 16 && slots != 32 && slots != 64) return fail(NATSL_ERR_UNSUPPORTED, "slots %d not in {16, 32, 64}", slots);
  if (window < 0 || window % 64 != 0)
    return fail(NATSL_ERR_UNSUPPORTED, "window %d must be a non-negative multiple of 64", window);
  *bytes = nha_ws_bytes(dims->B, dims->H, dims->L, dims->Dk, slots, window);
  return ok();
}

natsl_status natsl_nha_attention(const natsl_dims* dims, const void* q, const void* k, const void* v,
                                 const float* slot_gate, int slots, int window, void* out, void* ws, size_t ws_bytes,
                                 hipStream_t stream) {
  size_t need = 0;
  CHECK(natsl_nha_workspace_size(dims, slots, window, &need));
  if (dims->B == 0) return ok();  // empty batch: nothing to do, pointers may be NULL
  NEED(q, "q");
  NEED(k, "k");
  NEED(v, "v");
  NEED(slot_gate, "slot_gate");
  NEED(out, "out");
  CHECK(check_ws(ws, ws_bytes, need));
  HelperPool<Helper>::Lease lease;
  CHECK(acquire_helper(&lease));
  SideStream side;
  side.aux = lease.ctx->aux;
  side.fork = lease.ctx->fork;
  side.join = lease.ctx->join;
  const float sc = eff_scale(dims);
  const int B = dims->B, H = dims->H, L = dims->L;
  hipError_t e;
  auto prof = prof_fn();
  if (prof) prof(KID_NHA, stream, 0);
  if (dims->io == NATSL_BF16)
    e = dims->Dk == 64 ? launch_nha<bf16, bf16, 64>((const bf16*)q, (const bf16*)k, (const bf16*)v, slot_gate, slots,
                                                    (bf16*)out, ws, B, H, L, window, sc, stream, prof, side)
                       : launch_nha<bf16, bf16, 128>((const bf16*)q, (const bf16*)k, (const bf16*)v, slot_gate,
                                                     slots, (bf16*)out, ws, B, H, L, window, sc, stream, prof, side);
  else
    e = dims->Dk == 64 ? launch_nha<float, float, 64>((const float*)q, (const float*)k, (const float*)v, slot_gate,
                                                      slots, (float*)out, ws, B, H, L, window, sc, stream, prof, side)
                       : launch_nha<float, float, 128>((const float*)q, (const float*)k, (const float*)v, slot_gate,
                                                       slots, (float*)out, ws, B, H, L, window, sc, stream, prof, side);
  if (prof) prof(KID_NHA, stream, 1);
  if (e != hipSuccess) return dev_fail(e, "natsl_nha_attention");
  return done(stream, "natsl_nha_attention");
}

natsl_status natsl_set_sync_check(int level) {
  if (level < 0 || level > 2) return fail(NATSL_ERR_INVALID_ARG, "sync check level %d (0, 1 or 2)", level);
  g_sync_level.store(level, std::memory_order_release);
  return ok();
}

int natsl_get_sync_check(void) { return sync_level(); }

natsl_status natsl_profile_enable(int on) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (on && g_prof_pool.empty()) {
    g_prof_pool.resize(8192);
    for (auto& r : g_prof_pool) {
      hipError_t e;
      if ((e = hipEventCreate(&r.a)) != hipSuccess || (e = hipEventCreate(&r.b)) != hipSuccess) {
        g_prof_pool.clear();
        return dev_fail(e, "hipEventCreate");
      }
    }
  }
  g_prof_on = on != 0;
  g_prof_used = 0;
  return ok();
}

natsl_status natsl_profile_reset(void) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof_used = 0;
  return ok();
}

natsl_status natsl_profile_select(const char* name) {
  int kid = -1;
  if (name && name[0]) {
    for (int i = 0; i < KID_COUNT; ++i)
      if (strcmp(name, kKernelNames[i]) == 0) kid = i;
    if (kid < 0) return fail(NATSL_ERR_INVALID_ARG, "unknown kernel name '%s'", name);
  }
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof_only = kid;
  return ok();
}

natsl_status natsl_profile_read(const char* name, int* count, double* total_ms) {
  NEED(name, "name");
  NEED(count, "count");
  NEED(total_ms, "total_ms");
  int kid = -1;
  for (int i = 0; i < KID_COUNT; ++i)
    if (strcmp(name, kKernelNames[i]) == 0) kid = i;
  if (kid < 0) return fail(NATSL_ERR_INVALID_ARG, "unknown kernel name '%s'", name);
  std::lock_guard<std::mutex> lk(g_prof_mu);
  int n = 0;
  double tot = 0.0;
  for (size_t i = 0; i < g_prof_used; ++i) {
    const ProfRec& r = g_prof_pool[i];
    if (r.kid != kid) continue;
    hipError_t e = hipEventSynchronize(r.b);
    if (e != hipSuccess) return dev_fail(e, "hipEventSynchronize");
    float ms = 0.f;
    e = hipEventElapsedTime(&ms, r.a, r.b);
    if (e != hipSuccess) return dev_fail(e, "hipEventElapsedTime");
    tot += ms;
    ++n;
  }
  *count = n;
  *total_ms = tot;
  return ok();
}

}  // extern "C"
