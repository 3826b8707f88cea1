// Host-side launch helpers of the NAtS-L kernels (internal to the library).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace natsl {

// a helper stream and two events (all set or none): work that does not need
// the caller's stream's other launches runs on it, forked from and joined back
// into the caller's stream (the GDN gradient: the state scan beside the
// reverse scan, the workspace laid out for it; Native Hybrid Attention: the
// window's softmax beside the slot states)
struct SideStream {
  hipStream_t aux = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};

typedef __bf16 bf16;

// kernel ids for the optional launch timing
enum {
  KID_ROUTE = 0,
  KID_COMPACT,
  KID_GDN_PREP,
  KID_GDN_SCAN,
  KID_SOFTMAX,
  KID_MERGE,
  KID_DECODE_ROUTE,
  KID_DECODE_GDN,
  KID_DECODE_ATTN,
  KID_DECODE_COMBINE,
  KID_DECODE_COMMIT,
  KID_SOFTMAX_BWD,
  KID_HANDOFF,
  KID_GDN_BWD,
  KID_MERGE_BWD,
  KID_NHA,
  KID_NHA_WINDOW,
  KID_NHA_CHUNK,
  KID_NHA_SCAN,
  KID_NHA_SLOTS,
  KID_ROUTE_BWD,
  KID_COUNT
};

// Largest dynamic LDS a workgroup may request on gfx950 (160 KiB per CU).
constexpr int LDS_MAX_BYTES = 160 * 1024;

// Raises kernel fn's dynamic LDS limit to `bytes` on the current device,
// once per (device, kernel); safe to call from several host threads.
hipError_t set_lds_limit(const void* fn, int bytes);

// Most chunks per sequence the Gated DeltaNet branch supports for this io
// dtype and head dim (the bf16 D = 128 scan keeps one route byte per chunk in
// LDS); the C ABI rejects longer sequences before launching anything.
int gdn_max_chunks(int io_is_bf16, int D);

template <typename T>
hipError_t launch_route(const T* x, const float* w, const float* bsc, int B, int L, int d, int G,
                        int32_t* route_out, float* scores, hipStream_t st);
hipError_t launch_compact(const int32_t* route_in, int32_t* route_out, int B, int G, int nc,
                          int32_t* sel_idx, int32_t* nsel_before, hipStream_t st);
// router gradient (straight-through): ws holds ds [B, G, Nc, 2] and the chunk means [B, Nc, d]
size_t route_bwd_ws_bytes(int B, int G, int L, int d);
template <typename T>
hipError_t launch_route_backward(const T* x, const float* w, const float* scores, const float* dg_sm,
                                 const float* dg_lin, float* dx, float* dw, float* db, void* ws, int B, int H, int L,
                                 int d, int G, hipStream_t st);

// mixd (nullable): per-token z0 - z1 of the mixing scores q W_mix, already
// computed (by the softmax branch); then q and w_mix are not read
template <typename Tq, typename Tb, int D>
hipError_t launch_merge(const Tq* q, const Tb* o_sm, const Tb* o_gdn, const float* w_mix, int64_t hs,
                        const float* g_sm, const float* g_lin, Tq* out, int B, int H, int L,
                        float eps, hipStream_t st, const float* mixd = nullptr);

// merge gradient: d_out fp32; ws holds per-block partial sums
size_t merge_bwd_ws_bytes(int B, int H, int L, int D);
template <typename Tq, typename Tb, int D>
hipError_t launch_merge_backward(const Tq* q, const Tb* o_sm, const Tb* o_gdn, const float* w_mix, int64_t hs,
                                 const float* g_sm, const float* g_lin, const float* d_out, float* d_sm,
                                 float* d_gdn, float* dq, float* dw_mix, float* dg_sm, float* dg_lin, void* ws,
                                 int B, int H, int L, float eps, hipStream_t st);

// cached softmax rows a prefill segment also attends to (chunked prefill):
// n_committed[b, g] rows (a multiple of 64) of k, v [B, H, cap, D]
struct SmPrefix {
  const void* k = nullptr;
  const void* v = nullptr;
  const int32_t* n_committed = nullptr;
  int cap = 0;
};
// softmax branch gradient: o and d_o in the io dtype (To == T); ws holds delta
size_t sm_bwd_ws_bytes(int B, int H, int L);
template <typename T, typename To, int D>
hipError_t launch_softmax_backward(const T* q, const T* k, const T* v, const int32_t* sel_idx,
                                   const int32_t* nsel_before, const To* o, const float* lse, const T* d_o,
                                   float* dq, float* dk, float* dv, float* dgate, void* ws, int B, int H, int L,
                                   int G, float scale, hipStream_t st);
// the merge's mixing scores from the softmax branch's own q fragments: when
// d is set and the launch uses the bf16 D = 128 kernel, d[b, h, t] =
// q W_mix[:, 0] - q W_mix[:, 1] is written and *done set (false otherwise)
struct SmMix {
  const float* w_mix = nullptr;
  int64_t hs = 0;  // head stride of w_mix in floats (0 = shared)
  float* d = nullptr;
  bool* done = nullptr;
};
template <typename T, typename To, int D>
hipError_t launch_softmax_masked(const T* q, const T* k, const T* v, const int32_t* sel_idx,
                                 const int32_t* nsel_before, To* o_sm, float* lse, int B, int H,
                                 int L, int G, float scale, hipStream_t st, const SmPrefix& pre = SmPrefix(),
                                 const SmMix& mix = SmMix());

// sliding-window causal softmax (the generic kernel's window mode): a query
// sees the win_chunks * 64 most recent tokens including itself; lse nullable
template <typename T, typename To, int D>
hipError_t launch_softmax_window(const T* q, const T* k, const T* v, To* o, float* lse, int B, int H, int L,
                                 int win_chunks, float scale, hipStream_t st);

// Native Hybrid Attention (slots + sliding window, one softmax)
struct NhaWs {
  float* Sk;  // [B, H, ne, M, D] per chunk e: its slot-key change, then the slot keys before it
  float* Sv;  // [B, H, ne, M, D] the same for the slot values
  float* G;   // [B, H, ne, M]    the chunk's decay of every slot
};
size_t nha_ws_bytes(int B, int H, int L, int D, int M, int window);
template <typename T, typename To, int D>
hipError_t launch_nha(const T* q, const T* k, const T* v, const float* gate, int M, To* out, void* ws, int B, int H,
                      int L, int window, float scale, hipStream_t st, void (*prof)(int, hipStream_t, int),
                      const SideStream& side = SideStream());

size_t gdn_ws_bytes(int io_is_bf16, int D, int64_t nch);
// Gated DeltaNet branch gradient (chunk form): ws holds every chunk's start
// state S0 and U, then the chunk preps' region(s) and every chunk's carried
// gradient; `overlap` lays out separate regions for the two sweeps
size_t gdn_bwd_ws_bytes(int io_is_bf16, int B, int H, int L, int D, bool overlap);
// the forward in state mode: every chunk's start state s0 [B, H, Nc, D, D]
// and U [B, H, L, D] (io dtype), no outputs; ws as launch_gdn's
template <typename T, int D>
hipError_t launch_gdn_states(const T* q, const T* k, const T* v, const float* alpha, const float* beta,
                             const int32_t* route, const float* S_init, T* s0, T* u, void* ws, int B, int H, int L,
                             int G, hipStream_t st);
template <typename T, int D>
hipError_t launch_gdn_backward(const T* q, const T* k, const T* v, const float* alpha, const float* beta,
                               const int32_t* route, const float* S_init, const float* d_o, const float* dS_final,
                               float* dq, float* dk, float* dv, float* dalpha, float* dbeta, float* dS_init,
                               float* dgate, void* ws, int B, int H, int L, int G, hipStream_t st,
                               const SideStream& ov = SideStream());
template <typename T, typename To, int D>
hipError_t launch_gdn(const T* q, const T* k, const T* v, const float* alpha, const float* beta,
                      const int32_t* route, const float* S_init, To* o_gdn, float* S_final, void* ws,
                      int B, int H, int L, int G, hipStream_t st_prep, hipStream_t st_scan,
                      hipEvent_t prep_done, hipEvent_t scan_dep, void (*prof)(int, hipStream_t, int));

struct DecodeLaunch {
  int B, H, G, d, cap;
  float scale, eps;
  const void *x, *q, *k, *v;
  const float *alpha, *beta, *w_score, *b_score, *w_mix;
  int64_t w_mix_hs;
  const float *g_sm, *g_lin;
  void *k_cache, *v_cache;
  int32_t *n_committed, *n_open, *err_flag, *route_out;
  float *S_carry, *S_work, *x_sum;
  void* out;
  float *o_sm_dbg, *o_gdn_dbg;
};
size_t decode_ws_bytes(int B, int H, int G, int D, int cap);
// nullptr if a decode step supports these sizes, else why not
const char* decode_dims_problem(int B, int H, int cap);
// the allocation-free decode step's scratch: a DECODE_SCRATCH_BYTES array per
// device, 256-byte aligned; its device address on the current device
constexpr size_t DECODE_SCRATCH_BYTES = (size_t)16 << 20;
hipError_t decode_scratch_address(void** out);

// prefill -> decode handoff
struct HandoffLaunch {
  int B, H, G, L, D, d, cap, append;
  const int32_t* route;
  const void *k, *v;
  const float* S_final;
  void *k_cache, *v_cache;
  int32_t *n_committed, *n_open, *err_flag;
  float *S_carry, *S_work, *x_sum;
};
size_t handoff_ws_bytes(int B, int G, int nc);
template <typename T>
hipError_t launch_handoff(const HandoffLaunch& a, void* ws, hipStream_t st);
template <typename T, int D>
hipError_t launch_decode(const DecodeLaunch& a, void* ws, hipStream_t st,
                         void (*prof)(int, hipStream_t, int));

}  // namespace natsl
