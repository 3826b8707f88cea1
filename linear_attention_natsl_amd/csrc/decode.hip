// Single-token decode step.
//
// "Technische Samenvatting: Neural Attention Search Linear (NAtS-L)",
// Kernmechanismen 3 keeps two hidden states: the softmax operation's KV (only
// softmax-routed chunks are kept) and the linear operation's fixed-size state.
// Online, the new token joins the open chunk: it attends to the committed
// softmax rows, the open chunk's earlier rows and itself, and pseudo-updates
// the Gated DeltaNet state (from S_carry at a chunk's first token, else from
// S_work).  When the chunk reaches 64 tokens it is routed (Kernmechanismen 1)
// and either its rows (softmax) or its state (linear) are committed.
//
// The step is HBM-bound (the cached rows dominate):
//   k_decode_route    x_sum += x; on chunk completion score x_sum / 64
//   k_decode_gdn      one 64 KiB fp32 state read + write per (b, h)
//   k_decode_attn     split-KV flash decode: every workgroup streams 1024 rows
//                     of K and V (16 lanes per row, 16-byte loads, 16 rows per
//                     lane group in flight) and leaves (max, sum, o) partials
//   k_decode_combine  merge the partials and the new token, RMSNorm both
//                     branches, Q-derived weights, append the new k/v row
//   k_decode_commit   advance the counters
#include <mutex>

#include "common.hpp"
#include "kernels.hpp"

namespace natsl {

// Scratch of the allocation-free decode step: one array per device, in the
// code object's device memory, which every such call on that device uses.
// (Its name is a host-side stand-in in host code; kernels get the device
// address that hipGetSymbolAddress returns, kept per device below.)
static __device__ __align__(256) unsigned char scratch[DECODE_SCRATCH_BYTES];

template <typename T>
__global__ void __launch_bounds__(256) k_decode_route(const T* __restrict__ x, const float* __restrict__ w,
                                                      const float* __restrict__ bsc, int d, int G,
                                                      float* __restrict__ x_sum,
                                                      const int32_t* __restrict__ n_open,
                                                      int32_t* __restrict__ dec,
                                                      int32_t* __restrict__ route_out) {
  extern __shared__ float s_mean[];  // [d + 2G]
  const int b = bid_x();
  const bool complete = (n_open[b] + 1) == CHUNK;
  for (int col0 = tid_x() * 8; col0 < d; col0 += 256 * 8) {
    float xv[8];
    load8f<T>(x + (int64_t)b * d + col0, xv);
    float* xs = x_sum + (int64_t)b * d + col0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float s = xs[j] + xv[j];
      if (complete) {
        s_mean[col0 + j] = s * (1.0f / CHUNK);
        xs[j] = 0.f;
      } else {
        xs[j] = s;
      }
    }
  }
  if (!complete) {
    for (int gg = tid_x(); gg < G; gg += 256) {
      dec[b * G + gg] = -1;
      if (route_out) route_out[b * G + gg] = -1;
    }
    return;
  }
  __syncthreads();
  const int lane = lane_id(), wv = wave_id();
  for (int o = wv; o < 2 * G; o += 4) {
    float p = 0.f;
    for (int j = lane; j < d; j += 64) p += s_mean[j] * w[(int64_t)j * 2 * G + o];
    p = wave_sum64(p);
    if (bsc) p += bsc[o];
    if (lane == 0) s_mean[d + o] = p;
  }
  __syncthreads();
  for (int gg = tid_x(); gg < G; gg += 256) {
    const int r = (s_mean[d + 2 * gg] >= s_mean[d + 2 * gg + 1]) ? 0 : 1;
    dec[b * G + gg] = r;
    if (route_out) route_out[b * G + gg] = r;
  }
}

template <typename T, int D>
__global__ void __launch_bounds__(256) k_decode_gdn(const T* __restrict__ q, const T* __restrict__ k,
                                                    const T* __restrict__ v, const float* __restrict__ alpha,
                                                    const float* __restrict__ beta, float* S_carry,
                                                    float* S_work, const int32_t* __restrict__ n_open,
                                                    const int32_t* __restrict__ dec, int H, int G,
                                                    float* __restrict__ o_gdn) {
  constexpr int TPC = 256 / D;  // threads per column
  constexpr int RPT = D / TPC;  // rows per thread
  __shared__ float kq[3][D];
  __shared__ float red[TPC][D];
  const int bh = bid_x(), b = bh / H, h = bh % H;
  const int grp = (G == 1) ? 0 : h;
  const int t = tid_x(), col = t % D, part = t / D;
  if (t < D) {
    kq[0][t] = to_f32(k[(int64_t)bh * D + t]);
    kq[1][t] = to_f32(q[(int64_t)bh * D + t]);
    kq[2][t] = to_f32(v[(int64_t)bh * D + t]);
  }
  const float* src = (n_open[b] == 0) ? S_carry : S_work;
  const bool commit = dec[b * G + grp] == 1;
  const int64_t base = (int64_t)bh * D * D;
  float s[RPT];
#pragma unroll
  for (int r = 0; r < RPT; ++r) s[r] = src[base + (int64_t)(part * RPT + r) * D + col];
  __syncthreads();
  float ks = 0.f;
#pragma unroll
  for (int r = 0; r < RPT; ++r) ks += kq[0][part * RPT + r] * s[r];
  red[part][col] = ks;
  __syncthreads();
  float u = 0.f;
#pragma unroll
  for (int p = 0; p < TPC; ++p) u += red[p][col];
  const float a = alpha[bh], bt = beta[bh];
  const float vv = kq[2][col];
  float op = 0.f;
#pragma unroll
  for (int r = 0; r < RPT; ++r) {
    const float kr = kq[0][part * RPT + r];
    const float sn = a * (s[r] - bt * kr * u) + bt * kr * vv;
    const int64_t idx = base + (int64_t)(part * RPT + r) * D + col;
    S_work[idx] = sn;
    if (commit) S_carry[idx] = sn;
    op += sn * kq[1][part * RPT + r];
  }
  __syncthreads();
  red[part][col] = op;
  __syncthreads();
  if (part == 0) {
    float o = 0.f;
#pragma unroll
    for (int p = 0; p < TPC; ++p) o += red[p][col];
    o_gdn[(int64_t)bh * D + col] = o;
  }
}

constexpr int DEC_SPLIT = 1024;  // cached rows per workgroup
constexpr int DEC_UNROLL = 16;   // rows per lane group in flight

template <typename T, int D>
__global__ void __launch_bounds__(256) k_decode_attn(const T* __restrict__ q, const T* __restrict__ kc,
                                                     const T* __restrict__ vc, int cap,
                                                     const int32_t* __restrict__ n_committed,
                                                     const int32_t* __restrict__ n_open, int H, int G,
                                                     float scale_log2, int nsplit,
                                                     float* __restrict__ part_o,
                                                     float* __restrict__ part_ml) {
  constexpr int LPK = D / 8;        // lanes per row
  constexpr int GPW = 64 / LPK;     // row groups per wave
  constexpr int NGRP = 4 * GPW;     // row groups per workgroup
  __shared__ float red_o[NGRP][D];
  __shared__ float red_m[NGRP], red_l[NGRP];
  const unsigned bid = (unsigned)bid_x();  // (split, b * H + h) flattened, split fastest
  const int s = (int)(bid % (unsigned)nsplit), bh = (int)(bid / (unsigned)nsplit), b = bh / H, h = bh % H;
  const int grp = (G == 1) ? 0 : h;
  // rows actually present (after a capacity error the counters run past cap)
  const int n = min(n_committed[b * G + grp] + n_open[b], cap);
  const int lo = s * DEC_SPLIT;
  const int hi = min(n, lo + DEC_SPLIT);
  const int lane = lane_id(), w = wave_id();
  const int sub = lane % LPK, kslot = lane / LPK;
  const int grpid = w * GPW + kslot;
  float qv[8];
  load8f<T>(q + (int64_t)bh * D + 8 * sub, qv);
#pragma unroll
  for (int j = 0; j < 8; ++j) qv[j] *= scale_log2;
  float m = -INFINITY, l = 0.f, acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.f;
  const T* kb = kc + (int64_t)bh * cap * D + 8 * sub;
  const T* vb = vc + (int64_t)bh * cap * D + 8 * sub;
  for (int r0 = lo + grpid; r0 < hi; r0 += NGRP * DEC_UNROLL) {
    Frag<T> kf[DEC_UNROLL], vf[DEC_UNROLL];
#pragma unroll
    for (int u = 0; u < DEC_UNROLL; ++u) {
      const int r = r0 + u * NGRP;
      const int rr = (r < hi) ? r : lo;  // in-bounds row; masked below
      if constexpr (sizeof(T) == 2) {  // each cached row is read once per step: streaming (non-temporal) loads
        kf[u].v = __builtin_bit_cast(bf16x8, __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(kb + (int64_t)rr * D)));
        vf[u].v = __builtin_bit_cast(bf16x8, __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(vb + (int64_t)rr * D)));
      } else {
        kf[u] = load8<T>(kb + (int64_t)rr * D);
        vf[u] = load8<T>(vb + (int64_t)rr * D);
      }
    }
    float sc[DEC_UNROLL];
#pragma unroll
    for (int u = 0; u < DEC_UNROLL; ++u) {
      float p = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) p += qv[j] * to_f32(frag_get<T>(kf[u], j));
      p = dpp_group_sum<LPK>(p);
      sc[u] = (r0 + u * NGRP < hi) ? p : -INFINITY;
    }
    float mb = sc[0];
#pragma unroll
    for (int u = 1; u < DEC_UNROLL; ++u) mb = fmaxf(mb, sc[u]);
    const float mn = fmaxf(m, mb);  // finite: row r0 < hi is valid
    const float corr = exp2f(m - mn);
    l *= corr;
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] *= corr;
#pragma unroll
    for (int u = 0; u < DEC_UNROLL; ++u) {
      const float p = exp2f(sc[u] - mn);
      l += p;
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] += p * to_f32(frag_get<T>(vf[u], j));
    }
    m = mn;
  }
  if (sub == 0) {
    red_m[grpid] = m;
    red_l[grpid] = l;
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) red_o[grpid][8 * sub + j] = acc[j];
  __syncthreads();
  const int t = tid_x();
  if (t < D) {
    float M = -INFINITY;
#pragma unroll
    for (int gi = 0; gi < NGRP; ++gi) M = fmaxf(M, red_m[gi]);
    float Lt = 0.f, O = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int gi = 0; gi < NGRP; ++gi) {
        const float f = exp2f(red_m[gi] - M);
        Lt += red_l[gi] * f;
        O += red_o[gi][t] * f;
      }
    }
    const int64_t pidx = (int64_t)bh * nsplit + s;
    part_o[pidx * D + t] = O;
    if (t == 0) {
      part_ml[pidx * 2] = M;
      part_ml[pidx * 2 + 1] = Lt;
    }
  }
}

template <typename T, int D>
__global__ void __launch_bounds__(D) k_decode_combine(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, T* kc, T* vc, int cap,
    const int32_t* __restrict__ n_committed, const int32_t* __restrict__ n_open, int H, int G,
    float scale_log2, int nsplit, const float* __restrict__ part_o, const float* __restrict__ part_ml,
    const float* __restrict__ o_gdn, const float* __restrict__ w_mix, int64_t wmix_hs,
    const float* __restrict__ g_sm, const float* __restrict__ g_lin, float eps, T* __restrict__ out,
    float* __restrict__ o_sm_dbg, float* __restrict__ o_gdn_dbg, int32_t* __restrict__ err_flag) {
  __shared__ float red[4][D / 64 > 0 ? D / 64 : 1];
  const int bh = bid_x(), b = bh / H, h = bh % H;
  const int grp = (G == 1) ? 0 : h;
  const int t = tid_x(), lane = lane_id(), w = wave_id();
  constexpr int NW = D / 64;
  const int n = n_committed[b * G + grp] + n_open[b];
  const float qv = to_f32(q[(int64_t)bh * D + t]);
  const T kn = k[(int64_t)bh * D + t];
  const T vn = v[(int64_t)bh * D + t];
  const float* wm = w_mix + (int64_t)h * wmix_hs;
  // block reductions of: q.k_new, q.W_mix[:,0], q.W_mix[:,1]
  float r0 = qv * to_f32(kn), r1 = qv * wm[2 * t], r2 = qv * wm[2 * t + 1];
  r0 = wave_sum64(r0);
  r1 = wave_sum64(r1);
  r2 = wave_sum64(r2);
  if (lane == 0) {
    red[0][w] = r0;
    red[1][w] = r1;
    red[2][w] = r2;
  }
  __syncthreads();
  float qk = 0.f, z0 = 0.f, z1 = 0.f;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    qk += red[0][i];
    z0 += red[1][i];
    z1 += red[2][i];
  }
  const float s_new = qk * scale_log2;
  const int nsp = (min(n, cap) + DEC_SPLIT - 1) / DEC_SPLIT;
  float M = s_new;
  for (int s = 0; s < nsp; ++s) M = fmaxf(M, part_ml[((int64_t)bh * nsplit + s) * 2]);
  const float fn = exp2f(s_new - M);
  float Lt = fn, O = fn * to_f32(vn);
  for (int s = 0; s < nsp; ++s) {
    const int64_t pidx = (int64_t)bh * nsplit + s;
    const float f = exp2f(part_ml[pidx * 2] - M);
    Lt += part_ml[pidx * 2 + 1] * f;
    O += part_o[pidx * D + t] * f;
  }
  const float osm = O / Lt;
  const float og = o_gdn[(int64_t)bh * D + t];
  // RMS of both branches
  float a2 = osm * osm, b2 = og * og;
  a2 = wave_sum64(a2);
  b2 = wave_sum64(b2);
  __syncthreads();
  if (lane == 0) {
    red[0][w] = a2;
    red[1][w] = b2;
  }
  __syncthreads();
  float ssa = 0.f, ssb = 0.f;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    ssa += red[0][i];
    ssb += red[1][i];
  }
  const float ra = 1.0f / sqrtf(ssa * (1.0f / D) + eps);
  const float rb = 1.0f / sqrtf(ssb * (1.0f / D) + eps);
  const float zm = fmaxf(z0, z1);
  const float e0 = expf(z0 - zm), e1 = expf(z1 - zm);
  const float inv = 1.0f / (e0 + e1);
  const float gs = g_sm ? g_sm[t] : 1.f, gl = g_lin ? g_lin[t] : 1.f;
  const float o = e0 * inv * ra * osm * gs + e1 * inv * rb * og * gl;
  out[(int64_t)bh * D + t] = from_f32<T>(o);
  if (o_sm_dbg) o_sm_dbg[(int64_t)bh * D + t] = osm;
  if (o_gdn_dbg) o_gdn_dbg[(int64_t)bh * D + t] = og;
  if (n < cap) {
    kc[((int64_t)bh * cap + n) * D + t] = kn;
    vc[((int64_t)bh * cap + n) * D + t] = vn;
  } else if (t == 0) {
    err_flag[0] = 1;
  }
}

__global__ void k_decode_commit(int B, int G, int32_t* __restrict__ n_committed,
                                int32_t* __restrict__ n_open, const int32_t* __restrict__ dec) {
  const int b = bid_x() * block_dim_x() + tid_x();
  if (b >= B) return;
  int no = n_open[b] + 1;
  if (no == CHUNK) {
    for (int gg = 0; gg < G; ++gg)
      if (dec[b * G + gg] == 0) n_committed[b * G + gg] += CHUNK;
    no = 0;
  }
  n_open[b] = no;
}

hipError_t decode_scratch_address(void** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* ptrs[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(mu);
  if (!ptrs[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));  // with device `dev` current
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    ptrs[dev] = p;
  }
  *out = ptrs[dev];
  return hipSuccess;
}

const char* decode_dims_problem(int B, int H, int cap) {
  if (cap < 1 || cap > (1 << 30)) return "cache capacity must lie in [1, 2^30]";
  // the attention grid has one 256-lane workgroup per (split, b, h)
  if ((int64_t)B * H * ((cap + DEC_SPLIT - 1) / DEC_SPLIT) >= ((int64_t)1 << 24))
    return "B * H * ceil(capacity / 1024) must stay below 2^24";
  return nullptr;
}

size_t decode_ws_bytes(int B, int H, int G, int D, int cap) {
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const size_t nsplit = ((size_t)cap + DEC_SPLIT - 1) / DEC_SPLIT;
  return al((size_t)B * G * 4) + al((size_t)B * H * D * 4) + al((size_t)B * H * nsplit * D * 4) +
         al((size_t)B * H * nsplit * 2 * 4);
}

template <typename T, int D>
hipError_t launch_decode(const DecodeLaunch& a, void* wsp, hipStream_t st,
                         void (*prof)(int, hipStream_t, int)) {
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const int nsplit = (a.cap + DEC_SPLIT - 1) / DEC_SPLIT;
  char* p = (char*)wsp;
  int32_t* dec = (int32_t*)p; p += al((size_t)a.B * a.G * 4);
  float* o_gdn = (float*)p; p += al((size_t)a.B * a.H * D * 4);
  float* part_o = (float*)p; p += al((size_t)a.B * a.H * nsplit * D * 4);
  float* part_ml = (float*)p;
  hipError_t e;
#define LAUNCH_CHECK(kid, ...)           \
  if (prof) prof(kid, st, 0);            \
  hipLaunchKernelGGL(__VA_ARGS__);       \
  e = hipGetLastError();                 \
  if (e != hipSuccess) return e;         \
  if (prof) prof(kid, st, 1);
  LAUNCH_CHECK(KID_DECODE_ROUTE, k_decode_route<T>, dim3(a.B), dim3(256),
               (size_t)(a.d + 2 * a.G) * 4, st, (const T*)a.x, a.w_score, a.b_score, a.d, a.G, a.x_sum,
               a.n_open, dec, a.route_out);
  LAUNCH_CHECK(KID_DECODE_GDN, (k_decode_gdn<T, D>), dim3(a.B * a.H), dim3(256), 0, st, (const T*)a.q,
               (const T*)a.k, (const T*)a.v, a.alpha, a.beta, a.S_carry, a.S_work, a.n_open, dec, a.H,
               a.G, o_gdn);
  LAUNCH_CHECK(KID_DECODE_ATTN, (k_decode_attn<T, D>), dim3((unsigned)(nsplit * a.B * a.H)), dim3(256), 0, st,
               (const T*)a.q, (const T*)a.k_cache, (const T*)a.v_cache, a.cap, a.n_committed, a.n_open,
               a.H, a.G, a.scale * LOG2E, nsplit, part_o, part_ml);
  LAUNCH_CHECK(KID_DECODE_COMBINE, (k_decode_combine<T, D>), dim3(a.B * a.H), dim3(D), 0, st,
               (const T*)a.q, (const T*)a.k, (const T*)a.v, (T*)a.k_cache, (T*)a.v_cache, a.cap,
               a.n_committed, a.n_open, a.H, a.G, a.scale * LOG2E, nsplit, part_o, part_ml, o_gdn,
               a.w_mix, a.w_mix_hs, a.g_sm, a.g_lin, a.eps, (T*)a.out, a.o_sm_dbg, a.o_gdn_dbg,
               a.err_flag);
  LAUNCH_CHECK(KID_DECODE_COMMIT, k_decode_commit, dim3((a.B + 63) / 64), dim3(64), 0, st, a.B, a.G,
               a.n_committed, a.n_open, dec);
#undef LAUNCH_CHECK
  return hipSuccess;
}

template hipError_t launch_decode<float, 64>(const DecodeLaunch&, void*, hipStream_t,
                                             void (*)(int, hipStream_t, int));
template hipError_t launch_decode<float, 128>(const DecodeLaunch&, void*, hipStream_t,
                                              void (*)(int, hipStream_t, int));
template hipError_t launch_decode<bf16, 64>(const DecodeLaunch&, void*, hipStream_t,
                                            void (*)(int, hipStream_t, int));
template hipError_t launch_decode<bf16, 128>(const DecodeLaunch&, void*, hipStream_t,
                                             void (*)(int, hipStream_t, int));

}  // namespace natsl
