// Output merging: "Technische Samenvatting: Neural Attention Search Linear
// (NAtS-L)", Kernmechanismen 4 -- each branch output is RMS-normalised and the
// two are added with weights generated from the query.
//   n_x = o_x / sqrt(mean(o_x^2) + eps) * g_x,  (w_sm, w_lin) = softmax(q W_mix),
//   out = w_sm n_sm + w_lin n_lin.
// Bandwidth-bound: D/8 lanes per token, 8 elements per lane (16-byte bf16
// loads), reductions across the token's lanes in registers (DPP row ops).
#include "common.hpp"
#include "kernels.hpp"

namespace natsl {

template <typename Tq, typename Tb, typename To, int D>
__global__ void __launch_bounds__(256) k_merge(const Tq* __restrict__ q, const Tb* __restrict__ o_sm,
                                               const Tb* __restrict__ o_gdn,
                                               const float* __restrict__ w_mix, int64_t wmix_hs,
                                               const float* __restrict__ g_sm,
                                               const float* __restrict__ g_lin, To* __restrict__ out,
                                               int H, int L, float eps, int64_t ntok,
                                               const float* __restrict__ mixd) {
  constexpr int LPT = D / 8;  // lanes per token
  const int64_t gtid = (int64_t)bid_x() * 256 + tid_x();
  const int64_t tok = gtid / LPT;
  const int sub = (int)(gtid % LPT);
  const bool valid = tok < ntok;
  const int64_t t = valid ? tok : 0;
  const int h = (int)((t / L) % H);
  const int col = sub * 8;
  float a[8], b[8];
  load8f<Tb>(o_sm + t * D + col, a);
  load8f<Tb>(o_gdn + t * D + col, b);
  float ssa = 0.f, ssb = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    ssa += a[j] * a[j];
    ssb += b[j] * b[j];
  }
  ssa = dpp_group_sum<LPT>(ssa);
  ssb = dpp_group_sum<LPT>(ssb);
  const float ra = 1.0f / sqrtf(ssa * (1.0f / D) + eps);
  const float rb = 1.0f / sqrtf(ssb * (1.0f / D) + eps);
  // mixing weights softmax(z0, z1), z = q W_mix
  float m0, m1;
  if (mixd) {  // z0 - z1 given
    const float dz = mixd[t];
    const float e = expf(-fabsf(dz)), inv = 1.0f / (1.0f + e);
    m0 = dz >= 0.f ? inv : e * inv;
    m1 = dz >= 0.f ? e * inv : inv;
  } else {
    float qv[8];
    load8f<Tq>(q + t * D + col, qv);
    // the lane's 8 rows of W_mix [D, 2] are 16 consecutive floats
    const f32x4* wm4 = reinterpret_cast<const f32x4*>(w_mix + (int64_t)h * wmix_hs + col * 2);
    float wm[16];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x4 t4 = wm4[j];
      wm[4 * j] = t4[0]; wm[4 * j + 1] = t4[1]; wm[4 * j + 2] = t4[2]; wm[4 * j + 3] = t4[3];
    }
    float z0 = 0.f, z1 = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      z0 += qv[j] * wm[2 * j];
      z1 += qv[j] * wm[2 * j + 1];
    }
    z0 = dpp_group_sum<LPT>(z0);
    z1 = dpp_group_sum<LPT>(z1);
    const float zm = fmaxf(z0, z1);
    const float e0 = expf(z0 - zm), e1 = expf(z1 - zm);
    const float inv = 1.0f / (e0 + e1);
    m0 = e0 * inv;
    m1 = e1 * inv;
  }
  const float w0 = m0 * ra, w1 = m1 * rb;
  float gs[8], gl[8];
  if (g_sm) load8f<float>(g_sm + col, gs);
  else
#pragma unroll
    for (int j = 0; j < 8; ++j) gs[j] = 1.f;
  if (g_lin) load8f<float>(g_lin + col, gl);
  else
#pragma unroll
    for (int j = 0; j < 8; ++j) gl[j] = 1.f;
  float o[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) o[j] = w0 * a[j] * gs[j] + w1 * b[j] * gl[j];
  if (valid) {
    Frag<To> f;
#pragma unroll
    for (int j = 0; j < 8; ++j) frag_set(f, j, o[j]);
    store8<To>(out + t * D + col, f);
  }
}

template <typename Tq, typename Tb, int D>
hipError_t launch_merge(const Tq* q, const Tb* o_sm, const Tb* o_gdn, const float* w_mix, int64_t hs,
                        const float* g_sm, const float* g_lin, Tq* out, int B, int H, int L,
                        float eps, hipStream_t st, const float* mixd) {
  const int64_t ntok = (int64_t)B * H * L;
  const int64_t threads = ntok * (D / 8);
  const int64_t blocks = (threads + 255) / 256;
  hipLaunchKernelGGL((k_merge<Tq, Tb, Tq, D>), dim3((unsigned)blocks), dim3(256), 0, st, q, o_sm,
                     o_gdn, w_mix, hs, g_sm, g_lin, out, H, L, eps, ntok, mixd);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Gradient of the merge (the pages define the forward; this is its exact
// derivative).  With r_x = (mean(o_x^2) + eps)^(-1/2), n_x = o_x r_x g_x and
// (w_0, w_1) = softmax(q W_mix):
//   dn_x = w_x d_out,  dw_x = d_out . n_x,  dz_0 = w_0 w_1 (dw_0 - dw_1) = -dz_1
//   dq = dz_0 (W_mix[:, 0] - W_mix[:, 1]),   dW_mix[:, 0] = sum_t q dz_0 = -dW_mix[:, 1]
//   d o_x = r_x u - (r_x^3 / D) o_x (u . o_x) with u = dn_x g_x,   dg_x = sum_t dn_x o_x r_x
// One token per D/8 lanes as in the forward; a block's tokens belong to one
// head (L is a multiple of 64).  Each block writes its sums of q dz_0, dn_sm
// o_sm r_sm and dn_lin o_lin r_lin per column; k_merge_bwd_reduce adds the
// blocks' partials in block order (deterministic).
__device__ __forceinline__ void store8f(float* p, const float (&v)[8]) {
  *reinterpret_cast<f32x4*>(p) = f32x4{v[0], v[1], v[2], v[3]};
  *reinterpret_cast<f32x4*>(p + 4) = f32x4{v[4], v[5], v[6], v[7]};
}

template <typename Tq, typename Tb, int D>
__global__ void __launch_bounds__(256) k_merge_bwd(const Tq* __restrict__ q, const Tb* __restrict__ o_sm,
                                                   const Tb* __restrict__ o_gdn, const float* __restrict__ w_mix,
                                                   int64_t wmix_hs, const float* __restrict__ g_sm,
                                                   const float* __restrict__ g_lin, const float* __restrict__ d_out,
                                                   float* __restrict__ d_sm, float* __restrict__ d_gdn,
                                                   float* __restrict__ dq, float* __restrict__ part, int H, int L,
                                                   float eps) {
  constexpr int LPT = D / 8;         // lanes per token
  constexpr int TPB = 256 / LPT;     // tokens per block
  __shared__ float red[TPB][3 * D + 1];
  const int tl = tid_x() / LPT, sub = tid_x() % LPT, col = 8 * sub;
  const int64_t t = (int64_t)bid_x() * TPB + tl;  // token index in [B, H, L]
  const int h = (int)((t / L) % H);
  float qv[8], a[8], b[8], go[8], gs[8], gl[8], wm[16];
  load8f<Tq>(q + t * D + col, qv);
  load8f<Tb>(o_sm + t * D + col, a);
  load8f<Tb>(o_gdn + t * D + col, b);
  load8f<float>(d_out + t * D + col, go);
  if (g_sm) load8f<float>(g_sm + col, gs);
  else
#pragma unroll
    for (int j = 0; j < 8; ++j) gs[j] = 1.f;
  if (g_lin) load8f<float>(g_lin + col, gl);
  else
#pragma unroll
    for (int j = 0; j < 8; ++j) gl[j] = 1.f;
  const f32x4* wm4 = reinterpret_cast<const f32x4*>(w_mix + (int64_t)h * wmix_hs + col * 2);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const f32x4 t4 = wm4[j];
    wm[4 * j] = t4[0]; wm[4 * j + 1] = t4[1]; wm[4 * j + 2] = t4[2]; wm[4 * j + 3] = t4[3];
  }
  float ssa = 0.f, ssb = 0.f, z0 = 0.f, z1 = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    ssa += a[j] * a[j];
    ssb += b[j] * b[j];
    z0 += qv[j] * wm[2 * j];
    z1 += qv[j] * wm[2 * j + 1];
  }
  ssa = dpp_group_sum<LPT>(ssa);
  ssb = dpp_group_sum<LPT>(ssb);
  z0 = dpp_group_sum<LPT>(z0);
  z1 = dpp_group_sum<LPT>(z1);
  const float ra = 1.0f / sqrtf(ssa * (1.0f / D) + eps);
  const float rb = 1.0f / sqrtf(ssb * (1.0f / D) + eps);
  const float zm = fmaxf(z0, z1);
  const float e0 = expf(z0 - zm), e1 = expf(z1 - zm);
  const float inv = 1.0f / (e0 + e1);
  const float w0 = e0 * inv, w1 = e1 * inv;
  // dw_x = d_out . n_x and u_x . o_x with u_x = w_x d_out g_x
  float dw0 = 0.f, dw1 = 0.f, sua = 0.f, sub_ = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    dw0 += go[j] * a[j] * ra * gs[j];
    dw1 += go[j] * b[j] * rb * gl[j];
    sua += go[j] * gs[j] * a[j];
    sub_ += go[j] * gl[j] * b[j];
  }
  dw0 = dpp_group_sum<LPT>(dw0);
  dw1 = dpp_group_sum<LPT>(dw1);
  sua = dpp_group_sum<LPT>(sua) * w0;
  sub_ = dpp_group_sum<LPT>(sub_) * w1;
  const float dz0 = w0 * w1 * (dw0 - dw1);
  const float ca = ra * ra * ra * (1.0f / D) * sua, cb = rb * rb * rb * (1.0f / D) * sub_;
  float oa[8], ob[8], oq[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    oa[j] = ra * w0 * go[j] * gs[j] - ca * a[j];
    ob[j] = rb * w1 * go[j] * gl[j] - cb * b[j];
    oq[j] = dz0 * (wm[2 * j] - wm[2 * j + 1]);
    red[tl][col + j] = qv[j] * dz0;                      // W_mix column 0 (column 1 is its negative)
    red[tl][D + col + j] = w0 * go[j] * a[j] * ra;       // gain of the softmax branch
    red[tl][2 * D + col + j] = w1 * go[j] * b[j] * rb;   // gain of the linear branch
  }
  store8f(d_sm + t * D + col, oa);
  store8f(d_gdn + t * D + col, ob);
  store8f(dq + t * D + col, oq);
  __syncthreads();
  for (int e = tid_x(); e < 3 * D; e += 256) {
    float s = 0.f;
    for (int x = 0; x < TPB; ++x) s += red[x][e];
    part[(int64_t)bid_x() * 3 * D + e] = s;
  }
}

// dW_mix (per head when wmix_hs != 0, else over every head) and the gains'
// gradients from the blocks' partials, in two deterministic stages.  Output
// groups of 64 consecutive partial slots: the gains' 2D slots (over every
// block), then D / 64 groups of dW_mix slots per head (or once, shared).
// Stage 1: workgroup (group, range) adds the group's 64 slots over one of
// kMergeSplit contiguous block ranges (wave w takes every 4th block, so each
// wave reads 256 contiguous bytes per block), the 4 waves added in order.
// Stage 2: each slot's kMergeSplit range sums added in range order.
constexpr int kMergeSplit = 64;

__device__ __forceinline__ void merge_group(int g, int D, int per_head, int64_t nblk, int H, int& base, int& hh,
                                            bool& head_only, int64_t& count) {
  const int gains = 2 * D / 64;
  if (g < gains) {
    base = D + 64 * g;  // partial slots D .. 3D - 1: dg_sm, dg_lin
    hh = 0;
    head_only = false;
    count = nblk;
  } else {
    const int r = g - gains;
    hh = per_head ? r / (D / 64) : 0;
    base = 64 * (r % (D / 64));  // partial slots 0 .. D - 1: dW_mix column 0
    head_only = per_head != 0;
    count = head_only ? nblk / H : nblk;  // a head's blocks: B runs of blk_per_head
  }
}

template <int D>
__global__ void __launch_bounds__(256) k_merge_bwd_reduce(const float* __restrict__ part, int64_t nblk,
                                                          int64_t blk_per_head, int H, int per_head,
                                                          float* __restrict__ part2) {
  __shared__ float red[4][64];
  const int g = bid_x() / kMergeSplit, sp = bid_x() % kMergeSplit, t = tid_x(), el = t & 63, sb = t >> 6;
  int base, hh;
  bool head_only;
  int64_t count;
  merge_group(g, D, per_head, nblk, H, base, hh, head_only, count);
  const int64_t chunk = (count + kMergeSplit - 1) / kMergeSplit;
  const int64_t n0 = sp * chunk, n1 = min(count, n0 + chunk);
  auto slot_of = [&](int64_t n) {
    const int64_t x = head_only ? ((n / blk_per_head) * H + hh) * blk_per_head + n % blk_per_head : n;
    return part + x * 3 * D + base + el;
  };
  // 16 loads in flight per lane, added in block order (the same order as one
  // load at a time: the sums do not depend on the unrolling)
  constexpr int U = 16;
  float s = 0.f;
  int64_t n = n0 + sb;
  for (; n + 4 * (U - 1) < n1; n += 4 * U) {
    float v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = *slot_of(n + 4 * u);
#pragma unroll
    for (int u = 0; u < U; ++u) s += v[u];
  }
  for (; n < n1; n += 4) s += *slot_of(n);
  red[sb][el] = s;
  __syncthreads();
  if (t < 64) part2[(int64_t)bid_x() * 64 + t] = (red[0][t] + red[1][t]) + (red[2][t] + red[3][t]);
}

template <int D>
__global__ void __launch_bounds__(64) k_merge_bwd_final(const float* __restrict__ part2, int64_t nblk, int H,
                                                        int per_head, float* __restrict__ dw_mix,
                                                        float* __restrict__ dg_sm, float* __restrict__ dg_lin) {
  const int g = bid_x(), t = tid_x();
  int base, hh;
  bool head_only;
  int64_t count;
  merge_group(g, D, per_head, nblk, H, base, hh, head_only, count);
  float s = 0.f;
  for (int sp = 0; sp < kMergeSplit; ++sp) s += part2[((int64_t)g * kMergeSplit + sp) * 64 + t];
  const int slot = base + t;
  if (g < 2 * D / 64) {
    if (slot < 2 * D) {
      if (dg_sm) dg_sm[slot - D] = s;
    } else if (dg_lin) {
      dg_lin[slot - 2 * D] = s;
    }
  } else if (dw_mix) {
    dw_mix[((int64_t)hh * D + slot) * 2] = s;
    dw_mix[((int64_t)hh * D + slot) * 2 + 1] = -s;
  }
}

size_t merge_bwd_ws_bytes(int B, int H, int L, int D) {
  const int64_t tpb = 256 / (D / 8);
  const int64_t nblk = ((int64_t)B * H * L) / tpb;
  const int64_t ngroups = 2 * D / 64 + (int64_t)H * D / 64;  // the per-head case (the larger)
  const size_t part = ((size_t)nblk * 3 * D * 4 + 255) / 256 * 256;
  return part + (size_t)ngroups * kMergeSplit * 64 * 4;
}

template <typename Tq, typename Tb, int D>
hipError_t launch_merge_backward(const Tq* q, const Tb* o_sm, const Tb* o_gdn, const float* w_mix, int64_t hs,
                                 const float* g_sm, const float* g_lin, const float* d_out, float* d_sm,
                                 float* d_gdn, float* dq, float* dw_mix, float* dg_sm, float* dg_lin, void* ws,
                                 int B, int H, int L, float eps, hipStream_t st) {
  constexpr int TPB = 256 / (D / 8);
  const int64_t ntok = (int64_t)B * H * L;
  const int64_t nblk = ntok / TPB;  // L % 64 == 0: whole blocks, each within one head
  float* part = (float*)ws;
  float* part2 = (float*)((char*)ws + ((size_t)nblk * 3 * D * 4 + 255) / 256 * 256);
  hipLaunchKernelGGL((k_merge_bwd<Tq, Tb, D>), dim3((unsigned)nblk), dim3(256), 0, st, q, o_sm, o_gdn, w_mix, hs,
                     g_sm, g_lin, d_out, d_sm, d_gdn, dq, part, H, L, eps);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int per_head = hs != 0;
  const int ngroups = 2 * D / 64 + (per_head ? H : 1) * D / 64;
  hipLaunchKernelGGL((k_merge_bwd_reduce<D>), dim3((unsigned)(ngroups * kMergeSplit)), dim3(256), 0, st, part, nblk,
                     (int64_t)(L / TPB), H, per_head, part2);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL((k_merge_bwd_final<D>), dim3((unsigned)ngroups), dim3(64), 0, st, part2, nblk, H, per_head,
                     dw_mix, dg_sm, dg_lin);
  return hipGetLastError();
}

#define INSTB(Tq, Tb, D)                                                                                           \
  template hipError_t launch_merge_backward<Tq, Tb, D>(const Tq*, const Tb*, const Tb*, const float*, int64_t,     \
                                                       const float*, const float*, const float*, float*, float*,   \
                                                       float*, float*, float*, float*, void*, int, int, int, float, \
                                                       hipStream_t);
INSTB(float, float, 64)
INSTB(float, float, 128)
INSTB(bf16, bf16, 64)
INSTB(bf16, bf16, 128)
INSTB(bf16, float, 64)
INSTB(bf16, float, 128)
INSTB(float, bf16, 64)
INSTB(float, bf16, 128)
#undef INSTB

#define INST(Tq, Tb, D)                                                                          \
  template hipError_t launch_merge<Tq, Tb, D>(const Tq*, const Tb*, const Tb*, const float*,     \
                                              int64_t, const float*, const float*, Tq*, int, int, \
                                              int, float, hipStream_t, const float*);
INST(float, float, 64)
INST(float, float, 128)
INST(float, bf16, 64)
INST(float, bf16, 128)
INST(bf16, float, 64)
INST(bf16, float, 128)
INST(bf16, bf16, 64)
INST(bf16, bf16, 128)
#undef INST

}  // namespace natsl
