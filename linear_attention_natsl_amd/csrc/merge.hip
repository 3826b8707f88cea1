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
