// Gradient of the Gated DeltaNet branch through the per-chunk rollback.
//
// "Technische Samenvatting: Neural Attention Search Linear (NAtS-L)",
// Kernmechanismen 3 defines the forward: every chunk pseudo-updates the state
// token by token and keeps its end state only when it is routed to the linear
// operation (otherwise the chunk-start state is restored).  This is the exact
// derivative of that forward, taken token by token in reverse.  With
// G = d loss / d S_t (key-major [Dk, Dv]) and S = S_{t-1}, a = S^T k_t:
//   G += q_t do_t^T;  dq_t = S_t do_t;  w = G^T k_t;  dv_t = b_t w
//   dbeta_t = w . (v_t - a_t a);  dalpha_t = <G, S - b_t k_t a^T>
//   dk_t = b_t G v_t - a_t b_t (G a + S w);  G <- a_t (G - b_t k_t w^T)
// The carried state's gradient enters a chunk's last token when the chunk is
// linear-routed; otherwise it passes straight to the chunk start and the
// chunk's tokens see only their own outputs' gradients.
//
// One workgroup per (b, h) with 2 D threads: thread (j, half) holds rows
// half D/2 .. half D/2 + D/2 - 1 of state column j, so the column sums
// (S^T k, G^T k) are a register sum plus one LDS exchange, and the row sums
// (dq, dk) go through an LDS transpose.  Two launches:
//   k_gdn_bwd_ckpt  the forward, storing every chunk's starting (carried) state
//   k_gdn_bwd       chunks in reverse: recompute the chunk's per-token states
//                   into a scratch slot, then sweep its tokens backward
// Three barriers per token: this is the plain per-token form, a first
// correct GPU path for the gradient (the chunkwise form is not built).
#include "common.hpp"
#include "kernels.hpp"

namespace natsl {

constexpr int kRouteLinear = 1;  // route id of the linear (Gated DeltaNet) operation

template <int D>
struct GdnBwdCfg {
  static constexpr int NT = 2 * D;   // threads
  static constexpr int RPT = D / 2;  // state rows per thread
  static constexpr int XP = D + 1;   // pitch of the row-sum arrays
  // LDS (floats): vec[2][4][D] (k, v, q, do by token parity), part[2][4][D]
  // (column-sum halves of a and w), xq[D][XP], xk[D][XP], red[NT / 64][2]
  static constexpr int OFF_VEC = 0;
  static constexpr int OFF_PART = OFF_VEC + 2 * 4 * D;
  static constexpr int OFF_XQ = OFF_PART + 2 * 4 * D;
  static constexpr int OFF_XK = OFF_XQ + D * XP;
  static constexpr int OFF_RED = OFF_XK + D * XP;
  static constexpr int LDS_FLOATS = OFF_RED + 2 * (NT / 64);
  static constexpr int CKPT_LDS_FLOATS = OFF_XQ;  // the forward needs vec and part only
};

size_t gdn_bwd_ws_bytes(int B, int H, int L, int D) {
  const size_t nc = (size_t)L / CHUNK;
  return ((size_t)B * H * (nc + CHUNK) * D * D * 4 + 255) / 256 * 256;
}

// One forward token on the thread's rows of column j:
//   S <- a (S - b k (k^T S)) + b k v^T
// vec: this token's [k | v] (staged by the caller before the first barrier),
// part: this token's exchange buffer.
template <int D>
__device__ __forceinline__ void gdn_fwd_token(float (&S)[D / 2], const float* vec, float* part, int j, int hf,
                                              float al, float be) {
  constexpr int RPT = D / 2;
  const int r0 = hf * RPT;
  __syncthreads();  // vec staged
  float p4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < RPT; ++i) p4[i & 3] += S[i] * vec[r0 + i];
  part[hf * D + j] = (p4[0] + p4[1]) + (p4[2] + p4[3]);
  __syncthreads();  // column-sum halves exchanged
  const float a = part[j] + part[D + j], vj = vec[D + j];
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const float ki = vec[r0 + i];
    S[i] = al * (S[i] - be * ki * a) + be * ki * vj;
  }
}

template <typename T, int D>
__global__ void __launch_bounds__(2 * D) k_gdn_bwd_ckpt(const T* __restrict__ k, const T* __restrict__ v,
                                                        const float* __restrict__ alpha,
                                                        const float* __restrict__ beta,
                                                        const int32_t* __restrict__ route,
                                                        const float* __restrict__ S_init, float* __restrict__ ckpt,
                                                        int H, int L, int G) {
  using C = GdnBwdCfg<D>;
  extern __shared__ float lds_f[];
  const int nc = L / CHUNK;
  const int bh = bid_x(), b = bh / H, h = bh % H;
  const int grp = (G == 1) ? 0 : h;
  const int32_t* rt = route + ((int64_t)b * G + grp) * nc;
  const int t = tid_x(), j = t % D, hf = t / D, r0 = hf * C::RPT;
  const T* kh = k + (int64_t)bh * L * D;
  const T* vh = v + (int64_t)bh * L * D;
  const float* ah = alpha + (int64_t)bh * L;
  const float* bth = beta + (int64_t)bh * L;
  float* ck = ckpt + (int64_t)bh * nc * D * D;
  float S[C::RPT], carry[C::RPT];
#pragma unroll
  for (int i = 0; i < C::RPT; ++i) {
    S[i] = S_init ? S_init[((int64_t)bh * D + r0 + i) * D + j] : 0.f;
    carry[i] = S[i];
  }
  // this thread's staged value (k or v) and the decays, loaded a token ahead
  auto ld = [&](int tt) { return t < D ? to_f32(kh[(int64_t)tt * D + t]) : to_f32(vh[(int64_t)tt * D + (t - D)]); };
  float nx = ld(0), na = ah[0], nb = bth[0];
  for (int c = 0; c < nc; ++c) {
#pragma unroll
    for (int i = 0; i < C::RPT; ++i) ck[((int64_t)c * D + r0 + i) * D + j] = carry[i];
    for (int tt = c * CHUNK; tt < (c + 1) * CHUNK; ++tt) {
      float* vec = lds_f + C::OFF_VEC + (tt & 1) * 4 * D;
      float* part = lds_f + C::OFF_PART + (tt & 1) * 4 * D;
      const float cur = nx, al = na, be = nb;
      if (tt + 1 < L) {
        nx = ld(tt + 1);
        na = ah[tt + 1];
        nb = bth[tt + 1];
      }
      vec[t] = cur;
      gdn_fwd_token<D>(S, vec, part, j, hf, al, be);
    }
    const bool lin = rt[c] == kRouteLinear;
#pragma unroll
    for (int i = 0; i < C::RPT; ++i) {
      if (lin) carry[i] = S[i];
      else S[i] = carry[i];
    }
  }
}

template <typename T, int D>
__global__ void __launch_bounds__(2 * D) k_gdn_bwd(const T* __restrict__ q, const T* __restrict__ k,
                                                   const T* __restrict__ v, const float* __restrict__ alpha,
                                                   const float* __restrict__ beta, const int32_t* __restrict__ route,
                                                   const float* __restrict__ d_o, const float* __restrict__ dS_final,
                                                   const float* __restrict__ ckpt, float* __restrict__ scratch,
                                                   float* __restrict__ dq, float* __restrict__ dk,
                                                   float* __restrict__ dv, float* __restrict__ dalpha,
                                                   float* __restrict__ dbeta, float* __restrict__ dS_init, int H,
                                                   int L, int G) {
  using C = GdnBwdCfg<D>;
  extern __shared__ float lds_f[];
  float* xq = lds_f + C::OFF_XQ;
  float* xk = lds_f + C::OFF_XK;
  float* red = lds_f + C::OFF_RED;
  const int nc = L / CHUNK;
  const int bh = bid_x(), b = bh / H, h = bh % H;
  const int grp = (G == 1) ? 0 : h;
  const int32_t* rt = route + ((int64_t)b * G + grp) * nc;
  const int t = tid_x(), j = t % D, hf = t / D, r0 = hf * C::RPT;
  const int lane = lane_id(), wv = wave_id();
  const int64_t tok0 = (int64_t)bh * L;
  const T* qh = q + tok0 * D;
  const T* kh = k + tok0 * D;
  const T* vh = v + tok0 * D;
  const float* doh = d_o + tok0 * D;
  const float* ah = alpha + tok0;
  const float* bth = beta + tok0;
  const float* ck = ckpt + (int64_t)bh * nc * D * D;
  float* sc = scratch + (int64_t)bh * CHUNK * D * D;  // S_{t-1} of the chunk's tokens (own elements only)

  float Gc[C::RPT];  // gradient of the carried state after the current chunk
#pragma unroll
  for (int i = 0; i < C::RPT; ++i) Gc[i] = dS_final ? dS_final[((int64_t)bh * D + r0 + i) * D + j] : 0.f;

  for (int c = nc - 1; c >= 0; --c) {
    const int c0 = c * CHUNK;
    // recompute the chunk's states: slot s holds the state before token c0 + s
    float S[C::RPT];
#pragma unroll
    for (int i = 0; i < C::RPT; ++i) S[i] = ck[((int64_t)c * D + r0 + i) * D + j];
    auto ldf = [&](int tt) { return t < D ? to_f32(kh[(int64_t)tt * D + t]) : to_f32(vh[(int64_t)tt * D + (t - D)]); };
    float nx = ldf(c0), na = ah[c0], nb = bth[c0];
    for (int s = 0; s < CHUNK; ++s) {
      const int tt = c0 + s;
#pragma unroll
      for (int i = 0; i < C::RPT; ++i) sc[((int64_t)s * D + r0 + i) * D + j] = S[i];
      if (s == CHUNK - 1) break;  // the chunk's end state is not needed
      float* vec = lds_f + C::OFF_VEC + (tt & 1) * 4 * D;
      float* part = lds_f + C::OFF_PART + (tt & 1) * 4 * D;
      const float cur = nx, al = na, be = nb;
      nx = ldf(tt + 1);  // tt + 1 <= c0 + 63: inside the chunk
      na = ah[tt + 1];
      nb = bth[tt + 1];
      vec[t] = cur;
      gdn_fwd_token<D>(S, vec, part, j, hf, al, be);
    }
    __syncthreads();  // every read of the recompute's buffers is done
    const bool lin = rt[c] == kRouteLinear;
    float Gm[C::RPT];
#pragma unroll
    for (int i = 0; i < C::RPT; ++i) Gm[i] = lin ? Gc[i] : 0.f;
    // this thread's two staged values (k and q, or v and d_o) and the decays,
    // loaded a token ahead (the sweep runs backward)
    auto ld2 = [&](int tt, float& x0, float& x1) {
      if (t < D) {
        x0 = to_f32(kh[(int64_t)tt * D + t]);
        x1 = to_f32(qh[(int64_t)tt * D + t]);
      } else {
        x0 = to_f32(vh[(int64_t)tt * D + (t - D)]);
        x1 = doh[(int64_t)tt * D + (t - D)];
      }
    };
    float n0, n1;
    ld2(c0 + CHUNK - 1, n0, n1);
    float nal = ah[c0 + CHUNK - 1], nbe = bth[c0 + CHUNK - 1];
    for (int tt = c0 + CHUNK - 1; tt >= c0; --tt) {
      float* vec = lds_f + C::OFF_VEC + (tt & 1) * 4 * D;  // [k | v | q | do]
      float* part = lds_f + C::OFF_PART + (tt & 1) * 4 * D;  // [a halves | w halves]
      const float x0 = n0, x1 = n1, al = nal, be = nbe;
      if (tt > c0) {
        ld2(tt - 1, n0, n1);
        nal = ah[tt - 1];
        nbe = bth[tt - 1];
      }
      vec[t] = x0;
      vec[2 * D + t] = x1;  // q at 2D + t (t < D); d_o at 3D + (t - D) = 2D + t (t >= D)
      __syncthreads();  // vectors staged
      float Sp[C::RPT];
#pragma unroll
      for (int i = 0; i < C::RPT; ++i) Sp[i] = sc[((int64_t)(tt - c0) * D + r0 + i) * D + j];
      const float doj = vec[3 * D + j], vj = vec[D + j];
      float pa[4] = {0.f, 0.f, 0.f, 0.f}, pw[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < C::RPT; ++i) {
        const float ki = vec[r0 + i];
        Gm[i] += vec[2 * D + r0 + i] * doj;  // o_t = S_t^T q_t
        pa[i & 3] += Sp[i] * ki;
        pw[i & 3] += Gm[i] * ki;
      }
      part[hf * D + j] = (pa[0] + pa[1]) + (pa[2] + pa[3]);
      part[2 * D + hf * D + j] = (pw[0] + pw[1]) + (pw[2] + pw[3]);
      __syncthreads();  // column-sum halves exchanged
      const float a = part[j] + part[D + j];
      const float w = part[2 * D + j] + part[3 * D + j];
      const float cv = be * vj - al * be * a, cw = al * be * w;
      float pal = 0.f;
#pragma unroll
      for (int i = 0; i < C::RPT; ++i) {
        const float ki = vec[r0 + i];
        const float erased = Sp[i] - be * ki * a;
        xq[(r0 + i) * C::XP + j] = (al * erased + be * ki * vj) * doj;  // S_t do
        xk[(r0 + i) * C::XP + j] = Gm[i] * cv - cw * Sp[i];
        pal += Gm[i] * erased;
        Gm[i] = al * (Gm[i] - be * ki * w);  // the gradient of S_{t-1}
      }
      float pbe = (hf == 0) ? w * (vj - al * a) : 0.f;
      pal = wave_sum64(pal);
      pbe = wave_sum64(pbe);
      if (lane == 0) {
        red[2 * wv] = pal;
        red[2 * wv + 1] = pbe;
      }
      if (hf == 0) dv[((int64_t)tt) * D + tok0 * D + j] = be * w;
      __syncthreads();  // row-sum arrays and scalar partials written
      {
        const float* X = (t < D) ? xq : xk;
        const int r = t % D;
        float s4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
        for (int jj = 0; jj < D; ++jj) s4[jj & 3] += X[r * C::XP + jj];
        ((t < D) ? dq : dk)[(tok0 + tt) * D + r] = (s4[0] + s4[1]) + (s4[2] + s4[3]);
      }
      if (t == 0) {
        float sa = 0.f, sb = 0.f;
#pragma unroll
        for (int x = 0; x < C::NT / 64; ++x) {
          sa += red[2 * x];
          sb += red[2 * x + 1];
        }
        dalpha[tok0 + tt] = sa;
        dbeta[tok0 + tt] = sb;
      }
    }
#pragma unroll
    for (int i = 0; i < C::RPT; ++i) Gc[i] = Gm[i] + (lin ? 0.f : Gc[i]);
  }
  if (dS_init) {
#pragma unroll
    for (int i = 0; i < C::RPT; ++i) dS_init[((int64_t)bh * D + r0 + i) * D + j] = Gc[i];
  }
}

template <typename T, int D>
hipError_t launch_gdn_backward(const T* q, const T* k, const T* v, const float* alpha, const float* beta,
                               const int32_t* route, const float* S_init, const float* d_o, const float* dS_final,
                               float* dq, float* dk, float* dv, float* dalpha, float* dbeta, float* dS_init,
                               void* ws, int B, int H, int L, int G, hipStream_t st) {
  using C = GdnBwdCfg<D>;
  static bool attr = false;
  if (!attr) {
    hipError_t e = hipFuncSetAttribute((const void*)k_gdn_bwd<T, D>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       C::LDS_FLOATS * 4);
    if (e != hipSuccess) return e;
    e = hipFuncSetAttribute((const void*)k_gdn_bwd_ckpt<T, D>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            C::CKPT_LDS_FLOATS * 4);
    if (e != hipSuccess) return e;
    attr = true;
  }
  const int nc = L / CHUNK;
  float* ckpt = (float*)ws;
  float* scratch = ckpt + (size_t)B * H * nc * D * D;
  hipLaunchKernelGGL((k_gdn_bwd_ckpt<T, D>), dim3(B * H), dim3(2 * D), C::CKPT_LDS_FLOATS * 4, st, k, v, alpha,
                     beta, route, S_init, ckpt, H, L, G);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_gdn_bwd<T, D>), dim3(B * H), dim3(2 * D), C::LDS_FLOATS * 4, st, q, k, v, alpha, beta,
                     route, d_o, dS_final, ckpt, scratch, dq, dk, dv, dalpha, dbeta, dS_init, H, L, G);
  return hipGetLastError();
}

#define INST(T, D)                                                                                                \
  template hipError_t launch_gdn_backward<T, D>(const T*, const T*, const T*, const float*, const float*,         \
                                                const int32_t*, const float*, const float*, const float*, float*, \
                                                float*, float*, float*, float*, float*, void*, int, int, int, int, \
                                                hipStream_t);
INST(float, 64)
INST(float, 128)
INST(bf16, 64)
INST(bf16, 128)
#undef INST

}  // namespace natsl
