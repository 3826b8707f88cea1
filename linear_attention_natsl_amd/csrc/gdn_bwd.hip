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
// The columns of S (and of G) evolve independently, so each head's 16-column
// groups run in workgroups of their own (D / 16 per head).  Thread (jl, rg)
// holds rows rg D/16 .. of column 16 cg + jl: the column sums (S^T k, G^T k)
// are a row-swap sum over the wave's 4 lane groups plus one LDS exchange
// across the 4 waves; the row sums (dq, dk) and the scalar gradients (dalpha,
// dbeta) are per-group partials, added over the groups in a fixed order by a
// last kernel (so the result does not depend on scheduling).  Launches:
//   k_gdn_bwd_ckpt    the forward, storing every chunk's starting (carried) state
//   k_gdn_bwd         chunks in reverse: recompute the chunk's per-token states
//                     into a scratch slot, then sweep its tokens backward
//   k_gdn_bwd_reduce  dq, dk, dalpha, dbeta from the groups' partials
// Each thread reads its own rows of k and q and its column of v and d_o from
// global memory (a token ahead), so a token needs one barrier, for the
// column-sum exchange.  This is the plain per-token form (the chunkwise form
// on MFMA is not built).
#include "common.hpp"
#include "kernels.hpp"

namespace natsl {

constexpr int kRouteLinear = 1;  // route id of the linear (Gated DeltaNet) operation

template <int D>
struct GdnBwdCfg {
  static constexpr int CW = 16;       // state columns per workgroup
  static constexpr int NCG = D / CW;  // column groups (workgroups) per head
  static constexpr int NT = 256;      // 16 columns x 16 row groups
  static constexpr int RPT = D / 16;  // state rows per thread
  // LDS: part[2][2][4][CW] floats (per-wave column sums of a and w, by token
  // parity); every other per-token value reaches the threads from global
  // memory directly, so a token needs one barrier (the column-sum exchange)
  static constexpr int LDS_FLOATS = 2 * 2 * 4 * CW;
};

size_t gdn_bwd_ws_bytes(int B, int H, int L, int D) {
  const size_t nc = (size_t)L / CHUNK, ntok = (size_t)B * H * L, ncg = (size_t)D / 16;
  const size_t floats = (size_t)B * H * (nc + CHUNK) * D * D  // chunk-start states, chunk token states
                        + 2 * ntok * ncg * D                  // dq, dk partials
                        + 2 * ntok * ncg * 4;                 // dalpha, dbeta partials (per wave)
  return (floats * 4 + 255) / 256 * 256;
}

// sum over the workgroup's 16 row groups of a per-thread partial for the
// thread's column: the wave's 4 lane groups by row swaps, the 4 waves through
// LDS (part[4][16]); the caller's barrier separates the write and the reads
__device__ __forceinline__ void col_part(float x, float* part, int jl, int wv, int lane) {
  x = group4_sum(x);
  if (lane < 16) part[wv * 16 + jl] = x;
}
__device__ __forceinline__ float col_total(const float* part, int jl) {
  return (part[jl] + part[16 + jl]) + (part[32 + jl] + part[48 + jl]);
}

// A token's inputs as one thread needs them: k (and q) at its RPT rows, v
// (and d_o) at its column, the decays
template <int RPT>
struct TokIn {
  float k[RPT], q[RPT];
  float v, d_o, al, be;
};
template <typename T, int D, bool BWD>
__device__ __forceinline__ void load_tok(TokIn<D / 16>& x, const T* kh, const T* qh, const T* vh, const float* doh,
                                         const float* ah, const float* bth, int tt, int r0, int j) {
  constexpr int RPT = D / 16;
  if constexpr (RPT % 8 == 0) {  // whole 8-element vectors of the thread's rows
    float kk[8], qq[8];
#pragma unroll
    for (int h8 = 0; h8 < RPT; h8 += 8) {
      load8f<T>(kh + (int64_t)tt * D + r0 + h8, kk);
#pragma unroll
      for (int i = 0; i < 8; ++i) x.k[h8 + i] = kk[i];
      if (BWD) {
        load8f<T>(qh + (int64_t)tt * D + r0 + h8, qq);
#pragma unroll
        for (int i = 0; i < 8; ++i) x.q[h8 + i] = qq[i];
      }
    }
  } else {  // fewer rows than a vector: exactly the thread's rows
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      x.k[i] = to_f32(kh[(int64_t)tt * D + r0 + i]);
      if (BWD) x.q[i] = to_f32(qh[(int64_t)tt * D + r0 + i]);
    }
  }
  x.v = to_f32(vh[(int64_t)tt * D + j]);
  x.d_o = BWD ? doh[(int64_t)tt * D + j] : 0.f;
  x.al = ah[tt];
  x.be = bth[tt];
}

// One forward token on the thread's rows of its column:
//   S <- a (S - b k (k^T S)) + b k v^T
// part: this token's exchange buffer [4][16] (alternating by token parity)
template <int D>
__device__ __forceinline__ void gdn_fwd_token(float (&S)[D / 16], const TokIn<D / 16>& x, float* part, int jl, int wv,
                                              int lane) {
  constexpr int RPT = D / 16;
  float p4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < RPT; ++i) p4[i & 3] += S[i] * x.k[i];
  col_part((p4[0] + p4[1]) + (p4[2] + p4[3]), part, jl, wv, lane);
  __syncthreads();  // column sums exchanged
  const float a = col_total(part, jl);
#pragma unroll
  for (int i = 0; i < RPT; ++i) S[i] = x.al * (S[i] - x.be * x.k[i] * a) + x.be * x.k[i] * x.v;
}

template <typename T, int D>
__global__ void __launch_bounds__(256) k_gdn_bwd_ckpt(const T* __restrict__ k, const T* __restrict__ v,
                                                      const float* __restrict__ alpha, const float* __restrict__ beta,
                                                      const int32_t* __restrict__ route,
                                                      const float* __restrict__ S_init, float* __restrict__ ckpt,
                                                      int H, int L, int G) {
  using C = GdnBwdCfg<D>;
  extern __shared__ float lds_f[];
  const int nc = L / CHUNK;
  const int bh = bid_x() / C::NCG, cg = bid_x() % C::NCG, b = bh / H, h = bh % H;
  const int grp = (G == 1) ? 0 : h;
  const int32_t* rt = route + ((int64_t)b * G + grp) * nc;
  const int t = tid_x(), jl = t & 15, rg = t >> 4, wv = wave_id(), lane = lane_id();
  const int j = C::CW * cg + jl, r0 = rg * C::RPT;
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
  TokIn<C::RPT> nx;  // the next token's inputs, loaded a token ahead
  load_tok<T, D, false>(nx, kh, kh, vh, nullptr, ah, bth, 0, r0, j);
  for (int c = 0; c < nc; ++c) {
#pragma unroll
    for (int i = 0; i < C::RPT; ++i) ck[((int64_t)c * D + r0 + i) * D + j] = carry[i];
    for (int tt = c * CHUNK; tt < (c + 1) * CHUNK; ++tt) {
      const TokIn<C::RPT> cur = nx;
      if (tt + 1 < L) load_tok<T, D, false>(nx, kh, kh, vh, nullptr, ah, bth, tt + 1, r0, j);
      gdn_fwd_token<D>(S, cur, lds_f + (tt & 1) * 4 * C::CW, jl, wv, lane);
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
__global__ void __launch_bounds__(256) k_gdn_bwd(const T* __restrict__ q, const T* __restrict__ k,
                                                 const T* __restrict__ v, const float* __restrict__ alpha,
                                                 const float* __restrict__ beta, const int32_t* __restrict__ route,
                                                 const float* __restrict__ d_o, const float* __restrict__ dS_final,
                                                 const float* __restrict__ ckpt, float* __restrict__ scratch,
                                                 float* __restrict__ dq_p, float* __restrict__ dk_p,
                                                 float* __restrict__ da_p, float* __restrict__ db_p,
                                                 float* __restrict__ dv, float* __restrict__ dS_init, int H, int L,
                                                 int G) {
  using C = GdnBwdCfg<D>;
  extern __shared__ float lds_f[];
  const int nc = L / CHUNK;
  const int bh = bid_x() / C::NCG, cg = bid_x() % C::NCG, b = bh / H, h = bh % H;
  const int grp = (G == 1) ? 0 : h;
  const int32_t* rt = route + ((int64_t)b * G + grp) * nc;
  const int t = tid_x(), jl = t & 15, rg = t >> 4, wv = wave_id(), lane = lane_id();
  const int j = C::CW * cg + jl, r0 = rg * C::RPT;
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
    // the previous chunk's last sweep token read the parity-0 exchange buffer
    // that this chunk's first recompute token writes
    __syncthreads();
    // recompute the chunk's states: slot s holds the state before token c0 + s
    float S[C::RPT];
#pragma unroll
    for (int i = 0; i < C::RPT; ++i) S[i] = ck[((int64_t)c * D + r0 + i) * D + j];
    TokIn<C::RPT> nx;
    load_tok<T, D, false>(nx, kh, kh, vh, nullptr, ah, bth, c0, r0, j);
    for (int s = 0; s < CHUNK; ++s) {
      const int tt = c0 + s;
#pragma unroll
      for (int i = 0; i < C::RPT; ++i) sc[((int64_t)s * D + r0 + i) * D + j] = S[i];
      if (s == CHUNK - 1) break;  // the chunk's end state is not needed
      const TokIn<C::RPT> cur = nx;
      load_tok<T, D, false>(nx, kh, kh, vh, nullptr, ah, bth, tt + 1, r0, j);  // tt + 1 <= c0 + 63
      gdn_fwd_token<D>(S, cur, lds_f + (tt & 1) * 4 * C::CW, jl, wv, lane);
    }
    const bool lin = rt[c] == kRouteLinear;
    float Gm[C::RPT];
#pragma unroll
    for (int i = 0; i < C::RPT; ++i) Gm[i] = lin ? Gc[i] : 0.f;
    // inputs and the thread's elements of S_{t-1}, loaded a token ahead (the
    // sweep runs backward)
    TokIn<C::RPT> nt;
    load_tok<T, D, true>(nt, kh, qh, vh, doh, ah, bth, c0 + CHUNK - 1, r0, j);
    float nS[C::RPT];
#pragma unroll
    for (int i = 0; i < C::RPT; ++i) nS[i] = sc[((int64_t)(CHUNK - 1) * D + r0 + i) * D + j];
    for (int tt = c0 + CHUNK - 1; tt >= c0; --tt) {
      // (the recompute's last exchange buffer was token c0 + 62, parity 0; the
      // sweep's first is token c0 + 63, parity 1, and the parities alternate)
      float* part = lds_f + (tt & 1) * 2 * 4 * C::CW;  // [a: 4 x 16 | w: 4 x 16]
      const TokIn<C::RPT> x = nt;
      float Sp[C::RPT];
#pragma unroll
      for (int i = 0; i < C::RPT; ++i) Sp[i] = nS[i];
      if (tt > c0) {
        load_tok<T, D, true>(nt, kh, qh, vh, doh, ah, bth, tt - 1, r0, j);
#pragma unroll
        for (int i = 0; i < C::RPT; ++i) nS[i] = sc[((int64_t)(tt - 1 - c0) * D + r0 + i) * D + j];
      }
      float pa[4] = {0.f, 0.f, 0.f, 0.f}, pw[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < C::RPT; ++i) {
        Gm[i] += x.q[i] * x.d_o;  // o_t = S_t^T q_t
        pa[i & 3] += Sp[i] * x.k[i];
        pw[i & 3] += Gm[i] * x.k[i];
      }
      col_part((pa[0] + pa[1]) + (pa[2] + pa[3]), part, jl, wv, lane);
      col_part((pw[0] + pw[1]) + (pw[2] + pw[3]), part + 4 * C::CW, jl, wv, lane);
      __syncthreads();  // column sums exchanged
      const float a = col_total(part, jl), w = col_total(part + 4 * C::CW, jl);
      const float al = x.al, be = x.be, vj = x.v, doj = x.d_o;
      const float cv = be * vj - al * be * a, cw = al * be * w;
      float pal = 0.f;
      const int64_t tok = tok0 + tt;
#pragma unroll
      for (int i = 0; i < C::RPT; ++i) {
        const float ki = x.k[i];
        const float erased = Sp[i] - be * ki * a;
        // this group's share of the row sums dq = S_t d_o and dk
        const float rq = dpp_group_sum<16>((al * erased + be * ki * vj) * doj);
        const float rk = dpp_group_sum<16>(Gm[i] * cv - cw * Sp[i]);
        if (jl == 0) {
          dq_p[(tok * C::NCG + cg) * D + r0 + i] = rq;
          dk_p[(tok * C::NCG + cg) * D + r0 + i] = rk;
        }
        pal += Gm[i] * erased;
        Gm[i] = al * (Gm[i] - be * ki * w);  // the gradient of S_{t-1}
      }
      float pbe = (rg == 0) ? w * (vj - al * a) : 0.f;
      pal = wave_sum64(pal);
      pbe = wave_sum64(pbe);
      if (lane == 0) {  // per-wave partials, added by k_gdn_bwd_reduce
        da_p[(tok * C::NCG + cg) * 4 + wv] = pal;
        db_p[(tok * C::NCG + cg) * 4 + wv] = pbe;
      }
      if (rg == 0) dv[tok * D + j] = be * w;
    }
#pragma unroll
    for (int i = 0; i < C::RPT; ++i) Gc[i] = Gm[i] + (lin ? 0.f : Gc[i]);
  }
  if (dS_init) {
#pragma unroll
    for (int i = 0; i < C::RPT; ++i) dS_init[((int64_t)bh * D + r0 + i) * D + j] = Gc[i];
  }
}

// dq, dk, dalpha, dbeta: the column groups' (and waves') partials added in a
// fixed order
template <int D>
__global__ void __launch_bounds__(256) k_gdn_bwd_reduce(const float* __restrict__ dq_p, const float* __restrict__ dk_p,
                                                        const float* __restrict__ da_p, const float* __restrict__ db_p,
                                                        float* __restrict__ dq, float* __restrict__ dk,
                                                        float* __restrict__ dalpha, float* __restrict__ dbeta,
                                                        int64_t ntok) {
  constexpr int NCG = GdnBwdCfg<D>::NCG;
  const int64_t gid = (int64_t)bid_x() * 256 + tid_x();
  const int64_t tok = gid / D;
  const int i = (int)(gid % D);
  if (tok >= ntok) return;
  float sq = 0.f, sk = 0.f;
#pragma unroll
  for (int cg = 0; cg < NCG; ++cg) {
    sq += dq_p[(tok * NCG + cg) * D + i];
    sk += dk_p[(tok * NCG + cg) * D + i];
  }
  dq[tok * D + i] = sq;
  dk[tok * D + i] = sk;
  if (i == 0) {
    float sa = 0.f, sb = 0.f;
#pragma unroll
    for (int x = 0; x < NCG * 4; ++x) {
      sa += da_p[tok * NCG * 4 + x];
      sb += db_p[tok * NCG * 4 + x];
    }
    dalpha[tok] = sa;
    dbeta[tok] = sb;
  }
}

template <typename T, int D>
hipError_t launch_gdn_backward(const T* q, const T* k, const T* v, const float* alpha, const float* beta,
                               const int32_t* route, const float* S_init, const float* d_o, const float* dS_final,
                               float* dq, float* dk, float* dv, float* dalpha, float* dbeta, float* dS_init,
                               void* ws, int B, int H, int L, int G, hipStream_t st) {
  using C = GdnBwdCfg<D>;
  const int nc = L / CHUNK;
  const int64_t ntok = (int64_t)B * H * L;
  float* ckpt = (float*)ws;
  float* scratch = ckpt + (size_t)B * H * nc * D * D;
  float* dq_p = scratch + (size_t)B * H * CHUNK * D * D;
  float* dk_p = dq_p + (size_t)ntok * C::NCG * D;
  float* da_p = dk_p + (size_t)ntok * C::NCG * D;
  float* db_p = da_p + (size_t)ntok * C::NCG * 4;
  const size_t lds = C::LDS_FLOATS * 4;
  const unsigned grid = (unsigned)(B * H * C::NCG);
  hipLaunchKernelGGL((k_gdn_bwd_ckpt<T, D>), dim3(grid), dim3(C::NT), lds, st, k, v, alpha, beta, route, S_init,
                     ckpt, H, L, G);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_gdn_bwd<T, D>), dim3(grid), dim3(C::NT), lds, st, q, k, v, alpha, beta, route, d_o,
                     dS_final, ckpt, scratch, dq_p, dk_p, da_p, db_p, dv, dS_init, H, L, G);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int64_t threads = ntok * D;
  hipLaunchKernelGGL((k_gdn_bwd_reduce<D>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st, dq_p, dk_p,
                     da_p, db_p, dq, dk, dalpha, dbeta, ntok);
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
