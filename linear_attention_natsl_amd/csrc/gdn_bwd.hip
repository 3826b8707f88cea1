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
// The columns of S (and of G) evolve independently, so each head's CW-column
// groups (4 at D = 128, 8 at D = 64) run in workgroups of their own: one wave
// each.  Lane (jl, rg) holds the RPT = D CW / 64 rows rg RPT .. of column
// CW cg + jl, so the column sums (S^T k, G^T k) stay in registers (DPP rotates
// and two row swaps) and a token needs no barrier.  The row sums (dq, dk) are
// reduced over the CW lanes of a row group by a reduce-scatter that leaves each lane a contiguous run of
// rows (one vector store per token); they and the scalar gradients (dalpha,
// dbeta) are per-group partials, added over the groups in a fixed order by a
// last kernel (so the result does not depend on scheduling).  Launches:
//   k_gdn_bwd_ckpt    the forward, storing every chunk's starting (carried) state
//   k_gdn_bwd         chunks in reverse: recompute the chunk's per-token states
//                     into a scratch slot, then sweep its tokens backward
//   k_gdn_bwd_reduce  dq, dk, dalpha, dbeta from the groups' partials
// Each lane reads its own rows of k and q and its column of v and d_o from
// global memory a few tokens ahead through a ring of registers (the sweep
// reads its scratch states the same way); alpha and beta come from one load
// per chunk (lane s holds token s) and a lane broadcast.  The scratch holds
// each lane's rows contiguously, moved as 16-byte vectors.  This is the plain
// per-token form (the chunkwise form on MFMA is not built).
#include "common.hpp"
#include "kernels.hpp"

namespace natsl {

constexpr int kRouteLinear = 1;  // route id of the linear (Gated DeltaNet) operation

template <int D>
struct GdnBwdCfg {
  static constexpr int CW = D == 128 ? 4 : 8;  // state columns per workgroup (a lane's rows fill 16-byte words)
  static constexpr int NCG = D / CW;       // column groups (workgroups) per head
  static constexpr int NT = 64;            // one wave: CW columns x 64 / CW row groups
  static constexpr int RPT = D * CW / NT;  // state rows per thread
  static constexpr int PF = 16;            // forward tokens of inputs in flight (ring depth)
  static constexpr int PFB = 8;            // the same for the backward sweep (inputs and S_{t-1})
  static_assert((CW == 4 || CW == 8) && RPT % 8 == 0 && CHUNK % PF == 0 && CHUNK % PFB == 0,
                "4 or 8 columns, whole row vectors");
};

size_t gdn_bwd_ws_bytes(int B, int H, int L, int D) {
  const size_t nc = (size_t)L / CHUNK, ntok = (size_t)B * H * L, ncg = (size_t)(D == 128 ? GdnBwdCfg<128>::NCG : GdnBwdCfg<64>::NCG);
  const size_t floats = (size_t)B * H * (nc + CHUNK) * D * D  // chunk-start states, chunk token states
                        + 2 * ntok * ncg * D                  // dq, dk partials
                        + 2 * ntok * ncg                      // dalpha, dbeta partials
                        + (size_t)B * H * ncg * nc;           // linear-gate partials
  return (floats * 4 + 255) / 256 * 256;
}

// sum over the wave's row groups of a per-thread partial for the thread's
// column (the lanes l + CW i of each 16-lane row by DPP rotates, the 4 rows by
// row swaps); every lane receives its column's total
template <int CW>
__device__ __forceinline__ float col_sum(float x) {
  if (CW == 4) x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x124, 0xF, 0xF, true));  // row_ror 4
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x128, 0xF, 0xF, true));  // row_ror 8
  return group4_sum(x);
}

// One reduce-scatter step over lane pairs given by a DPP pattern: of the N
// values, the lane keeps the lower half (keep_lo) or the upper half, adds the
// partner's copy of that half, and leaves the result in v[0 .. N/2).
template <int N, int CTRL>
__device__ __forceinline__ void rs_step(float* v, bool keep_lo) {
#pragma unroll
  for (int k = 0; k < N / 2; ++k) {
    const float send = keep_lo ? v[k + N / 2] : v[k];
    const float keep = keep_lo ? v[k] : v[k + N / 2];
    v[k] = keep + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(send), CTRL, 0xF, 0xF, true));
  }
}
// Sum of each of the N values over the CW lanes of a row group (lanes jl =
// 0..CW-1, CW-aligned); lane jl is left with the sums of values jl N/CW ..
// (jl + 1) N/CW - 1 in v[0 .. N/CW).  The pairings are l <-> 7 - l (CW = 8),
// l <-> l ^ 2, l <-> l ^ 1, which together span the CW lanes.
template <int CW, int N>
__device__ __forceinline__ void group_reduce_scatter(float* v, int jl) {
  static_assert(N % CW == 0, "whole values per lane");
  if constexpr (CW == 8) {
    rs_step<N, 0x141>(v, (jl & 4) == 0);     // row_half_mirror
    rs_step<N / 2, 0x4E>(v, (jl & 2) == 0);  // quad_perm 2,3,0,1
    rs_step<N / 4, 0xB1>(v, (jl & 1) == 0);  // quad_perm 1,0,3,2
  } else {
    rs_step<N, 0x4E>(v, (jl & 2) == 0);
    rs_step<N / 2, 0xB1>(v, (jl & 1) == 0);
  }
}

// alpha or beta of token c0 + s, from the chunk's values held one per lane
__device__ __forceinline__ float lane_bcast(float x, int s) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), s));
}

// A token's inputs as one lane needs them: k (and q) at its RPT rows, v (and
// d_o) at its column, kept as loaded (raw 16-byte words) so that a load in
// the ring is not waited for until the token is reached; widened by tok_f32.
template <typename T, int RPT>
struct TokRaw {
  static constexpr int NW = RPT * (int)sizeof(T) / 16;  // 16-byte words of the lane's rows
  uint4 k[NW], q[NW];
  T v;
  float d_o;
};
template <int RPT>
struct TokIn {
  float k[RPT], q[RPT];
  float v, d_o;
};
template <typename T, int D, bool BWD>
__device__ __forceinline__ void load_tok(TokRaw<T, GdnBwdCfg<D>::RPT>& x, const T* kh, const T* qh, const T* vh,
                                         const float* doh, int tt, int r0, int j) {
  constexpr int NW = TokRaw<T, GdnBwdCfg<D>::RPT>::NW;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    x.k[w] = *(const uint4*)(kh + (int64_t)tt * D + r0 + w * (16 / (int)sizeof(T)));
    if (BWD) x.q[w] = *(const uint4*)(qh + (int64_t)tt * D + r0 + w * (16 / (int)sizeof(T)));
  }
  x.v = vh[(int64_t)tt * D + j];
  x.d_o = BWD ? doh[(int64_t)tt * D + j] : 0.f;
}
// element i of a run of raw 16-byte words holding T values
template <typename T>
__device__ __forceinline__ float raw_f32(const uint4* w, int i) {
  constexpr int E = 16 / (int)sizeof(T);  // elements per word
  const uint4 x = w[i / E];
  const int c = (i % E) * (int)sizeof(T) / 4;  // 32-bit component
  const uint32_t u = c == 0 ? x.x : c == 1 ? x.y : c == 2 ? x.z : x.w;
  if constexpr (sizeof(T) == 2) return __uint_as_float((i & 1) ? (u & 0xffff0000u) : (u << 16));  // bf16 -> fp32
  else return __uint_as_float(u);
}
template <typename T, int RPT, bool BWD>
__device__ __forceinline__ TokIn<RPT> tok_f32(const TokRaw<T, RPT>& r) {
  TokIn<RPT> x;
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    x.k[i] = raw_f32<T>(r.k, i);
    x.q[i] = BWD ? raw_f32<T>(r.q, i) : 0.f;
  }
  x.v = to_f32(r.v);
  x.d_o = r.d_o;
  return x;
}

// the thread's RPT state elements, contiguous in the scratch (16-byte aligned)
template <int RPT>
__device__ __forceinline__ void store_state(float* p, const float (&S)[RPT]) {
#pragma unroll
  for (int h = 0; h < RPT; h += 4) *(float4*)(p + h) = make_float4(S[h], S[h + 1], S[h + 2], S[h + 3]);
}
template <int RPT>
__device__ __forceinline__ void load_state(float (&S)[RPT], const float* p) {
#pragma unroll
  for (int h = 0; h < RPT; h += 4) {
    const float4 x = *(const float4*)(p + h);
    S[h] = x.x;
    S[h + 1] = x.y;
    S[h + 2] = x.z;
    S[h + 3] = x.w;
  }
}

// one forward token on the thread's elements: a = S^T k (column sums), then
// S <- al (S - be k a^T) + be k v^T
template <int D>
__device__ __forceinline__ void gdn_fwd_token(float (&S)[GdnBwdCfg<D>::RPT], const TokIn<GdnBwdCfg<D>::RPT>& x,
                                              float al, float be) {
  constexpr int RPT = GdnBwdCfg<D>::RPT;
  float p4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < RPT; ++i) p4[i & 3] += S[i] * x.k[i];
  const float a = col_sum<GdnBwdCfg<D>::CW>((p4[0] + p4[1]) + (p4[2] + p4[3]));
#pragma unroll
  for (int i = 0; i < RPT; ++i) S[i] = al * (S[i] - be * x.k[i] * a) + be * x.k[i] * x.v;
}

template <typename T, int D>
__global__ void __launch_bounds__(64) k_gdn_bwd_ckpt(const T* __restrict__ k, const T* __restrict__ v,
                                                      const float* __restrict__ alpha, const float* __restrict__ beta,
                                                      const int32_t* __restrict__ route,
                                                      const float* __restrict__ S_init, float* __restrict__ ckpt,
                                                      int H, int L, int G) {
  using C = GdnBwdCfg<D>;
  const int nc = L / CHUNK;
  const int bh = bid_x() / C::NCG, cg = bid_x() % C::NCG, b = bh / H, h = bh % H;
  const int grp = (G == 1) ? 0 : h;
  const int32_t* rt = route + ((int64_t)b * G + grp) * nc;
  const int t = tid_x(), jl = t % C::CW, rg = t / C::CW, lane = t;
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
  TokRaw<T, C::RPT> ring[C::PF];  // slot u: the token tt with tt % PF == u, PF tokens ahead
#pragma unroll
  for (int u = 0; u < C::PF; ++u) load_tok<T, D, false>(ring[u], kh, kh, vh, nullptr, u, r0, j);  // L >= 64
  for (int c = 0; c < nc; ++c) {
    const float al_c = ah[c * CHUNK + lane], be_c = bth[c * CHUNK + lane];  // lane s: token c0 + s
#pragma unroll
    for (int i = 0; i < C::RPT; ++i) ck[((int64_t)c * D + r0 + i) * D + j] = carry[i];
    for (int s0 = 0; s0 < CHUNK; s0 += C::PF) {
#pragma unroll
      for (int u = 0; u < C::PF; ++u) {
        const int s = s0 + u, tt = c * CHUNK + s;
        const TokIn<C::RPT> cur = tok_f32<T, C::RPT, false>(ring[u]);
        // (unconditional, clamped to the last token: a branch around the load
        // would make the compiler wait for it at the join)
        load_tok<T, D, false>(ring[u], kh, kh, vh, nullptr, min(tt + C::PF, L - 1), r0, j);
        gdn_fwd_token<D>(S, cur, lane_bcast(al_c, s), lane_bcast(be_c, s));
      }
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
__global__ void __launch_bounds__(64) k_gdn_bwd(const T* __restrict__ q, const T* __restrict__ k,
                                                 const T* __restrict__ v, const float* __restrict__ alpha,
                                                 const float* __restrict__ beta, const int32_t* __restrict__ route,
                                                 const float* __restrict__ d_o, const float* __restrict__ dS_final,
                                                 const float* __restrict__ ckpt, float* __restrict__ scratch,
                                                 float* __restrict__ dq_p, float* __restrict__ dk_p,
                                                 float* __restrict__ dab_p, float* __restrict__ dv,
                                                 float* __restrict__ dS_init, float* __restrict__ gate_p, int H,
                                                 int L, int G) {
  using C = GdnBwdCfg<D>;
  constexpr int NV = 2 * C::RPT;  // row-sum values per thread and token: dq, dk at its rows
  constexpr int VPL = NV / C::CW;  // of which each lane stores VPL after the row-group reduction
  const int nc = L / CHUNK;
  const int bh = bid_x() / C::NCG, cg = bid_x() % C::NCG, b = bh / H, h = bh % H;
  const int grp = (G == 1) ? 0 : h;
  const int32_t* rt = route + ((int64_t)b * G + grp) * nc;
  const int t = tid_x(), jl = t % C::CW, rg = t / C::CW, lane = t;
  const int j = C::CW * cg + jl, r0 = rg * C::RPT;
  // after the row-group reduction lane jl holds values jl VPL ..: dq (the lower half of the lanes) or dk
  // at rows r0 + (jl % (CW / 2)) VPL ..
  float* const dqk_p = (jl < C::CW / 2) ? dq_p : dk_p;
  const int rq0 = r0 + (jl % (C::CW / 2)) * VPL;
  const int64_t tok0 = (int64_t)bh * L;
  const T* qh = q + tok0 * D;
  const T* kh = k + tok0 * D;
  const T* vh = v + tok0 * D;
  const float* doh = d_o + tok0 * D;
  const float* ah = alpha + tok0;
  const float* bth = beta + tok0;
  const float* ck = ckpt + (int64_t)bh * nc * D * D;
  // S_{t-1} of the chunk's tokens: slot s of thread t at (s * 256 + t) * RPT
  float* sc = scratch + (int64_t)bid_x() * CHUNK * D * C::CW + (int64_t)t * C::RPT;

  float Gc[C::RPT];  // gradient of the carried state after the current chunk
#pragma unroll
  for (int i = 0; i < C::RPT; ++i) Gc[i] = dS_final ? dS_final[((int64_t)bh * D + r0 + i) * D + j] : 0.f;

  for (int c = nc - 1; c >= 0; --c) {
    const int c0 = c * CHUNK;
    const float al_c = ah[c0 + lane], be_c = bth[c0 + lane];  // lane s: token c0 + s
    // recompute the chunk's states: slot s holds the state before token c0 + s
    float S[C::RPT];
#pragma unroll
    for (int i = 0; i < C::RPT; ++i) S[i] = ck[((int64_t)c * D + r0 + i) * D + j];
    {
      TokRaw<T, C::RPT> ring[C::PF];  // slot u: the token c0 + s with s % PF == u
#pragma unroll
      for (int u = 0; u < C::PF; ++u) load_tok<T, D, false>(ring[u], kh, kh, vh, nullptr, c0 + u, r0, j);
      for (int s0 = 0; s0 < CHUNK; s0 += C::PF) {
#pragma unroll
        for (int u = 0; u < C::PF; ++u) {
          const int s = s0 + u, tt = c0 + s;
          store_state<C::RPT>(sc + (int64_t)s * C::NT * C::RPT, S);
          // (token c0 + 63 runs too, without a branch; its end state is not used)
          const TokIn<C::RPT> cur = tok_f32<T, C::RPT, false>(ring[u]);
          load_tok<T, D, false>(ring[u], kh, kh, vh, nullptr, c0 + min(s + C::PF, CHUNK - 1), r0, j);
          gdn_fwd_token<D>(S, cur, lane_bcast(al_c, s), lane_bcast(be_c, s));
        }
      }
    }
    // the linear gate's derivative (the chunk's end state committed as
    // S_start + h (S_end - S_start)): <d loss / d carried state after the
    // chunk, S_end - S_start>, this group's columns; S holds S_end here
    if (gate_p) {
      float pg = 0.f;
#pragma unroll
      for (int i = 0; i < C::RPT; ++i) pg += Gc[i] * (S[i] - ck[((int64_t)c * D + r0 + i) * D + j]);
      pg = wave_sum64(pg);
      if (lane == 0) gate_p[(int64_t)bid_x() * nc + c] = pg;
    }
    // (this thread's scratch stores complete before the sweep reads them back)
    __syncthreads();
    const bool lin = rt[c] == kRouteLinear;
    float Gm[C::RPT];
#pragma unroll
    for (int i = 0; i < C::RPT; ++i) Gm[i] = lin ? Gc[i] : 0.f;
    // inputs and S_{t-1}, PFB tokens ahead; the sweep runs backward: step r is
    // token c0 + 63 - r, in slot r % PFB
    TokRaw<T, C::RPT> ring[C::PFB];
    float ringS[C::PFB][C::RPT];
#pragma unroll
    for (int u = 0; u < C::PFB; ++u) {
      load_tok<T, D, true>(ring[u], kh, qh, vh, doh, c0 + CHUNK - 1 - u, r0, j);
      load_state<C::RPT>(ringS[u], sc + (int64_t)(CHUNK - 1 - u) * C::NT * C::RPT);
    }
    for (int r00 = 0; r00 < CHUNK; r00 += C::PFB) {
#pragma unroll
      for (int u = 0; u < C::PFB; ++u) {
        const int rs = r00 + u, s = CHUNK - 1 - rs, tt = c0 + s;
        const TokIn<C::RPT> x = tok_f32<T, C::RPT, true>(ring[u]);
        float Sp[C::RPT];
#pragma unroll
        for (int i = 0; i < C::RPT; ++i) Sp[i] = ringS[u][i];
        // the token PFB steps on, clamped to the chunk's first (unconditional)
        load_tok<T, D, true>(ring[u], kh, qh, vh, doh, c0 + max(s - C::PFB, 0), r0, j);
        load_state<C::RPT>(ringS[u], sc + (int64_t)max(s - C::PFB, 0) * C::NT * C::RPT);
        float pa[4] = {0.f, 0.f, 0.f, 0.f}, pw[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < C::RPT; ++i) {
          Gm[i] += x.q[i] * x.d_o;  // o_t = S_t^T q_t
          pa[i & 3] += Sp[i] * x.k[i];
          pw[i & 3] += Gm[i] * x.k[i];
        }
        const float a = col_sum<C::CW>((pa[0] + pa[1]) + (pa[2] + pa[3]));
        const float w = col_sum<C::CW>((pw[0] + pw[1]) + (pw[2] + pw[3]));
        const float al = lane_bcast(al_c, s), be = lane_bcast(be_c, s), vj = x.v, doj = x.d_o;
        const float cv = be * vj - al * be * a, cw = al * be * w;
        float pal = 0.f, rv[NV];
#pragma unroll
        for (int i = 0; i < C::RPT; ++i) {
          const float ki = x.k[i];
          const float erased = Sp[i] - be * ki * a;
          rv[i] = (al * erased + be * ki * vj) * doj;  // this column's share of dq = S_t d_o
          rv[C::RPT + i] = Gm[i] * cv - cw * Sp[i];    // and of dk
          pal += Gm[i] * erased;
          Gm[i] = al * (Gm[i] - be * ki * w);  // the gradient of S_{t-1}
        }
        group_reduce_scatter<C::CW, NV>(rv, jl);
        const int64_t tok = tok0 + tt;
        float* dst = dqk_p + (tok * C::NCG + cg) * D + rq0;
        if constexpr (VPL % 4 == 0) {
#pragma unroll
          for (int h = 0; h < VPL; h += 4) *(float4*)(dst + h) = make_float4(rv[h], rv[h + 1], rv[h + 2], rv[h + 3]);
        } else {
#pragma unroll
          for (int h = 0; h < VPL; h += 2) *(float2*)(dst + h) = make_float2(rv[h], rv[h + 1]);
        }
        float pbe = (rg == 0) ? w * (vj - al * a) : 0.f;
        pal = wave_sum64(pal);
        pbe = wave_sum64(pbe);
        if (lane < 2) dab_p[(tok * C::NCG + cg) * 2 + lane] = lane ? pbe : pal;  // this group's partials
        if (rg == 0) dv[tok * D + j] = be * w;
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

// dq, dk, dalpha, dbeta: the NCG groups' partials added in group order
// (dalpha and dbeta interleaved).  Threads [0, ntok D/4) take 4 consecutive
// rows of one token's dq and dk (16-byte loads from the workspace; scalar
// stores, the outputs carrying no alignment promise); threads
// [ntok D/4, ntok D/4 + ntok) take one token's dalpha and dbeta.
template <int D>
__global__ void __launch_bounds__(256) k_gdn_bwd_reduce(const float* __restrict__ dq_p, const float* __restrict__ dk_p,
                                                        const float* __restrict__ dab_p, float* __restrict__ dq,
                                                        float* __restrict__ dk, float* __restrict__ dalpha,
                                                        float* __restrict__ dbeta, int64_t ntok) {
  constexpr int NCG = GdnBwdCfg<D>::NCG;
  static_assert(NCG % 2 == 0 && D % 4 == 0, "whole 16-byte partial vectors");
  const int64_t gid = (int64_t)bid_x() * 256 + tid_x();
  const int64_t nvec = ntok * (D / 4);
  if (gid < nvec) {
    const int64_t tok = gid / (D / 4);
    const int i = (int)(gid % (D / 4)) * 4;
    float sq[4] = {0.f, 0.f, 0.f, 0.f}, sk[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int cg = 0; cg < NCG; ++cg) {
      const float4 a = *(const float4*)(dq_p + (tok * NCG + cg) * D + i);
      const float4 c = *(const float4*)(dk_p + (tok * NCG + cg) * D + i);
      sq[0] += a.x; sq[1] += a.y; sq[2] += a.z; sq[3] += a.w;
      sk[0] += c.x; sk[1] += c.y; sk[2] += c.z; sk[3] += c.w;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      dq[tok * D + i + r] = sq[r];
      dk[tok * D + i + r] = sk[r];
    }
  } else if (gid < nvec + ntok) {
    const int64_t tok = gid - nvec;
    float sa = 0.f, sb = 0.f;
#pragma unroll
    for (int x = 0; x < NCG; x += 2) {  // groups x and x + 1
      const float4 a = *(const float4*)(dab_p + (tok * NCG + x) * 2);
      sa += a.x;
      sb += a.y;
      sa += a.z;
      sb += a.w;
    }
    dalpha[tok] = sa;
    dbeta[tok] = sb;
  }
}

// the linear gates' derivative: the column groups' partials added in order
__global__ void __launch_bounds__(256) k_gdn_bwd_gate_reduce(const float* __restrict__ gate_p,
                                                             float* __restrict__ dgate, int ncg, int nc, int64_t n) {
  const int64_t i = (int64_t)bid_x() * 256 + tid_x();  // (bh, c)
  if (i >= n) return;
  const int64_t bh = i / nc, c = i % nc;
  float s = 0.f;
  for (int cg = 0; cg < ncg; ++cg) s += gate_p[(bh * ncg + cg) * nc + c];
  dgate[i] = s;
}

template <typename T, int D>
hipError_t launch_gdn_backward(const T* q, const T* k, const T* v, const float* alpha, const float* beta,
                               const int32_t* route, const float* S_init, const float* d_o, const float* dS_final,
                               float* dq, float* dk, float* dv, float* dalpha, float* dbeta, float* dS_init,
                               float* dgate, void* ws, int B, int H, int L, int G, hipStream_t st) {
  using C = GdnBwdCfg<D>;
  const int nc = L / CHUNK;
  const int64_t ntok = (int64_t)B * H * L;
  float* ckpt = (float*)ws;
  float* scratch = ckpt + (size_t)B * H * nc * D * D;
  float* dq_p = scratch + (size_t)B * H * CHUNK * D * D;
  float* dk_p = dq_p + (size_t)ntok * C::NCG * D;
  float* dab_p = dk_p + (size_t)ntok * C::NCG * D;  // ntok x NCG x (dalpha, dbeta)
  float* gate_p = dab_p + (size_t)ntok * C::NCG * 2;  // [B H][NCG][Nc]
  const size_t lds = 0;
  const unsigned grid = (unsigned)(B * H * C::NCG);
  hipLaunchKernelGGL((k_gdn_bwd_ckpt<T, D>), dim3(grid), dim3(C::NT), lds, st, k, v, alpha, beta, route, S_init,
                     ckpt, H, L, G);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_gdn_bwd<T, D>), dim3(grid), dim3(C::NT), lds, st, q, k, v, alpha, beta, route, d_o,
                     dS_final, ckpt, scratch, dq_p, dk_p, dab_p, dv, dS_init, dgate ? gate_p : nullptr, H, L, G);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (dgate) {
    const int64_t n = (int64_t)B * H * nc;
    hipLaunchKernelGGL(k_gdn_bwd_gate_reduce, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, gate_p, dgate,
                       C::NCG, nc, n);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const int64_t threads = ntok * (D / 4) + ntok;
  hipLaunchKernelGGL((k_gdn_bwd_reduce<D>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st, dq_p, dk_p,
                     dab_p, dq, dk, dalpha, dbeta, ntok);
  return hipGetLastError();
}

#define INST(T, D)                                                                                                \
  template hipError_t launch_gdn_backward<T, D>(const T*, const T*, const T*, const float*, const float*,         \
                                                const int32_t*, const float*, const float*, const float*, float*, \
                                                float*, float*, float*, float*, float*, float*, void*, int, int, int, int, \
                                                hipStream_t);
INST(float, 64)
INST(float, 128)
INST(bf16, 64)
INST(bf16, 128)
#undef INST

}  // namespace natsl
