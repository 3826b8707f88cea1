// Native Hybrid Attention ("Native Hybrid Attention for Efficient Sequence
// Modeling", section 2 Methodologie, "Unificatie van Intra-layer
// Hybridisatie"): long-term information compressed into m key-value slots by
// a gated linear RNN update, joined with the tokens of a sliding window into
// ONE key-value set, and one softmax attention over that set.
//
// Readings (the page gives no equations): a query t sees the keys of tokens
// t-w+1 .. t (window w, a multiple of 64 here) and the slots; token s enters
// the slots when it leaves the window (before query s + w), per slot i
//   K~[i] <- a_s[i] K~[i] + (1 - a_s[i]) k_s,   V~[i] likewise,
// with the token's gate a_s in [0, 1]^m; slots start at zero and join the
// key set once a token has entered them.
//
// With w = 64 nw, the queries of chunk c take their evictions from chunk
// e = c - nw: query 64 c + j sees the slots after tokens 64 e .. 64 e + j have
// entered.  Four launches:
//   window attention  the softmax kernel in window mode (o_w, lse_w);
//   k_nha_chunk       per chunk e: the slots' change over its 64 tokens,
//                     dK[i] = sum_s a(s..63] (1 - a_s) k_s (and dV), and the
//                     chunk's decay G[i] = prod_s a_s[i];
//   k_nha_scan        chunk-start slot states S_e = G_{e-1} S_{e-1} + d_{e-1},
//                     element by element (one thread per slot entry);
//   k_nha_slots       per query chunk: slot scores
//                       z[j][i] = q_j . K~_j[i] = prod_{r<=j} a_r[i] (q_j . K~_e[i])
//                                + sum_{s<=j} (1 - a_s[i]) prod_{s<r<=j} a_r[i] (q_j . k_s),
//                     one softmax over [slots, window] with the window's lse,
//                     and the slot values rolled forward token by token for
//                     the read-out, merged with o_w.
// Products of gates are taken by running multiplication (no division by
// cumulative products, no logarithms), so gates of exactly 0 or 1 are exact.
#include "common.hpp"
#include "kernels.hpp"

namespace natsl {

// per (b, h, chunk e < ne): the slots' change over the chunk and its decay.
// The weights W[s][i] = (1 - a_s[i]) prod_{s<r<64} a_r[i] come from suffix
// products (one thread per slot); dK = W^T K_e and dV = W^T V_e are matrix-
// core products (W as bf16 hi + lo parts for bf16 io), K_e and V_e staged as
// key groups (4 tokens of a column contiguous).
template <typename T, int D, int M>
__global__ void __launch_bounds__(256) k_nha_chunk(const T* __restrict__ k, const T* __restrict__ v,
                                                   const float* __restrict__ gate, NhaWs ws, int L, int ne) {
  constexpr int RL = kg_row<T, D>();
  constexpr bool SPLIT = sizeof(T) == 2;
  __shared__ __align__(16) float wg[CHUNK][M];  // gates, then the weights
  __shared__ __align__(16) T Kg[(CHUNK / 4) * RL * 4];
  __shared__ __align__(16) T Vg[(CHUNK / 4) * RL * 4];
  const int64_t bh = bid_x() / ne;
  const int e = bid_x() % ne;
  const int tid = tid_x(), lane = lane_id(), w = wave_id();
  const int g = lane >> 4, c = lane & 15;
  const int64_t row0 = bh * L + (int64_t)e * CHUNK;
  constexpr int NA = (CHUNK * M / 4 + 255) / 256;
  constexpr int VT = (CHUNK / 4) * (D / 8);
  static_assert(VT <= 256, "one task per thread");
  const int kg = tid / (D / 8), col = (tid % (D / 8)) * 8;
  {
    f32x4 av[NA];
    Frag<T> kr[4], vr[4];
#pragma unroll
    for (int u = 0; u < NA; ++u) {
      const int x = tid + 256 * u;
      if (x < CHUNK * M / 4) av[u] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(gate + row0 * M + 4 * x));
    }
    if (tid < VT) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        kr[i] = load8<T>(k + (row0 + 4 * kg + i) * D + col);
        vr[i] = load8<T>(v + (row0 + 4 * kg + i) * D + col);
      }
    }
#pragma unroll
    for (int u = 0; u < NA; ++u) {
      const int x = tid + 256 * u;
      if (x < CHUNK * M / 4) *reinterpret_cast<f32x4*>(&wg[0][0] + 4 * x) = av[u];
    }
    if (tid < VT) {
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        st4<T>(Kg + kg_index<RL>(kg, col + jj), to_f32(frag_get<T>(kr[0], jj)), to_f32(frag_get<T>(kr[1], jj)),
               to_f32(frag_get<T>(kr[2], jj)), to_f32(frag_get<T>(kr[3], jj)));
        st4<T>(Vg + kg_index<RL>(kg, col + jj), to_f32(frag_get<T>(vr[0], jj)), to_f32(frag_get<T>(vr[1], jj)),
               to_f32(frag_get<T>(vr[2], jj)), to_f32(frag_get<T>(vr[3], jj)));
      }
    }
  }
  __syncthreads();
  if (tid < M) {
    float suf = 1.f;
    for (int s = CHUNK - 1; s >= 0; --s) {
      const float a = wg[s][tid];
      wg[s][tid] = (1.f - a) * suf;
      suf *= a;
    }
    ws.G[(bh * ne + e) * M + tid] = suf;
  }
  __syncthreads();
  // tiles (K or V, 16 slots, 16 columns), wave w takes tiles w, w + 4, ...
  constexpr int RT = M / 16, CT = D / 16, NTL = 2 * RT * CT;
  for (int t = w; t < NTL; t += 4) {
    const int which = t / (RT * CT), rem = t % (RT * CT), rt = rem / CT, ct = rem % CT;
    const T* Xg = which ? Vg : Kg;
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
      Frag<T> ah, al;
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const float x = wg[32 * k2 + kmap_acc(g, jj)][16 * rt + c];
        frag_set(ah, jj, x);
        frag_set(al, jj, x - to_f32(frag_get<T>(ah, jj)));
      }
      const Frag<T> bx = ld4x2<T>(Xg + kg_index<RL>(8 * k2 + g, 16 * ct + c),
                                      Xg + kg_index<RL>(8 * k2 + 4 + g, 16 * ct + c));
      mma(acc, ah, bx);
      if constexpr (SPLIT) mma(acc, al, bx);
    }
    float* S = (which ? ws.Sv : ws.Sk) + (bh * ne + e) * M * D;
#pragma unroll
    for (int i = 0; i < 4; ++i) S[(16 * rt + 4 * g + i) * D + 16 * ct + c] = acc[i];
  }
}

// chunk-start slot states, in place: entry e holds the chunk's change on
// entry and the state before chunk e on exit (S_0 = 0).  One thread per
// (b, h, slot entry of K~ or V~); the chunk changes are loaded 8 ahead.
template <int D, int M>
__global__ void __launch_bounds__(256) k_nha_scan(NhaWs ws, int BH, int ne) {
  constexpr int PER = M * D;  // entries of K~ (or V~) per head
  const int64_t gid = (int64_t)bid_x() * 256 + tid_x();
  if (gid >= (int64_t)BH * 2 * PER) return;
  const int64_t bh = gid / (2 * PER);
  const int r = (int)(gid % (2 * PER));
  const bool isv = r >= PER;
  const int el = isv ? r - PER : r;
  const int slot = el / D;
  float* S = (isv ? ws.Sv : ws.Sk) + bh * ne * PER + el;
  const float* G = ws.G + bh * ne * M + slot;
  float state = 0.f;
  int e = 0;
  for (; e + 8 <= ne; e += 8) {
    float dl[8], g[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {  // each entry is read and rewritten once: non-temporal
      dl[u] = __builtin_nontemporal_load(S + (int64_t)(e + u) * PER);
      g[u] = G[(int64_t)(e + u) * M];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      __builtin_nontemporal_store(state, S + (int64_t)(e + u) * PER);
      state = fmaf(g[u], state, dl[u]);
    }
  }
  for (; e < ne; ++e) {
    const float dl = S[(int64_t)e * PER];
    S[(int64_t)e * PER] = state;
    state = fmaf(G[(int64_t)e * M], state, dl);
  }
}

// per (b, h, query chunk c): slot scores, one softmax with the window, the
// slot read-out and the merge, on the matrix cores where the work is a
// product.  o_w / lse_w: the window's normalised output and natural-log
// logsumexp (NULL: empty window, w = 0).  With Gamma[j][i] = prod_{r<=j}
// a_r[i] over chunk e's tokens and P the slot weights of the softmax:
//   X = Q [K~_e; K_e]^T                       (matrix cores)
//   z_j[i] by the recurrence over chunk e's tokens, softmax      (vector)
//   R[j][s] = sum_i P[j][i] (1 - a_s[i]) prod_{s<r<=j} a_r[i]   (vector, s <= j)
//   O = (P * Gamma) V~_e + R V_e + w_win o_w                    (matrix cores)
// R and Gamma come from running products (gates of exactly 0 or 1 stay exact).
// The slot states (fp32) enter the bf16 products as hi + lo parts.
// max / sum over aligned groups of M = 16, 32 or 64 lanes, in registers:
// the 16-lane rows by DPP (quad swaps, then the half-row and row mirrors),
// then the gfx950 row swaps (permlane16: rows 0-1 and 2-3; permlane32: rows
// 0-2 and 1-3); the result is in every lane of the group
template <int M>
__device__ __forceinline__ float lane_group_max(float x) {
  static_assert(M == 16 || M == 32 || M == 64, "groups of 16, 32 or 64 lanes");
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, true)));   // quad_perm 1,0,3,2
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, true)));   // quad_perm 2,3,0,1
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x141, 0xF, 0xF, true)));  // row_half_mirror
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x140, 0xF, 0xF, true)));  // row_mirror
  if constexpr (M >= 32) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  }
  if constexpr (M == 64) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  }
  return x;
}
template <int M>
__device__ __forceinline__ float lane_group_sum(float x) {
  static_assert(M == 16 || M == 32 || M == 64, "groups of 16, 32 or 64 lanes");
  x = dpp_group_sum<16>(x);
  if constexpr (M >= 32) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  if constexpr (M == 64) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  return x;
}

template <typename T, int D, int M>
struct NhaSlotCfg {
  static constexpr int MP = M < 32 ? 32 : M;        // slots padded to the 32-deep contraction
  static constexpr int P = D + 16 / (int)sizeof(T);  // row pitch (elements)
  static constexpr int RL = kg_row<T, D>();
  static constexpr int KGB = 16 * RL * 4 * (int)sizeof(T);         // key groups of 64 rows
  static constexpr int KGBM = (MP / 4) * RL * 4 * (int)sizeof(T);  // key groups of MP rows
  static constexpr bool SPLIT = sizeof(T) == 2;
  // One region serves three phases in turn (Q stays in registers, each
  // wave's 16 rows): (1) the score products' [K~_e hi; K_e] and K~_e lo
  // rows; (2) fp32 [64][*] arrays: the gates of chunk e, X's slot part / P /
  // P * Gamma, and q_j.k_s / R; (3) the read-out's key groups of V_e and of
  // V~_e hi / lo.  So two workgroups fit in a CU.
  static constexpr int RK = (M + CHUNK + (SPLIT ? M : 0)) * P * (int)sizeof(T);
  static constexpr int OFF_A = 0;                       // fp32 [64][M] gates of chunk e
  static constexpr int OFF_XS = CHUNK * M * 4;          // fp32 [64 j][M] X's slot part, P, P * Gamma
  static constexpr int OFF_QK = 2 * CHUNK * M * 4;      // fp32 [64 s][64 j] q_j.k_s, then R [64 j][64 s]
  static constexpr int RS = OFF_QK + CHUNK * CHUNK * 4;
  static constexpr int RV = KGB + KGBM * (SPLIT ? 2 : 1);
  static constexpr int R1 = RK > RS ? RK : RS;
  static constexpr int OFF_WW = (((R1 > RV ? R1 : RV) + 15) & ~15);  // fp32 [64] the window's weights
  static constexpr int LDS = OFF_WW + CHUNK * 4;
  static_assert(2 * LDS <= 160 * 1024, "two workgroups per CU");
};

template <typename T, typename To, int D, int M>
__global__ void __launch_bounds__(256, 2) k_nha_slots(const T* __restrict__ q, const T* __restrict__ k,
                                                      const T* __restrict__ v, const float* __restrict__ gate,
                                                      NhaWs ws, const float* __restrict__ o_w,
                                                      const float* __restrict__ lse_w, To* __restrict__ out, int L,
                                                      int nw, int ne, float scale) {
  using C = NhaSlotCfg<T, D, M>;
  constexpr int P = C::P, KF = D / 32, NCT = (M + CHUNK) / 16, MS = M / 16;
  extern __shared__ __align__(16) unsigned char lds[];
  T* KS = reinterpret_cast<T*>(lds);  // M slot rows (hi), then chunk e's 64 key rows
  T* KL = KS + (M + CHUNK) * P;       // M slot rows (lo)
  T* Vg = reinterpret_cast<T*>(lds);
  T* VTh = reinterpret_cast<T*>(lds + C::KGB);
  T* VTl = reinterpret_cast<T*>(lds + C::KGB + C::KGBM);
  float* A = reinterpret_cast<float*>(lds + C::OFF_A);
  float* XS = reinterpret_cast<float*>(lds + C::OFF_XS);
  float* QK = reinterpret_cast<float*>(lds + C::OFF_QK);
  float* WW = reinterpret_cast<float*>(lds + C::OFF_WW);
  const int nc = L / CHUNK;
  const int64_t bh = bid_x() / nc;
  const int qc = bid_x() % nc;
  const int e = qc - nw;
  const int tid = tid_x();
  const int64_t row0 = bh * L + (int64_t)qc * CHUNK;
  if (e < 0) {  // no token has left the window yet: the window's result stands
    constexpr int NO = CHUNK * D / 4 / 256;
    f32x4 ov[NO];
#pragma unroll
    for (int u = 0; u < NO; ++u) ov[u] = *reinterpret_cast<const f32x4*>(o_w + row0 * D + 4 * (tid + 256 * u));
#pragma unroll
    for (int u = 0; u < NO; ++u) {
      const float f[4] = {ov[u][0], ov[u][1], ov[u][2], ov[u][3]};
      store4f<To>(out + row0 * D + 4 * (tid + 256 * u), f);
    }
    return;
  }
  const int64_t erow0 = bh * L + (int64_t)e * CHUNK;
  const int lane = lane_id(), w = wave_id();
  const int g = lane >> 4, c = lane & 15;
  const float* Ske = ws.Sk + (bh * ne + e) * M * D;
  const float* Sve = ws.Sv + (bh * ne + e) * M * D;

  // ---- phase 1: the score products' rows; Q as this wave's A fragments and
  // the gates stay in registers until the rows are dead
  constexpr int NQ = CHUNK * D / 8 / 256;          // 8-element pieces of k per thread
  constexpr int NSK = (M * D / 8 + 255) / 256;     // 8-float pieces of K~_e per thread
  constexpr int NA = (CHUNK * M / 4 + 255) / 256;  // 4-float pieces of the gates per thread
  Frag<T> qa[KF];
  f32x4 av[NA];
  {
    Frag<T> kv[NQ];
    float skv[NSK][8];
#pragma unroll
    for (int u = 0; u < NQ; ++u) {
      const int x = tid + 256 * u, r = x / (D / 8), col = (x % (D / 8)) * 8;
      kv[u] = load8<T>(k + (erow0 + r) * D + col);
    }
#pragma unroll
    for (int u = 0; u < NSK; ++u) {
      const int x = tid + 256 * u, r = x / (D / 8), col = (x % (D / 8)) * 8;
      if (x < M * D / 8) {
        const f32x4 lo4 = *reinterpret_cast<const f32x4*>(Ske + r * D + col);
        const f32x4 hi4 = *reinterpret_cast<const f32x4*>(Ske + r * D + col + 4);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          skv[u][jj] = lo4[jj];
          skv[u][4 + jj] = hi4[jj];
        }
      }
    }
#pragma unroll
    for (int ks = 0; ks < KF; ++ks) qa[ks] = load8<T>(q + (row0 + 16 * w + c) * D + 32 * ks + 8 * g);
#pragma unroll
    for (int u = 0; u < NA; ++u) {
      const int x = tid + 256 * u;
      if (x < CHUNK * M / 4) av[u] = *reinterpret_cast<const f32x4*>(gate + erow0 * M + 4 * x);
    }
#pragma unroll
    for (int u = 0; u < NQ; ++u) {
      const int x = tid + 256 * u, r = x / (D / 8), col = (x % (D / 8)) * 8;
      store8<T>(KS + (M + r) * P + col, kv[u]);
    }
#pragma unroll
    for (int u = 0; u < NSK; ++u) {
      const int x = tid + 256 * u, r = x / (D / 8), col = (x % (D / 8)) * 8;
      if (x < M * D / 8) {
        Frag<T> hi, lo;
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          frag_set(hi, jj, skv[u][jj]);
          frag_set(lo, jj, skv[u][jj] - to_f32(frag_get<T>(hi, jj)));
        }
        store8<T>(KS + r * P + col, hi);
        if constexpr (C::SPLIT) store8<T>(KL + r * P + col, lo);
      }
    }
  }
  __syncthreads();
  // ---- X = Q [K~_e; K_e]^T: wave w takes query rows 16w .. 16w+15
  {
    f32x4 acc[NCT];
#pragma unroll
    for (int n = 0; n < NCT; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KF; ++ks) {
#pragma unroll
      for (int n = 0; n < NCT; ++n) {
        mma(acc[n], qa[ks], load8<T>(KS + (16 * n + c) * P + 32 * ks + 8 * g));
        if constexpr (C::SPLIT)
          if (n < MS) mma(acc[n], qa[ks], load8<T>(KL + (16 * n + c) * P + 32 * ks + 8 * g));
      }
    }
    __syncthreads();  // every wave is done with the rows: phase 2's arrays take the region
#pragma unroll
    for (int n = 0; n < NCT; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = 16 * w + 4 * g + i;
        if (n < MS) XS[j * M + 16 * n + c] = acc[n][i];
        else QK[(16 * (n - MS) + c) * CHUNK + j] = acc[n][i];
      }
#pragma unroll
    for (int u = 0; u < NA; ++u) {
      const int x = tid + 256 * u;
      if (x < CHUNK * M / 4) *reinterpret_cast<f32x4*>(A + 4 * x) = av[u];
    }
  }
  __syncthreads();
  // ---- slot scores: lane group grp (M lanes, lane i = slot i) takes the
  // JPG queries j = grp JPG .. and runs the slot key's recurrence over chunk
  // e's tokens for all of them at once,
  //   y_j(s) = a_s[i] y_j(s - 1) + (1 - a_s[i]) q_j.k_s,  y_j(-1) = q_j.K~_e[i],
  // so z_j = q_j.K~ after token j = y_j(j); then one softmax per query over
  // [slots, window] (the window through its lse)
  {
    constexpr int NG = 256 / M, JPG = CHUNK / NG;  // JPG = M / 4 queries per group
    const int i = tid % M, grp = tid / M;
    const int jb = grp * JPG;
    float y[JPG], z[JPG];
#pragma unroll
    for (int u = 0; u < JPG; ++u) y[u] = XS[(jb + u) * M + i];
#pragma unroll 4
    for (int st = 0; st < jb; ++st) {  // tokens before the group's first query: every query takes them
      const float a = A[st * M + i], b = 1.f - a;
      const float* qk = QK + st * CHUNK + jb;
#pragma unroll
      for (int u = 0; u < JPG; u += 4) {
        const f32x4 v4 = *reinterpret_cast<const f32x4*>(qk + u);
#pragma unroll
        for (int x = 0; x < 4; ++x) y[u + x] = fmaf(a, y[u + x], b * v4[x]);
      }
    }
#pragma unroll
    for (int u0 = 0; u0 < JPG; ++u0) {  // token jb + u0: queries jb + u0 .. take it, query jb + u0 is done
      const int st = jb + u0;
      const float a = A[st * M + i], b = 1.f - a;
      const float* qk = QK + st * CHUNK + jb;
#pragma unroll
      for (int u = u0; u < JPG; ++u) y[u] = fmaf(a, y[u], b * qk[u]);
      z[u0] = y[u0];
    }
    // (each group writes only its own queries' rows of XS, after reading them)
#pragma unroll
    for (int u = 0; u < JPG; ++u) {
      const int j = jb + u;
      const float zz = scale * z[u];
      const float lw = lse_w ? lse_w[row0 + j] : -INFINITY;
      const float mx = fmaxf(lane_group_max<M>(zz), lw);
      const float p = __expf(zz - mx);
      float den = lane_group_sum<M>(p);
      const float pw = __expf(lw - mx);  // 0 for an empty window
      den += pw;
      const float inv = 1.f / den;
      XS[j * M + i] = p * inv;
      if ((lane % M) == 0) WW[j] = pw * inv;
    }
  }
  __syncthreads();
  // the read-out's V_e and V~_e rows: loaded now (the R loop hides their
  // latency), stored as key groups once phase 2's arrays are dead
  constexpr int VT = (CHUNK / 4) * (D / 8);  // (key group, 8 columns) tasks of V_e
  constexpr int ST = (C::MP / 4) * (D / 8);  // ... of V~_e (rows past M are zero)
  static_assert(VT <= 256 && ST <= 256, "one task per thread");
  const int vkg = tid / (D / 8), vcol = (tid % (D / 8)) * 8;
  Frag<T> vr[4];
  float sr[4][8];
  if (tid < VT) {
#pragma unroll
    for (int i = 0; i < 4; ++i) vr[i] = load8<T>(v + (erow0 + 4 * vkg + i) * D + vcol);
  }
  if (tid < ST) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 4 * vkg + i;
      if (r < M) {
        const f32x4 lo4 = *reinterpret_cast<const f32x4*>(Sve + r * D + vcol);
        const f32x4 hi4 = *reinterpret_cast<const f32x4*>(Sve + r * D + vcol + 4);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          sr[i][jj] = lo4[jj];
          sr[i][4 + jj] = hi4[jj];
        }
      } else {
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) sr[i][jj] = 0.f;
      }
    }
  }
  // R[j][s] = sum_i P[j][i] (1 - a_s[i]) prod_{s<r<=j} a_r[i]: thread (s,
  // quarter of the slots) keeps its running weights in registers over j; the
  // four quarters of a token sit in adjacent lanes and are added by DPP
  {
    constexpr int SPQ = M / 4;
    const int s = tid >> 2, part = tid & 3, i0 = part * SPQ;
    static_assert(SPQ % 4 == 0, "whole float4 pieces");
    float cw[SPQ];
#pragma unroll
    for (int u = 0; u < SPQ; ++u) cw[u] = 1.f - A[s * M + i0 + u];
    // R[j][s] = 0 for j < s: wave w (tokens 16w .. 16w + 15) starts at j = 16w
    const int j0 = 16 * w;
    if (part == 0)
      for (int j = 0; j < j0; ++j) QK[j * CHUNK + s] = 0.f;
#pragma unroll 4
    for (int j = j0; j < CHUNK; ++j) {
      // branch-free (a guarded multiply became one exec-masked branch and
      // one LDS round trip per slot); four partial sums for the dot product
      const bool later = j > s;
      float ra[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int u4 = 0; u4 < SPQ / 4; ++u4) {
        const f32x4 a4 = *reinterpret_cast<const f32x4*>(A + j * M + i0 + 4 * u4);
        const f32x4 p4 = *reinterpret_cast<const f32x4*>(XS + j * M + i0 + 4 * u4);
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const int u = 4 * u4 + x;
          cw[u] *= later ? a4[x] : 1.f;
          ra[x] = fmaf(p4[x], cw[u], ra[x]);
        }
      }
      float r = (ra[0] + ra[1]) + (ra[2] + ra[3]);
      r += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(r), 0xB1, 0xF, 0xF, true));  // quad_perm 1,0,3,2
      r += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(r), 0x4E, 0xF, 0xF, true));  // quad_perm 2,3,0,1
      if (part == 0) QK[j * CHUNK + s] = (j >= s) ? r : 0.f;
    }
  }
  __syncthreads();
  // P * Gamma, in place (slot i's running product over the chunk's tokens)
  if (tid < M) {
    float gm = 1.f;
    for (int j = 0; j < CHUNK; ++j) {
      gm *= A[j * M + tid];
      XS[j * M + tid] *= gm;
    }
  }
  __syncthreads();
  // ---- O = (P * Gamma) V~_e + R V_e + w_win o_w: wave w takes rows 16w ..;
  // its R and P * Gamma fragments go to registers before phase 3 takes the region
  constexpr int MK = C::MP / 32;
  Frag<T> ar[2], ap[MK];
#pragma unroll
  for (int k2 = 0; k2 < 2; ++k2)
    ar[k2] = frag_fn<T>([&](int jj) { return QK[(16 * w + c) * CHUNK + 32 * k2 + kmap_acc(g, jj)]; });
#pragma unroll
  for (int kk = 0; kk < MK; ++kk)
    ap[kk] = frag_fn<T>([&](int jj) {
      const int i = 32 * kk + kmap_acc(g, jj);
      return i < M ? XS[(16 * w + c) * M + i] : 0.f;
    });
  __syncthreads();
  // V_e and V~_e (hi, lo) as key groups (4 rows of a column contiguous)
  if (tid < VT) {
#pragma unroll
    for (int jj = 0; jj < 8; ++jj)
      st4<T>(Vg + kg_index<C::RL>(vkg, vcol + jj), to_f32(frag_get<T>(vr[0], jj)), to_f32(frag_get<T>(vr[1], jj)),
             to_f32(frag_get<T>(vr[2], jj)), to_f32(frag_get<T>(vr[3], jj)));
  }
  if (tid < ST) {
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      float hv[4], lv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        hv[i] = to_f32(from_f32<T>(sr[i][jj]));
        lv[i] = sr[i][jj] - hv[i];
      }
      st4<T>(VTh + kg_index<C::RL>(vkg, vcol + jj), hv[0], hv[1], hv[2], hv[3]);
      if constexpr (C::SPLIT) st4<T>(VTl + kg_index<C::RL>(vkg, vcol + jj), lv[0], lv[1], lv[2], lv[3]);
    }
  }
  __syncthreads();
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) {
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2)
      mma(acc, ar[k2], ld4x2<T>(Vg + kg_index<C::RL>(8 * k2 + g, 16 * dt + c),
                                    Vg + kg_index<C::RL>(8 * k2 + 4 + g, 16 * dt + c)));
#pragma unroll
    for (int kk = 0; kk < MK; ++kk) {
      mma(acc, ap[kk], ld4x2<T>(VTh + kg_index<C::RL>(8 * kk + g, 16 * dt + c),
                                    VTh + kg_index<C::RL>(8 * kk + 4 + g, 16 * dt + c)));
      if constexpr (C::SPLIT)
        mma(acc, ap[kk], ld4x2<T>(VTl + kg_index<C::RL>(8 * kk + g, 16 * dt + c),
                                      VTl + kg_index<C::RL>(8 * kk + 4 + g, 16 * dt + c)));
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = 16 * w + 4 * g + i, d = 16 * dt + c;
      const float ow = o_w ? o_w[(row0 + j) * D + d] : 0.f;
      out[(row0 + j) * D + d] = from_f32<To>(fmaf(WW[j], ow, acc[i]));
    }
  }
}

size_t nha_ws_bytes(int B, int H, int L, int D, int M, int window) {
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const int nc = L / CHUNK, nw = window / CHUNK;
  const size_t ne = (size_t)(nc > nw ? nc - nw : 0);
  const size_t BH = (size_t)B * H;
  return 2 * al(BH * ne * M * D * 4) + al(BH * ne * M * 4) + al(BH * L * D * 4) + al(BH * L * 4);
}

template <typename T, typename To, int D>
hipError_t launch_nha_m(const T* q, const T* k, const T* v, const float* gate, int M, To* out, void* wsp, int B,
                        int H, int L, int window, float scale, hipStream_t st, void (*prof)(int, hipStream_t, int),
                        const SideStream& side) {
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const int nc = L / CHUNK, nw = window / CHUNK;
  const int ne = nc > nw ? nc - nw : 0;
  const int64_t BH = (int64_t)B * H;
  hipError_t e;
  if (ne == 0) {  // the window covers the sequence: causal softmax attention
    if (prof) prof(KID_NHA_WINDOW, st, 0);
    e = launch_softmax_window<T, To, D>(q, k, v, out, nullptr, B, H, L, nc, scale, st);
    if (e == hipSuccess && prof) prof(KID_NHA_WINDOW, st, 1);
    return e;
  }
  char* p = (char*)wsp;
  NhaWs ws;
  ws.Sk = (float*)p; p += al((size_t)BH * ne * M * D * 4);
  ws.Sv = (float*)p; p += al((size_t)BH * ne * M * D * 4);
  ws.G = (float*)p; p += al((size_t)BH * ne * M * 4);
  float* o_w = (float*)p; p += al((size_t)BH * L * D * 4);
  float* lse_w = (float*)p;
  // the window's softmax needs none of the slot states: with a side stream
  // it runs there beside the chunk and scan kernels, joined before the slots
  const bool fork = side.aux != nullptr && nw > 0;
  const hipStream_t sw = fork ? side.aux : st;
  if (fork) {
    if ((e = hipEventRecord(side.fork, st)) != hipSuccess) return e;
    if ((e = hipStreamWaitEvent(side.aux, side.fork, 0)) != hipSuccess) return e;
  }
  auto join = [&](hipError_t err) {  // also after a failed launch: nothing queued outlives the call's order
    if (!fork) return err;
    const hipError_t ej = hipEventRecord(side.join, side.aux);
    const hipError_t ew = ej == hipSuccess ? hipStreamWaitEvent(st, side.join, 0) : ej;
    return err != hipSuccess ? err : ew;
  };
  if (nw > 0) {
    if (prof) prof(KID_NHA_WINDOW, sw, 0);
    e = launch_softmax_window<T, float, D>(q, k, v, o_w, lse_w, B, H, L, nw, scale, sw);
    if (e != hipSuccess) return join(e);
    if (prof) prof(KID_NHA_WINDOW, sw, 1);
  }
  const float* ow = nw > 0 ? o_w : nullptr;
  const float* lw = nw > 0 ? lse_w : nullptr;
#define NHA_M(MM)                                                                                                  \
  do {                                                                                                             \
    const size_t lds = NhaSlotCfg<T, D, MM>::LDS;                                                                  \
    if ((e = set_lds_limit((const void*)k_nha_slots<T, To, D, MM>, (int)lds)) != hipSuccess) return join(e);      \
    if (prof) prof(KID_NHA_CHUNK, st, 0);                                                                          \
    hipLaunchKernelGGL((k_nha_chunk<T, D, MM>), dim3((unsigned)(BH * ne)), dim3(256), 0, st, k, v, gate, ws, L,     \
                       ne);                                                                                        \
    if ((e = hipGetLastError()) != hipSuccess) return join(e);                                                    \
    if (prof) prof(KID_NHA_CHUNK, st, 1);                                                                          \
    const int64_t nthr = BH * 2 * MM * D;                                                                          \
    if (prof) prof(KID_NHA_SCAN, st, 0);                                                                           \
    hipLaunchKernelGGL((k_nha_scan<D, MM>), dim3((unsigned)((nthr + 255) / 256)), dim3(256), 0, st, ws, (int)BH,   \
                       ne);                                                                                        \
    if ((e = hipGetLastError()) != hipSuccess) return join(e);                                                    \
    if (prof) prof(KID_NHA_SCAN, st, 1);                                                                           \
    if ((e = join(hipSuccess)) != hipSuccess) return e;                                                            \
    if (prof) prof(KID_NHA_SLOTS, st, 0);                                                                          \
    hipLaunchKernelGGL((k_nha_slots<T, To, D, MM>), dim3((unsigned)(BH * nc)), dim3(256), lds, st, q, k, v, gate,  \
                       ws, ow, lw, out, L, nw, ne, scale);                                                         \
    if ((e = hipGetLastError()) != hipSuccess) return e;                                                          \
    if (prof) prof(KID_NHA_SLOTS, st, 1);                                                                          \
    return hipSuccess;                                                                                             \
  } while (0)
  if (M == 16) NHA_M(16);
  if (M == 32) NHA_M(32);
  if (M == 64) NHA_M(64);
#undef NHA_M
  return join(hipErrorInvalidValue);
}

template <typename T, typename To, int D>
hipError_t launch_nha(const T* q, const T* k, const T* v, const float* gate, int M, To* out, void* ws, int B, int H,
                      int L, int window, float scale, hipStream_t st, void (*prof)(int, hipStream_t, int),
                      const SideStream& side) {
  return launch_nha_m<T, To, D>(q, k, v, gate, M, out, ws, B, H, L, window, scale, st, prof, side);
}

#define INST(T, To, D)                                                                                          \
  template hipError_t launch_nha<T, To, D>(const T*, const T*, const T*, const float*, int, To*, void*, int, int, \
                                           int, int, float, hipStream_t, void (*)(int, hipStream_t, int), \
                                           const SideStream&);
INST(float, float, 64)
INST(float, float, 128)
INST(bf16, bf16, 64)
INST(bf16, bf16, 128)
#undef INST

}  // namespace natsl
