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
//   window attention  the generic softmax kernel in window mode (o_w, lse_w);
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

// per (b, h, chunk e < ne): the slots' change over the chunk and its decay
template <typename T, int D, int M>
__global__ void __launch_bounds__(256) k_nha_chunk(const T* __restrict__ k, const T* __restrict__ v,
                                                   const float* __restrict__ gate, NhaWs ws, int L, int ne) {
  constexpr int TPC = 256 / D;   // threads per column
  constexpr int SPT = M / TPC;   // slots per thread
  __shared__ float wg[CHUNK][M];  // gates, then the weights (1 - a_s) prod_{s<r<64} a_r
  const int nc = L / CHUNK;
  const int64_t bh = bid_x() / ne;
  const int e = bid_x() % ne;
  const int tid = tid_x();
  const float* gc = gate + (bh * L + (int64_t)e * CHUNK) * M;
  for (int x = tid; x < CHUNK * M; x += 256) wg[x / M][x % M] = gc[x];
  __syncthreads();
  float* G = ws.G + (bh * ne + e) * M;
  if (tid < M) {
    float suf = 1.f;
    for (int s = CHUNK - 1; s >= 0; --s) {
      const float a = wg[s][tid];
      wg[s][tid] = (1.f - a) * suf;
      suf *= a;
    }
    G[tid] = suf;
  }
  __syncthreads();
  const int d = tid / TPC, part = tid % TPC;
  const T* kc = k + (bh * L + (int64_t)e * CHUNK) * D + d;
  const T* vc = v + (bh * L + (int64_t)e * CHUNK) * D + d;
  float ak[SPT], av[SPT];
#pragma unroll
  for (int u = 0; u < SPT; ++u) ak[u] = av[u] = 0.f;
  constexpr int PF = 8;  // tokens of k and v in flight (clamped, unconditional loads)
  float kr[PF], vr[PF];
#pragma unroll
  for (int u = 0; u < PF; ++u) {
    kr[u] = to_f32(kc[(int64_t)u * D]);
    vr[u] = to_f32(vc[(int64_t)u * D]);
  }
  for (int s0 = 0; s0 < CHUNK; s0 += PF) {
#pragma unroll
    for (int x = 0; x < PF; ++x) {
      const int s = s0 + x, sn = min(s + PF, CHUNK - 1);
      const float ks = kr[x], vs = vr[x];
      kr[x] = to_f32(kc[(int64_t)sn * D]);
      vr[x] = to_f32(vc[(int64_t)sn * D]);
#pragma unroll
      for (int u = 0; u < SPT; ++u) {
        const float w = wg[s][part * SPT + u];
        ak[u] = fmaf(w, ks, ak[u]);
        av[u] = fmaf(w, vs, av[u]);
      }
    }
  }
  float* dk = ws.Sk + ((bh * ne + e) * M) * D + d;
  float* dv = ws.Sv + ((bh * ne + e) * M) * D + d;
#pragma unroll
  for (int u = 0; u < SPT; ++u) {
    dk[(int64_t)(part * SPT + u) * D] = ak[u];
    dv[(int64_t)(part * SPT + u) * D] = av[u];
  }
  (void)nc;
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
    for (int u = 0; u < 8; ++u) {
      dl[u] = S[(int64_t)(e + u) * PER];
      g[u] = G[(int64_t)(e + u) * M];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      S[(int64_t)(e + u) * PER] = state;
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
// slot read-out and the merge.  o_w / lse_w: the window's normalised output
// and natural-log logsumexp (NULL: empty window, w = 0).
template <typename T, typename To, int D, int M>
__global__ void __launch_bounds__(256) k_nha_slots(const T* __restrict__ q, const T* __restrict__ k,
                                                   const T* __restrict__ v, const float* __restrict__ gate,
                                                   NhaWs ws, const float* __restrict__ o_w,
                                                   const float* __restrict__ lse_w, To* __restrict__ out, int L,
                                                   int nw, int ne, float scale) {
  constexpr int DP = D + 4;           // padded LDS row (16-byte aligned, rows spread over the banks)
  constexpr int NCOL = M + CHUNK;     // columns of the score products: M slots, then the chunk's 64 keys
  constexpr int TPC = 256 / D, SPT = M / TPC;
  extern __shared__ __align__(16) float sh[];
  float* Qs = sh;                     // [64][DP]   queries
  float* KC = Qs + CHUNK * DP;        // [NCOL][DP] slot keys K~_e, then chunk e's keys
  float* A = KC + NCOL * DP;          // [64][M]    gates of chunk e's tokens
  float* XS = A + CHUNK * M;          // [64 j][M]  q_j.K~_e[i], then P[j][i]
  float* QKT = XS + CHUNK * M;        // [64 s][64 j] q_j.k_s (transposed: a step s reads its queries' row)
  float* WW = QKT + CHUNK * CHUNK;    // [64] the window's weight per query
  const int nc = L / CHUNK;
  const int64_t bh = bid_x() / nc;
  const int c = bid_x() % nc;
  const int e = c - nw;
  const int tid = tid_x();
  const int64_t row0 = bh * L + (int64_t)c * CHUNK;
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
  // ---- stage q (chunk c), K~_e and chunk e's keys, chunk e's gates: every
  // load of the thread is issued before the first LDS store (a load, then its
  // store, one after the other kept a single load in flight per wave)
  {
    constexpr int NQ = CHUNK * D / 8 / 256;  // 8-element pieces of q and of k per thread
    constexpr int NS = M * D / 4 / 256;      // 4-float pieces of K~_e per thread
    constexpr int NA = CHUNK * M / 4 / 256;  // 4-float pieces of the gates per thread
    float qv[NQ][8], kv[NQ][8];
    f32x4 sv[NS], av[NA];
    const float* Ske = ws.Sk + (bh * ne + e) * M * D;
#pragma unroll
    for (int u = 0; u < NQ; ++u) {
      const int x = tid + 256 * u, r = x / (D / 8), col = (x % (D / 8)) * 8;
      load8f<T>(q + (row0 + r) * D + col, qv[u]);
      load8f<T>(k + (erow0 + r) * D + col, kv[u]);
    }
#pragma unroll
    for (int u = 0; u < NS; ++u) {
      const int x = tid + 256 * u, r = x / (D / 4), col = (x % (D / 4)) * 4;
      sv[u] = *reinterpret_cast<const f32x4*>(Ske + r * D + col);
    }
#pragma unroll
    for (int u = 0; u < NA; ++u) av[u] = *reinterpret_cast<const f32x4*>(gate + erow0 * M + 4 * (tid + 256 * u));
#pragma unroll
    for (int u = 0; u < NQ; ++u) {
      const int x = tid + 256 * u, r = x / (D / 8), col = (x % (D / 8)) * 8;
      *reinterpret_cast<f32x4*>(Qs + r * DP + col) = f32x4{qv[u][0], qv[u][1], qv[u][2], qv[u][3]};
      *reinterpret_cast<f32x4*>(Qs + r * DP + col + 4) = f32x4{qv[u][4], qv[u][5], qv[u][6], qv[u][7]};
      *reinterpret_cast<f32x4*>(KC + (M + r) * DP + col) = f32x4{kv[u][0], kv[u][1], kv[u][2], kv[u][3]};
      *reinterpret_cast<f32x4*>(KC + (M + r) * DP + col + 4) = f32x4{kv[u][4], kv[u][5], kv[u][6], kv[u][7]};
    }
#pragma unroll
    for (int u = 0; u < NS; ++u) {
      const int x = tid + 256 * u, r = x / (D / 4), col = (x % (D / 4)) * 4;
      *reinterpret_cast<f32x4*>(KC + r * DP + col) = sv[u];
    }
#pragma unroll
    for (int u = 0; u < NA; ++u) *reinterpret_cast<f32x4*>(A + 4 * (tid + 256 * u)) = av[u];
  }
  __syncthreads();
  // ---- X = Q [K~_e; K_e]^T (64 x NCOL): a 4 x (NCOL / 64) tile per thread
  {
    constexpr int CPT = NCOL / 16;  // columns per thread
    const int rg = tid / 16, cg = tid % 16;  // rows 4 rg .. 4 rg + 3; columns cg + 16 u
    float acc[4][CPT];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int u = 0; u < CPT; ++u) acc[a][u] = 0.f;
    for (int d0 = 0; d0 < D; d0 += 4) {
      f32x4 qv[4];
#pragma unroll
      for (int a = 0; a < 4; ++a) qv[a] = *reinterpret_cast<const f32x4*>(Qs + (4 * rg + a) * DP + d0);
#pragma unroll
      for (int u = 0; u < CPT; ++u) {
        const f32x4 kv = *reinterpret_cast<const f32x4*>(KC + (cg + 16 * u) * DP + d0);
#pragma unroll
        for (int a = 0; a < 4; ++a)
          acc[a][u] = fmaf(qv[a][0], kv[0], fmaf(qv[a][1], kv[1], fmaf(qv[a][2], kv[2], fmaf(qv[a][3], kv[3], acc[a][u]))));
      }
    }
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int u = 0; u < CPT; ++u) {
        const int col = cg + 16 * u, j = 4 * rg + a;
        if (u < M / 16) XS[j * M + col] = acc[a][u];
        else QKT[(col - M) * CHUNK + j] = acc[a][u];
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
    const int lane = lane_id();
    float y[JPG], z[JPG];
#pragma unroll
    for (int u = 0; u < JPG; ++u) y[u] = XS[(jb + u) * M + i];
    for (int st = 0; st < jb; ++st) {  // tokens before the group's first query: every query takes them
      const float a = A[st * M + i], b = 1.f - a;
      const float* qk = QKT + st * CHUNK + jb;
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
      const float* qk = QKT + st * CHUNK + jb;
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
      float mx = zz;
#pragma unroll
      for (int msk = M / 2; msk >= 1; msk >>= 1) mx = fmaxf(mx, __shfl_xor(mx, msk, 64));
      mx = fmaxf(mx, lw);
      const float p = __expf(zz - mx);
      float den = p;
#pragma unroll
      for (int msk = M / 2; msk >= 1; msk >>= 1) den += __shfl_xor(den, msk, 64);
      const float pw = __expf(lw - mx);  // 0 for an empty window
      den += pw;
      const float inv = 1.f / den;
      XS[j * M + i] = p * inv;
      if ((lane % M) == 0) WW[j] = pw * inv;
    }
  }
  __syncthreads();
  // ---- read-out: V~ rolled forward over chunk e's tokens, thread (column d,
  // slots part * SPT ..) keeps its slot values in registers
  {
    const int d = tid / TPC, part = tid % TPC;
    const float* Sve = ws.Sv + (bh * ne + e) * M * D + d;
    float vt[SPT];
#pragma unroll
    for (int u = 0; u < SPT; ++u) vt[u] = Sve[(int64_t)(part * SPT + u) * D];
    const T* vc = v + erow0 * D + d;
    const float* owc = o_w ? o_w + row0 * D + d : nullptr;
    // v and o_w of the next PF tokens in flight (unconditional loads at
    // clamped rows, so that the compiler does not wait for each right away)
    constexpr int PF = 8;
    float vr[PF], owr[PF];
#pragma unroll
    for (int u = 0; u < PF; ++u) {
      vr[u] = to_f32(vc[(int64_t)u * D]);
      owr[u] = owc ? owc[(int64_t)u * D] : 0.f;
    }
    for (int j0 = 0; j0 < CHUNK; j0 += PF) {
#pragma unroll
      for (int u = 0; u < PF; ++u) {
        const int j = j0 + u;
        const float vj = vr[u], ow = owr[u];
        const int jn = min(j + PF, CHUNK - 1);
        vr[u] = to_f32(vc[(int64_t)jn * D]);
        if (owc) owr[u] = owc[(int64_t)jn * D];
        const float* aj = A + j * M + part * SPT;
        const float* pj = XS + j * M + part * SPT;
        float acc = 0.f;
#pragma unroll
        for (int w = 0; w < SPT; ++w) {
          const float a = aj[w];
          vt[w] = fmaf(a, vt[w], (1.f - a) * vj);
          acc = fmaf(pj[w], vt[w], acc);
        }
#pragma unroll
        for (int msk = 1; msk < TPC; msk <<= 1) acc += __shfl_xor(acc, msk, 64);
        if (part == 0) out[(row0 + j) * D + d] = from_f32<To>(fmaf(WW[j], ow, acc));
      }
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
                        int H, int L, int window, float scale, hipStream_t st, void (*prof)(int, hipStream_t, int)) {
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
  if (nw > 0) {
    if (prof) prof(KID_NHA_WINDOW, st, 0);
    e = launch_softmax_window<T, float, D>(q, k, v, o_w, lse_w, B, H, L, nw, scale, st);
    if (e != hipSuccess) return e;
    if (prof) prof(KID_NHA_WINDOW, st, 1);
  }
  const float* ow = nw > 0 ? o_w : nullptr;
  const float* lw = nw > 0 ? lse_w : nullptr;
  const size_t lds = (size_t)(CHUNK * (D + 4) + (M + CHUNK) * (D + 4) + CHUNK * M + CHUNK * M + CHUNK * CHUNK + CHUNK) * 4;
#define NHA_M(MM)                                                                                                  \
  do {                                                                                                             \
    if ((e = set_lds_limit((const void*)k_nha_slots<T, To, D, MM>, (int)lds)) != hipSuccess) return e;            \
    if (prof) prof(KID_NHA_CHUNK, st, 0);                                                                          \
    hipLaunchKernelGGL((k_nha_chunk<T, D, MM>), dim3((unsigned)(BH * ne)), dim3(256), 0, st, k, v, gate, ws, L,     \
                       ne);                                                                                        \
    if ((e = hipGetLastError()) != hipSuccess) return e;                                                          \
    if (prof) prof(KID_NHA_CHUNK, st, 1);                                                                          \
    const int64_t nthr = BH * 2 * MM * D;                                                                          \
    if (prof) prof(KID_NHA_SCAN, st, 0);                                                                           \
    hipLaunchKernelGGL((k_nha_scan<D, MM>), dim3((unsigned)((nthr + 255) / 256)), dim3(256), 0, st, ws, (int)BH,   \
                       ne);                                                                                        \
    if ((e = hipGetLastError()) != hipSuccess) return e;                                                          \
    if (prof) prof(KID_NHA_SCAN, st, 1);                                                                           \
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
  return hipErrorInvalidValue;
}

template <typename T, typename To, int D>
hipError_t launch_nha(const T* q, const T* k, const T* v, const float* gate, int M, To* out, void* ws, int B, int H,
                      int L, int window, float scale, hipStream_t st, void (*prof)(int, hipStream_t, int)) {
  return launch_nha_m<T, To, D>(q, k, v, gate, M, out, ws, B, H, L, window, scale, st, prof);
}

#define INST(T, To, D)                                                                                          \
  template hipError_t launch_nha<T, To, D>(const T*, const T*, const T*, const float*, int, To*, void*, int, int, \
                                           int, int, float, hipStream_t, void (*)(int, hipStream_t, int));
INST(float, float, 64)
INST(float, float, 128)
INST(bf16, bf16, 64)
INST(bf16, bf16, 128)
#undef INST

}  // namespace natsl
