// Gradient of the Gated DeltaNet branch through the per-chunk rollback, in
// chunk form on the matrix cores.
//
// "Technische Samenvatting: Neural Attention Search Linear (NAtS-L)",
// Kernmechanismen 3 defines the forward: every chunk pseudo-updates the state
// and keeps its end state only when it is routed to the linear operation
// (otherwise the chunk-start state is restored).  In chunk form (gdn.hip),
// for a chunk with start state S0:
//   U = T (diag(b) V - diag(b gamma) K S0),  O = diag(gamma) Q S0 + P U,
//   S_end = gamma_C S0 + K~^T U,  K~ = diag(exp(g_C - g)) K.
// This file takes the exact derivative of that form, chunk by chunk in
// reverse.  With Gc = d loss / d carried state after chunk c and dSe = Gc for
// a linear-routed chunk (its end state is committed), 0 otherwise:
//   dU  = P^T dO + K~ dSe
//   Gc' = gamma_C dSe + Q^T diag(gamma) dO - W^T dU  (+ Gc if not committed)
// (W = T diag(b gamma) K) is a reverse recurrence over chunks whose columns
// evolve independently, like the forward's state.  Given every chunk's S0, U,
// Gc and dU, the token gradients of a chunk are local to it:
//   dP = tril(dO U^T), F = dP * Gamma;  dQ = diag(gamma) dO S0^T + F K
//   TdU = T^T dU;  dV = diag(b) TdU;  TdW = -TdU S0^T
//   VmR = U + diag(b) A U  (= diag(b) V - diag(b gamma) K S0)
//   dT = dU VmR^T;  dM = strict_tril(-T^T dT T^T);  E = diag(b) dM * Gamma
//   dK = diag(b gamma) TdW + E K + E^T K + F^T Q + [committed] diag(e) U Gc^T
// plus the per-token beta and log-decay gradients (row and column sums of the
// same products), the decay gradient reverse-summed into d log alpha, and
// the linear gate's derivative <Gc, S_end - S0> = (gamma_C - 1) <Gc, S0> +
// sum_s e_s k_s . (U Gc^T)_s.  (A = strict_tril(Gamma . K K^T), Gamma[t][s]
// = exp(g_t - g_s), g the in-chunk cumulative log decay.)
//
// Launches (one stream):
//   k_gdn_prep + scan    the forward in state mode (gdn.hip): every chunk's
//                        S0 and U, bf16 or fp32 as the io dtype
//   k_gdn_bwd_prep       one workgroup per chunk-head: the fragment copies of
//                        P^T and -W^T the reverse scan reads
//   k_gdn_bwd_scan       one workgroup per (head, 16-column slice), chunks in
//                        reverse: Gc of every chunk, and dS_init
//   k_gdn_bwd_chunk      one workgroup per chunk-head: T again (as the preps
//                        compute it) and dU = P^T dO + [committed] K~ Gc, then
//                        dq, dk, dv, dalpha, dbeta and the gate derivative
// Workspace: every chunk's S0 and U, then one region that holds the forward
// prep's output while the state scan runs and, once it is dead, the backward
// prep's output and every chunk's Gc.
#include "common.hpp"
#include "gdn_common.hpp"
#include "kernels.hpp"

namespace natsl {

constexpr int BWD_DVT = 16;  // state columns per reverse-scan workgroup
constexpr int GM_FLOATS = 144;  // gamma[64], gamma_C at 64, exp(g_C - g)[64] at 80

template <typename T, int D>
struct GdnBwdWs {
  T* pt;      // [nch][4 rs][2 k2][64][8]  P^T A fragments (rows s, contraction t, accumulator-shaped map)
  T* wtn;     // [nch][D/16][2 k2][64][8]  -W^T A fragments (rows d, contraction s)
  float* gm;  // [nch][GM_FLOATS]
  T* gst;     // [nch][D][D]               Gc of every chunk (the carried gradient after it)
};

static inline size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

// workspace: [S0 of every chunk][U of every chunk][region], where the region
// holds the forward prep's output (live during the state scan) or, after it,
// the backward prep's output followed by Gc.  With `overlap` the two uses get
// regions of their own, so that the state scan and the reverse scan (which
// reads neither S0 nor U) can run at the same time on two streams.
template <typename T, int D>
struct BwdLayout {
  size_t s0, u, region, pt, wtn, gm, gst, total;
  BwdLayout(int64_t nch, bool overlap) {
    const size_t n = (size_t)nch;
    s0 = 0;
    u = al256(n * D * D * sizeof(T));
    region = u + al256(n * CHUNK * D * sizeof(T));
    pt = overlap ? region + al256(carve_bytes<T, D>(nch)) : region;
    wtn = pt + al256(n * CHUNK * CHUNK * sizeof(T));
    gm = wtn + al256(n * CHUNK * D * sizeof(T));
    gst = gm + al256(n * GM_FLOATS * 4);
    const size_t bwd_end = gst + al256(n * D * D * sizeof(T));
    const size_t fwd_end = region + al256(carve_bytes<T, D>(nch));
    total = bwd_end > fwd_end ? bwd_end : fwd_end;
  }
  GdnBwdWs<T, D> carve(void* ws) const {
    char* p = (char*)ws;
    GdnBwdWs<T, D> w;
    w.pt = (T*)(p + pt);
    w.wtn = (T*)(p + wtn);
    w.gm = (float*)(p + gm);
    w.gst = (T*)(p + gst);
    return w;
  }
};

size_t gdn_bwd_ws_bytes(int io_is_bf16, int B, int H, int L, int D, bool overlap) {
  const int64_t nch = (int64_t)B * H * (L / CHUNK);
  if (io_is_bf16)
    return D == 64 ? BwdLayout<bf16, 64>(nch, overlap).total : BwdLayout<bf16, 128>(nch, overlap).total;
  return D == 64 ? BwdLayout<float, 64>(nch, overlap).total : BwdLayout<float, 128>(nch, overlap).total;
}

// ------------------------------------------------------------ backward prep
template <typename T, int D>
struct BwdPrepCfg {
  static constexpr int RL = kg_row<T, D>();
  static constexpr int KG_BYTES = 16 * RL * 4 * (int)sizeof(T);
  static constexpr int LTP = CHUNK + 1;
  static constexpr int OFF_KG = 0, OFF_LT = KG_BYTES;
  static constexpr int OFF_RS = OFF_LT + CHUNK * LTP * 4;
  static constexpr int OFF_GL = OFF_RS + 3 * 16 * 17 * 4;
  static constexpr int LDS = OFF_GL + 3 * CHUNK * 4;
  static constexpr int KF = D / 32, NT = D / 16;
};

// One workgroup per chunk-head: the per-token decays, L = diag(b) A and its
// inverse T (as the forward prep), P, and W = T diag(b gamma) K.  P^T and
// -W^T leave in the accumulator-shaped fragment order (row = s or d,
// contraction over tokens): wave w holds rows 16w + 4g + i of P and W, which
// are elements 4 (w & 1) + i of the fragments of token block w >> 1.
template <typename T, int D>
__global__ void __launch_bounds__(256) k_gdn_bwd_prep(const T* __restrict__ q, const T* __restrict__ k,
                                                      const float* __restrict__ alpha,
                                                      const float* __restrict__ beta, GdnBwdWs<T, D> bw, int L) {
  using C = BwdPrepCfg<T, D>;
  extern __shared__ __align__(16) unsigned char lds[];
  T* Kg = (T*)(lds + C::OFF_KG);
  float* LT = (float*)(lds + C::OFF_LT);
  float* Rs = (float*)(lds + C::OFF_RS);
  float* gl = (float*)(lds + C::OFF_GL);  // cumulative log2 decay
  float* bl = gl + CHUNK;                 // beta
  float* gbl = bl + CHUNK;                // beta * gamma
  const int nc = L / CHUNK;
  const int64_t ch = bid_x();
  const int64_t bh = ch / nc;
  const int cc = (int)(ch % nc);
  const int64_t tok0 = bh * L + (int64_t)cc * CHUNK;
  const int t = tid_x(), lane = lane_id(), w = wave_id();
  const int g = lane >> 4, c = lane & 15;

  constexpr int TASKS = (CHUNK / 4) * (D / 8);
  static_assert(TASKS <= 256, "one task per thread");
  const int kg = t / (D / 8), col = (t % (D / 8)) * 8;
  Frag<T> kr[4];
  if (t < TASKS) {
#pragma unroll
    for (int i = 0; i < 4; ++i) kr[i] = load8<T>(k + (tok0 + 4 * kg + i) * D + col);
  }
  Frag<T> ka[C::KF], qa[C::KF];
#pragma unroll
  for (int ks = 0; ks < C::KF; ++ks) {
    ka[ks] = load8<T>(k + (tok0 + 16 * w + c) * D + 32 * ks + 8 * g);
    qa[ks] = load8<T>(q + (tok0 + 16 * w + c) * D + 32 * ks + 8 * g);
  }
  if (w == 0) {
    const float a = alpha[tok0 + lane];
    const float bt = beta[tok0 + lane];
    float s = __builtin_amdgcn_logf(a);
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float o = __shfl_up(s, off, 64);
      if (lane >= off) s += o;
    }
    const float gC = __shfl(s, 63, 64);
    gl[lane] = s;
    bl[lane] = bt;
    gbl[lane] = bt * __builtin_amdgcn_exp2f(s);
    bw.gm[ch * GM_FLOATS + lane] = __builtin_amdgcn_exp2f(s);
    bw.gm[ch * GM_FLOATS + 80 + lane] = __builtin_amdgcn_exp2f(gC - s);
    if (lane == 0) bw.gm[ch * GM_FLOATS + 64] = __builtin_amdgcn_exp2f(gC);
  }
  if (t < TASKS) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      st4<T>(Kg + kg_index<C::RL>(kg, col + j), to_f32(frag_get<T>(kr[0], j)), to_f32(frag_get<T>(kr[1], j)),
             to_f32(frag_get<T>(kr[2], j)), to_f32(frag_get<T>(kr[3], j)));
    }
  }
  __syncthreads();

  // K K^T and Q K^T, rows 16w .. 16w+15 (B: key rows 16ct + c)
  f32x4 akk[4], apq[4];
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) {
    akk[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    apq[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int ks = 0; ks < C::KF; ++ks)
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      const Frag<T> bk = load8<T>(k + (tok0 + 16 * ct + c) * D + 32 * ks + 8 * g);
      mma(akk[ct], ka[ks], bk);
      mma(apq[ct], qa[ks], bk);
    }
  const int hb = w & 1, kb = w >> 1;
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) {
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * w + 4 * g + i, s = 16 * ct + c;
      const float gm_ = __builtin_amdgcn_exp2f(gl[r] - gl[s]);
      LT[r * C::LTP + s] = (s < r) ? bl[r] * gm_ * akk[ct][i] : 0.f;
      p[i] = (s <= r) ? gm_ * apq[ct][i] : 0.f;
    }
    st4<T>(bw.pt + ((ch * 4 + ct) * 2 + kb) * 512 + lane * 8 + hb * 4, p[0], p[1], p[2], p[3]);
  }
  __syncthreads();
  lt_inverse64<C::LTP>(LT, Rs);

  // W = T diag(b gamma) K, rows 16w .. 16w+15 (T split into bf16 hi + lo)
  constexpr bool SPLIT = sizeof(T) == 2;
  f32x4 wa[C::NT];
#pragma unroll
  for (int n = 0; n < C::NT; ++n) wa[n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k2 = 0; k2 < 2; ++k2) {
    Frag<T> a2, a2l;
    const float* trow = LT + (16 * w + c) * C::LTP;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int tk = 32 * k2 + kmap_acc(g, j);
      const float x2 = trow[tk] * gbl[tk];
      frag_set(a2, j, x2);
      frag_set(a2l, j, x2 - to_f32(frag_get<T>(a2, j)));
    }
#pragma unroll
    for (int n = 0; n < C::NT; ++n) {
      const Frag<T> bk = ld4x2<T>(Kg + kg_index<C::RL>(8 * k2 + g, 16 * n + c),
                                  Kg + kg_index<C::RL>(8 * k2 + 4 + g, 16 * n + c));
      mma(wa[n], a2, bk);
      if (SPLIT) mma(wa[n], a2l, bk);
    }
  }
#pragma unroll
  for (int n = 0; n < C::NT; ++n)
    st4<T>(bw.wtn + ((ch * C::NT + n) * 2 + kb) * 512 + lane * 8 + hb * 4, -wa[n][0], -wa[n][1], -wa[n][2],
           -wa[n][3]);
}

// -------------------------------------------------------------- reverse scan
template <typename T, int D, int DVT>
struct BwdScanOps {
  static constexpr int KF = D / 32, NV = DVT / 16, DTW = D / 64;
  Frag<T> ka[KF];      // K rows 16w + c (contraction d, contiguous)
  Frag<T> pt[2];       // P^T, row tile w
  Frag<T> wt[DTW][2];  // -W^T, d tiles DTW w + x
  // Q^T (rows d, tokens in the accumulator-shaped map).  bf16, D = 128: the
  // chunk's Q rows, 16 bytes per piece (pieces tid + 256 i), for the
  // transposed LDS reads; otherwise the fragments gathered from q directly
  static constexpr bool QTR = sizeof(T) == 2 && D == 128;
  bf16x8 qv[QTR ? 4 : 1];
  Frag<T> qt[QTR ? 1 : DTW][2];
  float dov[2][NV][8]; // d_o at tokens 32 k2 + kmap_acc(g, j), columns dv0 + 16 n + c
  f32x4 gk[2][2];      // gamma at tokens 32 k2 + 4g + i and 32 k2 + 16 + 4g + i
  f32x4 ek;            // exp(g_C - g) at rows 16w + 4g + i
  float gC;
  int route;
};

template <typename T, int D, int DVT>
__device__ __forceinline__ void bwd_scan_load(BwdScanOps<T, D, DVT>& op, const GdnBwdWs<T, D>& bw, const T* kh,
                                              const T* qh, const float* doh, const int32_t* rt, int64_t bh, int nc,
                                              int cc, int dv0) {
  using O = BwdScanOps<T, D, DVT>;
  constexpr int NT = D / 16;
  const int lane = lane_id(), w = wave_id();
  const int g = lane >> 4, c = lane & 15;
  const int64_t ch = bh * nc + cc;
  if constexpr (O::QTR) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = tid_x() + 256 * i;
      op.qv[i] = *reinterpret_cast<const bf16x8*>(qh + ((int64_t)cc * CHUNK + (e >> 4)) * D + 8 * (e & 15));
    }
  } else {
#pragma unroll
    for (int x = 0; x < O::DTW; ++x)
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
        for (int j = 0; j < 8; ++j)
          op.qt[x][k2].v[j] = qh[((int64_t)cc * CHUNK + 32 * k2 + kmap_acc(g, j)) * D + 16 * (O::DTW * w + x) + c];
  }
#pragma unroll
  for (int ks = 0; ks < O::KF; ++ks) op.ka[ks] = load8<T>(kh + ((int64_t)cc * CHUNK + 16 * w + c) * D + 32 * ks + 8 * g);
#pragma unroll
  for (int k2 = 0; k2 < 2; ++k2) op.pt[k2] = load8<T>(bw.pt + ((ch * 4 + w) * 2 + k2) * 512 + lane * 8);
#pragma unroll
  for (int x = 0; x < O::DTW; ++x)
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
      const int dt = O::DTW * w + x;
      op.wt[x][k2] = load8<T>(bw.wtn + ((ch * NT + dt) * 2 + k2) * 512 + lane * 8);
    }
#pragma unroll
  for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
    for (int n = 0; n < O::NV; ++n)
#pragma unroll
      for (int j = 0; j < 8; ++j)
        op.dov[k2][n][j] = doh[((int64_t)cc * CHUNK + 32 * k2 + kmap_acc(g, j)) * D + dv0 + 16 * n + c];
  const float* gm = bw.gm + ch * GM_FLOATS;
#pragma unroll
  for (int k2 = 0; k2 < 2; ++k2) {
    op.gk[k2][0] = *reinterpret_cast<const f32x4*>(gm + 32 * k2 + 4 * g);
    op.gk[k2][1] = *reinterpret_cast<const f32x4*>(gm + 32 * k2 + 16 + 4 * g);
  }
  op.ek = *reinterpret_cast<const f32x4*>(gm + 80 + 16 * w + 4 * g);
  op.gC = gm[64];
  op.route = rt[cc];
}

// One workgroup per (b, h, DVT-column slice of Dv), chunks in reverse.  The
// fp32 carried gradient lives in registers (rows d = 16 (DTW w + x) + 4g + i,
// columns dv0 + 16 n + c), a T copy transposed in LDS feeds K Gc; dU goes
// through LDS key groups into -W^T dU, and (bf16, D = 128) the chunk's Q rows
// (loaded with the chunk's other operands, one chunk ahead) through LDS into
// Q^T by transposed reads.  Per chunk: Gc -> workspace, then
//   Z = K Gc;  dU = P^T dO + [committed] diag(e) Z
//   Gc <- [committed ? gamma_C : 1] Gc + Q^T (gamma dO) + (-W^T) dU.
template <typename T, int D, int DVT>
__global__ void __launch_bounds__(256, 1)
    k_gdn_bwd_scan(const T* __restrict__ q, const T* __restrict__ k, const float* __restrict__ d_o,
                   const int32_t* __restrict__ route,
                   GdnBwdWs<T, D> bw, const float* __restrict__ dS_final, T* __restrict__ g_out,
                   float* __restrict__ dS_init, int H, int L, int G) {
  using O = BwdScanOps<T, D, DVT>;
  constexpr int SPP = D + 16 / (int)sizeof(T);
  __shared__ __align__(16) T Gp[2][DVT * SPP];
  constexpr int URL = kg_row<T, DVT>();
  __shared__ __align__(16) T Ug[(CHUNK / 4) * URL * 4];
  // Q rows of the chunk (bf16, D = 128): 16-byte piece q of row r at slot
  // q ^ ((r & 7) << 1), which keeps the transposed reads conflict-free
  __shared__ __align__(16) unsigned char Qs[O::QTR ? CHUNK * 256 : 16];

  const int nc = L / CHUNK;
  const int nvt = D / DVT;
  const int total = (int)grid_dim_x();
  const int BH = total / nvt;
  int logical = bid_x();
  if ((BH & 7) == 0) logical = (bid_x() & 7) * (total >> 3) + (bid_x() >> 3);
  const int64_t bh = logical / nvt;
  const int vt = logical % nvt;
  const int b = (int)(bh / H), h = (int)(bh % H);
  const int grp = (G == 1) ? 0 : h;
  const int32_t* rt = route + ((int64_t)b * G + grp) * nc;
  const int dv0 = vt * DVT;
  const T* kh = k + bh * L * D;
  const T* qh = q + bh * L * D;
  const float* doh = d_o + bh * L * D;
  const int lane = lane_id(), w = wave_id();
  const int g = lane >> 4, c = lane & 15;

  f32x4 sm[O::DTW][O::NV];
#pragma unroll
  for (int x = 0; x < O::DTW; ++x)
#pragma unroll
    for (int n = 0; n < O::NV; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int dk = 16 * (w * O::DTW + x) + 4 * g + i;
        sm[x][n][i] = dS_final ? dS_final[(bh * D + dk) * D + dv0 + 16 * n + c] : 0.f;
      }
  int sb = 0;
  auto write_g = [&](int buf) {
#pragma unroll
    for (int x = 0; x < O::DTW; ++x)
#pragma unroll
      for (int n = 0; n < O::NV; ++n)
        st4<T>(&Gp[buf][(16 * n + c) * SPP + 16 * (w * O::DTW + x) + 4 * g], sm[x][n][0], sm[x][n][1], sm[x][n][2],
               sm[x][n][3]);
  };
  write_g(0);
  lds_barrier();

  auto step = [&](const O& op, int cc) {
    const int64_t ch = bh * nc + cc;
    // Q rows -> LDS (the previous chunk's reads of Qs ended before its last
    // barrier; the barrier after the dU stores publishes these)
    if constexpr (O::QTR) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = tid_x() + 256 * i, r = e >> 4;
        *reinterpret_cast<bf16x8*>(Qs + r * 256 + (((e & 15) ^ ((r & 7) << 1)) * 16)) = op.qv[i];
      }
    }
#pragma unroll
    for (int x = 0; x < O::DTW; ++x)
#pragma unroll
      for (int n = 0; n < O::NV; ++n)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int dk = 16 * (w * O::DTW + x) + 4 * g + i;
          g_out[(ch * D + dk) * D + dv0 + 16 * n + c] = from_f32<T>(sm[x][n][i]);
        }
    Frag<T> bg[O::KF][O::NV];
#pragma unroll
    for (int ks = 0; ks < O::KF; ++ks)
#pragma unroll
      for (int n = 0; n < O::NV; ++n) bg[ks][n] = load8<T>(&Gp[sb][(16 * n + c) * SPP + 32 * ks + 8 * g]);
    f32x4 z[O::NV], xa[O::NV];
#pragma unroll
    for (int n = 0; n < O::NV; ++n) {
      z[n] = f32x4{0.f, 0.f, 0.f, 0.f};
      xa[n] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int ks = 0; ks < O::KF; ++ks)
#pragma unroll
      for (int n = 0; n < O::NV; ++n) mma(z[n], op.ka[ks], bg[ks][n]);
    Frag<T> bdo[2][O::NV], bdg[2][O::NV];
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
      for (int n = 0; n < O::NV; ++n)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float dv = op.dov[k2][n][j];
          const float gm_ = j < 4 ? op.gk[k2][0][j] : op.gk[k2][1][j - 4];
          frag_set(bdo[k2][n], j, dv);
          frag_set(bdg[k2][n], j, dv * gm_);
        }
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
      for (int n = 0; n < O::NV; ++n) mma(xa[n], op.pt[k2], bdo[k2][n]);
    const bool lin = op.route == 1;
    const float gce = lin ? op.gC : 1.f;
    f32x4 du[O::NV];
#pragma unroll
    for (int n = 0; n < O::NV; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i) du[n][i] = xa[n][i] + (lin ? op.ek[i] * z[n][i] : 0.f);
#pragma unroll
    for (int n = 0; n < O::NV; ++n) st4<T>(&Ug[kg_index<URL>(4 * w + g, 16 * n + c)], du[n][0], du[n][1], du[n][2], du[n][3]);
    lds_barrier();
    Frag<T> bu[2][O::NV];
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
      for (int n = 0; n < O::NV; ++n)
        bu[k2][n] = ld4x2<T>(&Ug[kg_index<URL>(8 * k2 + g, 16 * n + c)], &Ug[kg_index<URL>(8 * k2 + 4 + g, 16 * n + c)]);
    // Q^T A fragments (rows d, tokens in the accumulator-shaped map): lane c
    // of group g reads rows 32 k2 + 4g + c / 4 and +16, columns 16 dt + 4 (c % 4) .. +3
    Frag<T> qt[O::DTW][2];
#pragma unroll
    for (int x = 0; x < O::DTW; ++x)
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
        if constexpr (O::QTR) {
          const int dt = O::DTW * w + x;
          const int colq = (16 * dt + 4 * (c & 3)) >> 3, half = (c & 1) * 8;
          const int r0 = 32 * k2 + 4 * g + (c >> 2), r1 = r0 + 16;
          const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) v4i16*)(Qs + r0 * 256 + ((colq ^ ((r0 & 7) << 1)) * 16) + half));
          const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) v4i16*)(Qs + r1 * 256 + ((colq ^ ((r1 & 7) << 1)) * 16) + half));
          qt[x][k2].v = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        } else {
          qt[x][k2] = op.qt[x][k2];
        }
      }
#pragma unroll
    for (int x = 0; x < O::DTW; ++x)
#pragma unroll
      for (int n = 0; n < O::NV; ++n) {
        f32x4 acc = sm[x][n] * gce;
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
          mma(acc, qt[x][k2], bdg[k2][n]);
          mma(acc, op.wt[x][k2], bu[k2][n]);
        }
        sm[x][n] = acc;
      }
    write_g(sb ^ 1);
    sb ^= 1;
    lds_barrier();
  };

  O ops[2];
  bwd_scan_load<T, D, DVT>(ops[0], bw, kh, qh, doh, rt, bh, nc, nc - 1, dv0);
  int cc = nc - 1;
  for (; cc >= 1; cc -= 2) {
    bwd_scan_load<T, D, DVT>(ops[1], bw, kh, qh, doh, rt, bh, nc, cc - 1, dv0);
    step(ops[0], cc);
    bwd_scan_load<T, D, DVT>(ops[0], bw, kh, qh, doh, rt, bh, nc, cc >= 2 ? cc - 2 : 0, dv0);
    step(ops[1], cc - 1);
  }
  if (cc == 0) step(ops[0], 0);
  if (dS_init) {
#pragma unroll
    for (int x = 0; x < O::DTW; ++x)
#pragma unroll
      for (int n = 0; n < O::NV; ++n)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int dk = 16 * (w * O::DTW + x) + 4 * g + i;
          dS_init[(bh * D + dk) * D + dv0 + 16 * n + c] = sm[x][n][i];
        }
  }
}

// ------------------------------------------------------- per-chunk gradients
template <typename T, int D>
struct BwdChunkCfg {
  static constexpr int CT = D / 64;  // 16-column tiles per wave of a 64 x D product
  static constexpr int KV = D / 32;  // contraction steps over D
  static constexpr int PM = 68;      // pitch of the fp32 64 x 64 matrices (16-byte rows)
  static constexpr int PT = D + 16 / (int)sizeof(T);
  // U and K staged in LDS (else read from global memory); dU is computed
  // here and always lives in LDS
  static constexpr bool FIT = sizeof(T) == 2 || D == 64;
  static constexpr int M_BYTES = CHUNK * PM * 4;
  static constexpr int T_BYTES = CHUNK * PT * (int)sizeof(T);
  static constexpr int OFF_TL = 0, OFF_AL = M_BYTES, OFF_FL = 2 * M_BYTES, OFF_ML = 3 * M_BYTES;
  static constexpr int OFF_X1 = 4 * M_BYTES;
  static constexpr int OFF_DUL = OFF_X1 + T_BYTES;
  static constexpr int OFF_UL = OFF_DUL + T_BYTES;
  static constexpr int OFF_KL = OFF_UL + (FIT ? T_BYTES : 0);
  static constexpr int OFF_VEC = OFF_KL + (FIT ? T_BYTES : 0);
  static_assert(3 * 16 * 17 * 4 <= T_BYTES, "the inverse's scratch fits in X1");
  // g2, gamma, e, beta, beta gamma, alpha; partial row sums pbeta, pgam,
  // pts, cdg [4][64]; rdg, rbeta [64]; red [4]
  static constexpr int VEC_FLOATS = 6 * 64 + 4 * 4 * 64 + 2 * 64 + 4;
  static constexpr int LDS = OFF_VEC + VEC_FLOATS * 4;
  static_assert(LDS <= 160 * 1024, "LDS");
};

template <typename T>
__device__ __forceinline__ Frag<T> frag_f32(const float* p) {  // 8 contiguous fp32 (16-byte aligned)
  const f32x4 a = *reinterpret_cast<const f32x4*>(p), b = *reinterpret_cast<const f32x4*>(p + 4);
  Frag<T> f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    frag_set(f, j, a[j]);
    frag_set(f, 4 + j, b[j]);
  }
  return f;
}
// sum over the 16 lanes of a row group; lane c = 0 of group g writes the 4
// rows base + 4g + i
__device__ __forceinline__ void row_partials(const f32x4& v, float* dst, int g, int c) {
  f32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = dpp_group_sum<16>(v[i]);
  if (c == 0) *reinterpret_cast<f32x4*>(dst + 4 * g) = r;
}

// One workgroup per chunk-head.  Wave w owns row tile w of the 64 x 64
// products (rows t = 16w + 4g + i) and columns 16 (CT w + ct) + c of the
// 64 x D products (all four row tiles).  All contractions use the row map
// (8g + j), operands from LDS, or from global memory where they are read
// once (dO, the S0 / Gc fragments).  T and dU are computed here rather than
// stored by the preps and the reverse scan: T by the preps' own steps (so
// the same values), dU from the reverse scan's bf16 operands.
template <typename T, int D>
__global__ void __launch_bounds__(256, 1)
    k_gdn_bwd_chunk(const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
                    const float* __restrict__ alpha, const float* __restrict__ beta, const float* __restrict__ d_o,
                    const int32_t* __restrict__ route, GdnBwdWs<T, D> bw, const T* __restrict__ s0,
                    const T* __restrict__ u, float* __restrict__ dq,
                    float* __restrict__ dk, float* __restrict__ dv, float* __restrict__ dalpha,
                    float* __restrict__ dbeta, float* __restrict__ dgate, int H, int L, int G) {
  using C = BwdChunkCfg<T, D>;
  constexpr int CT = C::CT, KV = C::KV, PM = C::PM, PT = C::PT;
  extern __shared__ __align__(16) unsigned char lds[];
  float* Tl = (float*)(lds + C::OFF_TL);
  float* Al = (float*)(lds + C::OFF_AL);  // A (decayed), then dT, then E
  float* Fl = (float*)(lds + C::OFF_FL);
  float* Ml = (float*)(lds + C::OFF_ML);
  T* X1 = (T*)(lds + C::OFF_X1);          // TdU, then VmR
  float* vec = (float*)(lds + C::OFF_VEC);
  float* g2 = vec;
  float* gam = vec + 64;
  float* ekv = vec + 128;
  float* bet = vec + 192;
  float* bgm = vec + 256;
  float* alp = vec + 320;
  float* pbeta = vec + 384;
  float* pgam = pbeta + 256;
  float* pts = pgam + 256;
  float* cdg = pts + 256;
  float* rdg = cdg + 256;
  float* rbeta = rdg + 64;
  float* red = rbeta + 64;

  const int nc = L / CHUNK;
  const int64_t ch = bid_x();
  const int64_t bh = ch / nc;
  const int cc = (int)(ch % nc);
  const int b = (int)(bh / H), h = (int)(bh % H);
  const int grp = (G == 1) ? 0 : h;
  const bool lin = route[((int64_t)b * G + grp) * nc + cc] == 1;
  const int64_t tok0 = bh * L + (int64_t)cc * CHUNK;
  const int t = tid_x(), lane = lane_id(), w = wave_id();
  const int g = lane >> 4, c = lane & 15;

  const T* qc = q + tok0 * D;
  const T* kc = k + tok0 * D;
  const T* vc = v + tok0 * D;
  const float* doc = d_o + tok0 * D;
  const T* uc = u + tok0 * D;
  const T* gst = bw.gst;
  // U, K rows: LDS copies (pitch PT) or global memory (pitch D); dU rows in LDS (pitch PT)
  const T* Ub = C::FIT ? (const T*)(lds + C::OFF_UL) : uc;
  T* dUl = (T*)(lds + C::OFF_DUL);
  const T* dUb = dUl;
  const T* Kb = C::FIT ? (const T*)(lds + C::OFF_KL) : kc;
  constexpr int UP = C::FIT ? PT : D;

  // ---- phase 0: decays, staging, the S0^T / Gc^T fragments
  if (w == 0) {
    const float a = alpha[tok0 + lane];
    const float bt = beta[tok0 + lane];
    float s = __builtin_amdgcn_logf(a);
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float o = __shfl_up(s, off, 64);
      if (lane >= off) s += o;
    }
    const float gC = __shfl(s, 63, 64);
    const float gm_ = __builtin_amdgcn_exp2f(s);
    g2[lane] = s;
    gam[lane] = gm_;
    ekv[lane] = __builtin_amdgcn_exp2f(gC - s);
    bet[lane] = bt;
    bgm[lane] = bt * gm_;
    alp[lane] = a;
  }
  if constexpr (C::FIT) {
    // a fixed trip count, so that every load is in flight before the first
    // LDS store (one workgroup per CU: nothing else hides their latency)
    constexpr int PER = 16 / (int)sizeof(T), NP = CHUNK * D / PER, NI = NP / 256;
    static_assert(NP % 256 == 0, "staging loop");
    T* Ul = (T*)(lds + C::OFF_UL);
    T* Kl = (T*)(lds + C::OFF_KL);
    f32x4 us[NI], ks[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int e = t + 256 * i, r = e / (D / PER), cl = (e % (D / PER)) * PER;
      us[i] = *reinterpret_cast<const f32x4*>(uc + r * D + cl);
      ks[i] = *reinterpret_cast<const f32x4*>(kc + r * D + cl);
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int e = t + 256 * i, r = e / (D / PER), cl = (e % (D / PER)) * PER;
      *reinterpret_cast<f32x4*>(Ul + r * PT + cl) = us[i];
      *reinterpret_cast<f32x4*>(Kl + r * PT + cl) = ks[i];
    }
  }
  // S0^T and Gc^T B fragments of this wave's columns: column d = 16 (CT w +
  // ct) + c, contraction over v = 32 kv + 8g + j (contiguous rows of S0, Gc)
  Frag<T> s0f[CT][KV], gf[CT][KV];
  float sg = 0.f;
#pragma unroll
  for (int ct = 0; ct < CT; ++ct)
#pragma unroll
    for (int kv = 0; kv < KV; ++kv) {
      const int64_t off = (ch * D + 16 * (CT * w + ct) + c) * D + 32 * kv + 8 * g;
      s0f[ct][kv] = load8<T>(s0 + off);
      gf[ct][kv] = load8<T>(gst + off);
#pragma unroll
      for (int j = 0; j < 8; ++j) sg += to_f32(frag_get<T>(s0f[ct][kv], j)) * to_f32(frag_get<T>(gf[ct][kv], j));
    }
  sg = wave_sum64(sg);
  if (lane == 0) red[w] = sg;
  __syncthreads();

  // ---- phase 1 (row tile w): A, L = diag(b) A (-> Tl), P (-> Ml), dP
  f32x4 akk[4], apq[4], dpa[4];
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) {
    akk[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    apq[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    dpa[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int kv = 0; kv < KV; ++kv) {
    const Frag<T> ak = load8<T>(Kb + (16 * w + c) * UP + 32 * kv + 8 * g);
    const Frag<T> aq = load8<T>(qc + (16 * w + c) * D + 32 * kv + 8 * g);
    const Frag<T> ad = frag_f32<T>(doc + (16 * w + c) * D + 32 * kv + 8 * g);
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      const Frag<T> bk = load8<T>(Kb + (16 * ct + c) * UP + 32 * kv + 8 * g);
      const Frag<T> bu = load8<T>(Ub + (16 * ct + c) * UP + 32 * kv + 8 * g);
      mma(akk[ct], ak, bk);
      mma(apq[ct], aq, bk);
      mma(dpa[ct], ad, bu);
    }
  }
  {
    f32x4 rsum = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      float csum = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * w + 4 * g + i, s = 16 * ct + c;
        const float gmx = __builtin_amdgcn_exp2f(g2[r] - g2[s]);
        Al[r * PM + s] = (s < r) ? gmx * akk[ct][i] : 0.f;
        Tl[r * PM + s] = (s < r) ? bet[r] * gmx * akk[ct][i] : 0.f;  // as the preps form it
        const float p = (s <= r) ? gmx * apq[ct][i] : 0.f;
        Ml[r * PM + s] = p;
        const float dp = (s <= r) ? dpa[ct][i] : 0.f;
        Fl[r * PM + s] = dp * gmx;
        rsum[i] += dp * p;
        csum += dp * p;
      }
      csum = group4_sum(csum);
      if (g == 0) cdg[w * 64 + 16 * ct + c] = csum;
    }
    row_partials(rsum, rdg + 16 * w, g, c);
  }
  __syncthreads();

  // ---- phase 1b (columns of wave w): dU = P^T dO + [committed] diag(e) K Gc
  // -> dUl, the reverse scan's dU from the same bf16 operands (dO rounded to
  // T, Gc as stored); then T = (I + L)^-1 in place in Tl, whose barriers also
  // publish dUl
  // (one 16-column tile at a time: 32 accumulator registers)
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    const int col = 16 * (CT * w + ct) + c;
    f32x4 dua[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) dua[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
      const int s0_ = 32 * k2 + 8 * g;
      const Frag<T> bdo = frag_fn<T>([&](int j) { return doc[(s0_ + j) * D + col]; });
#pragma unroll
      for (int rt = 0; rt < 4; ++rt)
        mma(dua[rt], frag_fn<T>([&](int j) { return Ml[(s0_ + j) * PM + 16 * rt + c]; }), bdo);
    }
    if (lin) {
      f32x4 kga[4];
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) kga[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kv = 0; kv < KV; ++kv) {
        const int d0 = 32 * kv + 8 * g;
        const Frag<T> bgc = frag_fn<T>([&](int j) { return to_f32(gst[(ch * D + d0 + j) * D + col]); });
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) mma(kga[rt], load8<T>(Kb + (16 * rt + c) * UP + 32 * kv + 8 * g), bgc);
      }
#pragma unroll
      for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) dua[rt][i] += ekv[16 * rt + 4 * g + i] * kga[rt][i];
    }
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) dUl[(16 * rt + 4 * g + i) * PT + col] = from_f32<T>(dua[rt][i]);
  }
  __builtin_amdgcn_sched_barrier(0);
  lt_inverse64<PM>(Tl, (float*)X1);

  // ---- phase 2 (columns of wave w): dO S0^T, U Gc^T, T^T dU, A U, TdU S0^T
  f32x4 dqa[4][CT], dka[4][CT];
  f32x4 vb[4], vg[4];  // per-row partial sums for dbeta, dgamma
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    vb[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
    vg[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  {
    f32x4 vt[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      f32x4 dos[CT], ug[CT];
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        dos[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
        ug[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int kv = 0; kv < KV; ++kv) {
        const Frag<T> ad = frag_f32<T>(doc + (16 * rt + c) * D + 32 * kv + 8 * g);
        const Frag<T> au = load8<T>(Ub + (16 * rt + c) * UP + 32 * kv + 8 * g);
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          mma(dos[ct], ad, s0f[ct][kv]);
          mma(ug[ct], au, gf[ct][kv]);
        }
      }
      vt[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        const int col = 16 * (CT * w + ct) + c;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * rt + 4 * g + i;
          const float qv = to_f32(qc[r * D + col]);
          const float kv_ = to_f32(Kb[r * UP + col]);
          dqa[rt][ct][i] = gam[r] * dos[ct][i];
          dka[rt][ct][i] = lin ? ekv[r] * ug[ct][i] : 0.f;
          vg[rt][i] += qv * dos[ct][i];
          vt[rt][i] += ekv[r] * kv_ * ug[ct][i];
        }
      }
    }
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) row_partials(vt[rt], pts + w * 64 + 16 * rt, g, c);
  }
  // TdU = T^T dU -> dv, X1;  A U -> VmR (held until X1 is free).  The B
  // fragments (columns of dU and U) do not depend on the row tile.
  f32x4 vmr[4][CT];
  {
    f32x4 tdu[4][CT], au[4][CT];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        tdu[rt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
        au[rt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
      const int t0 = 32 * k2 + 8 * g;
      Frag<T> bdu[CT], bu[CT];
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        const int col = 16 * (CT * w + ct) + c;
        bdu[ct] = frag_fn<T>([&](int j) { return to_f32(dUb[(t0 + j) * PT + col]); });
        bu[ct] = frag_fn<T>([&](int j) { return to_f32(Ub[(t0 + j) * UP + col]); });
      }
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        const Frag<T> at = frag_fn<T>([&](int j) { return Tl[(t0 + j) * PM + 16 * rt + c]; });
        const Frag<T> aa = frag_f32<T>(Al + (16 * rt + c) * PM + t0);
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          mma(tdu[rt][ct], at, bdu[ct]);
          mma(au[rt][ct], aa, bu[ct]);
        }
      }
    }
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        const int col = 16 * (CT * w + ct) + c;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * rt + 4 * g + i;
          dv[(tok0 + r) * D + col] = bet[r] * tdu[rt][ct][i];
          vb[rt][i] += to_f32(vc[r * D + col]) * tdu[rt][ct][i];
          X1[r * PT + col] = from_f32<T>(tdu[rt][ct][i]);
          vmr[rt][ct][i] = to_f32(Ub[r * UP + col]) + bet[r] * au[rt][ct][i];
        }
      }
  }
  __syncthreads();
  // TdW = -TdU S0^T
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    f32x4 tw[CT];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) tw[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kv = 0; kv < KV; ++kv) {
      const Frag<T> ax = load8<T>(X1 + (16 * rt + c) * PT + 32 * kv + 8 * g);
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) mma(tw[ct], ax, s0f[ct][kv]);
    }
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      const int col = 16 * (CT * w + ct) + c;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * rt + 4 * g + i;
        const float tdw = -tw[ct][i];
        const float kw = to_f32(Kb[r * UP + col]) * tdw;
        dka[rt][ct][i] += bgm[r] * tdw;
        vb[rt][i] += gam[r] * kw;
        vg[rt][i] += bet[r] * kw;
      }
    }
  }
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    row_partials(vb[rt], pbeta + w * 64 + 16 * rt, g, c);
    row_partials(vg[rt], pgam + w * 64 + 16 * rt, g, c);
  }
  __syncthreads();
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int i = 0; i < 4; ++i) X1[(16 * rt + 4 * g + i) * PT + 16 * (CT * w + ct) + c] = from_f32<T>(vmr[rt][ct][i]);
  __syncthreads();

  // ---- phase 3 (row tile w): dT = dU VmR^T, M1 = T^T dT, dM = -M1 T^T
  {
    f32x4 dta[4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) dta[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kv = 0; kv < KV; ++kv) {
      const Frag<T> a = load8<T>(dUb + (16 * w + c) * PT + 32 * kv + 8 * g);
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) mma(dta[ct], a, load8<T>(X1 + (16 * ct + c) * PT + 32 * kv + 8 * g));
    }
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
#pragma unroll
      for (int i = 0; i < 4; ++i) Al[(16 * w + 4 * g + i) * PM + 16 * ct + c] = dta[ct][i];
  }
  __syncthreads();
  {
    f32x4 m1[4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) m1[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
      const int t0 = 32 * k2 + 8 * g;
      const Frag<T> a = frag_fn<T>([&](int j) { return Tl[(t0 + j) * PM + 16 * w + c]; });
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
        mma(m1[ct], a, frag_fn<T>([&](int j) { return Al[(t0 + j) * PM + 16 * ct + c]; }));
    }
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
#pragma unroll
      for (int i = 0; i < 4; ++i) Ml[(16 * w + 4 * g + i) * PM + 16 * ct + c] = m1[ct][i];
  }
  __syncthreads();
  {
    f32x4 dma[4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) dma[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
      const int k0 = 32 * k2 + 8 * g;
      const Frag<T> a = frag_f32<T>(Ml + (16 * w + c) * PM + k0);
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) mma(dma[ct], a, frag_f32<T>(Tl + (16 * ct + c) * PM + k0));
    }
    f32x4 rb = f32x4{0.f, 0.f, 0.f, 0.f}, rg = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      float csum = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * w + 4 * g + i, s = 16 * ct + c;
        const float gmx = __builtin_amdgcn_exp2f(g2[r] - g2[s]);
        const float adec = (s < r) ? gmx * akk[ct][i] : 0.f;
        const float dm = (s < r) ? -dma[ct][i] : 0.f;
        const float da = bet[r] * dm;
        rb[i] += dm * adec;
        rg[i] += da * adec;
        csum += da * adec;
        Al[r * PM + s] = da * gmx;  // E
      }
      csum = group4_sum(csum);
      if (g == 0) cdg[w * 64 + 16 * ct + c] += csum;
    }
    f32x4 r1, r2;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      r1[i] = dpp_group_sum<16>(rb[i]);
      r2[i] = dpp_group_sum<16>(rg[i]);
    }
    if (c == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        rbeta[16 * w + 4 * g + i] = r1[i];
        rdg[16 * w + 4 * g + i] += r2[i];
      }
    }
  }
  __syncthreads();

  // ---- phase 4 (columns of wave w): E K, E^T K, F K, F^T Q; store dq, dk.
  // The B fragments (columns of K and Q) do not depend on the row tile.
#pragma unroll
  for (int k2 = 0; k2 < 2; ++k2) {
    const int t0 = 32 * k2 + 8 * g;
    Frag<T> bk[CT], bq[CT];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      const int col = 16 * (CT * w + ct) + c;
      bk[ct] = frag_fn<T>([&](int j) { return to_f32(Kb[(t0 + j) * UP + col]); });
      bq[ct] = frag_fn<T>([&](int j) { return to_f32(qc[(t0 + j) * D + col]); });
    }
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      const Frag<T> ae = frag_f32<T>(Al + (16 * rt + c) * PM + t0);
      const Frag<T> aet = frag_fn<T>([&](int j) { return Al[(t0 + j) * PM + 16 * rt + c]; });
      const Frag<T> af = frag_f32<T>(Fl + (16 * rt + c) * PM + t0);
      const Frag<T> aft = frag_fn<T>([&](int j) { return Fl[(t0 + j) * PM + 16 * rt + c]; });
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        mma(dka[rt][ct], ae, bk[ct]);
        mma(dka[rt][ct], aet, bk[ct]);
        mma(dqa[rt][ct], af, bk[ct]);
        mma(dka[rt][ct], aft, bq[ct]);
      }
    }
  }
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      const int col = 16 * (CT * w + ct) + c;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t o = (tok0 + 16 * rt + 4 * g + i) * D + col;
        dq[o] = dqa[rt][ct][i];
        dk[o] = dka[rt][ct][i];
      }
    }
  __syncthreads();

  // ---- phase 5 (wave 0, lane = token): dbeta, d log-decay, dalpha, gate
  if (w == 0) {
    const int r = lane;
    float db_ = rbeta[r], dgm = 0.f, ts = 0.f, cd = 0.f;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) {
      db_ += pbeta[ww * 64 + r];
      dgm += pgam[ww * 64 + r];
      ts += pts[ww * 64 + r];
      cd += cdg[ww * 64 + r];
    }
    const float sgt = red[0] + red[1] + red[2] + red[3];
    const float tsum = wave_sum64(ts);
    float dg = rdg[r] - cd + gam[r] * dgm - (lin ? ts : 0.f);
    if (r == CHUNK - 1 && lin) dg += tsum + gam[CHUNK - 1] * sgt;
    // d log alpha_r = sum over t >= r of dg_t
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float o = __shfl_down(dg, off, 64);
      if (lane + off < 64) dg += o;
    }
    dalpha[tok0 + r] = dg / alp[r];
    dbeta[tok0 + r] = db_;
    if (dgate && lane == 0) dgate[bh * nc + cc] = (gam[CHUNK - 1] - 1.f) * sgt + tsum;
  }
}

template <typename T, int D>
hipError_t launch_gdn_backward(const T* q, const T* k, const T* v, const float* alpha, const float* beta,
                               const int32_t* route, const float* S_init, const float* d_o, const float* dS_final,
                               float* dq, float* dk, float* dv, float* dalpha, float* dbeta, float* dS_init,
                               float* dgate, void* ws, int B, int H, int L, int G, hipStream_t st,
                               const SideStream& ov) {
  const int nc = L / CHUNK;
  const int64_t nch = (int64_t)B * H * nc;
  const bool overlap = ov.aux != nullptr;
  const BwdLayout<T, D> lay(nch, overlap);
  T* s0 = (T*)((char*)ws + lay.s0);
  T* u = (T*)((char*)ws + lay.u);
  GdnBwdWs<T, D> bw = lay.carve(ws);
  using PC = BwdPrepCfg<T, D>;
  hipError_t e = set_lds_limit((const void*)k_gdn_bwd_prep<T, D>, PC::LDS);
  if (e != hipSuccess) return e;
  // the backward prep and the reverse scan: on the helper stream beside the
  // forward's state mode (own regions), else after it on st (shared region)
  hipStream_t sb = overlap ? ov.aux : st;
  if (overlap) {
    if ((e = hipEventRecord(ov.fork, st)) != hipSuccess) return e;
    if ((e = hipStreamWaitEvent(ov.aux, ov.fork, 0)) != hipSuccess) return e;
  }
  auto reverse = [&]() -> hipError_t {
    hipLaunchKernelGGL((k_gdn_bwd_prep<T, D>), dim3((unsigned)nch), dim3(256), PC::LDS, sb, q, k, alpha, beta, bw,
                       L);
    hipError_t r = hipGetLastError();
    if (r != hipSuccess) return r;
    hipLaunchKernelGGL((k_gdn_bwd_scan<T, D, BWD_DVT>), dim3((unsigned)(B * H * (D / BWD_DVT))), dim3(256), 0, sb, q,
                       k, d_o, route, bw, dS_final, bw.gst, dS_init, H, L, G);
    return hipGetLastError();
  };
  if (overlap) e = reverse();
  if (e == hipSuccess)
    e = launch_gdn_states<T, D>(q, k, v, alpha, beta, route, S_init, s0, u, (char*)ws + lay.region, B, H, L, G, st);
  if (e == hipSuccess && !overlap) e = reverse();
  if (overlap) {  // joined also after a failed launch, so that nothing queued outlives the call's stream order
    const hipError_t ej = hipEventRecord(ov.join, ov.aux);
    if (ej == hipSuccess) {
      const hipError_t ew = hipStreamWaitEvent(st, ov.join, 0);
      if (e == hipSuccess) e = ew;
    } else if (e == hipSuccess) {
      e = ej;
    }
  }
  if (e != hipSuccess) return e;
  using CC = BwdChunkCfg<T, D>;
  if ((e = set_lds_limit((const void*)k_gdn_bwd_chunk<T, D>, CC::LDS)) != hipSuccess) return e;
  hipLaunchKernelGGL((k_gdn_bwd_chunk<T, D>), dim3((unsigned)nch), dim3(256), CC::LDS, st, q, k, v, alpha, beta, d_o,
                     route, bw, (const T*)s0, (const T*)u, dq, dk, dv, dalpha, dbeta, dgate, H, L, G);
  return hipGetLastError();
}

#define INST(T, D)                                                                                                  \
  template hipError_t launch_gdn_backward<T, D>(const T*, const T*, const T*, const float*, const float*,           \
                                                const int32_t*, const float*, const float*, const float*, float*,   \
                                                float*, float*, float*, float*, float*, float*, void*, int, int,    \
                                                int, int, hipStream_t, const SideStream&);
INST(float, 64)
INST(float, 128)
INST(bf16, 64)
INST(bf16, 128)
#undef INST

}  // namespace natsl
