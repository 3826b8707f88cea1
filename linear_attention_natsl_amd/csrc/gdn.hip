// Gated DeltaNet branch with per-chunk rollback.
//
// "Technische Samenvatting: Neural Attention Search Linear (NAtS-L)",
// Kernmechanismen 3: the model keeps a hidden state for the linear operation,
// pseudo-updates it through every chunk, and resets it to the chunk start when
// the chunk was not routed to the linear operation.  The recurrence itself is
// the gated delta rule (Gated DeltaNet is named in Kernmechanismen 1; the
// "Systematische Analyse van Hybride Lineaire Aandacht" summary describes this
// family as data-dependent gating plus a delta rule that erases stale content):
//   S_t = a_t (S_{t-1} - b_t k_t (k_t^T S_{t-1})) + b_t k_t v_t^T,  o_t = S_t^T q_t.
//
// Chunkwise form (exact up to rounding) for a chunk starting from state S0,
// with g_r = sum_{i<=r} log a_i and gamma_r = exp(g_r):
//   A = strict_tril(exp(g_r - g_i) k_r.k_i),  T = (I + diag(b) A)^-1
//   W = T diag(b gamma) K,  U~ = T diag(b) V,  U = U~ - W S0
//   P = tril(exp(g_r - g_i) q_r.k_i),  O = diag(gamma) Q S0 + P U
//   S_end = gamma_C S0 + K~^T U,  K~ = diag(exp(g_C - g_i)) K
// S_end replaces S0 only for linear-routed chunks (rollback otherwise).
//
// Two kernels:
//   k_gdn_prep  one workgroup per (b, h, chunk), fully parallel: K K^T and
//               Q K^T on MFMA, the 64x64 unit-lower-triangular inverse T in
//               LDS (fp32: 16x16 diagonal blocks by forward substitution, then
//               block rows), T diag(b) V and T diag(b gamma) K on MFMA; writes
//               -W, U~, P, the per-token decays and (except for the head form,
//               which reads K itself) K^T in exactly the per-lane fragment
//               order the scan consumes (every scan load is 16 B per lane,
//               1 KiB contiguous per wave).  T diag(b) and
//               T diag(b gamma) are split into bf16 hi + lo parts for their
//               products, so neither is rounded to bf16 precision; P is
//               stored as hi + lo except for the bf16 head-form scan, which
//               takes P in bf16 like -W and U; K^T stays exact (its
//               exp(g_C - g) scale is applied to U in fp32 by the scan).
//   k_gdn_scan_head (bf16, D = 128) and k_gdn_scan (otherwise): the scan,
//               sequential over chunks (see each kernel).  k_gdn_scan takes
//               one workgroup per (b, h, 32-column slice of Dv).  Columns of S evolve independently under the
//               delta rule, so slicing Dv needs no communication.  The fp32
//               master state lives in registers, a bf16 copy in LDS feeds the
//               MFMAs; the next chunk's operands are loaded while the current
//               chunk is computed (the barriers order LDS only, so those loads
//               stay in flight across them).
#include "common.hpp"
#include "gdn_common.hpp"
#include "kernels.hpp"

namespace natsl {

size_t gdn_ws_bytes(int io_is_bf16, int D, int64_t nch) {
  if (io_is_bf16) return D == 64 ? carve_bytes<bf16, 64>(nch) : carve_bytes<bf16, 128>(nch);
  return D == 64 ? carve_bytes<float, 64>(nch) : carve_bytes<float, 128>(nch);
}

// ---------------------------------------------------------------- prep ----
template <typename T, int D>
__global__ void __launch_bounds__(256, (GdnCfg<T, D>::PREP_WGS))
    k_gdn_prep(const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
               const float* __restrict__ alpha, const float* __restrict__ beta, GdnWs<T, D> ws,
               int L) {
  using C = GdnCfg<T, D>;
  extern __shared__ __align__(16) unsigned char lds[];
  T* Ks = (T*)(lds + C::OFF_KS);
  T* Kg = (T*)(lds + C::OFF_KG);
  T* Vg = (T*)(lds + C::OFF_VG);
  float* LT = (float*)(lds + C::OFF_LT);
  float* Rs = (float*)(lds + C::OFF_RS);
  float* gl = (float*)(lds + C::OFF_GL);  // cumulative log2 decay
  float* bl = gl + CHUNK;                 // beta
  float* gbl = bl + CHUNK;                // beta * gamma

  const int nc = L / CHUNK;
  const int64_t ch = bid_x();
  const int64_t bh = ch / nc;
  const int cc = (int)(ch % nc);
  const int64_t tok0 = bh * L + (int64_t)cc * CHUNK;  // row index into [B*H*L]
  const int t = tid_x(), lane = lane_id(), w = wave_id();
  const int g = lane >> 4, c = lane & 15;

  // Every global load of the chunk is issued first (one memory latency
  // instead of one per copy loop): thread t loads key group kg = t / (D / 8)
  // (rows 4kg .. 4kg+3) of K and V at columns col .. col+7, plus its Q
  // fragments; wave 0 also loads alpha and beta.
  constexpr int TASKS = (CHUNK / 4) * (D / 8);
  static_assert(TASKS <= 256, "one task per thread");
  const T* kc = k + tok0 * D;
  const T* vc = v + tok0 * D;
  const int kg = t / (D / 8), col = (t % (D / 8)) * 8;
  Frag<T> kr[4], vr[4];
  if (t < TASKS) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      kr[i] = load8<T>(kc + (4 * kg + i) * D + col);
      vr[i] = load8<T>(vc + (4 * kg + i) * D + col);
    }
  }
  Frag<T> qa[C::KF];
#pragma unroll
  for (int ks = 0; ks < C::KF; ++ks) qa[ks] = load8<T>(q + (tok0 + 16 * w + c) * D + 32 * ks + 8 * g);
  // cumulative log decay in log2 units (wave 0), beta: every decay below is
  // one v_exp_f32 of a difference (the library expf is a dozen VALU ops)
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
    ws.gm[ch * C::GM + lane] = __builtin_amdgcn_exp2f(s);
    ws.gm[ch * C::GM + 80 + lane] = __builtin_amdgcn_exp2f(gC - s);
    if (lane == 0) ws.gm[ch * C::GM + 64] = __builtin_amdgcn_exp2f(gC);
  }
  // K -> row layout and key-group layout, V -> key-group layout (the
  // key-group copies only after the inverse when they share the K rows' LDS)
  auto store_kv_groups = [&]() {
    if (t < TASKS) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        st4<T>(Kg + kg_index<C::RL>(kg, col + j), to_f32(frag_get<T>(kr[0], j)), to_f32(frag_get<T>(kr[1], j)),
               to_f32(frag_get<T>(kr[2], j)), to_f32(frag_get<T>(kr[3], j)));
        st4<T>(Vg + kg_index<C::RL>(kg, col + j), to_f32(frag_get<T>(vr[0], j)), to_f32(frag_get<T>(vr[1], j)),
               to_f32(frag_get<T>(vr[2], j)), to_f32(frag_get<T>(vr[3], j)));
      }
    }
  };
  if (t < TASKS) {
#pragma unroll
    for (int i = 0; i < 4; ++i) store8<T>(Ks + (4 * kg + i) * C::KP + col, kr[i]);
  }
  if constexpr (!C::ALIAS) store_kv_groups();
  __syncthreads();

  // K K^T rows 16w .. 16w+15, and P^T = K Q^T for the queries 16w .. 16w+15:
  // the transposed product leaves P's A fragments for the scan (row = query,
  // contraction over keys, accumulator-shaped map) directly in the
  // accumulators, with no LDS round trip
  f32x4 akk[4], apt[4];
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) {
    akk[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    apt[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int ks = 0; ks < C::KF; ++ks) {
    const Frag<T> ak = load8<T>(Ks + (16 * w + c) * C::KP + 32 * ks + 8 * g);
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      const Frag<T> bk = load8<T>(Ks + (16 * ct + c) * C::KP + 32 * ks + 8 * g);
      mma(akk[ct], ak, bk);
      mma(apt[ct], bk, qa[ks]);
    }
  }
  // L = diag(beta) strict_tril(Gamma . KK^T) -> LT (fp32)
#pragma unroll
  for (int ct = 0; ct < 4; ++ct)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * w + 4 * g + i, col = 16 * ct + c;
      LT[r * C::LTP + col] = (col < r) ? bl[r] * __builtin_amdgcn_exp2f(gl[r] - gl[col]) * akk[ct][i] : 0.f;
    }
  // P = tril(Gamma . QK^T): apt[ct][i] is (query 16w + c, key 16ct + 4g + i); the
  // fragment of key half k2 holds keys 32k2 + 4g + j and 32k2 + 16 + 4g + j.
  // The head-form scan takes P in bf16 (as it takes -W); otherwise P is split
  // into a bf16 part and the remainder bf16 could not hold (zero for fp32)
  {
    Frag<T> ph[2], pl[2];
    const int r = 16 * w + c;
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int col = 16 * ct + 4 * g + i;
        const float pv = (col <= r) ? __builtin_amdgcn_exp2f(gl[r] - gl[col]) * apt[ct][i] : 0.f;
        const int k2 = ct >> 1, j = (ct & 1) * 4 + i;
        frag_set(ph[k2], j, pv);
        if constexpr (!scan_head_form<T, D>()) frag_set(pl[k2], j, pv - to_f32(frag_get<T>(ph[k2], j)));
      }
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
      if constexpr (scan_head_form<T, D>()) {
        store8<T>(ws.pm + ch * C::PM + (w * 2 + k2) * 512 + lane * 8, ph[k2]);
      } else {
        store8<T>(ws.pm + (((ch * 4 + w) * 2 + k2) * 2 + 0) * 512 + lane * 8, ph[k2]);
        store8<T>(ws.pm + (((ch * 4 + w) * 2 + k2) * 2 + 1) * 512 + lane * 8, pl[k2]);
      }
    }
  }
  __syncthreads();

  lt_inverse64<C::LTP>(LT, Rs);

  // this lane's T values: row 16w + c, columns 32 k2 + kmap_acc(g, j)
  float tvr[2][8];
#pragma unroll
  for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
    for (int j = 0; j < 8; ++j) tvr[k2][j] = LT[(16 * w + c) * C::LTP + 32 * k2 + kmap_acc(g, j)];
  if constexpr (C::ALIAS) {  // the key-group copies overwrite the inverse's scratch and T
    __syncthreads();
    store_kv_groups();
    __syncthreads();
  }
  // U~ = T diag(b) V and W = T diag(b gamma) K, rows 16w .. 16w+15
  f32x4 ut[C::NT], wa[C::NT];
#pragma unroll
  for (int n = 0; n < C::NT; ++n) {
    ut[n] = f32x4{0.f, 0.f, 0.f, 0.f};
    wa[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  constexpr bool SPLIT = sizeof(T) == 2;  // bf16 operands: add the rounding remainder
#pragma unroll
  for (int k2 = 0; k2 < 2; ++k2) {
    Frag<T> a1, a2, a1l, a2l;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int tk = 32 * k2 + kmap_acc(g, j);
      const float tv = tvr[k2][j];
      const float x1 = tv * bl[tk], x2 = tv * gbl[tk];
      frag_set(a1, j, x1);
      frag_set(a2, j, x2);
      frag_set(a1l, j, x1 - to_f32(frag_get<T>(a1, j)));
      frag_set(a2l, j, x2 - to_f32(frag_get<T>(a2, j)));
    }
#pragma unroll
    for (int n = 0; n < C::NT; ++n) {
      const Frag<T> bv = ld4x2<T>(Vg + kg_index<C::RL>(8 * k2 + g, 16 * n + c),
                                  Vg + kg_index<C::RL>(8 * k2 + 4 + g, 16 * n + c));
      const Frag<T> bk = ld4x2<T>(Kg + kg_index<C::RL>(8 * k2 + g, 16 * n + c),
                                  Kg + kg_index<C::RL>(8 * k2 + 4 + g, 16 * n + c));
      mma(ut[n], a1, bv);
      if (SPLIT) mma(ut[n], a1l, bv);
      if constexpr (scan_head_form<T, D>()) {
        // W^T = K^T (T diag(b gamma))^T: wa[n][i] is W(token 16w + c, d 16n + 4g + i)
        mma(wa[n], bk, a2);
        if (SPLIT) mma(wa[n], bk, a2l);
      } else {
        mma(wa[n], a2, bk);
        if (SPLIT) mma(wa[n], a2l, bk);
      }
    }
  }
  // U~ in accumulator order (the scan uses it as the C operand): [rt][n][lane][4]
  // (fp32: in bf16 it added a third to the bf16 workloads' largest
  // RMS-normalised error for under 1% of the forward's time)
#pragma unroll
  for (int n = 0; n < C::NT; ++n)
    *reinterpret_cast<f32x4*>(ws.ut + ((ch * 4 + w) * C::NT + n) * 256 + lane * 4) = ut[n];
  // -W -> A fragments with contraction over d.  Head form: straight from the
  // transposed accumulators (d 32 ks + 4g + j from tile 2 ks, d 32 ks + 16 +
  // 4g + j from tile 2 ks + 1); otherwise through Ks (row layout, 8
  // contiguous d per lane)
  if constexpr (scan_head_form<T, D>()) {
#pragma unroll
    for (int ks = 0; ks < C::KF; ++ks) {
      Frag<T> f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        frag_set(f, j, -wa[2 * ks][j]);
        frag_set(f, 4 + j, -wa[2 * ks + 1][j]);
      }
      store8<T>(ws.wn + ((ch * 4 + w) * C::KF + ks) * 512 + lane * 8, f);
    }
  } else {
#pragma unroll
    for (int n = 0; n < C::NT; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i) Ks[(16 * w + 4 * g + i) * C::KP + 16 * n + c] = from_f32<T>(-wa[n][i]);
  }
  // K^T fragments: rows = d, contraction over tokens (KMAP_ACC); exact copies
  // of K (the exp(g_C - g) row scale is applied to U by the scan).  The
  // head-form scan reads K itself (transposed LDS reads) and needs none.
  if constexpr (!scan_head_form<T, D>())
  for (int f = w; f < C::NT * 2; f += 4) {
    const int n = f >> 1, k2 = f & 1;
    store8<T>(ws.kt + ((ch * C::NT + n) * 2 + k2) * 512 + lane * 8,
              ld4x2<T>(Kg + kg_index<C::RL>(8 * k2 + g, 16 * n + c), Kg + kg_index<C::RL>(8 * k2 + 4 + g, 16 * n + c)));
  }
  if constexpr (!scan_head_form<T, D>()) {
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < C::KF; ++ks)
      store8<T>(ws.wn + ((ch * 4 + w) * C::KF + ks) * 512 + lane * 8,
                load8<T>(Ks + (16 * w + c) * C::KP + 32 * ks + 8 * g));
  }
}

// ---------------------------------------------------------------- scan ----
template <typename T, int D, int DVT>
struct ScanOps {
  static constexpr int KF = D / 32;
  static constexpr int NV = DVT / 16;
  static constexpr int DTW = D / 64;  // 16-row d tiles of the state per wave
  Frag<T> wn[KF];
  f32x4 ut[NV];
  Frag<T> qa[KF];
  Frag<T> pa[2][2];  // [k2][hi, lo]
  Frag<T> kt[DTW][2];
  f32x4 gam;  // gamma of the wave's 4 rows
  f32x4 ek;   // exp(g_C - g) of the wave's 4 rows
  float gC;
  int route;
};

template <typename T, int D, int DVT>
__device__ __forceinline__ void scan_load(ScanOps<T, D, DVT>& op, const GdnWs<T, D>& ws,
                                          const T* qh, const int32_t* rt, int64_t bh, int nc,
                                          int cc, int nv0) {
  using C = GdnCfg<T, D>;
  using O = ScanOps<T, D, DVT>;
  const int lane = lane_id(), w = wave_id();
  const int g = lane >> 4, c = lane & 15;
  const int64_t ch = bh * nc + cc;
#pragma unroll
  for (int ks = 0; ks < O::KF; ++ks) {
    op.wn[ks] = load8<T>(ws.wn + ((ch * 4 + w) * C::KF + ks) * 512 + lane * 8);
    op.qa[ks] = load8<T>(qh + ((int64_t)cc * CHUNK + 16 * w + c) * D + 32 * ks + 8 * g);
  }
#pragma unroll
  for (int n = 0; n < O::NV; ++n)
    op.ut[n] = *reinterpret_cast<const f32x4*>(ws.ut + ((ch * 4 + w) * C::NT + nv0 + n) * 256 + lane * 4);
#pragma unroll
  for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
    for (int hl = 0; hl < 2; ++hl) op.pa[k2][hl] = load8<T>(ws.pm + (((ch * 4 + w) * 2 + k2) * 2 + hl) * 512 + lane * 8);
#pragma unroll
  for (int x = 0; x < O::DTW; ++x)
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2)
      op.kt[x][k2] = load8<T>(ws.kt + ((ch * C::NT + w * O::DTW + x) * 2 + k2) * 512 + lane * 8);
  op.gam = *reinterpret_cast<const f32x4*>(ws.gm + ch * C::GM + 16 * w + 4 * g);
  op.ek = *reinterpret_cast<const f32x4*>(ws.gm + ch * C::GM + 80 + 16 * w + 4 * g);
  op.gC = ws.gm[ch * C::GM + 64];
  op.route = rt[cc];
}

// The scan keeps global stores out of its chunk loop: on this GPU loads and
// stores share one completion counter, and while both kinds are outstanding
// a wait for a load can only be a wait for everything, which would drain the
// operand prefetch every chunk.  Outputs therefore go to an LDS ring of
// OUT_RING chunks that is flushed to memory (followed by one full wait)
// every OUT_RING chunks; between flushes only loads are in flight and the
// prefetch of NS - 1 chunks ahead stays in flight across chunks.
constexpr int OUT_RING = 8;

// State mode (ST, for the gradient): the outputs are replaced by the chunks'
// U = U~ - W S (through the same ring into o_gdn), and every chunk's start
// state is written to s0_out ([B, H, Nc, D, D] in T, row-major); the output
// products are skipped.
template <typename T, typename To, int D, int DVT, int NS, bool ST>
__global__ void __launch_bounds__(256, 1)
    k_gdn_scan(const T* __restrict__ q, const int32_t* __restrict__ route, GdnWs<T, D> ws,
               const float* __restrict__ S_init, To* __restrict__ o_gdn, float* __restrict__ S_final,
               T* __restrict__ s0_out, int H, int L, int G) {
  using O = ScanOps<T, D, DVT>;
  constexpr int SPP = D + 16 / (int)sizeof(T);  // pitch of the transposed bf16 state [dv][dk]
  __shared__ __align__(16) T Sp[2][DVT * SPP];
  constexpr int URL = kg_row<T, DVT>();
  __shared__ __align__(16) To Ob[OUT_RING * CHUNK * DVT];  // output ring
  __shared__ __align__(16) T Up[(CHUNK / 4) * URL * 4];   // U (B operand of P U)
  __shared__ __align__(16) T Ue[(CHUNK / 4) * URL * 4];   // exp(g_C - g) U (of K^T U)
  constexpr bool SPLIT = sizeof(T) == 2;

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
  const int nv0 = vt * (DVT / 16);
  const int dv0 = vt * DVT;
  const T* qh = q + bh * L * D;
  To* oh = o_gdn + bh * L * D;

  const int lane = lane_id(), w = wave_id();
  const int g = lane >> 4, c = lane & 15;

  // fp32 master state: rows d = 16 (w*DTW + x) + 4g + i, columns dv0 + 16n + c
  f32x4 sm[O::DTW][O::NV];
#pragma unroll
  for (int x = 0; x < O::DTW; ++x)
#pragma unroll
    for (int n = 0; n < O::NV; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int dk = 16 * (w * O::DTW + x) + 4 * g + i;
        sm[x][n][i] = S_init ? S_init[(bh * D + dk) * D + dv0 + 16 * n + c] : 0.f;
      }
  int sb = 0;
  auto write_state = [&](int buf) {
#pragma unroll
    for (int x = 0; x < O::DTW; ++x)
#pragma unroll
      for (int n = 0; n < O::NV; ++n)
        st4<T>(&Sp[buf][(16 * n + c) * SPP + 16 * (w * O::DTW + x) + 4 * g], sm[x][n][0], sm[x][n][1],
               sm[x][n][2], sm[x][n][3]);
  };
  write_state(0);
  lds_barrier();

  // One chunk.  Branch-free: for a softmax-routed chunk the state update runs
  // with decay 1 and zero operands (U scaled to zero and K^T replaced by zero
  // by selection, not by multiplication, so that a non-finite U or K cannot
  // leak in as 0 * inf), which leaves S bit-identical (x*1 + 0*0), so every
  // prefetched operand is consumed unconditionally (a use inside a branch
  // lets the compiler sink the load into it, defeating the prefetch).
  auto step = [&](const ScanOps<T, D, DVT>& op, int cc) {
    if constexpr (ST) {
#pragma unroll
      for (int x = 0; x < O::DTW; ++x)
#pragma unroll
        for (int n = 0; n < O::NV; ++n)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int dk = 16 * (w * O::DTW + x) + 4 * g + i;
            s0_out[((bh * nc + cc) * D + dk) * D + dv0 + 16 * n + c] = from_f32<T>(sm[x][n][i]);
          }
    }
    // S fragments (B operand, contraction over d): shared by U and Q S
    Frag<T> bs[O::KF][O::NV];
#pragma unroll
    for (int ks = 0; ks < O::KF; ++ks)
#pragma unroll
      for (int n = 0; n < O::NV; ++n) bs[ks][n] = load8<T>(&Sp[sb][(16 * n + c) * SPP + 32 * ks + 8 * g]);
    f32x4 u[O::NV], oa[O::NV];
#pragma unroll
    for (int n = 0; n < O::NV; ++n) {
      u[n] = op.ut[n];
      oa[n] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int ks = 0; ks < O::KF; ++ks)
#pragma unroll
      for (int n = 0; n < O::NV; ++n) {
        mma(u[n], op.wn[ks], bs[ks][n]);   // U = U~ - W S
        if constexpr (!ST) mma(oa[n], op.qa[ks], bs[ks][n]);  // Q S
      }
    const bool lin = op.route == 1;
    const float gce = lin ? op.gC : 1.f;
#pragma unroll
    for (int n = 0; n < O::NV; ++n) {
      f32x4 ue;
#pragma unroll
      for (int i = 0; i < 4; ++i) ue[i] = lin ? u[n][i] * op.ek[i] : 0.f;
      st4<T>(&Up[kg_index<URL>(4 * w + g, 16 * n + c)], u[n][0], u[n][1], u[n][2], u[n][3]);
      st4<T>(&Ue[kg_index<URL>(4 * w + g, 16 * n + c)], ue[0], ue[1], ue[2], ue[3]);
#pragma unroll
      for (int i = 0; i < 4; ++i) oa[n][i] *= op.gam[i];
    }
    lds_barrier();
    Frag<T> bu[2][O::NV], be[2][O::NV];
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
      for (int n = 0; n < O::NV; ++n) {
        bu[k2][n] = ld4x2<T>(&Up[kg_index<URL>(8 * k2 + g, 16 * n + c)], &Up[kg_index<URL>(8 * k2 + 4 + g, 16 * n + c)]);
        be[k2][n] = ld4x2<T>(&Ue[kg_index<URL>(8 * k2 + g, 16 * n + c)], &Ue[kg_index<URL>(8 * k2 + 4 + g, 16 * n + c)]);
      }
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
      for (int n = 0; n < O::NV; ++n) {
        if constexpr (!ST) {
          mma(oa[n], op.pa[k2][0], bu[k2][n]);  // + P U
          if (SPLIT) mma(oa[n], op.pa[k2][1], bu[k2][n]);
        }
      }
    To* ob = Ob + (cc % OUT_RING) * CHUNK * DVT;
#pragma unroll
    for (int n = 0; n < O::NV; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        ob[(16 * w + 4 * g + i) * DVT + 16 * n + c] = from_f32<To>(ST ? u[n][i] : oa[n][i]);
    // S <- gamma_C S + K^T diag(exp(g_C - g)) U   (linear-routed), else S unchanged
#pragma unroll
    for (int x = 0; x < O::DTW; ++x)
#pragma unroll
      for (int n = 0; n < O::NV; ++n) {
        f32x4 acc = sm[x][n] * gce;
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) mma(acc, frag_select(lin, op.kt[x][k2]), be[k2][n]);
        sm[x][n] = acc;
      }
    write_state(sb ^ 1);
    sb ^= 1;
    lds_barrier();
  };
  // Output ring -> memory for chunks c_first .. c_last, then one full wait so
  // that no store stays outstanding next to the operand loads.
  auto flush = [&](int c_first, int c_last) {
    const int rows = (c_last - c_first + 1) * CHUNK;
    constexpr int PER = 16 / (int)sizeof(To);  // elements per 16-byte store
    for (int e = tid_x(); e < rows * (DVT / PER); e += 256) {
      const int r = e / (DVT / PER), cl = (e % (DVT / PER)) * PER;
      const To* src = Ob + ((c_first % OUT_RING) * CHUNK + r) * DVT + cl;
      To* dst = oh + ((int64_t)c_first * CHUNK + r) * D + dv0 + cl;
      *reinterpret_cast<f32x4*>(dst) = *reinterpret_cast<const f32x4*>(src);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  };

  // NS operand sets rotate: the loads for chunk c + NS - 1 are issued before
  // chunk c is computed (clamped to the last chunk near the end; the extra
  // loads are harmless).  Main loop: OUT_RING chunks per iteration, no
  // branches but the loop itself; then a generic tail.
  static_assert(OUT_RING % NS == 0, "ring must hold whole operand rotations");
  ScanOps<T, D, DVT> ops[NS];
#pragma unroll
  for (int j = 0; j < NS - 1; ++j) scan_load<T, D, DVT>(ops[j], ws, qh, rt, bh, nc, min(j, nc - 1), nv0);
  int c0 = 0;
  for (; c0 + OUT_RING <= nc; c0 += OUT_RING) {
#pragma unroll
    for (int j = 0; j < OUT_RING; ++j) {
      scan_load<T, D, DVT>(ops[(j + NS - 1) % NS], ws, qh, rt, bh, nc, min(c0 + j + NS - 1, nc - 1), nv0);
      __builtin_amdgcn_sched_barrier(0);
      step(ops[j % NS], c0 + j);
    }
    flush(c0, c0 + OUT_RING - 1);
  }
  // tail (fewer than OUT_RING chunks): ops[0 .. NS-2] hold chunks c0 .. c0+NS-2
  for (int cc = c0; cc < nc; ++cc) {
    const int j = cc - c0;
    ScanOps<T, D, DVT> cur;
    if (j < NS - 1) {
      // pick the already-loaded set (j is small and runtime: select by copy)
#pragma unroll
      for (int jj = 0; jj < NS - 1; ++jj)
        if (jj == j) cur = ops[jj];
    } else {
      scan_load<T, D, DVT>(cur, ws, qh, rt, bh, nc, cc, nv0);
    }
    step(cur, cc);
  }
  if (c0 < nc) flush(c0, nc - 1);
  if (S_final) {
#pragma unroll
    for (int x = 0; x < O::DTW; ++x)
#pragma unroll
      for (int n = 0; n < O::NV; ++n)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int dk = 16 * (w * O::DTW + x) + 4 * g + i;
          S_final[(bh * D + dk) * D + dv0 + 16 * n + c] = sm[x][n][i];
        }
  }
}

// --------------------------------------------------- scan, head form ----
// bf16, D = 128: NSPLIT workgroups of NW waves per (b, h).  Wave w of part p
// owns the state columns dv0 .. dv0 + 16 NV - 1, dv0 = 16 NV (NW p + w)
// (NV = 128 / (16 NW NSPLIT) column tiles, all 128 rows) and runs the whole
// chunk recurrence for them in registers: columns
// of S evolve independently, so the waves never exchange state, and the
// dependency chain of a chunk (S -> U = U~ - W S -> S' = gamma_C S +
// K^T diag(exp(g_C - g)) U) has no barrier and no LDS round trip.  The state's
// B operand (contraction over d) is packed from the fp32 accumulators directly
// (accumulator-shaped map, which is how the chunk prep writes -W for this
// form); U's B operand (contraction over tokens) likewise.
// The operands every wave needs (-W, Q, P, K^T: 56 KiB in bf16, plus the
// decays) go through a 2-stage LDS ring by direct global -> LDS loads issued
// one chunk ahead, and so do the workgroup's U~ columns (16 KiB).  All loads
// of a chunk, and the output stores of the previous one, are
// issued a whole chunk before the single vmcnt(0) wait at the top of the next
// chunk.
constexpr int SCH_WN = 0;              // -W fragments [rt 4][ks 4][lane][8]
constexpr int SCH_Q = 16384;           // Q rows, 16-byte chunk q of row r at slot q ^ (r & 15)
constexpr int SCH_PM = 2 * 16384;      // P fragments (bf16) [rt 4][k2 2][lane][8]
constexpr int SCH_KT = SCH_PM + 8192;  // K rows, 16-byte chunk q of row r at slot q ^ ((r & 7) << 1)
constexpr int SCH_UT = SCH_KT + 16384; // the workgroup's U~ columns (fp32 accumulator order) [rt 4][tile 4][lane][4]
constexpr int SCH_GM = SCH_UT + 16384; // gamma[64], gamma_C at 64, exp(g_C - g)[64] at 80 (fp32)
constexpr int SCH_STAGE = SCH_GM + 576;
constexpr int SCH_ROUTE = 2 * SCH_STAGE;
// route bytes of the head's chunks fill the rest of the LDS after the ring
constexpr int SCH_MAX_NC = (LDS_MAX_BYTES - SCH_ROUTE) & ~15;
constexpr int SCH_NW = 4;              // waves per workgroup
constexpr int SCH_NSPLIT = 2;          // workgroups per head
// One workgroup of eight waves per head (for many heads, where two
// workgroups per head would hold most of the GPU): its 32 KiB of U~ columns
// would not fit in both stages, so the stages hold no U~ and one U~ buffer
// follows them, refilled for the next chunk once every wave has read its
// columns.
constexpr int SCH1_NW = 8;
constexpr int SCH1_GM = SCH_UT;        // the decays right after K
constexpr int SCH1_STAGE = SCH1_GM + 576;
constexpr int SCH1_UT = 2 * SCH1_STAGE;
static_assert(SCH1_UT + 32768 <= SCH_ROUTE, "the one-workgroup layout ends before the route bytes");
// (every wave reads all 64 KiB of shared operands from LDS per chunk, so LDS
// traffic per CU grows with the waves per workgroup: two workgroups of four
// waves per head halve it against one of eight, at the price of loading the
// shared operands twice from L2)

__device__ __forceinline__ Frag<bf16> pack_acc2(const f32x4& a, const f32x4& b) {
  Frag<bf16> f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    f.v[j] = (bf16)a[j];
    f.v[4 + j] = (bf16)b[j];
  }
  return f;
}

// (launch bounds of two waves per SIMD cap the wave at 256 VGPRs, so that the
// compiler keeps the matrix products in their VGPR form: with 512 registers it
// moves the accumulators to AGPRs and copies them back and forth for every
// VALU touch of the state)
// State mode (ST, for the gradient): the outputs are replaced by the chunks'
// U = U~ - W S (written where o_gdn would go, [B, H, L, D] bf16), and every
// chunk's start state is written to s0_out ([B, H, Nc, D, D] bf16, row-major);
// the output products are skipped.
template <typename To, int NW, int NSPLIT, bool ST>
__global__ void __launch_bounds__(64 * NW, 8 / NW)
    k_gdn_scan_head(const bf16* __restrict__ q, const bf16* __restrict__ k, const int32_t* __restrict__ route,
                    GdnWs<bf16, 128> ws,
                    const float* __restrict__ S_init, To* __restrict__ o_gdn, float* __restrict__ S_final,
                    bf16* __restrict__ s0_out, int H, int L, int G) {
  constexpr int D = 128;
  constexpr int NV = D / (16 * NW * NSPLIT);  // 16-column state tiles per wave
  static_assert(NV >= 1 && NW >= 4, "the Q swizzle assumes 4 KiB-aligned load groups");
  constexpr int NB = 16 / NW;        // 1 KiB blocks of each 16 KiB operand per wave
  constexpr bool UT1 = NSPLIT == 1;  // one U~ buffer after the stages (see SCH1_*)
  constexpr int STAGE = UT1 ? SCH1_STAGE : SCH_STAGE;
  constexpr int OFF_GM = UT1 ? SCH1_GM : SCH_GM;
  static_assert(!UT1 || 4 * NV * NW * 1024 == 32768, "one U~ buffer of 32 KiB");
  using C = GdnCfg<bf16, D>;
  extern __shared__ __align__(16) unsigned char lds[];
  unsigned char* rl = lds + SCH_ROUTE;  // one route byte per chunk

  const int nc = L / CHUNK;
  // the NSPLIT workgroups of a head go to one XCD (workgroup p runs on XCD
  // p % 8), so the second reads the shared operands from that XCD's L2
  int64_t bh;
  int part;
  // (unsigned: with signed division here the chunk loop below spills)
  const unsigned bid = (unsigned)bid_x();
  if ((((unsigned)grid_dim_x() / NSPLIT) & 7) == 0) {
    const unsigned x = bid & 7, r = bid >> 3;
    part = (int)(r % NSPLIT);
    bh = (int64_t)(r / NSPLIT) * 8 + x;
  } else {
    bh = bid / NSPLIT;
    part = (int)(bid % NSPLIT);
  }
  const int b = (int)(bh / H), h = (int)(bh % H);
  const int grp = (G == 1) ? 0 : h;
  const int32_t* rt_g = route + ((int64_t)b * G + grp) * nc;
  const bf16* qh = q + bh * L * D;
  const bf16* kh = k + bh * L * D;
  To* oh = o_gdn + bh * L * D;
  const int lane = lane_id(), w = wave_id();
  const int g = lane >> 4, c = lane & 15;
  const int dv0 = 16 * NV * (NW * part + w);

  for (int i = tid_x(); i < nc; i += 64 * NW) rl[i] = (unsigned char)(rt_g[i] == 1);

  // fp32 state: rows d = 16 dt + 4g + i, columns dv0 + 16 nn + c
  f32x4 sm[8][NV];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
#pragma unroll
    for (int nn = 0; nn < NV; ++nn) sm[dt][nn] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (S_init) {
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int nn = 0; nn < NV; ++nn)
#pragma unroll
        for (int i = 0; i < 4; ++i) sm[dt][nn][i] = S_init[(bh * D + 16 * dt + 4 * g + i) * D + dv0 + 16 * nn + c];
  }

  // chunk cc's operands -> stage st, all by direct global -> LDS loads (so
  // that the waits below can count them).  Wave w loads the 1 KiB blocks
  // NW i + w of each 16 KiB operand; for Q, LDS position e = 64 blk + lane
  // holds 16-byte chunk (e & 15) ^ (r & 15) of row r = e / 16, and r & 15 does
  // not depend on i; K likewise with slot (e & 15) ^ ((r & 7) << 1).  Per
  // wave: NB blocks each of -W, Q and K, 4 NV of U~, NB / 2 of P and one
  // partial block of the decays.
  const uint32_t off_lin = (uint32_t)(w * 1024 + lane * 16);
  const int qr = 4 * w + (lane >> 4);
  const uint32_t off_q = (uint32_t)(w * 1024 + (lane >> 4) * 256 + (((lane & 15) ^ (qr & 15)) * 16));
  const uint32_t off_k = (uint32_t)(w * 1024 + (lane >> 4) * 256 + (((lane & 15) ^ ((qr & 7) << 1)) * 16));
  constexpr int GMW = (36 + NW - 1) / NW;  // 16-byte pieces of the 576 decay bytes per wave (fewer for the last)
  static_assert((NW - 1) * GMW < 36, "every wave loads a piece of the decays (one DMA operation each)");
  // op 0: -W, 1: Q, 2: P (8 KiB) and the decays, 3: K, 4: this
  // workgroup's U~ columns ([rt][16-column tile] blocks)
  auto load_part = [&](int cc, int st, int op) {
    const int64_t ch = bh * nc + cc;
    unsigned char* sb = lds + opaque_sgpr(st * STAGE);
    if (op == 4) {
      const unsigned char* ub = reinterpret_cast<const unsigned char*>(ws.ut + ch * 4 * C::NT * 256);
#pragma unroll
      for (int i = 0; i < 4 * NV; ++i) {
        const int j = NW * i + w;  // block: row tile j / (NV NW), local column tile j % (NV NW)
        const int rt = j / (NV * NW), tl = j % (NV * NW);
        gload_lds16_s_nt(ub + (rt * C::NT + NV * NW * part + tl) * 1024, (uint32_t)(lane * 16),
                         (UT1 ? lds + SCH1_UT : sb + SCH_UT) + j * 1024);
      }
      return;
    }
    const unsigned char* src;
    uint32_t off = off_lin;
    int dst;
    if (op == 0) {
      src = reinterpret_cast<const unsigned char*>(ws.wn + ch * C::WN);
      dst = SCH_WN;
    } else if (op == 1) {
      src = reinterpret_cast<const unsigned char*>(qh + (int64_t)cc * CHUNK * D);
      off = off_q;
      dst = SCH_Q;
    } else if (op == 2) {
      src = reinterpret_cast<const unsigned char*>(ws.pm + ch * C::PM);
      dst = SCH_PM;
    } else {
      src = reinterpret_cast<const unsigned char*>(kh + (int64_t)cc * CHUNK * D);
      off = off_k;
      dst = SCH_KT;
    }
    const int nb = op == 2 ? NB / 2 : NB;  // P: 8 KiB
#pragma unroll
    for (int i = 0; i < NB; ++i)
      if (i < nb) {  // the prep's operands (-W, P) are read once, here; q and k also by the softmax branch
        if (op == 0 || op == 2)
          gload_lds16_s_nt(src + i * NW * 1024, off, sb + dst + (NW * i + w) * 1024);
        else
          gload_lds16_s(src + i * NW * 1024, off, sb + dst + (NW * i + w) * 1024);
      }
    if (op == 2 && lane < GMW && w * GMW + lane < 36)  // 576 bytes of decays, a share per wave
      gload_lds16_s_nt(reinterpret_cast<const unsigned char*>(ws.gm + ch * C::GM) + w * GMW * 16,
                       (uint32_t)(lane * 16), sb + OFF_GM + w * GMW * 16);
  };
  // DMA operations a wave issues per part
  constexpr int N_W = NB, N_Q = NB, N_U = 4 * NV, N_P = NB / 2 + 1, N_KT = NB;
  static_assert(N_W + N_Q + N_U + N_P + N_KT + 16 * NV + (ST ? 16 * NV : 0) < 64, "vmcnt range");
  // outputs: a uniform base per store plus one 32-bit byte offset per lane
  // (the SGPR-base store form; 64-bit lane addresses per store cost registers)
  const uint32_t o_boff = (uint32_t)((4 * g * D + dv0 + c) * sizeof(To));
  auto store_o = [&](int cc, const f32x4 (&o)[4][NV]) {
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int nn = 0; nn < NV; ++nn)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          unsigned char* base =
              reinterpret_cast<unsigned char*>(oh + (int64_t)cc * CHUNK * D + (16 * rt + i) * D + 16 * nn);
          *reinterpret_cast<To*>(base + o_boff) = from_f32<To>(o[rt][nn][i]);
        }
  };
  // state mode: the chunk-start state, bf16 row-major, two columns per
  // 4-byte store (lanes c and c ^ 1 trade values: the even lane writes rows
  // 4g and 4g + 2, the odd one rows 4g + 1 and 4g + 3)
  const bool codd = (c & 1) != 0;
  const uint32_t s_boff = (uint32_t)((((4 * g + (codd ? 1 : 0)) * D) + (c & ~1)) * 2);
  auto store_state = [&](int cc) {
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int nn = 0; nn < NV; ++nn) {
        const f32x4 x = sm[dt][nn];
        const float r0 = __int_as_float(
            __builtin_amdgcn_mov_dpp(__float_as_int(codd ? x[0] : x[1]), 0xB1, 0xF, 0xF, false));  // quad_perm 1,0,3,2
        const float r1 = __int_as_float(
            __builtin_amdgcn_mov_dpp(__float_as_int(codd ? x[2] : x[3]), 0xB1, 0xF, 0xF, false));
        const bf16x2 a = codd ? bf16x2{(bf16)r0, (bf16)x[1]} : bf16x2{(bf16)x[0], (bf16)r0};
        const bf16x2 b2 = codd ? bf16x2{(bf16)r1, (bf16)x[3]} : bf16x2{(bf16)x[2], (bf16)r1};
        unsigned char* base = reinterpret_cast<unsigned char*>(
            s0_out + (((int64_t)bh * nc + cc) * D + 16 * dt) * D + dv0 + 16 * nn);
        *reinterpret_cast<bf16x2*>(base + s_boff) = a;
        *reinterpret_cast<bf16x2*>(base + s_boff + 2 * D * 2) = b2;
      }
  };
  // Operand fragments from LDS are read ahead of the products that use them
  // (two (row tile, d step) steps ahead for -W and Q, two d tiles ahead for
  // K^T, a row-tile pair ahead for P); sched_barrier fences pin that order:
  // left free, the scheduler hoists every read of the chunk and runs out of
  // registers; fenced without a lead, every step waits out the LDS latency.
  struct FragP { Frag<bf16> p[2][2]; };  // P for two row tiles: [tile][k2]
  auto read_p = [&](const unsigned char* sb, int rt0, FragP& f) {
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2)
        f.p[t][k2] = load8<bf16>(reinterpret_cast<const bf16*>(sb + SCH_PM + (((rt0 + t) * 2 + k2) * 64 + lane) * 16));
  };
  auto read_wq = [&](const unsigned char* sb, int s_, Frag<bf16>& fw, Frag<bf16>& fq) {
    const int rt = s_ >> 2, ks = s_ & 3;
    fw = load8<bf16>(reinterpret_cast<const bf16*>(sb + SCH_WN + ((rt * 4 + ks) * 64 + lane) * 16));
    const unsigned char* qrow = sb + SCH_Q + (16 * rt + c) * 256;
    const int q1 = 4 * ks + (g >> 1), q2 = q1 + 2, half = (g & 1) * 8;
    fq = ld4x2<bf16>(reinterpret_cast<const bf16*>(qrow + ((q1 ^ c) * 16) + half),
                     reinterpret_cast<const bf16*>(qrow + ((q2 ^ c) * 16) + half));
  };
  // K^T fragments of d tile dt (rows d = 16 dt + c, tokens 32 k2 + 4g + j and
  // 32 k2 + 16 + 4g + j) from the row-major K by transposed reads, which swap
  // 4 x 4 blocks of 16-bit values across each 16-lane group: lane c of group g
  // reads token row 32 k2 + 4g + c / 4 (+16), columns 16 dt + 4 (c % 4) .. +3
  auto read_k1 = [&](const unsigned char* sb, int dt, Frag<bf16> (&f)[2]) {
    const unsigned char* kl = sb + SCH_KT;
    const int colq = (16 * dt + 4 * (c & 3)) >> 3;  // 16-byte chunk of the 4 columns
    const int half = (c & 1) * 8;                    // byte offset inside it
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
      const int r0 = 32 * k2 + 4 * g + (c >> 2), r1 = r0 + 16;
      const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) v4i16*)(kl + r0 * 256 + ((colq ^ ((r0 & 7) << 1)) * 16) + half));
      const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) v4i16*)(kl + r1 * 256 + ((colq ^ ((r1 & 7) << 1)) * 16) + half));
      f[k2].v = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
  };
  auto fence = []() { __builtin_amdgcn_sched_barrier(0); };

  // chunk cc from stage st.  Order of the loads for chunk cc + 1 (issued
  // during chunk cc): -W, Q, U~, P and the decays, spread over the first half;
  // K^T last, after this chunk's K^T is in.  So the wait at the top of a chunk
  // leaves that chunk's K^T in flight (N_KT), and the state update waits for
  // it behind everything issued after it.  o_prev holds the previous chunk's
  // outputs on entry (stored here); o receives this chunk's.
  auto step = [&](int cc, int st, f32x4 (&o)[4][NV], f32x4 (&o_prev)[4][NV]) {
    wait_vmcnt<N_KT>();  // all of chunk cc's operands but K^T (and older stores) are in
    lds_barrier();       // ... for every wave; every wave is done with chunk cc - 1
    const unsigned char* sb = lds + opaque_sgpr(st * STAGE);
    const unsigned char* ub = UT1 ? lds + SCH1_UT : sb + SCH_UT;
    f32x4 u[4][NV];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int nn = 0; nn < NV; ++nn)
        u[rt][nn] = *reinterpret_cast<const f32x4*>(ub + ((rt * NV * NW + NV * w + nn) * 64 + lane) * 16);
    const bool more = cc + 1 < nc;
    if constexpr (UT1) lds_barrier();  // every wave holds its U~ columns: the one buffer may be refilled
    if (cc > 0) store_o(cc - 1, o_prev);  // outputs of chunk cc - 1 (state mode: its U)
    if constexpr (ST) store_state(cc);
    // (one buffer: chunk cc + 1's U~ goes first, after the stores, so that the
    // K^T wait below, which counts the operand loads issued after K^T but not
    // the stores, leaves it in flight)
    if (UT1 && more) load_part(cc + 1, st ^ 1, 4);
    if (more) load_part(cc + 1, st ^ 1, 0);
    const float* gm = reinterpret_cast<const float*>(sb + OFF_GM);
    const bool lin = rl[cc] == 1;

    // state B operand, contraction over d
    Frag<bf16> bs[4][NV];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int nn = 0; nn < NV; ++nn) bs[ks][nn] = pack_acc2(sm[2 * ks][nn], sm[2 * ks + 1][nn]);
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int nn = 0; nn < NV; ++nn) o[rt][nn] = f32x4{0.f, 0.f, 0.f, 0.f};

    // U = U~ - W S  and  Q S: 16 (row tile, d step) steps, operands read two
    // steps ahead
    Frag<bf16> fw[3], fq[3];
    FragP fp[2];
    read_wq(sb, 0, fw[0], fq[0]);
    read_wq(sb, 1, fw[1], fq[1]);
    fence();
#pragma unroll
    for (int s_ = 0; s_ < 16; ++s_) {
      const int rt = s_ >> 2, ks = s_ & 3;
      if (s_ + 2 < 16) read_wq(sb, s_ + 2, fw[(s_ + 2) % 3], fq[(s_ + 2) % 3]);
      if (s_ == 13) read_p(sb, 0, fp[0]);
      if (more && s_ == 3) load_part(cc + 1, st ^ 1, 1);
      if (!UT1 && more && s_ == 7) load_part(cc + 1, st ^ 1, 4);
      if (more && s_ == 11) load_part(cc + 1, st ^ 1, 2);
      fence();
#pragma unroll
      for (int nn = 0; nn < NV; ++nn) {
        mma(u[rt][nn], fw[s_ % 3], bs[ks][nn]);
        if constexpr (!ST) mma(o[rt][nn], fq[s_ % 3], bs[ks][nn]);
      }
      fence();
    }
    // branch-free rollback: a softmax-routed chunk updates with decay 1 and
    // zero operands (scaled U and K^T both replaced by zero by selection, so
    // that a non-finite U or K cannot leak in as 0 * inf), which leaves S
    // bit-identical
    const float gce = lin ? gm[64] : 1.f;
    Frag<bf16> bu[2][NV], be[2][NV];
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
      const f32x4 ek0 = *reinterpret_cast<const f32x4*>(gm + 80 + 32 * k2 + 4 * g);
      const f32x4 ek1 = *reinterpret_cast<const f32x4*>(gm + 80 + 32 * k2 + 16 + 4 * g);
#pragma unroll
      for (int nn = 0; nn < NV; ++nn) {
        bu[k2][nn] = pack_acc2(u[2 * k2][nn], u[2 * k2 + 1][nn]);
        f32x4 e0, e1;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          e0[i] = lin ? u[2 * k2][nn][i] * ek0[i] : 0.f;
          e1[i] = lin ? u[2 * k2 + 1][nn][i] * ek1[i] : 0.f;
        }
        be[k2][nn] = pack_acc2(e0, e1);
      }
    }
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      const f32x4 gam = *reinterpret_cast<const f32x4*>(gm + 16 * rt + 4 * g);
#pragma unroll
      for (int nn = 0; nn < NV; ++nn) {
        if constexpr (ST)
          o[rt][nn] = u[rt][nn];
        else
          o[rt][nn] *= gam;
      }
    }
    // O += P U, two row tiles per group
    Frag<bf16> fk[3][2];
#pragma unroll
    for (int gp = 0; gp < 2; ++gp) {
      if (gp == 0) {
        read_p(sb, 2, fp[1]);
      } else {
        // this chunk's K^T: everything issued after it may stay in flight
        if (more) wait_vmcnt<N_W + N_Q + N_U + N_P>();
        else wait_vmcnt<0>();
        lds_barrier();
        if (more) load_part(cc + 1, st ^ 1, 3);
        read_k1(sb, 0, fk[0]);
        read_k1(sb, 1, fk[1]);
      }
      fence();
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
          for (int nn = 0; nn < NV; ++nn)
            if constexpr (!ST) mma(o[2 * gp + t][nn], fp[gp].p[t][k2], bu[k2][nn]);
      fence();
    }
    // S <- gamma_C S + K^T diag(exp(g_C - g)) U, four d tiles per group
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int nn = 0; nn < NV; ++nn) sm[dt][nn] *= gce;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      if (dt + 2 < 8) read_k1(sb, dt + 2, fk[(dt + 2) % 3]);
      fence();
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
        for (int nn = 0; nn < NV; ++nn) mma(sm[dt][nn], frag_select(lin, fk[dt % 3][k2]), be[k2][nn]);
      fence();
    }
  };

  f32x4 oA[4][NV], oB[4][NV];
  // prologue in the order the chunk loop issues: K^T last
  load_part(0, 0, 0);
  load_part(0, 0, 1);
  load_part(0, 0, 4);
  load_part(0, 0, 2);
  load_part(0, 0, 3);
  int cc = 0;
  for (; cc + 2 <= nc; cc += 2) {
    step(cc, 0, oA, oB);
    step(cc + 1, 1, oB, oA);
  }
  const bool odd = cc < nc;
  if (odd) step(cc, 0, oA, oB);
  // outputs of the last chunk
  if (odd)
    store_o(nc - 1, oA);
  else
    store_o(nc - 1, oB);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // no load may still be in flight into LDS at the end
  if (S_final) {
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int nn = 0; nn < NV; ++nn)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          S_final[(bh * D + 16 * dt + 4 * g + i) * D + dv0 + 16 * nn + c] = sm[dt][nn][i];
  }
}

template <typename T, typename To, int D>
hipError_t launch_gdn(const T* q, const T* k, const T* v, const float* alpha, const float* beta,
                      const int32_t* route, const float* S_init, To* o_gdn, float* S_final, void* wsp,
                      int B, int H, int L, int G, hipStream_t st_prep, hipStream_t st_scan,
                      hipEvent_t prep_done, hipEvent_t scan_dep, void (*prof)(int, hipStream_t, int)) {
  using C = GdnCfg<T, D>;
  constexpr int DVT = 32;
  constexpr int SCAN_NS = sizeof(T) == 2 ? 4 : 2;  // operand sets in flight in the scan
  const int nc = L / CHUNK;
  // (the C ABI has already rejected longer sequences; nothing is launched
  // when this fails)
  if (nc > gdn_max_chunks(sizeof(T) == 2, D)) return hipErrorInvalidValue;
  hipError_t e = set_lds_limit((const void*)k_gdn_prep<T, D>, C::PREP_LDS);
  if (e != hipSuccess) return e;
  // the head-form scan: two workgroups per head, or one of eight waves when
  // two per head would not fit the GPU at once (256 CUs, one scan workgroup
  // each).  The one-workgroup form is slower per chunk (every wave reads all
  // shared operands, for half the state columns); at 64 heads it freed CUs
  // that sped the softmax branch by 10%, but the longer scan then bounded
  // the step (B = 4, H = 16, L = 4096: 0.424 vs 0.419 ms)
  const bool one_wg = (int64_t)B * H >= 128;
  if constexpr (scan_head_form<T, D>()) {
    e = one_wg ? set_lds_limit((const void*)k_gdn_scan_head<To, SCH1_NW, 1, false>, SCH_ROUTE + SCH_MAX_NC)
               : set_lds_limit((const void*)k_gdn_scan_head<To, SCH_NW, SCH_NSPLIT, false>, SCH_ROUTE + SCH_MAX_NC);
    if (e != hipSuccess) return e;
  }
  const int64_t nch = (int64_t)B * H * nc;
  GdnWs<T, D> ws = carve<T, D>(wsp, nch);
  if (prof) prof(KID_GDN_PREP, st_prep, 0);
  hipLaunchKernelGGL((k_gdn_prep<T, D>), dim3((unsigned)nch), dim3(256), C::PREP_LDS, st_prep, q, k, v,
                     alpha, beta, ws, L);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (prof) prof(KID_GDN_PREP, st_prep, 1);
  if (st_scan != st_prep) {
    e = hipEventRecord(prep_done, st_prep);
    if (e != hipSuccess) return e;
    e = hipStreamWaitEvent(st_scan, prep_done, 0);
    if (e != hipSuccess) return e;
  }
  if (scan_dep) {  // the routes come from another stream
    e = hipStreamWaitEvent(st_scan, scan_dep, 0);
    if (e != hipSuccess) return e;
  }
  if (prof) prof(KID_GDN_SCAN, st_scan, 0);
  if constexpr (scan_head_form<T, D>()) {
    const size_t lds = SCH_ROUTE + ((size_t)nc + 15) / 16 * 16;
    if (one_wg)
      hipLaunchKernelGGL((k_gdn_scan_head<To, SCH1_NW, 1, false>), dim3((unsigned)(B * H)), dim3(64 * SCH1_NW), lds,
                         st_scan, (const bf16*)q, (const bf16*)k, route, ws, S_init, o_gdn, S_final, (bf16*)nullptr,
                         H, L, G);
    else
      hipLaunchKernelGGL((k_gdn_scan_head<To, SCH_NW, SCH_NSPLIT, false>), dim3((unsigned)(B * H * SCH_NSPLIT)),
                         dim3(64 * SCH_NW), lds, st_scan, (const bf16*)q, (const bf16*)k, route, ws, S_init, o_gdn,
                         S_final, (bf16*)nullptr, H, L, G);
  } else {
    hipLaunchKernelGGL((k_gdn_scan<T, To, D, DVT, SCAN_NS, false>), dim3((unsigned)(B * H * (D / DVT))), dim3(256),
                       0, st_scan, q, route, ws, S_init, o_gdn, S_final, (T*)nullptr, H, L, G);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (prof) prof(KID_GDN_SCAN, st_scan, 1);
  return hipSuccess;
}

// The forward in state mode, for the gradient: the chunk prep, then the scan
// writing every chunk's start state (s0, [B, H, Nc, D, D] in T) and U (u,
// [B, H, L, D] in T) instead of the outputs; one stream.
template <typename T, int D>
hipError_t launch_gdn_states(const T* q, const T* k, const T* v, const float* alpha, const float* beta,
                             const int32_t* route, const float* S_init, T* s0, T* u, void* wsp, int B, int H, int L,
                             int G, hipStream_t st) {
  using C = GdnCfg<T, D>;
  constexpr int DVT = 32;
  constexpr int SCAN_NS = sizeof(T) == 2 ? 4 : 2;
  const int nc = L / CHUNK;
  if (nc > gdn_max_chunks(sizeof(T) == 2, D)) return hipErrorInvalidValue;
  hipError_t e = set_lds_limit((const void*)k_gdn_prep<T, D>, C::PREP_LDS);
  if (e != hipSuccess) return e;
  const int64_t nch = (int64_t)B * H * nc;
  GdnWs<T, D> ws = carve<T, D>(wsp, nch);
  hipLaunchKernelGGL((k_gdn_prep<T, D>), dim3((unsigned)nch), dim3(256), C::PREP_LDS, st, q, k, v, alpha, beta, ws,
                     L);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if constexpr (scan_head_form<T, D>()) {
    e = set_lds_limit((const void*)k_gdn_scan_head<bf16, SCH_NW, SCH_NSPLIT, true>, SCH_ROUTE + SCH_MAX_NC);
    if (e != hipSuccess) return e;
    const size_t lds = SCH_ROUTE + ((size_t)nc + 15) / 16 * 16;
    hipLaunchKernelGGL((k_gdn_scan_head<bf16, SCH_NW, SCH_NSPLIT, true>), dim3((unsigned)(B * H * SCH_NSPLIT)),
                       dim3(64 * SCH_NW), lds, st, (const bf16*)q, (const bf16*)k, route, ws, S_init, (bf16*)u,
                       (float*)nullptr, (bf16*)s0, H, L, G);
  } else {
    hipLaunchKernelGGL((k_gdn_scan<T, T, D, DVT, SCAN_NS, true>), dim3((unsigned)(B * H * (D / DVT))), dim3(256), 0,
                       st, q, route, ws, S_init, u, (float*)nullptr, s0, H, L, G);
  }
  return hipGetLastError();
}
template hipError_t launch_gdn_states<float, 64>(const float*, const float*, const float*, const float*, const float*,
                                                 const int32_t*, const float*, float*, float*, void*, int, int, int,
                                                 int, hipStream_t);
template hipError_t launch_gdn_states<float, 128>(const float*, const float*, const float*, const float*,
                                                  const float*, const int32_t*, const float*, float*, float*, void*,
                                                  int, int, int, int, hipStream_t);
template hipError_t launch_gdn_states<bf16, 64>(const bf16*, const bf16*, const bf16*, const float*, const float*,
                                                const int32_t*, const float*, bf16*, bf16*, void*, int, int, int, int,
                                                hipStream_t);
template hipError_t launch_gdn_states<bf16, 128>(const bf16*, const bf16*, const bf16*, const float*, const float*,
                                                 const int32_t*, const float*, bf16*, bf16*, void*, int, int, int,
                                                 int, hipStream_t);

int gdn_max_chunks(int io_is_bf16, int D) {
  return (io_is_bf16 && D == 128) ? SCH_MAX_NC : (1 << 30);
}

#define INST(T, To, D)                                                                            \
  template hipError_t launch_gdn<T, To, D>(const T*, const T*, const T*, const float*, const float*, \
                                           const int32_t*, const float*, To*, float*, void*, int,  \
                                           int, int, int, hipStream_t, hipStream_t, hipEvent_t,     \
                                           hipEvent_t, void (*)(int, hipStream_t, int));
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
