// Definitions shared by the Gated DeltaNet forward (gdn.hip) and its
// gradient (gdn_bwd.hip): the chunk-prep configuration and workspace layout,
// fragment load / store helpers, and the 64 x 64 unit-lower-triangular
// inverse of the chunk form (T = (I + diag(beta) A)^-1).
#pragma once
#include "common.hpp"

namespace natsl {

template <typename T, int D>
struct GdnCfg {
  static constexpr int KP = D + 16 / (int)sizeof(T);   // row-layout pitch (elements)
  static constexpr int PP = CHUNK + 16 / (int)sizeof(T);
  static constexpr int LTP = CHUNK + 1;                 // fp32 pitch of L / T
  static constexpr int KF = D / 32;
  static constexpr int NT = D / 16;                     // 16-wide column tiles of D
  // LDS layout of the prep kernel (bytes).  The bf16, D = 128 form (the one
  // the head-form scan reads) keeps its buffers live one after the other in
  // one region: the K rows and L / T (products and inverse), the inverse's
  // block scratch over the dead K rows, then the K / V key-group copies over
  // everything (K and V wait in registers until the inverse is done, and each
  // lane holds the 16 values of T it needs in registers by then), so that four
  // workgroups fit in a CU's 160 KiB.
  static constexpr bool ALIAS = sizeof(T) == 2 && D == 128;
  static constexpr int RL = kg_row<T, D>();             // padded key-group row (columns)
  static constexpr int KS_BYTES = CHUNK * KP * (int)sizeof(T);
  static constexpr int KG_BYTES = 16 * RL * 4 * (int)sizeof(T);
  static constexpr int LT_BYTES = CHUNK * LTP * 4;
  static constexpr int RS_BYTES = 3 * 16 * 17 * 4;
  static constexpr int OFF_KS = 0;
  static constexpr int OFF_KG = ALIAS ? 0 : OFF_KS + KS_BYTES;
  static constexpr int OFF_VG = OFF_KG + KG_BYTES;
  static constexpr int OFF_LT = ALIAS ? KS_BYTES : OFF_VG + KG_BYTES;
  static constexpr int OFF_RS = ALIAS ? 0 : OFF_LT + LT_BYTES;
  static constexpr int OFF_GL = ALIAS ? (OFF_LT + LT_BYTES > 2 * KG_BYTES ? OFF_LT + LT_BYTES : 2 * KG_BYTES)
                                      : OFF_RS + RS_BYTES;
  static constexpr int PREP_LDS = OFF_GL + 3 * CHUNK * 4;
  static constexpr int PREP_WGS = ALIAS ? 4 : 2;        // workgroups per CU the launch bounds ask for
  static_assert(!ALIAS || (KS_BYTES % 16 == 0 && RS_BYTES <= KS_BYTES), "layout");
  static_assert(!ALIAS || PREP_WGS * PREP_LDS <= 160 * 1024, "four prep workgroups per CU");
  // per chunk-head workspace (elements).  The head-form scan (bf16, D = 128)
  // reads K itself and takes P in bf16: no K^T copy, no P remainder.
  static constexpr bool HEAD = sizeof(T) == 2 && D == 128;
  static constexpr int64_t WN = (int64_t)CHUNK * D;   // T
  static constexpr int64_t UT = (int64_t)CHUNK * D;   // float
  static constexpr int64_t KT = HEAD ? 0 : (int64_t)D * CHUNK;                 // T
  static constexpr int64_t PM = (HEAD ? 1 : 2) * (int64_t)CHUNK * CHUNK;       // T: P, and its remainder
  static constexpr int64_t GM = 144;  // float: gamma[64], gamma_C at 64, exp(g_C - g)[64] at 80
};

template <typename T, int D>
struct GdnWs {
  T* wn;
  float* ut;
  T* kt;
  T* pm;
  float* gm;
};

// The chunk prep's workspace for nch chunk-heads: carve() lays it out (from
// a 256-byte aligned base), carve_bytes() is its size.
template <typename T, int D>
static GdnWs<T, D> carve(void* ws, int64_t nch) {
  using C = GdnCfg<T, D>;
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  char* p = (char*)ws;
  GdnWs<T, D> w;
  w.wn = (T*)p; p += al(C::WN * nch * sizeof(T));
  w.ut = (float*)p; p += al(C::UT * nch * sizeof(float));
  w.kt = C::KT ? (T*)p : nullptr; p += al(C::KT * nch * sizeof(T));
  w.pm = (T*)p; p += al(C::PM * nch * sizeof(T));
  w.gm = (float*)p;
  return w;
}
template <typename T, int D>
static size_t carve_bytes(int64_t nch) {
  using C = GdnCfg<T, D>;
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  return al(C::WN * nch * sizeof(T)) + al(C::UT * nch * sizeof(float)) + al(C::KT * nch * sizeof(T)) +
         al(C::PM * nch * sizeof(T)) + al(C::GM * nch * sizeof(float));
}

// The scan runs one workgroup per head for bf16 with D = 128, and one per
// (head, 32-column slice) otherwise; the two read -W in different orders.
template <typename T, int D> constexpr bool scan_head_form() { return sizeof(T) == 2 && D == 128; }

// T = (I + L)^-1 in place in LT (fp32, pitch LTP, L strictly lower
// triangular, zero elsewhere; the diagonal blocks' upper halves are written
// with zeros by the solve), for a 256-thread workgroup; Rs is scratch of 3 x
// 16 x 17 floats.  Ends with a barrier.
//   (a) 16x16 diagonal blocks: lane j of wave w solves column j of block w by
//       forward substitution.
//   (b) block rows a = 1..3:  T_ab = -T_aa * sum_{b<=m<a} L_am T_mb, on fp32
//       MFMA (16x16x4: in step j lane (g, c) gives A[c][4j + g] and B[4j +
//       g][c], and holds C[4g + i][c]).  Wave w owns the target block (a, w)
//       of every round a > w.  All L_am and T_aa fragments a wave needs are
//       read before the first round writes, so a round's writes (which
//       replace L_ab by T_ab) never race with reads of the blocks they
//       replace: one barrier per round.
template <int LTP>
__device__ __forceinline__ void lt_inverse64(float* LT, float* Rs) {
  const int lane = lane_id(), w = wave_id();
  const int g = lane >> 4, c = lane & 15;
  if (lane < 16) {
    const int j = lane, o = 16 * w;
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float acc = (r == j) ? 1.f : 0.f;
#pragma unroll
      for (int i = 0; i < r; ++i) acc -= LT[(o + r) * LTP + o + i] * x[i];
      x[r] = acc;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) LT[(o + r) * LTP + o + j] = x[r];
  }
  __syncthreads();
  float la[3][3][4], ta[3][4];
#pragma unroll
  for (int a = 1; a < 4; ++a) {
    if (w < a) {
#pragma unroll
      for (int m = 0; m < 3; ++m)
        if (m >= w && m < a) {
#pragma unroll
          for (int j = 0; j < 4; ++j) la[a - 1][m][j] = LT[(16 * a + c) * LTP + 16 * m + 4 * j + g];
        }
#pragma unroll
      for (int j = 0; j < 4; ++j) ta[a - 1][j] = LT[(16 * a + c) * LTP + 16 * a + 4 * j + g];
    }
  }
  float* Rw = Rs + w * 16 * 17;  // wave-private 16 x 16 scratch (waves 0..2)
#pragma unroll
  for (int a = 1; a < 4; ++a) {
    if (w < a) {
      f32x4 r = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int m = 0; m < 3; ++m)
        if (m >= w && m < a) {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            r = __builtin_amdgcn_mfma_f32_16x16x4f32(la[a - 1][m][j], LT[(16 * m + 4 * j + g) * LTP + 16 * w + c], r, 0,
                                                     0, 0);
        }
      // R (accumulator layout) -> B operand layout through the wave's scratch
#pragma unroll
      for (int i = 0; i < 4; ++i) Rw[(4 * g + i) * 17 + c] = r[i];
      f32x4 tt = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 4; ++j)
        tt = __builtin_amdgcn_mfma_f32_16x16x4f32(ta[a - 1][j], Rw[(4 * j + g) * 17 + c], tt, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) LT[(16 * a + 4 * g + i) * LTP + 16 * w + c] = -tt[i];
    }
    __syncthreads();
  }
}

}  // namespace natsl
