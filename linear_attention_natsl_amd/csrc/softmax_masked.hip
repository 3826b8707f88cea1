// Softmax branch: "Technische Samenvatting: Neural Attention Search Linear
// (NAtS-L)", Kernmechanismen 3 -- inside every chunk both correlations are
// computed, and the softmax operation keeps only the KV of the chunks routed to
// it.  A query of chunk c therefore attends to the tokens of the softmax chunks
// before c (the compacted list sel_idx[0 .. nsel_before[c])) plus the causal
// prefix of its own chunk.
//
// Flash-style online softmax on MFMA (gfx950, wave64):
//   * one workgroup = 4 waves = 128 queries (two chunks c0 = 2p, c1 = 2p + 1);
//     wave w owns queries 32w .. 32w+31 of the block;
//   * the key loop walks the compacted chunk list, then c0, then c1; every key
//     tile is exactly one 64-token chunk (contiguous 16 KiB bf16 rows, so the
//     gather through sel_idx costs nothing in coalescing);
//   * per tile a wave is FULL (all keys visible), DIAG (causal mask inside its
//     own chunk) or SKIP (c1's queries and c0's tile when c0 is linear-routed;
//     c0's queries never see c1);
//   * S^T = K Q^T with K from LDS (A operand) and Q held in registers
//     (B operand); its accumulator layout (lane = query, 4 keys per lane) is
//     directly the B operand of O^T = V^T P^T, so P never leaves registers and
//     the per-query rescale is lane-local;
//   * V is stored in LDS in the key-group layout (4 keys of one column in 8
//     bytes, swizzled) that the A operand of V^T needs;
//   * K/V tiles are double-buffered: the next tile's global loads are in flight
//     while the current tile is computed;
//   * blocks are issued longest-first (later query chunks see more keys), and
//     on the 8 XCDs every XCD serves a fixed set of heads so the K/V tiles those
//     blocks stream stay in that XCD's L2.
#include "common.hpp"
#include "kernels.hpp"

namespace natsl {

template <typename T, int D>
struct SmCfg {
  static constexpr int KP = D + 16 / (int)sizeof(T);   // K row pitch (elements), 16 B pad
  static constexpr int KTILE = CHUNK * KP;              // elements
  static constexpr int VRL = kg_row<T, D>();            // padded key-group row (columns)
  static constexpr int VTILE = (CHUNK / 4) * VRL * 4;   // elements (key-group layout)
  static constexpr int BUF = KTILE + VTILE;
  static constexpr int LDS_BYTES = 2 * BUF * (int)sizeof(T);
  static constexpr int KF = D / 32;                     // contraction steps over D
  static constexpr int KLOADS = (CHUNK * D / 8) / 256;  // 8-element K loads per thread
  static constexpr int VTASKS = (CHUNK / 4) * (D / 8);  // (key group, 8 columns) tasks
  static constexpr int VT = (VTASKS + 255) / 256;
};

// store 4 elements (one per token of a key group) for one column
template <typename T> __device__ __forceinline__ void store_col4(T* p, T a, T b, T c, T d);
template <> __device__ __forceinline__ void store_col4<bf16>(bf16* p, bf16 a, bf16 b, bf16 c, bf16 d) {
  bf16x4 v = {a, b, c, d};
  *reinterpret_cast<bf16x4*>(p) = v;
}
template <> __device__ __forceinline__ void store_col4<float>(float* p, float a, float b, float c, float d) {
  f32x4 v = {a, b, c, d};
  *reinterpret_cast<f32x4*>(p) = v;
}

template <typename T, int D>
struct TileRegs {
  Frag<T> k[SmCfg<T, D>::KLOADS];
  Frag<T> v[SmCfg<T, D>::VT][4];
};

template <typename T, int D>
__device__ __forceinline__ void tile_gload(TileRegs<T, D>& r, const T* kbase, const T* vbase) {
  using C = SmCfg<T, D>;
  const int t = tid_x();
#pragma unroll
  for (int i = 0; i < C::KLOADS; ++i) {
    const int e = t + 256 * i;
    const int row = e / (D / 8), col = (e % (D / 8)) * 8;
    r.k[i] = load8<T>(kbase + row * D + col);
  }
#pragma unroll
  for (int i = 0; i < C::VT; ++i) {
    const int task = t + 256 * i;
    if (task < C::VTASKS) {
      const int kg = task / (D / 8), col = (task % (D / 8)) * 8;
#pragma unroll
      for (int tk = 0; tk < 4; ++tk) r.v[i][tk] = load8<T>(vbase + (4 * kg + tk) * D + col);
    }
  }
}

template <typename T, int D>
__device__ __forceinline__ void tile_sstore(const TileRegs<T, D>& r, T* buf) {
  using C = SmCfg<T, D>;
  const int t = tid_x();
  T* ks = buf;
  T* vs = buf + C::KTILE;
#pragma unroll
  for (int i = 0; i < C::KLOADS; ++i) {
    const int e = t + 256 * i;
    const int row = e / (D / 8), col = (e % (D / 8)) * 8;
    store8<T>(ks + row * C::KP + col, r.k[i]);
  }
#pragma unroll
  for (int i = 0; i < C::VT; ++i) {
    const int task = t + 256 * i;
    if (task < C::VTASKS) {
      const int kg = task / (D / 8), col = (task % (D / 8)) * 8;
      if constexpr (sizeof(T) == 2) {
        // 4 tokens x 8 columns of bf16 transposed in registers: word m of
        // token tk holds columns 2m (low half) and 2m + 1 (high half); v_perm
        // pairs the halves of two tokens (element extraction from the bf16
        // vectors went through scratch memory)
        uint32_t w[4][4];
#pragma unroll
        for (int tk = 0; tk < 4; ++tk) {
          const uint4 u = __builtin_bit_cast(uint4, r.v[i][tk].v);
          w[tk][0] = u.x; w[tk][1] = u.y; w[tk][2] = u.z; w[tk][3] = u.w;
        }
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const uint2 lo = {__builtin_amdgcn_perm(w[1][m], w[0][m], 0x05040100u),
                            __builtin_amdgcn_perm(w[3][m], w[2][m], 0x05040100u)};
          const uint2 hi = {__builtin_amdgcn_perm(w[1][m], w[0][m], 0x07060302u),
                            __builtin_amdgcn_perm(w[3][m], w[2][m], 0x07060302u)};
          *reinterpret_cast<uint2*>(vs + kg_index<C::VRL>(kg, col + 2 * m)) = lo;
          *reinterpret_cast<uint2*>(vs + kg_index<C::VRL>(kg, col + 2 * m + 1)) = hi;
        }
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j)
          store_col4<T>(vs + kg_index<C::VRL>(kg, col + j), frag_get<T>(r.v[i][0], j),
                        frag_get<T>(r.v[i][1], j), frag_get<T>(r.v[i][2], j),
                        frag_get<T>(r.v[i][3], j));
      }
    }
  }
}

enum { MODE_SKIP = 0, MODE_FULL = 1, MODE_DIAG = 2, MODE_WSTART = 3 };
constexpr float RESCALE_TH = 8.0f;  // log2 units

template <typename T, typename To, int D>
__global__ void __launch_bounds__(256, 2)
    k_softmax_masked(const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
                     const int32_t* __restrict__ sel_idx, const int32_t* __restrict__ nsel_before,
                     To* __restrict__ o_sm, float* __restrict__ lse, int H, int L, int G,
                     float scale_log2, const T* __restrict__ pre_k, const T* __restrict__ pre_v,
                     const int32_t* __restrict__ pnc, int pcap, int win) {
  // win > 0: sliding-window mode instead of the routed key set: a query of
  // chunk c at offset j sees chunk c - win from offset j + 1 on, the chunks
  // in between in full and chunk c up to offset j (the win * 64 most recent
  // tokens including itself); sel_idx, nsel_before and the prefix are unused
  using C = SmCfg<T, D>;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  T* smem = reinterpret_cast<T*>(smem_raw);

  const int nc = L / CHUNK;
  const int nb = (nc + 1) / 2;
  const int BH = (int)(grid_dim_x() / nb);
  const int p = bid_x();
  int qblk, bh;
  if ((BH & 7) == 0) {
    const int xcd = p & 7, slot = p >> 3, hpx = BH >> 3;
    qblk = nb - 1 - slot / hpx;
    bh = (slot % hpx) * 8 + xcd;
  } else {
    qblk = nb - 1 - p / BH;
    bh = p % BH;
  }
  const int b = bh / H, h = bh % H;
  const int grp = (G == 1) ? 0 : h;
  const int c0 = 2 * qblk, c1 = c0 + 1;
  const bool has_c1 = c1 < nc;
  const int32_t* sel = win > 0 ? nullptr : sel_idx + ((int64_t)b * G + grp) * nc;
  const int32_t* nsbp = win > 0 ? nullptr : nsel_before + ((int64_t)b * G + grp) * (nc + 1);
  // key tiles: the prefix cache's rows (npre tiles), the softmax chunks
  // before c0, c0, c1
  // (rows of a cache that overflowed were never written: at most cap rows);
  // window mode: chunks c1 (or c0) down to wlo, newest first, so that every
  // query meets its own (diagonal) chunk before the chunk where its window
  // starts, which may hide all of its keys from it
  const int wlo = max(0, c0 - win);
  const int whi = has_c1 ? c1 : c0;
  const int npre = (win == 0 && pnc) ? min(pnc[(int64_t)b * G + grp], pcap) / CHUNK : 0;
  const int nsel = win > 0 ? 0 : nsbp[c0];
  const int nsb = npre + nsel;
  const bool c0_sm = win > 0 ? false : nsbp[c0 + 1] > nsel;
  const int ntiles = win > 0 ? whi - wlo + 1 : nsb + 1 + (has_c1 ? 1 : 0);

  const int lane = lane_id(), w = wave_id();
  const int g = lane >> 4, c = lane & 15;
  const bool my_c1 = w >= 2;
  const bool active = !my_c1 || has_c1;
  const int64_t head_off = (int64_t)bh * L * D;
  const T* qh = q + head_off;
  const T* kh = k + head_off;
  const T* vh = v + head_off;

  // Q fragments: B operand of S^T = K Q^T (column = query, rows = d)
  Frag<T> qf[2][C::KF];
  const int qtok0 = c0 * CHUNK + 32 * w;
#pragma unroll
  for (int qs = 0; qs < 2; ++qs)
#pragma unroll
    for (int ks = 0; ks < C::KF; ++ks) {
      if (active) qf[qs][ks] = load8<T>(qh + (int64_t)(qtok0 + 16 * qs + c) * D + 32 * ks + 8 * g);
      else qf[qs][ks] = load8<T>(qh + 32 * ks + 8 * g);  // any in-bounds row; unused
    }

  f32x4 o[D / 16][2];
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
    for (int qs = 0; qs < 2; ++qs) o[dt][qs] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run[2] = {-INFINITY, -INFINITY};
  float l_run[2] = {0.f, 0.f};

  const int64_t pre_off = (int64_t)bh * pcap * D;
  auto tile_load = [&](TileRegs<T, D>& r, int it) {
    if (win > 0) {
      const int kc = whi - it;
      tile_gload<T, D>(r, kh + (int64_t)kc * CHUNK * D, vh + (int64_t)kc * CHUNK * D);
    } else if (it < npre) {
      tile_gload<T, D>(r, pre_k + pre_off + (int64_t)it * CHUNK * D, pre_v + pre_off + (int64_t)it * CHUNK * D);
    } else {
      const int j = it - npre;
      const int kc = j < nsel ? sel[j] : (j == nsel ? c0 : c1);
      tile_gload<T, D>(r, kh + (int64_t)kc * CHUNK * D, vh + (int64_t)kc * CHUNK * D);
    }
  };

  TileRegs<T, D> pre;
  tile_load(pre, 0);
  tile_sstore<T, D>(pre, smem);
  __syncthreads();

  const int qrow_base = 32 * (w & 1);  // query row inside its own chunk, minus 16qs + c
  for (int it = 0; it < ntiles; ++it) {
    const bool more = it + 1 < ntiles;
    if (more) tile_load(pre, it + 1);
    int mode;
    if (win > 0) {
      const int kc = whi - it, cw = my_c1 ? c1 : c0;
      mode = (kc > cw || kc < cw - win) ? MODE_SKIP : (kc == cw) ? MODE_DIAG : (kc == cw - win) ? MODE_WSTART
                                                                                                   : MODE_FULL;
    } else if (it < nsb) mode = MODE_FULL;
    else if (it == nsb) mode = my_c1 ? (c0_sm ? MODE_FULL : MODE_SKIP) : MODE_DIAG;
    else mode = my_c1 ? MODE_DIAG : MODE_SKIP;
    if (!active) mode = MODE_SKIP;

    if (mode != MODE_SKIP) {
      const T* ks_lds = smem + (it & 1) * C::BUF;
      const T* vs_lds = ks_lds + C::KTILE;
      f32x4 s[4][2];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int qs = 0; qs < 2; ++qs) s[kt][qs] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < C::KF; ++ks)
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
          const Frag<T> a = load8<T>(ks_lds + (16 * kt + c) * C::KP + 32 * ks + 8 * g);
#pragma unroll
          for (int qs = 0; qs < 2; ++qs) mma(s[kt][qs], a, qf[qs][ks]);
        }

      // Online softmax in log2 units.  The running max only moves when a
      // row's tile max exceeds it by more than RESCALE_TH, so p = 2^(s - m)
      // stays <= 2^RESCALE_TH (exact enough in fp32 and bf16) and the O
      // rescale (D/16 x 4 multiplies per row block) is skipped for most
      // tiles; the final division by the matching row sum is unaffected.
      Frag<T> pf[2][2];
#pragma unroll
      for (int qs = 0; qs < 2; ++qs) {
        const int qrow = qrow_base + 16 * qs + c;
        if (mode == MODE_DIAG) {
#pragma unroll
          for (int kt = 0; kt < 4; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if ((16 * kt + 4 * g + i) > qrow) s[kt][qs][i] = -INFINITY;
        } else if (mode == MODE_WSTART) {  // keys already past the window's start
#pragma unroll
          for (int kt = 0; kt < 4; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if ((16 * kt + 4 * g + i) <= qrow) s[kt][qs][i] = -INFINITY;
        }
        float mt = fmaxf(fmaxf(s[0][qs][0], s[0][qs][1]), fmaxf(s[0][qs][2], s[0][qs][3]));
#pragma unroll
        for (int kt = 1; kt < 4; ++kt)
          mt = fmaxf(mt, fmaxf(fmaxf(s[kt][qs][0], s[kt][qs][1]), fmaxf(s[kt][qs][2], s[kt][qs][3])));
        mt = wave_max_xor(mt, 16);
        mt = wave_max_xor(mt, 32);
        mt *= scale_log2;  // scale > 0: max commutes with scaling
        if (__ballot(mt > m_run[qs] + RESCALE_TH) != 0) {
          const float m_new = fmaxf(m_run[qs], mt);
          // 0 on a row's first visible tile; a row that has still seen no
          // visible key (m stays -inf) keeps its zeros
          const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run[qs] - m_new);
          m_run[qs] = m_new;
          l_run[qs] *= alpha;
#pragma unroll
          for (int dt = 0; dt < D / 16; ++dt) o[dt][qs] *= alpha;
        }
        // (a row that has seen no visible key yet keeps m = -inf: its
        // weights are 0, not 2^(-inf + inf))
        const float nm = m_run[qs] == -INFINITY ? 0.f : -m_run[qs];
        float ls = 0.f;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float pv = __builtin_amdgcn_exp2f(fmaf(s[kt][qs][i], scale_log2, nm));
            s[kt][qs][i] = pv;
            ls += pv;
          }
        l_run[qs] += ls;
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            frag_set(pf[qs][k2], j, s[2 * k2][qs][j]);
            frag_set(pf[qs][k2], 4 + j, s[2 * k2 + 1][qs][j]);
          }
      }
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
          const Frag<T> a = ld4x2<T>(vs_lds + kg_index<C::VRL>(8 * k2 + g, 16 * dt + c),
                                       vs_lds + kg_index<C::VRL>(8 * k2 + 4 + g, 16 * dt + c));
#pragma unroll
          for (int qs = 0; qs < 2; ++qs) mma(o[dt][qs], a, pf[qs][k2]);
        }
    }
    if (more) tile_sstore<T, D>(pre, smem + ((it + 1) & 1) * C::BUF);
    __syncthreads();
  }

  if (!active) return;
#pragma unroll
  for (int qs = 0; qs < 2; ++qs) {
    float lt = l_run[qs];
    lt = wave_sum_xor(lt, 16);
    lt = wave_sum_xor(lt, 32);
    const float inv = 1.0f / lt;
    const int64_t tok = qtok0 + 16 * qs + c;
    To* orow = o_sm + head_off + tok * D;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      float vals[4] = {o[dt][qs][0] * inv, o[dt][qs][1] * inv, o[dt][qs][2] * inv,
                       o[dt][qs][3] * inv};
      store4f<To>(orow + 16 * dt + 4 * g, vals);
    }
    if (lse && g == 0) lse[(int64_t)bh * L + tok] = (m_run[qs] + log2f(lt)) * LN2;
  }
}


// ---------------------------------------------------------------------------
// bf16, D = 128: deep-pipelined variant.
//
// Measured on the kernel above, a tile costs ~9.4k cycles of which ~5.3k are
// spent issuing and waiting for the next tile's global loads: every block of
// a head streams the same K/V chunks in lockstep, so each tile is an L2 miss
// for someone and one tile of prefetch cannot cover it.  Here the K/V tiles
// go straight from global memory into a 4-stage LDS ring
// (global_load_lds_dwordx4, no register staging) three tiles ahead.  Rows are
// stored contiguously with a 16-byte-chunk XOR swizzle (the direct loads fill
// 1 KiB of LDS per wave instruction, so rows cannot be padded):
//   K: chunk q of row r at slot q ^ (r & 15)        (conflict-free A reads)
//   V: chunk q of row r at slot q ^ ((r & 7) << 1)  (conflict-free transposed reads)
// V stays row-major; the A operand of O^T = V^T P^T (4 keys of one column per
// 8 bytes) comes from ds_read_b64_tr_b16, which transposes 4 x 4 blocks of
// 16-bit values across each group of 16 lanes.
// One workgroup = 8 waves = 4 chunks; waves 2m and 2m+1 own the 64 queries of
// chunk c0 + m (32 each), so register use matches the kernel above.
// Window mode (win > 0 chunks, no routes): the key tiles are chunks c0 - win
// .. c0 + 3, newest first, so that every query's first visible tile is its
// own (causal) chunk; chunk c - win keeps only keys past the query's offset.
constexpr int SM2_STAGES = 4;
constexpr int SM2_TILE_BYTES = 2 * CHUNK * 128 * 2;  // K + V, bf16, D = 128
constexpr int SM2_LIST = 4096;  // key-tile list entries (prefix tiles + softmax chunks + own chunks)
constexpr int SM2_LDS = SM2_STAGES * SM2_TILE_BYTES + 4 * SM2_LIST;
static_assert(SM2_LDS <= LDS_MAX_BYTES, "ring + tile list exceed the LDS");

__device__ __forceinline__ int sm2_kslot(int r, int q) { return q ^ (r & 15); }
__device__ __forceinline__ int sm2_vslot(int r, int q) { return q ^ ((r & 7) << 1); }

template <typename To>
__global__ void __launch_bounds__(512, 1)
    k_softmax_v2(const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
                 const int32_t* __restrict__ sel_idx, const int32_t* __restrict__ nsel_before,
                 To* __restrict__ o_sm, float* __restrict__ lse, int H, int L, int G, float scale_log2,
                 const bf16* __restrict__ pre_k, const bf16* __restrict__ pre_v, const int32_t* __restrict__ pnc,
                 int pcap, const float* __restrict__ w_mix, int64_t wmix_hs, float* __restrict__ mixd, int win) {
  constexpr int D = 128;
  extern __shared__ __align__(16) unsigned char lds[];
  int32_t* sel_l = reinterpret_cast<int32_t*>(lds + SM2_STAGES * SM2_TILE_BYTES);

  const int nc = L / CHUNK;
  const int nb = (nc + 3) / 4;
  const int BH = (int)(grid_dim_x() / nb);
  const int p = bid_x();
  int qblk, bh;
  if ((BH & 7) == 0) {
    const int xcd = p & 7, slot = p >> 3, hpx = BH >> 3;
    qblk = nb - 1 - slot / hpx;
    bh = (slot % hpx) * 8 + xcd;
  } else {
    qblk = nb - 1 - p / BH;
    bh = p % BH;
  }
  const int b = bh / H, h = bh % H;
  const int grp = (G == 1) ? 0 : h;
  const int c0 = 4 * qblk;
  const int nown = min(4, nc - c0);
  // key tiles: the prefix cache's rows (npre tiles), the softmax chunks
  // before c0, then the block's own chunks
  // (rows of a cache that overflowed were never written: at most cap rows)
  int npre = 0, nsel = 0, nsb = 0, ntiles, sm_bits = 0;
  const int32_t* sel = nullptr;
  if (win > 0) {
    ntiles = c0 + nown - max(0, c0 - win);
  } else {
    sel = sel_idx + ((int64_t)b * G + grp) * nc;
    const int32_t* nsbp = nsel_before + ((int64_t)b * G + grp) * (nc + 1);
    npre = pnc ? min(pnc[(int64_t)b * G + grp], pcap) / CHUNK : 0;
    nsel = nsbp[c0];
    nsb = npre + nsel;
    ntiles = nsb + nown;
    for (int j = 0; j < nown; ++j) sm_bits |= (nsbp[c0 + j + 1] > nsbp[c0 + j]) ? (1 << j) : 0;
  }

  const int lane = lane_id(), w = wave_id();
  const int g = lane >> 4, c = lane & 15;
  const int mch = w >> 1;            // chunk of this wave within the block
  const bool active = mch < nown;
  const int64_t head_off = (int64_t)bh * L * D;
  const bf16* kh = k + head_off;
  const bf16* vh = v + head_off;

  // tile list in LDS (keeps its reads out of the vector-memory counter):
  // prefix tile j is stored as -1 - j
  if (win > 0) {
    for (int i = tid_x(); i < ntiles; i += 512) sel_l[i] = c0 + nown - 1 - i;  // newest first
  } else {
    for (int i = tid_x(); i < npre; i += 512) sel_l[i] = -1 - i;
    for (int i = tid_x(); i < nsel; i += 512) sel_l[npre + i] = sel[i];
    for (int i = tid_x(); i < nown; i += 512) sel_l[nsb + i] = c0 + i;
  }
  const int64_t pre_off = (int64_t)bh * pcap * D;

  Frag<bf16> qf[2][4];
  const int qtok0 = (c0 + (active ? mch : 0)) * CHUNK + 32 * (w & 1);
#pragma unroll
  for (int qs = 0; qs < 2; ++qs)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qf[qs][ks] = load8<bf16>(q + head_off + (int64_t)(qtok0 + 16 * qs + c) * D + 32 * ks + 8 * g);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): nothing of ours outstanding before the ring starts
  __syncthreads();

  // tile `it` -> stage it % STAGES: 2 K + 2 V 16-byte loads per thread
  auto issue = [&](int it) {
    const int kc = sel_l[it];
    unsigned char* st = lds + (it % SM2_STAGES) * SM2_TILE_BYTES;
    const bf16* kg = kc >= 0 ? kh + (int64_t)kc * CHUNK * D : pre_k + pre_off + (int64_t)(-1 - kc) * CHUNK * D;
    const bf16* vg = kc >= 0 ? vh + (int64_t)kc * CHUNK * D : pre_v + pre_off + (int64_t)(-1 - kc) * CHUNK * D;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int e0 = w * 128 + i * 64;  // first 16-byte chunk of this wave instruction
      const int e = e0 + lane, r = e >> 4, sl = e & 15;
      gload_lds16(kg + r * D + sm2_kslot(r, sl) * 8, st + e0 * 16);
      gload_lds16(vg + r * D + sm2_vslot(r, sl) * 8, st + CHUNK * D * 2 + e0 * 16);
    }
  };

  f32x4 o[D / 16][2];
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
    for (int qs = 0; qs < 2; ++qs) o[dt][qs] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run[2] = {-INFINITY, -INFINITY};
  float l_run[2] = {0.f, 0.f};

#pragma unroll
  for (int j = 0; j < SM2_STAGES - 1; ++j)
    if (j < ntiles) issue(j);

  const int qrow_base = 32 * (w & 1);
  Frag<bf16> va[D / 16][2];
  Frag<bf16> pf[2][2];
  auto pv = [&]() {
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
        for (int qs = 0; qs < 2; ++qs) mma(o[dt][qs], va[dt][k2], pf[qs][k2]);
  };
  for (int it = 0; it < ntiles; ++it) {
    wait_vm(4 * (min(it + SM2_STAGES - 2, ntiles - 1) - it));  // this tile's loads have landed
    lds_barrier();                                              // ... for every wave
    if (it + SM2_STAGES - 1 < ntiles) issue(it + SM2_STAGES - 1);  // into the stage read last iteration

    int mode;
    if (win > 0) {
      const int dm = mch - (nown - 1 - it);  // query chunk - key chunk
      mode = dm < 0 ? MODE_SKIP : dm == 0 ? MODE_DIAG : dm < win ? MODE_FULL : dm == win ? MODE_WSTART : MODE_SKIP;
    } else if (it < nsb) {
      mode = MODE_FULL;
    } else {
      const int j = it - nsb;
      mode = (j == mch) ? MODE_DIAG : (j < mch && ((sm_bits >> j) & 1)) ? MODE_FULL : MODE_SKIP;
    }
    if (!active) mode = MODE_SKIP;
    if (mode == MODE_SKIP) continue;

    const unsigned char* st = lds + (it % SM2_STAGES) * SM2_TILE_BYTES;
    const bf16* ks_l = reinterpret_cast<const bf16*>(st);
    const unsigned char* vs_l = st + CHUNK * D * 2;
    f32x4 s[4][2];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int qs = 0; qs < 2; ++qs) s[kt][qs] = f32x4{0.f, 0.f, 0.f, 0.f};
    // all 16 K fragments of the tile are read before the 32 products, so the
    // reads' latency overlaps instead of stalling each pair of products
    {
      Frag<bf16> ka[4][4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
          const int r = 16 * kt + c;
          ka[ks][kt] = load8<bf16>(ks_l + r * D + sm2_kslot(r, 4 * ks + g) * 8);
        }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int qs = 0; qs < 2; ++qs) mma(s[kt][qs], ka[ks][kt], qf[qs][ks]);
    }

    // V^T fragments by transposed reads, issued before the softmax work so
    // that it hides their latency: lane c of group g reads row
    // 32 k2 + 4 g + c / 4 (+16 for the second half), columns 16 dt + 4 (c % 4) .. +3
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      const int colq = (16 * dt + 4 * (c & 3)) >> 3;  // 16-byte chunk of the 4 columns
      const int half = ((c & 3) & 1) * 8;            // byte offset inside it
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
        const int r0 = 32 * k2 + 4 * g + (c >> 2), r1 = r0 + 16;
        const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) v4i16*)(vs_l + r0 * 256 + sm2_vslot(r0, colq) * 16 + half));
        const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) v4i16*)(vs_l + r1 * 256 + sm2_vslot(r1, colq) * 16 + half));
        va[dt][k2].v = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if (mode == MODE_DIAG) {
#pragma unroll
      for (int qs = 0; qs < 2; ++qs)
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if ((16 * kt + 4 * g + i) > qrow_base + 16 * qs + c) s[kt][qs][i] = -INFINITY;
    } else if (mode == MODE_WSTART) {  // only keys past the window's start
#pragma unroll
      for (int qs = 0; qs < 2; ++qs)
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if ((16 * kt + 4 * g + i) <= qrow_base + 16 * qs + c) s[kt][qs][i] = -INFINITY;
    }
    // tile max per query (its 4 lane groups hold 16 keys each), one rescale
    // decision for the wave
    float mt[2];
    bool up = false;
#pragma unroll
    for (int qs = 0; qs < 2; ++qs) {
      float x = fmaxf(fmaxf(s[0][qs][0], s[0][qs][1]), fmaxf(s[0][qs][2], s[0][qs][3]));
#pragma unroll
      for (int kt = 1; kt < 4; ++kt)
        x = fmaxf(x, fmaxf(fmaxf(s[kt][qs][0], s[kt][qs][1]), fmaxf(s[kt][qs][2], s[kt][qs][3])));
      mt[qs] = group4_max(x) * scale_log2;
      up |= mt[qs] > m_run[qs] + RESCALE_TH;
    }
    if (__ballot(up) != 0) {
#pragma unroll
      for (int qs = 0; qs < 2; ++qs) {
        const float m_new = fmaxf(m_run[qs], mt[qs]);
        const float alpha = __builtin_amdgcn_exp2f(m_run[qs] - m_new);
        m_run[qs] = m_new;
        l_run[qs] *= alpha;
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) o[dt][qs] *= alpha;
      }
    }
#pragma unroll
    for (int qs = 0; qs < 2; ++qs) {
      const float nm = -m_run[qs];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) s[kt][qs][i] = __builtin_amdgcn_exp2f(fmaf(s[kt][qs][i], scale_log2, nm));
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          frag_set(pf[qs][k2], j, s[2 * k2][qs][j]);
          frag_set(pf[qs][k2], 4 + j, s[2 * k2 + 1][qs][j]);
        }
      // row sum of the bf16 weights the product uses, two per dot2 (fp32 accumulate)
      float ls = l_run[qs];
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const bf16x2 pr = {pf[qs][k2].v[2 * j], pf[qs][k2].v[2 * j + 1]};
          ls = __builtin_amdgcn_fdot2_f32_bf16(pr, bf16x2{(bf16)1.f, (bf16)1.f}, ls, false);
        }
      l_run[qs] = ls;
    }
    // O^T += V^T P^T
    pv();
  }

  if (!active) return;
#pragma unroll
  for (int qs = 0; qs < 2; ++qs) {
    const float lt = group4_sum(l_run[qs]);
    const float inv = 1.0f / lt;
    const int64_t tok = qtok0 + 16 * qs + c;
    To* orow = o_sm + head_off + tok * D;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      float vals[4] = {o[dt][qs][0] * inv, o[dt][qs][1] * inv, o[dt][qs][2] * inv, o[dt][qs][3] * inv};
      store4f<To>(orow + 16 * dt + 4 * g, vals);
    }
    if (lse && g == 0) lse[(int64_t)bh * L + tok] = (m_run[qs] + log2f(lt)) * LN2;
  }
  // the merge's mixing scores, from the q fragments already in registers:
  // lane group g holds q[t][32 ks + 8 g + j], whose W_mix rows are 16
  // consecutive floats per ks
  if (mixd) {
    const float* wm = w_mix + (int64_t)h * wmix_hs;
#pragma unroll
    for (int qs = 0; qs < 2; ++qs) {
      float z0 = 0.f, z1 = 0.f;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const f32x4* w4 = reinterpret_cast<const f32x4*>(wm + (32 * ks + 8 * g) * 2);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const f32x4 ww = w4[jj];  // W_mix rows 32 ks + 8 g + 2 jj and + 1, both columns
          const float qa = (float)qf[qs][ks].v[2 * jj], qb = (float)qf[qs][ks].v[2 * jj + 1];
          z0 += qa * ww[0] + qb * ww[2];
          z1 += qa * ww[1] + qb * ww[3];
        }
      }
      z0 = group4_sum(z0);
      z1 = group4_sum(z1);
      if (g == 0) mixd[(int64_t)bh * L + qtok0 + 16 * qs + c] = z0 - z1;
    }
  }
}

template <typename T, typename To, int D>
hipError_t launch_softmax_masked(const T* q, const T* k, const T* v, const int32_t* sel_idx,
                                 const int32_t* nsel_before, To* o_sm, float* lse, int B, int H,
                                 int L, int G, float scale, hipStream_t st, const SmPrefix& pre,
                                 const SmMix& mix) {
  using C = SmCfg<T, D>;
  if (mix.done) *mix.done = false;
  if constexpr (sizeof(T) == 2 && D == 128) {
    const int nc = L / CHUNK;
    // the tile list (prefix tiles + chunks) lives in an SM2_LIST-entry LDS
    // array; a longer list (a prefix cache of more than 4096 - nc chunks)
    // takes the kernel below, which reads the chunk list from global memory
    if ((int64_t)nc + (pre.n_committed ? pre.cap / CHUNK : 0) <= SM2_LIST) {
      hipError_t e = set_lds_limit((const void*)k_softmax_v2<To>, SM2_LDS);
      if (e != hipSuccess) return e;
      const int64_t grid = (int64_t)B * H * ((nc + 3) / 4);
      hipLaunchKernelGGL(k_softmax_v2<To>, dim3((unsigned)grid), dim3(512), SM2_LDS, st, (const bf16*)q,
                         (const bf16*)k, (const bf16*)v, sel_idx, nsel_before, o_sm, lse, H, L, G, scale * LOG2E,
                         (const bf16*)pre.k, (const bf16*)pre.v, pre.n_committed, pre.cap, mix.w_mix, mix.hs,
                         mix.w_mix ? mix.d : nullptr, 0);
      e = hipGetLastError();
      if (e == hipSuccess && mix.done) *mix.done = mix.w_mix && mix.d;
      return e;
    }
  }
  const hipError_t ea = set_lds_limit((const void*)k_softmax_masked<T, To, D>, C::LDS_BYTES);
  if (ea != hipSuccess) return ea;
  const int nc = L / CHUNK;
  const int nb = (nc + 1) / 2;
  const int64_t grid = (int64_t)B * H * nb;
  hipLaunchKernelGGL((k_softmax_masked<T, To, D>), dim3((unsigned)grid), dim3(256), C::LDS_BYTES,
                     st, q, k, v, sel_idx, nsel_before, o_sm, lse, H, L, G, scale * LOG2E, (const T*)pre.k,
                     (const T*)pre.v, pre.n_committed, pre.cap, 0);
  return hipGetLastError();
}

template <typename T, typename To, int D>
hipError_t launch_softmax_window(const T* q, const T* k, const T* v, To* o, float* lse, int B, int H, int L,
                                 int win_chunks, float scale, hipStream_t st) {
  using C = SmCfg<T, D>;
  if (win_chunks < 1) return hipErrorInvalidValue;
  const int nc = L / CHUNK;
  if constexpr (sizeof(T) == 2 && D == 128) {
    if (min(nc, win_chunks + 4) <= SM2_LIST) {  // the fast kernel's tile list holds the window
      const hipError_t e = set_lds_limit((const void*)k_softmax_v2<To>, SM2_LDS);
      if (e != hipSuccess) return e;
      const int64_t grid = (int64_t)B * H * ((nc + 3) / 4);
      hipLaunchKernelGGL(k_softmax_v2<To>, dim3((unsigned)grid), dim3(512), SM2_LDS, st, (const bf16*)q,
                         (const bf16*)k, (const bf16*)v, (const int32_t*)nullptr, (const int32_t*)nullptr, o, lse, H,
                         L, 1, scale * LOG2E, (const bf16*)nullptr, (const bf16*)nullptr, (const int32_t*)nullptr, 0,
                         (const float*)nullptr, (int64_t)0, (float*)nullptr, win_chunks);
      return hipGetLastError();
    }
  }
  const hipError_t ea = set_lds_limit((const void*)k_softmax_masked<T, To, D>, C::LDS_BYTES);
  if (ea != hipSuccess) return ea;
  const int64_t grid = (int64_t)B * H * ((nc + 1) / 2);
  hipLaunchKernelGGL((k_softmax_masked<T, To, D>), dim3((unsigned)grid), dim3(256), C::LDS_BYTES, st, q, k, v,
                     (const int32_t*)nullptr, (const int32_t*)nullptr, o, lse, H, L, 1, scale * LOG2E,
                     (const T*)nullptr, (const T*)nullptr, (const int32_t*)nullptr, 0, win_chunks);
  return hipGetLastError();
}
#define INSTW(T, To, D)                                                                                \
  template hipError_t launch_softmax_window<T, To, D>(const T*, const T*, const T*, To*, float*, int, int, \
                                                      int, int, float, hipStream_t);
INSTW(float, float, 64)
INSTW(float, float, 128)
INSTW(bf16, float, 64)
INSTW(bf16, float, 128)
INSTW(float, bf16, 64)
INSTW(float, bf16, 128)
INSTW(bf16, bf16, 64)
INSTW(bf16, bf16, 128)
#undef INSTW

#define INST(T, To, D)                                                                         \
  template hipError_t launch_softmax_masked<T, To, D>(const T*, const T*, const T*,            \
                                                      const int32_t*, const int32_t*, To*,     \
                                                      float*, int, int, int, int, float,       \
                                                      hipStream_t, const SmPrefix&, const SmMix&);
INST(float, float, 64)
INST(float, float, 128)
INST(float, bf16, 64)
INST(float, bf16, 128)
INST(bf16, float, 64)
INST(bf16, float, 128)
INST(bf16, bf16, 64)
INST(bf16, bf16, 128)
#undef INST


// ---------------------------------------------------------------------------
// Gradient of the softmax branch.  The pages define the forward only; this is
// its exact derivative.  With p = exp(scale s - lse) over the visible keys
// (lse from the forward pass), upstream gradient dO and delta = rowsum(dO * O):
//   dP = dO V^T,   dS = P * (dP - delta),
//   dQ = scale dS K,   dK = scale dS^T Q,   dV = P^T dO.
// Three launches: delta per query; dQ with one workgroup per query chunk (4
// waves x 16 queries) walking that chunk's visible key tiles (the forward's
// tile list); dK and dV with one workgroup per key chunk (4 waves x 16 keys)
// walking the query chunks that see it (every later chunk if the chunk is
// softmax-routed, else only its own).  Products contracting over d take K, V,
// Q, dO with 8 contiguous d per lane (row layout); products contracting over
// tokens take the accumulator-shaped B operand (P^T or dS^T straight from the
// accumulators) and the other operand in the key-group layout, as in the
// forward's O^T = V^T P^T.  Gradients are written in fp32.

// delta = rowsum(dO * O): D / 8 lanes per token, each with 8 contiguous
// values of both rows (one 16-byte bf16 load each), summed across the lane
// group in registers (DPP), so a wave reads whole rows contiguously
template <typename To, int D>
__global__ void __launch_bounds__(256) k_sm_bwd_delta(const To* __restrict__ o, const To* __restrict__ d_o,
                                                      float* __restrict__ delta, int64_t ntok) {
  constexpr int LPT = D / 8;  // lanes per token (8 or 16)
  const int tid = tid_x();
  const int64_t t = (int64_t)bid_x() * (256 / LPT) + tid / LPT;
  const int c = (tid % LPT) * 8;
  const bool in = t < ntok;
  const int64_t tt = in ? t : ntok - 1;  // in-bounds row for the group's shuffle partners
  float a[8], b[8];
  load8f<To>(o + tt * D + c, a);
  load8f<To>(d_o + tt * D + c, b);
  float acc = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) acc = fmaf(a[j], b[j], acc);
  acc = dpp_group_sum<LPT>(acc);
  if (in && (tid % LPT) == 0) delta[t] = acc;
}

// One 64-token tile loaded once and written to LDS in both layouts: thread t
// takes 4 consecutive tokens 4 (t / (D/8)) .. +3 of the 8 columns
// 8 (t % (D/8)) .. +7 (threads past the 64 tokens idle), writes them as rows
// (pitch KP) and, if kg is given, as one key group (4 tokens of each column
// contiguous).
template <typename T, int D>
struct Stage4 {
  Frag<T> f[4];
};
template <typename T, int D>
__device__ __forceinline__ void stage_load(Stage4<T, D>& st, const T* src) {
  const int t = tid_x(), rg = t / (D / 8), cc = t % (D / 8);
  if (4 * rg < CHUNK)
#pragma unroll
    for (int i = 0; i < 4; ++i) st.f[i] = load8<T>(src + (int64_t)(4 * rg + i) * D + 8 * cc);
}
template <typename T, int D>
__device__ __forceinline__ void stage_store(const Stage4<T, D>& st, T* rows, T* kg) {
  using C = SmCfg<T, D>;
  const int t = tid_x(), rg = t / (D / 8), cc = t % (D / 8);
  if (4 * rg >= CHUNK) return;
#pragma unroll
  for (int i = 0; i < 4; ++i) store8<T>(rows + (4 * rg + i) * C::KP + 8 * cc, st.f[i]);
  if (!kg) return;
  if constexpr (sizeof(T) == 2) {
    uint32_t w[4][4];
#pragma unroll
    for (int tk = 0; tk < 4; ++tk) {
      const uint4 u = __builtin_bit_cast(uint4, st.f[tk].v);
      w[tk][0] = u.x; w[tk][1] = u.y; w[tk][2] = u.z; w[tk][3] = u.w;
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const uint2 lo = {__builtin_amdgcn_perm(w[1][m], w[0][m], 0x05040100u),
                        __builtin_amdgcn_perm(w[3][m], w[2][m], 0x05040100u)};
      const uint2 hi = {__builtin_amdgcn_perm(w[1][m], w[0][m], 0x07060302u),
                        __builtin_amdgcn_perm(w[3][m], w[2][m], 0x07060302u)};
      *reinterpret_cast<uint2*>(kg + kg_index<C::VRL>(rg, 8 * cc + 2 * m)) = lo;
      *reinterpret_cast<uint2*>(kg + kg_index<C::VRL>(rg, 8 * cc + 2 * m + 1)) = hi;
    }
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      store_col4<T>(kg + kg_index<C::VRL>(rg, 8 * cc + j), frag_get<T>(st.f[0], j), frag_get<T>(st.f[1], j),
                    frag_get<T>(st.f[2], j), frag_get<T>(st.f[3], j));
  }
}

template <typename T, int D>
__global__ void __launch_bounds__(256, sizeof(T) == 2 ? 2 : 1) k_sm_bwd_dq(const T* __restrict__ q, const T* __restrict__ k,
                                                   const T* __restrict__ v, const T* __restrict__ d_o,
                                                   const int32_t* __restrict__ sel_idx,
                                                   const int32_t* __restrict__ nsel_before,
                                                   const float* __restrict__ lse, const float* __restrict__ delta,
                                                   float* __restrict__ dq, int H, int L, int G, float scale) {
  using C = SmCfg<T, D>;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  T* kbuf = reinterpret_cast<T*>(smem_raw);  // K rows, K key groups
  T* vbuf = kbuf + C::BUF;                   // V rows (its key-group part unused)
  const int nc = L / CHUNK;
  const int BH = (int)(grid_dim_x() / nc);
  const int p = bid_x();
  const int qc = nc - 1 - p / BH;  // later query chunks see more keys: first
  const int bh = p % BH;
  const int b = bh / H, h = bh % H;
  const int grp = (G == 1) ? 0 : h;
  const int32_t* sel = sel_idx + ((int64_t)b * G + grp) * nc;
  const int nsb = nsel_before[((int64_t)b * G + grp) * (nc + 1) + qc];
  const int lane = lane_id(), w = wave_id();
  const int g = lane >> 4, c = lane & 15;
  const int64_t head_off = (int64_t)bh * L * D;
  const int64_t tok = (int64_t)qc * CHUNK + 16 * w + c;
  Frag<T> qf[C::KF], df[C::KF];
#pragma unroll
  for (int ks = 0; ks < C::KF; ++ks) {
    qf[ks] = load8<T>(q + head_off + tok * D + 32 * ks + 8 * g);
    df[ks] = load8<T>(d_o + head_off + tok * D + 32 * ks + 8 * g);
  }
  const float lse2 = lse[(int64_t)bh * L + tok] * LOG2E;
  const float dlt = delta[(int64_t)bh * L + tok];
  const float scale_log2 = scale * LOG2E;
  const int qrow = 16 * w + c;
  f32x4 acc[D / 16];
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  // the next tile's global loads are issued before this tile's products
  Stage4<T, D> rk, rv;
  auto gload = [&](int it) {
    const int kc = it < nsb ? sel[it] : qc;
    stage_load<T, D>(rk, k + head_off + (int64_t)kc * CHUNK * D);
    stage_load<T, D>(rv, v + head_off + (int64_t)kc * CHUNK * D);
  };
  gload(0);
  for (int it = 0; it <= nsb; ++it) {
    const bool diag = it == nsb;
    __syncthreads();  // the previous tile's reads are done
    stage_store<T, D>(rk, kbuf, kbuf + C::KTILE);
    stage_store<T, D>(rv, vbuf, nullptr);
    __syncthreads();
    if (it < nsb) gload(it + 1);
    // S^T and dP^T for 64 keys x this wave's 16 queries
    f32x4 s[4], dp[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) s[kt] = dp[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < C::KF; ++ks)
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        mma(s[kt], load8<T>(kbuf + (16 * kt + c) * C::KP + 32 * ks + 8 * g), qf[ks]);
        mma(dp[kt], load8<T>(vbuf + (16 * kt + c) * C::KP + 32 * ks + 8 * g), df[ks]);
      }
    // dS^T = P^T (dP^T - delta), packed as the B operand (keys in accumulator order)
    Frag<T> dsf[2];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool vis = !diag || (16 * kt + 4 * g + i) <= qrow;
        const float pp = vis ? __builtin_amdgcn_exp2f(fmaf(s[kt][i], scale_log2, -lse2)) : 0.f;
        frag_set(dsf[kt >> 1], 4 * (kt & 1) + i, pp * (dp[kt][i] - dlt));
      }
    // dQ^T += K^T dS^T
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
        const T* kg = kbuf + C::KTILE;
        const Frag<T> a = ld4x2<T>(kg + kg_index<C::VRL>(8 * k2 + g, 16 * dt + c),
                                     kg + kg_index<C::VRL>(8 * k2 + 4 + g, 16 * dt + c));
        mma(acc[dt], a, dsf[k2]);
      }
  }
  float* out = dq + head_off + tok * D;
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) {
    f32x4 r = acc[dt] * scale;
    *reinterpret_cast<f32x4*>(out + 16 * dt + 4 * g) = r;
  }
}

template <typename T, int D>
__global__ void __launch_bounds__(256, sizeof(T) == 2 ? 2 : 1) k_sm_bwd_dkdv(const T* __restrict__ q, const T* __restrict__ k,
                                                     const T* __restrict__ v, const T* __restrict__ d_o,
                                                     const int32_t* __restrict__ nsel_before,
                                                     const float* __restrict__ lse, const float* __restrict__ delta,
                                                     float* __restrict__ dk, float* __restrict__ dv, int H, int L,
                                                     int G, float scale, float* __restrict__ dgate) {
  // dgate (nullable) [B, H, Nc]: the derivative with respect to the chunk's
  // softmax gate (its keys weighted by the gate for the queries of later
  // chunks): the sum of dS = p (dP - delta) over every later query chunk, with
  // p = exp(scale q.k - lse) whether or not the key chunk is softmax-routed;
  // a linear-routed key chunk then visits the later query chunks for that sum
  // only (its keys receive no dK / dV from them)
  using C = SmCfg<T, D>;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  T* qbuf = reinterpret_cast<T*>(smem_raw);  // Q rows, dO key groups
  T* dbuf = qbuf + C::BUF;                   // dO rows, Q key groups
  float* lse_s = reinterpret_cast<float*>(dbuf + C::BUF);
  float* dlt_s = lse_s + CHUNK;
  const int nc = L / CHUNK;
  const int BH = (int)(grid_dim_x() / nc);
  const int p = bid_x();
  const int kc = p / BH;  // earlier key chunks are seen by more queries: first
  const int bh = p % BH;
  const int b = bh / H, h = bh % H;
  const int grp = (G == 1) ? 0 : h;
  const int32_t* nsbp = nsel_before + ((int64_t)b * G + grp) * (nc + 1);
  const bool kc_sm = nsbp[kc + 1] > nsbp[kc];
  const int qlast = (kc_sm || dgate) ? nc - 1 : kc;
  float gsum = 0.f;  // this lane's share of the gate derivative
  const int lane = lane_id(), w = wave_id();
  const int g = lane >> 4, c = lane & 15;
  const int64_t head_off = (int64_t)bh * L * D;
  const int64_t key = (int64_t)kc * CHUNK + 16 * w + c;
  Frag<T> kf[C::KF], vf[C::KF];
#pragma unroll
  for (int ks = 0; ks < C::KF; ++ks) {
    kf[ks] = load8<T>(k + head_off + key * D + 32 * ks + 8 * g);
    vf[ks] = load8<T>(v + head_off + key * D + 32 * ks + 8 * g);
  }
  const float scale_log2 = scale * LOG2E;
  const int kcol = 16 * w + c;
  f32x4 adk[D / 16], adv[D / 16];
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) adk[dt] = adv[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  // the next query chunk's global loads are issued before this one's products
  Stage4<T, D> ra, rb;
  float lse_r = 0.f, dlt_r = 0.f;
  auto gload = [&](int qcx) {
    stage_load<T, D>(ra, q + head_off + (int64_t)qcx * CHUNK * D);
    stage_load<T, D>(rb, d_o + head_off + (int64_t)qcx * CHUNK * D);
    if (tid_x() < CHUNK) {
      lse_r = lse[(int64_t)bh * L + (int64_t)qcx * CHUNK + tid_x()] * LOG2E;
      dlt_r = delta[(int64_t)bh * L + (int64_t)qcx * CHUNK + tid_x()];
    }
  };
  gload(kc);
  for (int qcx = kc; qcx <= qlast; ++qcx) {
    const bool diag = qcx == kc;
    __syncthreads();  // the previous chunk's reads are done
    stage_store<T, D>(ra, qbuf, dbuf + C::KTILE);  // Q rows; Q key groups next to dO rows
    stage_store<T, D>(rb, dbuf, qbuf + C::KTILE);  // dO rows; dO key groups next to Q rows
    if (tid_x() < CHUNK) {
      lse_s[tid_x()] = lse_r;
      dlt_s[tid_x()] = dlt_r;
    }
    __syncthreads();
    if (qcx < qlast) gload(qcx + 1);
    // S and dP for 64 queries x this wave's 16 keys: rows = queries
    f32x4 pm[4], dsm[4];
#pragma unroll
    for (int qt = 0; qt < 4; ++qt) {
      f32x4 s = {0.f, 0.f, 0.f, 0.f}, dp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < C::KF; ++ks) {
        mma(s, load8<T>(qbuf + (16 * qt + c) * C::KP + 32 * ks + 8 * g), kf[ks]);
        mma(dp, load8<T>(dbuf + (16 * qt + c) * C::KP + 32 * ks + 8 * g), vf[ks]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int qrow = 16 * qt + 4 * g + i;
        const bool vis = !diag || kcol <= qrow;
        const float pp = vis ? __builtin_amdgcn_exp2f(fmaf(s[i], scale_log2, -lse_s[qrow])) : 0.f;
        pm[qt][i] = pp;
        dsm[qt][i] = pp * (dp[i] - dlt_s[qrow]);
        if (!diag) gsum += dsm[qt][i];
      }
    }
    if (!diag && !kc_sm) continue;  // only the gate's sum: these keys are not visible in the forward
    // dV^T += dO^T P and dK^T += Q^T dS, contraction over the 64 queries
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
      Frag<T> pf, dsf;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        frag_set(pf, j, pm[2 * k2][j]);
        frag_set(pf, 4 + j, pm[2 * k2 + 1][j]);
        frag_set(dsf, j, dsm[2 * k2][j]);
        frag_set(dsf, 4 + j, dsm[2 * k2 + 1][j]);
      }
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) {
        const T* dgk = qbuf + C::KTILE;  // dO key groups
        const T* qgk = dbuf + C::KTILE;  // Q key groups
        mma(adv[dt], ld4x2<T>(dgk + kg_index<C::VRL>(8 * k2 + g, 16 * dt + c),
                                dgk + kg_index<C::VRL>(8 * k2 + 4 + g, 16 * dt + c)), pf);
        mma(adk[dt], ld4x2<T>(qgk + kg_index<C::VRL>(8 * k2 + g, 16 * dt + c),
                                qgk + kg_index<C::VRL>(8 * k2 + 4 + g, 16 * dt + c)), dsf);
      }
    }
  }
  float* okr = dk + head_off + key * D;
  float* ovr = dv + head_off + key * D;
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) {
    f32x4 r = adk[dt] * scale;
    *reinterpret_cast<f32x4*>(okr + 16 * dt + 4 * g) = r;
    *reinterpret_cast<f32x4*>(ovr + 16 * dt + 4 * g) = adv[dt];
  }
  if (dgate) {  // the wave sums, then the 4 waves in order (deterministic)
    gsum = wave_sum64(gsum);
    __syncthreads();  // lse_s is free again
    if (lane == 0) lse_s[w] = gsum;
    __syncthreads();
    if (tid_x() == 0) dgate[(int64_t)bh * nc + kc] = (lse_s[0] + lse_s[1]) + (lse_s[2] + lse_s[3]);
  }
}

// bf16, D = 128: dQ on the forward kernel's layout.  8 waves own 4 query
// chunks (waves 2m, 2m + 1: 32 queries each of chunk c0 + m); the key tiles
// (the softmax chunks before the block, then its own chunks) stream through
// the 4-stage direct-to-LDS ring three tiles ahead; blocks run longest-first
// and XCD-aware.  K rows carry the V swizzle (row reads for S^T = K Q^T,
// transposed reads for dQ^T += K^T dS^T), V rows the K swizzle (row reads for
// dP^T = V dO^T).  The tile list sits in LDS so that its reads stay out of
// the vector-memory counter (up to SM2_LIST tiles).  (This layout replaced
// one workgroup of 4 waves per query chunk, 16 queries per wave and a 2-stage
// ring: same tiles in the same order per query, bit-identical, 17% faster.)
__global__ void __launch_bounds__(512, 1)
    k_sm_bwd_dq2(const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
                 const bf16* __restrict__ d_o, const int32_t* __restrict__ sel_idx,
                 const int32_t* __restrict__ nsel_before, const float* __restrict__ lse,
                 const float* __restrict__ delta, float* __restrict__ dq, int H, int L, int G, float scale) {
  constexpr int D = 128;
  extern __shared__ __align__(16) unsigned char lds[];
  int32_t* sel_l = reinterpret_cast<int32_t*>(lds + SM2_STAGES * SM2_TILE_BYTES);
  const int nc = L / CHUNK;
  const int nb = (nc + 3) / 4;
  const int BH = (int)(grid_dim_x() / nb);
  const int p = bid_x();
  int qblk, bh;
  if ((BH & 7) == 0) {
    const int xcd = p & 7, slot = p >> 3, hpx = BH >> 3;
    qblk = nb - 1 - slot / hpx;
    bh = (slot % hpx) * 8 + xcd;
  } else {
    qblk = nb - 1 - p / BH;
    bh = p % BH;
  }
  const int b = bh / H, h = bh % H;
  const int grp = (G == 1) ? 0 : h;
  const int c0 = 4 * qblk;
  const int nown = min(4, nc - c0);
  const int32_t* sel = sel_idx + ((int64_t)b * G + grp) * nc;
  const int32_t* nsbp = nsel_before + ((int64_t)b * G + grp) * (nc + 1);
  const int nsb = nsbp[c0];
  const int ntiles = nsb + nown;
  int sm_bits = 0;
  for (int j = 0; j < nown; ++j) sm_bits |= (nsbp[c0 + j + 1] > nsbp[c0 + j]) ? (1 << j) : 0;

  const int lane = lane_id(), w = wave_id();
  const int g = lane >> 4, c = lane & 15;
  const int mch = w >> 1;  // chunk of this wave within the block
  const bool active = mch < nown;
  const int64_t head_off = (int64_t)bh * L * D;
  const bf16* kh = k + head_off;
  const bf16* vh = v + head_off;
  for (int i = tid_x(); i < nsb; i += 512) sel_l[i] = sel[i];
  for (int i = tid_x(); i < nown; i += 512) sel_l[nsb + i] = c0 + i;

  Frag<bf16> qf[2][4], df[2][4];
  float lse2[2], dlt[2];
  const int qtok0 = (c0 + (active ? mch : 0)) * CHUNK + 32 * (w & 1);
#pragma unroll
  for (int qs = 0; qs < 2; ++qs) {
    const int64_t tok = qtok0 + 16 * qs + c;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      qf[qs][ks] = load8<bf16>(q + head_off + tok * D + 32 * ks + 8 * g);
      df[qs][ks] = load8<bf16>(d_o + head_off + tok * D + 32 * ks + 8 * g);
    }
    lse2[qs] = lse[(int64_t)bh * L + tok] * LOG2E;
    dlt[qs] = delta[(int64_t)bh * L + tok];
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): nothing of ours outstanding before the ring starts
  __syncthreads();

  // tile `it` -> stage it % STAGES: 2 K + 2 V 16-byte loads per thread
  auto issue = [&](int it) {
    const int kc = sel_l[it];
    unsigned char* st = lds + (it % SM2_STAGES) * SM2_TILE_BYTES;
    const bf16* kg = kh + (int64_t)kc * CHUNK * D;
    const bf16* vg = vh + (int64_t)kc * CHUNK * D;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int e0 = w * 128 + i * 64;  // first 16-byte chunk of this wave instruction
      const int e = e0 + lane, r = e >> 4, sl = e & 15;
      gload_lds16(kg + r * D + sm2_vslot(r, sl) * 8, st + e0 * 16);
      gload_lds16(vg + r * D + sm2_kslot(r, sl) * 8, st + CHUNK * D * 2 + e0 * 16);
    }
  };
  const float scale_log2 = scale * LOG2E;
  const int qrow_base = 32 * (w & 1);
  f32x4 acc[D / 16][2];
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
    for (int qs = 0; qs < 2; ++qs) acc[dt][qs] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < SM2_STAGES - 1; ++j)
    if (j < ntiles) issue(j);
  for (int it = 0; it < ntiles; ++it) {
    wait_vm(4 * (min(it + SM2_STAGES - 2, ntiles - 1) - it));  // this tile's loads have landed
    lds_barrier();                                              // ... for every wave
    if (it + SM2_STAGES - 1 < ntiles) issue(it + SM2_STAGES - 1);  // into the stage read last iteration
    int mode;
    if (it < nsb) {
      mode = MODE_FULL;
    } else {
      const int j = it - nsb;
      mode = (j == mch) ? MODE_DIAG : (j < mch && ((sm_bits >> j) & 1)) ? MODE_FULL : MODE_SKIP;
    }
    if (!active) mode = MODE_SKIP;
    if (mode == MODE_SKIP) continue;

    const unsigned char* st = lds + (it % SM2_STAGES) * SM2_TILE_BYTES;
    const unsigned char* ks_l = st;
    const unsigned char* vs_l = st + CHUNK * D * 2;
    f32x4 s_[4][2], dp[4][2];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int qs = 0; qs < 2; ++qs) s_[kt][qs] = f32x4{0.f, 0.f, 0.f, 0.f};
    // S^T = K Q^T, the K fragments in two halves of the contraction
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      Frag<bf16> ka[2][4];
#pragma unroll
      for (int k = 0; k < 2; ++k)
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
          const int r = 16 * kt + c, ks = 2 * hf + k;
          ka[k][kt] = *reinterpret_cast<const Frag<bf16>*>(ks_l + r * 256 + sm2_vslot(r, 4 * ks + g) * 16);
        }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int k = 0; k < 2; ++k)
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int qs = 0; qs < 2; ++qs) mma(s_[kt][qs], ka[k][kt], qf[qs][2 * hf + k]);
    }
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int qs = 0; qs < 2; ++qs) dp[kt][qs] = f32x4{0.f, 0.f, 0.f, 0.f};
    // dP^T = V dO^T, the V fragments in two halves of the contraction
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      Frag<bf16> va[2][4];
#pragma unroll
      for (int k = 0; k < 2; ++k)
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
          const int r = 16 * kt + c, ks = 2 * hf + k;
          va[k][kt] = *reinterpret_cast<const Frag<bf16>*>(vs_l + r * 256 + sm2_kslot(r, 4 * ks + g) * 16);
        }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int k = 0; k < 2; ++k)
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int qs = 0; qs < 2; ++qs) mma(dp[kt][qs], va[k][kt], df[qs][2 * hf + k]);
    }
    // dS^T = P^T (dP^T - delta), packed as the B operand (keys in accumulator order)
    Frag<bf16> dsf[2][2];
#pragma unroll
    for (int qs = 0; qs < 2; ++qs)
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bool vis = mode != MODE_DIAG || (16 * kt + 4 * g + i) <= qrow_base + 16 * qs + c;
          const float pp = vis ? __builtin_amdgcn_exp2f(fmaf(s_[kt][qs][i], scale_log2, -lse2[qs])) : 0.f;
          frag_set(dsf[qs][kt >> 1], 4 * (kt & 1) + i, pp * (dp[kt][qs][i] - dlt[qs]));
        }
    // dQ^T += K^T dS^T: K^T fragments by transposed reads (rows d = 16 dt + c,
    // keys 32 k2 + 4g + j and 32 k2 + 16 + 4g + j)
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
      const int r0 = 32 * k2 + 4 * g + (c >> 2), r1 = r0 + 16;
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) {
        const int colq = (16 * dt + 4 * (c & 3)) >> 3;
        const int half = (c & 1) * 8;
        const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) v4i16*)(ks_l + r0 * 256 + sm2_vslot(r0, colq) * 16 + half));
        const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) v4i16*)(ks_l + r1 * 256 + sm2_vslot(r1, colq) * 16 + half));
        Frag<bf16> a;
        a.v = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int qs = 0; qs < 2; ++qs) mma(acc[dt][qs], a, dsf[qs][k2]);
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // no load may still be in flight into LDS at the end
  if (!active) return;
#pragma unroll
  for (int qs = 0; qs < 2; ++qs) {
    float* out = dq + head_off + (int64_t)(qtok0 + 16 * qs + c) * D;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      f32x4 r = acc[dt][qs] * scale;
      *reinterpret_cast<f32x4*>(out + 16 * dt + 4 * g) = r;
    }
  }
}

// bf16, D = 128: dK and dV with one workgroup of 2 waves per key chunk, 32
// keys per wave (two 16-key sub-tiles, so every Q or dO fragment read from
// LDS feeds two products; one wave per SIMD with 512 registers, two
// workgroups per CU), the query chunks' Q and dO streamed straight from
// global memory into a 2-stage LDS ring (global_load_lds_dwordx4, one tile
// ahead), rows stored with the forward's V swizzle (chunk q of row r at slot
// q ^ ((r & 7) << 1)): row reads give the A operands of S = Q K^T and
// dP = dO V^T, transposed reads (ds_read_b64_tr_b16) the A operands of
// dV^T += dO^T P and dK^T += Q^T dS.  One barrier per query chunk, no
// register staging; lse and delta of the chunk ride in the same ring.
// (4 waves of 16 keys each, two per SIMD, read twice the LDS per product and
// were 3% slower for the whole gradient; the per-key arithmetic is the same.)
constexpr int DK2_STAGES = 2;
constexpr int DK2_TILE = 2 * CHUNK * 128 * 2 + 1024;  // Q, dO rows; lse, delta (+ two spare slots)
constexpr int DK2_LDS = DK2_STAGES * DK2_TILE + 16;
__global__ void __launch_bounds__(128, 1)
    k_sm_bwd_dkdv2(const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
                   const bf16* __restrict__ d_o, const int32_t* __restrict__ nsel_before,
                   const float* __restrict__ lse, const float* __restrict__ delta, float* __restrict__ dk,
                   float* __restrict__ dv, int H, int L, int G, float scale, float* __restrict__ dgate) {
  constexpr int D = 128;
  extern __shared__ __align__(16) unsigned char lds[];
  float* red = reinterpret_cast<float*>(lds + DK2_STAGES * DK2_TILE);
  const int nc = L / CHUNK;
  const int BH = (int)(grid_dim_x() / nc);
  const int p = bid_x();
  const int kc = p / BH;  // earlier key chunks are seen by more queries: first
  const int bh = p % BH;
  const int b = bh / H, h = bh % H;
  const int grp = (G == 1) ? 0 : h;
  const int32_t* nsbp = nsel_before + ((int64_t)b * G + grp) * (nc + 1);
  const bool kc_sm = nsbp[kc + 1] > nsbp[kc];
  const int qlast = (kc_sm || dgate) ? nc - 1 : kc;
  const int ntl = qlast - kc + 1;
  float gsum = 0.f;
  const int lane = lane_id(), w = wave_id();
  const int g = lane >> 4, c = lane & 15;
  const int64_t head_off = (int64_t)bh * L * D;
  // wave w owns keys 32 w .. 32 w + 31 of the chunk, as two 16-key sub-tiles kq
  Frag<bf16> kf[2][4], vf[2][4];
#pragma unroll
  for (int kq = 0; kq < 2; ++kq)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int64_t key = (int64_t)kc * CHUNK + 32 * w + 16 * kq + c;
      kf[kq][ks] = load8<bf16>(k + head_off + key * D + 32 * ks + 8 * g);
      vf[kq][ks] = load8<bf16>(v + head_off + key * D + 32 * ks + 8 * g);
    }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): nothing of ours outstanding before the ring starts
  const float scale_log2 = scale * LOG2E;
  f32x4 adk[2][D / 16], adv[2][D / 16];
#pragma unroll
  for (int kq = 0; kq < 2; ++kq)
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) adk[kq][dt] = adv[kq][dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // tile j (query chunk kc + j) -> stage j % DK2_STAGES: per wave 8 + 8
  // row-block loads and one 256-byte vector load (wave 0: lse, wave 1: delta)
  auto issue = [&](int j) {
    const int qcx = kc + j;
    unsigned char* st = lds + (j % DK2_STAGES) * DK2_TILE;
    const bf16* qg = q + head_off + (int64_t)qcx * CHUNK * D;
    const bf16* dg = d_o + head_off + (int64_t)qcx * CHUNK * D;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int e0 = w * 512 + i * 64;
      const int e = e0 + lane, r = e >> 4, sl = e & 15;
      gload_lds16(qg + r * D + sm2_vslot(r, sl) * 8, st + e0 * 16);
      gload_lds16(dg + r * D + sm2_vslot(r, sl) * 8, st + CHUNK * D * 2 + e0 * 16);
    }
    const float* src = ((w & 1) ? delta : lse) + (int64_t)bh * L + (int64_t)qcx * CHUNK + 4 * (lane & 15);
    if (lane < 16) gload_lds16(src, st + 2 * CHUNK * D * 2 + w * 256);
  };
  __syncthreads();
  issue(0);
  for (int j = 0; j < ntl; ++j) {
    const int qcx = kc + j;
    const bool diag = qcx == kc;
    __builtin_amdgcn_s_waitcnt(0x0F70);  // this tile's loads have landed (vmcnt(0))
    lds_barrier();                       // ... for every wave; every wave is done with tile j - 1
    if (j + 1 < ntl) issue(j + 1);       // into the stage tile j - 1 used
    const unsigned char* st = lds + opaque_sgpr((j % DK2_STAGES) * DK2_TILE);
    const unsigned char* qs_l = st;
    const unsigned char* ds_l = st + CHUNK * D * 2;
    const float* lse_s = reinterpret_cast<const float*>(st + 2 * CHUNK * D * 2);
    const float* dlt_s = lse_s + CHUNK;
    f32x4 pm[2][4], dsm[2][4];
#pragma unroll
    for (int qt = 0; qt < 4; ++qt) {
      f32x4 s_[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
      f32x4 dp[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
      const int r = 16 * qt + c;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int off = r * 256 + sm2_vslot(r, 4 * ks + g) * 16;
        const Frag<bf16> aq = *reinterpret_cast<const Frag<bf16>*>(qs_l + off);
        const Frag<bf16> ad = *reinterpret_cast<const Frag<bf16>*>(ds_l + off);
#pragma unroll
        for (int kq = 0; kq < 2; ++kq) {
          mma(s_[kq], aq, kf[kq][ks]);
          mma(dp[kq], ad, vf[kq][ks]);
        }
      }
#pragma unroll
      for (int kq = 0; kq < 2; ++kq)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int qrow = 16 * qt + 4 * g + i;
          const bool vis = !diag || 32 * w + 16 * kq + c <= qrow;
          const float pp = vis ? __builtin_amdgcn_exp2f(fmaf(s_[kq][i], scale_log2, -lse_s[qrow] * LOG2E)) : 0.f;
          pm[kq][qt][i] = pp;
          dsm[kq][qt][i] = pp * (dp[kq][i] - dlt_s[qrow]);
          if (!diag) gsum += dsm[kq][qt][i];
        }
    }
    if (!diag && !kc_sm) continue;  // only the gate's sum: these keys are not visible in the forward
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
      Frag<bf16> pf[2], dsf[2];
#pragma unroll
      for (int kq = 0; kq < 2; ++kq)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          frag_set(pf[kq], jj, pm[kq][2 * k2][jj]);
          frag_set(pf[kq], 4 + jj, pm[kq][2 * k2 + 1][jj]);
          frag_set(dsf[kq], jj, dsm[kq][2 * k2][jj]);
          frag_set(dsf[kq], 4 + jj, dsm[kq][2 * k2 + 1][jj]);
        }
      // dO^T and Q^T fragments (rows d = 16 dt + c, queries 32 k2 + 4g + j
      // and 32 k2 + 16 + 4g + j) by transposed reads: lane c of group g reads
      // row 32 k2 + 4g + c / 4 (+16), columns 16 dt + 4 (c % 4) .. +3
      const int r0 = 32 * k2 + 4 * g + (c >> 2), r1 = r0 + 16;
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) {
        const int colq = (16 * dt + 4 * (c & 3)) >> 3;
        const int half = (c & 1) * 8;
        const int o0 = r0 * 256 + sm2_vslot(r0, colq) * 16 + half, o1 = r1 * 256 + sm2_vslot(r1, colq) * 16 + half;
        Frag<bf16> ad, aq;
        {
          const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)(ds_l + o0));
          const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)(ds_l + o1));
          ad.v = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
        {
          const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)(qs_l + o0));
          const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)(qs_l + o1));
          aq.v = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
#pragma unroll
        for (int kq = 0; kq < 2; ++kq) {
          mma(adv[kq][dt], ad, pf[kq]);
          mma(adk[kq][dt], aq, dsf[kq]);
        }
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // no load may still be in flight into LDS at the end
#pragma unroll
  for (int kq = 0; kq < 2; ++kq) {
    const int64_t key = (int64_t)kc * CHUNK + 32 * w + 16 * kq + c;
    float* okr = dk + head_off + key * D;
    float* ovr = dv + head_off + key * D;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      f32x4 r = adk[kq][dt] * scale;
      *reinterpret_cast<f32x4*>(okr + 16 * dt + 4 * g) = r;
      *reinterpret_cast<f32x4*>(ovr + 16 * dt + 4 * g) = adv[kq][dt];
    }
  }
  if (dgate) {  // the wave sums, then the 2 waves in order (deterministic)
    gsum = wave_sum64(gsum);
    if (lane == 0) red[w] = gsum;
    __syncthreads();
    if (tid_x() == 0) dgate[(int64_t)bh * nc + kc] = red[0] + red[1];
  }
}

size_t sm_bwd_ws_bytes(int B, int H, int L) { return (size_t)B * H * L * sizeof(float); }

template <typename T, typename To, int D>
hipError_t launch_softmax_backward(const T* q, const T* k, const T* v, const int32_t* sel_idx,
                                   const int32_t* nsel_before, const To* o, const float* lse, const T* d_o,
                                   float* dq, float* dk, float* dv, float* dgate, void* ws, int B, int H, int L,
                                   int G, float scale, hipStream_t st) {
  using C = SmCfg<T, D>;
  // the delta pass reads dO in the output dtype: only io == output dtype here
  static_assert(sizeof(To) > 0, "");
  float* delta = static_cast<float*>(ws);
  const int64_t ntok = (int64_t)B * H * L;
  const int nc = L / CHUNK;
  constexpr int LDS_DQ = 2 * C::BUF * (int)sizeof(T);
  constexpr int LDS_DKDV = 2 * C::BUF * (int)sizeof(T) + 2 * CHUNK * 4;
  hipError_t e = set_lds_limit((const void*)k_sm_bwd_dq<T, D>, LDS_DQ);
  if (e == hipSuccess) e = set_lds_limit((const void*)k_sm_bwd_dkdv<T, D>, LDS_DKDV);
  if (e != hipSuccess) return e;
  constexpr int TPB = 256 / (D / 8);  // tokens per block
  hipLaunchKernelGGL((k_sm_bwd_delta<To, D>), dim3((unsigned)((ntok + TPB - 1) / TPB)), dim3(256), 0, st, o,
                     (const To*)d_o, delta, ntok);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t grid = (int64_t)B * H * nc;
  if (sizeof(T) == 2 && D == 128 && nc <= SM2_LIST) {
    if ((e = set_lds_limit((const void*)k_sm_bwd_dq2, SM2_LDS)) != hipSuccess) return e;
    hipLaunchKernelGGL(k_sm_bwd_dq2, dim3((unsigned)((int64_t)B * H * ((nc + 3) / 4))), dim3(512), SM2_LDS, st,
                       (const bf16*)q, (const bf16*)k, (const bf16*)v, (const bf16*)d_o, sel_idx, nsel_before, lse,
                       delta, dq, H, L, G, scale);
  } else {
    hipLaunchKernelGGL((k_sm_bwd_dq<T, D>), dim3((unsigned)grid), dim3(256), LDS_DQ, st, q, k, v, d_o, sel_idx,
                       nsel_before, lse, delta, dq, H, L, G, scale);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if constexpr (sizeof(T) == 2 && D == 128) {
    if ((e = set_lds_limit((const void*)k_sm_bwd_dkdv2, DK2_LDS)) != hipSuccess) return e;
    hipLaunchKernelGGL(k_sm_bwd_dkdv2, dim3((unsigned)grid), dim3(128), DK2_LDS, st, (const bf16*)q, (const bf16*)k,
                       (const bf16*)v, (const bf16*)d_o, nsel_before, lse, delta, dk, dv, H, L, G, scale, dgate);
  } else {
    hipLaunchKernelGGL((k_sm_bwd_dkdv<T, D>), dim3((unsigned)grid), dim3(256), LDS_DKDV, st, q, k, v, d_o,
                       nsel_before, lse, delta, dk, dv, H, L, G, scale, dgate);
  }
  return hipGetLastError();
}

#define INSTB(T, D)                                                                                    \
  template hipError_t launch_softmax_backward<T, T, D>(const T*, const T*, const T*, const int32_t*,  \
                                                       const int32_t*, const T*, const float*, const T*, \
                                                       float*, float*, float*, float*, void*, int, int, int, int, \
                                                       float, hipStream_t);
INSTB(float, 64)
INSTB(float, 128)
INSTB(bf16, 64)
INSTB(bf16, 128)
#undef INSTB

}  // namespace natsl
