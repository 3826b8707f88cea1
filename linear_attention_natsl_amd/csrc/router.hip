// Router and compaction.
//
// Router: "Technische Samenvatting: Neural Attention Search Linear (NAtS-L)",
// Kernmechanismen 1 -- every 64-token chunk is mean-pooled and scored by a
// linear layer, one score per operation; the higher score picks the chunk's
// operation (ties: softmax, the first maximum).
// Compaction: Kernmechanismen 3 -- only the softmax-routed chunks' KV is kept
// for the softmax operation; in prefill that is an ordered index list.
//
// The router is bandwidth-bound: one pass over x.  One workgroup per (b, c)
// streams the chunk's 64 x d values with 16-byte loads (each thread owns 8
// columns), sums in fp32 in a fixed order, stores the mean in LDS, and the
// four waves form the 2G dot products with W_score (fixed-order wave
// reductions), so the result is deterministic.
//
// Router gradient (straight-through; the pages leave the argmax's derivative
// open): one pass over x that also writes dx (the chunk's score gradient
// broadcast over its rows, fp32), then dW and db as fixed-order sums over
// chunks.  Bandwidth-bound: 2 + 4 bytes per element of x (bf16 io).
#include "common.hpp"
#include "kernels.hpp"

namespace natsl {

template <typename T>
__global__ void __launch_bounds__(256) k_route(const T* __restrict__ x, const float* __restrict__ w,
                                               const float* __restrict__ bsc, int L, int d, int G,
                                               int nc, int32_t* __restrict__ route_out,
                                               float* __restrict__ scores) {
  extern __shared__ float s_mean[];  // [d]
  const unsigned bid = (unsigned)bid_x();  // one-dimensional grid: chunk fastest
  const int c = (int)(bid % (unsigned)nc), b = (int)(bid / (unsigned)nc);
  const T* xc = x + ((int64_t)b * L + (int64_t)c * CHUNK) * d;
  for (int col0 = tid_x() * 8; col0 < d; col0 += 256 * 8) {
    float acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = 0.f;
#pragma unroll 8
    for (int r = 0; r < CHUNK; ++r) {
      float v[8];
      load8f<T>(xc + (int64_t)r * d + col0, v);
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] += v[j];
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) s_mean[col0 + j] = acc[j] * (1.0f / CHUNK);
  }
  __syncthreads();
  const int lane = lane_id(), wv = wave_id();
  for (int o = wv; o < 2 * G; o += 4) {
    float p = 0.f;
    for (int j = lane; j < d; j += 64) p += s_mean[j] * w[(int64_t)j * 2 * G + o];
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) p = wave_sum_xor(p, m);
    if (bsc) p += bsc[o];
    if (lane == 0) s_mean[d + o] = p;  // scores live after the mean
  }
  __syncthreads();
  for (int gg = tid_x(); gg < G; gg += 256) {
    const float s0 = s_mean[d + 2 * gg], s1 = s_mean[d + 2 * gg + 1];
    const int64_t idx = ((int64_t)b * G + gg) * nc + c;
    route_out[idx] = (s0 >= s1) ? 0 : 1;
    if (scores) {
      scores[idx * 2] = s0;
      scores[idx * 2 + 1] = s1;
    }
  }
}

// Fast path for d_model = 8 * 2^k <= 8192: 1024 threads per chunk.  The d/8
// column groups of 8 contiguous values (16-byte loads) times RS = 8192 / d
// row slices cover the chunk's 64 x d values once; each thread issues all of
// its 64 / RS loads before adding any, so the whole chunk is in flight at
// once.  The RS partial sums of a column are then added in slice order
// through LDS (fixed order: deterministic).
template <typename T>
__global__ void __launch_bounds__(1024, 2) k_route_wide(const T* __restrict__ x, const float* __restrict__ w,
                                                     const float* __restrict__ bsc, int L, int d, int G, int nc,
                                                     int32_t* __restrict__ route_out, float* __restrict__ scores) {
  extern __shared__ float s_part[];  // [RS][d] partial sums, then the mean [d] and 2G scores; W_score [d][2G]
  const unsigned bid = (unsigned)bid_x();  // one-dimensional grid: chunk fastest
  const int c = (int)(bid % (unsigned)nc), b = (int)(bid / (unsigned)nc);
  const int tid = tid_x();
  const int ncg = d >> 3;          // column groups
  const int rs = 1024 / ncg;       // row slices (1 .. 64 ... capped below)
  const int rows = CHUNK / rs;     // rows per thread
  const int cg = tid % ncg, sl = tid / ncg;
  const T* xc = x + ((int64_t)b * L + (int64_t)c * CHUNK + (int64_t)sl * rows) * d + cg * 8;
  // W_score goes to LDS (when it fits, 16 KiB at G = 1): its loads are issued
  // first and stored while the chunk's rows are in flight, so the scores do
  // not wait on one global load per step
  const int nw4 = d * 2 * G / 4;
  float* s_w = s_part + ((rs * d + d + 2 * G + 3) & ~3);
  const bool w_lds = nw4 <= 4 * 1024 && ((uintptr_t)w & 15) == 0;
  f32x4 wreg[4];
  if (w_lds) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int x4 = tid + 1024 * u;
      if (x4 < nw4) wreg[u] = *reinterpret_cast<const f32x4*>(w + 4 * x4);
    }
  }
  float acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.f;
  {
    // batches of 8 independent 16-byte loads (two workgroups per CU keep
    // 16 per column group in flight)
    for (int r = 0; r < rows; r += 8) {
      Frag<T> v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {  // x is read once, here: non-temporal loads (bf16)
        const T* px = xc + (int64_t)min(r + u, rows - 1) * d;
        if constexpr (sizeof(T) == 2)
          v[u].v = __builtin_bit_cast(bf16x8, __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(px)));
        else
          v[u] = load8<T>(px);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (r + u < rows)
#pragma unroll
          for (int j = 0; j < 8; ++j) acc[j] += to_f32(frag_get<T>(v[u], j));
    }
  }
  float* mine = s_part + sl * d + cg * 8;
#pragma unroll
  for (int j = 0; j < 8; ++j) mine[j] = acc[j];
  if (w_lds) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int x4 = tid + 1024 * u;
      if (x4 < nw4) *reinterpret_cast<f32x4*>(s_w + 4 * x4) = wreg[u];
    }
  }
  __syncthreads();
  float* s_mean = s_part + rs * d;
  for (int col = tid; col < d; col += 1024) {
    float t = 0.f;
    for (int k = 0; k < rs; ++k) t += s_part[k * d + col];
    s_mean[col] = t * (1.0f / CHUNK);
  }
  __syncthreads();
  const int lane = lane_id(), wv = wave_id();
  const float* wsrc = w_lds ? s_w : w;
  for (int o = wv; o < 2 * G; o += 16) {
    float p = 0.f;
#pragma unroll 8
    for (int j = lane; j < d; j += 64) p += s_mean[j] * wsrc[(int64_t)j * 2 * G + o];
    p = wave_sum64(p);
    if (bsc) p += bsc[o];
    if (lane == 0) s_mean[d + o] = p;
  }
  __syncthreads();
  for (int gg = tid; gg < G; gg += 1024) {
    const float s0 = s_mean[d + 2 * gg], s1 = s_mean[d + 2 * gg + 1];
    const int64_t idx = ((int64_t)b * G + gg) * nc + c;
    route_out[idx] = (s0 >= s1) ? 0 : 1;
    if (scores) {
      scores[idx * 2] = s0;
      scores[idx * 2 + 1] = s1;
    }
  }
}

// One wave per (b, g): ordered list of softmax chunks and exclusive prefix counts.
__global__ void __launch_bounds__(64) k_compact(const int32_t* __restrict__ route_in,
                                                int32_t* __restrict__ route_out, int nc,
                                                int32_t* __restrict__ sel_idx,
                                                int32_t* __restrict__ nsel_before) {
  const int bg = bid_x();
  const int lane = tid_x();
  const int32_t* r = route_in + (int64_t)bg * nc;
  int32_t* ro = route_out + (int64_t)bg * nc;
  int32_t* sel = sel_idx + (int64_t)bg * nc;
  int32_t* nsb = nsel_before + (int64_t)bg * (nc + 1);
  int base = 0;
  for (int c0 = 0; c0 < nc; c0 += 64) {
    const int c = c0 + lane;
    const int rv = (c < nc) ? r[c] : 1;
    const bool is_sm = (c < nc) && (rv == 0);
    const uint64_t mask = __ballot(is_sm);
    const int before = __popcll(mask & ((1ull << lane) - 1ull));
    if (c < nc) {
      if (ro != r) ro[c] = rv;
      nsb[c] = base + before;
      if (is_sm) sel[base + before] = c;
    }
    base += __popcll(mask);
  }
  for (int c = base + lane; c < nc; c += 64) sel[c] = -1;
  if (lane == 0) nsb[nc] = base;
}

// ---------------------------------------------------------------------------
// Router gradient ("Technische Samenvatting: Neural Attention Search Linear
// (NAtS-L)", Kernmechanismen 5: the selection is learned end to end, with
// gradients for the attention score layer).  Straight-through reading: the
// route of chunk c is a one-hot gate h_c whose derivative with respect to the
// scores is taken to be the Jacobian of softmax(s_c).  From the branches' gate
// derivatives dh (per head, summed over the heads of the route group):
//   ds = pi (dh - pi . dh),  pi = softmax(s_c)
//   dW[:, 2g + o] = sum_{b, c} mean_c(x) ds[b, g, c, o],   db = sum ds,
//   dx_t = W ds_{c(t)} / 64
// Every sum runs in a fixed order: deterministic.

// ds [B, G, Nc, 2], one thread per (b, g, c)
// per (b, c, 2048-column slice): the straight-through step for the chunk's
// score pairs, the chunk mean of x (kept for dW) and dx of the chunk's rows.
// The gate derivatives of a group's heads are summed (dh), and ds = J^T dh
// with J the Jacobian of the two-way softmax of the scores: ds_o = p_o (dh_o -
// p . dh).  Each thread owns 8 columns (d_model is a multiple of 8): 16-byte
// (bf16) or 2 x 16-byte (fp32) loads, eight rows in flight, each column
// summed over the rows in order; dx of a chunk is one row (the mean's
// gradient, d pooled / d x = 1/64) written to all 64 rows.
template <typename T>
__global__ void __launch_bounds__(256) k_route_bwd_x(const T* __restrict__ x, const float* __restrict__ w,
                                                     const float* __restrict__ scores,
                                                     const float* __restrict__ dg_sm,
                                                     const float* __restrict__ dg_lin, int L, int d, int H, int G,
                                                     int nc, float* __restrict__ ds, float* __restrict__ pooled,
                                                     float* __restrict__ dx) {
  extern __shared__ float s_ds[];  // [G][2]
  const unsigned bid = (unsigned)bid_x();  // (chunk, batch) flattened, chunk fastest; z: column block
  const int c = (int)(bid % (unsigned)nc), b = (int)(bid / (unsigned)nc), z = (int)__builtin_amdgcn_workgroup_id_z();
  const int col = (z * 256 + tid_x()) * 8;
  // the gate sums' loads are issued first, the x rows' next; the barrier
  // before dx waits for both
  float dh[2] = {0.f, 0.f};
  const int g_own = tid_x() < G ? tid_x() : -1;
  if (g_own >= 0) {
    const int hpg = H / G;
    for (int h = g_own * hpg; h < (g_own + 1) * hpg; ++h) {
      const int64_t j = ((int64_t)b * H + h) * nc + c;
      dh[0] += dg_sm[j];
      dh[1] += dg_lin[j];
    }
  }
  if (col < d) {
    const T* xc = x + ((int64_t)b * L + (int64_t)c * CHUNK) * d + col;
    float sx[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int r0 = 0; r0 < CHUNK; r0 += 8) {
      Frag<T> raw[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) raw[u] = load8<T>(xc + (int64_t)(r0 + u) * d);
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int j = 0; j < 8; ++j) sx[j] += to_f32(frag_get<T>(raw[u], j));
    }
    float4* pc4 = reinterpret_cast<float4*>(pooled + ((int64_t)b * nc + c) * d + col);
    pc4[0] = make_float4(sx[0] * (1.0f / CHUNK), sx[1] * (1.0f / CHUNK), sx[2] * (1.0f / CHUNK),
                         sx[3] * (1.0f / CHUNK));
    pc4[1] = make_float4(sx[4] * (1.0f / CHUNK), sx[5] * (1.0f / CHUNK), sx[6] * (1.0f / CHUNK),
                         sx[7] * (1.0f / CHUNK));
  }
  // G > 256 groups: the remaining ones in further passes (no x loads beside them)
  for (int g = g_own >= 0 ? g_own : tid_x(); g < G; g += 256) {
    if (g != g_own) {
      dh[0] = dh[1] = 0.f;
      const int hpg = H / G;
      for (int h = g * hpg; h < (g + 1) * hpg; ++h) {
        const int64_t j = ((int64_t)b * H + h) * nc + c;
        dh[0] += dg_sm[j];
        dh[1] += dg_lin[j];
      }
    }
    const int64_t i = ((int64_t)b * G + g) * nc + c;
    const float s0 = scores[i * 2], s1 = scores[i * 2 + 1];
    const float m = fmaxf(s0, s1);
    const float e0 = __expf(s0 - m), e1 = __expf(s1 - m);
    const float p0 = e0 / (e0 + e1), p1 = e1 / (e0 + e1);
    const float pd = p0 * dh[0] + p1 * dh[1];
    const float d0 = p0 * (dh[0] - pd), d1 = p1 * (dh[1] - pd);
    s_ds[2 * g] = d0;
    s_ds[2 * g + 1] = d1;
    if (z == 0) {
      ds[i * 2] = d0;
      ds[i * 2 + 1] = d1;
    }
  }
  __syncthreads();
  if (col >= d || !dx) return;
  float gx[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float* wr = w + (int64_t)(col + j) * 2 * G;
    float a = 0.f;
    for (int g = 0; g < G; ++g) a += wr[2 * g] * s_ds[2 * g] + wr[2 * g + 1] * s_ds[2 * g + 1];
    gx[j] = a * (1.0f / CHUNK);
  }
  const float4 g0 = make_float4(gx[0], gx[1], gx[2], gx[3]), g1 = make_float4(gx[4], gx[5], gx[6], gx[7]);
  float* dxc = dx + ((int64_t)b * L + (int64_t)c * CHUNK) * d + col;
#pragma unroll 8
  for (int r = 0; r < CHUNK; ++r) {
    float4* o = reinterpret_cast<float4*>(dxc + (int64_t)r * d);
    o[0] = g0;
    o[1] = g1;
  }
}

// dW [d, 2G] = sum over (b, c) of pooled[b, c, :] x ds[b, g, c, :]: the
// (b, c) range split into RB_SLICES interleaved slices (grid z), one thread
// per (column, group), each slice's sum in order of (b, c); the slices are
// then added in order by k_route_bwd_w_final, so the result is deterministic.
constexpr int RB_SLICES = 16;
__global__ void __launch_bounds__(256) k_route_bwd_w(const float* __restrict__ pooled, const float* __restrict__ ds,
                                                     int B, int G, int nc, int d, float* __restrict__ part) {
  const int col = bid_x() * 256 + tid_x(), g = bid_y(), s = (int)__builtin_amdgcn_workgroup_id_z();
  if (col >= d) return;
  const int nbc = B * nc;
  float a0 = 0.f, a1 = 0.f;
  int bc = s;
  for (; bc + 7 * RB_SLICES < nbc; bc += 8 * RB_SLICES) {
    float p[8];
    float2 q[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = bc + u * RB_SLICES, bb = i / nc, c = i - bb * nc;
      p[u] = pooled[(int64_t)i * d + col];
      q[u] = *reinterpret_cast<const float2*>(ds + (((int64_t)bb * G + g) * nc + c) * 2);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      a0 += p[u] * q[u].x;
      a1 += p[u] * q[u].y;
    }
  }
  for (; bc < nbc; bc += RB_SLICES) {
    const int bb = bc / nc, c = bc - bb * nc;
    const float p = pooled[(int64_t)bc * d + col];
    a0 += p * ds[(((int64_t)bb * G + g) * nc + c) * 2];
    a1 += p * ds[(((int64_t)bb * G + g) * nc + c) * 2 + 1];
  }
  part[((int64_t)s * 2 * G + 2 * g) * d + col] = a0;
  part[((int64_t)s * 2 * G + 2 * g + 1) * d + col] = a1;
}

// the slices' partial dW added in slice order (blocks below nbw); db [2G] as
// the (b, c) sum of ds, one wave per output: lane-strided sums, then a
// fixed-order wave reduction
__global__ void __launch_bounds__(256) k_route_bwd_w_final(const float* __restrict__ part,
                                                           const float* __restrict__ ds, int B, int G, int nc, int d,
                                                           int nbw, float* __restrict__ dw, float* __restrict__ db) {
  if (bid_x() < nbw) {
    const int64_t i = (int64_t)bid_x() * 256 + tid_x();
    if (i >= (int64_t)d * 2 * G) return;
    const int col = (int)(i / (2 * G)), o = (int)(i % (2 * G));
    float acc = 0.f;
    for (int s = 0; s < RB_SLICES; ++s) acc += part[((int64_t)s * 2 * G + o) * d + col];
    dw[i] = acc;
    return;
  }
  const int o = (bid_x() - nbw) * 4 + wave_id();
  if (o >= 2 * G) return;
  const int g = o / 2, oo = o % 2;
  float acc = 0.f;
  for (int bc = lane_id(); bc < B * nc; bc += 64) {
    const int bb = bc / nc, c = bc - bb * nc;
    acc += ds[(((int64_t)bb * G + g) * nc + c) * 2 + oo];
  }
  acc = wave_sum64(acc);
  if (lane_id() == 0) db[o] = acc;
}

size_t route_bwd_ws_bytes(int B, int G, int L, int d) {
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const size_t nc = (size_t)L / CHUNK;
  return al((size_t)B * G * nc * 2 * 4) + al((size_t)B * nc * d * 4) + al((size_t)RB_SLICES * 2 * G * d * 4);
}

template <typename T>
hipError_t launch_route_backward(const T* x, const float* w, const float* scores, const float* dg_sm,
                                 const float* dg_lin, float* dx, float* dw, float* db, void* wsp, int B, int H, int L,
                                 int d, int G, hipStream_t st) {
  auto al = [](size_t v) { return (v + 255) & ~(size_t)255; };
  const int nc = L / CHUNK;
  float* ds = (float*)wsp;
  float* pooled = (float*)((char*)wsp + al((size_t)B * G * nc * 2 * 4));
  float* part = (float*)((char*)pooled + al((size_t)B * nc * d * 4));
  hipLaunchKernelGGL(k_route_bwd_x<T>, dim3((unsigned)(nc * B), 1, (d + 2047) / 2048), dim3(256), (size_t)G * 2 * sizeof(float), st,
                     x, w, scores, dg_sm, dg_lin, L, d, H, G, nc, ds, pooled, dx);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_route_bwd_w, dim3((d + 255) / 256, G, RB_SLICES), dim3(256), 0, st, pooled, ds, B, G, nc, d,
                     part);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int nbw = (int)(((int64_t)d * 2 * G + 255) / 256);
  const int nbb = db ? (2 * G + 3) / 4 : 0;
  hipLaunchKernelGGL(k_route_bwd_w_final, dim3((unsigned)(nbw + nbb)), dim3(256), 0, st, part, ds, B, G, nc, d, nbw,
                     dw, db);
  return hipGetLastError();
}
template hipError_t launch_route_backward<float>(const float*, const float*, const float*, const float*,
                                                 const float*, float*, float*, float*, void*, int, int, int, int,
                                                 int, hipStream_t);
template hipError_t launch_route_backward<bf16>(const bf16*, const float*, const float*, const float*, const float*,
                                                float*, float*, float*, void*, int, int, int, int, int, hipStream_t);

template <typename T>
hipError_t launch_route(const T* x, const float* w, const float* bsc, int B, int L, int d, int G,
                        int32_t* route_out, float* scores, hipStream_t st) {
  const int nc = L / CHUNK;
  // wide path: d = 8 * 2^k with 64 <= d <= 8192 (1 to 16 row slices of 64 / rs rows)
  const bool pow2 = (d & (d - 1)) == 0;
  if (pow2 && d >= 512 && d <= 8192) {
    const int rs = 8192 / d;
    const size_t nw = (size_t)d * 2 * G;
    const size_t lds = (size_t)(rs * d + d + 2 * G + 3 + (nw <= 4 * 1024 * 4 ? nw : 0)) * sizeof(float);
    if (lds <= (size_t)LDS_MAX_BYTES) {
      const hipError_t e = set_lds_limit((const void*)k_route_wide<T>, (int)lds);
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL(k_route_wide<T>, dim3((unsigned)(nc * B)), dim3(1024), lds, st, x, w, bsc, L, d, G, nc, route_out,
                         scores);
      return hipGetLastError();
    }
  }
  const size_t lds = (size_t)(d + 2 * G) * sizeof(float);
  hipLaunchKernelGGL(k_route<T>, dim3((unsigned)(nc * B)), dim3(256), lds, st, x, w, bsc, L, d, G, nc, route_out,
                     scores);
  return hipGetLastError();
}
template hipError_t launch_route<float>(const float*, const float*, const float*, int, int, int, int,
                                        int32_t*, float*, hipStream_t);
template hipError_t launch_route<bf16>(const bf16*, const float*, const float*, int, int, int, int,
                                       int32_t*, float*, hipStream_t);

hipError_t launch_compact(const int32_t* route_in, int32_t* route_out, int B, int G, int nc,
                          int32_t* sel_idx, int32_t* nsel_before, hipStream_t st) {
  hipLaunchKernelGGL(k_compact, dim3(B * G), dim3(64), 0, st, route_in, route_out, nc, sel_idx,
                     nsel_before);
  return hipGetLastError();
}

}  // namespace natsl
