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
#include "common.hpp"
#include "kernels.hpp"

namespace natsl {

template <typename T>
__global__ void __launch_bounds__(256) k_route(const T* __restrict__ x, const float* __restrict__ w,
                                               const float* __restrict__ bsc, int L, int d, int G,
                                               int nc, int32_t* __restrict__ route_out,
                                               float* __restrict__ scores) {
  extern __shared__ float s_mean[];  // [d]
  const int c = bid_x(), b = bid_y();
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
  extern __shared__ float s_part[];  // [RS][d] partial sums, then the mean [d] and 2G scores
  const int c = bid_x(), b = bid_y();
  const int tid = tid_x();
  const int ncg = d >> 3;          // column groups
  const int rs = 1024 / ncg;       // row slices (1 .. 64 ... capped below)
  const int rows = CHUNK / rs;     // rows per thread
  const int cg = tid % ncg, sl = tid / ncg;
  const T* xc = x + ((int64_t)b * L + (int64_t)c * CHUNK + (int64_t)sl * rows) * d + cg * 8;
  float acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.f;
  {
    // batches of 8 independent 16-byte loads (two workgroups per CU keep
    // 16 per column group in flight)
    for (int r = 0; r < rows; r += 8) {
      Frag<T> v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = load8<T>(xc + (int64_t)min(r + u, rows - 1) * d);
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
  __syncthreads();
  float* s_mean = s_part + rs * d;
  for (int col = tid; col < d; col += 1024) {
    float t = 0.f;
    for (int k = 0; k < rs; ++k) t += s_part[k * d + col];
    s_mean[col] = t * (1.0f / CHUNK);
  }
  __syncthreads();
  const int lane = lane_id(), wv = wave_id();
  for (int o = wv; o < 2 * G; o += 16) {
    float p = 0.f;
    for (int j = lane; j < d; j += 64) p += s_mean[j] * w[(int64_t)j * 2 * G + o];
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
__global__ void __launch_bounds__(256) k_route_bwd_ds(const float* __restrict__ scores,
                                                      const float* __restrict__ dg_sm,
                                                      const float* __restrict__ dg_lin, int B, int H, int G, int nc,
                                                      float* __restrict__ ds) {
  const int64_t i = (int64_t)bid_x() * 256 + tid_x();
  if (i >= (int64_t)B * G * nc) return;
  const int c = (int)(i % nc), g = (int)((i / nc) % G), b = (int)(i / ((int64_t)nc * G));
  const int hpg = H / G;
  float dh0 = 0.f, dh1 = 0.f;
  for (int h = g * hpg; h < (g + 1) * hpg; ++h) {
    const int64_t j = ((int64_t)b * H + h) * nc + c;
    dh0 += dg_sm[j];
    dh1 += dg_lin[j];
  }
  const float s0 = scores[i * 2], s1 = scores[i * 2 + 1];
  const float m = fmaxf(s0, s1);
  const float e0 = __expf(s0 - m), e1 = __expf(s1 - m);
  const float p0 = e0 / (e0 + e1), p1 = e1 / (e0 + e1);
  const float pd = p0 * dh0 + p1 * dh1;
  ds[i * 2] = p0 * (dh0 - pd);
  ds[i * 2 + 1] = p1 * (dh1 - pd);
}

// per (b, c): the chunk mean of x (kept for dW) and dx of the chunk's rows
template <typename T>
__global__ void __launch_bounds__(256) k_route_bwd_x(const T* __restrict__ x, const float* __restrict__ w,
                                                     const float* __restrict__ ds, int L, int d, int G, int nc,
                                                     float* __restrict__ pooled, float* __restrict__ dx) {
  const int c = bid_x(), b = bid_y();
  const T* xc = x + ((int64_t)b * L + (int64_t)c * CHUNK) * d;
  const float* dsc = ds + ((int64_t)b * G * nc + c) * 2;  // + (g nc) * 2 + o
  for (int col = tid_x(); col < d; col += 256) {
    float sx = 0.f;
    for (int r = 0; r < CHUNK; ++r) sx += to_f32(xc[(int64_t)r * d + col]);
    pooled[((int64_t)b * nc + c) * d + col] = sx * (1.0f / CHUNK);
    if (dx) {
      float gx = 0.f;
      for (int g = 0; g < G; ++g)
        gx += w[(int64_t)col * 2 * G + 2 * g] * dsc[(int64_t)g * nc * 2] +
              w[(int64_t)col * 2 * G + 2 * g + 1] * dsc[(int64_t)g * nc * 2 + 1];
      gx *= 1.0f / CHUNK;
      float* dxc = dx + ((int64_t)b * L + (int64_t)c * CHUNK) * d + col;
      for (int r = 0; r < CHUNK; ++r) dxc[(int64_t)r * d] = gx;
    }
  }
}

// dW [d, 2G] and db [2G]: one thread per output, the (b, c) sum in order
__global__ void __launch_bounds__(256) k_route_bwd_w(const float* __restrict__ pooled, const float* __restrict__ ds,
                                                     int B, int G, int nc, int d, float* __restrict__ dw,
                                                     float* __restrict__ db) {
  const int64_t i = (int64_t)bid_x() * 256 + tid_x();
  const int64_t nw = (int64_t)d * 2 * G;
  if (i < nw) {
    const int col = (int)(i / (2 * G)), o = (int)(i % (2 * G)), g = o / 2, oo = o % 2;
    float acc = 0.f;
    for (int b = 0; b < B; ++b)
      for (int c = 0; c < nc; ++c)
        acc += pooled[((int64_t)b * nc + c) * d + col] * ds[(((int64_t)b * G + g) * nc + c) * 2 + oo];
    dw[i] = acc;
  } else if (db && i < nw + 2 * G) {
    const int o = (int)(i - nw), g = o / 2, oo = o % 2;
    float acc = 0.f;
    for (int b = 0; b < B; ++b)
      for (int c = 0; c < nc; ++c) acc += ds[(((int64_t)b * G + g) * nc + c) * 2 + oo];
    db[o] = acc;
  }
}

size_t route_bwd_ws_bytes(int B, int G, int L, int d) {
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const size_t nc = (size_t)L / CHUNK;
  return al((size_t)B * G * nc * 2 * 4) + al((size_t)B * nc * d * 4);
}

template <typename T>
hipError_t launch_route_backward(const T* x, const float* w, const float* scores, const float* dg_sm,
                                 const float* dg_lin, float* dx, float* dw, float* db, void* wsp, int B, int H, int L,
                                 int d, int G, hipStream_t st) {
  auto al = [](size_t v) { return (v + 255) & ~(size_t)255; };
  const int nc = L / CHUNK;
  float* ds = (float*)wsp;
  float* pooled = (float*)((char*)wsp + al((size_t)B * G * nc * 2 * 4));
  const int64_t n = (int64_t)B * G * nc;
  hipLaunchKernelGGL(k_route_bwd_ds, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, scores, dg_sm, dg_lin, B,
                     H, G, nc, ds);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_route_bwd_x<T>, dim3(nc, B), dim3(256), 0, st, x, w, ds, L, d, G, nc, pooled, dx);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int64_t nt = (int64_t)d * 2 * G + 2 * G;
  hipLaunchKernelGGL(k_route_bwd_w, dim3((unsigned)((nt + 255) / 256)), dim3(256), 0, st, pooled, ds, B, G, nc, d,
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
    const size_t lds = (size_t)(rs * d + d + 2 * G) * sizeof(float);
    if (lds <= (size_t)LDS_MAX_BYTES) {
      const hipError_t e = set_lds_limit((const void*)k_route_wide<T>, (int)lds);
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL(k_route_wide<T>, dim3(nc, B), dim3(1024), lds, st, x, w, bsc, L, d, G, nc, route_out,
                         scores);
      return hipGetLastError();
    }
  }
  const size_t lds = (size_t)(d + 2 * G) * sizeof(float);
  hipLaunchKernelGGL(k_route<T>, dim3(nc, B), dim3(256), lds, st, x, w, bsc, L, d, G, nc, route_out,
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
