// Prefill -> decode handoff.
//
// "Technische Samenvatting: Neural Attention Search Linear (NAtS-L)",
// Kernmechanismen 3: after a prefix the softmax operation keeps the KV of the
// chunks routed to it and the linear operation keeps its fixed-size state.  A
// prefill of L tokens (a whole number of 64-token chunks) therefore leaves the
// decode cache as:
//   K/V rows   the rows of the softmax-routed chunks, in chunk order
//              (n_committed = 64 x their number, per sequence and route group);
//   S_carry    the Gated DeltaNet state after the prefix (only linear-routed
//              chunks moved it), i.e. the forward pass's final state;
//   open chunk empty: n_open = 0, S_work = 0, x_sum = 0.
// Appended to a cache that already holds a prefix at a chunk boundary (chunked
// prefill), the segment's rows go after the cache's n_committed rows and the
// counts add up.  Three launches on the caller's stream: the compaction of the
// routes (chunk list per (b, g)), then the states and counters and the row
// copies (copies first when appending: they read the old row counts).
#include "common.hpp"
#include "kernels.hpp"

namespace natsl {

// S_carry <- S_final (or zero), S_work <- 0, x_sum <- 0, counters, error flag
// (cleared unless appending).  Thread i handles four state floats, four x_sum
// floats and counter i.
__global__ void __launch_bounds__(256) k_handoff_state(const float* __restrict__ S_final, int64_t n_state,
                                                       float* __restrict__ S_carry, float* __restrict__ S_work,
                                                       float* __restrict__ x_sum, int64_t n_x,
                                                       const int32_t* __restrict__ nsel_before, int BG, int nc,
                                                       int32_t* __restrict__ n_committed,
                                                       int32_t* __restrict__ n_open, int B,
                                                       int32_t* __restrict__ err_flag, int append) {
  const int64_t i = (int64_t)bid_x() * 256 + tid_x();
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  if (4 * i < n_state) {
    reinterpret_cast<f32x4*>(S_carry)[i] = S_final ? reinterpret_cast<const f32x4*>(S_final)[i] : zero;
    reinterpret_cast<f32x4*>(S_work)[i] = zero;
  }
  if (4 * i < n_x) reinterpret_cast<f32x4*>(x_sum)[i] = zero;
  if (i < BG) n_committed[i] = (append ? n_committed[i] : 0) + CHUNK * nsel_before[i * (nc + 1) + nc];
  if (i < B) n_open[i] = 0;
  if (i == 0 && !append) err_flag[0] = 0;
}

// One workgroup per (list position, b * H + h): copies the 64 K and V rows of
// the position-th softmax chunk of (b, g) to cache rows base + 64 * position
// (base = the cache's n_committed[b, g] when appending, else 0).  Rows at or
// beyond the capacity are not written and raise the error flag, as does an
// append to a cache with an open chunk (every writer stores the same 1, no
// atomics).
template <typename T>
__global__ void __launch_bounds__(256) k_handoff_kv(const T* __restrict__ k, const T* __restrict__ v,
                                                    const int32_t* __restrict__ sel_idx,
                                                    const int32_t* __restrict__ nsel_before, int H, int G, int L,
                                                    int D, int nc, int cap, T* __restrict__ k_cache,
                                                    T* __restrict__ v_cache, int32_t* __restrict__ err_flag,
                                                    const int32_t* __restrict__ base_rows,
                                                    const int32_t* __restrict__ n_open) {
  const unsigned bid = (unsigned)bid_x();  // (list position, b * H + h) flattened, position fastest
  const int pos = (int)(bid % (unsigned)nc), bh = (int)(bid / (unsigned)nc);
  const int b = bh / H, h = bh % H, g = (G == 1) ? 0 : h;
  const int64_t bg = (int64_t)b * G + g;
  if (pos >= nsel_before[bg * (nc + 1) + nc]) return;
  if (base_rows && n_open[b] != 0 && tid_x() == 0) err_flag[0] = 1;
  const int c = sel_idx[bg * nc + pos];
  const int64_t row0l = (base_rows ? (int64_t)base_rows[bg] : 0) + (int64_t)pos * CHUNK;
  if (row0l < 0 || row0l >= cap) {
    if (tid_x() == 0) err_flag[0] = 1;
    return;
  }
  const int row0 = (int)row0l;
  const int rows = min(CHUNK, cap - row0);
  if (rows < CHUNK && tid_x() == 0) err_flag[0] = 1;
  const int64_t src = ((int64_t)bh * L + (int64_t)c * CHUNK) * D;
  const int64_t dst = ((int64_t)bh * cap + row0) * D;
  const int per_row = D * (int)sizeof(T) / 16;  // 16-byte pieces of a row
  const int total = rows * per_row;
  const uint4* ks = reinterpret_cast<const uint4*>(k + src);
  const uint4* vs = reinterpret_cast<const uint4*>(v + src);
  uint4* kd = reinterpret_cast<uint4*>(k_cache + dst);
  uint4* vd = reinterpret_cast<uint4*>(v_cache + dst);
  for (int i = tid_x(); i < total; i += 256) {
    kd[i] = ks[i];
    vd[i] = vs[i];
  }
}

size_t handoff_ws_bytes(int B, int G, int nc) { return (size_t)B * G * (2 * nc + 1) * sizeof(int32_t); }

template <typename T>
hipError_t launch_handoff(const HandoffLaunch& a, void* ws, hipStream_t st) {
  const int nc = a.L / CHUNK;
  const int BG = a.B * a.G;
  int32_t* sel = static_cast<int32_t*>(ws);
  int32_t* nsb = sel + (size_t)BG * nc;
  // the route list is only read (route_out == route_in skips the copy)
  hipError_t e = launch_compact(a.route, const_cast<int32_t*>(a.route), a.B, a.G, nc, sel, nsb, st);
  if (e != hipSuccess) return e;
  const int64_t n_state = (int64_t)a.B * a.H * a.D * a.D;
  const int64_t n_x = (int64_t)a.B * a.d;
  int64_t items = n_state / 4;
  if (n_x / 4 > items) items = n_x / 4;
  if (BG > items) items = BG;
  if (a.B > items) items = a.B;
  auto state = [&]() {
    hipLaunchKernelGGL(k_handoff_state, dim3((unsigned)((items + 255) / 256)), dim3(256), 0, st, a.S_final,
                       n_state, a.S_carry, a.S_work, a.x_sum, n_x, nsb, BG, nc, a.n_committed, a.n_open, a.B,
                       a.err_flag, a.append);
    return hipGetLastError();
  };
  auto rows = [&]() {
    hipLaunchKernelGGL(k_handoff_kv<T>, dim3((unsigned)(nc * a.B * a.H)), dim3(256), 0, st, (const T*)a.k, (const T*)a.v, sel,
                       nsb, a.H, a.G, a.L, a.D, nc, a.cap, (T*)a.k_cache, (T*)a.v_cache, a.err_flag,
                       a.append ? (const int32_t*)a.n_committed : nullptr, (const int32_t*)a.n_open);
    return hipGetLastError();
  };
  if (a.append) {
    if ((e = rows()) != hipSuccess) return e;
    return state();
  }
  if ((e = state()) != hipSuccess) return e;
  return rows();
}

template hipError_t launch_handoff<float>(const HandoffLaunch&, void*, hipStream_t);
template hipError_t launch_handoff<bf16>(const HandoffLaunch&, void*, hipStream_t);

}  // namespace natsl
