// Device helpers shared by the NAtS-L kernels (gfx950 / CDNA4).
//
// Matrix products use 16x16 MFMA tiles with a 32-deep contraction step:
//   bf16: one v_mfma_f32_16x16x32_bf16 per step (8 bf16 per lane per operand)
//   fp32: eight v_mfma_f32_16x16x4_f32 per step (one fp32 per lane each)
// A lane l (g = l / 16, c = l % 16) holds, for a step,
//   A operand: row c of the 16x32 A tile, 8 contraction indices kmap(g, 0..7)
//   B operand: column c of the 32x16 B tile, the same 8 contraction indices
// and the fp32 accumulator holds C[4g + i][c], i = 0..3.
// Any bijective kmap works as long as A and B use the same one, because the
// hardware pairs A's and B's values by (lane group, slot).  Two maps are used:
//   KMAP_ROW: kmap(g, j) = 8g + j            (contiguous: 16 B of a row)
//   KMAP_ACC: kmap(g, j) = 4g + j      (j<4)  (the layout an accumulator has:
//             kmap(g, j) = 16 + 4g + j-4 (j>=4) two stacked 16-row C tiles)
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace natsl {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short v4i16 __attribute__((ext_vector_type(4)));  // ds_read_b64_tr_b16 result
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int CHUNK = 64;
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }

// One lane's share of an MFMA operand for one 32-deep step.
template <typename T> struct Frag;
template <> struct Frag<bf16> { bf16x8 v; };
template <> struct Frag<float> { float v[8]; };

__device__ __forceinline__ void mma(f32x4& c, const Frag<bf16>& a, const Frag<bf16>& b) {
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, c, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x4& c, const Frag<float>& a, const Frag<float>& b) {
#pragma unroll
  for (int j = 0; j < 8; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[j], b.v[j], c, 0, 0, 0);
}

// f when keep, else a zero fragment: a selection, never a product, so that a
// non-finite fragment cannot survive as 0 * inf
__device__ __forceinline__ Frag<bf16> frag_select(bool keep, const Frag<bf16>& f) {
  typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
  const u32x4_t u = __builtin_bit_cast(u32x4_t, f.v);
  u32x4_t r;
#pragma unroll
  for (int j = 0; j < 4; ++j) r[j] = keep ? u[j] : 0u;
  Frag<bf16> o;
  o.v = __builtin_bit_cast(bf16x8, r);
  return o;
}
__device__ __forceinline__ Frag<float> frag_select(bool keep, const Frag<float>& f) {
  Frag<float> o;
#pragma unroll
  for (int j = 0; j < 8; ++j) o.v[j] = keep ? f.v[j] : 0.f;
  return o;
}

template <typename T> __device__ __forceinline__ T frag_get(const Frag<T>& f, int j);
template <> __device__ __forceinline__ bf16 frag_get<bf16>(const Frag<bf16>& f, int j) { return f.v[j]; }
template <> __device__ __forceinline__ float frag_get<float>(const Frag<float>& f, int j) { return f.v[j]; }
__device__ __forceinline__ void frag_set(Frag<bf16>& f, int j, float x) { f.v[j] = (bf16)x; }
__device__ __forceinline__ void frag_set(Frag<float>& f, int j, float x) { f.v[j] = x; }

// 8 contiguous elements (16 B bf16 / 32 B fp32) <-> Frag
template <typename T> __device__ __forceinline__ Frag<T> load8(const T* p);
template <> __device__ __forceinline__ Frag<bf16> load8<bf16>(const bf16* p) {
  Frag<bf16> f;
  f.v = *reinterpret_cast<const bf16x8*>(p);
  return f;
}
template <> __device__ __forceinline__ Frag<float> load8<float>(const float* p) {
  Frag<float> f;
  f32x4 a = *reinterpret_cast<const f32x4*>(p);
  f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
  f.v[0] = a[0]; f.v[1] = a[1]; f.v[2] = a[2]; f.v[3] = a[3];
  f.v[4] = b[0]; f.v[5] = b[1]; f.v[6] = b[2]; f.v[7] = b[3];
  return f;
}
template <typename T> __device__ __forceinline__ void store8(T* p, const Frag<T>& f);
template <> __device__ __forceinline__ void store8<bf16>(bf16* p, const Frag<bf16>& f) {
  *reinterpret_cast<bf16x8*>(p) = f.v;
}
template <> __device__ __forceinline__ void store8<float>(float* p, const Frag<float>& f) {
  f32x4 a = {f.v[0], f.v[1], f.v[2], f.v[3]};
  f32x4 b = {f.v[4], f.v[5], f.v[6], f.v[7]};
  *reinterpret_cast<f32x4*>(p) = a;
  *reinterpret_cast<f32x4*>(p + 4) = b;
}

// 4 contiguous elements <-> floats
template <typename T> __device__ __forceinline__ void load4f(const T* p, float* o);
template <> __device__ __forceinline__ void load4f<bf16>(const bf16* p, float* o) {
  bf16x4 v = *reinterpret_cast<const bf16x4*>(p);
  o[0] = (float)v[0]; o[1] = (float)v[1]; o[2] = (float)v[2]; o[3] = (float)v[3];
}
template <> __device__ __forceinline__ void load4f<float>(const float* p, float* o) {
  f32x4 v = *reinterpret_cast<const f32x4*>(p);
  o[0] = v[0]; o[1] = v[1]; o[2] = v[2]; o[3] = v[3];
}
template <typename T> __device__ __forceinline__ void store4f(T* p, const float* o);
template <> __device__ __forceinline__ void store4f<bf16>(bf16* p, const float* o) {
  bf16x4 v = {(bf16)o[0], (bf16)o[1], (bf16)o[2], (bf16)o[3]};
  *reinterpret_cast<bf16x4*>(p) = v;
}
template <> __device__ __forceinline__ void store4f<float>(float* p, const float* o) {
  f32x4 v = {o[0], o[1], o[2], o[3]};
  *reinterpret_cast<f32x4*>(p) = v;
}

// 8 contiguous elements -> floats
template <typename T> __device__ __forceinline__ void load8f(const T* p, float* o) {
  Frag<T> f = load8<T>(p);
#pragma unroll
  for (int j = 0; j < 8; ++j) o[j] = to_f32(frag_get<T>(f, j));
}

// two 4-element pieces (e.g. two key groups of one column) -> one fragment
template <typename T> __device__ __forceinline__ Frag<T> ld4x2(const T* p0, const T* p1);
template <> __device__ __forceinline__ Frag<bf16> ld4x2<bf16>(const bf16* p0, const bf16* p1) {
  bf16x4 a = *reinterpret_cast<const bf16x4*>(p0);
  bf16x4 b = *reinterpret_cast<const bf16x4*>(p1);
  Frag<bf16> f;
  f.v = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  return f;
}
template <> __device__ __forceinline__ Frag<float> ld4x2<float>(const float* p0, const float* p1) {
  f32x4 a = *reinterpret_cast<const f32x4*>(p0);
  f32x4 b = *reinterpret_cast<const f32x4*>(p1);
  Frag<float> f;
  f.v[0] = a[0]; f.v[1] = a[1]; f.v[2] = a[2]; f.v[3] = a[3];
  f.v[4] = b[0]; f.v[5] = b[1]; f.v[6] = b[2]; f.v[7] = b[3];
  return f;
}
// 4 values -> 4 contiguous elements (e.g. one key group of a column)
template <typename T> __device__ __forceinline__ void st4(T* p, float a, float b, float c, float d);
template <> __device__ __forceinline__ void st4<bf16>(bf16* p, float a, float b, float c, float d) {
  bf16x4 v = {(bf16)a, (bf16)b, (bf16)c, (bf16)d};
  *reinterpret_cast<bf16x4*>(p) = v;
}
template <> __device__ __forceinline__ void st4<float>(float* p, float a, float b, float c, float d) {
  f32x4 v = {a, b, c, d};
  *reinterpret_cast<f32x4*>(p) = v;
}

// a fragment from a function of the element index (scattered reads)
template <typename T, typename Fn>
__device__ __forceinline__ Frag<T> frag_fn(Fn fn) {
  Frag<T> f;
#pragma unroll
  for (int j = 0; j < 8; ++j) frag_set(f, j, fn(j));
  return f;
}

__device__ __forceinline__ int kmap_acc(int g, int j) { return (j < 4) ? (4 * g + j) : (16 + 4 * g + (j - 4)); }

// "Key-group" LDS layout for an operand whose contraction index runs over
// tokens (rows of a row-major [64 x NCOL] tile): element (tok, col) is stored at
//   ((tok / 4) * RL + swz(col)) * 4 + tok % 4,   RL = kg_row<T, NCOL>
// so the 4 tokens 4kg..4kg+3 of one column are contiguous (one 8-byte bf16 /
// 16-byte fp32 read).  swz permutes columns inside each group of 16 so that
// 16 lanes reading 16 consecutive columns, or 16 lanes writing columns
// 8m + i (m = 0..15), hit distinct banks; each key-group row is padded by
// 128 bytes so that the next 16 lanes (the next key group) land on the other
// half of the 64 banks.
template <typename T, int NCOL> constexpr int kg_row() { return NCOL + 32 / (int)sizeof(T); }
__device__ __forceinline__ int kg_swz(int col) {
  const int hi = col >> 4;
  return (col & ~15) | ((col ^ hi) & 15);
}
template <int RL> __device__ __forceinline__ int kg_index(int kg, int col) {
  return (kg * RL + kg_swz(col)) * 4;
}

// Wave-level helpers (wave64).
__device__ __forceinline__ float wave_max_xor(float v, int mask) {
  return fmaxf(v, __shfl_xor(v, mask, 64));
}
__device__ __forceinline__ float wave_sum_xor(float v, int mask) { return v + __shfl_xor(v, mask, 64); }
// Sum over aligned groups of N = 8 or 16 lanes, in registers (DPP), result in
// every lane of the group: quad xor 1, quad xor 2, then the half-row mirror
// (lane i <-> 7 - i pairs the two quads of each 8) and, for 16, the row
// mirror (i <-> 15 - i pairs the two halves).
template <int N>
__device__ __forceinline__ float dpp_group_sum(float x) {
  static_assert(N == 8 || N == 16, "groups of 8 or 16 lanes");
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, true));   // quad_perm 1,0,3,2
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, true));   // quad_perm 2,3,0,1
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x141, 0xF, 0xF, true));  // row_half_mirror
  if (N == 16)
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x140, 0xF, 0xF, true));  // row_mirror
  return x;
}
// max / sum over the 4 lanes c, c + 16, c + 32, c + 48 (the 4 lane groups of
// an MFMA accumulator column), with the gfx950 row swaps instead of LDS
// permutes: permlane16_swap pairs rows 0-1 and 2-3, permlane32_swap rows 0-2
// and 1-3
__device__ __forceinline__ float group4_max(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  auto r2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r2[0]), __uint_as_float(r2[1]));
}
__device__ __forceinline__ float group4_sum(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  auto r2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r2[0]) + __uint_as_float(r2[1]);
}
// sum over the whole wave, in registers: rows of 16 by DPP, then the 4 rows
__device__ __forceinline__ float wave_sum64(float x) { return group4_sum(dpp_group_sum<16>(x)); }

// Workgroup barrier that orders LDS only: waits for this wave's LDS accesses
// and meets the other waves, but leaves global loads in flight (a plain
// __syncthreads() also drains outstanding global loads, which would defeat
// prefetching the next step's operands).  The memory clobber keeps the
// compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// 16-byte global -> LDS load of this lane to lds_wave_base + 16 * lane (the
// wave writes 1 KiB of LDS contiguously).  Issued from inline assembly so that
// the compiler's wait insertion, which cannot tell ring stages apart, does not
// drain every outstanding load before each LDS read; kernels that use it wait
// for these loads themselves (wait_vm, then a barrier for the other waves).
__device__ __forceinline__ void gload_lds16(const void* gptr, const void* lds_wave_base) {
  const uint32_t base = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)lds_wave_base);
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(base), "v"(gptr) : "memory", "m0");
}
// The same with a wave-uniform 64-bit base in SGPRs and a 32-bit lane offset
// (one VGPR per distinct offset pattern instead of a 64-bit address per load).
// readfirstlane returns int: both halves are zero-extended before they are
// joined, a sign-extended low half would corrupt the high one.
__device__ __forceinline__ void gload_lds16_s(const void* gbase, uint32_t voff, const void* lds_wave_base) {
  const uint32_t base = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)lds_wave_base);
  const uint64_t gp = (uint64_t)(uintptr_t)gbase;
  const uint32_t ghi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(gp >> 32));
  const uint32_t glo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)gp);
  const uint64_t gs = ((uint64_t)ghi << 32) | (uint64_t)glo;
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(base), "v"(voff), "s"(gs)
               : "memory", "m0");
}
// The same, non-temporal: for operands that one kernel reads once, so that
// streaming them does not displace lines other kernels reuse.
__device__ __forceinline__ void gload_lds16_s_nt(const void* gbase, uint32_t voff, const void* lds_wave_base) {
  const uint32_t base = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)lds_wave_base);
  const uint64_t gp = (uint64_t)(uintptr_t)gbase;
  const uint32_t ghi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(gp >> 32));
  const uint32_t glo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)gp);
  const uint64_t gs = ((uint64_t)ghi << 32) | (uint64_t)glo;
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2 nt" ::"s"(base), "v"(voff), "s"(gs)
               : "memory", "m0");
}
// s_waitcnt until at most N vector memory operations of this wave are
// outstanding (they complete in issue order); expcnt / lgkmcnt not waited
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}
// s_waitcnt with vmcnt = n (expcnt / lgkmcnt not waited); n in {0, 4, 8}
__device__ __forceinline__ void wait_vm(int n) {
  if (n >= 8) __builtin_amdgcn_s_waitcnt(0x0F78);
  else if (n >= 4) __builtin_amdgcn_s_waitcnt(0x0F74);
  else __builtin_amdgcn_s_waitcnt(0x0F70);
}
// Hides a wave-uniform value from the optimiser.  A ring stage offset is one
// of a few values; left visible, the compiler precomputes the addresses of
// every stage and keeps them all live.
__device__ __forceinline__ int opaque_sgpr(int x) {
  x = __builtin_amdgcn_readfirstlane(x);
  asm volatile("" : "+s"(x));
  return x;
}
// Work-item and workgroup indices straight from the hardware.  HIP's
// threadIdx / blockIdx / gridDim are device-library functions built with the
// default target features; this library is compiled with packed fp32 ops
// disabled, so they are not inlined into its kernels: every use becomes a call
// whose result the compiler must take as divergent, which turns all control
// flow derived from the block index into exec-mask branches.
__device__ __forceinline__ int tid_x() { return (int)__builtin_amdgcn_workitem_id_x(); }
__device__ __forceinline__ int bid_x() { return (int)__builtin_amdgcn_workgroup_id_x(); }
__device__ __forceinline__ int bid_y() { return (int)__builtin_amdgcn_workgroup_id_y(); }
// HSA kernel dispatch packet: workgroup_size_x (u16) at byte 4, grid_size_x
// (u32, in work-items) at byte 12
typedef const __attribute__((address_space(4))) char* dispatch_bytes;
__device__ __forceinline__ int block_dim_x() {
  const dispatch_bytes dp = (dispatch_bytes)__builtin_amdgcn_dispatch_ptr();
  return *(const __attribute__((address_space(4))) uint16_t*)(dp + 4);
}
__device__ __forceinline__ int grid_dim_x() {
  const dispatch_bytes dp = (dispatch_bytes)__builtin_amdgcn_dispatch_ptr();
  return (int)(*(const __attribute__((address_space(4))) uint32_t*)(dp + 12) /
               *(const __attribute__((address_space(4))) uint16_t*)(dp + 4));
}
__device__ __forceinline__ int lane_id() { return tid_x() & 63; }
// wave-uniform by construction; readfirstlane lets the compiler know it, so
// branches on the wave index are scalar branches
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(tid_x() >> 6); }

}  // namespace natsl
